// Checks make_div32/div32 (the kernels' 32-bit division by a launch-fixed
// divisor) against exact division: every divisor up to 4096, powers of two
// and their neighbours, divisors near 2^31 and 2^32, and pseudo-random ones;
// for each, dividends at 0, around every multiple of the divisor near the
// ends of the 32-bit range, at 2^32-1, and pseudo-random.  Prints "ok <n>"
// or the first mismatch.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "ccv_internal.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next32() {  // xorshift64*
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return static_cast<uint32_t>((state * 0x2545F4914F6CDD1Dull) >> 32);
}

int main() {
    std::vector<uint32_t> divisors;
    for (uint32_t d = 1; d <= 4096; ++d) divisors.push_back(d);
    for (int k = 12; k < 32; ++k)
        for (int64_t e = -2; e <= 2; ++e) divisors.push_back(static_cast<uint32_t>((int64_t(1) << k) + e));
    for (uint32_t e = 0; e < 8; ++e) divisors.push_back(0xFFFFFFFFu - e);
    for (int i = 0; i < 2000; ++i) divisors.push_back(next32() | 1u);
    for (int i = 0; i < 2000; ++i) divisors.push_back((next32() >> (next32() % 31)) + 1u);
    uint64_t checked = 0;
    for (uint32_t d : divisors) {
        const ccv::Div32 v = ccv::make_div32(d);
        std::vector<uint32_t> ns = {0u, 1u, d - 1u, d, d + 1u, 0xFFFFFFFFu, 0xFFFFFFFEu, 0x80000000u,
                                    0x7FFFFFFFu};
        const uint64_t top = 0xFFFFFFFFull / d;
        for (uint64_t q : {uint64_t(1), uint64_t(2), top / 2, top - 1, top}) {
            const uint64_t m = q * d;
            for (int64_t e = -1; e <= 1; ++e) {
                const int64_t n = static_cast<int64_t>(m) + e;
                if (n >= 0 && n <= 0xFFFFFFFFll) ns.push_back(static_cast<uint32_t>(n));
            }
        }
        for (int i = 0; i < 64; ++i) ns.push_back(next32());
        for (uint32_t n : ns) {
            ++checked;
            if (ccv::div32(n, v) != n / d) {
                std::printf("mismatch n=%u d=%u got=%u want=%u\n", n, d, ccv::div32(n, v), n / d);
                return 1;
            }
        }
    }
    std::printf("ok %llu\n", static_cast<unsigned long long>(checked));
    return 0;
}

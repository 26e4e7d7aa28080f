// ccv_misc.hip — width-independent launches (offset validation, the fixed-
// order dW reduction) and the switch from a call's filter width to the
// kernels built for it.
#include <atomic>
#include <mutex>

#include "ccv_device.h"

namespace ccv {

// Scratch of the allocation-free backward (ccv_bwd_noalloc): the partials of
// the deterministic dW/dB route live here instead of in a caller workspace.
// Every device the library runs on holds its own copy, at its own address,
// until the process ends.  Host code must never pass `scratch` itself to a
// kernel or a copy (on the host the name is only a stand-in): it uses the
// device address looked up below.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t noalloc_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

// Resident blocks of a kernel on the current device (CUs x blocks per CU),
// from the occupancy the compiled kernel allows; 0 when it cannot be told.
int64_t device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

int64_t resident_blocks(const void *kernel, unsigned dyn_lds) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, dyn_lds) != hipSuccess)
        return 0;
    return static_cast<int64_t>(cus) * per_cu;
}

hipError_t launch_fwd(const FwdArgs &a, int vec, int silu, int rows, hipStream_t s) {
    switch (a.width) {
    case 2: return fwd_dispatch_w2(a, vec, silu, rows, s, nullptr);
    case 3: return fwd_dispatch_w3(a, vec, silu, rows, s, nullptr);
    case 4: return fwd_dispatch_w4(a, vec, silu, rows, s, nullptr);
    default: return hipErrorInvalidValue;
    }
}

int64_t fwd_resident_blocks(const FwdArgs &a, int vec, int silu, int rows) {
    int64_t cap = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (a.width) {
    case 2: e = fwd_dispatch_w2(a, vec, silu, rows, kQueryStream, &cap); break;
    case 3: e = fwd_dispatch_w3(a, vec, silu, rows, kQueryStream, &cap); break;
    case 4: e = fwd_dispatch_w4(a, vec, silu, rows, kQueryStream, &cap); break;
    default: break;
    }
    return e == hipSuccess ? cap : 0;
}

hipError_t launch_bwd(const BwdArgs &a, int vec, int silu, int rows, hipStream_t s) {
    switch (a.width) {
    case 2: return bwd_dispatch_w2(a, vec, silu, rows, s, nullptr);
    case 3: return bwd_dispatch_w3(a, vec, silu, rows, s, nullptr);
    case 4: return bwd_dispatch_w4(a, vec, silu, rows, s, nullptr);
    default: return hipErrorInvalidValue;
    }
}

int64_t bwd_resident_blocks(const BwdArgs &a, int vec, int silu, int rows) {
    int64_t cap = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (a.width) {
    case 2: e = bwd_dispatch_w2(a, vec, silu, rows, kQueryStream, &cap); break;
    case 3: e = bwd_dispatch_w3(a, vec, silu, rows, kQueryStream, &cap); break;
    case 4: e = bwd_dispatch_w4(a, vec, silu, rows, kQueryStream, &cap); break;
    default: break;
    }
    return e == hipSuccess ? cap : 0;
}

hipError_t launch_update(const UpdArgs &a, int vec, int silu, hipStream_t s) {
    switch (a.width) {
    case 2: return update_dispatch_w2(a, vec, silu, s);
    case 3: return update_dispatch_w3(a, vec, silu, s);
    case 4: return update_dispatch_w4(a, vec, silu, s);
    default: return hipErrorInvalidValue;
    }
}

int update_rows_per_lane() { return CCV_UPD_ROWS; }

hipError_t launch_validate(const int32_t *cu, int64_t n_seq, int64_t total, uint32_t *flags,
                           int overwrite, hipStream_t s) {
    hipLaunchKernelGGL(k_validate, dim3(1), dim3(256), 0, s, cu, n_seq, total, flags, overwrite);
    return hipGetLastError();
}

hipError_t launch_dw_reduce(const float *partial, int64_t n_part, int64_t n_ch, int w, int kp,
                            float *dw, float *db, const uint32_t *err, hipStream_t s) {
    // 16-byte lanes when every partial row is a whole number of 16-byte
    // vectors (the partials start 256-byte aligned); 64 lanes per block.
    const int64_t n_elem = n_ch * kp;
    if (n_elem % 4 == 0) {
        const int64_t blocks = (n_elem / 4 + kWaveSize - 1) / kWaveSize;
        hipLaunchKernelGGL(k_dw_reduce<4>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           partial, n_part, n_ch, w, kp, dw, db, err);
    } else {
        const int64_t blocks = (n_elem + kWaveSize - 1) / kWaveSize;
        hipLaunchKernelGGL(k_dw_reduce<1>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           partial, n_part, n_ch, w, kp, dw, db, err);
    }
    return hipGetLastError();
}

}  // namespace ccv

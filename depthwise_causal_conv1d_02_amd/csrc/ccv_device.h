// ccv_device.h — gfx950 device code of the depthwise causal conv1d (all
// kernels as templates; ccv_width.hip and ccv_misc.hip instantiate them).
//
// Operation (cuDNN FE "Causal Conv1d", tensor/state semantics and the
// optimized route; tap order from the POPCORNBENCH trace's causal left-pad
// derivation):  z = bias + sum_k w[k] * x_ext[t-(W-1)+k],  y = act(z).
//
// Mapping ("channel-lane" kernels).  A lane owns VEC consecutive channels
// (VEC = 8: one 16-byte BF16 vector per token when channels are unit-stride,
// i.e. the [B,T,D] storage behind a transpose(1,2) view; VEC = 1: any
// strides).  A wavefront owns 64*VEC channels and walks a chunk of L time
// steps in order, keeping the W-1 previous tokens (and, backward, the W-1
// previous SiLU gradients) in registers, so every input element is loaded
// once by its chunk plus a W-1 token halo at chunk edges.  Each wave-wide
// load or store touches 64*VEC*2 contiguous bytes.  Four waves of a block
// take four consecutive chunks of the same channel group; block ids are
// remapped so that each XCD (own L2) streams a contiguous range of
// chunks, which keeps the halo re-reads inside one L2.
//
// Packed rows (cu_seqlens) are handled inside a chunk: the chunk is split at
// sequence starts and every piece restarts its window from that sequence's
// initial state (or zeros).  The offsets are staged in LDS, validated there
// by every block (no host read) and searched there.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ccv_internal.h"

namespace ccv {
namespace {
constexpr uint32_t kFirstNonzero = 0x1u, kLastMismatch = 0x2u, kDecreasing = 0x4u,
                   kEmpty = 0x8u;

#ifndef CCV_FWD_UNROLL
#define CCV_FWD_UNROLL 4
#endif
// The software-pipelined forward (inputs of 256 MB and more, 16-step
// chunks): two batches of 8 steps per chunk measured faster than four of 4
// (large 350.8 -> 346.7 us, packed 127.9 -> 123.4 us).
#ifndef CCV_FWD_PIPE_UNROLL
#define CCV_FWD_PIPE_UNROLL 8
#endif
#ifndef CCV_FWD_PIPE_UNROLL_DENSE
#define CCV_FWD_PIPE_UNROLL_DENSE CCV_FWD_PIPE_UNROLL
#endif
// Dense rows on 4-channel lanes (the small-input forward): longer batches,
// more loads in flight from HBM (measured with cold caches).
#ifndef CCV_FWD_SMALL_UNROLL
#define CCV_FWD_SMALL_UNROLL 16
#endif
#ifndef CCV_BWD_UNROLL
#define CCV_BWD_UNROLL 4
#endif
// Measured per row mode: packed rows do best with batches of 2, seq_idx
// rows with software-pipelined batches of 4 (1.2% faster than unpipelined
// batches of 8; pipelined batches of 8 spill).
#ifndef CCV_BWD_UNROLL_PACKED
#define CCV_BWD_UNROLL_PACKED 2
#endif
#ifndef CCV_BWD_UNROLL_SEQ
#define CCV_BWD_UNROLL_SEQ 4
#endif
#ifndef CCV_BWD_SEQ_PIPE
#define CCV_BWD_SEQ_PIPE 1
#endif
#ifndef CCV_TC_BWD_WAVES
#define CCV_TC_BWD_WAVES 6      // time-lane backward: waves per SIMD it must fit (8: 2.5% slower on 200 MB)
#endif
#ifndef CCV_BWD_PIPE
#define CCV_BWD_PIPE 1
#endif
// Interior heads and tails of a backward chunk take a path without the
// row-edge checks (dinit, final-state term, row end).
#ifndef CCV_BWD_FAST_EDGES
#define CCV_BWD_FAST_EDGES 1
#endif
// Lower bound on resident waves per SIMD (register budget), measured best:
// the forward keeps 4 waves; the software-pipelined forward (two batches of
// 8 steps) gets a 2-wave budget, within which its bias-free variants fit in
// 164 registers (3 waves per SIMD) without spilling; a 3-wave budget spills.
#ifndef CCV_FWD_MIN_WAVES
#define CCV_FWD_MIN_WAVES 4
#endif
#ifndef CCV_FWD_PIPE_MIN_WAVES
#define CCV_FWD_PIPE_MIN_WAVES 2
#endif
// Variants that spilled under the 4-wave budget take the 3-wave one.
#ifndef CCV_FWD_SPILL_MIN_WAVES
#define CCV_FWD_SPILL_MIN_WAVES 3
#endif
#ifndef CCV_BWD_MIN_WAVES
#define CCV_BWD_MIN_WAVES 2
#endif
// Variants that would spill under the 4-wave budget (no activation, seq_idx
// rows, packed rows with a bias) take the 3-wave budget instead.
#define CCV_FWD_ATTR                                                                 \
    __attribute__((amdgpu_waves_per_eu(                                              \
        PIPE ? CCV_FWD_PIPE_MIN_WAVES                                                \
        : (!SILU || ROWS == kRowsSeq || (ROWS == kRowsPacked && fk_bias(FK)))        \
            ? CCV_FWD_SPILL_MIN_WAVES                                                \
            : CCV_FWD_MIN_WAVES)))
#ifdef CCV_BWD_MIN_WAVES
#define CCV_BWD_ATTR __attribute__((amdgpu_waves_per_eu(CCV_BWD_MIN_WAVES)))
#else
#define CCV_BWD_ATTR
#endif
// Dynamic LDS (bytes) given to the backward and to the pipelined forward to
// cap their blocks per CU (0: the registers alone decide).
#ifndef CCV_BWD_DYN_LDS
#define CCV_BWD_DYN_LDS 0
#endif
#ifndef CCV_FWD_PIPE_DYN_LDS
#define CCV_FWD_PIPE_DYN_LDS 0
#endif
// Wave index through readfirstlane in the seq_idx kernels.
#ifndef CCV_WAVE_UNIFORM
#define CCV_WAVE_UNIFORM 1
#endif
// Row modes (bit 1 << mode) whose forward / backward take the wave index
// through readfirstlane.
#ifndef CCV_FWD_UNIFORM_ROWS
#define CCV_FWD_UNIFORM_ROWS (1 << 2)
#endif
#ifndef CCV_BWD_UNIFORM_ROWS
#define CCV_BWD_UNIFORM_ROWS (1 << 2)
#endif

// ---------------------------------------------------------------------------
// BF16 <-> FP32.  Widening is exact (the BF16 bits are the top half of the
// FP32 word); narrowing uses gfx950's v_cvt_pk_bf16_f32 (round to nearest
// even), reached through the __bf16 vector conversion.
// ---------------------------------------------------------------------------
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t to_bf16_bits(float a) {
    return static_cast<uint16_t>(pack2_bf16(a, 0.0f) & 0xffffu);
}

// VEC channels of one token as raw BF16 bits (clang vector types, so the
// non-temporal builtins apply).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <int VEC> struct Raw;
template <> struct Raw<8> { u32x4_t v; };
template <> struct Raw<4> { u32x2_t v; };
template <> struct Raw<1> { uint16_t v; };

// Loads and stores of one token's VEC channels.  STREAM selects the
// non-temporal cache policy for data touched once (the bulk of x, dy, y and
// dx); halo and state accesses use the default policy so that re-reads of a
// neighbour chunk's tokens can hit in cache.
#ifndef CCV_NT_LOAD
#define CCV_NT_LOAD 1
#endif
#ifndef CCV_NT_STORE
#define CCV_NT_STORE 1
#endif

template <int VEC, bool STREAM = false>
__device__ __forceinline__ Raw<VEC> load_raw(const uint16_t *p, int64_t) {
    using V = decltype(Raw<VEC>::v);
    const V *q = reinterpret_cast<const V *>(p);
    if constexpr (STREAM && CCV_NT_LOAD) return Raw<VEC>{__builtin_nontemporal_load(q)};
    else return Raw<VEC>{*q};
}

template <int VEC>
__device__ __forceinline__ void unpack(const Raw<VEC> &r, float (&v)[VEC]) {
    if constexpr (VEC == 1) {
        v[0] = bf16_bits_to_f32(r.v);
    } else {
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) {
            v[2 * i] = lo_bf16(r.v[i]);
            v[2 * i + 1] = hi_bf16(r.v[i]);
        }
    }
}

template <int VEC, bool STREAM = false>
__device__ __forceinline__ void store_vec(uint16_t *p, int64_t, const float (&v)[VEC]) {
    using V = decltype(Raw<VEC>::v);
    V r;
    if constexpr (VEC == 1) {
        r = to_bf16_bits(v[0]);
    } else {
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) r[i] = pack2_bf16(v[2 * i], v[2 * i + 1]);
    }
    V *q = reinterpret_cast<V *>(p);
    if constexpr (STREAM && CCV_NT_STORE) __builtin_nontemporal_store(r, q);
    else *q = r;
}

// ---------------------------------------------------------------------------
// Activation and its slope.  SiLU(z) = z * s, s = 1 / (1 + e^-z);
// SiLU'(z) = s * (1 + z (1 - s)) = s + z (s - s^2).  One v_exp_f32 and one
// v_rcp_f32 each.
// ---------------------------------------------------------------------------
template <bool SILU>
__device__ __forceinline__ float act(float z) {
    if constexpr (SILU) return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
    else return z;
}
template <bool SILU>
__device__ __forceinline__ float act_slope(float z) {
    if constexpr (SILU) {
        const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
        return fmaf(z, fmaf(-s, s, s), s);
    } else {
        return 1.0f;
    }
}

// Block id -> logical tile id such that XCD x (hardware dispatches block i
// to XCD i % 8) receives one contiguous range of logical tiles.
#ifndef CCV_XCD_REMAP
#define CCV_XCD_REMAP 1
#endif
#ifndef CCV_BWD_PACKED_TILE_ORDER
#define CCV_BWD_PACKED_TILE_ORDER 0
#endif
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nb) {
    if (!CCV_XCD_REMAP) return bid;
    constexpr int64_t X = 8;
    const int64_t q = nb / X, r = nb % X;
    const int64_t x = bid % X, j = bid / X;
    return x * q + (x < r ? x : r) + j;
}

// Logical tile -> (row b, channel block, time block) in the CCV_TILE_ORDER.
template <int ORDER = CCV_TILE_ORDER>
__device__ __forceinline__ void decode_tile(int64_t tile, int64_t n_t, int64_t n_c, int64_t &b,
                                            int64_t &cb, int64_t &tb) {
    if constexpr (ORDER == 0) {
        tb = tile % n_t;
        cb = (tile / n_t) % n_c;
    } else {
        cb = tile % n_c;
        tb = (tile / n_c) % n_t;
    }
    b = tile / (n_t * n_c);
}

// A block's place in a launch split into main and tail chunks (see
// FwdArgs): the first n_block_m blocks tile [0, Tm) with chunks of L steps,
// the rest tile [Tm, T) with chunks of Lt steps.  Each range is remapped over
// the XCDs on its own, so both spread over every XCD.  `bt` comes back as
// the time block among all n_tblk + n_tblk_t of a (row, channel block): a
// fixed function of the block id, so per-block partials stay shape-determined.
struct TileSpan {
    int64_t b, c, bt;   // row, channel block, time block
    int64_t t0, L, end; // first step of wave 0's chunk, chunk length, range end
};
template <int ORDER, typename A>
__device__ __forceinline__ TileSpan split_tile(const A &a, int64_t n_c, int wt) {
    TileSpan s;
    const int64_t bid = blockIdx.x;
    if (bid < a.n_block_m) {
        decode_tile<ORDER>(xcd_remap(bid, a.n_block_m), a.n_tblk, n_c, s.b, s.c, s.bt);
        s.L = a.L;
        s.t0 = s.bt * wt * a.L;
        s.end = a.Tm;
    } else {
        int64_t bt;
        decode_tile<ORDER>(xcd_remap(bid - a.n_block_m, a.n_block - a.n_block_m), a.n_tblk_t, n_c,
                           s.b, s.c, bt);
        s.L = a.Lt;
        s.t0 = a.Tm + bt * wt * a.Lt;
        s.end = a.T;
        s.bt = a.n_tblk + bt;
    }
    return s;
}

// Filter kinds: the weight dtype and whether a bias is present.  The bias
// has the weight's dtype (an FP32 filter with an FP32 bias is an opt-in of
// the boundary).
enum FilterKind { kBf16 = 0, kBf16Bias = 1, kF32 = 2, kF32Bias = 3 };
// Row modes: dense batch rows, rows packed by cu_seqlens, or rows whose
// tokens carry sequence ids (seq_idx).
enum RowMode { kRowsDense = 0, kRowsPacked = 1, kRowsSeq = 2 };
constexpr bool fk_f32(int fk) { return fk == kF32 || fk == kF32Bias; }
constexpr bool fk_bias(int fk) { return fk == kBf16Bias || fk == kF32Bias; }

// Filter taps and bias of a lane's VEC channels, widened to FP32.  With
// VEC >= 4 the host has verified a contiguous [D,W] filter and a contiguous
// bias, both 16-byte aligned: every load is a vector load, all issued before
// the first conversion.
template <int W, int VEC, int FK>
__device__ __forceinline__ void load_filter(const void *wp, int64_t sd, int64_t sk,
                                            const void *bp, int64_t bs, int64_t c0,
                                            float (&w)[W][VEC], float (&bias)[VEC]) {
    constexpr int kEl = fk_f32(FK) ? 4 : 2;                     // bytes per tap / bias
    constexpr int kBytes = VEC * W * kEl;                       // a lane's filter bytes
    if constexpr (VEC >= 4 && kBytes % 16 == 0) {
        constexpr int kVecs = kBytes / 16;                      // 16-byte loads
        constexpr int kBiasVecs = (VEC * kEl + 15) / 16;
        const u32x4_t *q = reinterpret_cast<const u32x4_t *>(
            static_cast<const char *>(wp) + c0 * W * kEl);
        u32x4_t wv[kVecs];
#pragma unroll
        for (int i = 0; i < kVecs; ++i) wv[i] = q[i];
        Raw<VEC> bv{};
        u32x4_t bf[kBiasVecs];
        if constexpr (FK == kBf16Bias)
            bv = load_raw<VEC>(static_cast<const uint16_t *>(bp) + c0, 1);
        if constexpr (FK == kF32Bias) {
            const u32x4_t *bq =
                reinterpret_cast<const u32x4_t *>(static_cast<const float *>(bp) + c0);
#pragma unroll
            for (int i = 0; i < kBiasVecs; ++i) bf[i] = bq[i];
        }
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int e2 = c * W + k;
                if constexpr (fk_f32(FK)) {
                    w[k][c] = __uint_as_float(wv[e2 / 4][e2 % 4]);
                } else {
                    const uint32_t word = wv[e2 / 8][(e2 % 8) / 2];
                    w[k][c] = (e2 % 2) ? hi_bf16(word) : lo_bf16(word);
                }
            }
        }
        if constexpr (FK == kBf16Bias) {
            unpack<VEC>(bv, bias);
        } else if constexpr (FK == kF32Bias) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) bias[c] = __uint_as_float(bf[c / 4][c % 4]);
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) bias[c] = 0.0f;
        }
    } else {
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int64_t off = (c0 + c) * sd + k * sk;
                w[k][c] = fk_f32(FK) ? static_cast<const float *>(wp)[off]
                                     : bf16_bits_to_f32(static_cast<const uint16_t *>(wp)[off]);
            }
            if constexpr (FK == kBf16Bias)
                bias[c] = bf16_bits_to_f32(static_cast<const uint16_t *>(bp)[(c0 + c) * bs]);
            else if constexpr (FK == kF32Bias)
                bias[c] = static_cast<const float *>(bp)[(c0 + c) * bs];
            else
                bias[c] = 0.0f;
        }
    }
}

// z = bias + sum_k w[k] * v[k] with v = (win[0..W-2], cur), FP32 fused.
template <int W, int VEC>
__device__ __forceinline__ float preact(const float (&w)[W][VEC], const float (&bias)[VEC],
                                        const float (&win)[W - 1][VEC], const float (&cur)[VEC],
                                        int c) {
    float z = bias[c];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) z = fmaf(w[k][c], win[k][c], z);
    return fmaf(w[W - 1][c], cur[c], z);
}

template <int W, int VEC>
__device__ __forceinline__ void shift_in(float (&win)[W - 1][VEC], const float (&cur)[VEC]) {
#pragma unroll
    for (int k = 0; k < W - 2; ++k)
#pragma unroll
        for (int c = 0; c < VEC; ++c) win[k][c] = win[k + 1][c];
#pragma unroll
    for (int c = 0; c < VEC; ++c) win[W - 2][c] = cur[c];
}

// Left halo of a piece that starts at position ta of the row [s, e) whose
// state row is r: x_ext[ta-(W-1) .. ta-1] from the input where inside the
// row, else from the initial state (slot p - s + W - 1), else zeros.  The
// input loads use addresses clamped into the row, so they can be issued
// early and together (issue_left_halo); finish_left_halo then replaces the
// values that lie before the row.
template <int W, int VEC>
__device__ __forceinline__ void issue_left_halo(const uint16_t *xb, int64_t xs_d, int64_t xs_t,
                                                int64_t s, int64_t ta, Raw<VEC> (&raw)[W - 1]) {
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int64_t p = ta - (W - 1) + j;
        raw[j] = load_raw<VEC>(xb + (p >= s ? p : s) * xs_t, xs_d);
    }
}

template <int W, int VEC>
__device__ __forceinline__ void finish_left_halo(const Raw<VEC> (&raw)[W - 1],
                                                 const Strided3 &init, int64_t r, int64_t s,
                                                 int64_t ta, int64_t c0,
                                                 float (&win)[W - 1][VEC]) {
#pragma unroll
    for (int j = 0; j < W - 1; ++j) unpack<VEC>(raw[j], win[j]);
    if (ta - (W - 1) < s) {
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int64_t p = ta - (W - 1) + j;
            if (p >= s) continue;
            if (init.ptr) {
                const uint16_t *ip = static_cast<const uint16_t *>(init.ptr) + r * init.s0 +
                                     c0 * init.s1 + (p - s + W - 1) * init.s2;
#pragma unroll
                for (int c = 0; c < VEC; ++c) win[j][c] = bf16_bits_to_f32(ip[c * init.s1]);
            } else {
#pragma unroll
                for (int c = 0; c < VEC; ++c) win[j][c] = 0.0f;
            }
        }
    }
}

// cu_seqlens staged in LDS and validated there (the whole array, by every
// block, so no block depends on another).  Returns the violation bits of
// this call ORed with the sticky flag word; block 0 publishes its bits.
// s_bad[0] collects this call's bits, s_bad[1] receives the flag word, read
// by one thread of the block: the word is one address that every block of
// a launch reads at agent scope (past the XCDs' own L2s), so a read per wave
// would queue a launch's waves on one memory channel.
__device__ __forceinline__ uint32_t stage_and_validate(const int32_t *cu, int64_t n_seq,
                                                       int64_t total, uint32_t *err,
                                                       int32_t *s_cu, uint32_t (&s_bad)[2],
                                                       int in_lds, bool publish) {
    const int tid = threadIdx.x;
    if (tid == 0) s_bad[0] = 0u;
    if (in_lds) {
        for (int64_t i = tid; i <= n_seq; i += blockDim.x) s_cu[i] = cu[i];
    }
    __syncthreads();
    uint32_t bad = 0u;
    if (in_lds) {
        for (int64_t i = tid; i < n_seq; i += blockDim.x) {
            const int32_t a = s_cu[i], b = s_cu[i + 1];
            if (b < a) bad |= kDecreasing;
            if (b == a) bad |= kEmpty;
        }
        if (tid == 0) {
            if (s_cu[0] != 0) bad |= kFirstNonzero;
            if (static_cast<int64_t>(s_cu[n_seq]) != total) bad |= kLastMismatch;
        }
        if (bad) atomicOr(&s_bad[0], bad);
    }
    // The word may hold bits of an earlier call (sticky) or, when the
    // offsets did not fit in LDS, of the validation kernel run just before.
    if (tid == 0) s_bad[1] = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    bad = s_bad[0];
    if (publish && tid == 0 && bad) atomicOr(err, bad);
    return bad | s_bad[1];
}

// Largest i in [0, n) with cu[i] <= t, for offsets already validated
// (strictly increasing from 0 to the total, so cu[0] <= t < cu[n]).
__device__ __forceinline__ int64_t find_row(const int32_t *cu, int64_t n, int64_t t) {
    int64_t lo = 0, hi = n;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (static_cast<int64_t>(cu[mid]) <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// ===========================================================================
// Forward
// ===========================================================================
template <int W, int VEC, bool SILU, bool NTL, bool PIPE, int U>
__device__ __forceinline__ void fwd_piece(const FwdArgs &a, int64_t b, int64_t r, int64_t s,
                                          int64_t e, int64_t ta, int64_t tb, int64_t c0,
                                          const float (&w)[W][VEC], const float (&bias)[VEC]) {
    const uint16_t *xb = static_cast<const uint16_t *>(a.x.ptr) + b * a.x.s0 + c0 * a.x.s1;
    uint16_t *yb = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.y.ptr)) + b * a.y.s0 +
                   c0 * a.y.s1;
    const int64_t xs_t = a.x.s2, ys_t = a.y.s2, xs_d = a.x.s1, ys_d = a.y.s1;
    float win[W - 1][VEC];

    auto run_batch = [&](int64_t t, const Raw<VEC> (&raw)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float cur[VEC], out[VEC];
            unpack<VEC>(raw[u], cur);
#pragma unroll
            for (int c = 0; c < VEC; ++c) out[c] = act<SILU>(preact<W, VEC>(w, bias, win, cur, c));
            store_vec<VEC, true>(yb + (t + u) * ys_t, ys_d, out);
            shift_in<W, VEC>(win, cur);
        }
    };

    // The halo loads go out together with the first batch's.
    Raw<VEC> halo[W - 1];
    issue_left_halo<W, VEC>(xb, xs_d, xs_t, s, ta, halo);
    int64_t t = ta;
    if (t + U <= tb) {
        Raw<VEC> raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = load_raw<VEC, NTL>(xb + (t + u) * xs_t, xs_d);
        finish_left_halo<W, VEC>(halo, a.init, r, s, ta, c0, win);
        run_batch(t, raw);
        t += U;
    } else {
        finish_left_halo<W, VEC>(halo, a.init, r, s, ta, c0, win);
    }
    if constexpr (PIPE) {
        // Software pipeline: the next batch's loads are in flight while the
        // current batch computes.
        if (t + U <= tb) {
            Raw<VEC> cur_raw[U];
#pragma unroll
            for (int u = 0; u < U; ++u) cur_raw[u] = load_raw<VEC, NTL>(xb + (t + u) * xs_t, xs_d);
            for (; t + 2 * U <= tb; t += U) {
                Raw<VEC> nxt[U];
#pragma unroll
                for (int u = 0; u < U; ++u) nxt[u] = load_raw<VEC, NTL>(xb + (t + U + u) * xs_t, xs_d);
                run_batch(t, cur_raw);
#pragma unroll
                for (int u = 0; u < U; ++u) cur_raw[u] = nxt[u];
            }
            run_batch(t, cur_raw);
            t += U;
        }
    } else {
        for (; t + U <= tb; t += U) {
            Raw<VEC> raw[U];
#pragma unroll
            for (int u = 0; u < U; ++u) raw[u] = load_raw<VEC, NTL>(xb + (t + u) * xs_t, xs_d);
            run_batch(t, raw);
        }
    }
    for (; t < tb; ++t) {
        float cur[VEC], out[VEC];
        unpack<VEC>(load_raw<VEC, NTL>(xb + t * xs_t, xs_d), cur);
#pragma unroll
        for (int c = 0; c < VEC; ++c) out[c] = act<SILU>(preact<W, VEC>(w, bias, win, cur, c));
        store_vec<VEC, true>(yb + t * ys_t, ys_d, out);
        shift_in<W, VEC>(win, cur);
    }
    // The row ends inside this piece: its last W-1 extended tokens are the
    // window (cuDNN FE "Causal Conv1d": returned final_states).
    if (tb == e && a.fin.ptr) {
        uint16_t *fp = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.fin.ptr)) +
                       r * a.fin.s0 + c0 * a.fin.s1;
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
#pragma unroll
            for (int c = 0; c < VEC; ++c)
                fp[c * a.fin.s1 + j * a.fin.s2] = to_bf16_bits(win[j][c]);
    }
}

// ---------------------------------------------------------------------------
// seq_idx rows (per-token sequence ids; no states).  Tap k of output t sees
// x[t-(W-1)+k] only when that token carries t's id, so the window keeps the
// ids of its W-1 tokens next to their values.  An id is the same for every
// lane of a wave (one token of one row), so its load is a single broadcast.
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ void shift_id(int32_t (&idw)[W - 1], int32_t id) {
#pragma unroll
    for (int k = 0; k < W - 2; ++k) idw[k] = idw[k + 1];
    idw[W - 2] = id;
}

// Ids of the W-1 positions before ta (0 before the row start, where the
// values are zeros and the id is never used).
template <int W>
__device__ __forceinline__ void load_id_halo(const int32_t *sq, int64_t st, int64_t ta,
                                             int32_t (&idw)[W - 1]) {
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int64_t p = ta - (W - 1) + j;
        idw[j] = p >= 0 ? sq[p * st] : 0;
    }
}

// z with the taps of other sequences masked: the same FP32 chain as preact
// with a zero in place of a masked value.
template <int W, int VEC>
__device__ __forceinline__ float preact_seq(const float (&w)[W][VEC], const float (&bias)[VEC],
                                            const float (&win)[W - 1][VEC],
                                            const int32_t (&idw)[W - 1], int32_t id,
                                            const float (&cur)[VEC], int c) {
    float z = bias[c];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) z = fmaf(w[k][c], idw[k] == id ? win[k][c] : 0.0f, z);
    return fmaf(w[W - 1][c], cur[c], z);
}

template <int W, int VEC, bool SILU, bool NTL, int U>
__device__ __forceinline__ void fwd_seq_piece(const FwdArgs &a, int64_t b, int64_t ta,
                                              int64_t tb, int64_t c0, const float (&w)[W][VEC],
                                              const float (&bias)[VEC]) {
    const uint16_t *xb = static_cast<const uint16_t *>(a.x.ptr) + b * a.x.s0 + c0 * a.x.s1;
    uint16_t *yb = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.y.ptr)) + b * a.y.s0 +
                   c0 * a.y.s1;
    const int32_t *sq = a.seq + b * a.seq_sb;
    const int64_t xs_t = a.x.s2, ys_t = a.y.s2, xs_d = a.x.s1, ys_d = a.y.s1, st = a.seq_st;
    float win[W - 1][VEC];
    int32_t idw[W - 1];
    {
        Raw<VEC> halo[W - 1];
        issue_left_halo<W, VEC>(xb, xs_d, xs_t, 0, ta, halo);
        load_id_halo<W>(sq, st, ta, idw);
        finish_left_halo<W, VEC>(halo, a.init, b, 0, ta, c0, win);  // no state: zeros
    }
    auto step = [&](int64_t t, const Raw<VEC> &raw, int32_t id) {
        float cur[VEC], out[VEC];
        unpack<VEC>(raw, cur);
#pragma unroll
        for (int c = 0; c < VEC; ++c)
            out[c] = act<SILU>(preact_seq<W, VEC>(w, bias, win, idw, id, cur, c));
        store_vec<VEC, true>(yb + t * ys_t, ys_d, out);
        shift_in<W, VEC>(win, cur);
        shift_id<W>(idw, id);
    };
    int64_t t = ta;
    for (; t + U <= tb; t += U) {
        Raw<VEC> raw[U];
        int32_t ids[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            raw[u] = load_raw<VEC, NTL>(xb + (t + u) * xs_t, xs_d);
            ids[u] = sq[(t + u) * st];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) step(t + u, raw[u], ids[u]);
    }
    for (; t < tb; ++t) step(t, load_raw<VEC, NTL>(xb + t * xs_t, xs_d), sq[t * st]);
}

template <int W, int VEC, bool SILU, int ROWS, int FK, bool PIPE>
__global__ __launch_bounds__(256) CCV_FWD_ATTR void k_fwd_chan(FwdArgs a) {
    constexpr bool PACKED = ROWS == kRowsPacked;
    __shared__ int32_t s_cu[PACKED ? kLdsCuMax : 1];
    __shared__ uint32_t s_bad[2];
    const TileSpan ts = split_tile<CCV_TILE_ORDER>(a, a.n_gblk, kFwdWavesT);
    const int64_t b = ts.b, gb = ts.c;
    // The wave index is uniform over the wave; readfirstlane tells the
    // compiler so, which keeps the time bounds and row offsets in scalars.
    // Measured: it frees the registers the seq_idx walk needs, but slows
    // the dense and packed streams on large inputs, so only seq_idx uses it.
    const int wave = (((CCV_FWD_UNIFORM_ROWS >> ROWS) & 1) && CCV_WAVE_UNIFORM)
                         ? __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize)
                         : static_cast<int>(threadIdx.x / kWaveSize);
    const int lane = threadIdx.x % kWaveSize;

    if constexpr (PACKED) {
        if (stage_and_validate(a.cu, a.n_seq, a.T, a.err, s_cu, s_bad, a.cu_in_lds,
                               blockIdx.x == 0))
            return;  // malformed or sticky: write nothing
    }
    const int64_t g = gb * kFwdWavesC + wave / kFwdWavesT;
    const int64_t t0 = ts.t0 + (wave % kFwdWavesT) * ts.L;
    const int64_t c0 = g * (kWaveSize * VEC) + lane * VEC;
    if (t0 >= ts.end || c0 >= a.D) return;
    const int64_t t1 = min(t0 + ts.L, ts.end);

    float w[W][VEC], bias[VEC];
    load_filter<W, VEC, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, c0, w, bias);

    // Non-temporal loads only when the operands exceed what caches can keep.
    auto run = [&](auto ntl) {
        constexpr bool NTL = decltype(ntl)::value;
        if constexpr (ROWS == kRowsSeq) {
            constexpr int U = VEC == 4 ? CCV_FWD_SMALL_UNROLL : CCV_FWD_UNROLL;
            fwd_seq_piece<W, VEC, SILU, NTL, U>(a, b, t0, t1, c0, w, bias);
        } else if constexpr (!PACKED) {
            constexpr int U = PIPE ? CCV_FWD_PIPE_UNROLL_DENSE
                              : VEC == 4 ? CCV_FWD_SMALL_UNROLL : CCV_FWD_UNROLL;
            fwd_piece<W, VEC, SILU, NTL, PIPE, U>(a, b, b, 0, a.T, t0, t1, c0, w, bias);
        } else {
            const int32_t *cu = a.cu_in_lds ? s_cu : a.cu;
            for (int64_t i = find_row(cu, a.n_seq, t0); i < a.n_seq; ++i) {
                const int64_t s = cu[i], e = cu[i + 1];
                if (s >= t1) break;
                fwd_piece<W, VEC, SILU, NTL, PIPE, PIPE ? CCV_FWD_PIPE_UNROLL : CCV_FWD_UNROLL>(
                    a, 0, i, s, e, s > t0 ? s : t0, e < t1 ? e : t1, c0, w, bias);
            }
        }
    };
    if (a.nt_load) run(std::true_type{});
    else run(std::false_type{});
}

// ===========================================================================
// Backward
//
// g[t] = dy[t] * act'(z[t]);  dx_ext[p] = sum_k w[k] * g[p + W-1 - k] over the
// row, plus dfinal[j] at p = e-(W-1)+j;  dx[p] = dx_ext[p] (p in the row),
// dinit[j] = dx_ext[s-(W-1)+j];  dW[k] += g[t] x_ext[t-(W-1)+k], dB += g[t].
//
// A piece [ta, tb) of row [s, e) walks tau over [ta, tb + W-1): step tau
// computes g[tau] (zero past the row end; past tb it is a right halo) and
// emits dx_ext[tau-(W-1)] from the W-1 previous g's held in registers.
// Emission before ta happens only when the piece starts the row (dinit).
// ===========================================================================
template <int W, int VEC, bool SILU, bool BIAS>
struct BwdLane {
    float w[W][VEC], bias[VEC];
    float dw[W][VEC], db[VEC];
};

template <int W, int VEC, bool SILU, bool BIAS, bool NTL, int U>
__device__ __forceinline__ void bwd_piece(const BwdArgs &a, BwdLane<W, VEC, SILU, BIAS> &L,
                                          int64_t b, int64_t r, int64_t s, int64_t e,
                                          int64_t ta, int64_t tb, int64_t c0) {
    const uint16_t *xb = static_cast<const uint16_t *>(a.x.ptr) + b * a.x.s0 + c0 * a.x.s1;
    const uint16_t *dyb = static_cast<const uint16_t *>(a.dy.ptr) + b * a.dy.s0 + c0 * a.dy.s1;
    uint16_t *dxb = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dx.ptr)) +
                    b * a.dx.s0 + c0 * a.dx.s1;
    const int64_t xs_d = a.x.s1, xs_t = a.x.s2, ys_d = a.dy.s1, ys_t = a.dy.s2;
    const int64_t ds_d = a.dx.s1, ds_t = a.dx.s2;

    float xw[W - 1][VEC], gw[W - 1][VEC];
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
#pragma unroll
        for (int c = 0; c < VEC; ++c) gw[j][c] = 0.0f;

    // dx_ext[p] from g[p .. p+W-1] = (gw[0..W-2], gcur).
    auto emit_value = [&](const float (&gcur)[VEC], float (&v)[VEC]) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            float acc = L.w[0][c] * gcur[c];
#pragma unroll
            for (int j = W - 2; j >= 0; --j) acc = fmaf(L.w[W - 1 - j][c], gw[j][c], acc);
            v[c] = acc;
        }
    };
    auto shift_g = [&](const float (&gcur)[VEC]) {
#pragma unroll
        for (int k = 0; k < W - 2; ++k)
#pragma unroll
            for (int c = 0; c < VEC; ++c) gw[k][c] = gw[k + 1][c];
#pragma unroll
        for (int c = 0; c < VEC; ++c) gw[W - 2][c] = gcur[c];
    };
    // g at tau from (xw, cur, dy); accumulates dW/dB when `count`.
    // SiLU'(z) = s + z s (1 - s), with s (1 - s) formed as s - s^2.
    auto grad_step = [&](const float (&cur)[VEC], const float (&dyv)[VEC], float (&gcur)[VEC],
                         bool count) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            const float z = preact<W, VEC>(L.w, L.bias, xw, cur, c);
            gcur[c] = dyv[c] * act_slope<SILU>(z);
        }
        if (count) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
#pragma unroll
                for (int k = 0; k < W - 1; ++k) L.dw[k][c] = fmaf(gcur[c], xw[k][c], L.dw[k][c]);
                L.dw[W - 1][c] = fmaf(gcur[c], cur[c], L.dw[W - 1][c]);
                if constexpr (BIAS) L.db[c] += gcur[c];
            }
        }
    };
    // Fully checked step (head and tail of a piece) on preloaded tokens.
    auto generic_step = [&](int64_t tau, const Raw<VEC> &rxv, const Raw<VEC> &rdv) {
        float gcur[VEC];
        if (tau < e) {
            float cur[VEC], dyv[VEC];
            unpack<VEC>(rxv, cur);
            unpack<VEC>(rdv, dyv);
            grad_step(cur, dyv, gcur, tau < tb);
            shift_in<W, VEC>(xw, cur);
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) gcur[c] = 0.0f;
        }
        const int64_t p = tau - (W - 1);
        const bool to_dx = p >= ta;
        const bool to_dinit = !to_dx && ta == s && a.dinit.ptr != nullptr;
        if (to_dx || to_dinit) {
            float v[VEC];
            emit_value(gcur, v);
            if (a.dfin.ptr && p >= e - (W - 1)) {
                const uint16_t *fp = static_cast<const uint16_t *>(a.dfin.ptr) + r * a.dfin.s0 +
                                     c0 * a.dfin.s1 + (p - (e - (W - 1))) * a.dfin.s2;
#pragma unroll
                for (int c = 0; c < VEC; ++c) v[c] += bf16_bits_to_f32(fp[c * a.dfin.s1]);
            }
            if (to_dx) {
                store_vec<VEC>(dxb + p * ds_t, ds_d, v);
            } else {
                uint16_t *ip = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dinit.ptr)) +
                               r * a.dinit.s0 + c0 * a.dinit.s1 + (p - s + W - 1) * a.dinit.s2;
#pragma unroll
                for (int c = 0; c < VEC; ++c) ip[c * a.dinit.s1] = to_bf16_bits(v[c]);
            }
        }
        shift_g(gcur);
    };
    // x and dy of the W-1 steps from tau0, addresses clamped into the row so
    // that the loads can be issued together (values past the row are unused).
    auto load_steps = [&](int64_t tau0, Raw<VEC> (&rx)[W - 1], Raw<VEC> (&rd)[W - 1]) {
#pragma unroll
        for (int h = 0; h < W - 1; ++h) {
            const int64_t tc = tau0 + h < e ? tau0 + h : e - 1;
            rx[h] = load_raw<VEC>(xb + tc * xs_t, xs_d);
            rd[h] = load_raw<VEC>(dyb + tc * ys_t, ys_d);
        }
    };
    // Body step: inside the row, emits dx[tau-(W-1)] with no final-state
    // term (tau - (W-1) < e - (W-1)).
    auto body_batch = [&](int64_t tau, const Raw<VEC> (&rx)[U], const Raw<VEC> (&rd)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float cur[VEC], dyv[VEC], gcur[VEC], v[VEC];
            unpack<VEC>(rx[u], cur);
            unpack<VEC>(rd[u], dyv);
            grad_step(cur, dyv, gcur, true);
            shift_in<W, VEC>(xw, cur);
            emit_value(gcur, v);
            store_vec<VEC, true>(dxb + (tau + u - (W - 1)) * ds_t, ds_d, v);
            shift_g(gcur);
        }
    };
    auto load_batch = [&](int64_t tau, Raw<VEC> (&rx)[U], Raw<VEC> (&rd)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            rx[u] = load_raw<VEC, NTL>(xb + (tau + u) * xs_t, xs_d);
            rd[u] = load_raw<VEC, NTL>(dyb + (tau + u) * ys_t, ys_d);
        }
    };

    // Prologue: the left halo, the head (tau in [ta, ta + W-1)) and the first
    // body batch are all requested before anything waits.
    Raw<VEC> halo[W - 1], hx[W - 1], hd[W - 1];
    issue_left_halo<W, VEC>(xb, xs_d, xs_t, s, ta, halo);
    load_steps(ta, hx, hd);
    int64_t tau = ta + (W - 1);
    if (tau + U <= tb) {
        Raw<VEC> rx[U], rd[U];
        load_batch(tau, rx, rd);
        finish_left_halo<W, VEC>(halo, a.init, r, s, ta, c0, xw);
        if (CCV_BWD_FAST_EDGES && ta > s) {
            // Interior head (this branch has tb >= ta + W-1 + U): every head
            // token is in the row and counted, and its dx belongs to the
            // chunk before, so nothing is emitted.
#pragma unroll
            for (int h = 0; h < W - 1; ++h) {
                float cur[VEC], dyv[VEC], gcur[VEC];
                unpack<VEC>(hx[h], cur);
                unpack<VEC>(hd[h], dyv);
                grad_step(cur, dyv, gcur, true);
                shift_in<W, VEC>(xw, cur);
                shift_g(gcur);
            }
        } else {
#pragma unroll
            for (int h = 0; h < W - 1; ++h) generic_step(ta + h, hx[h], hd[h]);
        }
        body_batch(tau, rx, rd);
        tau += U;
    } else {
        finish_left_halo<W, VEC>(halo, a.init, r, s, ta, c0, xw);
#pragma unroll
        for (int h = 0; h < W - 1; ++h) generic_step(ta + h, hx[h], hd[h]);
    }
    if constexpr (CCV_BWD_PIPE) {
        // Software pipeline: the next batch's loads are in flight while the
        // current batch computes.
        if (tau + U <= tb) {
            Raw<VEC> rx[U], rd[U];
            load_batch(tau, rx, rd);
            for (; tau + 2 * U <= tb; tau += U) {
                Raw<VEC> nx[U], nd[U];
                load_batch(tau + U, nx, nd);
                body_batch(tau, rx, rd);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    rx[u] = nx[u];
                    rd[u] = nd[u];
                }
            }
            body_batch(tau, rx, rd);
            tau += U;
        }
    } else {
        for (; tau + U <= tb; tau += U) {
            Raw<VEC> rx[U], rd[U];
            load_batch(tau, rx, rd);
            body_batch(tau, rx, rd);
        }
    }
    for (; tau < tb; ++tau) {
        float cur[VEC], dyv[VEC], gcur[VEC], v[VEC];
        unpack<VEC>(load_raw<VEC, NTL>(xb + tau * xs_t, xs_d), cur);
        unpack<VEC>(load_raw<VEC, NTL>(dyb + tau * ys_t, ys_d), dyv);
        grad_step(cur, dyv, gcur, true);
        shift_in<W, VEC>(xw, cur);
        emit_value(gcur, v);
        store_vec<VEC, true>(dxb + (tau - (W - 1)) * ds_t, ds_d, v);
        shift_g(gcur);
    }
    // Tail: tau in [max(tb, ta + W-1), tb + W-1): at most W-1 steps.
    {
        const int64_t tt = tb > ta + (W - 1) ? tb : ta + (W - 1);
        Raw<VEC> rx[W - 1], rd[W - 1];
        load_steps(tt, rx, rd);
        if (CCV_BWD_FAST_EDGES && tb >= ta + (W - 1) && tb + (W - 1) <= e) {
            // Interior tail: the W-1 right-halo tokens are in the row and not
            // counted, and the dx they complete (p < tb) carry no
            // final-state term (p < e - (W-1)).
#pragma unroll
            for (int h = 0; h < W - 1; ++h) {
                float cur[VEC], dyv[VEC], gcur[VEC], v[VEC];
                unpack<VEC>(rx[h], cur);
                unpack<VEC>(rd[h], dyv);
                grad_step(cur, dyv, gcur, false);
                shift_in<W, VEC>(xw, cur);
                emit_value(gcur, v);
                store_vec<VEC, true>(dxb + (tb + h - (W - 1)) * ds_t, ds_d, v);
                shift_g(gcur);
            }
        } else {
#pragma unroll
            for (int h = 0; h < W - 1; ++h)
                if (tt + h < tb + (W - 1)) generic_step(tt + h, rx[h], rd[h]);
        }
    }
}

// seq_idx rows: the walk of bwd_piece (tau over [ta, tb + W-1), g[tau] in
// registers, dx[tau-(W-1)] emitted) with the ids of the window's tokens kept
// beside their values.  x[p] reaches output t only when id[p] == id[t], in
// the forward (z), in dW, and in dx[p] = sum_k w[k] g[p+W-1-k] [same id].
template <int W, int VEC, bool SILU, bool BIAS, bool NTL, int U>
__device__ __forceinline__ void bwd_seq_piece(const BwdArgs &a, BwdLane<W, VEC, SILU, BIAS> &L,
                                              int64_t b, int64_t ta, int64_t tb, int64_t c0) {
    const uint16_t *xb = static_cast<const uint16_t *>(a.x.ptr) + b * a.x.s0 + c0 * a.x.s1;
    const uint16_t *dyb = static_cast<const uint16_t *>(a.dy.ptr) + b * a.dy.s0 + c0 * a.dy.s1;
    uint16_t *dxb = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dx.ptr)) +
                    b * a.dx.s0 + c0 * a.dx.s1;
    const int32_t *sq = a.seq + b * a.seq_sb;
    const int64_t xs_d = a.x.s1, xs_t = a.x.s2, ys_d = a.dy.s1, ys_t = a.dy.s2;
    const int64_t ds_d = a.dx.s1, ds_t = a.dx.s2, st = a.seq_st;

    float xw[W - 1][VEC], gw[W - 1][VEC];
    int32_t idw[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
#pragma unroll
        for (int c = 0; c < VEC; ++c) gw[j][c] = 0.0f;
    {
        Raw<VEC> halo[W - 1];
        issue_left_halo<W, VEC>(xb, xs_d, xs_t, 0, ta, halo);
        load_id_halo<W>(sq, st, ta, idw);
        finish_left_halo<W, VEC>(halo, a.init, b, 0, ta, c0, xw);  // no state: zeros
    }
    // One step at tau: g[tau] (zero past the row end), dW/dB when `count`,
    // dx[tau-(W-1)] when `emit`.
    auto step = [&](int64_t tau, const Raw<VEC> &rxv, const Raw<VEC> &rdv, int32_t id,
                    bool in_row, bool count, bool emit, bool stream) {
        float cur[VEC], gcur[VEC];
        if (in_row) {
            float dyv[VEC];
            unpack<VEC>(rxv, cur);
            unpack<VEC>(rdv, dyv);
#pragma unroll
            for (int c = 0; c < VEC; ++c)
                gcur[c] = dyv[c] * act_slope<SILU>(preact_seq<W, VEC>(L.w, L.bias, xw, idw, id,
                                                                      cur, c));
            if (count) {
#pragma unroll
                for (int c = 0; c < VEC; ++c) {
#pragma unroll
                    for (int k = 0; k < W - 1; ++k)
                        L.dw[k][c] = fmaf(gcur[c], idw[k] == id ? xw[k][c] : 0.0f, L.dw[k][c]);
                    L.dw[W - 1][c] = fmaf(gcur[c], cur[c], L.dw[W - 1][c]);
                    if constexpr (BIAS) L.db[c] += gcur[c];
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) cur[c] = gcur[c] = 0.0f;
        }
        if (emit) {
            // dx at p = tau-(W-1): its id is the window's oldest, idw[0].
            const int32_t idp = idw[0];
            float v[VEC];
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                float acc = L.w[0][c] * (id == idp ? gcur[c] : 0.0f);
#pragma unroll
                for (int j = W - 2; j >= 0; --j)
                    acc = fmaf(L.w[W - 1 - j][c], idw[j] == idp ? gw[j][c] : 0.0f, acc);
                v[c] = acc;
            }
            if (stream) store_vec<VEC, true>(dxb + (tau - (W - 1)) * ds_t, ds_d, v);
            else store_vec<VEC>(dxb + (tau - (W - 1)) * ds_t, ds_d, v);
        }
        shift_in<W, VEC>(xw, cur);
        shift_id<W>(idw, id);
#pragma unroll
        for (int k = 0; k < W - 2; ++k)
#pragma unroll
            for (int c = 0; c < VEC; ++c) gw[k][c] = gw[k + 1][c];
#pragma unroll
        for (int c = 0; c < VEC; ++c) gw[W - 2][c] = gcur[c];
    };
    // Fully checked step: head (no emission yet), right halo past tb.
    auto generic = [&](int64_t tau) {
        const bool in_row = tau < a.T;
        Raw<VEC> rx{}, rd{};
        int32_t id = 0;
        if (in_row) {
            rx = load_raw<VEC>(xb + tau * xs_t, xs_d);
            rd = load_raw<VEC>(dyb + tau * ys_t, ys_d);
            id = sq[tau * st];
        }
        step(tau, rx, rd, id, in_row, tau < tb, tau - (W - 1) >= ta, false);
    };
    const int64_t end = tb + (W - 1);
    const int64_t head_end = ta + (W - 1) < end ? ta + (W - 1) : end;
    int64_t tau = ta;
    for (; tau < head_end; ++tau) generic(tau);
    auto load_seq_batch = [&](int64_t t, Raw<VEC> (&rx)[U], Raw<VEC> (&rd)[U],
                              int32_t (&ids)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            rx[u] = load_raw<VEC, NTL>(xb + (t + u) * xs_t, xs_d);
            rd[u] = load_raw<VEC, NTL>(dyb + (t + u) * ys_t, ys_d);
            ids[u] = sq[(t + u) * st];
        }
    };
    if constexpr (CCV_BWD_SEQ_PIPE) {
        // The next batch's loads are in flight while the current one computes.
        if (tau + U <= tb) {
            Raw<VEC> rx[U], rd[U];
            int32_t ids[U];
            load_seq_batch(tau, rx, rd, ids);
            for (; tau + 2 * U <= tb; tau += U) {
                Raw<VEC> nx[U], nd[U];
                int32_t nids[U];
                load_seq_batch(tau + U, nx, nd, nids);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    step(tau + u, rx[u], rd[u], ids[u], true, true, true, true);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    rx[u] = nx[u];
                    rd[u] = nd[u];
                    ids[u] = nids[u];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) step(tau + u, rx[u], rd[u], ids[u], true, true, true, true);
            tau += U;
        }
    } else {
        for (; tau + U <= tb; tau += U) {
            Raw<VEC> rx[U], rd[U];
            int32_t ids[U];
            load_seq_batch(tau, rx, rd, ids);
#pragma unroll
            for (int u = 0; u < U; ++u)
                step(tau + u, rx[u], rd[u], ids[u], true, true, true, true);
        }
    }
    for (; tau < end; ++tau) generic(tau);
}

template <int W, int VEC, bool SILU, int ROWS, int FK>
__global__ __launch_bounds__(256) CCV_BWD_ATTR void k_bwd_chan(BwdArgs a) {
    constexpr bool PACKED = ROWS == kRowsPacked;
    constexpr bool BIAS = fk_bias(FK);
    constexpr int CH = kWaveSize * VEC;  // channels of a block
    // One LDS buffer: the staged offsets during the walk, then the dW/dB
    // reduction (a barrier separates the two uses).
    constexpr int kRed = kWavesPerBlock * (W + 1) * (CH + 1);
    constexpr int kBuf = (PACKED && kLdsCuMax > kRed) ? kLdsCuMax : kRed;
    __shared__ float s_buf[kBuf];
    __shared__ uint32_t s_bad[2];
    int32_t *s_cu = reinterpret_cast<int32_t *>(s_buf);
    float (*s_red)[W + 1][CH + 1] = reinterpret_cast<float (*)[W + 1][CH + 1]>(s_buf);
    // Packed rows measured faster with time blocks innermost, the others
    // with channel blocks innermost.
    const TileSpan ts = split_tile<PACKED ? CCV_BWD_PACKED_TILE_ORDER : CCV_TILE_ORDER>(
        a, a.n_group, kWavesPerBlock);
    const int64_t b = ts.b, g = ts.c, bt = ts.bt;
    // The wave index is uniform over the wave; readfirstlane tells the
    // compiler so, which keeps the time bounds and row offsets in scalars.
    // Measured: it frees the registers the seq_idx walk needs, but slows
    // the dense and packed streams on large inputs, so only seq_idx uses it.
    const int wave = (((CCV_BWD_UNIFORM_ROWS >> ROWS) & 1) && CCV_WAVE_UNIFORM)
                         ? __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize)
                         : static_cast<int>(threadIdx.x / kWaveSize);
    const int lane = threadIdx.x % kWaveSize;

    if constexpr (PACKED) {
        if (stage_and_validate(a.cu, a.n_seq, a.T, a.err, s_cu, s_bad, a.cu_in_lds,
                               blockIdx.x == 0))
            return;  // uniform over the block: no barrier is left waiting
    }
    const int64_t t0 = ts.t0 + wave * ts.L;
    const int64_t c0 = g * CH + lane * VEC;

    BwdLane<W, VEC, SILU, BIAS> L;
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
#pragma unroll
        for (int k = 0; k < W; ++k) L.dw[k][c] = 0.0f;
        L.db[c] = 0.0f;
    }
    if (t0 < ts.end && c0 < a.D) {
        const int64_t t1 = min(t0 + ts.L, ts.end);
        load_filter<W, VEC, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, c0, L.w, L.bias);
        auto run = [&](auto ntl) {
            constexpr bool NTL = decltype(ntl)::value;
            if constexpr (ROWS == kRowsSeq) {
                bwd_seq_piece<W, VEC, SILU, BIAS, NTL, CCV_BWD_UNROLL_SEQ>(a, L, b, t0, t1, c0);
            } else if constexpr (!PACKED) {
                bwd_piece<W, VEC, SILU, BIAS, NTL, CCV_BWD_UNROLL>(a, L, b, b, 0, a.T, t0, t1, c0);
            } else {
                const int32_t *cu = a.cu_in_lds ? s_cu : a.cu;
                for (int64_t i = find_row(cu, a.n_seq, t0); i < a.n_seq; ++i) {
                    const int64_t s = cu[i], e = cu[i + 1];
                    if (s >= t1) break;
                    bwd_piece<W, VEC, SILU, BIAS, NTL, CCV_BWD_UNROLL_PACKED>(
                        a, L, 0, i, s, e, s > t0 ? s : t0, e < t1 ? e : t1, c0);
                }
            }
        };
        if (a.nt_load) run(std::true_type{});
        else run(std::false_type{});
    }

    // dW/dB: the block's waves cover the same channels over consecutive
    // chunks; sum them through LDS in wave order, then one atomic (or one
    // unique partial) per (channel, tap) of the block.
    if constexpr (PACKED) __syncthreads();  // every wave is done with s_cu
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
#pragma unroll
        for (int k = 0; k < W; ++k) s_red[wave][k][lane * VEC + c] = L.dw[k][c];
        s_red[wave][W][lane * VEC + c] = L.db[c];
    }
    __syncthreads();
    const int64_t ch0 = g * CH;
    const int64_t pidx = b * (a.n_tblk + a.n_tblk_t) + bt;
    if (a.partial) {
        // One unique partial row per block: [channel][tap] (+ the bias slot
        // when dbias goes through the deterministic route too).
        const int kp = a.part_stride;
        for (int i = threadIdx.x; i < CH * kp; i += blockDim.x) {
            const int ch = i / kp, k = i % kp;
            if (ch0 + ch >= a.D) continue;
            float v = s_red[0][k][ch];
#pragma unroll
            for (int q = 1; q < kWavesPerBlock; ++q) v += s_red[q][k][ch];
            a.partial[(pidx * a.D + ch0 + ch) * kp + k] = v;
        }
        return;
    }
    for (int i = threadIdx.x; i < CH * W; i += blockDim.x) {
        const int ch = i / W, k = i % W;
        if (ch0 + ch >= a.D) continue;
        float v = s_red[0][k][ch];
#pragma unroll
        for (int q = 1; q < kWavesPerBlock; ++q) v += s_red[q][k][ch];
        atomicAdd(a.dw + (ch0 + ch) * W + k, v);
    }
    if constexpr (BIAS) {
        for (int ch = threadIdx.x; ch < CH; ch += blockDim.x) {
            if (ch0 + ch >= a.D) continue;
            float v = s_red[0][W][ch];
#pragma unroll
            for (int q = 1; q < kWavesPerBlock; ++q) v += s_red[q][W][ch];
            atomicAdd(a.db + ch0 + ch, v);
        }
    }
}

// ===========================================================================
// Time-contiguous rows (unit stride along T, e.g. a contiguous [B,D,T]).
//
// Lanes run along time: a lane owns kTcE = 8 consecutive tokens of one
// (b, d) row (one 16-byte vector), a wave one tile of 512 consecutive tokens,
// and a wave walks a chunk of kTcTilesFwd (forward) or kTcTilesBwd tiles in
// order, all of whose loads are issued before the first use.  The W-1 tokens
// before a lane's first token come from the lane before (a cross-lane shift);
// lane 0 takes them from the previous tile's lane 63, or at the chunk start
// from memory (the input, the initial state, or zeros).  The filter taps and
// the bias belong to the row, so they are wave-uniform.
// ===========================================================================
// Cross-lane moves on the VALU (DPP), not through the LDS crossbar.  With
// `bound_ctrl` off, a lane whose source lies outside the wave (or, for the
// row shifts, outside its row of 16 lanes) keeps `edge`.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float edge, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(edge), __float_as_int(v),
                                                      CTRL, 0xf, 0xf, false));
}
constexpr int kDppWaveShr1 = 0x138;  // lane i <- lane i-1
constexpr int kDppWaveShl1 = 0x130;  // lane i <- lane i+1
constexpr int kDppRowShr = 0x110;    // + n: lane i <- lane i-n of the same row
// Lane i gets lane i-1's v; lane 0 gets `first`.
__device__ __forceinline__ float lane_up(float v, float first) {
    return dpp_move<kDppWaveShr1>(first, v);
}
// Lane i gets lane i+1's v; lane 63 gets `last`.
__device__ __forceinline__ float lane_down(float v, float last) {
    return dpp_move<kDppWaveShl1>(last, v);
}
__device__ __forceinline__ float from_lane(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Sum over the wave, in every lane: an inclusive scan within each row of 16
// lanes (shifts of 1, 2, 4, 8), then the four row totals (lanes 15, 31, 47,
// 63) added in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_move<kDppRowShr + 1>(0.0f, v);
    v += dpp_move<kDppRowShr + 2>(0.0f, v);
    v += dpp_move<kDppRowShr + 4>(0.0f, v);
    v += dpp_move<kDppRowShr + 8>(0.0f, v);
    return (from_lane(v, 15) + from_lane(v, 31)) + (from_lane(v, 47) + from_lane(v, 63));
}

// A lane's kTcE tokens from t on a unit-stride row; the tokens at or past
// `end` read as zeros.  `align` is the byte alignment of the row's start
// (tc_align: 16, 4 or 2); t is a multiple of kTcE, so a lane's tokens start
// at that alignment too.  16: one aligned 16-byte
// vector; 4: one 16-byte access at 4-byte alignment (the memory pipeline
// takes dword-aligned vectors); 2: a load of the token before and the
// first 7 (dword-aligned) plus one of the last token, shifted into place by
// two bytes, and a store of the first token, the next six (three dwords)
// and the last.  The lane that starts a row reads its tokens one by one (no
// token before the row is read).
typedef uint32_t u32x4_a4_t __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3_a4_t __attribute__((ext_vector_type(3), aligned(4)));

__device__ __forceinline__ int tc_align(const uint16_t *row) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(row);
    return (a & 15u) == 0 ? 16 : (a & 3u) == 0 ? 4 : 2;
}

template <bool NTL>
__device__ __forceinline__ Raw<8> tc_load(const uint16_t *row, int64_t t, int64_t end,
                                          int align) {
    Raw<8> r;
    if (t + kTcE <= end && align >= 4) {
        if (align >= 16) return load_raw<8, NTL>(row + t, 1);
        const u32x4_a4_t *q = reinterpret_cast<const u32x4_a4_t *>(row + t);
        u32x4_a4_t v;
        if constexpr (NTL && CCV_NT_LOAD) v = __builtin_nontemporal_load(q);
        else v = *q;
        r.v = u32x4_t{v[0], v[1], v[2], v[3]};
        return r;
    }
    if (t + kTcE <= end && t > 0) {
        // 2-byte rows: tokens t-1 .. t+6 from the dword boundary before t
        const u32x4_a4_t *q = reinterpret_cast<const u32x4_a4_t *>(row + t - 1);
        u32x4_a4_t v;
        uint32_t last;
        if constexpr (NTL && CCV_NT_LOAD) {
            v = __builtin_nontemporal_load(q);
            last = __builtin_nontemporal_load(row + t + kTcE - 1);
        } else {
            v = *q;
            last = row[t + kTcE - 1];
        }
        r.v = u32x4_t{__builtin_amdgcn_alignbyte(v[1], v[0], 2),
                      __builtin_amdgcn_alignbyte(v[2], v[1], 2),
                      __builtin_amdgcn_alignbyte(v[3], v[2], 2),
                      __builtin_amdgcn_alignbyte(last, v[3], 2)};
        return r;
    }
    r.v = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kTcE; ++i)
        if (t + i < end) r.v[i / 2] |= static_cast<uint32_t>(row[t + i]) << (16 * (i % 2));
    return r;
}

template <bool STREAM>
__device__ __forceinline__ void tc_store(uint16_t *row, int64_t t, int64_t end,
                                         const float (&v)[kTcE], int align) {
    if (t + kTcE <= end && align >= 4) {
        if (align >= 16) {
            store_vec<8, STREAM>(row + t, 1, v);
            return;
        }
        u32x4_a4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack2_bf16(v[2 * i], v[2 * i + 1]);
        u32x4_a4_t *q = reinterpret_cast<u32x4_a4_t *>(row + t);
        if constexpr (STREAM && CCV_NT_STORE) __builtin_nontemporal_store(w, q);
        else *q = w;
        return;
    }
    if (t + kTcE <= end) {
        // 2-byte rows: token t, tokens t+1 .. t+6 (dword-aligned), token t+7
        const u32x3_a4_t mid = {pack2_bf16(v[1], v[2]), pack2_bf16(v[3], v[4]),
                                pack2_bf16(v[5], v[6])};
        u32x3_a4_t *q = reinterpret_cast<u32x3_a4_t *>(row + t + 1);
        if constexpr (STREAM && CCV_NT_STORE) {
            __builtin_nontemporal_store(to_bf16_bits(v[0]), row + t);
            __builtin_nontemporal_store(mid, q);
            __builtin_nontemporal_store(to_bf16_bits(v[kTcE - 1]), row + t + kTcE - 1);
        } else {
            row[t] = to_bf16_bits(v[0]);
            *q = mid;
            row[t + kTcE - 1] = to_bf16_bits(v[kTcE - 1]);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kTcE; ++i)
        if (t + i < end) row[t + i] = to_bf16_bits(v[i]);
}

// Dwords q .. q+3 of the 8 in c, each moved down by `sh` bytes (0 or 2).
template <int Q>
__device__ __forceinline__ u32x4_t tc_funnel(const uint32_t (&c)[8], uint32_t sh) {
    return u32x4_t{__builtin_amdgcn_alignbyte(c[Q + 1], c[Q], sh),
                   __builtin_amdgcn_alignbyte(c[Q + 2], c[Q + 1], sh),
                   __builtin_amdgcn_alignbyte(c[Q + 3], c[Q + 2], sh),
                   __builtin_amdgcn_alignbyte(c[Q + 4], c[Q + 3], sh)};
}
// Lanes 0..62 take lane l+1's v, lane 63 takes `last`.
__device__ __forceinline__ int32_t tc_lane_down_u32(int32_t v, int32_t last) {
    return __builtin_amdgcn_update_dpp(last, v, kDppWaveShl1, 0xf, 0xf, false);
}

// Time-lane loads of rows that do not start on a 16-byte boundary.  A 16-byte
// access that is only 4- or 2-byte aligned costs the memory pipeline about
// as much again as an aligned one, so such rows are read in aligned blocks:
// with s tokens between the 16-byte boundary at or before a lane's first
// token t and t (s is the same for every lane of a row), the lane loads the
// aligned block of tokens t-s .. t-s+7, takes the next lane's block (lane 63:
// lane 0's block of the next tile, or the chunk's tail block) by a DPP shift,
// and assembles t .. t+7 from the two with a byte shift.  Block tokens
// outside [0, T) read as zero and are never accessed.
template <bool NTL>
__device__ __forceinline__ Raw<8> tc_block(const uint16_t *row, int64_t b0, int64_t T) {
    if (b0 >= 0 && b0 + kTcE <= T) return load_raw<8, NTL>(row + b0, 1);  // 16-byte aligned
    Raw<8> r;
    r.v = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kTcE; ++i)
        if (b0 + i >= 0 && b0 + i < T)
            r.v[i / 2] |= static_cast<uint32_t>(row[b0 + i]) << (16 * (i % 2));
    return r;
}

template <bool NTL, bool A16>
struct TcLoads {
    const uint16_t *row;
    int64_t T;  // the row's length
    int s;      // 0: the row starts on a 16-byte boundary
    __device__ __forceinline__ TcLoads(const uint16_t *r, int64_t row_len)
        : row(r),
          T(row_len),
          s(A16 ? 0 : static_cast<int>((reinterpret_cast<uintptr_t>(r) & 15u) >> 1)) {}
    // The lane's tokens t .. t+7 (aligned rows; zero from `end`), or its block.
    __device__ __forceinline__ Raw<8> load(int64_t t, int64_t end) const {
        if (A16 || s == 0) {
            if (t < end) return tc_load<NTL>(row, t, end, 16);
            Raw<8> z;
            z.v = u32x4_t{0u, 0u, 0u, 0u};
            return z;
        }
        return tc_block<NTL>(row, t - s, T);
    }
    // Lane 0's block of the tile at t (the chunk's tail; unused for aligned rows).
    __device__ __forceinline__ Raw<8> tail(int64_t t) const {
        if (A16 || s == 0) {
            Raw<8> z;
            z.v = u32x4_t{0u, 0u, 0u, 0u};
            return z;
        }
        return tc_block<NTL>(row, t - s, T);
    }
    // Block -> tokens t .. t+7, given the next tile's blocks (lane 0's is
    // used).  Every lane of the wave calls it.
    __device__ __forceinline__ void fix(Raw<8> &r, const Raw<8> &next_tile) const {
        if (A16 || s == 0) return;
        uint32_t c[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c[k] = r.v[k];
            const int32_t first = __builtin_amdgcn_readlane(static_cast<int32_t>(next_tile.v[k]), 0);
            c[4 + k] = static_cast<uint32_t>(tc_lane_down_u32(static_cast<int32_t>(r.v[k]), first));
        }
        const uint32_t sh = (s & 1) ? 2u : 0u;
        switch (s >> 1) {
            case 0: r.v = tc_funnel<0>(c, sh); break;
            case 1: r.v = tc_funnel<1>(c, sh); break;
            case 2: r.v = tc_funnel<2>(c, sh); break;
            default: r.v = tc_funnel<3>(c, sh); break;
        }
    }
};

// Single extended tokens of one row (b, d): x_ext at p < T is the input for
// p >= 0, else the initial state's slot p + W-1, else zero.  The source is
// picked by selects and every case has a valid address (a zero token reads
// the row's first input and is dropped after the load), so these loads are
// issued without a branch, before the bulk loads, and no wait comes between
// them: the first tile can start as soon as its own data is in.
template <int W>
struct TcRowExt {
    const uint16_t *xr;  // the row's input, T >= 1 tokens
    const uint16_t *ir;  // the row's initial state, or null
    int64_t is2;         // its slot stride
    __device__ __forceinline__ TcRowExt(const uint16_t *x_row, const Strided3 &init, int64_t b,
                                        int64_t d)
        : xr(x_row),
          ir(init.ptr ? static_cast<const uint16_t *>(init.ptr) + b * init.s0 + d * init.s1
                      : nullptr),
          is2(init.s2) {}
    // Raw bits of x_ext[p]; `keep` false where x_ext[p] is zero.
    __device__ __forceinline__ uint16_t load(int64_t p, bool &keep) const {
        keep = p >= 0 || ir;
        const uint16_t *src = p >= 0 ? xr + p : ir ? ir + (p + W - 1) * is2 : xr;
        return *src;
    }
};
__device__ __forceinline__ float kept_f32(uint16_t bits, bool keep) {
    return keep ? bf16_bits_to_f32(bits) : 0.0f;
}

// Work item of a time-lane wave: row (b, d) and chunk [t0, t1).
struct TcItem {
    int64_t b, d, chunk, t0, t1;
};
template <typename A>
__device__ __forceinline__ bool tc_item(const A &a, TcItem &it) {
    const int64_t wid = xcd_remap(blockIdx.x, a.n_block) * kWavesPerBlock +
                        __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    if (wid >= a.B * a.D * a.n_chunk) return false;
    if (a.tc_div32) {
        const uint32_t w32 = static_cast<uint32_t>(wid);
        const uint32_t row = div32(w32, a.tc_chunks);
        const uint32_t b = div32(row, a.tc_rows);
        it.chunk = w32 - row * static_cast<uint32_t>(a.n_chunk);
        it.b = b;
        it.d = row - b * static_cast<uint32_t>(a.D);
    } else {
        const int64_t row = wid / a.n_chunk;
        it.chunk = wid % a.n_chunk;
        it.b = row / a.D;
        it.d = row % a.D;
    }
    it.t0 = it.chunk * a.L;
    it.t1 = min(it.t0 + a.L, a.T);
    return true;
}

// No check: dense rows.  A packed chunk's check runs once the chunk's loads
// are issued and says whether the chunk may write.
struct TcNoCheck {
    __device__ __forceinline__ bool ok() const { return true; }
};

// Runs f(ntl, a16) with the call's cache policy for the bulk loads and
// whether every row start of every tensor is 16-byte aligned (then the
// tiles move as whole vectors with no alignment test in the kernel).
template <typename A, typename F>
__device__ __forceinline__ void tc_run(const A &a, F &&f) {
    if (a.tc_vec16) {
        if (a.nt_load) f(std::true_type{}, std::true_type{});
        else f(std::false_type{}, std::true_type{});
    } else {
        if (a.nt_load) f(std::true_type{}, std::false_type{});
        else f(std::false_type{}, std::false_type{});
    }
}

template <int W, bool SILU, int FK, bool NTL, bool A16, typename Check>
__device__ __forceinline__ void fwd_tc_chunk(const FwdArgs &a, const TcItem &it,
                                             const Check &check) {
    const int lane = threadIdx.x % kWaveSize;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x.ptr) + it.b * a.x.s0 + it.d * a.x.s1;
    uint16_t *yr = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.y.ptr)) +
                   it.b * a.y.s0 + it.d * a.y.s1;
    const int ay = A16 ? 16 : tc_align(yr);
    const TcLoads<NTL, A16> lx(xr, a.T);
    // Left halo, the final state's tokens (lanes 0..W-2 of the chunk that
    // ends the row copy the row's last W-1 extended tokens bit for bit; the
    // other lanes repeat lane W-2's address), the filter, then the tiles.
    const TcRowExt<W> ext(xr, a.init, it.b, it.d);
    uint16_t lh[W - 1];
    bool lh_keep[W - 1], fin_keep;
#pragma unroll
    for (int j = 0; j < W - 1; ++j) lh[j] = ext.load(it.t0 - (W - 1) + j, lh_keep[j]);
    const uint16_t fin_bits = ext.load(a.T - (W - 1) + min(lane, W - 2), fin_keep);
    float w[W][1], bias[1];
    load_filter<W, 1, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, it.d, w, bias);
    Raw<8> raw[kTcTilesFwd];
#pragma unroll
    for (int c = 0; c < kTcTilesFwd; ++c) {
        const int64_t t = it.t0 + c * kTcTile + lane * kTcE;
        raw[c] = lx.load(t, it.t1);
    }
    const Raw<8> xtail = lx.tail(it.t0 + kTcTilesFwd * kTcTile);
    if (!check.ok()) return;
    float carry[W - 1];  // x_ext of the W-1 tokens before the current tile
#pragma unroll
    for (int j = 0; j < W - 1; ++j) carry[j] = kept_f32(lh[j], lh_keep[j]);

#pragma unroll
    for (int c = 0; c < kTcTilesFwd; ++c) {
        const int64_t tt = it.t0 + c * kTcTile;
        if (tt >= it.t1) break;
        float v[kTcE], xe[W - 1 + kTcE], out[kTcE];
        lx.fix(raw[c], c + 1 < kTcTilesFwd ? raw[c + 1 < kTcTilesFwd ? c + 1 : c] : xtail);
        unpack<8>(raw[c], v);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) xe[j] = lane_up(v[kTcE - (W - 1) + j], carry[j]);
#pragma unroll
        for (int i = 0; i < kTcE; ++i) xe[W - 1 + i] = v[i];
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) z = fmaf(w[k][0], xe[i + k], z);
            out[i] = act<SILU>(z);
        }
        const int64_t t = tt + lane * kTcE;
        if (t < it.t1) tc_store<true>(yr, t, it.t1, out, ay);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) carry[j] = from_lane(v[kTcE - (W - 1) + j], kWaveSize - 1);
    }
    if (it.t1 == a.T && a.fin.ptr && lane < W - 1)
        const_cast<uint16_t *>(static_cast<const uint16_t *>(a.fin.ptr))
            [it.b * a.fin.s0 + it.d * a.fin.s1 + lane * a.fin.s2] = fin_keep ? fin_bits : 0;
}

template <int W, bool SILU, int FK>
__global__ __launch_bounds__(256) void k_fwd_tc(FwdArgs a) {
    TcItem it;
    if (!tc_item(a, it)) return;
    tc_run(a, [&](auto ntl, auto a16) {
        fwd_tc_chunk<W, SILU, FK, decltype(ntl)::value, decltype(a16)::value>(a, it, TcNoCheck{});
    });
}

// Backward on time lanes.  Per tile: z and g = dy * act'(z) for the lane's
// tokens, dW/dB accumulated per lane; dx[p] = sum_k w[k] g[p+W-1-k] needs
// the next W-1 g's, from the next lane or, for lane 63, from the next tile,
// so a tile's dx is emitted once the next tile's g is known.  After the
// chunk's last tile the W-1 g's past the chunk are computed directly (the
// right halo).  dW/dB: one wave sum per chunk, then an atomic or a unique
// partial.
template <int W, bool SILU, int FK, bool NTL, bool A16, typename Check>
__device__ __forceinline__ void bwd_tc_chunk(const BwdArgs &a, const TcItem &it,
                                             const Check &check) {
    constexpr bool BIAS = fk_bias(FK);
    const int lane = threadIdx.x % kWaveSize;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x.ptr) + it.b * a.x.s0 + it.d * a.x.s1;
    const uint16_t *dyr = static_cast<const uint16_t *>(a.dy.ptr) + it.b * a.dy.s0 + it.d * a.dy.s1;
    uint16_t *dxr = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dx.ptr)) +
                    it.b * a.dx.s0 + it.d * a.dx.s1;
    const int adx = A16 ? 16 : tc_align(dxr);
    const TcLoads<NTL, A16> lx(xr, a.T), ld(dyr, a.T);
    // Single-token loads first, without branches (as in the forward): the
    // left halo; the right halo (lane j < W-1 reads token t1 + j of x and dy;
    // the other lanes, and tokens past the row, read an in-row token that is
    // dropped); the row's final-state gradient (every lane holds all W-1
    // values; a row without one reads its first input token W-1 times).
    const TcRowExt<W> ext(xr, a.init, it.b, it.d);
    uint16_t lh[W - 1];
    bool lh_keep[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) lh[j] = ext.load(it.t0 - (W - 1) + j, lh_keep[j]);
    const int64_t rq = min(it.t1 + lane, a.T - 1);
    const uint16_t rh_x = xr[rq], rh_dy = dyr[rq];
    const uint16_t *dfr = a.dfin.ptr ? static_cast<const uint16_t *>(a.dfin.ptr) +
                                           it.b * a.dfin.s0 + it.d * a.dfin.s1
                                     : xr;
    const int64_t dfs = a.dfin.ptr ? a.dfin.s2 : 0;
    uint16_t dfb[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) dfb[j] = dfr[j * dfs];
    Raw<8> rx[kTcTilesBwd], rd[kTcTilesBwd];
#pragma unroll
    for (int c = 0; c < kTcTilesBwd; ++c) {
        const int64_t t = it.t0 + c * kTcTile + lane * kTcE;
        rx[c] = lx.load(t, it.t1);
        rd[c] = ld.load(t, it.t1);
    }
    const Raw<8> xtail = lx.tail(it.t0 + kTcTilesBwd * kTcTile),
                 dtail = ld.tail(it.t0 + kTcTilesBwd * kTcTile);
    float w[W][1], bias[1];
    load_filter<W, 1, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, it.d, w, bias);
    if (!check.ok()) return;
    float carry[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) carry[j] = kept_f32(lh[j], lh_keep[j]);
    float dfv[W - 1];  // dfinal of the row (zeros without one)
#pragma unroll
    for (int j = 0; j < W - 1; ++j) dfv[j] = kept_f32(dfb[j], a.dfin.ptr != nullptr);
    float dwacc[W], dbacc = 0.0f;
#pragma unroll
    for (int k = 0; k < W; ++k) dwacc[k] = 0.0f;
    const int64_t fin0 = a.T - (W - 1);  // first position a final-state gradient reaches

    // dx of the lane's tokens of the tile at tt from its g and the W-1 g's
    // that follow the lane (gn: the next lane's, or `after` for lane 63).
    auto emit = [&](int64_t tt, const float (&g)[kTcE], const float (&after)[W - 1]) {
        float ge[kTcE + W - 1], v[kTcE];
#pragma unroll
        for (int i = 0; i < kTcE; ++i) ge[i] = g[i];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) ge[kTcE + j] = lane_down(g[j], after[j]);
        const int64_t t = tt + lane * kTcE;
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            float acc = w[0][0] * ge[i + W - 1];
#pragma unroll
            for (int j = W - 2; j >= 0; --j) acc = fmaf(w[W - 1 - j][0], ge[i + j], acc);
            v[i] = acc;
        }
        if (a.dfin.ptr && t + kTcE > fin0) {
#pragma unroll
            for (int i = 0; i < kTcE; ++i) {
                const int64_t m = t + i - fin0;  // final-state slot of the token, if any
#pragma unroll
                for (int j = 0; j < W - 1; ++j)
                    if (m == j) v[i] += dfv[j];
            }
        }
        if (t < it.t1) tc_store<true>(dxr, t, it.t1, v, adx);
    };

    float gprev[kTcE];
    int64_t tprev = -1;
#pragma unroll
    for (int c = 0; c < kTcTilesBwd; ++c) {
        const int64_t tt = it.t0 + c * kTcTile;
        if (tt >= it.t1) break;
        float v[kTcE], dyv[kTcE], xe[W - 1 + kTcE], g[kTcE];
        lx.fix(rx[c], c + 1 < kTcTilesBwd ? rx[c + 1 < kTcTilesBwd ? c + 1 : c] : xtail);
        ld.fix(rd[c], c + 1 < kTcTilesBwd ? rd[c + 1 < kTcTilesBwd ? c + 1 : c] : dtail);
        unpack<8>(rx[c], v);
        unpack<8>(rd[c], dyv);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) xe[j] = lane_up(v[kTcE - (W - 1) + j], carry[j]);
#pragma unroll
        for (int i = 0; i < kTcE; ++i) xe[W - 1 + i] = v[i];
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) z = fmaf(w[k][0], xe[i + k], z);
            g[i] = dyv[i] * act_slope<SILU>(z);  // zero past the chunk (dy reads 0)
#pragma unroll
            for (int k = 0; k < W; ++k) dwacc[k] = fmaf(g[i], xe[i + k], dwacc[k]);
            if constexpr (BIAS) dbacc += g[i];
        }
        if (tprev >= 0) {
            float after[W - 1];
#pragma unroll
            for (int j = 0; j < W - 1; ++j) after[j] = from_lane(g[j], 0);
            emit(tprev, gprev, after);
        }
        // The gradient of the initial state: dx_ext at -(W-1)..-1 from the
        // row's first g's (lane 0 of the first tile).
        if (tt == 0 && a.dinit.ptr && lane == 0) {
#pragma unroll
            for (int j = 0; j < W - 1; ++j) {
                const int64_t p = j - (W - 1);
                float acc = w[0][0] * (p + W - 1 < kTcE ? g[p + W - 1] : 0.0f);
#pragma unroll
                for (int m = W - 2; m >= 0; --m)
                    acc = fmaf(w[W - 1 - m][0], p + m >= 0 ? g[p + m] : 0.0f, acc);
                if (a.dfin.ptr && p >= fin0) {
#pragma unroll
                    for (int m = 0; m < W - 1; ++m)
                        if (p - fin0 == m) acc += dfv[m];
                }
                const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dinit.ptr))
                    [it.b * a.dinit.s0 + it.d * a.dinit.s1 + j * a.dinit.s2] = to_bf16_bits(acc);
            }
        }
#pragma unroll
        for (int i = 0; i < kTcE; ++i) gprev[i] = g[i];
        tprev = tt;
#pragma unroll
        for (int j = 0; j < W - 1; ++j) carry[j] = from_lane(v[kTcE - (W - 1) + j], kWaveSize - 1);
    }
    // Right halo: g at t1 .. t1+W-2 (zero past the row) for the last tile's
    // lane 63, computed in every lane from the prefetched tokens.  A chunk
    // that does not end the row is a whole number of tiles, so `carry` now
    // holds x at t1-(W-1) .. t1-1.
    {
        float xw[2 * (W - 1)], after[W - 1];
        const float hx = bf16_bits_to_f32(rh_x), hd = bf16_bits_to_f32(rh_dy);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            xw[j] = carry[j];
            xw[W - 1 + j] = from_lane(hx, j);
        }
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) z = fmaf(w[k][0], xw[j + k], z);
            after[j] = it.t1 + j < a.T ? from_lane(hd, j) * act_slope<SILU>(z) : 0.0f;
        }
        emit(tprev, gprev, after);
    }
    // dW/dB of the chunk: a wave sum, then one atomic or one partial per tap.
#pragma unroll
    for (int k = 0; k < W; ++k) dwacc[k] = wave_sum(dwacc[k]);
    if constexpr (BIAS) dbacc = wave_sum(dbacc);
    if (lane == 0) {
        if (a.partial) {
            const int64_t pidx = it.b * a.n_chunk + it.chunk;
            float *pr = a.partial + (pidx * a.D + it.d) * a.part_stride;
#pragma unroll
            for (int k = 0; k < W; ++k) pr[k] = dwacc[k];
            if (a.part_stride > W) pr[W] = dbacc;
        } else {
#pragma unroll
            for (int k = 0; k < W; ++k) atomicAdd(a.dw + it.d * W + k, dwacc[k]);
            if constexpr (BIAS) atomicAdd(a.db + it.d, dbacc);
        }
    }
}

template <int W, bool SILU, int FK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CCV_TC_BWD_WAVES)))
void k_bwd_tc(BwdArgs a) {
    TcItem it;
    if (!tc_item(a, it)) return;
    tc_run(a, [&](auto ntl, auto a16) {
        bwd_tc_chunk<W, SILU, FK, decltype(ntl)::value, decltype(a16)::value>(a, it, TcNoCheck{});
    });
}

// ===========================================================================
// Time lanes for seq_idx rows (unit stride along T)
//
// The lanes, tiles and chunks of the dense time-lane kernels, with the
// seq_idx entry of every token beside its value.  A tap contributes the input
// only when its token has the output token's id, otherwise zero.  Ids move
// across lanes with the same DPP shifts as the values.  Positions outside the
// row carry kNoId; an entry equal to it meets only zero inputs (before the
// row) or zero gradients (past it).
// ===========================================================================
constexpr int32_t kNoId = -1;

__device__ __forceinline__ int32_t lane_up_id(int32_t v, int32_t first) {
    return __builtin_amdgcn_update_dpp(first, v, kDppWaveShr1, 0xf, 0xf, false);
}
__device__ __forceinline__ int32_t lane_down_id(int32_t v, int32_t last) {
    return __builtin_amdgcn_update_dpp(last, v, kDppWaveShl1, 0xf, 0xf, false);
}
__device__ __forceinline__ int32_t from_lane_id(int32_t v, int l) {
    return __builtin_amdgcn_readlane(v, l);
}

// The seq_idx entries of one row.
struct TcSeqIds {
    const int32_t *sq;  // this row's entries
    int64_t st;         // their stride
    bool vec;           // unit stride and 16-byte aligned rows
    int64_t T;
    __device__ __forceinline__ int32_t at(int64_t p) const {
        return p < 0 || p >= T ? kNoId : sq[p * st];
    }
    // The ids of the kTcE tokens from t (kNoId past the row).
    __device__ __forceinline__ void lane_ids(int64_t t, int32_t (&id)[kTcE]) const {
        if (vec && t + kTcE <= T) {
            // t is a multiple of kTcE: two 16-byte loads
            const u32x4_t *q = reinterpret_cast<const u32x4_t *>(sq + t);
            const u32x4_t lo = q[0], hi = q[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                id[e] = static_cast<int32_t>(lo[e]);
                id[4 + e] = static_cast<int32_t>(hi[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < kTcE; ++e) id[e] = t + e < T ? sq[(t + e) * st] : kNoId;
        }
    }
};

template <typename A>
__device__ __forceinline__ TcSeqIds tc_seq_ids(const A &a, const TcItem &it) {
    TcSeqIds ids;
    ids.sq = a.seq + it.b * a.seq_sb;
    ids.st = a.seq_st;
    ids.vec = a.seq_vec != 0;
    ids.T = a.T;
    return ids;
}

// Tap values of output token i of a window (xe/ie: values and ids of the
// W-1 tokens before the lane's first token, then its kTcE tokens).
template <int W>
__device__ __forceinline__ void tc_taps(const float (&xe)[W - 1 + kTcE],
                                        const int32_t (&ie)[W - 1 + kTcE], int i,
                                        float (&xv)[W]) {
    const int32_t own = ie[i + W - 1];
#pragma unroll
    for (int k = 0; k < W; ++k) xv[k] = ie[i + k] == own ? xe[i + k] : 0.0f;
}

template <int W, bool SILU, int FK, bool NTL, bool A16>
__device__ __forceinline__ void fwd_tcs_chunk(const FwdArgs &a, const TcItem &it,
                                              const TcSeqIds &ids) {
    const int lane = threadIdx.x % kWaveSize;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x.ptr) + it.b * a.x.s0 + it.d * a.x.s1;
    uint16_t *yr = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.y.ptr)) +
                   it.b * a.y.s0 + it.d * a.y.s1;
    const int ay = A16 ? 16 : tc_align(yr);
    const TcLoads<NTL, A16> lx(xr, a.T);
    // Left halo (values and ids of the W-1 tokens before the chunk; before
    // the row, zero and kNoId), the filter, then the tiles and their ids.
    uint16_t lh[W - 1];
    int32_t cid[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int64_t p = it.t0 - (W - 1) + j;
        lh[j] = xr[p >= 0 ? p : 0];
        cid[j] = ids.at(p);
    }
    float w[W][1], bias[1];
    load_filter<W, 1, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, it.d, w, bias);
    Raw<8> raw[kTcTilesFwd];
    int32_t tid[kTcTilesFwd][kTcE];
#pragma unroll
    for (int c = 0; c < kTcTilesFwd; ++c) {
        const int64_t t = it.t0 + c * kTcTile + lane * kTcE;
        raw[c] = lx.load(t, it.t1);
        ids.lane_ids(t < it.t1 ? t : a.T, tid[c]);
    }
    const Raw<8> xtail = lx.tail(it.t0 + kTcTilesFwd * kTcTile);
    float carry[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
        carry[j] = it.t0 - (W - 1) + j >= 0 ? bf16_bits_to_f32(lh[j]) : 0.0f;

#pragma unroll
    for (int c = 0; c < kTcTilesFwd; ++c) {
        const int64_t tt = it.t0 + c * kTcTile;
        if (tt >= it.t1) break;
        const int64_t t = tt + lane * kTcE;
        float v[kTcE], xe[W - 1 + kTcE], out[kTcE];
        int32_t ie[W - 1 + kTcE];
        lx.fix(raw[c], c + 1 < kTcTilesFwd ? raw[c + 1 < kTcTilesFwd ? c + 1 : c] : xtail);
        unpack<8>(raw[c], v);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            xe[j] = lane_up(v[kTcE - (W - 1) + j], carry[j]);
            ie[j] = lane_up_id(tid[c][kTcE - (W - 1) + j], cid[j]);
        }
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            xe[W - 1 + i] = v[i];
            ie[W - 1 + i] = tid[c][i];
        }
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            float xv[W];
            tc_taps<W>(xe, ie, i, xv);
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) z = fmaf(w[k][0], xv[k], z);
            out[i] = act<SILU>(z);
        }
        if (t < it.t1) tc_store<true>(yr, t, it.t1, out, ay);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            carry[j] = from_lane(v[kTcE - (W - 1) + j], kWaveSize - 1);
            cid[j] = from_lane_id(tid[c][kTcE - (W - 1) + j], kWaveSize - 1);
        }
    }
}

template <int W, bool SILU, int FK, bool NTL, bool A16>
__device__ __forceinline__ void bwd_tcs_chunk(const BwdArgs &a, const TcItem &it,
                                              const TcSeqIds &ids) {
    constexpr bool BIAS = fk_bias(FK);
    const int lane = threadIdx.x % kWaveSize;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x.ptr) + it.b * a.x.s0 + it.d * a.x.s1;
    const uint16_t *dyr = static_cast<const uint16_t *>(a.dy.ptr) + it.b * a.dy.s0 + it.d * a.dy.s1;
    uint16_t *dxr = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dx.ptr)) +
                    it.b * a.dx.s0 + it.d * a.dx.s1;
    const int adx = A16 ? 16 : tc_align(dxr);
    const TcLoads<NTL, A16> lx(xr, a.T), ld(dyr, a.T);
    // Single tokens first: the left halo (values, ids); the right halo (lane
    // j < W-1 reads token t1 + j of x and dy, the other lanes and tokens
    // past the row an in-row token that is dropped) and its ids.
    uint16_t lh[W - 1];
    int32_t cid[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int64_t p = it.t0 - (W - 1) + j;
        lh[j] = xr[p >= 0 ? p : 0];
        cid[j] = ids.at(p);
    }
    const int64_t rq = min(it.t1 + lane, a.T - 1);
    const uint16_t rh_x = xr[rq], rh_dy = dyr[rq];
    float w[W][1], bias[1];
    load_filter<W, 1, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, it.d, w, bias);
    Raw<8> rx[kTcTilesBwd], rd[kTcTilesBwd];
    int32_t tid[kTcTilesBwd][kTcE];
#pragma unroll
    for (int c = 0; c < kTcTilesBwd; ++c) {
        const int64_t t = it.t0 + c * kTcTile + lane * kTcE;
        rx[c] = lx.load(t, it.t1);
        rd[c] = ld.load(t, it.t1);
        ids.lane_ids(t < it.t1 ? t : a.T, tid[c]);
    }
    const Raw<8> xtail = lx.tail(it.t0 + kTcTilesBwd * kTcTile),
                 dtail = ld.tail(it.t0 + kTcTilesBwd * kTcTile);
    const int32_t rh_id = ids.at(it.t1 + lane);  // lane j < W-1: the id of token t1 + j
    float carry[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
        carry[j] = it.t0 - (W - 1) + j >= 0 ? bf16_bits_to_f32(lh[j]) : 0.0f;
    float dwacc[W], dbacc = 0.0f;
#pragma unroll
    for (int k = 0; k < W; ++k) dwacc[k] = 0.0f;

    // dx of the lane's tokens of the tile at tt from its g's and ids, and
    // the W-1 g's and ids that follow the lane (`after`: the next tile's, or
    // the right halo's, for lane 63).
    auto emit = [&](int64_t tt, const float (&g)[kTcE], const int32_t (&id)[kTcE],
                    const float (&after)[W - 1], const int32_t (&after_id)[W - 1]) {
        float ge[kTcE + W - 1], v[kTcE];
        int32_t ige[kTcE + W - 1];
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            ge[i] = g[i];
            ige[i] = id[i];
        }
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            ge[kTcE + j] = lane_down(g[j], after[j]);
            ige[kTcE + j] = lane_down_id(id[j], after_id[j]);
        }
        const int64_t t = tt + lane * kTcE;
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            const int32_t own = ige[i];
            float acc = w[0][0] * (ige[i + W - 1] == own ? ge[i + W - 1] : 0.0f);
#pragma unroll
            for (int j = W - 2; j >= 0; --j)
                acc = fmaf(w[W - 1 - j][0], ige[i + j] == own ? ge[i + j] : 0.0f, acc);
            v[i] = acc;
        }
        if (t < it.t1) tc_store<true>(dxr, t, it.t1, v, adx);
    };

    float gprev[kTcE];
    int32_t idprev[kTcE];
    int64_t tprev = -1;
#pragma unroll
    for (int c = 0; c < kTcTilesBwd; ++c) {
        const int64_t tt = it.t0 + c * kTcTile;
        if (tt >= it.t1) break;
        float v[kTcE], dyv[kTcE], xe[W - 1 + kTcE], g[kTcE];
        int32_t ie[W - 1 + kTcE];
        lx.fix(rx[c], c + 1 < kTcTilesBwd ? rx[c + 1 < kTcTilesBwd ? c + 1 : c] : xtail);
        ld.fix(rd[c], c + 1 < kTcTilesBwd ? rd[c + 1 < kTcTilesBwd ? c + 1 : c] : dtail);
        unpack<8>(rx[c], v);
        unpack<8>(rd[c], dyv);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            xe[j] = lane_up(v[kTcE - (W - 1) + j], carry[j]);
            ie[j] = lane_up_id(tid[c][kTcE - (W - 1) + j], cid[j]);
        }
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            xe[W - 1 + i] = v[i];
            ie[W - 1 + i] = tid[c][i];
        }
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            float xv[W];
            tc_taps<W>(xe, ie, i, xv);
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) z = fmaf(w[k][0], xv[k], z);
            g[i] = dyv[i] * act_slope<SILU>(z);  // zero past the chunk (dy reads 0)
#pragma unroll
            for (int k = 0; k < W; ++k) dwacc[k] = fmaf(g[i], xv[k], dwacc[k]);
            if constexpr (BIAS) dbacc += g[i];
        }
        if (tprev >= 0) {
            float after[W - 1];
            int32_t after_id[W - 1];
#pragma unroll
            for (int j = 0; j < W - 1; ++j) {
                after[j] = from_lane(g[j], 0);
                after_id[j] = from_lane_id(tid[c][j], 0);
            }
            emit(tprev, gprev, idprev, after, after_id);
        }
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            gprev[i] = g[i];
            idprev[i] = tid[c][i];
        }
        tprev = tt;
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            carry[j] = from_lane(v[kTcE - (W - 1) + j], kWaveSize - 1);
            cid[j] = from_lane_id(tid[c][kTcE - (W - 1) + j], kWaveSize - 1);
        }
    }
    // Right halo: g at t1 .. t1+W-2 (zero past the row), in every lane.  A
    // chunk that does not end the row is a whole number of tiles, so
    // `carry`/`cid` hold the W-1 tokens before t1.
    {
        float xw[2 * (W - 1)], after[W - 1];
        int32_t iw[2 * (W - 1)], after_id[W - 1];
        const float hx = bf16_bits_to_f32(rh_x), hd = bf16_bits_to_f32(rh_dy);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            xw[j] = carry[j];
            iw[j] = cid[j];
            xw[W - 1 + j] = from_lane(hx, j);
            iw[W - 1 + j] = from_lane_id(rh_id, j);
        }
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int32_t own = iw[j + W - 1];
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) z = fmaf(w[k][0], iw[j + k] == own ? xw[j + k] : 0.0f, z);
            after[j] = it.t1 + j < a.T ? from_lane(hd, j) * act_slope<SILU>(z) : 0.0f;
            after_id[j] = own;
        }
        emit(tprev, gprev, idprev, after, after_id);
    }
    // dW/dB of the chunk: a wave sum, then one atomic or one partial per tap.
#pragma unroll
    for (int k = 0; k < W; ++k) dwacc[k] = wave_sum(dwacc[k]);
    if constexpr (BIAS) dbacc = wave_sum(dbacc);
    if (lane == 0) {
        if (a.partial) {
            const int64_t pidx = it.b * a.n_chunk + it.chunk;
            float *pr = a.partial + (pidx * a.D + it.d) * a.part_stride;
#pragma unroll
            for (int k = 0; k < W; ++k) pr[k] = dwacc[k];
            if (a.part_stride > W) pr[W] = dbacc;
        } else {
#pragma unroll
            for (int k = 0; k < W; ++k) atomicAdd(a.dw + it.d * W + k, dwacc[k]);
            if constexpr (BIAS) atomicAdd(a.db + it.d, dbacc);
        }
    }
}

// ---------------------------------------------------------------------------
// The same lanes with block-shared tap masks (CCV_TCS_MASKS_FWD/_BWD).  A block's four
// waves take four consecutive rows (b, d) of one chunk, so they share the
// chunk's seq_idx entries: wave w reads the entries of tile w only and turns
// them into one tap-mask word per lane (bit 3i + l-1: token i of the lane and
// the token l places before it carry the same entry, l = 1..W-1), and the
// block exchanges the words through LDS.  A wave past the last row only
// builds masks.  The backward also needs the words of the W-1 tokens past the
// chunk (the right halo), built by wave 0.
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ uint32_t tcm_word(const int32_t (&ie)[W - 1 + kTcE]) {
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < kTcE; ++i)
#pragma unroll
        for (int l = 1; l < W; ++l)
            if (ie[i + W - 1 - l] == ie[i + W - 1]) m |= 1u << (3 * i + l - 1);
    return m;
}
// v where bit b of m is set, else +0 (an AND with the bit spread to 32).
__device__ __forceinline__ float tcm_keep(float v, uint32_t m, int b) {
    return __int_as_float(__float_as_int(v) &
                          __builtin_amdgcn_sbfe(static_cast<int>(m), static_cast<unsigned>(b), 1u));
}

// Work item: block q = (b, chunk, row group), row groups innermost (32-bit
// decode by tc_rows = n_rg and tc_chunks = n_chunk); wave w takes row
// d = 4 rg + w, `live` when d < D (else d is clamped and nothing is loaded
// or written for it).
template <typename A>
__device__ __forceinline__ void tcm_item(const A &a, TcItem &it, bool &live) {
    const int64_t q = xcd_remap(blockIdx.x, a.n_block);
    const int64_t n_rg = (a.D + kWavesPerBlock - 1) / kWavesPerBlock;
    int64_t rg;
    if (a.tc_div32) {
        const uint32_t q32 = static_cast<uint32_t>(q);
        const uint32_t bc = div32(q32, a.tc_rows);
        rg = q32 - bc * static_cast<uint32_t>(n_rg);
        const uint32_t b = div32(bc, a.tc_chunks);
        it.chunk = bc - b * static_cast<uint32_t>(a.n_chunk);
        it.b = b;
    } else {
        const int64_t bc = q / n_rg;
        rg = q % n_rg;
        it.chunk = bc % a.n_chunk;
        it.b = bc / a.n_chunk;
    }
    it.d = rg * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    live = it.d < a.D;
    if (!live) it.d = a.D - 1;
    it.t0 = it.chunk * a.L;
    it.t1 = min(it.t0 + a.L, a.T);
}

// Build the block's mask words (tile w by wave w; the right halo's by wave 0
// when RH) and make them visible to the block.  Every wave of the block
// calls it.
template <int W, int TILES, bool RH>
__device__ __forceinline__ void tcm_build(const TcItem &it, const TcSeqIds &ids, int64_t T,
                                          uint32_t (&s_mask)[TILES][kWaveSize],
                                          uint32_t &s_rh) {
    static_assert(W <= 4, "3 mask bits per token");
    static_assert(TILES <= kWavesPerBlock, "one tile per wave");
    const int wave = threadIdx.x / kWaveSize, lane = threadIdx.x % kWaveSize;
    const int64_t tt = it.t0 + static_cast<int64_t>(wave) * kTcTile;
    if (wave < TILES && tt < it.t1) {
        const int64_t t = tt + lane * kTcE;
        int32_t id[kTcE], hid[W - 1], ie[W - 1 + kTcE];
        ids.lane_ids(t < it.t1 ? t : T, id);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) hid[j] = ids.at(tt - (W - 1) + j);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) ie[j] = lane_up_id(id[kTcE - (W - 1) + j], hid[j]);
#pragma unroll
        for (int i = 0; i < kTcE; ++i) ie[W - 1 + i] = id[i];
        s_mask[wave][lane] = tcm_word<W>(ie);
    }
    if (RH && wave == 0) {
        // tokens t1 + j (j < W-1) against the W-1 tokens before each
        int32_t iw[2 * (W - 1)];
#pragma unroll
        for (int k = 0; k < 2 * (W - 1); ++k) iw[k] = ids.at(it.t1 - (W - 1) + k);
        uint32_t m = 0u;
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
#pragma unroll
            for (int l = 1; l < W; ++l)
                if (iw[j + W - 1 - l] == iw[j + W - 1]) m |= 1u << (3 * j + l - 1);
        if (lane == 0) s_rh = m;
    }
    __syncthreads();
}

template <int W, bool SILU, int FK, bool NTL, bool A16>
__device__ __forceinline__ void fwd_tcm_chunk(const FwdArgs &a, const TcItem &it, bool live,
                                              const TcSeqIds &ids,
                                              uint32_t (&s_mask)[kTcTilesFwd][kWaveSize],
                                              uint32_t &s_rh) {
    const int lane = threadIdx.x % kWaveSize;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x.ptr) + it.b * a.x.s0 + it.d * a.x.s1;
    uint16_t *yr = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.y.ptr)) +
                   it.b * a.y.s0 + it.d * a.y.s1;
    const int ay = A16 ? 16 : tc_align(yr);
    const TcLoads<NTL, A16> lx(xr, a.T);
    uint16_t lh[W - 1];
    float w[W][1], bias[1];
    Raw<8> raw[kTcTilesFwd], xtail;
    if (live) {
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int64_t p = it.t0 - (W - 1) + j;
            lh[j] = xr[p >= 0 ? p : 0];
        }
        load_filter<W, 1, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, it.d, w, bias);
#pragma unroll
        for (int c = 0; c < kTcTilesFwd; ++c) {
            const int64_t t = it.t0 + c * kTcTile + lane * kTcE;
            raw[c] = lx.load(t, it.t1);
        }
        xtail = lx.tail(it.t0 + kTcTilesFwd * kTcTile);
    }
    tcm_build<W, kTcTilesFwd, false>(it, ids, a.T, s_mask, s_rh);
    if (!live) return;
    float carry[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
        carry[j] = it.t0 - (W - 1) + j >= 0 ? bf16_bits_to_f32(lh[j]) : 0.0f;
#pragma unroll
    for (int c = 0; c < kTcTilesFwd; ++c) {
        const int64_t tt = it.t0 + c * kTcTile;
        if (tt >= it.t1) break;
        const int64_t t = tt + lane * kTcE;
        const uint32_t mc = s_mask[c][lane];
        float v[kTcE], xe[W - 1 + kTcE], out[kTcE];
        lx.fix(raw[c], c + 1 < kTcTilesFwd ? raw[c + 1 < kTcTilesFwd ? c + 1 : c] : xtail);
        unpack<8>(raw[c], v);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) xe[j] = lane_up(v[kTcE - (W - 1) + j], carry[j]);
#pragma unroll
        for (int i = 0; i < kTcE; ++i) xe[W - 1 + i] = v[i];
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int lag = W - 1 - k;
                z = fmaf(w[k][0], lag == 0 ? xe[i + k] : tcm_keep(xe[i + k], mc, 3 * i + lag - 1),
                         z);
            }
            out[i] = act<SILU>(z);
        }
        if (t < it.t1) tc_store<true>(yr, t, it.t1, out, ay);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) carry[j] = from_lane(v[kTcE - (W - 1) + j], kWaveSize - 1);
    }
}

template <int W, bool SILU, int FK, bool NTL, bool A16>
__device__ __forceinline__ void bwd_tcm_chunk(const BwdArgs &a, const TcItem &it, bool live,
                                              const TcSeqIds &ids,
                                              uint32_t (&s_mask)[kTcTilesBwd][kWaveSize],
                                              uint32_t &s_rh) {
    constexpr bool BIAS = fk_bias(FK);
    const int lane = threadIdx.x % kWaveSize;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x.ptr) + it.b * a.x.s0 + it.d * a.x.s1;
    const uint16_t *dyr = static_cast<const uint16_t *>(a.dy.ptr) + it.b * a.dy.s0 + it.d * a.dy.s1;
    uint16_t *dxr = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dx.ptr)) +
                    it.b * a.dx.s0 + it.d * a.dx.s1;
    const int adx = A16 ? 16 : tc_align(dxr);
    const TcLoads<NTL, A16> lx(xr, a.T), ld(dyr, a.T);
    uint16_t lh[W - 1], rh_x = 0, rh_dy = 0;
    float w[W][1], bias[1];
    Raw<8> rx[kTcTilesBwd], rd[kTcTilesBwd], xtail, dtail;
    if (live) {
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int64_t p = it.t0 - (W - 1) + j;
            lh[j] = xr[p >= 0 ? p : 0];
        }
        const int64_t rq = min(it.t1 + lane, a.T - 1);
        rh_x = xr[rq];
        rh_dy = dyr[rq];
        load_filter<W, 1, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, it.d, w, bias);
#pragma unroll
        for (int c = 0; c < kTcTilesBwd; ++c) {
            const int64_t t = it.t0 + c * kTcTile + lane * kTcE;
            rx[c] = lx.load(t, it.t1);
            rd[c] = ld.load(t, it.t1);
        }
        xtail = lx.tail(it.t0 + kTcTilesBwd * kTcTile);
        dtail = ld.tail(it.t0 + kTcTilesBwd * kTcTile);
    }
    tcm_build<W, kTcTilesBwd, true>(it, ids, a.T, s_mask, s_rh);
    if (!live) return;
    float carry[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
        carry[j] = it.t0 - (W - 1) + j >= 0 ? bf16_bits_to_f32(lh[j]) : 0.0f;
    float dwacc[W], dbacc = 0.0f;
#pragma unroll
    for (int k = 0; k < W; ++k) dwacc[k] = 0.0f;

    // dx of the lane's tokens of the tile at tt from its g's and mask word,
    // and the W-1 g's and the mask word that follow the lane (`after`,
    // `after_m`: the next tile's lane 0, or the right halo's, for lane 63).
    // Term l of dx[i] is g of token i+l through its tap l, kept when token
    // i+l has token i's entry: bit 3(i+l) + l-1 of this lane's word, or of
    // the next lane's for i+l >= kTcE.
    auto emit = [&](int64_t tt, const float (&g)[kTcE], uint32_t mw, const float (&after)[W - 1],
                    uint32_t after_m) {
        float ge[kTcE + W - 1], v[kTcE];
#pragma unroll
        for (int i = 0; i < kTcE; ++i) ge[i] = g[i];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) ge[kTcE + j] = lane_down(g[j], after[j]);
        const uint32_t mn = static_cast<uint32_t>(
            lane_down_id(static_cast<int32_t>(mw), static_cast<int32_t>(after_m)));
        const int64_t t = tt + lane * kTcE;
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            float acc = 0.0f;
#pragma unroll
            for (int l = W - 1; l >= 0; --l) {
                const int u = i + l;  // the output token whose tap l meets token i
                float gv = ge[u];
                if (l > 0) gv = u < kTcE ? tcm_keep(gv, mw, 3 * u + l - 1)
                                         : tcm_keep(gv, mn, 3 * (u - kTcE) + l - 1);
                acc = l == W - 1 ? w[0][0] * gv : fmaf(w[W - 1 - l][0], gv, acc);
            }
            v[i] = acc;
        }
        if (t < it.t1) tc_store<true>(dxr, t, it.t1, v, adx);
    };

    float gprev[kTcE];
    uint32_t mprev = 0u;
    int64_t tprev = -1;
#pragma unroll
    for (int c = 0; c < kTcTilesBwd; ++c) {
        const int64_t tt = it.t0 + c * kTcTile;
        if (tt >= it.t1) break;
        const uint32_t mc = s_mask[c][lane];
        float v[kTcE], dyv[kTcE], xe[W - 1 + kTcE], g[kTcE];
        lx.fix(rx[c], c + 1 < kTcTilesBwd ? rx[c + 1 < kTcTilesBwd ? c + 1 : c] : xtail);
        ld.fix(rd[c], c + 1 < kTcTilesBwd ? rd[c + 1 < kTcTilesBwd ? c + 1 : c] : dtail);
        unpack<8>(rx[c], v);
        unpack<8>(rd[c], dyv);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) xe[j] = lane_up(v[kTcE - (W - 1) + j], carry[j]);
#pragma unroll
        for (int i = 0; i < kTcE; ++i) xe[W - 1 + i] = v[i];
#pragma unroll
        for (int i = 0; i < kTcE; ++i) {
            float xv[W];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int lag = W - 1 - k;
                xv[k] = lag == 0 ? xe[i + k] : tcm_keep(xe[i + k], mc, 3 * i + lag - 1);
            }
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) z = fmaf(w[k][0], xv[k], z);
            g[i] = dyv[i] * act_slope<SILU>(z);  // zero past the chunk (dy reads 0)
#pragma unroll
            for (int k = 0; k < W; ++k) dwacc[k] = fmaf(g[i], xv[k], dwacc[k]);
            if constexpr (BIAS) dbacc += g[i];
        }
        if (tprev >= 0) {
            float after[W - 1];
#pragma unroll
            for (int j = 0; j < W - 1; ++j) after[j] = from_lane(g[j], 0);
            emit(tprev, gprev, mprev,
                 after, static_cast<uint32_t>(from_lane_id(static_cast<int32_t>(mc), 0)));
        }
#pragma unroll
        for (int i = 0; i < kTcE; ++i) gprev[i] = g[i];
        mprev = mc;
        tprev = tt;
#pragma unroll
        for (int j = 0; j < W - 1; ++j) carry[j] = from_lane(v[kTcE - (W - 1) + j], kWaveSize - 1);
    }
    // Right halo: g at t1 .. t1+W-2 (zero past the row), in every lane; a
    // chunk that does not end the row is a whole number of tiles, so `carry`
    // holds the W-1 tokens before t1.
    {
        const uint32_t rh = s_rh;
        float xw[2 * (W - 1)], after[W - 1];
        const float hx = bf16_bits_to_f32(rh_x), hd = bf16_bits_to_f32(rh_dy);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            xw[j] = carry[j];
            xw[W - 1 + j] = from_lane(hx, j);
        }
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int lag = W - 1 - k;
                z = fmaf(w[k][0], lag == 0 ? xw[j + k] : tcm_keep(xw[j + k], rh, 3 * j + lag - 1),
                         z);
            }
            after[j] = it.t1 + j < a.T ? from_lane(hd, j) * act_slope<SILU>(z) : 0.0f;
        }
        emit(tprev, gprev, mprev, after, rh);
    }
    // dW/dB of the chunk: a wave sum, then one atomic or one partial per tap.
#pragma unroll
    for (int k = 0; k < W; ++k) dwacc[k] = wave_sum(dwacc[k]);
    if constexpr (BIAS) dbacc = wave_sum(dbacc);
    if (lane == 0) {
        if (a.partial) {
            const int64_t pidx = it.b * a.n_chunk + it.chunk;
            float *pr = a.partial + (pidx * a.D + it.d) * a.part_stride;
#pragma unroll
            for (int k = 0; k < W; ++k) pr[k] = dwacc[k];
            if (a.part_stride > W) pr[W] = dbacc;
        } else {
#pragma unroll
            for (int k = 0; k < W; ++k) atomicAdd(a.dw + it.d * W + k, dwacc[k]);
            if constexpr (BIAS) atomicAdd(a.db + it.d, dbacc);
        }
    }
}

template <int W, bool SILU, int FK>
__global__ __launch_bounds__(256) void k_fwd_tcs(FwdArgs a) {
    if constexpr (CCV_TCS_MASKS_FWD) {
        __shared__ uint32_t s_mask[kTcTilesFwd][kWaveSize];
        __shared__ uint32_t s_rh;
        TcItem it;
        bool live;
        tcm_item(a, it, live);
        const TcSeqIds ids = tc_seq_ids(a, it);
        tc_run(a, [&](auto ntl, auto a16) {
            fwd_tcm_chunk<W, SILU, FK, decltype(ntl)::value, decltype(a16)::value>(
                a, it, live, ids, s_mask, s_rh);
        });
    } else {
        TcItem it;
        if (!tc_item(a, it)) return;
        tc_run(a, [&](auto ntl, auto a16) {
            fwd_tcs_chunk<W, SILU, FK, decltype(ntl)::value, decltype(a16)::value>(
                a, it, tc_seq_ids(a, it));
        });
    }
}

template <int W, bool SILU, int FK>
__global__ __launch_bounds__(256) void k_bwd_tcs(BwdArgs a) {
    if constexpr (CCV_TCS_MASKS_BWD) {
        __shared__ uint32_t s_mask[kTcTilesBwd][kWaveSize];
        __shared__ uint32_t s_rh;
        TcItem it;
        bool live;
        tcm_item(a, it, live);
        const TcSeqIds ids = tc_seq_ids(a, it);
        tc_run(a, [&](auto ntl, auto a16) {
            bwd_tcm_chunk<W, SILU, FK, decltype(ntl)::value, decltype(a16)::value>(
                a, it, live, ids, s_mask, s_rh);
        });
    } else {
        TcItem it;
        if (!tc_item(a, it)) return;
        tc_run(a, [&](auto ntl, auto a16) {
            bwd_tcs_chunk<W, SILU, FK, decltype(ntl)::value, decltype(a16)::value>(
                a, it, tc_seq_ids(a, it));
        });
    }
}

// ===========================================================================
// Time lanes for packed rows (B = 1, unit stride along T)
//
// Two launches.  The first is the dense rows' chunk code unchanged: the
// row's initial state is sequence 0's, and it writes no final state and no
// state gradient.  The second repairs what the sequence boundaries change,
// with one lane per (channel, boundary): a boundary changes only the W-1
// tokens on either side of it.  So the tiles run at the dense code's
// registers, occupancy and speed, and the repair's stores come after the
// first launch's by stream order.  With at most 64 offsets the chunk launch
// validates them itself (every wave, see TcpCheck); otherwise the validation
// launch runs first.  The repair launch reads the flag word first and writes
// nothing when it is set.
//
// Forward, for a sequence j = [s, e): the outputs at s .. s+W-2 take their
// taps before s from the sequence's initial state (or zeros), and the
// repair writes the sequence's final state.
//
// Backward, at a boundary s between A = [sa, s) and B = [s, eb): A's last
// W-1 tokens get dx without B's gradients and with A's final-state
// gradient; B's first W-1 tokens get g, dx and their dW/dB terms from B's
// own taps, and the dense pass's terms for them are taken out again; dinit
// of B is worked out from those g's (plus, for a sequence shorter than W-1,
// the final-state gradient slots that are initial-state slots).  Boundary 0
// is the row's start (dinit of sequence 0) and boundary N its end (the last
// sequence's final-state gradient).  A wave's dW/dB terms are summed and
// added like a chunk's: by atomics, or as partial rows after the first
// launch's, in the order the fixed-order reduction reads them.
// ===========================================================================

// v[i] for 0 <= i < M, zero otherwise; i is known only at run time.
template <int M>
__device__ __forceinline__ float pick(const float (&v)[M], int64_t i) {
    float r = 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m) r = i == m ? v[m] : r;
    return r;
}

// Token p of a row of T, zero outside [0, T) (the load reads an in-row
// address either way).
__device__ __forceinline__ float tcp_tok(const uint16_t *row, int64_t p, int64_t T) {
    const uint16_t bits = row[p < 0 ? 0 : p >= T ? T - 1 : p];
    return p >= 0 && p < T ? bf16_bits_to_f32(bits) : 0.0f;
}

// The W-1 slots of sequence j, channel d, of a [N, D, W-1] state tensor
// (zeros without one).
template <int W>
__device__ __forceinline__ void tcp_slots(const Strided3 &st, int64_t j, int64_t d,
                                          float (&v)[W - 1]) {
    if (st.ptr) {
        const uint16_t *r = static_cast<const uint16_t *>(st.ptr) + j * st.s0 + d * st.s1;
#pragma unroll
        for (int m = 0; m < W - 1; ++m) v[m] = bf16_bits_to_f32(r[m * st.s2]);
    } else {
#pragma unroll
        for (int m = 0; m < W - 1; ++m) v[m] = 0.0f;
    }
}

// The sticky flag word (this call's validation, or an earlier call's).
__device__ __forceinline__ bool tcp_flag_set(const uint32_t *err) { return *err != 0u; }

// The repair launches' work item: a wave per (row r < rows, group g of 64
// lanes), and the lane's index j = 64 g + lane along the groups.  The
// backward's rows are channels and its lanes boundaries; the forward's rows
// are sequences and its lanes channels.
struct TcpItem {
    int64_t d, g, j;  // row, group, lane index
};
__device__ __forceinline__ bool tcp_item(int64_t rows, int64_t groups, TcpItem &it) {
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock +
                        __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    if (wid >= rows * groups) return false;
    it.d = wid / groups;
    it.g = wid - it.d * groups;
    it.j = it.g * kWaveSize + threadIdx.x % kWaveSize;
    return true;
}

// The packed chunk launch's check.  With the validation launch before it, a
// wave only reads the sticky flag word (and stops at once when it is set).
// With at most 64 offsets (cu_in_wave) the wave validates them itself, one
// per lane, loaded before the chunk's bulk loads and looked at after them:
// the conditions of the validation kernel, by two ballots and two lane
// reads; the launch's first wave publishes the bits into the word.  A wave
// writes nothing when the offsets are malformed or the word was set.
template <typename A>
struct TcpCheck {
    const A *a;
    bool first;           // the launch's first wave
    uint32_t sticky = 0;  // the flag word before the call
    int32_t cl = 0;       // cu_in_wave: lane l holds cu[min(l, N)]

    // false: stop now
    __device__ __forceinline__ bool start() {
        sticky = *a->err;
        if (!a->cu_in_wave) return sticky == 0u;
        cl = a->cu[min(static_cast<int64_t>(threadIdx.x % kWaveSize), a->n_seq)];
        return true;
    }

    __device__ __forceinline__ bool ok() const {
        if (!a->cu_in_wave) return true;
        const int64_t lane = threadIdx.x % kWaveSize, n = a->n_seq;
        const int32_t next = lane_down_id(cl, cl);  // lane l: cu[l+1]
        uint32_t bad = 0u;
        if (__ballot(lane < n && next < cl)) bad |= kDecreasing;
        if (__ballot(lane < n && next == cl)) bad |= kEmpty;
        if (__builtin_amdgcn_readlane(cl, 0) != 0) bad |= kFirstNonzero;
        if (static_cast<int64_t>(__builtin_amdgcn_readlane(cl, static_cast<int>(n))) != a->T)
            bad |= kLastMismatch;
        if (bad && first && lane == 0) atomicOr(a->err, bad);
        return (bad | sticky) == 0u;
    }
};

template <int W, bool SILU, int FK>
__global__ __launch_bounds__(256) void k_fwd_tcp(FwdArgs a) {
    TcItem it;
    if (!tc_item(a, it)) return;
    TcpCheck<FwdArgs> check{&a, it.b == 0 && it.d == 0 && it.chunk == 0};
    if (!check.start()) return;  // a set flag word: write nothing
    FwdArgs da = a;
    da.fin.ptr = nullptr;  // final states come from the repair
    tc_run(a, [&](auto ntl, auto a16) {
        fwd_tc_chunk<W, SILU, FK, decltype(ntl)::value, decltype(a16)::value>(da, it, check);
    });
}

// Forward repair: a wave per sequence j = [s, e) and group of 64 channels,
// lane l channel 64 g + l (the state reads and final-state writes of a
// wave are contiguous).
template <int W, bool SILU, int FK>
__global__ __launch_bounds__(256) void k_fwd_tcp_fix(FwdArgs a) {
    TcpItem it;
    if (!tcp_item(a.n_seq, (a.D + kWaveSize - 1) / kWaveSize, it)) return;
    if (tcp_flag_set(a.err)) return;
    const int64_t j = it.d, d = it.j;  // (item row, lane) = (sequence, channel)
    if (d >= a.D) return;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x.ptr) + d * a.x.s1;
    uint16_t *yr = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.y.ptr)) + d * a.y.s1;
    const int64_t s = a.cu[j], e = a.cu[j + 1];
    float w[W][1], bias[1];
    load_filter<W, 1, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, d, w, bias);
    if (j > 0) {
        // x_ext of sequence j at s-(W-1) .. s+W-2
        float st[W - 1], xe[2 * (W - 1)];
        tcp_slots<W>(a.init, j, d, st);
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            xe[i] = st[i];
            xe[W - 1 + i] = s + i < e ? tcp_tok(xr, s + i, a.T) : 0.0f;
        }
#pragma unroll
        for (int l = 0; l < W - 1; ++l) {
            if (s + l < e) {
                float z = bias[0];
#pragma unroll
                for (int k = 0; k < W; ++k) z = fmaf(w[k][0], xe[l + k], z);
                yr[s + l] = to_bf16_bits(act<SILU>(z));
            }
        }
    }
    if (a.fin.ptr) {
        // the sequence's last W-1 extended tokens, bit for bit
        const uint16_t *ir = a.init.ptr ? static_cast<const uint16_t *>(a.init.ptr) +
                                              j * a.init.s0 + d * a.init.s1
                                        : nullptr;
        uint16_t *fr = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.fin.ptr)) +
                       j * a.fin.s0 + d * a.fin.s1;
#pragma unroll
        for (int m = 0; m < W - 1; ++m) {
            const int64_t p = e - (W - 1) + m;
            uint16_t bits = 0;
            if (p >= s) bits = xr[p];
            else if (ir) bits = ir[(p - s + W - 1) * a.init.s2];
            fr[m * a.fin.s2] = bits;
        }
    }
}

template <int W, bool SILU, int FK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CCV_TC_BWD_WAVES)))
void k_bwd_tcp(BwdArgs a) {
    TcItem it;
    if (!tc_item(a, it)) return;
    TcpCheck<BwdArgs> check{&a, it.b == 0 && it.d == 0 && it.chunk == 0};
    if (!check.start()) return;  // a set flag word: write nothing
    BwdArgs da = a;
    da.dfin.ptr = nullptr;  // the state gradients come from the repair
    da.dinit.ptr = nullptr;
    tc_run(a, [&](auto ntl, auto a16) {
        bwd_tc_chunk<W, SILU, FK, decltype(ntl)::value, decltype(a16)::value>(da, it, check);
    });
}

// Backward repair of boundary j (s = cu[j]) in one lane, adding its dW/dB
// terms to the lane's sums.
template <int W, bool SILU, int FK>
__device__ __forceinline__ void bwd_tcp_boundary(const BwdArgs &a, int64_t d, int64_t j,
                                                 const float (&w)[W][1], const float (&bias)[1],
                                                 float (&dwacc)[W], float &dbacc) {
    constexpr bool BIAS = fk_bias(FK);
    const int64_t n = a.n_seq, T = a.T;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x.ptr) + d * a.x.s1;
    const uint16_t *dyr = static_cast<const uint16_t *>(a.dy.ptr) + d * a.dy.s1;
    uint16_t *dxr = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dx.ptr)) + d * a.dx.s1;
    const bool has_a = j > 0, has_b = j < n;
    const int64_t s = a.cu[j], sa = a.cu[has_a ? j - 1 : j], eb = a.cu[has_b ? j + 1 : j];
    // x at s-2(W-1) .. s+2(W-1)-1, dy at s-(W-1) .. s+2(W-1)-1, the
    // initial-state slots of A, B and sequence 0, the final-state gradients
    // of A and B (zeros for what the call does not have)
    float X[4 * (W - 1)], Dy[3 * (W - 1)];
#pragma unroll
    for (int i = 0; i < 4 * (W - 1); ++i) X[i] = tcp_tok(xr, s - 2 * (W - 1) + i, T);
#pragma unroll
    for (int i = 0; i < 3 * (W - 1); ++i) Dy[i] = tcp_tok(dyr, s - (W - 1) + i, T);
    float ia[W - 1], ib[W - 1], i0[W - 1], fa[W - 1], fb[W - 1];
    tcp_slots<W>(a.init, has_a ? j - 1 : 0, d, ia);
    tcp_slots<W>(a.init, has_b ? j : 0, d, ib);
    tcp_slots<W>(a.init, 0, d, i0);
    tcp_slots<W>(a.dfin, has_a ? j - 1 : 0, d, fa);
    tcp_slots<W>(a.dfin, has_b ? j : 0, d, fb);

    if (has_a) {
        // A's last W-1 tokens u = s-(W-1)+i (those at or after sa)
        float ga[W - 1];
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            const int64_t u = s - (W - 1) + i;
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int64_t p = u - (W - 1) + k;
                z = fmaf(w[k][0], p >= sa ? X[i + k] : pick(ia, p - sa + W - 1), z);
            }
            ga[i] = u >= sa ? Dy[i] * act_slope<SILU>(z) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            const int64_t u = s - (W - 1) + i;
            if (u >= sa) {
                float acc = 0.0f;
#pragma unroll
                for (int m = W - 2; m >= 0; --m)
                    if (i + m < W - 1) acc = fmaf(w[W - 1 - m][0], ga[i + m], acc);
                dxr[u] = to_bf16_bits(acc + fa[i]);
            }
        }
    }
    if (has_b) {
        // B's first 2(W-1) tokens v = s+i, with B's taps (zero from eb on)
        float gb[2 * (W - 1)];
#pragma unroll
        for (int i = 0; i < 2 * (W - 1); ++i) {
            float z = bias[0];
#pragma unroll
            for (int k = 0; k < W; ++k)
                z = fmaf(w[k][0], i + k >= W - 1 ? X[i + k + W - 1] : ib[i + k], z);
            gb[i] = s + i < eb ? Dy[i + W - 1] * act_slope<SILU>(z) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            const int64_t v = s + i;
            if (v < eb) {
                float acc = w[0][0] * gb[i + W - 1];
#pragma unroll
                for (int m = W - 2; m >= 0; --m) acc = fmaf(w[W - 1 - m][0], gb[i + m], acc);
                dxr[v] = to_bf16_bits(acc + pick(fb, v - (eb - (W - 1))));
                if (has_a) {
                    // take out the dense pass's dW/dB terms of v (its taps were
                    // the row's tokens, or sequence 0's state before the row)
                    // and put in B's
                    float zd = bias[0], xd[W];
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        const int64_t p = v - (W - 1) + k;
                        xd[k] = p >= 0 ? X[i + k + W - 1] : pick(i0, p + W - 1);
                        zd = fmaf(w[k][0], xd[k], zd);
                    }
                    const float gd = Dy[i + W - 1] * act_slope<SILU>(zd);
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        const float xb = i + k >= W - 1 ? X[i + k + W - 1] : ib[i + k];
                        dwacc[k] = fmaf(gb[i], xb, dwacc[k]);
                        dwacc[k] = fmaf(-gd, xd[k], dwacc[k]);
                    }
                    if constexpr (BIAS) dbacc += gb[i] - gd;
                }
            }
        }
        if (a.dinit.ptr) {
            uint16_t *di = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dinit.ptr)) +
                           j * a.dinit.s0 + d * a.dinit.s1;
#pragma unroll
            for (int m = 0; m < W - 1; ++m) {
                // dx_ext at s-(W-1)+m: the g's at s+m-k for k <= m, plus a
                // final-state slot that lands there
                float acc = w[0][0] * gb[m];
#pragma unroll
                for (int k = W - 2; k >= 0; --k)
                    if (m - (W - 1) + k >= 0) acc = fmaf(w[W - 1 - k][0], gb[m - (W - 1) + k], acc);
                di[m * a.dinit.s2] = to_bf16_bits(acc + pick(fb, m - (eb - s)));
            }
        }
    }
}

// Backward repair: lane j is boundary j in [0, N].  Boundary 0 needs work
// only for dinit, boundary N only for a final-state gradient.
template <int W, bool SILU, int FK>
__global__ __launch_bounds__(256) void k_bwd_tcp_fix(BwdArgs a) {
    constexpr bool BIAS = fk_bias(FK);
    TcpItem it;
    if (!tcp_item(a.D, (a.n_seq + kWaveSize) / kWaveSize, it)) return;
    if (tcp_flag_set(a.err)) return;
    const int64_t j = it.j, d = it.d, n = a.n_seq;
    float w[W][1], bias[1];
    load_filter<W, 1, FK>(a.w, a.w_sd, a.w_sk, a.bias, a.b_s, d, w, bias);
    float dwacc[W], dbacc = 0.0f;
#pragma unroll
    for (int k = 0; k < W; ++k) dwacc[k] = 0.0f;
    if (j <= n && (j > 0 || a.dinit.ptr) && (j < n || a.dfin.ptr))
        bwd_tcp_boundary<W, SILU, FK>(a, d, j, w, bias, dwacc, dbacc);
    // the wave's dW/dB terms, like a chunk's
#pragma unroll
    for (int k = 0; k < W; ++k) dwacc[k] = wave_sum(dwacc[k]);
    if constexpr (BIAS) dbacc = wave_sum(dbacc);
    if (threadIdx.x % kWaveSize == 0) {
        if (a.partial) {
            float *pr = a.partial + ((a.n_chunk + it.g) * a.D + d) * a.part_stride;
#pragma unroll
            for (int k = 0; k < W; ++k) pr[k] = dwacc[k];
            if (a.part_stride > W) pr[W] = dbacc;
        } else {
#pragma unroll
            for (int k = 0; k < W; ++k) atomicAdd(a.dw + d * W + k, dwacc[k]);
            if constexpr (BIAS) atomicAdd(a.db + d, dbacc);
        }
    }
}

// ===========================================================================
// Single-token update (in place on the [B,D,W-1] state)
//
// One lane per VEC channels of one batch row.  With VEC = 8 the host has
// verified unit channel strides, a contiguous [B,D,W-1] state, a contiguous
// [D,W] filter and 16-byte alignment, so a lane's state is 3 x 16 contiguous
// bytes and every load below is issued before the first wait.
// ===========================================================================
#ifndef CCV_UPD_MAX_WAVES
#define CCV_UPD_MAX_WAVES 4
#endif
#ifndef CCV_UPD_NT
#define CCV_UPD_NT 0
#endif
#ifndef CCV_UPD_ROWS
#define CCV_UPD_ROWS 2          // batch rows an 8-channel update lane serves
#endif
#ifndef CCV_UPD_STAGED
#define CCV_UPD_STAGED 1        // coalesced (LDS-staged) update when D % 512 == 0
#endif
// Cache policy of the staged update's accesses (bits): 1 = non-temporal
// state loads, 2 = non-temporal state stores, 4 = non-temporal token loads.
// Measured on the decode shape with cold states (interleaved runs): all
// three 6.8 us, state loads and stores 7.3 us, state stores alone 8.4 us,
// none 8.6 us.
#ifndef CCV_UPD_STAGED_NT
#define CCV_UPD_STAGED_NT 7
#endif
// ... and from this many (row, channel) pairs (12 MiB of update traffic at
// width 4).  Measured with cold states: the staged kernel loses about 0.5 us
// to the plain one up to 1 MB, 0.1 us at 8 MB, and wins 0.15 us at 16 MB and
// 0.7 us at 34 MB (its LDS round trips lengthen a launch-bound kernel, and
// shorten the L2 request stream of a bandwidth-bound one).
#ifndef CCV_UPD_STAGED_MIN_BD
#define CCV_UPD_STAGED_MIN_BD (int64_t(3) << 18)
#endif

// Per-lane pieces of the 8-channel update, shared by both kernels below.
// Filter taps and bias of 8 channels from their raw 16-byte vectors (the
// bias has the filter's dtype).
template <int W, bool WF32>
struct UpdVecs {
    static constexpr int kState = 8 * (W - 1) / 8;           // 16-byte vectors of state
    static constexpr int kFilter = 8 * W * (WF32 ? 4 : 2) / 16;
    static constexpr int kBias = WF32 ? 2 : 1;
};

template <int W, bool WF32>
__device__ __forceinline__ void upd_unpack_filter(
    const u32x4_t (&wv)[UpdVecs<W, WF32>::kFilter], const u32x4_t (&bv)[UpdVecs<W, WF32>::kBias],
    float (&w)[W][8], float (&bias)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const int e2 = c * W + k;
            if constexpr (WF32) {
                w[k][c] = __uint_as_float(wv[e2 / 4][e2 % 4]);
            } else {
                const uint32_t word = wv[e2 / 8][(e2 % 8) / 2];
                w[k][c] = (e2 % 2) ? hi_bf16(word) : lo_bf16(word);
            }
        }
        if constexpr (WF32) bias[c] = __uint_as_float(bv[c / 4][c % 4]);
        else bias[c] = (c % 2) ? hi_bf16(bv[0][c / 2]) : lo_bf16(bv[0][c / 2]);
    }
}

// One row of 8 channels: y from the state (s_0 .. s_{W-2}) and the token x,
// and the new state (s_1 .. s_{W-2}, x) as raw bits (a copy, never re-rounded).
template <int W, bool SILU, bool WF32>
__device__ __forceinline__ void upd_row(const float (&w)[W][8], const float (&bias)[8],
                                        const u32x4_t (&sv)[UpdVecs<W, WF32>::kState],
                                        const u32x4_t &xv, float (&out)[8],
                                        u32x4_t (&nv)[UpdVecs<W, WF32>::kState]) {
    constexpr int VEC = 8;
    uint16_t st[VEC][W - 1], xr[VEC];
#pragma unroll
    for (int e2 = 0; e2 < VEC * (W - 1); ++e2)
        st[e2 / (W - 1)][e2 % (W - 1)] =
            static_cast<uint16_t>(sv[e2 / 8][(e2 % 8) / 2] >> (16 * (e2 % 2)));
#pragma unroll
    for (int c = 0; c < VEC; ++c) xr[c] = static_cast<uint16_t>(xv[c / 2] >> (16 * (c % 2)));
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
        float z = bias[c];
#pragma unroll
        for (int k = 0; k < W - 1; ++k) z = fmaf(w[k][c], bf16_bits_to_f32(st[c][k]), z);
        z = fmaf(w[W - 1][c], bf16_bits_to_f32(xr[c]), z);
        out[c] = act<SILU>(z);
    }
#pragma unroll
    for (int i = 0; i < VEC * (W - 1) / 2; ++i) {
        uint16_t h[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e2 = 2 * i + q, c = e2 / (W - 1), j = e2 % (W - 1);
            h[q] = j < W - 2 ? st[c][j + 1] : xr[c];
        }
        nv[i / 4][i % 4] = static_cast<uint32_t>(h[0]) | (static_cast<uint32_t>(h[1]) << 16);
    }
}

// The register budget of up to CCV_UPD_MAX_WAVES waves per SIMD leaves room
// for every load of a lane to be in flight at once.  With 8 channels per lane
// the host has verified unit channel strides, a contiguous [B,D,W-1] state, a
// contiguous [D,W] filter and bias, and 16-byte alignment: a lane's state is
// 3 x 16 contiguous bytes.  A lane serves RPL batch rows of the same
// channels, so their filter and bias are loaded once.
template <int W, bool SILU, bool WF32, bool BIAS, int RPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, CCV_UPD_MAX_WAVES)))
void k_update_vec(UpdArgs a) {
    using V = UpdVecs<W, WF32>;
    constexpr int VEC = 8;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t rg = gid / a.n_lane_per_row;
    if (rg >= a.n_row_groups) return;
    const int64_t c0 = (gid % a.n_lane_per_row) * VEC;
    const int64_t b0 = rg * RPL;

    // Every load first: filter, bias, then each row's state and token.
    const u32x4_t *wq = reinterpret_cast<const u32x4_t *>(
        static_cast<const char *>(a.w) + c0 * W * (WF32 ? 4 : 2));
    u32x4_t wv[V::kFilter], bv[V::kBias];
#pragma unroll
    for (int i = 0; i < V::kFilter; ++i) wv[i] = wq[i];
#pragma unroll
    for (int i = 0; i < V::kBias; ++i) bv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (BIAS) {
        const u32x4_t *bq = reinterpret_cast<const u32x4_t *>(
            static_cast<const char *>(a.bias) + c0 * (WF32 ? 4 : 2));
#pragma unroll
        for (int i = 0; i < V::kBias; ++i) bv[i] = bq[i];
    }
    u32x4_t sv[RPL][V::kState], xv[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        if (b0 + r >= a.B) break;
        const u32x4_t *sq = reinterpret_cast<const u32x4_t *>(
            static_cast<const uint16_t *>(a.state) + (b0 + r) * a.s_sb + c0 * (W - 1));
#pragma unroll
        for (int i = 0; i < V::kState; ++i)
            sv[r][i] = CCV_UPD_NT ? __builtin_nontemporal_load(sq + i) : sq[i];
        const u32x4_t *xq = reinterpret_cast<const u32x4_t *>(
            static_cast<const uint16_t *>(a.x) + (b0 + r) * a.x_sb + c0);
        xv[r] = CCV_UPD_NT ? __builtin_nontemporal_load(xq) : *xq;
    }

    float w[W][VEC], bias[VEC];
    upd_unpack_filter<W, WF32>(wv, bv, w, bias);
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        if (b0 + r >= a.B) break;
        float out[VEC];
        u32x4_t nv[V::kState];
        upd_row<W, SILU, WF32>(w, bias, sv[r], xv[r], out, nv);
        store_vec<VEC, true>(static_cast<uint16_t *>(a.y) + (b0 + r) * a.y_sb + c0, 1, out);
        u32x4_t *sq = reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(a.state) +
                                                  (b0 + r) * a.s_sb + c0 * (W - 1));
#pragma unroll
        for (int i = 0; i < V::kState; ++i) {
            if (CCV_UPD_NT) __builtin_nontemporal_store(nv[i], sq + i);
            else sq[i] = nv[i];
        }
    }
}

// The same update with every global access coalesced: a wave owns 512
// consecutive channels (the host has verified D % 512 == 0, so a wave never
// straddles two row groups), and its state rows and filter are contiguous
// byte ranges.  Lane l loads the 16-byte vectors l, l + 64, ... of each range
// (each wave-wide load is 1 KB contiguous), the vectors pass through LDS to
// the lane that owns their channels, and the new state goes back the same
// way.  The four waves of a block take the same 512 channels of four
// consecutive row groups, so the block loads their filter once.  (The
// strided per-lane form touches every 128-byte line of a range with each of
// its loads.)
template <int W, bool SILU, bool WF32, bool BIAS, int RPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, CCV_UPD_MAX_WAVES)))
void k_update_staged(UpdArgs a) {
    using V = UpdVecs<W, WF32>;
    constexpr int VEC = 8;
    constexpr int kFiltVecs = kWaveSize * V::kFilter;  // the block's filter, 16-byte vectors
    __shared__ u32x4_t s_state[kWavesPerBlock][RPL][kWaveSize * V::kState];
    __shared__ u32x4_t s_filt[kFiltVecs];
    const int wave = threadIdx.x / kWaveSize, lane = threadIdx.x % kWaveSize;
    const int64_t ranges = a.n_lane_per_row / kWaveSize;   // 512-channel ranges per row
    const int64_t cb = blockIdx.x % ranges;
    const int64_t rg = (blockIdx.x / ranges) * kWavesPerBlock + wave;
    // Uniform over the wave; waves past the end still reach every barrier.
    const bool live = rg < a.n_row_groups;
    const int64_t cw = cb * (kWaveSize * VEC);  // the block's first channel
    const int64_t b0 = rg * RPL;

    const u32x4_t *wq = reinterpret_cast<const u32x4_t *>(
        static_cast<const char *>(a.w) + cw * W * (WF32 ? 4 : 2));
    constexpr int kPerThread = (kFiltVecs + 255) / 256;
    u32x4_t fv[kPerThread], bv[V::kBias], sv[RPL][V::kState], xv[RPL];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
        if (threadIdx.x + 256 * i < kFiltVecs) fv[i] = wq[threadIdx.x + 256 * i];
#pragma unroll
    for (int i = 0; i < V::kBias; ++i) bv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (live) {
        if constexpr (BIAS) {
            const u32x4_t *bq = reinterpret_cast<const u32x4_t *>(
                static_cast<const char *>(a.bias) + (cw + lane * VEC) * (WF32 ? 4 : 2));
#pragma unroll
            for (int i = 0; i < V::kBias; ++i) bv[i] = bq[i];
        }
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            if (b0 + r >= a.B) break;
            const u32x4_t *sq = reinterpret_cast<const u32x4_t *>(
                static_cast<const uint16_t *>(a.state) + (b0 + r) * a.s_sb + cw * (W - 1));
#pragma unroll
            for (int i = 0; i < V::kState; ++i) {
                if constexpr (CCV_UPD_STAGED_NT & 1)
                    sv[r][i] = __builtin_nontemporal_load(sq + lane + kWaveSize * i);
                else
                    sv[r][i] = sq[lane + kWaveSize * i];
            }
            const u32x4_t *xq = reinterpret_cast<const u32x4_t *>(
                static_cast<const uint16_t *>(a.x) + (b0 + r) * a.x_sb + cw + lane * VEC);
            if constexpr (CCV_UPD_STAGED_NT & 4) xv[r] = __builtin_nontemporal_load(xq);
            else xv[r] = *xq;
        }
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
        if (threadIdx.x + 256 * i < kFiltVecs) s_filt[threadIdx.x + 256 * i] = fv[i];
    if (live) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            if (b0 + r >= a.B) break;
#pragma unroll
            for (int i = 0; i < V::kState; ++i) s_state[wave][r][lane + kWaveSize * i] = sv[r][i];
        }
    }
    __syncthreads();
    float w[W][VEC], bias[VEC];
    u32x4_t nv[RPL][V::kState];
    if (live) {
        u32x4_t wv[V::kFilter];
#pragma unroll
        for (int i = 0; i < V::kFilter; ++i) wv[i] = s_filt[lane * V::kFilter + i];
        upd_unpack_filter<W, WF32>(wv, bv, w, bias);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            if (b0 + r >= a.B) break;
            u32x4_t own[V::kState];
#pragma unroll
            for (int i = 0; i < V::kState; ++i) own[i] = s_state[wave][r][lane * V::kState + i];
            float out[VEC];
            upd_row<W, SILU, WF32>(w, bias, own, xv[r], out, nv[r]);
            store_vec<VEC, true>(static_cast<uint16_t *>(a.y) + (b0 + r) * a.y_sb + cw +
                                     lane * VEC, 1, out);
        }
    }
    __syncthreads();  // every lane has read its slice before it is overwritten
    if (live) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            if (b0 + r >= a.B) break;
#pragma unroll
            for (int i = 0; i < V::kState; ++i) s_state[wave][r][lane * V::kState + i] = nv[r][i];
        }
    }
    __syncthreads();
    if (live) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            if (b0 + r >= a.B) break;
            u32x4_t *sq = reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(a.state) +
                                                      (b0 + r) * a.s_sb + cw * (W - 1));
#pragma unroll
            for (int i = 0; i < V::kState; ++i) {
                if constexpr (CCV_UPD_STAGED_NT & 2)
                    __builtin_nontemporal_store(s_state[wave][r][lane + kWaveSize * i],
                                                sq + lane + kWaveSize * i);
                else
                    sq[lane + kWaveSize * i] = s_state[wave][r][lane + kWaveSize * i];
            }
        }
    }
}

// Any strides: one lane per channel of one row; the row's L tokens in
// order, the state in registers until the end.
template <int W, bool SILU, bool WF32, bool BIAS>
__global__ __launch_bounds__(256) void k_update_any(UpdArgs a) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t b = gid / a.n_lane_per_row;
    if (b >= a.B) return;
    const int64_t c = gid % a.n_lane_per_row;
    const uint16_t *xp = static_cast<const uint16_t *>(a.x) + b * a.x_sb + c * a.x_sd;
    uint16_t *yp = static_cast<uint16_t *>(a.y) + b * a.y_sb + c * a.y_sd;
    uint16_t *sp = static_cast<uint16_t *>(a.state) + b * a.s_sb + c * a.s_sd;
    uint16_t st[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) st[j] = sp[j * a.s_sj];
    float w[W], bias = 0.0f;
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const int64_t off = c * a.w_sd + k * a.w_sk;
        w[k] = WF32 ? static_cast<const float *>(a.w)[off]
                    : bf16_bits_to_f32(static_cast<const uint16_t *>(a.w)[off]);
    }
    if constexpr (BIAS)
        bias = WF32 ? static_cast<const float *>(a.bias)[c * a.b_s]
                    : bf16_bits_to_f32(static_cast<const uint16_t *>(a.bias)[c * a.b_s]);
    for (int64_t l = 0; l < a.L; ++l) {
        const uint16_t xr = xp[l * a.x_st];
        float z = bias;
#pragma unroll
        for (int k = 0; k < W; ++k) z = fmaf(w[k], bf16_bits_to_f32(k < W - 1 ? st[k] : xr), z);
        yp[l * a.y_st] = to_bf16_bits(act<SILU>(z));
#pragma unroll
        for (int j = 0; j < W - 2; ++j) st[j] = st[j + 1];
        st[W - 2] = xr;
    }
#pragma unroll
    for (int j = 0; j < W - 1; ++j) sp[j * a.s_sj] = st[j];
}

// Several tokens per row (x [B,D,L], L > 1) on 8-channel lanes: the state
// window stays in registers (raw bits) across the row's tokens and is written
// once at the end.  The lane's state (W-1 16-byte vectors), its filter and
// bias vectors and the first 8 tokens are all requested before the first
// wait; later tokens follow in batches of 8.  Token loads, output stores and
// state stores are non-temporal, state loads are not: measured on 8 calls of
// 8 tokens at B=256 D=8192 (cold), 20.3 us against 20.5 (state stores
// cached too), 22.4 (all four non-temporal) and 23.8 (none); the scalar
// state accesses and batches of 4 tokens before, 22.0 us.
#ifndef CCV_UPD_TOK_STAGED
#define CCV_UPD_TOK_STAGED 1
#endif
#ifndef CCV_UPD_TOK_NT
#define CCV_UPD_TOK_NT 14  // non-temporal: 1 state loads, 2 state stores, 4 token loads, 8 outputs
#endif
template <int W, bool SILU, bool WF32, bool BIAS>
__global__ __launch_bounds__(256) void k_update_tokens(UpdArgs a) {
    using V = UpdVecs<W, WF32>;
    constexpr int VEC = 8, U = 8;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t b = gid / a.n_lane_per_row;
    if (b >= a.B) return;
    const int64_t c0 = (gid % a.n_lane_per_row) * VEC;
    const uint16_t *xb = static_cast<const uint16_t *>(a.x) + b * a.x_sb + c0;
    uint16_t *yb = static_cast<uint16_t *>(a.y) + b * a.y_sb + c0;
    u32x4_t *sq = reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(a.state) + b * a.s_sb +
                                              c0 * (W - 1));
    // With whole waves per row (D % 512 == 0) the wave's state is one
    // contiguous range: lane l moves its vectors l, l + 64, ..., and the
    // lanes swap them through the wave's LDS slice (LDS operations of a
    // wave complete in order, so no barrier is needed).  8 calls of 8
    // tokens at B=256 D=8192: 20.3 -> 19.5 us (state loads non-temporal
    // too: 19.9 us).
    __shared__ u32x4_t s_st[kWavesPerBlock][kWaveSize * V::kState];
    const int wave = threadIdx.x / kWaveSize, lane = threadIdx.x % kWaveSize;
    const bool staged = CCV_UPD_TOK_STAGED && a.n_lane_per_row % kWaveSize == 0;
    u32x4_t *wsq = sq - lane * V::kState;  // the wave's first state vector (when staged)
    u32x4_t sv[V::kState];
#pragma unroll
    for (int i = 0; i < V::kState; ++i) {
        u32x4_t *p = staged ? wsq + lane + kWaveSize * i : sq + i;
        sv[i] = (CCV_UPD_TOK_NT & 1) ? __builtin_nontemporal_load(p) : *p;
    }
    const u32x4_t *wq = reinterpret_cast<const u32x4_t *>(
        static_cast<const char *>(a.w) + c0 * W * (WF32 ? 4 : 2));
    u32x4_t wv[V::kFilter], bv[V::kBias];
#pragma unroll
    for (int i = 0; i < V::kFilter; ++i) wv[i] = wq[i];
#pragma unroll
    for (int i = 0; i < V::kBias; ++i) bv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (BIAS) {
        const u32x4_t *bq = reinterpret_cast<const u32x4_t *>(
            static_cast<const char *>(a.bias) + c0 * (WF32 ? 4 : 2));
#pragma unroll
        for (int i = 0; i < V::kBias; ++i) bv[i] = bq[i];
    }
    Raw<VEC> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (u < a.L) raw[u] = load_raw<VEC, (CCV_UPD_TOK_NT & 4) != 0>(xb + u * a.x_st, 1);

    float w[W][VEC], bias[VEC];
    upd_unpack_filter<W, WF32>(wv, bv, w, bias);
    if (staged) {
#pragma unroll
        for (int i = 0; i < V::kState; ++i) s_st[wave][lane + kWaveSize * i] = sv[i];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < V::kState; ++i) sv[i] = s_st[wave][lane * V::kState + i];
    }
    // state element (c, j) is 16-bit word c*(W-1) + j of the lane's vectors
    uint16_t st[VEC][W - 1];
#pragma unroll
    for (int c = 0; c < VEC; ++c)
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int e = c * (W - 1) + j;
            st[c][j] = static_cast<uint16_t>(sv[e / 8][(e % 8) / 2] >> (16 * (e % 2)));
        }
    auto step = [&](int64_t l, const Raw<VEC> &r) {
        uint16_t xr[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) xr[c] = static_cast<uint16_t>(r.v[c / 2] >> (16 * (c % 2)));
        float out[VEC];
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            float z = bias[c];
#pragma unroll
            for (int k = 0; k < W - 1; ++k) z = fmaf(w[k][c], bf16_bits_to_f32(st[c][k]), z);
            z = fmaf(w[W - 1][c], bf16_bits_to_f32(xr[c]), z);
            out[c] = act<SILU>(z);
        }
        store_vec<VEC, (CCV_UPD_TOK_NT & 8) != 0>(yb + l * a.y_st, 1, out);
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
#pragma unroll
            for (int j = 0; j < W - 2; ++j) st[c][j] = st[c][j + 1];
            st[c][W - 2] = xr[c];
        }
    };
    for (int64_t l = 0; l < a.L; l += U) {
        if (l > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (l + u < a.L)
                    raw[u] = load_raw<VEC, (CCV_UPD_TOK_NT & 4) != 0>(xb + (l + u) * a.x_st, 1);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (l + u < a.L) step(l + u, raw[u]);
    }
    u32x4_t nv[V::kState];
#pragma unroll
    for (int i = 0; i < V::kState; ++i) nv[i] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < VEC; ++c)
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            const int e = c * (W - 1) + j;
            nv[e / 8][(e % 8) / 2] |= static_cast<uint32_t>(st[c][j]) << (16 * (e % 2));
        }
    if (staged) {
#pragma unroll
        for (int i = 0; i < V::kState; ++i) s_st[wave][lane * V::kState + i] = nv[i];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < V::kState; ++i) nv[i] = s_st[wave][lane + kWaveSize * i];
    }
#pragma unroll
    for (int i = 0; i < V::kState; ++i) {
        u32x4_t *p = staged ? wsq + lane + kWaveSize * i : sq + i;
        if (CCV_UPD_TOK_NT & 2) __builtin_nontemporal_store(nv[i], p);
        else *p = nv[i];
    }
}

// ===========================================================================
// Small kernels
// ===========================================================================
__global__ __launch_bounds__(256) void k_validate(const int32_t *cu, int64_t n_seq, int64_t total,
                                                  uint32_t *flags, int overwrite) {
    __shared__ uint32_t s_bad;
    if (threadIdx.x == 0) s_bad = 0u;
    __syncthreads();
    uint32_t bad = 0u;
    for (int64_t i = threadIdx.x; i < n_seq; i += blockDim.x) {
        const int32_t x0 = cu[i], x1 = cu[i + 1];
        if (x1 < x0) bad |= kDecreasing;
        if (x1 == x0) bad |= kEmpty;
    }
    if (threadIdx.x == 0) {
        if (cu[0] != 0) bad |= kFirstNonzero;
        if (static_cast<int64_t>(cu[n_seq]) != total) bad |= kLastMismatch;
    }
    if (bad) atomicOr(&s_bad, bad);
    __syncthreads();
    if (threadIdx.x == 0) {
        if (overwrite) *flags = s_bad;
        else if (s_bad) atomicOr(flags, s_bad);
    }
}

// Fixed-order reduction of unique partials [P][D][kp] into dw[d][k] (k < W)
// and, with kp = W+1, db[d].  The P partials of every element are split into
// 16 groups (4 waves x 4 accumulators): group q sums p = q, q+16, q+32, ...
// in increasing p, then the 16 group sums are added in increasing q.  The
// order depends on P only, never on scheduling, so the result is the same
// bits run to run.
//
// A lane owns V consecutive elements (V = 4: one 16-byte load per partial,
// when the element count is a multiple of 4; else V = 1), a block 64 lanes'
// columns.  Each lane issues the loads of 8 partials per group (32 loads)
// before it adds any, so a block keeps its whole share of the partials in
// flight at once; a last partial round (P not a multiple of 128) loads from
// indices clamped into range and adds only the partials that exist.  The
// lane's dweight/dbias values are read before the partials, so that their
// update does not wait for one more memory round trip.
//
// `err` is the packed call's flag word (nullptr for dense rows).  When it is
// non-zero the backward blocks wrote no partials, so the reduction adds
// nothing either: dweight and dbias keep their values.  The word is read once
// per block and shared through LDS, so the whole block takes one branch.
template <int V> struct RedVec;
template <> struct RedVec<4> { typedef float T __attribute__((ext_vector_type(4))); };
template <> struct RedVec<1> { typedef float T; };

// The register budget of at most 2 waves per SIMD lets every load of a lane
// be in flight together (a higher occupancy target makes the scheduler wait
// on each load before the next).
template <int V>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_dw_reduce(const float *part, int64_t n_part,
                                                   int64_t n_ch, int w, int kp, float *dw,
                                                   float *db, const uint32_t *err) {
    using T = typename RedVec<V>::T;
    constexpr int kAcc = 4, kGroups = kWavesPerBlock * kAcc, kUnroll = 8;
    __shared__ T s_acc[kGroups][kWaveSize];
    __shared__ uint32_t s_err;
    if (err != nullptr) {
        if (threadIdx.x == 0)
            s_err = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (s_err != 0u) return;  // uniform over the block
    }
    const int lane = threadIdx.x % kWaveSize, wave = threadIdx.x / kWaveSize;
    const int64_t n_vec = n_ch * kp / V;
    const int64_t c = static_cast<int64_t>(blockIdx.x) * kWaveSize + lane;
    // wave 0 writes the sums: element e = c*V + i is (channel e / kp, tap e % kp)
    float *dst[V];
    float old[V];
    if (wave == 0 && c < n_vec) {
        int64_t ch = c * V / kp;
        int k = static_cast<int>(c * V - ch * kp);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            dst[i] = k < w ? dw + ch * w + k : db + ch;
            old[i] = *dst[i];
            if (++k == kp) {
                k = 0;
                ++ch;
            }
        }
    }
    T acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = T{};
    if (c < n_vec) {
        const T *col = reinterpret_cast<const T *>(part) + c;
        int64_t p0 = 0;
        for (; p0 + kGroups * kUnroll <= n_part; p0 += kGroups * kUnroll) {
            T v[kUnroll][kAcc];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int j = 0; j < kAcc; ++j)
                    v[u][j] = col[(p0 + u * kGroups + wave * kAcc + j) * n_vec];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int j = 0; j < kAcc; ++j) acc[j] += v[u][j];
        }
        if (p0 < n_part) {
            // the last, partial round: same order, absent partials skipped
            T v[kUnroll][kAcc];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int j = 0; j < kAcc; ++j) {
                    const int64_t p = p0 + u * kGroups + wave * kAcc + j;
                    v[u][j] = col[(p < n_part ? p : n_part - 1) * n_vec];
                }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int j = 0; j < kAcc; ++j)
                    if (p0 + u * kGroups + wave * kAcc + j < n_part) acc[j] += v[u][j];
        }
    }
#pragma unroll
    for (int j = 0; j < kAcc; ++j) s_acc[wave * kAcc + j][lane] = acc[j];
    __syncthreads();
    if (wave != 0 || c >= n_vec) return;
    T sum = T{};
#pragma unroll
    for (int q = 0; q < kGroups; ++q) sum += s_acc[q][lane];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        float v;
        if constexpr (V == 1) v = sum;
        else v = sum[i];
        *dst[i] = old[i] + v;
    }
}

// A stream value that never names a real stream: dispatch without launching.
hipStream_t const kQueryStream = reinterpret_cast<hipStream_t>(~uintptr_t(0));

// `lds` bytes of dynamic LDS (unused by the kernel) cap the blocks that fit
// on one CU, i.e. the kernel's occupancy.
template <typename K, typename A>
hipError_t launch(K kernel, int64_t blocks, const A &args, hipStream_t s, unsigned lds = 0) {
    if (blocks <= 0) return hipSuccess;
    if (blocks > int64_t(UINT32_MAX)) return hipErrorInvalidConfiguration;  // beyond one grid
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), lds, s, args);
    return hipGetLastError();
}

}  // namespace
}  // namespace ccv

// ccv_kernels.hip — gfx950 kernels of the depthwise causal conv1d.
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
#include <hip/hip_runtime.h>

#include "ccv_internal.h"

namespace ccv {
namespace {

constexpr int W = kWidth;
constexpr uint32_t kFirstNonzero = 0x1u, kLastMismatch = 0x2u, kDecreasing = 0x4u,
                   kEmpty = 0x8u;

#ifndef CCV_FWD_UNROLL
#define CCV_FWD_UNROLL 8
#endif
#ifndef CCV_BWD_UNROLL
#define CCV_BWD_UNROLL 4
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

// VEC channels of one token as raw BF16 bits.
template <int VEC> struct Raw;
template <> struct Raw<8> { uint4 v; };
template <> struct Raw<1> { uint16_t v; };

template <int VEC>
__device__ __forceinline__ Raw<VEC> load_raw(const uint16_t *p, int64_t sd);
template <>
__device__ __forceinline__ Raw<8> load_raw<8>(const uint16_t *p, int64_t) {
    return Raw<8>{*reinterpret_cast<const uint4 *>(p)};
}
template <>
__device__ __forceinline__ Raw<1> load_raw<1>(const uint16_t *p, int64_t) {
    return Raw<1>{*p};
}

template <int VEC>
__device__ __forceinline__ void unpack(const Raw<VEC> &r, float (&v)[VEC]);
template <>
__device__ __forceinline__ void unpack<8>(const Raw<8> &r, float (&v)[8]) {
    v[0] = lo_bf16(r.v.x); v[1] = hi_bf16(r.v.x);
    v[2] = lo_bf16(r.v.y); v[3] = hi_bf16(r.v.y);
    v[4] = lo_bf16(r.v.z); v[5] = hi_bf16(r.v.z);
    v[6] = lo_bf16(r.v.w); v[7] = hi_bf16(r.v.w);
}
template <>
__device__ __forceinline__ void unpack<1>(const Raw<1> &r, float (&v)[1]) {
    v[0] = bf16_bits_to_f32(r.v);
}

template <int VEC>
__device__ __forceinline__ void store_vec(uint16_t *p, int64_t sd, const float (&v)[VEC]);
template <>
__device__ __forceinline__ void store_vec<8>(uint16_t *p, int64_t, const float (&v)[8]) {
    uint4 r;
    r.x = pack2_bf16(v[0], v[1]);
    r.y = pack2_bf16(v[2], v[3]);
    r.z = pack2_bf16(v[4], v[5]);
    r.w = pack2_bf16(v[6], v[7]);
    *reinterpret_cast<uint4 *>(p) = r;
}
template <>
__device__ __forceinline__ void store_vec<1>(uint16_t *p, int64_t, const float (&v)[1]) {
    *p = to_bf16_bits(v[0]);
}

// ---------------------------------------------------------------------------
// Activation and its slope.  SiLU(z) = z * s, s = 1 / (1 + e^-z);
// SiLU'(z) = s * (1 + z (1 - s)).  One v_exp_f32 and one v_rcp_f32 each.
// ---------------------------------------------------------------------------
template <bool SILU>
__device__ __forceinline__ float act(float z) {
    if constexpr (SILU) return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
    else return z;
}
template <bool SILU>
__device__ __forceinline__ float act_slope(float z) {
    if constexpr (SILU) {
        float s = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
        return s * fmaf(z, 1.0f - s, 1.0f);
    } else {
        return 1.0f;
    }
}

// Block id -> logical tile id such that XCD x (hardware dispatches block i
// to XCD i % 8) receives one contiguous range of logical tiles.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nb) {
    constexpr int64_t X = 8;
    const int64_t q = nb / X, r = nb % X;
    const int64_t x = bid % X, j = bid / X;
    return x * q + (x < r ? x : r) + j;
}

// Filter taps and bias of a lane's VEC channels, widened to FP32.
// `wvec`: the host found the filter contiguous [D,W] and 16-byte aligned.
template <int VEC>
__device__ __forceinline__ void load_filter(const void *wp, int64_t sd, int64_t sk, int wf32,
                                            int wvec, const void *bp, int64_t bs, int64_t c0,
                                            float (&w)[W][VEC], float (&bias)[VEC]) {
    if (wf32) {
        const float *p = static_cast<const float *>(wp);
        if (VEC == 8 && wvec) {
            const float4 *q = reinterpret_cast<const float4 *>(p + c0 * W);
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                float4 t = q[c];
                w[0][c] = t.x; w[1][c] = t.y; w[2][c] = t.z; w[3][c] = t.w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c)
#pragma unroll
                for (int k = 0; k < W; ++k) w[k][c] = p[(c0 + c) * sd + k * sk];
        }
    } else {
        const uint16_t *p = static_cast<const uint16_t *>(wp);
        if (VEC == 8 && wvec) {
            const uint2 *q = reinterpret_cast<const uint2 *>(p + c0 * W);
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                uint2 t = q[c];
                w[0][c] = lo_bf16(t.x); w[1][c] = hi_bf16(t.x);
                w[2][c] = lo_bf16(t.y); w[3][c] = hi_bf16(t.y);
            }
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c)
#pragma unroll
                for (int k = 0; k < W; ++k) w[k][c] = bf16_bits_to_f32(p[(c0 + c) * sd + k * sk]);
        }
    }
#pragma unroll
    for (int c = 0; c < VEC; ++c)
        bias[c] = bp ? bf16_bits_to_f32(static_cast<const uint16_t *>(bp)[(c0 + c) * bs]) : 0.0f;
}

// z = bias + sum_k w[k] * v[k] with v = (win[0..W-2], cur), FP32 fused.
template <int VEC>
__device__ __forceinline__ float preact(const float (&w)[W][VEC], const float (&bias)[VEC],
                                        const float (&win)[W - 1][VEC], const float (&cur)[VEC],
                                        int c) {
    float z = bias[c];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) z = fmaf(w[k][c], win[k][c], z);
    return fmaf(w[W - 1][c], cur[c], z);
}

template <int VEC>
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
// row, else from the initial state (slot p - s + W - 1), else zeros.
template <int VEC>
__device__ __forceinline__ void load_left_halo(const uint16_t *xb, int64_t xs_d, int64_t xs_t,
                                               const Strided3 &init, int64_t r, int64_t s,
                                               int64_t ta, int64_t c0, float (&win)[W - 1][VEC]) {
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int64_t p = ta - (W - 1) + j;
        if (p >= s) {
            unpack<VEC>(load_raw<VEC>(xb + p * xs_t, xs_d), win[j]);
        } else if (init.ptr) {
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

// cu_seqlens staged in LDS and validated there (the whole array, by every
// block, so no block depends on another).  Returns the violation bits of
// this call ORed with the sticky flag word; block 0 publishes its bits.
__device__ __forceinline__ uint32_t stage_and_validate(const int32_t *cu, int64_t n_seq,
                                                       int64_t total, uint32_t *err,
                                                       int32_t *s_cu, uint32_t *s_bad,
                                                       int in_lds, bool publish) {
    const int tid = threadIdx.x;
    if (tid == 0) *s_bad = 0u;
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
        if (bad) atomicOr(s_bad, bad);
    }
    __syncthreads();
    bad = *s_bad;
    if (publish && tid == 0 && bad) atomicOr(err, bad);
    // The word may hold bits of an earlier call (sticky) or, when the
    // offsets did not fit in LDS, of the validation kernel run just before.
    const uint32_t prior = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return bad | prior;
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
template <int VEC, bool SILU>
__device__ __forceinline__ void fwd_piece(const FwdArgs &a, int64_t b, int64_t r, int64_t s,
                                          int64_t e, int64_t ta, int64_t tb, int64_t c0,
                                          const float (&w)[W][VEC], const float (&bias)[VEC]) {
    constexpr int U = CCV_FWD_UNROLL;
    const uint16_t *xb = static_cast<const uint16_t *>(a.x.ptr) + b * a.x.s0 + c0 * a.x.s1;
    uint16_t *yb = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.y.ptr)) + b * a.y.s0 +
                   c0 * a.y.s1;
    const int64_t xs_t = a.x.s2, ys_t = a.y.s2;
    float win[W - 1][VEC];
    load_left_halo<VEC>(xb, a.x.s1, xs_t, a.init, r, s, ta, c0, win);

    int64_t t = ta;
    for (; t + U <= tb; t += U) {
        Raw<VEC> raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = load_raw<VEC>(xb + (t + u) * xs_t, a.x.s1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float cur[VEC], out[VEC];
            unpack<VEC>(raw[u], cur);
#pragma unroll
            for (int c = 0; c < VEC; ++c) out[c] = act<SILU>(preact<VEC>(w, bias, win, cur, c));
            store_vec<VEC>(yb + (t + u) * ys_t, a.y.s1, out);
            shift_in<VEC>(win, cur);
        }
    }
    for (; t < tb; ++t) {
        float cur[VEC], out[VEC];
        unpack<VEC>(load_raw<VEC>(xb + t * xs_t, a.x.s1), cur);
#pragma unroll
        for (int c = 0; c < VEC; ++c) out[c] = act<SILU>(preact<VEC>(w, bias, win, cur, c));
        store_vec<VEC>(yb + t * ys_t, a.y.s1, out);
        shift_in<VEC>(win, cur);
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

template <int VEC, bool SILU, bool PACKED>
__global__ __launch_bounds__(256) void k_fwd_chan(FwdArgs a) {
    __shared__ int32_t s_cu[PACKED ? kLdsCuMax : 1];
    __shared__ uint32_t s_bad;
    const int64_t tile = xcd_remap(blockIdx.x, a.n_block);
    const int64_t bt = tile % a.n_tblk;
    const int64_t g = (tile / a.n_tblk) % a.n_group;
    const int64_t b = tile / (a.n_tblk * a.n_group);
    const int wave = threadIdx.x / kWaveSize, lane = threadIdx.x % kWaveSize;

    if constexpr (PACKED) {
        if (stage_and_validate(a.cu, a.n_seq, a.T, a.err, s_cu, &s_bad, a.cu_in_lds,
                               blockIdx.x == 0))
            return;  // malformed or sticky: write nothing
    }
    const int64_t t0 = (bt * kWavesPerBlock + wave) * a.L;
    const int64_t c0 = g * (kWaveSize * VEC) + lane * VEC;
    if (t0 >= a.T || c0 >= a.D) return;
    const int64_t t1 = min(t0 + a.L, a.T);

    float w[W][VEC], bias[VEC];
    load_filter<VEC>(a.w, a.w_sd, a.w_sk, a.w_f32, a.w_vec, a.bias, a.b_s, c0, w, bias);

    if constexpr (!PACKED) {
        fwd_piece<VEC, SILU>(a, b, b, 0, a.T, t0, t1, c0, w, bias);
    } else {
        const int32_t *cu = a.cu_in_lds ? s_cu : a.cu;
        for (int64_t i = find_row(cu, a.n_seq, t0); i < a.n_seq; ++i) {
            const int64_t s = cu[i], e = cu[i + 1];
            if (s >= t1) break;
            fwd_piece<VEC, SILU>(a, 0, i, s, e, s > t0 ? s : t0, e < t1 ? e : t1, c0, w, bias);
        }
    }
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
template <int VEC, bool SILU, bool BIAS>
struct BwdLane {
    float w[W][VEC], bias[VEC];
    float dw[W][VEC], db[VEC];
};

template <int VEC, bool SILU, bool BIAS>
__device__ __forceinline__ void bwd_piece(const BwdArgs &a, BwdLane<VEC, SILU, BIAS> &L,
                                          int64_t b, int64_t r, int64_t s, int64_t e,
                                          int64_t ta, int64_t tb, int64_t c0) {
    constexpr int U = CCV_BWD_UNROLL;
    const uint16_t *xb = static_cast<const uint16_t *>(a.x.ptr) + b * a.x.s0 + c0 * a.x.s1;
    const uint16_t *dyb = static_cast<const uint16_t *>(a.dy.ptr) + b * a.dy.s0 + c0 * a.dy.s1;
    uint16_t *dxb = const_cast<uint16_t *>(static_cast<const uint16_t *>(a.dx.ptr)) +
                    b * a.dx.s0 + c0 * a.dx.s1;
    const int64_t xs_d = a.x.s1, xs_t = a.x.s2, ys_d = a.dy.s1, ys_t = a.dy.s2;
    const int64_t ds_d = a.dx.s1, ds_t = a.dx.s2;

    float xw[W - 1][VEC], gw[W - 1][VEC];
    load_left_halo<VEC>(xb, xs_d, xs_t, a.init, r, s, ta, c0, xw);
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
    auto grad_step = [&](const float (&cur)[VEC], const float (&dyv)[VEC], float (&gcur)[VEC],
                         bool count) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            const float z = preact<VEC>(L.w, L.bias, xw, cur, c);
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
    // Fully checked step (head and tail of a piece).
    auto generic_step = [&](int64_t tau) {
        float gcur[VEC];
        if (tau < e) {
            float cur[VEC], dyv[VEC];
            unpack<VEC>(load_raw<VEC>(xb + tau * xs_t, xs_d), cur);
            unpack<VEC>(load_raw<VEC>(dyb + tau * ys_t, ys_d), dyv);
            grad_step(cur, dyv, gcur, tau < tb);
            shift_in<VEC>(xw, cur);
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

    // Head: tau in [ta, ta + W-1).
#pragma unroll
    for (int h = 0; h < W - 1; ++h) generic_step(ta + h);
    // Body: tau in [ta + W-1, tb): inside the row, emits dx[tau-(W-1)] with
    // no final-state term (tau - (W-1) < e - (W-1)).
    int64_t tau = ta + (W - 1);
    for (; tau + U <= tb; tau += U) {
        Raw<VEC> rx[U], rd[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            rx[u] = load_raw<VEC>(xb + (tau + u) * xs_t, xs_d);
            rd[u] = load_raw<VEC>(dyb + (tau + u) * ys_t, ys_d);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float cur[VEC], dyv[VEC], gcur[VEC], v[VEC];
            unpack<VEC>(rx[u], cur);
            unpack<VEC>(rd[u], dyv);
            grad_step(cur, dyv, gcur, true);
            shift_in<VEC>(xw, cur);
            emit_value(gcur, v);
            store_vec<VEC>(dxb + (tau + u - (W - 1)) * ds_t, ds_d, v);
            shift_g(gcur);
        }
    }
    for (; tau < tb; ++tau) {
        float cur[VEC], dyv[VEC], gcur[VEC], v[VEC];
        unpack<VEC>(load_raw<VEC>(xb + tau * xs_t, xs_d), cur);
        unpack<VEC>(load_raw<VEC>(dyb + tau * ys_t, ys_d), dyv);
        grad_step(cur, dyv, gcur, true);
        shift_in<VEC>(xw, cur);
        emit_value(gcur, v);
        store_vec<VEC>(dxb + (tau - (W - 1)) * ds_t, ds_d, v);
        shift_g(gcur);
    }
    // Tail: tau in [max(tb, ta + W-1), tb + W-1).
    for (tau = tb > ta + (W - 1) ? tb : ta + (W - 1); tau < tb + (W - 1); ++tau) generic_step(tau);
}

template <int VEC, bool SILU, bool PACKED, bool BIAS>
__global__ __launch_bounds__(256) void k_bwd_chan(BwdArgs a) {
    constexpr int CH = kWaveSize * VEC;  // channels of a block
    // One LDS buffer: the staged offsets during the walk, then the dW/dB
    // reduction (a barrier separates the two uses).
    constexpr int kRed = kWavesPerBlock * (W + 1) * (CH + 1);
    constexpr int kBuf = (PACKED && kLdsCuMax > kRed) ? kLdsCuMax : kRed;
    __shared__ float s_buf[kBuf];
    __shared__ uint32_t s_bad;
    int32_t *s_cu = reinterpret_cast<int32_t *>(s_buf);
    float (*s_red)[W + 1][CH + 1] = reinterpret_cast<float (*)[W + 1][CH + 1]>(s_buf);
    const int64_t tile = xcd_remap(blockIdx.x, a.n_block);
    const int64_t bt = tile % a.n_tblk;
    const int64_t g = (tile / a.n_tblk) % a.n_group;
    const int64_t b = tile / (a.n_tblk * a.n_group);
    const int wave = threadIdx.x / kWaveSize, lane = threadIdx.x % kWaveSize;

    if constexpr (PACKED) {
        if (stage_and_validate(a.cu, a.n_seq, a.T, a.err, s_cu, &s_bad, a.cu_in_lds,
                               blockIdx.x == 0))
            return;  // uniform over the block: no barrier is left waiting
    }
    const int64_t t0 = (bt * kWavesPerBlock + wave) * a.L;
    const int64_t c0 = g * CH + lane * VEC;

    BwdLane<VEC, SILU, BIAS> L;
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
#pragma unroll
        for (int k = 0; k < W; ++k) L.dw[k][c] = 0.0f;
        L.db[c] = 0.0f;
    }
    if (t0 < a.T && c0 < a.D) {
        const int64_t t1 = min(t0 + a.L, a.T);
        load_filter<VEC>(a.w, a.w_sd, a.w_sk, a.w_f32, a.w_vec, a.bias, a.b_s, c0, L.w, L.bias);
        if constexpr (!PACKED) {
            bwd_piece<VEC, SILU, BIAS>(a, L, b, b, 0, a.T, t0, t1, c0);
        } else {
            const int32_t *cu = a.cu_in_lds ? s_cu : a.cu;
            for (int64_t i = find_row(cu, a.n_seq, t0); i < a.n_seq; ++i) {
                const int64_t s = cu[i], e = cu[i + 1];
                if (s >= t1) break;
                bwd_piece<VEC, SILU, BIAS>(a, L, 0, i, s, e, s > t0 ? s : t0, e < t1 ? e : t1, c0);
            }
        }
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
    const int64_t pidx = b * a.n_tblk + bt;
    for (int i = threadIdx.x; i < CH * W; i += blockDim.x) {
        const int ch = i / W, k = i % W;
        if (ch0 + ch >= a.D) continue;
        float v = s_red[0][k][ch];
#pragma unroll
        for (int q = 1; q < kWavesPerBlock; ++q) v += s_red[q][k][ch];
        if (a.partial) a.partial[(pidx * a.D + ch0 + ch) * W + k] = v;
        else atomicAdd(a.dw + (ch0 + ch) * W + k, v);
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
// Single-token update (in place on the [B,D,W-1] state)
// ===========================================================================
template <int VEC, bool SILU>
__global__ __launch_bounds__(256) void k_update(UpdArgs a) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t b = gid / a.n_lane_per_row;
    if (b >= a.B) return;
    const int64_t c0 = (gid % a.n_lane_per_row) * VEC;

    float w[W][VEC], bias[VEC];
    load_filter<VEC>(a.w, a.w_sd, a.w_sk, a.w_f32, a.w_vec, a.bias, a.b_s, c0, w, bias);
    const uint16_t *xp = static_cast<const uint16_t *>(a.x) + b * a.x_sb + c0 * a.x_sd;
    uint16_t *sp = static_cast<uint16_t *>(a.state) + b * a.s_sb + c0 * a.s_sd;
    uint16_t *yp = static_cast<uint16_t *>(a.y) + b * a.y_sb + c0 * a.y_sd;

    // Raw bits: the shifted state is a copy, never re-rounded.
    uint16_t st[VEC][W - 1], xr[VEC];
    // VEC == 8: the host verified unit channel strides, a contiguous
    // [B,D,W-1] state and 16-byte alignment of every row.
    if constexpr (VEC == 8) {
        // The lane's VEC*(W-1) state values are contiguous: 3 x 16 bytes.
        const uint4 *q = reinterpret_cast<const uint4 *>(sp);
        uint32_t words[VEC * (W - 1) / 2];
#pragma unroll
        for (int i = 0; i < VEC * (W - 1) / 8; ++i) {
            uint4 t = q[i];
            words[4 * i] = t.x; words[4 * i + 1] = t.y; words[4 * i + 2] = t.z; words[4 * i + 3] = t.w;
        }
#pragma unroll
        for (int e2 = 0; e2 < VEC * (W - 1); ++e2)
            st[e2 / (W - 1)][e2 % (W - 1)] = static_cast<uint16_t>(words[e2 / 2] >> (16 * (e2 % 2)));
    } else {
#pragma unroll
        for (int c = 0; c < VEC; ++c)
#pragma unroll
            for (int j = 0; j < W - 1; ++j) st[c][j] = sp[c * a.s_sd + j * a.s_sj];
    }
    if constexpr (VEC == 8) {
        uint4 t = *reinterpret_cast<const uint4 *>(xp);
        const uint32_t words[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int c = 0; c < VEC; ++c) xr[c] = static_cast<uint16_t>(words[c / 2] >> (16 * (c % 2)));
    } else {
#pragma unroll
        for (int c = 0; c < VEC; ++c) xr[c] = xp[c * a.x_sd];
    }

    float out[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
        float z = bias[c];
#pragma unroll
        for (int k = 0; k < W - 1; ++k) z = fmaf(w[k][c], bf16_bits_to_f32(st[c][k]), z);
        z = fmaf(w[W - 1][c], bf16_bits_to_f32(xr[c]), z);
        out[c] = act<SILU>(z);
    }
    if constexpr (VEC == 8) {
        store_vec<VEC>(yp, 1, out);
    } else {
#pragma unroll
        for (int c = 0; c < VEC; ++c) yp[c * a.y_sd] = to_bf16_bits(out[c]);
    }
    // New state (s_1 .. s_{W-2}, x).
    uint16_t ns[VEC][W - 1];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
#pragma unroll
        for (int j = 0; j < W - 2; ++j) ns[c][j] = st[c][j + 1];
        ns[c][W - 2] = xr[c];
    }
    if constexpr (VEC == 8) {
        uint32_t words[VEC * (W - 1) / 2];
#pragma unroll
        for (int i = 0; i < VEC * (W - 1) / 2; ++i) {
            const int e0 = 2 * i, e1 = 2 * i + 1;
            words[i] = static_cast<uint32_t>(ns[e0 / (W - 1)][e0 % (W - 1)]) |
                       (static_cast<uint32_t>(ns[e1 / (W - 1)][e1 % (W - 1)]) << 16);
        }
        uint4 *q = reinterpret_cast<uint4 *>(sp);
#pragma unroll
        for (int i = 0; i < VEC * (W - 1) / 8; ++i)
            q[i] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
    } else {
#pragma unroll
        for (int c = 0; c < VEC; ++c)
#pragma unroll
            for (int j = 0; j < W - 1; ++j) sp[c * a.s_sd + j * a.s_sj] = ns[c][j];
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

// Fixed-order reduction of unique partials: out[e] += sum_{p=0}^{P-1} part[p][e],
// always in increasing p, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void k_dw_reduce(const float *part, int64_t n_part,
                                                   int64_t n_elem, float *out) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= n_elem) return;
    float acc = 0.0f;
    for (int64_t p = 0; p < n_part; ++p) acc += part[p * n_elem + e];
    out[e] += acc;
}

template <typename K, typename A>
hipError_t launch(K kernel, int64_t blocks, const A &args, hipStream_t s) {
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, int vec, int silu, int packed, hipStream_t s) {
#define CCV_FWD(V, S, P) \
    if (vec == V && !!silu == S && !!packed == P) return launch(k_fwd_chan<V, S, P>, a.n_block, a, s);
    CCV_FWD(8, true, false) CCV_FWD(8, true, true) CCV_FWD(8, false, false) CCV_FWD(8, false, true)
    CCV_FWD(1, true, false) CCV_FWD(1, true, true) CCV_FWD(1, false, false) CCV_FWD(1, false, true)
#undef CCV_FWD
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs &a, int vec, int silu, int packed, hipStream_t s) {
    const bool bias = a.db != nullptr;
#define CCV_BWD(V, S, P, B)                                            \
    if (vec == V && !!silu == S && !!packed == P && bias == B) \
        return launch(k_bwd_chan<V, S, P, B>, a.n_block, a, s);
    CCV_BWD(8, true, false, true) CCV_BWD(8, true, false, false)
    CCV_BWD(8, true, true, true) CCV_BWD(8, true, true, false)
    CCV_BWD(8, false, false, true) CCV_BWD(8, false, false, false)
    CCV_BWD(8, false, true, true) CCV_BWD(8, false, true, false)
    CCV_BWD(1, true, false, true) CCV_BWD(1, true, false, false)
    CCV_BWD(1, true, true, true) CCV_BWD(1, true, true, false)
    CCV_BWD(1, false, false, true) CCV_BWD(1, false, false, false)
    CCV_BWD(1, false, true, true) CCV_BWD(1, false, true, false)
#undef CCV_BWD
    return hipErrorInvalidValue;
}

hipError_t launch_update(const UpdArgs &a, int vec, int silu, hipStream_t s) {
    const int64_t lanes = a.B * a.n_lane_per_row;
    const int64_t blocks = (lanes + 255) / 256;
    if (vec == 8) return silu ? launch(k_update<8, true>, blocks, a, s) : launch(k_update<8, false>, blocks, a, s);
    if (vec == 1) return silu ? launch(k_update<1, true>, blocks, a, s) : launch(k_update<1, false>, blocks, a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_validate(const int32_t *cu, int64_t n_seq, int64_t total, uint32_t *flags,
                           int overwrite, hipStream_t s) {
    hipLaunchKernelGGL(k_validate, dim3(1), dim3(256), 0, s, cu, n_seq, total, flags, overwrite);
    return hipGetLastError();
}

hipError_t launch_dw_reduce(const float *partial, int64_t n_part, int64_t n_elem, float *out,
                            hipStream_t s) {
    const int64_t blocks = (n_elem + 255) / 256;
    hipLaunchKernelGGL(k_dw_reduce, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, partial,
                       n_part, n_elem, out);
    return hipGetLastError();
}

}  // namespace ccv

// ccv_dispatch.h — host-side selection of the kernel instance for one filter
// width W (a template argument here; ccv_width.hip instantiates it for each
// width the library is built for).
#pragma once

#include "ccv_device.h"

namespace ccv {
namespace {

// Filter kind of an argument block (see FilterKind).
template <typename A>
int filter_kind(const A &a) {
    if (a.w_f32) return a.bias != nullptr ? kF32Bias : kF32;
    return a.bias != nullptr ? kBf16Bias : kBf16;
}

template <typename K>
int64_t capacity_of(K kernel, unsigned lds) {
    return resident_blocks(reinterpret_cast<const void *>(kernel), lds);
}

template <int W, int V, bool S, int P, int F, bool Q>
hipError_t fwd_one(const FwdArgs &a, hipStream_t s, int64_t *cap) {
    if constexpr (P == kRowsSeq && Q) {
        return hipErrorInvalidValue;  // seq_idx rows have no pipelined body
    } else {
        constexpr unsigned lds = Q ? CCV_FWD_PIPE_DYN_LDS : 0;
        if (cap) *cap = capacity_of(k_fwd_chan<W, V, S, P, F, Q>, lds);
        if (s == kQueryStream) return hipSuccess;
        return launch(k_fwd_chan<W, V, S, P, F, Q>, a.n_block, a, s, lds);
    }
}

template <int W, int V, bool Q>
hipError_t fwd_vec(const FwdArgs &a, int silu, int rows, int fk, hipStream_t s, int64_t *cap) {
#define CCV_FWD(S, P, F) \
    if (!!silu == S && rows == P && fk == F) return fwd_one<W, V, S, P, F, Q>(a, s, cap);
#define CCV_FWD_K(S, P) \
    CCV_FWD(S, P, kBf16) CCV_FWD(S, P, kBf16Bias) CCV_FWD(S, P, kF32) CCV_FWD(S, P, kF32Bias)
    CCV_FWD_K(true, kRowsDense) CCV_FWD_K(true, kRowsPacked) CCV_FWD_K(false, kRowsDense)
    CCV_FWD_K(false, kRowsPacked)
    if constexpr (!Q) {
        CCV_FWD_K(true, kRowsSeq) CCV_FWD_K(false, kRowsSeq)
    }
#undef CCV_FWD_K
#undef CCV_FWD
    return hipErrorInvalidValue;
}

// The software-pipelined forward is built for 8-channel lanes of dense and
// packed rows only.
// Time-lane kernels: dense rows, packed rows (the dense code, then a repair
// at the sequence boundaries) and seq_idx rows (per-token ids).
// Blocks of a packed rows' repair launch: a wave per row and group of 64
// lanes over `items` (backward: channels x boundaries; forward: sequences x
// channels).
inline int64_t tcp_blocks(int64_t rows, int64_t items) {
    return (rows * ((items + kWaveSize - 1) / kWaveSize) + kWavesPerBlock - 1) / kWavesPerBlock;
}

template <int W>
hipError_t fwd_tc(const FwdArgs &a, int silu, int fk, int rows, hipStream_t s) {
#define CCV_TC(S, F)                                                                    \
    if (!!silu == S && fk == F) {                                                       \
        if (rows == kRowsDense) return launch(k_fwd_tc<W, S, F>, a.n_block, a, s);       \
        if (rows == kRowsPacked) {                                                      \
            const hipError_t e = launch(k_fwd_tcp<W, S, F>, a.n_block, a, s);           \
            if (e != hipSuccess) return e;                                              \
            return launch(k_fwd_tcp_fix<W, S, F>, tcp_blocks(a.n_seq, a.D), a, s);       \
        }                                                                               \
        if (rows == kRowsSeq) return launch(k_fwd_tcs<W, S, F>, a.n_block, a, s);        \
    }
    CCV_TC(true, kBf16) CCV_TC(true, kBf16Bias) CCV_TC(true, kF32) CCV_TC(true, kF32Bias)
    CCV_TC(false, kBf16) CCV_TC(false, kBf16Bias) CCV_TC(false, kF32) CCV_TC(false, kF32Bias)
#undef CCV_TC
    return hipErrorInvalidValue;
}

template <int W>
hipError_t bwd_tc(const BwdArgs &a, int silu, int fk, int rows, hipStream_t s) {
#define CCV_TC(S, F)                                                                    \
    if (!!silu == S && fk == F) {                                                       \
        if (rows == kRowsDense) return launch(k_bwd_tc<W, S, F>, a.n_block, a, s);       \
        if (rows == kRowsPacked) {                                                      \
            const hipError_t e = launch(k_bwd_tcp<W, S, F>, a.n_block, a, s);           \
            if (e != hipSuccess) return e;                                              \
            return launch(k_bwd_tcp_fix<W, S, F>, tcp_blocks(a.D, a.n_seq + 1), a, s);   \
        }                                                                               \
        if (rows == kRowsSeq) return launch(k_bwd_tcs<W, S, F>, a.n_block, a, s);        \
    }
    CCV_TC(true, kBf16) CCV_TC(true, kBf16Bias) CCV_TC(true, kF32) CCV_TC(true, kF32Bias)
    CCV_TC(false, kBf16) CCV_TC(false, kBf16Bias) CCV_TC(false, kF32) CCV_TC(false, kF32Bias)
#undef CCV_TC
    return hipErrorInvalidValue;
}

template <int W>
hipError_t fwd_dispatch(const FwdArgs &a, int vec, int silu, int rows, hipStream_t s,
                        int64_t *cap) {
    const int fk = filter_kind(a);
    if (vec == kVecTime) {
        if (cap) *cap = 0;
        if (s == kQueryStream) return hipSuccess;
        return fwd_tc<W>(a, silu, fk, rows, s);
    }
    if (vec == 8 && a.pipe && rows != kRowsSeq)
        return fwd_vec<W, 8, true>(a, silu, rows, fk, s, cap);
    if (vec == 8) return fwd_vec<W, 8, false>(a, silu, rows, fk, s, cap);
    if (vec == 4) return fwd_vec<W, 4, false>(a, silu, rows, fk, s, cap);
    if (vec == 1) return fwd_vec<W, 1, false>(a, silu, rows, fk, s, cap);
    return hipErrorInvalidValue;
}

template <int W, int V, bool S, int P, int F>
hipError_t bwd_one(const BwdArgs &a, hipStream_t s, int64_t *cap) {
    if (cap) *cap = capacity_of(k_bwd_chan<W, V, S, P, F>, CCV_BWD_DYN_LDS);
    if (s == kQueryStream) return hipSuccess;
    return launch(k_bwd_chan<W, V, S, P, F>, a.n_block, a, s, CCV_BWD_DYN_LDS);
}

template <int W, int V>
hipError_t bwd_vec(const BwdArgs &a, int silu, int rows, int fk, hipStream_t s, int64_t *cap) {
#define CCV_BWD(S, P, F) \
    if (!!silu == S && rows == P && fk == F) return bwd_one<W, V, S, P, F>(a, s, cap);
#define CCV_BWD_K(S, P) \
    CCV_BWD(S, P, kBf16) CCV_BWD(S, P, kBf16Bias) CCV_BWD(S, P, kF32) CCV_BWD(S, P, kF32Bias)
    CCV_BWD_K(true, kRowsDense) CCV_BWD_K(true, kRowsPacked) CCV_BWD_K(true, kRowsSeq)
    CCV_BWD_K(false, kRowsDense) CCV_BWD_K(false, kRowsPacked) CCV_BWD_K(false, kRowsSeq)
#undef CCV_BWD_K
#undef CCV_BWD
    return hipErrorInvalidValue;
}

// Backward lanes own 4 channels (or 1): with 8, the window, gradient window
// and dW accumulators leave too few registers for latency hiding.
template <int W>
hipError_t bwd_dispatch(const BwdArgs &a, int vec, int silu, int rows, hipStream_t s,
                        int64_t *cap) {
    const int fk = filter_kind(a);
    if (vec == kVecTime) {
        if (cap) *cap = 0;
        if (s == kQueryStream) return hipSuccess;
        return bwd_tc<W>(a, silu, fk, rows, s);
    }
    if (vec == 4) return bwd_vec<W, 4>(a, silu, rows, fk, s, cap);
    if (vec == 1) return bwd_vec<W, 1>(a, silu, rows, fk, s, cap);
    return hipErrorInvalidValue;
}

template <int W>
hipError_t update_dispatch(const UpdArgs &a, int vec, int silu, hipStream_t s) {
    const bool wf32 = a.w_f32 != 0, bias = a.bias != nullptr;
    if (vec == 8 && a.L > 1) {
        const int64_t blocks = (a.B * a.n_lane_per_row + 255) / 256;
#define CCV_UPD(S, F, B) \
        if (!!silu == S && wf32 == F && bias == B) return launch(k_update_tokens<W, S, F, B>, blocks, a, s);
        CCV_UPD(true, false, true) CCV_UPD(true, false, false) CCV_UPD(true, true, false)
        CCV_UPD(true, true, true) CCV_UPD(false, false, true) CCV_UPD(false, false, false)
        CCV_UPD(false, true, false) CCV_UPD(false, true, true)
#undef CCV_UPD
    } else if (vec == 8 && CCV_UPD_STAGED && a.n_lane_per_row % kWaveSize == 0 &&
               a.B * a.D >= CCV_UPD_STAGED_MIN_BD) {
        // Whole waves per row group (D % 512 == 0) and a large enough batch:
        // the coalesced kernel.
        // A block: one 512-channel range of kWavesPerBlock row groups.
        const int64_t blocks = (a.n_lane_per_row / kWaveSize) *
                               ((a.n_row_groups + kWavesPerBlock - 1) / kWavesPerBlock);
#define CCV_UPD(S, F, B)                                                                      \
        if (!!silu == S && wf32 == F && bias == B)                                            \
            return launch(k_update_staged<W, S, F, B, CCV_UPD_ROWS>, blocks, a, s);
        CCV_UPD(true, false, true) CCV_UPD(true, false, false) CCV_UPD(true, true, false)
        CCV_UPD(true, true, true) CCV_UPD(false, false, true) CCV_UPD(false, false, false)
        CCV_UPD(false, true, false) CCV_UPD(false, true, true)
#undef CCV_UPD
    } else if (vec == 8) {
        const int64_t blocks = (a.n_row_groups * a.n_lane_per_row + 255) / 256;
#define CCV_UPD(S, F, B)                                                                      \
        if (!!silu == S && wf32 == F && bias == B)                                            \
            return launch(k_update_vec<W, S, F, B, CCV_UPD_ROWS>, blocks, a, s);
        CCV_UPD(true, false, true) CCV_UPD(true, false, false) CCV_UPD(true, true, false)
        CCV_UPD(true, true, true) CCV_UPD(false, false, true) CCV_UPD(false, false, false)
        CCV_UPD(false, true, false) CCV_UPD(false, true, true)
#undef CCV_UPD
    } else if (vec == 1) {
        const int64_t blocks = (a.B * a.n_lane_per_row + 255) / 256;
#define CCV_UPD(S, F, B) \
        if (!!silu == S && wf32 == F && bias == B) return launch(k_update_any<W, S, F, B>, blocks, a, s);
        CCV_UPD(true, false, true) CCV_UPD(true, false, false) CCV_UPD(true, true, false)
        CCV_UPD(true, true, true) CCV_UPD(false, false, true) CCV_UPD(false, false, false)
        CCV_UPD(false, true, false) CCV_UPD(false, true, true)
#undef CCV_UPD
    }
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace ccv

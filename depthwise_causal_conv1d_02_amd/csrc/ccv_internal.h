// ccv_internal.h — argument blocks shared by the host layer (ccv_api.cpp)
// and the gfx950 kernels (ccv_device.h).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "ccv.h"

namespace ccv {

constexpr int kMinWidth = 2, kMaxWidth = 4;  // filter widths the kernels are built for
constexpr int kWaveSize = 64;      // CDNA wavefront
constexpr int kWavesPerBlock = 4;  // channel-lane kernels: 4 waves per block
// Forward blocks: kFwdWavesT waves along time x kFwdWavesC along channel
// groups.  Backward blocks put all 4 waves on one channel group (consecutive
// chunks), so that their dW/dB partials can be summed in LDS.
#ifndef CCV_FWD_WAVES_T
#define CCV_FWD_WAVES_T 2
#endif
constexpr int kFwdWavesT = CCV_FWD_WAVES_T;
constexpr int kFwdWavesC = kWavesPerBlock / kFwdWavesT;
// Order of blocks in a launch: 0 = time blocks innermost (a block's
// neighbours in time are its neighbours in dispatch order), 1 = channel
// blocks innermost (concurrent blocks cover whole [B,T,D] rows).
#ifndef CCV_TILE_ORDER
#define CCV_TILE_ORDER 1
#endif
constexpr int kLdsCuMax = 4096;    // cu_seqlens entries staged in LDS (16 KB)
// Time-lane kernels (unit stride along T): tokens per lane, per wave step
// (a tile), and tiles per wave chunk in the forward and the backward (the
// backward's per-chunk work, its right halo and its dW/dB sum, favours
// longer chunks).
constexpr int kTcE = 8;
constexpr int kTcTile = kWaveSize * kTcE;
#ifndef CCV_TC_TILES_FWD
#define CCV_TC_TILES_FWD 2
#endif
#ifndef CCV_TC_TILES_BWD
#define CCV_TC_TILES_BWD 4
#endif
constexpr int kTcTilesFwd = CCV_TC_TILES_FWD;
constexpr int kTcTilesBwd = CCV_TC_TILES_BWD;
// `vec` value that selects the time-lane kernels.
constexpr int kVecTime = 0;
// seq_idx rows on time lanes: a block's four waves take four rows of one
// chunk and share its tap masks through LDS (1), or every wave reads its own
// seq_idx entries (0), per direction.  The host's grid follows the same
// choice.  Measured on seqidx_tc (B4 D4096 T2048, 8 segments a row): the
// backward 54.0 -> 49.9 us with shared masks, the forward 26.5 -> 26.7 us.
#ifndef CCV_TCS_MASKS_FWD
#define CCV_TCS_MASKS_FWD 0
#endif
#ifndef CCV_TCS_MASKS_BWD
#define CCV_TCS_MASKS_BWD 1
#endif

// Unsigned 32-bit division by a divisor fixed for a launch, as a multiply
// and two shifts, exact for every 0 <= n < 2^32 (Granlund and Montgomery,
// "Division by Invariant Integers using Multiplication", PLDI 1994, section
// 4: m = floor(2^32 (2^l - d) / d) + 1 with l = ceil(log2 d)).  The host
// builds it; a kernel applies it to wave-uniform indices, where it replaces a
// 64-bit division routine that would precede the wave's first load.
struct Div32 {
    uint32_t mul, sh1, sh2;
};
constexpr Div32 make_div32(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return Div32{static_cast<uint32_t>(m), l < 1 ? l : 1u, l > 1 ? l - 1 : 0u};
}
constexpr uint32_t div32(uint32_t n, const Div32 &v) {
    const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(v.mul) * n) >> 32);
    return (t + ((n - t) >> v.sh1)) >> v.sh2;
}

// One BF16 activation-like tensor [B,D,T] (or [R,D,W-1] for states) in
// element strides.  ptr == nullptr means absent.
struct Strided3 {
    const void *ptr;
    int64_t s0, s1, s2;
};

struct FwdArgs {
    int width;                 // filter taps W (2..4)
    Strided3 x, y, init, fin;  // y/fin are written through const_cast in the kernels
    const void *w;             // [D,W], BF16 or FP32
    int64_t w_sd, w_sk;
    int w_f32, w_vec;          // w_vec: contiguous [D,W], 16-byte aligned
    const void *bias;          // [D] BF16 or nullptr
    int64_t b_s;
    const int32_t *cu;         // packed offsets or nullptr
    int64_t n_seq;             // N (packed) ; unused dense
    const int32_t *seq;        // seq_idx [B,T] or nullptr
    int64_t seq_sb, seq_st;
    int seq_vec;               // unit id stride, 16-byte aligned id rows
    uint32_t *err;             // flag word (packed) or nullptr
    int64_t B, D, T;           // T = tokens per batch row (dense) or the packed total
    int64_t L;                 // time steps per wave
    int64_t n_chunk;           // ceil(T / L)
    int64_t n_tblk;            // blocks along time: ceil(n_chunk / kFwdWavesT)
    int64_t n_group;           // channel groups of 64*VEC channels
    int64_t n_gblk;            // blocks along channels: ceil(n_group / kFwdWavesC)
    int64_t n_block;           // grid size
    // Main and tail chunks: the first n_block_m blocks take chunks of L steps
    // over [0, Tm); the others take chunks of Lt steps over [Tm, T), n_tblk_t
    // blocks along time per (row, channel block).  Tm == T: no tail.
    int64_t Tm, Lt, n_tblk_t, n_block_m;
    int cu_in_lds;             // stage + validate cu_seqlens in LDS
    int cu_in_wave;            // packed time lanes: every wave validates the N+1 <= 64 offsets
    int nt_load;               // stream the bulk loads with the non-temporal policy
    int pipe;                  // software-pipelined body (8-channel lanes, large inputs)
    // Time lanes: wave index -> (row, chunk) -> (b, d) in 32 bits when the
    // B*D*n_chunk waves fit (tc_div32), by these divisors (n_chunk, D).
    int tc_div32;
    Div32 tc_chunks, tc_rows;
    int tc_vec16;              // time lanes: every row start of every tensor is 16-byte aligned
};

struct BwdArgs {
    int width;
    Strided3 x, dy, dx, init, dfin, dinit;
    const void *w;
    int64_t w_sd, w_sk;
    int w_f32, w_vec;
    const void *bias;
    int64_t b_s;
    float *dw;                 // [D,W] FP32, contiguous, accumulated into
    float *db;                 // [D] FP32 or nullptr
    float *partial;            // deterministic path: [P][D][part_stride] FP32, else nullptr
    int part_stride;           // W, or W+1 when dbias is reduced deterministically too
    const int32_t *cu;
    int64_t n_seq;
    const int32_t *seq;        // seq_idx [B,T] or nullptr
    int64_t seq_sb, seq_st;
    int seq_vec;               // as in FwdArgs
    uint32_t *err;
    int64_t B, D, T, L, n_chunk, n_tblk, n_group, n_gblk, n_block;
    int64_t Tm, Lt, n_tblk_t, n_block_m;  // main and tail chunks, as in FwdArgs
    int cu_in_lds;
    int cu_in_wave;                       // as in FwdArgs
    int nt_load;
    int tc_div32;                         // as in FwdArgs
    Div32 tc_chunks, tc_rows;
    int tc_vec16;                         // as in FwdArgs
};

struct UpdArgs {
    int width;
    const void *x;        // [B,D] or [B,D,L]
    int64_t x_sb, x_sd;
    void *state;          // [B,D,W-1]
    int64_t s_sb, s_sd, s_sj;
    const void *w;
    int64_t w_sd, w_sk;
    int w_f32, w_vec;
    const void *bias;
    int64_t b_s;
    void *y;              // [B,D] or [B,D,L]
    int64_t y_sb, y_sd;
    int64_t L;            // tokens per row (1: x and y are [B,D])
    int64_t x_st, y_st;   // token strides when L > 1
    int64_t B, D;
    int64_t n_lane_per_row;  // D / VEC
    int64_t n_row_groups;    // ceil(B / rows per lane), 8-channel lanes
};

// Launchers (ccv_misc.hip).  `vec` is the channels per lane (8, 4 or 1); the
// filter width comes from the argument block; `rows` is the row mode
// (0 dense, 1 packed by cu_seqlens, 2 seq_idx).
hipError_t launch_fwd(const FwdArgs &a, int vec, int silu, int rows, hipStream_t s);
hipError_t launch_bwd(const BwdArgs &a, int vec, int silu, int rows, hipStream_t s);
hipError_t launch_update(const UpdArgs &a, int vec, int silu, hipStream_t s);
int update_rows_per_lane();  // batch rows an 8-channel update lane serves
// Blocks of the kernel launch_fwd / launch_bwd would pick that fit on the
// current device at once (0 if the runtime cannot tell).  Host queries only.
int64_t fwd_resident_blocks(const FwdArgs &a, int vec, int silu, int rows);
int64_t bwd_resident_blocks(const BwdArgs &a, int vec, int silu, int rows);
hipError_t launch_validate(const int32_t *cu, int64_t n_seq, int64_t total, uint32_t *flags,
                           int overwrite, hipStream_t s);
// `err`: the packed call's flag word, or nullptr; a non-zero word skips the
// reduction (the backward wrote no partials).
hipError_t launch_dw_reduce(const float *partial, int64_t n_part, int64_t n_ch, int w, int kp,
                            float *dw, float *db, const uint32_t *err, hipStream_t s);
int64_t resident_blocks(const void *kernel, unsigned dyn_lds);
int64_t device_cus();  // compute units of the current device (0 if unknown)

// Bytes of the per-device scratch behind ccv_bwd_noalloc (CCV_NOALLOC_SCRATCH_BYTES),
// and the device address of that scratch on the current device (ccv_misc.hip).
constexpr size_t kNoallocScratchBytes = CCV_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void **ptr);

// Per-width kernel selection (ccv_width.hip, built once per width).  With
// `cap` set, the resident-block capacity of the selected kernel is stored
// there; the stream kQueryStream selects without launching.
#define CCV_DECLARE_WIDTH(W)                                                                   \
    hipError_t fwd_dispatch_w##W(const FwdArgs &a, int vec, int silu, int rows, hipStream_t s, \
                                 int64_t *cap);                                                \
    hipError_t bwd_dispatch_w##W(const BwdArgs &a, int vec, int silu, int rows, hipStream_t s, \
                                 int64_t *cap);                                                \
    hipError_t update_dispatch_w##W(const UpdArgs &a, int vec, int silu, hipStream_t s);
CCV_DECLARE_WIDTH(2)
CCV_DECLARE_WIDTH(3)
CCV_DECLARE_WIDTH(4)
#undef CCV_DECLARE_WIDTH

}  // namespace ccv

// ccv_api.cpp — the C-ABI of libccv: host-side argument checks, the alias
// and determinism rules, launch geometry, and the launches.  Nothing here
// reads device memory or synchronises.
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "ccv.h"
#include "ccv_internal.h"

// Launch geometry of the channel-lane kernels (measured on MI355X): the
// chunk of time steps per wave aims for a number of waves per launch, within
// [min, max] steps; lanes own VEC channels when the layout allows.
#ifndef CCV_FWD_TARGET_WAVES
#define CCV_FWD_TARGET_WAVES 16384
#endif
#ifndef CCV_FWD_MIN_CHUNK
#define CCV_FWD_MIN_CHUNK 16
#endif
#ifndef CCV_BWD_TARGET_WAVES
#define CCV_BWD_TARGET_WAVES 16384
#endif
#ifndef CCV_BWD_MIN_CHUNK
#define CCV_BWD_MIN_CHUNK 16
#endif
// The deterministic backward's grid (and so its partials) depends on the
// shape alone: a whole number of nominal rounds of CCV_BWD_DET_ROUND_WAVES
// waves (the backward's resident waves on MI355X: two per SIMD; packed rows
// three), with chunks of at most about CCV_BWD_DET_ROUND_STEPS steps.
// Measured (interleaved, cold): against a plain 16384-wave target, the
// dense shape 54.5 -> 46.3 us, seq_idx rows 67.0 -> 52.4 us, packed rows
// 228 -> 216 us (one round of 256-step chunks), the large shape unchanged
// (8 rounds of 128 steps either way).  0 waves: the plain target.
#ifndef CCV_BWD_DET_ROUND_WAVES
#define CCV_BWD_DET_ROUND_WAVES 2048
#endif
#ifndef CCV_BWD_DET_ROUND_STEPS
#define CCV_BWD_DET_ROUND_STEPS 128
#endif
#ifndef CCV_BWD_DET_PACKED_ROUND_WAVES
#define CCV_BWD_DET_PACKED_ROUND_WAVES 3072
#endif
#ifndef CCV_BWD_DET_PACKED_ROUND_STEPS
#define CCV_BWD_DET_PACKED_ROUND_STEPS 256
#endif
#ifndef CCV_MAX_CHUNK
#define CCV_MAX_CHUNK 1024
#endif
#ifndef CCV_FWD_ROUNDS
#define CCV_FWD_ROUNDS 0        // 0: size the grid by target waves
#endif
#ifndef CCV_FWD_PACKED_MIN_CHUNK
#define CCV_FWD_PACKED_MIN_CHUNK CCV_FWD_MIN_CHUNK
#endif
#ifndef CCV_FWD_PACKED_TARGET_WAVES
#define CCV_FWD_PACKED_TARGET_WAVES CCV_FWD_TARGET_WAVES
#endif
// Inputs large enough for the pipelined forward: more waves of shorter
// chunks (16 steps on the large and packed workloads) keep the dispatcher
// refilling CUs until the end of the launch.
#ifndef CCV_FWD_PIPE_TARGET_WAVES
#define CCV_FWD_PIPE_TARGET_WAVES 65536
#endif
#ifndef CCV_BWD_PACKED_ROUNDS
#define CCV_BWD_PACKED_ROUNDS CCV_BWD_ROUNDS
#endif
#ifndef CCV_BWD_ROUNDS
#define CCV_BWD_ROUNDS 1
#endif
// Blocks per CU counted in the atomic backward's round (dense and seq_idx
// rows; 0: as many as fit).  The width-4 kernels fit 2 (two waves per SIMD);
// narrower filters need fewer registers and fit 3, and a round of 3 blocks
// per CU (shorter chunks) measured slower: widths 3 and 2 on the dense
// shape 41.9 -> 40.7 and 40.8 -> 39.8 us with the cap, seq_idx rows 46.7 ->
// 45.8 us, width 4 unchanged.  Packed rows keep 3 (measured best there).
#ifndef CCV_BWD_ROUND_BLOCKS_PER_CU
#define CCV_BWD_ROUND_BLOCKS_PER_CU 2
#endif
#ifndef CCV_FWD_VEC
#define CCV_FWD_VEC 8
#endif
// Small dense forwards (whose 8-channel geometry would already sit at the
// minimum chunk) measured faster on 4-channel lanes with 32-step chunks.
#ifndef CCV_FWD_SMALL_VEC
#define CCV_FWD_SMALL_VEC 4
#endif
#ifndef CCV_FWD_SMALL_CHUNK
#define CCV_FWD_SMALL_CHUNK 32
#endif
// Bulk loads use the non-temporal policy once an op streams at least this
// many input bytes.  Measured with cold caches (the operands in HBM, not in
// the memory-side cache): from the first byte for dense and packed rows;
// seq_idx rows from twice the 256 MB memory-side cache.
#ifndef CCV_NT_LOAD_MIN_BYTES
#define CCV_NT_LOAD_MIN_BYTES 0
#endif
#ifndef CCV_NT_LOAD_MIN_BYTES_SEQ
#define CCV_NT_LOAD_MIN_BYTES_SEQ (int64_t(1) << 29)    // forward
#endif
#ifndef CCV_NT_LOAD_MIN_BYTES_SEQ_BWD
#define CCV_NT_LOAD_MIN_BYTES_SEQ_BWD 0
#endif
// The small-input forward geometry for seq_idx rows too.
#ifndef CCV_FWD_SMALL_SEQ
#define CCV_FWD_SMALL_SEQ 1
#endif
#ifndef CCV_UPD_VEC
#define CCV_UPD_VEC 8
#endif
// The forward software-pipelines its loads (fewer, fatter waves) from this
// many input bytes on; smaller inputs keep more waves per SIMD instead.
#ifndef CCV_FWD_PIPE_MIN_BYTES
#define CCV_FWD_PIPE_MIN_BYTES (int64_t(1) << 28)
#endif
#ifndef CCV_BWD_VEC
#define CCV_BWD_VEC 4           // the backward kernels are built for 4 or 1
#endif
// Tail chunks (percent of each row's steps, and their length): the main
// chunks shrink to cover the rest, and the tail chunks' blocks are numbered
// after every main block, so the dispatcher hands them to whichever CUs
// finish first.  0 = no tail.
#ifndef CCV_FWD_TAIL_PCT
#define CCV_FWD_TAIL_PCT 0
#endif
#ifndef CCV_FWD_TAIL_CHUNK
#define CCV_FWD_TAIL_CHUNK 16
#endif
#ifndef CCV_FWD_TAIL_PIPE_ONLY
#define CCV_FWD_TAIL_PIPE_ONLY 1  // only inputs large enough for the pipelined forward
#endif
#ifndef CCV_BWD_TAIL_PCT
#define CCV_BWD_TAIL_PCT 0
#endif
#ifndef CCV_BWD_TAIL_CHUNK
#define CCV_BWD_TAIL_CHUNK 16
#endif

namespace {

constexpr uint32_t kKnownOptions = CCV_OPT_F32_FILTER_BIAS | CCV_OPT_DETERMINISTIC_DBIAS;


bool present(const ccv_tensor *t) { return t != nullptr && t->data != nullptr; }

int64_t elem_bytes(int32_t dt) {
    switch (dt) {
    case CCV_DTYPE_BF16: return 2;
    case CCV_DTYPE_F32: return 4;
    case CCV_DTYPE_I32: return 4;
    default: return 0;
    }
}

// Descriptor sanity: rank, dtype, non-negative sizes and strides.
bool well_formed(const ccv_tensor *t, int ndim) {
    if (t->ndim != ndim || elem_bytes(t->dtype) == 0) return false;
    for (int i = 0; i < ndim; ++i)
        if (t->shape[i] < 0 || t->stride[i] < 0) return false;
    return true;
}

bool shape_is(const ccv_tensor *t, int64_t a, int64_t b = -1, int64_t c = -1) {
    const int64_t want[3] = {a, b, c};
    for (int i = 0; i < t->ndim; ++i)
        if (t->shape[i] != want[i]) return false;
    return true;
}

// Byte span [lo, hi) covered by a tensor (empty when any extent is 0).
struct Span {
    uintptr_t lo = 0, hi = 0;
};

Span span_of(const ccv_tensor *t) {
    Span s;
    if (!present(t)) return s;
    int64_t last = 0;
    for (int i = 0; i < t->ndim; ++i) {
        if (t->shape[i] == 0) return s;
        last += (t->shape[i] - 1) * t->stride[i];
    }
    const int64_t eb = elem_bytes(t->dtype);
    s.lo = reinterpret_cast<uintptr_t>(t->data);
    s.hi = s.lo + static_cast<uintptr_t>((last + 1) * eb);
    return s;
}

Span span_raw(const void *p, size_t bytes) {
    Span s;
    if (p && bytes) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + bytes;
    }
    return s;
}

bool overlaps(const Span &a, const Span &b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

// No two index tuples of an output may name the same element.  Dimensions
// sorted by stride must each step over everything the smaller ones span.
bool injective(const ccv_tensor *t) {
    int64_t st[3], sh[3];
    int n = 0;
    for (int i = 0; i < t->ndim; ++i)
        if (t->shape[i] > 1) { st[n] = t->stride[i]; sh[n] = t->shape[i]; ++n; }
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if (st[j] < st[i]) { std::swap(st[i], st[j]); std::swap(sh[i], sh[j]); }
    int64_t reach = 0;  // largest offset reachable with the smaller dims
    for (int i = 0; i < n; ++i) {
        if (st[i] <= reach) return false;
        reach += (sh[i] - 1) * st[i];
    }
    return true;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A [B,D,T] BF16 tensor that lanes owning `vec` channels can read with
// vec*2-byte vectors: unit channel stride, and every row start aligned.
bool vec_ok(const ccv_tensor *t, int vec) {
    if (!present(t)) return true;
    const int64_t B = t->shape[0], D = t->shape[1], T = t->shape[2];
    const uintptr_t a = reinterpret_cast<uintptr_t>(t->data);
    return t->stride[1] == 1 && D % vec == 0 && a % (2 * vec) == 0 &&
           (B == 1 || t->stride[0] % vec == 0) && (T == 1 || t->stride[2] % vec == 0);
}

bool filter_vec(const ccv_tensor *w) {
    return w->stride[1] == 1 && w->stride[0] == w->shape[1] && aligned16(w->data);
}

// The widest lane width (preferred first, then 4, else 1) every tensor
// allows.  Vector lanes also load the filter and bias as vectors.
int pick_vec(int preferred, const ccv_tensor *weight, const ccv_tensor *bias,
             const ccv_tensor *a, const ccv_tensor *b, const ccv_tensor *c) {
    if (!filter_vec(weight) || (present(bias) && (bias->stride[0] != 1 || !aligned16(bias->data))))
        return 1;
    for (int v : {preferred, 4}) {
        if (v <= 1) continue;
        if (vec_ok(a, v) && vec_ok(b, v) && vec_ok(c, v)) return v;
    }
    return 1;
}

// Time lanes (lanes along T): every activation tensor has unit time stride
// and rows that are not channel-contiguous (dense, packed or seq_idx rows),
// at any row alignment (each wave moves its rows' tokens in the widest
// pieces their starts allow).
bool time_lanes_ok(const ccv_tensor *a, const ccv_tensor *b, const ccv_tensor *c) {
    for (const ccv_tensor *t : {a, b, c}) {
        if (t == nullptr) continue;
        if (t->stride[2] != 1 || (t->stride[1] == 1 && t->shape[1] > 1)) return false;
    }
    return true;
}

// Every row start of these tensors is 16-byte aligned.
bool rows_aligned16(const ccv_tensor *a, const ccv_tensor *b, const ccv_tensor *c) {
    for (const ccv_tensor *t : {a, b, c}) {
        if (t == nullptr) continue;
        if (!aligned16(t->data) || (t->shape[0] > 1 && t->stride[0] % 8 != 0) ||
            (t->shape[1] > 1 && t->stride[1] % 8 != 0))
            return false;
    }
    return true;
}

ccv::Strided3 s3(const ccv_tensor *t) {
    ccv::Strided3 s{nullptr, 0, 0, 0};
    if (present(t)) {
        s.ptr = t->data;
        s.s0 = t->stride[0];
        s.s1 = t->stride[1];
        s.s2 = t->stride[2];
    }
    return s;
}

// Shared checks of the full-sequence calls (forward and backward inputs).
struct Problem {
    int64_t B = 0, D = 0, T = 0, N = 0, R = 0, W = 0;
    bool packed = false;  // rows packed by cu_seqlens
    bool seq = false;     // tokens carry seq_idx sequence ids
    int rows() const { return packed ? 1 : (seq ? 2 : 0); }  // the kernels' row mode
};

// The filter and bias dtypes: a BF16 filter takes a BF16 bias; an FP32
// filter takes no bias, or (with CCV_OPT_F32_FILTER_BIAS) an FP32 one.
// Called after the shape checks; returns INVALID or the explicit decline.
int check_filter_dtypes(const ccv_tensor *weight, const ccv_tensor *bias, uint32_t options) {
    if (!present(bias)) return CCV_OK;
    if (weight->dtype == CCV_DTYPE_BF16)
        return bias->dtype == CCV_DTYPE_BF16 ? CCV_OK : CCV_ERR_INVALID_ARG;
    if (bias->dtype != CCV_DTYPE_BF16 && bias->dtype != CCV_DTYPE_F32) return CCV_ERR_INVALID_ARG;
    if (!(options & CCV_OPT_F32_FILTER_BIAS)) return CCV_ERR_UNSUPPORTED;
    return bias->dtype == CCV_DTYPE_F32 ? CCV_OK : CCV_ERR_INVALID_ARG;
}

int check_inputs(const ccv_tensor *x, const ccv_tensor *weight, const ccv_tensor *bias,
                 const ccv_tensor *cu, const ccv_tensor *seq_idx, const ccv_tensor *init,
                 int activation, const uint32_t *err_flag, uint32_t options, Problem &p) {
    if (!present(x) || !well_formed(x, 3) || x->dtype != CCV_DTYPE_BF16) return CCV_ERR_INVALID_ARG;
    p.B = x->shape[0];
    p.D = x->shape[1];
    p.T = x->shape[2];
    if (p.B < 1 || p.D < 1 || p.T < 1) return CCV_ERR_INVALID_ARG;
    if (!present(weight) || !well_formed(weight, 2) || weight->shape[0] != p.D ||
        weight->shape[1] < 1 ||
        (weight->dtype != CCV_DTYPE_BF16 && weight->dtype != CCV_DTYPE_F32))
        return CCV_ERR_INVALID_ARG;
    if (present(bias) && (!well_formed(bias, 1) || !shape_is(bias, p.D)))
        return CCV_ERR_INVALID_ARG;
    if (options & ~kKnownOptions) return CCV_ERR_INVALID_ARG;
    // seq_idx and cu_seqlens are mutually exclusive.
    if (present(seq_idx) && present(cu)) return CCV_ERR_INVALID_ARG;
    if (present(seq_idx)) {
        if (!well_formed(seq_idx, 2) || seq_idx->dtype != CCV_DTYPE_I32 ||
            !shape_is(seq_idx, p.B, p.T))
            return CCV_ERR_INVALID_ARG;
        p.seq = true;
    }
    if (present(cu)) {
        if (!well_formed(cu, 1) || cu->dtype != CCV_DTYPE_I32 || cu->stride[0] != 1 ||
            cu->shape[0] < 2 || p.B != 1 || err_flag == nullptr || cu->shape[0] - 1 > INT32_MAX)
            return CCV_ERR_INVALID_ARG;
        p.packed = true;
        p.N = cu->shape[0] - 1;
    }
    p.R = p.packed ? p.N : p.B;
    if (present(init) && (!well_formed(init, 3) || init->dtype != CCV_DTYPE_BF16 ||
                          !shape_is(init, p.R, p.D, weight->shape[1] - 1)))
        return CCV_ERR_INVALID_ARG;
    // Declines: states with seq_idx (undefined there), the width, FP32 filter
    // with a bias (unless opted in), the activation set.
    if (p.seq && present(init)) return CCV_ERR_UNSUPPORTED;
    p.W = weight->shape[1];
    if (p.W < ccv::kMinWidth || p.W > ccv::kMaxWidth) return CCV_ERR_UNSUPPORTED;
    if (int rc = check_filter_dtypes(weight, bias, options)) return rc;
    if (activation != CCV_ACT_NONE && activation != CCV_ACT_SILU) return CCV_ERR_UNSUPPORTED;
    return CCV_OK;
}

int check_state_out(const ccv_tensor *t, const Problem &p) {
    if (!present(t)) return CCV_OK;
    if (!well_formed(t, 3) || t->dtype != CCV_DTYPE_BF16 || !shape_is(t, p.R, p.D, p.W - 1) ||
        !injective(t))
        return CCV_ERR_INVALID_ARG;
    return CCV_OK;
}

int check_act_tensor(const ccv_tensor *t, const Problem &p, bool output) {
    if (!present(t) || !well_formed(t, 3) || t->dtype != CCV_DTYPE_BF16 ||
        !shape_is(t, p.B, p.D, p.T))
        return CCV_ERR_INVALID_ARG;
    if (output && !injective(t)) return CCV_ERR_INVALID_ARG;
    return CCV_OK;
}

// The seq_idx fields of an argument block.
template <typename A>
void set_seq(A &a, const ccv_tensor *seq_idx, const Problem &p) {
    a.seq = p.seq ? static_cast<const int32_t *>(seq_idx->data) : nullptr;
    a.seq_sb = p.seq ? seq_idx->stride[0] : 0;
    a.seq_st = p.seq ? seq_idx->stride[1] : 0;
    a.seq_vec = p.seq && a.seq_st == 1 && a.seq_sb % 4 == 0 && aligned16(seq_idx->data);
}

// Every output span against every input span and every other output span.
bool any_alias(const Span *outs, int n_out, const Span *ins, int n_in) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j)
            if (overlaps(outs[i], ins[j])) return true;
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i], outs[j])) return true;
    }
    return false;
}

// Time steps per wave (L).  With `rounds` > 0 and the device's resident
// block capacity known, L makes the grid `rounds` whole rounds of resident
// blocks, so that no last round runs partly empty.  Otherwise L aims for
// `target_waves` waves.  Never fewer than `min_chunk` steps per wave.
// A block holds `wt` waves along time times `wc` waves along channel groups.
struct Geometry {
    int64_t L, n_chunk, n_tblk, n_group, n_gblk, n_block;
    int64_t Tm, Lt, n_tblk_t, n_block_m;  // main / tail split (Tm == T: none)
};

Geometry geometry(const Problem &p, int vec, int wt, int wc, int64_t capacity, int rounds,
                  int64_t target_waves, int64_t min_chunk) {
    Geometry g;
    g.n_group = (p.D + ccv::kWaveSize * vec - 1) / (ccv::kWaveSize * vec);
    g.n_gblk = (g.n_group + wc - 1) / wc;
    const int64_t rows = p.packed ? 1 : p.B;
    const int64_t work = rows * g.n_group * p.T;
    int64_t L = 0;
    if (capacity > 0 && rounds > 0) {
        const int64_t per_row_gblk = capacity * rounds / (rows * g.n_gblk);
        if (per_row_gblk >= 1) {
            const int64_t chunks = per_row_gblk * wt;
            L = (p.T + chunks - 1) / chunks;
        }
    }
    if (L == 0) {
        L = (work + target_waves - 1) / target_waves;
        L = (L + 7) / 8 * 8;
    }
    L = std::max<int64_t>(min_chunk, std::min<int64_t>(CCV_MAX_CHUNK, L));
    g.L = L;
    g.n_chunk = (p.T + L - 1) / L;
    g.n_tblk = (g.n_chunk + wt - 1) / wt;
    g.n_block = rows * g.n_gblk * g.n_tblk;
    g.Tm = p.T;
    g.Lt = 0;
    g.n_tblk_t = 0;
    g.n_block_m = g.n_block;
    return g;
}

// Target waves of the deterministic backward: as many nominal rounds as
// chunks of at most the round's steps need, up to the plain target (the
// large workload: 8 rounds of 128-step chunks, which is the plain target;
// the dense one: 1 round of 64-step chunks; the packed one: 1 round of 3072
// waves).
int64_t det_target_waves(const Problem &p, int vec) {
    const int64_t waves = p.packed ? CCV_BWD_DET_PACKED_ROUND_WAVES : CCV_BWD_DET_ROUND_WAVES;
    const int64_t steps = p.packed ? CCV_BWD_DET_PACKED_ROUND_STEPS : CCV_BWD_DET_ROUND_STEPS;
    if (waves <= 0) return CCV_BWD_TARGET_WAVES;
    const int64_t groups = (p.D + ccv::kWaveSize * vec - 1) / (ccv::kWaveSize * vec);
    const int64_t work = (p.packed ? 1 : p.B) * groups * p.T;
    const int64_t per_round = waves * steps;
    // never more waves (so never more partials) than the plain target
    return std::min<int64_t>(std::max<int64_t>(1, (work + per_round - 1) / per_round) * waves,
                             CCV_BWD_TARGET_WAVES);
}

// Split off tail chunks: the main chunks keep their number (whole blocks of
// `wt`) and shrink to cover (100 - pct)% of the steps; the rest is cut into
// chunks of `lt` steps.  No split when pct or lt is 0, or when the main
// chunks would fall below `min_chunk` steps.
void add_tail(Geometry &g, const Problem &p, int wt, int pct, int64_t lt, int64_t min_chunk) {
    if (pct <= 0 || pct >= 100 || lt <= 0) return;
    const int64_t n_chunk_m = g.n_tblk * wt;
    const int64_t Lm = p.T * (100 - pct) / 100 / n_chunk_m;
    if (Lm < min_chunk) return;
    const int64_t Tm = Lm * n_chunk_m;
    if (Tm >= p.T) return;
    const int64_t per = (p.packed ? 1 : p.B) * g.n_gblk;
    const int64_t n_chunk_t = (p.T - Tm + lt - 1) / lt;
    g.L = Lm;
    g.Tm = Tm;
    g.Lt = lt;
    g.n_tblk_t = (n_chunk_t + wt - 1) / wt;
    g.n_chunk = n_chunk_m + n_chunk_t;
    g.n_block_m = per * g.n_tblk;
    g.n_block = g.n_block_m + per * g.n_tblk_t;
}

// seq_idx rows on time lanes with block-shared tap masks: a block takes
// kWavesPerBlock consecutive channels of one (batch row, chunk).
bool seq_mask_blocks(const Problem &p, bool bwd) {
    return (bwd ? CCV_TCS_MASKS_BWD : CCV_TCS_MASKS_FWD) && p.seq && !p.packed;
}
int64_t row_groups(const Problem &p) {
    return (p.D + ccv::kWavesPerBlock - 1) / ccv::kWavesPerBlock;
}

// Time-lane geometry: one wave per (row, chunk of `tiles` tiles).
Geometry time_geometry(const Problem &p, int tiles, bool bwd) {
    Geometry g;
    g.L = static_cast<int64_t>(tiles) * ccv::kTcTile;
    g.n_chunk = (p.T + g.L - 1) / g.L;
    g.n_tblk = g.n_chunk;  // partials per batch row: one per chunk
    g.n_group = p.D;
    g.n_gblk = p.D;
    g.n_block = seq_mask_blocks(p, bwd)
                    ? p.B * g.n_chunk * row_groups(p)
                    : (p.B * p.D * g.n_chunk + ccv::kWavesPerBlock - 1) / ccv::kWavesPerBlock;
    g.Tm = p.T;
    g.Lt = 0;
    g.n_tblk_t = 0;
    g.n_block_m = g.n_block;
    return g;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CCV_OK : CCV_ERR_HIP; }

// Where packed offsets are validated: inside every block of the launch (in
// LDS, channel lanes, N+1 <= 4096), by every wave (time lanes, one offset per
// lane, N+1 <= 64), or by the validation launch before it.  The first two
// need the launch to run at least one wave.
template <typename A>
void set_validation(A &a, const Problem &p, bool time_lanes) {
    const bool waves = p.B * p.D * p.T > 0;
    a.cu_in_lds = p.packed && !time_lanes && waves && p.N + 1 <= ccv::kLdsCuMax;
    a.cu_in_wave = p.packed && time_lanes && waves && p.N + 1 <= ccv::kWaveSize;
}

// The time lanes decode their wave index in 32 bits when all B*D*n_chunk
// wave indices fit; with block-shared masks, their block index (B*n_chunk
// blocks per row group, divided by the row groups, then by n_chunk).
template <typename A>
void set_tc_div(A &a, const Problem &p, bool bwd) {
    const bool blocks = seq_mask_blocks(p, bwd);
    const int64_t per = blocks ? row_groups(p) : a.D;
    a.tc_div32 = a.B * per * a.n_chunk <= int64_t(UINT32_MAX);
    if (a.tc_div32) {
        a.tc_chunks = ccv::make_div32(static_cast<uint32_t>(a.n_chunk));
        a.tc_rows = ccv::make_div32(static_cast<uint32_t>(per));
    }
}

}  // namespace

extern "C" {

int ccv_abi_version(void) { return CCV_ABI_VERSION; }

const char *ccv_status_string(int status) {
    switch (status) {
    case CCV_OK: return "CCV_OK";
    case CCV_WARN_NONDETERMINISTIC: return "CCV_WARN_NONDETERMINISTIC";
    case CCV_ERR_INVALID_ARG: return "CCV_ERR_INVALID_ARG";
    case CCV_ERR_ALIAS: return "CCV_ERR_ALIAS";
    case CCV_ERR_UNSUPPORTED: return "CCV_ERR_UNSUPPORTED";
    case CCV_ERR_NONDETERMINISTIC: return "CCV_ERR_NONDETERMINISTIC";
    case CCV_ERR_HIP: return "CCV_ERR_HIP";
    case CCV_ERR_TOO_LARGE: return "CCV_ERR_TOO_LARGE";
    default: return "CCV_UNKNOWN_STATUS";
    }
}

int ccv_fwd(const ccv_tensor *x, const ccv_tensor *weight, const ccv_tensor *bias,
            const ccv_tensor *cu_seqlens, const ccv_tensor *seq_idx,
            const ccv_tensor *initial_states, const ccv_tensor *y,
            const ccv_tensor *final_states, int activation, uint32_t options,
            uint32_t *err_flag, hipStream_t stream) {
    Problem p;
    int rc = check_inputs(x, weight, bias, cu_seqlens, seq_idx, initial_states, activation,
                          err_flag, options, p);
    if (rc != CCV_OK) return rc;
    if ((rc = check_act_tensor(y, p, true)) != CCV_OK) return rc;
    if ((rc = check_state_out(final_states, p)) != CCV_OK) return rc;
    if (p.seq && present(final_states)) return CCV_ERR_UNSUPPORTED;

    const Span outs[] = {span_of(y), span_of(final_states),
                         p.packed ? span_raw(err_flag, 4) : Span{}};
    const Span ins[] = {span_of(x), span_of(weight), span_of(bias), span_of(cu_seqlens),
                        span_of(initial_states), span_of(seq_idx)};
    if (any_alias(outs, 3, ins, 6)) return CCV_ERR_ALIAS;

    const bool time_lanes = time_lanes_ok(x, y, nullptr);
    const bool pipe = p.B * p.D * p.T * 2 >= CCV_FWD_PIPE_MIN_BYTES;
    const int64_t groups8 = (p.D + ccv::kWaveSize * 8 - 1) / (ccv::kWaveSize * 8);
    const bool small_dense = !p.packed && (!p.seq || CCV_FWD_SMALL_SEQ) && !pipe &&
                             p.B * groups8 * p.T <= int64_t(CCV_FWD_TARGET_WAVES) * CCV_FWD_MIN_CHUNK;
    const int vec = time_lanes ? ccv::kVecTime
                               : pick_vec(small_dense ? CCV_FWD_SMALL_VEC : CCV_FWD_VEC, weight,
                                          bias, x, y, nullptr);
    ccv::FwdArgs a;
    memset(&a, 0, sizeof(a));
    a.width = static_cast<int>(p.W);
    a.x = s3(x);
    a.y = s3(y);
    a.init = s3(initial_states);
    a.fin = s3(final_states);
    a.w = weight->data;
    a.w_sd = weight->stride[0];
    a.w_sk = weight->stride[1];
    a.w_f32 = weight->dtype == CCV_DTYPE_F32;
    a.w_vec = filter_vec(weight);
    a.bias = present(bias) ? bias->data : nullptr;
    a.b_s = present(bias) ? bias->stride[0] : 0;
    a.cu = p.packed ? static_cast<const int32_t *>(cu_seqlens->data) : nullptr;
    a.n_seq = p.N;
    a.err = p.packed ? err_flag : nullptr;
    set_seq(a, seq_idx, p);
    a.pipe = pipe;
    const int silu = activation == CCV_ACT_SILU;
    const int64_t cap = CCV_FWD_ROUNDS > 0 && !time_lanes
                            ? ccv::fwd_resident_blocks(a, vec, silu, p.rows())
                            : 0;
    const Geometry g = time_lanes ? time_geometry(p, ccv::kTcTilesFwd, false)
                                  : geometry(p, vec, ccv::kFwdWavesT, ccv::kFwdWavesC, cap,
                                             CCV_FWD_ROUNDS,
                                             pipe && vec == 8 && !p.seq
                                                 ? CCV_FWD_PIPE_TARGET_WAVES
                                             : p.packed ? CCV_FWD_PACKED_TARGET_WAVES
                                                        : CCV_FWD_TARGET_WAVES,
                                             p.packed ? CCV_FWD_PACKED_MIN_CHUNK
                                             : small_dense && vec == CCV_FWD_SMALL_VEC
                                                 ? CCV_FWD_SMALL_CHUNK
                                                 : CCV_FWD_MIN_CHUNK);
    Geometry gs = g;
    if (!time_lanes && (pipe || !CCV_FWD_TAIL_PIPE_ONLY))
        add_tail(gs, p, ccv::kFwdWavesT, CCV_FWD_TAIL_PCT, CCV_FWD_TAIL_CHUNK, 1);
    a.B = p.B;
    a.D = p.D;
    a.T = p.T;
    a.L = gs.L;
    a.n_chunk = gs.n_chunk;
    a.n_tblk = gs.n_tblk;
    a.n_group = gs.n_group;
    a.n_gblk = gs.n_gblk;
    a.n_block = gs.n_block;
    a.Tm = gs.Tm;
    a.Lt = gs.Lt;
    a.n_tblk_t = gs.n_tblk_t;
    a.n_block_m = gs.n_block_m;
    if (time_lanes) set_tc_div(a, p, false);
    a.tc_vec16 = time_lanes && rows_aligned16(x, y, nullptr);
    set_validation(a, p, time_lanes);
    a.nt_load = p.B * p.D * p.T * 2 >=
                (p.seq ? CCV_NT_LOAD_MIN_BYTES_SEQ : CCV_NT_LOAD_MIN_BYTES);
    if (p.packed && !a.cu_in_lds && !a.cu_in_wave) {
        rc = hip_status(ccv::launch_validate(a.cu, p.N, p.T, err_flag, 0, stream));
        if (rc != CCV_OK) return rc;
    }
    return hip_status(ccv::launch_fwd(a, vec, silu, p.rows(), stream));
}

}  // extern "C"

namespace {

// The backward behind ccv_bwd and ccv_bwd_noalloc.  With `noalloc` the
// deterministic route's partials go to the library's per-device scratch
// (no size query; calls that need more than it holds are refused before
// any HIP call).
int bwd_call(const ccv_tensor *x, const ccv_tensor *weight, const ccv_tensor *bias,
             const ccv_tensor *cu_seqlens, const ccv_tensor *seq_idx,
             const ccv_tensor *initial_states, const ccv_tensor *dy,
             const ccv_tensor *dfinal_states, const ccv_tensor *dx, const ccv_tensor *dweight,
             const ccv_tensor *dbias, const ccv_tensor *dinitial_states, int activation,
             int deterministic, int warn_only, uint32_t options, void *workspace,
             size_t *workspace_bytes, uint32_t *err_flag, hipStream_t stream, bool noalloc) {
    Problem p;
    int rc = check_inputs(x, weight, bias, cu_seqlens, seq_idx, initial_states, activation,
                          err_flag, options, p);
    if (rc != CCV_OK) return rc;
    if ((rc = check_act_tensor(dy, p, false)) != CCV_OK) return rc;
    if ((rc = check_act_tensor(dx, p, true)) != CCV_OK) return rc;
    if (present(dfinal_states) &&
        (!well_formed(dfinal_states, 3) || dfinal_states->dtype != CCV_DTYPE_BF16 ||
         !shape_is(dfinal_states, p.R, p.D, p.W - 1)))
        return CCV_ERR_INVALID_ARG;
    if ((rc = check_state_out(dinitial_states, p)) != CCV_OK) return rc;
    if (present(dinitial_states) && !present(initial_states)) return CCV_ERR_INVALID_ARG;
    if (p.seq && present(dfinal_states)) return CCV_ERR_UNSUPPORTED;
    // dweight [D,W] and dbias [D]: FP32, contiguous.
    if (!present(dweight) || !well_formed(dweight, 2) || dweight->dtype != CCV_DTYPE_F32 ||
        !shape_is(dweight, p.D, p.W) || dweight->stride[0] != p.W || dweight->stride[1] != 1)
        return CCV_ERR_INVALID_ARG;
    if (present(bias) != present(dbias)) return CCV_ERR_INVALID_ARG;
    if (present(dbias) && (!well_formed(dbias, 1) || dbias->dtype != CCV_DTYPE_F32 ||
                           !shape_is(dbias, p.D) || dbias->stride[0] != 1))
        return CCV_ERR_INVALID_ARG;

    // Determinism policy (cuDNN FE "Causal Conv1d", the determinism
    // paragraph): a bias has no deterministic dbias route unless the caller
    // opts into dbias partials (one more FP32 column per channel).
    int status = CCV_OK;
    bool use_partials = false;
    if (deterministic) {
        if (present(bias) && !(options & CCV_OPT_DETERMINISTIC_DBIAS)) {
            if (!warn_only) return CCV_ERR_NONDETERMINISTIC;
            status = CCV_WARN_NONDETERMINISTIC;
        } else {
            use_partials = true;
        }
    }
    const int64_t kp = p.W + (present(bias) ? 1 : 0);  // partial columns per channel
    const bool time_lanes = time_lanes_ok(x, dy, dx);
    const int vec = time_lanes ? ccv::kVecTime : pick_vec(CCV_BWD_VEC, weight, bias, x, dy, dx);
    // The partials of the deterministic route depend on the shape only (a
    // grid sized by target waves); the atomic route sizes its grid by the
    // device's resident capacity below.
    Geometry g = time_lanes ? time_geometry(p, ccv::kTcTilesBwd, true)
                            : geometry(p, vec, ccv::kWavesPerBlock, 1, 0, 0,
                                       det_target_waves(p, vec), CCV_BWD_MIN_CHUNK);
    if (!time_lanes)
        add_tail(g, p, ccv::kWavesPerBlock, CCV_BWD_TAIL_PCT, CCV_BWD_TAIL_CHUNK, 1);
    // packed rows on time lanes: the boundary repair's partial rows follow
    // the chunks' (one per channel and group of 64 boundaries)
    const int64_t n_part = (p.packed ? 1 : p.B) * (g.n_tblk + g.n_tblk_t) +
                           (p.packed && time_lanes ? (p.N + 1 + ccv::kWaveSize - 1) / ccv::kWaveSize
                                                   : 0);
    const size_t need = use_partials
                            ? static_cast<size_t>(n_part) * static_cast<size_t>(p.D * kp) * 4
                            : 0;
    if (noalloc) {
        // The partials go to the library's scratch (looked up after every
        // host check below); it is private, so it takes no part in the
        // alias test.
        if (need > ccv::kNoallocScratchBytes) return CCV_ERR_TOO_LARGE;
        workspace = nullptr;
        workspace_bytes = nullptr;
    } else if (workspace == nullptr && workspace_bytes != nullptr) {  // size query
        *workspace_bytes = need;
        return CCV_OK;
    }
    if (need > 0 && !noalloc) {
        if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
            return CCV_ERR_INVALID_ARG;
        if (workspace_bytes != nullptr && *workspace_bytes < need) return CCV_ERR_INVALID_ARG;
    }

    const Span outs[] = {span_of(dx), span_of(dweight), span_of(dbias), span_of(dinitial_states),
                         p.packed ? span_raw(err_flag, 4) : Span{}, span_raw(workspace, need)};
    const Span ins[] = {span_of(x), span_of(weight), span_of(bias), span_of(cu_seqlens),
                        span_of(initial_states), span_of(dy), span_of(dfinal_states),
                        span_of(seq_idx)};
    if (any_alias(outs, 6, ins, 8)) return CCV_ERR_ALIAS;

    if (noalloc && need > 0) {
        rc = hip_status(ccv::noalloc_scratch(&workspace));
        if (rc != CCV_OK) return rc;
    }

    ccv::BwdArgs a;
    memset(&a, 0, sizeof(a));
    a.width = static_cast<int>(p.W);
    a.x = s3(x);
    a.dy = s3(dy);
    a.dx = s3(dx);
    a.init = s3(initial_states);
    a.dfin = s3(dfinal_states);
    a.dinit = s3(dinitial_states);
    a.w = weight->data;
    a.w_sd = weight->stride[0];
    a.w_sk = weight->stride[1];
    a.w_f32 = weight->dtype == CCV_DTYPE_F32;
    a.w_vec = filter_vec(weight);
    a.bias = present(bias) ? bias->data : nullptr;
    a.b_s = present(bias) ? bias->stride[0] : 0;
    a.dw = static_cast<float *>(dweight->data);
    a.db = present(dbias) ? static_cast<float *>(dbias->data) : nullptr;
    a.partial = use_partials ? static_cast<float *>(workspace) : nullptr;
    a.part_stride = static_cast<int>(kp);
    a.cu = p.packed ? static_cast<const int32_t *>(cu_seqlens->data) : nullptr;
    a.n_seq = p.N;
    a.err = p.packed ? err_flag : nullptr;
    set_seq(a, seq_idx, p);
    a.nt_load = 2 * p.B * p.D * p.T * 2 >=
                (p.seq ? CCV_NT_LOAD_MIN_BYTES_SEQ_BWD : CCV_NT_LOAD_MIN_BYTES);
    const int silu = activation == CCV_ACT_SILU;
    const int rounds = p.packed ? CCV_BWD_PACKED_ROUNDS : CCV_BWD_ROUNDS;
    if (!use_partials && rounds > 0 && !time_lanes) {
        int64_t cap = ccv::bwd_resident_blocks(a, vec, silu, p.rows());
        if (CCV_BWD_ROUND_BLOCKS_PER_CU > 0 && !p.packed)
            cap = std::min<int64_t>(cap, ccv::device_cus() * CCV_BWD_ROUND_BLOCKS_PER_CU);
        g = geometry(p, vec, ccv::kWavesPerBlock, 1, cap, rounds, CCV_BWD_TARGET_WAVES,
                     CCV_BWD_MIN_CHUNK);
        add_tail(g, p, ccv::kWavesPerBlock, CCV_BWD_TAIL_PCT, CCV_BWD_TAIL_CHUNK, 1);
    }
    a.B = p.B;
    a.D = p.D;
    a.T = p.T;
    a.L = g.L;
    a.n_chunk = g.n_chunk;
    a.n_tblk = g.n_tblk;
    a.n_group = g.n_group;
    a.n_gblk = g.n_gblk;
    a.n_block = g.n_block;
    a.Tm = g.Tm;
    a.Lt = g.Lt;
    a.n_tblk_t = g.n_tblk_t;
    a.n_block_m = g.n_block_m;
    if (time_lanes) set_tc_div(a, p, true);
    a.tc_vec16 = time_lanes && rows_aligned16(x, dy, dx);
    set_validation(a, p, time_lanes);

    if (p.packed && !a.cu_in_lds && !a.cu_in_wave) {
        rc = hip_status(ccv::launch_validate(a.cu, p.N, p.T, err_flag, 0, stream));
        if (rc != CCV_OK) return rc;
    }
    rc = hip_status(ccv::launch_bwd(a, vec, silu, p.rows(), stream));
    if (rc != CCV_OK) return rc;
    if (use_partials) {
        rc = hip_status(ccv::launch_dw_reduce(a.partial, n_part, p.D, static_cast<int>(p.W),
                                              static_cast<int>(kp), a.dw, a.db, a.err, stream));
        if (rc != CCV_OK) return rc;
    }
    return status;
}

}  // namespace

extern "C" {

int ccv_bwd(const ccv_tensor *x, const ccv_tensor *weight, const ccv_tensor *bias,
            const ccv_tensor *cu_seqlens, const ccv_tensor *seq_idx,
            const ccv_tensor *initial_states, const ccv_tensor *dy,
            const ccv_tensor *dfinal_states, const ccv_tensor *dx,
            const ccv_tensor *dweight, const ccv_tensor *dbias,
            const ccv_tensor *dinitial_states, int activation, int deterministic,
            int warn_only, uint32_t options, void *workspace, size_t *workspace_bytes,
            uint32_t *err_flag, hipStream_t stream) {
    return bwd_call(x, weight, bias, cu_seqlens, seq_idx, initial_states, dy, dfinal_states, dx,
                    dweight, dbias, dinitial_states, activation, deterministic, warn_only, options,
                    workspace, workspace_bytes, err_flag, stream, false);
}

int ccv_bwd_noalloc(const ccv_tensor *x, const ccv_tensor *weight, const ccv_tensor *bias,
                    const ccv_tensor *cu_seqlens, const ccv_tensor *seq_idx,
                    const ccv_tensor *initial_states, const ccv_tensor *dy,
                    const ccv_tensor *dfinal_states, const ccv_tensor *dx,
                    const ccv_tensor *dweight, const ccv_tensor *dbias,
                    const ccv_tensor *dinitial_states, int activation, int deterministic,
                    int warn_only, uint32_t options, uint32_t *err_flag, hipStream_t stream) {
    return bwd_call(x, weight, bias, cu_seqlens, seq_idx, initial_states, dy, dfinal_states, dx,
                    dweight, dbias, dinitial_states, activation, deterministic, warn_only, options,
                    nullptr, nullptr, err_flag, stream, true);
}

int ccv_update(const ccv_tensor *x, const ccv_tensor *conv_state, const ccv_tensor *weight,
               const ccv_tensor *bias, const ccv_tensor *y, int activation, uint32_t options,
               hipStream_t stream) {
    // x and y: [B,D] (one token) or [B,D,L] (L tokens in order).
    if (!present(x) || (x->ndim != 2 && x->ndim != 3) || !well_formed(x, x->ndim) ||
        x->dtype != CCV_DTYPE_BF16)
        return CCV_ERR_INVALID_ARG;
    const int nd = x->ndim;
    const int64_t B = x->shape[0], D = x->shape[1], L = nd == 3 ? x->shape[2] : 1;
    if (B < 1 || D < 1 || L < 1) return CCV_ERR_INVALID_ARG;
    if (!present(weight) || !well_formed(weight, 2) || weight->shape[0] != D ||
        weight->shape[1] < 1 ||
        (weight->dtype != CCV_DTYPE_BF16 && weight->dtype != CCV_DTYPE_F32))
        return CCV_ERR_INVALID_ARG;
    if (present(bias) && (!well_formed(bias, 1) || !shape_is(bias, D)))
        return CCV_ERR_INVALID_ARG;
    if (options & ~kKnownOptions) return CCV_ERR_INVALID_ARG;
    if (!present(conv_state) || !well_formed(conv_state, 3) ||
        conv_state->dtype != CCV_DTYPE_BF16 ||
        !shape_is(conv_state, B, D, weight->shape[1] - 1) || !injective(conv_state))
        return CCV_ERR_INVALID_ARG;
    if (!present(y) || !well_formed(y, nd) || y->dtype != CCV_DTYPE_BF16 ||
        !shape_is(y, B, D, nd == 3 ? L : -1) || !injective(y))
        return CCV_ERR_INVALID_ARG;
    const int64_t W = weight->shape[1];
    if (W < ccv::kMinWidth || W > ccv::kMaxWidth) return CCV_ERR_UNSUPPORTED;
    if (int rc = check_filter_dtypes(weight, bias, options)) return rc;
    if (activation != CCV_ACT_NONE && activation != CCV_ACT_SILU) return CCV_ERR_UNSUPPORTED;
    // conv_state is in/out by design; y and the state must not overlap any
    // other argument.
    const Span outs[] = {span_of(y), span_of(conv_state)};
    const Span ins[] = {span_of(x), span_of(weight), span_of(bias)};
    if (any_alias(outs, 2, ins, 3)) return CCV_ERR_ALIAS;

    // 8-channel lanes need unit channel strides, a contiguous state, a
    // contiguous filter and bias, and 16-byte aligned rows everywhere.
    // With several tokens, their strides keep the rows aligned too.
    const bool vec = CCV_UPD_VEC == 8 && D % 8 == 0 && x->stride[1] == 1 && y->stride[1] == 1 &&
                     conv_state->stride[2] == 1 && conv_state->stride[1] == W - 1 &&
                     aligned16(x->data) && aligned16(y->data) && aligned16(conv_state->data) &&
                     (B == 1 || (x->stride[0] % 8 == 0 && y->stride[0] % 8 == 0 &&
                                 conv_state->stride[0] % 8 == 0)) &&
                     (L == 1 || (x->stride[2] % 8 == 0 && y->stride[2] % 8 == 0)) &&
                     filter_vec(weight) &&
                     (!present(bias) || (bias->stride[0] == 1 && aligned16(bias->data)));
    ccv::UpdArgs a;
    memset(&a, 0, sizeof(a));
    a.width = static_cast<int>(W);
    a.x = x->data;
    a.x_sb = x->stride[0];
    a.x_sd = x->stride[1];
    a.state = conv_state->data;
    a.s_sb = conv_state->stride[0];
    a.s_sd = conv_state->stride[1];
    a.s_sj = conv_state->stride[2];
    a.w = weight->data;
    a.w_sd = weight->stride[0];
    a.w_sk = weight->stride[1];
    a.w_f32 = weight->dtype == CCV_DTYPE_F32;
    a.w_vec = filter_vec(weight);
    a.bias = present(bias) ? bias->data : nullptr;
    a.b_s = present(bias) ? bias->stride[0] : 0;
    a.y = y->data;
    a.y_sb = y->stride[0];
    a.y_sd = y->stride[1];
    a.L = L;
    a.x_st = nd == 3 ? x->stride[2] : 0;
    a.y_st = nd == 3 ? y->stride[2] : 0;
    a.B = B;
    a.D = D;
    a.n_lane_per_row = vec ? D / 8 : D;
    const int64_t rpl = ccv::update_rows_per_lane();
    a.n_row_groups = (B + rpl - 1) / rpl;
    return hip_status(ccv::launch_update(a, vec ? 8 : 1, activation == CCV_ACT_SILU, stream));
}

int ccv_validate_cu_seqlens(const int32_t *cu_seqlens, int64_t n_seqs, int64_t total_tokens,
                            uint32_t *flags, hipStream_t stream) {
    if (cu_seqlens == nullptr || flags == nullptr || n_seqs < 1 || total_tokens < 1 ||
        n_seqs > INT32_MAX)
        return CCV_ERR_INVALID_ARG;
    if (overlaps(span_raw(cu_seqlens, static_cast<size_t>(n_seqs + 1) * 4), span_raw(flags, 4)))
        return CCV_ERR_ALIAS;
    return hip_status(ccv::launch_validate(cu_seqlens, n_seqs, total_tokens, flags, 1, stream));
}

}  // extern "C"

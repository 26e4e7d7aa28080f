/*
 * ccv.h — C-ABI of libccv, the MI355X (gfx950) depthwise causal conv1d.
 *
 * The operation (cuDNN FE "Causal Conv1d" page, the bullet list of tensor and
 * state semantics, the paragraph on the optimized route, and the
 * POPCORNBENCH causal conv1d trace's derivation of the causal left pad for
 * the tap order):
 *
 *   z[b,d,t] = bias[d] + sum_{k=0}^{W-1} weight[d,k] * x_ext[b,d,t-(W-1)+k]
 *   y[b,d,t] = act(z[b,d,t]),   act in {identity, SiLU}
 *
 * x_ext is a row of x extended on the left by its W-1 initial-state values
 * (oldest first) or by zeros.  A row is one batch entry (dense) or one
 * sequence [cu_seqlens[i], cu_seqlens[i+1]) of a B == 1 input packed along T.
 * Tap W-1 multiplies the current token.  final_states holds the last W-1
 * entries of each extended row, oldest first.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor is described by a ccv_tensor: a DEVICE pointer, a dtype,
 *   and shape and strides in elements, in the logical index order of the
 *   pages' shapes.  x, y, dy and dx are [B,D,T]; channel-last [B,T,D]
 *   storage seen through transpose(1,2) has stride[1] == 1 and is consumed
 *   as is, without a copy (cuDNN FE "Causal Conv1d", the paragraph on
 *   transpose views).  Any non-negative strides are accepted; outputs must
 *   not overlap themselves.
 * - An optional tensor is absent when its descriptor pointer is NULL or its
 *   data pointer is NULL.
 * - All memory is owned by the caller.  The library allocates nothing,
 *   keeps no pointer after returning, and holds no handle or state; the
 *   one exception is the fixed device scratch behind ccv_bwd_noalloc,
 *   which is part of the loaded code and never allocated by a call.
 * - Every kernel is launched on `stream` (NULL = the default stream).
 *   Calls are asynchronous: no synchronisation, no device-to-host copy and
 *   no read of device memory on the host (cuDNN FE overview, the stream
 *   convention).
 * - The return value is a status (ccv_status).  Argument checks run on the
 *   host before any launch; when a call returns a negative status nothing
 *   was launched.  Problems with device-resident metadata are reported
 *   through a device flag word, never through the return value.
 * - Arithmetic: inputs are widened exactly to FP32, accumulation is FP32,
 *   and BF16 outputs are rounded to nearest even.
 */
#ifndef CCV_H
#define CCV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CCV_ABI_VERSION 3

typedef enum ccv_dtype {
    CCV_DTYPE_BF16 = 0,
    CCV_DTYPE_F32 = 1,
    CCV_DTYPE_I32 = 2
} ccv_dtype;

typedef enum ccv_activation {
    CCV_ACT_NONE = 0,
    CCV_ACT_SILU = 1
} ccv_activation;

typedef enum ccv_status {
    CCV_OK = 0,
    /* Deterministic dweight was requested with a bias under warn_only: the
     * call ran with FP32 atomics (cuDNN FE "Causal Conv1d", determinism). */
    CCV_WARN_NONDETERMINISTIC = 1,
    /* Bad shape, stride, dtype or pointer; B != 1 with cu_seqlens; both
     * seq_idx and cu_seqlens; B, D, T or N < 1 (empty inputs: PyTorch hands
     * an empty tensor a null data pointer, which reads as absent here); a
     * too-small workspace. */
    CCV_ERR_INVALID_ARG = -1,
    /* An output's byte span overlaps an input's or another output's
     * (cuDNN FE "Causal Conv1d", the paragraph on final_states_out). */
    CCV_ERR_ALIAS = -2,
    /* Declined explicitly (cuDNN FE "Causal Conv1d", the optimized route):
     * state tensors together with seq_idx; FP32 weight with a bias (without
     * CCV_OPT_F32_FILTER_BIAS); a width outside 2..4; an activation other
     * than none or SiLU. */
    CCV_ERR_UNSUPPORTED = -3,
    /* Deterministic dweight requested with a bias, without warn_only and
     * without CCV_OPT_DETERMINISTIC_DBIAS. */
    CCV_ERR_NONDETERMINISTIC = -4,
    /* A HIP launch failed (hipGetLastError after the launch). */
    CCV_ERR_HIP = -5,
    /* ccv_bwd_noalloc: the call needs more scratch than the library holds
     * (CCV_NOALLOC_SCRATCH_BYTES); nothing was launched. */
    CCV_ERR_TOO_LARGE = -6
} ccv_status;

/* Bits of the cu_seqlens flag word (cuDNN FE "Causal Conv1d", the paragraph
 * on device-side validation of packed offsets; "non-increasing" is split
 * into DECREASING (a strict decrease) and EMPTY (two equal offsets)). */
#define CCV_CU_FIRST_NONZERO 0x1u /* cu_seqlens[0] != 0 */
#define CCV_CU_LAST_MISMATCH 0x2u /* cu_seqlens[N] != token total */
#define CCV_CU_DECREASING    0x4u /* cu_seqlens[i+1] <  cu_seqlens[i] */
#define CCV_CU_EMPTY         0x8u /* cu_seqlens[i+1] == cu_seqlens[i] */

/* Option bits (the `options` argument).  Both widen what the pages' route
 * declines (cuDNN FE "Causal Conv1d", the paragraph on the optimized route
 * and the determinism paragraph), so each is opt-in; any other bit is
 * CCV_ERR_INVALID_ARG.
 *   CCV_OPT_F32_FILTER_BIAS      admit an FP32 weight together with an FP32
 *                                bias (ccv_fwd, ccv_bwd, ccv_update).  The
 *                                bias is then FP32 too; a BF16 bias with an
 *                                FP32 weight stays invalid.
 *   CCV_OPT_DETERMINISTIC_DBIAS  (ccv_bwd) with deterministic = 1 and a
 *                                bias, reduce dbias through the workspace
 *                                partials as well, in the same fixed order
 *                                as dweight. */
#define CCV_OPT_F32_FILTER_BIAS     0x1u
#define CCV_OPT_DETERMINISTIC_DBIAS 0x2u

typedef struct ccv_tensor {
    void *data;        /* device pointer; NULL = absent */
    int32_t dtype;     /* ccv_dtype */
    int32_t ndim;      /* number of used entries in shape/stride (1..3) */
    int64_t shape[3];
    int64_t stride[3]; /* in elements, >= 0 */
} ccv_tensor;

/*
 * ccv_fwd — full-sequence forward (cuDNN FE "Causal Conv1d": causal_conv1d).
 *
 *   x               [B,D,T]  BF16, read.
 *   weight          [D,W]    BF16, or FP32 (with a bias only under
 *                            CCV_OPT_F32_FILTER_BIAS); W in 2..4 (the page's
 *                            optimized route is W = 4; 2 and 3 use the same
 *                            kernels built for their width).
 *   bias            [D]      optional; BF16, or FP32 with an FP32 weight
 *                            under CCV_OPT_F32_FILTER_BIAS.
 *   cu_seqlens      [N+1]    I32, optional; packs N sequences along T of a
 *                            B == 1 input.  Mutually exclusive with seq_idx.
 *   seq_idx         [B,T]    I32, optional: the id of the sequence each token
 *                            belongs to; tap k of output t sees position
 *                            t-(W-1)+k only when that token has t's id (a
 *                            reading of the page's compatibility keyword: only
 *                            equality of ids matters).  Mutually exclusive
 *                            with cu_seqlens; with it, initial_states and
 *                            final_states are declined.
 *   initial_states  [R,D,W-1] BF16, optional; R = B dense, N packed.
 *   y               [B,D,T]  BF16, written.  Any layout; usually x's.
 *   final_states    [R,D,W-1] BF16, optional, written.
 *   activation      CCV_ACT_NONE or CCV_ACT_SILU.
 *   options         CCV_OPT_* bits (0 = the pages' route).
 *   err_flag        device uint32, required with cu_seqlens, else ignored.
 *
 * Packed inputs are validated on the device (no host read).  The bits of
 * the violations found are ORed into *err_flag.  The flag is sticky: when
 * it is non-zero at kernel start, or this call's offsets are malformed, the
 * kernels write no output and touch no memory outside the inputs'
 * bounds.  The caller clears the word to resume.
 */
int ccv_fwd(const ccv_tensor *x, const ccv_tensor *weight, const ccv_tensor *bias,
            const ccv_tensor *cu_seqlens, const ccv_tensor *seq_idx,
            const ccv_tensor *initial_states, const ccv_tensor *y,
            const ccv_tensor *final_states, int activation, uint32_t options,
            uint32_t *err_flag, hipStream_t stream);

/*
 * ccv_bwd — backward of L = <dy, y> + <dfinal_states, final_states>
 * (cuDNN FE "Causal Conv1d": the optimized route covers backward with the
 * W-1 initial and final state; the determinism paragraph).
 *
 *   x, weight, bias, cu_seqlens, seq_idx, initial_states: as in ccv_fwd
 *                   (with seq_idx, dfinal_states is declined).
 *   dy              [B,D,T]  BF16, read.
 *   dfinal_states   [R,D,W-1] BF16, optional, read.
 *   dx              [B,D,T]  BF16, written.
 *   dweight         [D,W]    FP32, ACCUMULATED into (+=), like an autograd
 *                            .grad; zero it first for a plain gradient.
 *   dbias           [D]      FP32, accumulated into; required iff bias is
 *                            given.
 *   dinitial_states [R,D,W-1] BF16, written; optional, only with
 *                            initial_states.
 *   deterministic   0: dweight/dbias accumulate with FP32 atomics (not
 *                   bitwise reproducible).  1: bias-free calls write unique
 *                   FP32 partials into the workspace and add their sum, taken
 *                   in a fixed order, to dweight (bit-exact run to run for
 *                   the same starting dweight); with a bias the call
 *                   returns CCV_ERR_NONDETERMINISTIC, or, with warn_only,
 *                   runs with atomics and returns CCV_WARN_NONDETERMINISTIC,
 *                   or, under CCV_OPT_DETERMINISTIC_DBIAS, reduces dbias
 *                   through the partials too (W+1 columns per channel).
 *   options         CCV_OPT_* bits.
 *   workspace / workspace_bytes:
 *                   query: workspace == NULL and workspace_bytes != NULL
 *                   -> *workspace_bytes = bytes needed, CCV_OK, nothing
 *                   launched.  Run: workspace_bytes == NULL, or workspace
 *                   != NULL with *workspace_bytes >= the bytes needed.  The
 *                   workspace is device memory, 256-byte aligned.
 *   err_flag        as in ccv_fwd.
 */
int ccv_bwd(const ccv_tensor *x, const ccv_tensor *weight, const ccv_tensor *bias,
            const ccv_tensor *cu_seqlens, const ccv_tensor *seq_idx,
            const ccv_tensor *initial_states, const ccv_tensor *dy,
            const ccv_tensor *dfinal_states, const ccv_tensor *dx,
            const ccv_tensor *dweight, const ccv_tensor *dbias,
            const ccv_tensor *dinitial_states, int activation, int deterministic,
            int warn_only, uint32_t options, void *workspace, size_t *workspace_bytes,
            uint32_t *err_flag, hipStream_t stream);

/*
 * ccv_bwd_noalloc — ccv_bwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The arguments and results are those of ccv_bwd without the
 * workspace: the deterministic route writes its partials to a scratch array
 * the library keeps in device memory, CCV_NOALLOC_SCRATCH_BYTES on each
 * device it runs on, for the life of the process.  The call itself allocates
 * nothing (its first call on a device looks up that device's scratch
 * address).
 *
 *   Limit: a deterministic call whose partials exceed the scratch (ccv_bwd's
 *   workspace query gives the size) returns CCV_ERR_TOO_LARGE before any
 *   launch.  The atomic route uses no scratch and has no limit.
 *   Sharing: every call on one device uses the same scratch; calls that
 *   overlap in time on one device (two streams, two threads) race and must
 *   be serialised by the caller.  Nothing in the scratch has to start at
 *   zero: a call writes every partial it reads.
 */
#define CCV_NOALLOC_SCRATCH_BYTES (32u << 20)
int ccv_bwd_noalloc(const ccv_tensor *x, const ccv_tensor *weight, const ccv_tensor *bias,
                    const ccv_tensor *cu_seqlens, const ccv_tensor *seq_idx,
                    const ccv_tensor *initial_states, const ccv_tensor *dy,
                    const ccv_tensor *dfinal_states, const ccv_tensor *dx,
                    const ccv_tensor *dweight, const ccv_tensor *dbias,
                    const ccv_tensor *dinitial_states, int activation, int deterministic,
                    int warn_only, uint32_t options, uint32_t *err_flag, hipStream_t stream);

/*
 * ccv_update — decode step (cuDNN FE "Causal Conv1d": the returned
 * width-four final_states feed causal_conv1d_update, which mutates the state
 * in place with no layout conversion).  One token, or L tokens in order
 * (exactly L single-token steps).
 *
 *   x           [B,D]      BF16, the new token, read; or [B,D,L], L >= 1
 *                          tokens (oldest first), read.
 *   conv_state  [B,D,W-1]  BF16, read and written in place: the state
 *                          (s_0..s_{W-2}, oldest first) becomes
 *                          (s_1..s_{W-2}, x): the last W-1 entries of
 *                          (state, tokens).
 *   weight      [D,W]      BF16 or FP32; W in 2..4.
 *   bias        [D]        optional; as in ccv_fwd (FP32 with an FP32
 *                          weight under CCV_OPT_F32_FILTER_BIAS).
 *   y           x's shape, BF16, written: act(bias + sum_k w_k v_k) over
 *                          v = (s_0..s_{W-2}, x) for each token in turn.
 *                          Must not overlap any other argument.
 */
int ccv_update(const ccv_tensor *x, const ccv_tensor *conv_state, const ccv_tensor *weight,
               const ccv_tensor *bias, const ccv_tensor *y, int activation, uint32_t options,
               hipStream_t stream);

/*
 * ccv_validate_cu_seqlens — device-side check of packed offsets (cuDNN FE
 * "Causal Conv1d", the paragraph on device-side validation).
 *
 *   cu_seqlens    device int32[n_seqs + 1], read.
 *   n_seqs        N >= 1.
 *   total_tokens  the token total the last offset must equal (T >= 1).
 *   flags         device uint32, OVERWRITTEN with the CCV_CU_* bit mask
 *                 (0 = well formed).  Read it after synchronising the stream.
 */
int ccv_validate_cu_seqlens(const int32_t *cu_seqlens, int64_t n_seqs, int64_t total_tokens,
                            uint32_t *flags, hipStream_t stream);

/* Library version (CCV_ABI_VERSION) and a static name for a status code. */
int ccv_abi_version(void);
const char *ccv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CCV_H */

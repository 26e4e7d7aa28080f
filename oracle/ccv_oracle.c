/*
 * ccv_oracle.c — plain fp64 CPU oracle for the depthwise causal conv1d.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never links, includes or calls anything here, and nothing here includes
 * or calls the GPU library.
 *
 * What is computed (cuDNN FE "Causal Conv1d" page, the bullet list of tensor
 * and state semantics and the paragraph on the optimized route):
 *
 *   z[b,d,t] = sum_{k=0}^{W-1} w[d,k] * x_ext[b,d,t-(W-1)+k]   (+ bias[d])
 *   y        = act(z),  act in {identity, SiLU}
 *
 * where x_ext extends each row (a batch row when dense, a sequence when
 * packed by cu_seqlens) to the left with its W-1 initial-state values
 * (oldest first) or with zeros when no initial state is given.  The tap
 * order is PyTorch's cross-correlation after a left pad of W-1: tap W-1
 * multiplies the current token and tap 0 the oldest (POPCORNBENCH causal
 * conv1d trace, the derivation of the causal left pad, which settles that
 * the last kernel tap meets input position t).
 *
 * Everything is written as the definition, in the order the definition
 * states it: exact widening of the inputs to double, sequential sums
 * "acc = 0; acc += w[k] * v[k] for k = 0..W-1; acc += bias", the logistic
 * function through exp() in double.  No blocking, no fusion, no reordering.
 *
 * All arrays are dense, row-major, in the logical index order of the
 * pages' shapes:
 *   x, y, dy, dx      [B][D][T]
 *   w, dw             [D][W]
 *   bias, dbias       [D]
 *   init/final/dinit/dfinal states   [R][D][W-1]
 *                     R = B (dense) or N = len(cu_seqlens)-1 (packed, B==1)
 *   update: x, y      [B][D];  state [B][D][W-1]
 *
 * Every function returns 0 on success and a negative value on an argument
 * it cannot handle (the oracle checks nothing else; metadata validity is
 * the caller's concern, except for oracle_validate_cu_seqlens).
 */
#include "ccv_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* ---- activations (cuDNN FE "Causal Conv1d": activation="silu") ---------- */

/* SiLU(z) = z * logistic(z) = z / (1 + e^{-z}). */
static double act_value(int act, double z)
{
    if (act == ORACLE_ACT_SILU)
        return z / (1.0 + exp(-z));
    return z;
}

/* d/dz SiLU(z) = s + z s (1 - s) with s = 1/(1+e^{-z}); identity' = 1. */
static double act_slope(int act, double z)
{
    if (act == ORACLE_ACT_SILU) {
        double s = 1.0 / (1.0 + exp(-z));
        return s * (1.0 + z * (1.0 - s));
    }
    return 1.0;
}

/* ---- row geometry ------------------------------------------------------- */

/* The row that holds global position t of batch b.
 * Dense: row b spans [0, T).  Packed (B == 1): row i spans
 * [cu[i], cu[i+1]); the row is found by a plain linear scan. */
typedef struct { int64_t r, s, e; } row_t;

static row_t row_of(int64_t b, int64_t t, int64_t T, const int32_t *cu, int64_t N)
{
    row_t row;
    if (!cu) {
        row.r = b; row.s = 0; row.e = T;
        return row;
    }
    int64_t i = 0;
    while (i + 1 < N && (int64_t)cu[i + 1] <= t)
        ++i;
    row.r = i; row.s = cu[i]; row.e = cu[i + 1];
    return row;
}

static row_t row_by_index(int64_t r, int64_t T, const int32_t *cu)
{
    row_t row;
    row.r = r;
    if (!cu) { row.s = 0; row.e = T; }
    else     { row.s = cu[r]; row.e = cu[r + 1]; }
    return row;
}

/* x_ext at global position p for row `row` of batch b, channel d:
 * p >= s: the input itself; p < s: initial state slot p - s + (W-1)
 * (oldest first), or 0 when no initial state is given. */
static double x_ext(const double *x, const double *init, int64_t b, int64_t d,
                    int64_t p, row_t row, int64_t D, int64_t T, int64_t W)
{
    if (p >= row.s)
        return x[(b * D + d) * T + p];
    if (!init)
        return 0.0;
    int64_t j = p - row.s + (W - 1);
    return init[(row.r * D + d) * (W - 1) + j];
}

/* The pre-activation z at position t (definition above, canonical order). */
static double pre_act(const double *x, const double *w, const double *bias,
                      const double *init, int64_t b, int64_t d, int64_t t,
                      row_t row, int64_t D, int64_t T, int64_t W)
{
    double acc = 0.0;
    for (int64_t k = 0; k < W; ++k)
        acc += w[d * W + k] * x_ext(x, init, b, d, t - (W - 1) + k, row, D, T, W);
    if (bias)
        acc += bias[d];
    return acc;
}

static int check_shape(int64_t B, int64_t D, int64_t T, int64_t W,
                       const int32_t *cu, int64_t N)
{
    if (B < 1 || D < 1 || T < 0 || W < 1)
        return -1;
    if (cu && (B != 1 || N < 1))
        return -1;
    return 0;
}

/* ---- forward ------------------------------------------------------------ */

int oracle_fwd(int64_t B, int64_t D, int64_t T, int64_t W,
               const double *x, const double *w, const double *bias,
               const int32_t *cu, int64_t N, const double *init, int act,
               double *y, double *final_states)
{
    if (check_shape(B, D, T, W, cu, N))
        return -1;
    /* Outputs, one global position at a time (packed rows by lookup). */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d)
            for (int64_t t = 0; t < T; ++t) {
                row_t row = row_of(b, t, T, cu, N);
                double z = pre_act(x, w, bias, init, b, d, t, row, D, T, W);
                y[(b * D + d) * T + t] = act_value(act, z);
            }
    /* Final state: the last W-1 entries of each extended row, oldest first
     * (cuDNN FE "Causal Conv1d": returned final_states[.., W-1]). */
    if (final_states && W > 1) {
        int64_t R = cu ? N : B;
        for (int64_t r = 0; r < R; ++r) {
            row_t row = row_by_index(r, T, cu);
            int64_t b = cu ? 0 : r;
            for (int64_t d = 0; d < D; ++d)
                for (int64_t j = 0; j < W - 1; ++j)
                    final_states[(r * D + d) * (W - 1) + j] =
                        x_ext(x, init, b, d, row.e - (W - 1) + j, row, D, T, W);
        }
    }
    return 0;
}

/* ---- backward ----------------------------------------------------------- */

/* Gradient of L = sum dy * y + sum dfinal * final_states with respect to
 * x, w, bias and the initial states.
 *   g[t]        = dy[t] * act'(z[t])
 *   dx_ext[tau] = sum_k w[d,k] * g[tau + (W-1) - k]   over in-row terms
 *                 + dfinal[.., j] where tau = e - (W-1) + j
 *   dx[t]       = dx_ext[t]  (t inside the row)
 *   dinit[.., j]= dx_ext[s - (W-1) + j]
 *   dw[d,k]     = sum over all rows and t of g[t] * x_ext[t - (W-1) + k]
 *   dbias[d]    = sum over all rows and t of g[t]                        */

static double grad_out(const double *x, const double *w, const double *bias,
                       const double *init, const double *dy, int act,
                       int64_t b, int64_t d, int64_t t, row_t row,
                       int64_t D, int64_t T, int64_t W)
{
    double z = pre_act(x, w, bias, init, b, d, t, row, D, T, W);
    return dy[(b * D + d) * T + t] * act_slope(act, z);
}

/* dx_ext at position tau of row `row` (tau in [s-(W-1), e)). */
static double dx_ext_at(const double *x, const double *w, const double *bias,
                        const double *init, const double *dy,
                        const double *dfinal, int act, int64_t b, int64_t d,
                        int64_t tau, row_t row, int64_t D, int64_t T, int64_t W)
{
    double acc = 0.0;
    for (int64_t k = 0; k < W; ++k) {
        int64_t t = tau + (W - 1) - k;
        if (t >= row.s && t < row.e)
            acc += w[d * W + k] * grad_out(x, w, bias, init, dy, act, b, d, t, row, D, T, W);
    }
    if (dfinal) {
        int64_t j = tau - (row.e - (W - 1));
        if (j >= 0 && j < W - 1)
            acc += dfinal[(row.r * D + d) * (W - 1) + j];
    }
    return acc;
}

int oracle_bwd(int64_t B, int64_t D, int64_t T, int64_t W,
               const double *x, const double *w, const double *bias,
               const int32_t *cu, int64_t N, const double *init,
               const double *dy, const double *dfinal, int act,
               double *dx, double *dw, double *dbias, double *dinit)
{
    if (check_shape(B, D, T, W, cu, N))
        return -1;
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t k = 0; k < W; ++k)
            dw[d * W + k] = 0.0;
        if (dbias)
            dbias[d] = 0.0;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d)
            for (int64_t t = 0; t < T; ++t) {
                row_t row = row_of(b, t, T, cu, N);
                dx[(b * D + d) * T + t] =
                    dx_ext_at(x, w, bias, init, dy, dfinal, act, b, d, t, row, D, T, W);
                double g = grad_out(x, w, bias, init, dy, act, b, d, t, row, D, T, W);
                for (int64_t k = 0; k < W; ++k)
                    dw[d * W + k] += g * x_ext(x, init, b, d, t - (W - 1) + k, row, D, T, W);
                if (dbias)
                    dbias[d] += g;
            }
    if (dinit && W > 1) {
        int64_t R = cu ? N : B;
        for (int64_t r = 0; r < R; ++r) {
            row_t row = row_by_index(r, T, cu);
            int64_t b = cu ? 0 : r;
            for (int64_t d = 0; d < D; ++d)
                for (int64_t j = 0; j < W - 1; ++j)
                    dinit[(r * D + d) * (W - 1) + j] =
                        dx_ext_at(x, w, bias, init, dy, dfinal, act, b, d,
                                  row.s - (W - 1) + j, row, D, T, W);
        }
    }
    return 0;
}

/* ---- per-token sequence ids (seq_idx) ----------------------------------- */
/*
 * cuDNN FE "Causal Conv1d": the tensor list names a seq_idx[B, T] keyword,
 * kept for compatibility and mutually exclusive with cu_seqlens, i.e. a
 * second way to pack several sequences into one row: seq[b][t] is the id of
 * the sequence that token t of row b belongs to.  The page gives no further
 * semantics; the reading taken here is the plainest one: tap k of output t
 * sees input position p = t-(W-1)+k only when p >= 0 and seq[b][p] ==
 * seq[b][t]; any other tap sees zero.  With ids that are constant over
 * contiguous runs this is the packed route with zero initial states, one
 * sequence per run.  No state tensors go with seq_idx.
 */

/* x at position p as seen from output position t (row b, channel d). */
static double x_seen(const double *x, const int32_t *seq, int64_t b, int64_t d,
                     int64_t p, int64_t t, int64_t D, int64_t T)
{
    if (p < 0 || seq[b * T + p] != seq[b * T + t])
        return 0.0;
    return x[(b * D + d) * T + p];
}

static double pre_act_seq(const double *x, const double *w, const double *bias,
                          const int32_t *seq, int64_t b, int64_t d, int64_t t,
                          int64_t D, int64_t T, int64_t W)
{
    double acc = 0.0;
    for (int64_t k = 0; k < W; ++k)
        acc += w[d * W + k] * x_seen(x, seq, b, d, t - (W - 1) + k, t, D, T);
    if (bias)
        acc += bias[d];
    return acc;
}

int oracle_fwd_seq(int64_t B, int64_t D, int64_t T, int64_t W,
                   const double *x, const double *w, const double *bias,
                   const int32_t *seq, int act, double *y)
{
    if (B < 1 || D < 1 || T < 0 || W < 1 || !seq)
        return -1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d)
            for (int64_t t = 0; t < T; ++t)
                y[(b * D + d) * T + t] =
                    act_value(act, pre_act_seq(x, w, bias, seq, b, d, t, D, T, W));
    return 0;
}

/* Gradient of L = sum dy * y for the forward above:
 *   g[t]     = dy[t] * act'(z[t])
 *   dx[p]    = sum_k w[d,k] * g[t] over t = p + (W-1) - k < T with
 *              seq[t] == seq[p]   (the taps that saw x[p])
 *   dw[d,k]  = sum_t g[t] * (x[t-(W-1)+k] as seen from t)
 *   dbias[d] = sum_t g[t]                                                   */
int oracle_bwd_seq(int64_t B, int64_t D, int64_t T, int64_t W,
                   const double *x, const double *w, const double *bias,
                   const int32_t *seq, const double *dy, int act,
                   double *dx, double *dw, double *dbias)
{
    if (B < 1 || D < 1 || T < 0 || W < 1 || !seq)
        return -1;
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t k = 0; k < W; ++k)
            dw[d * W + k] = 0.0;
        if (dbias)
            dbias[d] = 0.0;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d)
            for (int64_t p = 0; p < T; ++p) {
                double acc = 0.0;
                for (int64_t k = 0; k < W; ++k) {
                    int64_t t = p + (W - 1) - k;
                    if (t < T && seq[b * T + t] == seq[b * T + p]) {
                        double z = pre_act_seq(x, w, bias, seq, b, d, t, D, T, W);
                        acc += w[d * W + k] * dy[(b * D + d) * T + t] * act_slope(act, z);
                    }
                }
                dx[(b * D + d) * T + p] = acc;
            }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d)
            for (int64_t t = 0; t < T; ++t) {
                double z = pre_act_seq(x, w, bias, seq, b, d, t, D, T, W);
                double g = dy[(b * D + d) * T + t] * act_slope(act, z);
                for (int64_t k = 0; k < W; ++k)
                    dw[d * W + k] += g * x_seen(x, seq, b, d, t - (W - 1) + k, t, D, T);
                if (dbias)
                    dbias[d] += g;
            }
    return 0;
}

/* ---- single-token update ------------------------------------------------ */

/* cuDNN FE "Causal Conv1d", the paragraph on causal_conv1d_update: the state
 * holds the previous W-1 tokens, oldest first; the new token x is appended,
 * the output is act(bias + sum_k w[k] * v[k]) over v = (state, x), and the
 * state becomes the last W-1 entries of v, in place. */
int oracle_update(int64_t B, int64_t D, int64_t W,
                  const double *x, double *state, const double *w,
                  const double *bias, int act, double *y)
{
    if (B < 1 || D < 1 || W < 1)
        return -1;
    double *v = (double *)malloc((size_t)W * sizeof(double));
    if (!v)
        return -2;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d) {
            double *s = state + (b * D + d) * (W - 1);
            for (int64_t k = 0; k < W - 1; ++k)
                v[k] = s[k];
            v[W - 1] = x[b * D + d];
            double acc = 0.0;
            for (int64_t k = 0; k < W; ++k)
                acc += w[d * W + k] * v[k];
            if (bias)
                acc += bias[d];
            y[b * D + d] = act_value(act, acc);
            for (int64_t k = 0; k < W - 1; ++k)
                s[k] = v[k + 1];
        }
    free(v);
    return 0;
}

/* ---- cu_seqlens validation ---------------------------------------------- */

/* cuDNN FE "Causal Conv1d", the paragraph on device-side validation: the
 * offsets are malformed when the first is not zero, the last is not the
 * token total, they decrease, or a sequence is empty.  "Non-increasing" is
 * split into two independent bits: a strict decrease and an equal pair. */
uint32_t oracle_validate_cu_seqlens(const int32_t *cu, int64_t N, int64_t total)
{
    uint32_t flags = 0;
    if (N < 1)
        return ORACLE_CU_EMPTY;
    if (cu[0] != 0)
        flags |= ORACLE_CU_FIRST_NONZERO;
    if ((int64_t)cu[N] != total)
        flags |= ORACLE_CU_LAST_MISMATCH;
    for (int64_t i = 0; i < N; ++i) {
        if (cu[i + 1] < cu[i])
            flags |= ORACLE_CU_DECREASING;
        if (cu[i + 1] == cu[i])
            flags |= ORACLE_CU_EMPTY;
    }
    return flags;
}

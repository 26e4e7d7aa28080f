/*
 * ccv_oracle.h — fp64 CPU oracle for the depthwise causal conv1d.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).
 * Shares no code, header or constant with the GPU library.
 * Layouts and semantics are documented in ccv_oracle.c.
 */
#ifndef CCV_ORACLE_H
#define CCV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_SILU 1

#define ORACLE_CU_FIRST_NONZERO 1u
#define ORACLE_CU_LAST_MISMATCH 2u
#define ORACLE_CU_DECREASING    4u
#define ORACLE_CU_EMPTY         8u

int oracle_fwd(int64_t B, int64_t D, int64_t T, int64_t W,
               const double *x, const double *w, const double *bias,
               const int32_t *cu, int64_t N, const double *init, int act,
               double *y, double *final_states);

int oracle_bwd(int64_t B, int64_t D, int64_t T, int64_t W,
               const double *x, const double *w, const double *bias,
               const int32_t *cu, int64_t N, const double *init,
               const double *dy, const double *dfinal, int act,
               double *dx, double *dw, double *dbias, double *dinit);

int oracle_fwd_seq(int64_t B, int64_t D, int64_t T, int64_t W,
                   const double *x, const double *w, const double *bias,
                   const int32_t *seq, int act, double *y);

int oracle_bwd_seq(int64_t B, int64_t D, int64_t T, int64_t W,
                   const double *x, const double *w, const double *bias,
                   const int32_t *seq, const double *dy, int act,
                   double *dx, double *dw, double *dbias);

int oracle_update(int64_t B, int64_t D, int64_t W,
                  const double *x, double *state, const double *w,
                  const double *bias, int act, double *y);

uint32_t oracle_validate_cu_seqlens(const int32_t *cu, int64_t N, int64_t total);

#ifdef __cplusplus
}
#endif

#endif

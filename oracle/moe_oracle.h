/*
 * moe_oracle.h -- declarations of the CPU fp64 oracle (moe_oracle.c).
 *
 * TEST INFRASTRUCTURE ONLY: for the tests' native programs.  The GPU library
 * never includes this header nor links the oracle.
 *
 * dtype: ORACLE_F32 (binary32 inputs) or ORACLE_BF16 (bfloat16 bit patterns).
 * Layouts as in the GPU library: x [T,d], w_router [d,E], w1 and w3 [E,d,f],
 * w2 [E,f,d], all row-major.  Results are double.  Each returns 0 on success.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

int oracle_num_threads(void);

/* Routing of every token: logits [T,E] (may be NULL), ids [T,k], gates [T,k]. */
int oracle_route(const void *x, const void *w_router, const float *bias, int dtype,
                 int64_t T, int64_t d, int64_t E, int64_t k,
                 double *logits, int32_t *ids, double *gates);

/*
 * The layer on n tokens (tokens == NULL: tokens 0..n-1): ids [n,k] and
 * gates [n,k] (inputs when forced != 0), out [n,d], optional y [n,k,d] and
 * h [n,k,f].
 */
int oracle_moe_tokens(const void *x, const void *w_router, const float *bias,
                      const void *w1, const void *w3, const void *w2, int dtype,
                      int64_t T, int64_t d, int64_t f, int64_t E, int64_t k,
                      const int64_t *tokens, int64_t n, int forced,
                      int32_t *ids, double *gates, double *out, double *y, double *h);

/* Unit-gain RMSNorm of each row of h [T,d]: out [T,d]. */
int oracle_rmsnorm(const void *hsrc, int dtype, int64_t T, int64_t d, double eps, double *out);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */

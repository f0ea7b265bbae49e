/*
 * moe_abi_check.c -- the layer driven from a plain C program through the C ABI
 * of libmoe_ffn.so (no Python), checked against the CPU oracle.
 *
 * Test infrastructure: built by __graft_entry__.build() (gcc, linked against
 * the HIP runtime, libmoe_ffn.so and the oracle) and run on a GPU by
 * tests/test_gpu_zz_native.py.  Prints one line per check and exits 0 only if
 * every check passed.
 *
 * Inputs come from a seeded splitmix64 stream (Box-Muller normals), the same
 * bits handed to the GPU and to the oracle.  Acceptance as in the Python
 * parity tests: expert ids equal wherever the oracle's k-th / (k+1)-th logit
 * gap exceeds 1e-3, outputs within tol * max|ref| on those tokens (tol 2e-2
 * for bf16 storage, 1e-4 for fp32).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_ffn.h"
#include "moe_oracle.h"

static int g_failures = 0;

static void check(int ok, const char *what)
{
    printf("[%s] %s\n", ok ? "ok" : "FAIL", what);
    fflush(stdout);
    if (!ok)
        ++g_failures;
}

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            printf("[FAIL] %s: %s\n", #call, hipGetErrorString(e_));              \
            exit(2);                                                              \
        }                                                                         \
    } while (0)

static uint64_t splitmix64(uint64_t *s)
{
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double normal01(uint64_t *s)
{
    double u1 = ((splitmix64(s) >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
    double u2 = (splitmix64(s) >> 11) * 0x1.0p-53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static uint16_t bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* n normals of standard deviation sd, as bf16 bits or fp32. */
static void *make_tensor(int64_t n, double sd, int bf16, uint64_t seed)
{
    uint64_t s = seed;
    void *p = malloc((size_t)n * (bf16 ? 2 : 4));
    for (int64_t i = 0; i < n; ++i) {
        float v = (float)(sd * normal01(&s));
        if (bf16)
            ((uint16_t *)p)[i] = bf16_bits(v);
        else
            ((float *)p)[i] = v;
    }
    return p;
}

static void *to_device(const void *h, size_t bytes)
{
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}

static int cmp_int(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

static int cmp_desc(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

/* One layer through moe_ffn_forward_ex (and the plain entry point) against
 * the oracle. */
static void run_case(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k, int bf16,
                     uint64_t seed)
{
    char what[256];
    const size_t es = bf16 ? 2 : 4;
    void *x = make_tensor(T * d, 1.0, bf16, seed + 1);
    void *wr = make_tensor(d * E, 1.0 / sqrt((double)d), bf16, seed + 2);
    void *w1 = make_tensor(E * d * f, 1.0 / sqrt((double)d), bf16, seed + 3);
    void *w3 = make_tensor(E * d * f, 1.0 / sqrt((double)d), bf16, seed + 4);
    void *w2 = make_tensor(E * f * d, 1.0 / sqrt((double)f), bf16, seed + 5);

    void *dx = to_device(x, (size_t)T * d * es);
    void *dwr = to_device(wr, (size_t)d * E * es);
    void *dw1 = to_device(w1, (size_t)E * d * f * es);
    void *dw3 = to_device(w3, (size_t)E * d * f * es);
    void *dw2 = to_device(w2, (size_t)E * f * d * es);
    void *dout = NULL, *dout2 = NULL, *dids = NULL;
    HIP_OK(hipMalloc(&dout, (size_t)T * d * es));
    HIP_OK(hipMalloc(&dout2, (size_t)T * d * es));
    HIP_OK(hipMalloc(&dids, (size_t)T * k * 4));

    moe_ffn_opts_t opts;
    memset(&opts, 0, sizeof opts);
    opts.dtype = bf16 ? MOE_DTYPE_BF16 : MOE_DTYPE_F32;
    opts.topk_ids = (int32_t *)dids;
    moe_status_t st = moe_ffn_forward_ex(dx, dwr, dw1, dw3, dw2, T, d, f, E, k, dout, NULL, &opts);
    snprintf(what, sizeof what, "T=%lld d=%lld f=%lld E=%lld k=%lld %s: moe_ffn_forward_ex status %d",
             (long long)T, (long long)d, (long long)f, (long long)E, (long long)k,
             bf16 ? "bf16" : "fp32", (int)st);
    check(st == MOE_OK, what);
    if (bf16)
        st = moe_ffn_forward(dx, dwr, dw1, dw3, dw2, T, d, f, E, k, dout2, NULL);
    else
        st = moe_ffn_forward_f32((const float *)dx, (const float *)dwr, (const float *)dw1,
                                 (const float *)dw3, (const float *)dw2, T, d, f, E, k,
                                 (float *)dout2, NULL);
    check(st == MOE_OK, "  plain entry point status");
    HIP_OK(hipDeviceSynchronize());

    void *out = malloc((size_t)T * d * es);
    void *out2 = malloc((size_t)T * d * es);
    int32_t *ids = (int32_t *)malloc((size_t)T * k * 4);
    HIP_OK(hipMemcpy(out, dout, (size_t)T * d * es, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out2, dout2, (size_t)T * d * es, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ids, dids, (size_t)T * k * 4, hipMemcpyDeviceToHost));
    check(memcmp(out, out2, (size_t)T * d * es) == 0, "  plain and _ex entry points give the same bits");

    const int odt = bf16 ? ORACLE_BF16 : ORACLE_F32;
    double *logits = (double *)malloc((size_t)T * E * sizeof(double));
    int32_t *oids = (int32_t *)malloc((size_t)T * k * 4);
    double *ogates = (double *)malloc((size_t)T * k * sizeof(double));
    double *oout = (double *)malloc((size_t)T * d * sizeof(double));
    int rc = oracle_route(x, wr, NULL, odt, T, d, E, k, logits, oids, ogates);
    rc |= oracle_moe_tokens(x, wr, NULL, w1, w3, w2, odt, T, d, f, E, k, NULL, T, 0, oids, ogates,
                            oout, NULL, NULL);
    check(rc == 0, "  oracle ran");

    int64_t exempt = 0, id_mismatch = 0;
    double max_ref = 0.0, max_err = 0.0;
    double *srt = (double *)malloc((size_t)E * sizeof(double));
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < d; ++c)
            if (fabs(oout[t * d + c]) > max_ref)
                max_ref = fabs(oout[t * d + c]);
    for (int64_t t = 0; t < T; ++t) {
        memcpy(srt, logits + t * E, (size_t)E * sizeof(double));
        qsort(srt, (size_t)E, sizeof(double), cmp_desc);
        if (k < E && srt[k - 1] - srt[k] <= 1e-3) {
            ++exempt;
            continue;
        }
        int32_t a[64], b[64];
        memcpy(a, ids + t * k, (size_t)k * 4);
        memcpy(b, oids + t * k, (size_t)k * 4);
        qsort(a, (size_t)k, 4, cmp_int);
        qsort(b, (size_t)k, 4, cmp_int);
        if (memcmp(a, b, (size_t)k * 4) != 0) {
            ++id_mismatch;
            continue;
        }
        for (int64_t c = 0; c < d; ++c) {
            const double g = bf16 ? bf16_value(((uint16_t *)out)[t * d + c])
                                  : (double)((float *)out)[t * d + c];
            const double e = fabs(g - oout[t * d + c]);
            if (e > max_err)
                max_err = e;
        }
    }
    snprintf(what, sizeof what, "  expert ids match the oracle off near ties (%lld exempt, %lld differ)",
             (long long)exempt, (long long)id_mismatch);
    check(id_mismatch == 0, what);
    const double tol = bf16 ? 2e-2 : 1e-4;
    snprintf(what, sizeof what, "  max|err| / max|ref| = %.3g (bar %.0e)", max_err / max_ref, tol);
    check(max_err <= tol * max_ref, what);

    free(srt);
    free(logits);
    free(oids);
    free(ogates);
    free(oout);
    free(out);
    free(out2);
    free(ids);
    free(x);
    free(wr);
    free(w1);
    free(w3);
    free(w2);
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dwr));
    HIP_OK(hipFree(dw1));
    HIP_OK(hipFree(dw3));
    HIP_OK(hipFree(dw2));
    HIP_OK(hipFree(dout));
    HIP_OK(hipFree(dout2));
    HIP_OK(hipFree(dids));
}

int main(void)
{
    int n = 0;
    HIP_OK(hipGetDeviceCount(&n));
    if (n < 1) {
        printf("[FAIL] no GPU\n");
        return 2;
    }
    HIP_OK(hipSetDevice(0));
    printf("library %s, oracle threads %d\n", moe_ffn_version(), oracle_num_threads());

    /* argument checking through the ABI */
    check(moe_ffn_forward(NULL, NULL, NULL, NULL, NULL, 0, 128, 128, 8, 2, NULL, NULL) == MOE_OK,
          "T = 0 is a no-op");
    check(moe_ffn_forward(NULL, NULL, NULL, NULL, NULL, 4, 128, 128, 2, 3, NULL, NULL) ==
              MOE_ERR_UNSUPPORTED && moe_ffn_last_error()[0] != '\0',
          "k > E is refused with a message");

    run_case(300, 256, 512, 8, 2, 1, 100);  /* 256-row tile GEMMs */
    run_case(20, 256, 512, 8, 2, 1, 200);   /* streamed-weight GEMMs */
    run_case(150, 192, 320, 16, 4, 1, 300); /* E = 16, k = 4 */
    run_case(64, 128, 256, 8, 2, 0, 400);   /* fp32 */
    moe_ffn_release_workspace();

    printf("%s: %d failure(s)\n", g_failures ? "FAILED" : "PASSED", g_failures);
    return g_failures ? 1 : 0;
}

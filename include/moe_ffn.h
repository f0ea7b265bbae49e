/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts
 * feed-forward library, libmoe_ffn.so.
 *
 * The layer (Mixtral of Experts, wikillm.com card, "Method", sparse MoE layer
 * of section 2.1, the moe_feed_forward and swiglu_expert pseudocode):
 *   logits = x . w_router                       bias-free linear router
 *   ids    = the k largest logits               section 2.1 display 2
 *   g      = softmax over those k logits only   section 2.1 display 2
 *   out    = sum_j g_j * w2[ids_j] . (SiLU(x . w1[ids_j]) * (x . w3[ids_j]))
 *                                               section 2.1 displays 1 and 3
 * applied to a whole batch at once, grouped by expert, with no capacity
 * limit: every token is processed by exactly k experts ("Method": steps for
 * one token, and "Pitfalls": no capacity limit or token dropping).
 *
 * Conventions for every entry point:
 *   - Tensors are dense row-major device pointers owned by the caller:
 *       x [T,d], w_router [d,E], w1 [E,d,f], w3 [E,d,f], w2 [E,f,d], out [T,d].
 *     The pages write the same products as W.x with transposed shapes.
 *   - Element type: bfloat16 for moe_ffn_forward, binary32 for
 *     moe_ffn_forward_f32, either for moe_ffn_forward_ex (opts->dtype).
 *     bf16 paths accumulate in fp32; router logits, top-k and softmax are fp32.
 *   - Top-k ties break toward the lower expert index; the k picks are stored
 *     by descending logit.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the default
 *     stream) and return without waiting for the GPU.  Nothing is copied back
 *     to the host inside a call, so a call can be captured in a HIP graph
 *     once its workspace exists (pass one via moe_ffn_forward_ex).
 *   - `out` is overwritten.  out == x is allowed; out must not overlap a weight.
 *   - Validation happens before any GPU work:
 *       T == 0                                   -> MOE_OK, nothing enqueued
 *       NULL tensor pointer with T > 0, or d, f, E, k < 1, or T < 0
 *                                                -> MOE_ERR_INVALID_ARG
 *       k > E, E > 64, d or f not a multiple of 64 (bf16) or of 4 (fp32),
 *       a pointer not 16-byte aligned            -> MOE_ERR_UNSUPPORTED
 *     A failing HIP call returns MOE_ERR_HIP; a failed workspace allocation
 *     MOE_ERR_OUT_OF_MEMORY.  moe_ffn_last_error() then describes it.
 *   - Inputs must be finite; non-finite values give undefined results.
 *   - The library keeps one cached workspace per device, grown on demand.
 *     Calls that use it from several host threads or streams at once race;
 *     such callers pass their own workspace through moe_ffn_forward_ex.
 *   - Tuning overrides, read once per process from the environment (unset or
 *     0: the library's own choice; results stay within the same tolerance,
 *     only the summation split changes): MOE_FFN_STREAM_SPLITS = K slices of
 *     the second expert GEMM on the few-rows-per-expert path (1..16, clamped
 *     to f/128; the workspace grows by one T*k x d fp32 slice each), and
 *     MOE_FFN_STREAM_K_WAVES = 1, 2 or 4 wavefronts splitting K per 128-column
 *     slab in its first GEMM (at most 12 rows per expert).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_HIP = 3,
    MOE_ERR_OUT_OF_MEMORY = 4
} moe_status_t;

typedef enum { MOE_DTYPE_BF16 = 0, MOE_DTYPE_F32 = 1 } moe_dtype_t;

/*
 * The whole layer in bfloat16 (fp32 accumulation).  Mixtral of Experts,
 * wikillm.com card, "Method", section 2.1 displays 1-3 and the pseudocode.
 */
moe_status_t moe_ffn_forward(const void *x, const void *w_router, const void *w1,
                             const void *w3, const void *w2, int64_t T, int64_t d,
                             int64_t f, int64_t E, int64_t k, void *out, void *stream);

/* The same layer with binary32 storage and arithmetic. */
moe_status_t moe_ffn_forward_f32(const float *x, const float *w_router, const float *w1,
                                 const float *w3, const float *w2, int64_t T, int64_t d,
                                 int64_t f, int64_t E, int64_t k, float *out, void *stream);

/*
 * Options for moe_ffn_forward_ex.  Zero-initialise, then set what is needed;
 * every pointer may be NULL.  All pointers are device pointers.
 *   dtype          MOE_DTYPE_BF16 or MOE_DTYPE_F32 (storage of x, weights, out,
 *                  residual, h_out).
 *   router_bias    [E] fp32 added to the logits before top-k.  The method's
 *                  router is bias-free (section 2.1); this exists so a workload
 *                  can force imbalanced routing.
 *   topk_ids       [T,k] int32 out: selected experts, descending logit.
 *   topk_weights   [T,k] fp32 out: their softmax weights (sum to 1 per token).
 *   expert_counts  [E] int32 out: tokens routed to each expert.
 *   expert_offsets [E+1] int32 out: exclusive prefix sum of expert_counts; the
 *                  rows of expert e are [offsets[e], offsets[e+1]) of the
 *                  grouped (expert-sorted) order, tokens ascending within e.
 *   row_token      [T*k] int32 out: token of each grouped row.
 *   slot_row       [T*k] int32 out: grouped row of token t's j-th pick, at t*k+j.
 *   h_out          [T*k, f] out (dtype): SwiGLU activations of each grouped row.
 *   y_out          [T*k, d] fp32 out: expert output of each grouped row, before
 *                  gating.
 *   residual       [T,d] (dtype): when set, out = residual + layer(x), the sum
 *                  formed in fp32 and rounded once.  residual == out is allowed.
 *   workspace      caller-owned device scratch of workspace_bytes bytes, at
 *                  least moe_ffn_workspace_bytes(...); NULL = library cache.
 *   rmsnorm_input  nonzero: x holds the residual stream h of the stacked
 *                  block h = h + MoE(RMSNorm(h)), and the layer runs on
 *                  RMSNorm(h) with unit gain and eps = rmsnorm_eps (>= 0,
 *                  finite), formed by the router while it reads h, with the
 *                  same bits as moe_rmsnorm.  The pages leave normalisation
 *                  details to the code ("Method", steps for one token, item 5).
 *                  With residual == out == x, one call is one whole block.
 *   rmsnorm_eps    see rmsnorm_input.
 *   x_norm_out     [T,d] out (dtype), used only with rmsnorm_input: receives
 *                  RMSNorm(h).  Must not overlap x, out or residual.  NULL =
 *                  kept in the workspace.
 */
typedef struct moe_ffn_opts {
    int32_t dtype;
    const float *router_bias;
    int32_t *topk_ids;
    float *topk_weights;
    int32_t *expert_counts;
    int32_t *expert_offsets;
    int32_t *row_token;
    int32_t *slot_row;
    void *h_out;
    float *y_out;
    const void *residual;
    void *workspace;
    size_t workspace_bytes;
    int32_t rmsnorm_input;
    float rmsnorm_eps;
    void *x_norm_out;
} moe_ffn_opts_t;

/* The layer with options; opts == NULL behaves as moe_ffn_forward. */
moe_status_t moe_ffn_forward_ex(const void *x, const void *w_router, const void *w1,
                                const void *w3, const void *w2, int64_t T, int64_t d,
                                int64_t f, int64_t E, int64_t k, void *out, void *stream,
                                const moe_ffn_opts_t *opts);

/*
 * For callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * moe_ffn_forward_ex with the workspace taken from a scratch array that the
 * library holds in device memory -- a file-scope array of
 * moe_ffn_noalloc_scratch_bytes() = 64 MiB, one copy on each GPU the library
 * runs on, kept until the process ends.  No call allocates or frees memory:
 * the first call on a device only looks up that device's copy of the array.
 * Same arguments, layouts and results as moe_ffn_forward_ex (opts may be
 * NULL: bf16, no options); opts->workspace must be NULL.  Sizes whose
 * workspace (moe_ffn_workspace_bytes) exceeds 64 MiB return
 * MOE_ERR_UNSUPPORTED before any launch; at d = 4096, f = 14336, E = 8,
 * k = 2 that admits every batch up to T = 207 tokens (the streamed-weight
 * path).  Nothing in the scratch needs to start zeroed.  Every call on one
 * GPU uses that GPU's one array: calls that overlap on a GPU (several host
 * threads, or streams that run concurrently) race and give undefined
 * results; serialise them, or give each its own workspace through
 * moe_ffn_forward_ex.
 */
moe_status_t moe_ffn_forward_noalloc(const void *x, const void *w_router, const void *w1,
                                     const void *w3, const void *w2, int64_t T, int64_t d,
                                     int64_t f, int64_t E, int64_t k, void *out, void *stream,
                                     const moe_ffn_opts_t *opts);

/* Bytes of the scratch array moe_ffn_forward_noalloc works in (64 MiB). */
size_t moe_ffn_noalloc_scratch_bytes(void);

/* Bytes of scratch one forward call needs for these sizes (0 on bad sizes). */
size_t moe_ffn_workspace_bytes(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k,
                               moe_dtype_t dtype);

/*
 * Unit-gain RMSNorm of each row, x[t,i] = h[t,i] / sqrt(mean_i h[t,i]^2 + eps),
 * computed in fp32 and rounded once to dtype.  For the stacked-block form
 * h = h + MoE(RMSNorm(h)); the pages leave normalisation details to the code
 * ("Method": steps for one token, item 5).  h [T,d] in, x [T,d] out; x == h
 * is allowed.  Same validation rules as above (d a multiple of 8 for bf16,
 * of 4 for fp32; eps >= 0).
 */
moe_status_t moe_rmsnorm(const void *h, void *x, int64_t T, int64_t d, float eps,
                         moe_dtype_t dtype, void *stream);

/*
 * Per-stage timing with HIP events, for benchmarks and tools.  Between
 * moe_ffn_profile_begin and moe_ffn_profile_end, the first max_calls forward
 * calls (any entry point, any stream) record an event on their own stream at
 * the start and at the end of each stage whose bit (1 << stage) is set in
 * stage_mask (0 means every stage).  Each recorded event costs a few
 * microseconds of GPU time, so a timing run should ask only for the stages it
 * needs.  moe_ffn_profile_end waits for those events and writes the summed
 * milliseconds of each stage over the recorded calls into
 * stage_ms[MOE_NUM_STAGES] (-1 for stages not in the mask; a stage that a
 * call skips, such as gather_rows on the streamed bf16 path or sum_splits
 * without y_out, adds nothing) and the number of recorded calls into *calls.
 * Stages, in launch order: 0 router_topk, 1 route_scan, 2 gather_rows,
 * 3 gemm1_swiglu, 4 gemm2, 5 sum_splits (runs only when y_out is asked for),
 * 6 combine.  max_calls must be in [1, 1e6];
 * a second begin before end, or an end without begin, is MOE_ERR_INVALID_ARG.
 * Not for concurrent use from several host threads.
 */
#define MOE_NUM_STAGES 7
moe_status_t moe_ffn_profile_begin(int32_t max_calls, uint32_t stage_mask);
moe_status_t moe_ffn_profile_end(float *stage_ms, int32_t *calls);
const char *moe_ffn_stage_name(int32_t stage);

/*
 * Measurement aid, not part of the layer: a streaming read of `bytes` bytes
 * of device memory at buf (16-byte aligned, bytes a multiple of 16) by
 * `blocks` workgroups of 256 threads (1..65536), each reading 16-byte vectors
 * marked nontemporal in a grid-stride loop.  *sink (a device uint32) receives an XOR fold of the
 * data, which only keeps the loads live.  Timing it over a buffer far larger
 * than the 256 MiB MALL gives the read rate a streaming kernel can reach on
 * this GPU, the measured ceiling beside the 8 TB/s datasheet figure.
 * Enqueued on `stream`; bytes == 0 is a no-op.
 */
moe_status_t moe_hbm_read_probe(const void *buf, size_t bytes, int32_t blocks, uint32_t *sink,
                                void *stream);

/*
 * Measurement aid, not part of the layer: bf16 matrix-core work with no
 * memory traffic, the ceiling the MFMA-bound grouped GEMMs are compared with
 * beside the 2.5 PFLOP/s datasheet figure (that figure assumes 2.4 GHz; a
 * dense MFMA stream on random data runs at the clock the part's power limit
 * allows).  `blocks` workgroups (1..65536; one per compute unit measures the
 * whole chip) of 4 wavefronts; each wavefront issues iters (1..2^24) x 128
 * v_mfma_f32_16x16x32_bf16 (16384 flops each) on operand fragments read once
 * from `operands` (device, 16-byte aligned, operand_bytes >= 16 KiB and a
 * multiple of 16; random bf16 data gives realistic power).  *sink (a device
 * uint32) receives an XOR fold of the results, which keeps them live.
 * clocks (device, optional): per workgroup two uint64, the shader-clock
 * cycles and the 100 MHz real-time ticks of its MFMA loop.  Enqueued on
 * `stream`.
 */
moe_status_t moe_mfma_probe(const void *operands, size_t operand_bytes, int32_t iters,
                            int32_t blocks, uint32_t *sink, uint64_t *clocks, void *stream);

/* Text describing the last non-OK status returned on this host thread. */
const char *moe_ffn_last_error(void);

/* Free the cached workspace of every device (waits for the device first). */
void moe_ffn_release_workspace(void);

/* Library version, "major.minor.patch". */
const char *moe_ffn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */

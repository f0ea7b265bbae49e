// api.hip -- the C ABI of libmoe_ffn: argument validation, workspace, and the
// launch sequence of the layer on one stream.
//
// Mixtral of Experts (wikillm.com card, "Method"): router, top-k with a
// softmax over the kept logits, SwiGLU experts, gate-weighted sum (section
// 2.1 displays 1-3), applied to a whole batch grouped by expert.  One call
// enqueues, in stream order:
//   1. router_topk    x, w_router        -> ids [T,k], gates [T,k]
//   2. route_scan     ids                -> counts, offsets, slot_row, row_token
//   3. gather_rows    x, row_token       -> x_perm [T*k, d] (the streamed
//                                            GEMM 1 reads x through row_token
//                                            instead, and this step is skipped)
//   4. gemm1_swiglu   x_perm, w1, w3     -> h [T*k, f]
//   5. gemm2          h, w2              -> y [splits][T*k, d] (fp32)
//   6. combine        y, gates, slot_row -> out [T,d] (+ residual)
// Nothing is read back to the host, so the host never waits for the GPU
// (except when the cached workspace has to grow).
#include <algorithm>
#include <cmath>
#include <mutex>
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include "common.h"
#include "moe_ffn.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

moe_status_t hip_fail(hipError_t e, const char* where) {
    return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

struct Plan {
    int variant = GEMM_LARGE_M;
    int splits = 1;
    int g1_k_waves = 1;  // streamed GEMM 1: waves that split K for one slab (1, 2 or 4)
    size_t ids = 0, gates = 0, counts = 0, offsets = 0, slot_row = 0, row_token = 0, scan = 0;
    size_t x_perm = 0, h = 0, y = 0, partials = 0, total = 0;
};

// Tile variant and K-split of the bf16 GEMMs, and the workspace layout.
// Rows per expert below which GEMM 1's tile kernel marks its weight DMA
// nontemporal: each expert then holds about one row tile, so each weight
// panel is read once (measured at 64 and 100 rows per expert: GEMM 1 3-5%
// faster; at two or more row tiles per expert 6-11% slower).
constexpr int64_t kNtWeightRows = 192;

// Overrides of the streamed path's kernel choices, for tuning runs:
// MOE_FFN_STREAM_SPLITS sets GEMM 2's K slices (1..16, at most f/128) and
// MOE_FFN_STREAM_K_WAVES the waves that split K per slab in GEMM 1 (1, 2 or
// 4; 2 and 4 only where the tiles hold 16 rows, at most 12 rows per
// expert).  Read once per process; unset or 0 keeps the plan's own choice.
static int plan_override(int which) {
    static const int splits = [] {
        const char* v = getenv("MOE_FFN_STREAM_SPLITS");
        return v ? atoi(v) : 0;
    }();
    static const int k_waves = [] {
        const char* v = getenv("MOE_FFN_STREAM_K_WAVES");
        return v ? atoi(v) : 0;
    }();
    return which == 0 ? splits : k_waves;
}

Plan make_plan(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k, int dtype) {
    Plan p;
    const int64_t R = T * k;
    const size_t es = dtype == MOE_DTYPE_BF16 ? 2 : 4;
    if (dtype == MOE_DTYPE_BF16) {
        const int64_t busy_experts = R < E ? R : E;
        const bool tile_ok = R * (d > f ? d : f) * 2 < ((int64_t)1 << 31) &&
                             d * f * 2 < ((int64_t)1 << 31);
        if (R < 52 * E) {
            // Under 52 rows per expert: stream the weights, in row tiles of
            // up to 64 rows (1, 2 or 4 fragments of 16, chosen per tile on the
            // device from the expert's row count).  Measured at Mixtral
            // shapes: 0.485 ms against 0.570 for the 256-row tiles at 48
            // rows per expert, 0.483 against 0.583 at 52; at 56 routing
            // spread puts experts past 64 rows (a second tile re-reads their
            // weights) and the tiles win, 0.584 against 0.619.
            p.variant = GEMM_STREAM;
            // GEMM 1 gives each wave a 128-column slab over all of K.  With
            // one or two tokens that leaves most CUs idle; then 2 or 4 waves
            // split K for each slab (2 or 1 slabs per workgroup, 16-row
            // tiles): the most K-split shape whose workgroups fit in one
            // round of 256 even if every assignment reaches its own expert
            // (a second round of a few dozen workgroups streams alone, at a
            // fraction of the HBM rate).  Measured at Mixtral shapes: T = 1
            // 4 waves (224 workgroups); T = 2 2 waves, GEMM 1 148 -> 116 us
            // against 4 waves; T = 3 1 wave (2 waves: 238 against ~215 us
            // when 6 experts hold rows).
            int64_t mt16 = (R + 15) / 16;
            if (mt16 < busy_experts) mt16 = busy_experts;
            if (R <= 12 * E) {
                for (int kw : {4, 2}) {
                    if (mt16 * ((f + 512 / kw - 1) / (512 / kw)) <= 256) {
                        p.g1_k_waves = kw;
                        break;
                    }
                }
                const int kw_o = plan_override(1);
                if (kw_o == 1 || kw_o == 2 || kw_o == 4) p.g1_k_waves = kw_o;
            }
            // GEMM 2 gives each wave a 128-column slab, the 4 waves of a
            // workgroup 4 adjacent slabs (512 contiguous columns of every w2
            // row, as GEMM 1 reads w1 and w3), and cuts K across workgroups;
            // the combine adds the K-slice partials.  The cut is sized for
            // about 208 streaming workgroups (256 above 12 rows per expert),
            // counting the experts expected to hold rows when R assignments
            // spread evenly over E (the routing itself is not known on the
            // host; workgroups of empty experts exit at once).  Measured at
            // Mixtral shapes: 3 slices at 8 rows per expert (decode), 4 at
            // 16-40 rows per expert streamed fastest.
            const double e_act = std::max(std::min((double)k, (double)E),
                                          E * (1.0 - std::pow(1.0 - 1.0 / E, (double)R)));
            const double rows_per = (double)R / e_act;
            const double mt_act = std::max(1.0, std::ceil(rows_per / 64.0));
            const double tiles2 = (double)((d + 511) / 512) * e_act * mt_act;
            int64_t s = std::lround((rows_per > 12.0 ? 256.0 : 208.0) / tiles2);
            int64_t smax = f / 128;
            if (smax > 16) smax = 16;
            if (smax < 1) smax = 1;
            if (plan_override(0) > 0) s = plan_override(0);
            if (s > smax) s = smax;
            if (s < 1) s = 1;
            p.splits = (int)s;
        } else if (tile_ok) {
            // (the 256-row tile kernels address x_perm, h and each weight
            // matrix with 32-bit buffer offsets: each must stay under 2 GiB)
            // Many rows per expert: 256x256 macro tiles; each XCD's last
            // partial round of tiles may be cut into K pieces, summed by a
            // fixup kernel (y stays one slice).
            p.variant = GEMM_TILE256;
            p.splits = 1;
        } else {
            // Operands past 2 GiB: 128-row tiles with 64-bit addressing.
            p.variant = (R <= 64 * E) ? GEMM_SMALL_M : GEMM_LARGE_M;
            const int64_t bm = gemm_bm(p.variant);
            const int64_t nt2 = (d + gemm2_bn(p.variant) - 1) / gemm2_bn(p.variant);
            int64_t mt = (R + bm - 1) / bm;
            if (mt < busy_experts) mt = busy_experts;
            const int64_t tiles = nt2 * mt;
            // Cut the w2 contraction when GEMM 2 alone would not give every CU
            // a couple of workgroups; keep at least 4 K steps per slice.
            int64_t s = (512 + tiles - 1) / tiles;
            const int64_t kt = f / 64;
            int64_t smax = kt / 4 < 8 ? kt / 4 : 8;
            if (smax < 1) smax = 1;
            if (s > smax) s = smax;
            if (s < 1) s = 1;
            p.splits = (int)s;
        }
    }
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    p.ids = take((size_t)R * 4);
    p.gates = take((size_t)R * 4);
    p.counts = take((size_t)E * 4);
    p.offsets = take((size_t)(E + 1) * 4);
    p.slot_row = take((size_t)R * 4);
    p.row_token = take((size_t)R * 4);
    p.scan = take(route_scan_scratch_bytes((int)R, (int)E));
    p.x_perm = take((size_t)R * d * es);
    p.h = take((size_t)R * f * es);
    p.y = take((size_t)p.splits * R * d * 4);
    p.partials = p.variant == GEMM_TILE256 ? take(tile_partials_bytes((int)R, (int)E, (int)d, (int)f)) : 0;
    p.total = off;
    return p;
}

moe_status_t check_sizes(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k, int dtype) {
    if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_F32)
        return fail(MOE_ERR_INVALID_ARG, "dtype %d is neither MOE_DTYPE_BF16 nor MOE_DTYPE_F32", dtype);
    if (T < 0 || d < 1 || f < 1 || E < 1 || k < 1)
        return fail(MOE_ERR_INVALID_ARG, "sizes must be T >= 0 and d, f, E, k >= 1 (got T=%lld d=%lld f=%lld E=%lld k=%lld)",
                    (long long)T, (long long)d, (long long)f, (long long)E, (long long)k);
    if (k > E) return fail(MOE_ERR_UNSUPPORTED, "k=%lld exceeds E=%lld", (long long)k, (long long)E);
    if (E > 64) return fail(MOE_ERR_UNSUPPORTED, "E=%lld exceeds 64", (long long)E);
    const int64_t mult = dtype == MOE_DTYPE_BF16 ? 64 : 4;
    if (d % mult != 0 || f % mult != 0)
        return fail(MOE_ERR_UNSUPPORTED, "d=%lld and f=%lld must be multiples of %lld", (long long)d,
                    (long long)f, (long long)mult);
    const int64_t lim = (int64_t)1 << 30;
    if (T * k >= lim || d >= lim || f >= lim)
        return fail(MOE_ERR_UNSUPPORTED, "T*k, d and f must each be below 2^30");
    return MOE_OK;
}

struct WorkspaceCache {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mu;
WorkspaceCache g_ws[64];

moe_status_t cached_workspace(size_t need, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d >= 64", dev);
    std::lock_guard<std::mutex> lk(g_ws_mu);
    WorkspaceCache& c = g_ws[dev];
    if (c.bytes < need) {
        if (c.ptr != nullptr) {
            // Work already enqueued may still use the old buffer.
            e = hipDeviceSynchronize();
            if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
            e = hipFree(c.ptr);
            c.ptr = nullptr;
            c.bytes = 0;
            if (e != hipSuccess) return hip_fail(e, "hipFree");
        }
        void* p = nullptr;
        e = hipMalloc(&p, need);
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return fail(MOE_ERR_OUT_OF_MEMORY, "hipMalloc of %zu workspace bytes failed: %s", need,
                        hipGetErrorString(e));
        }
        c.ptr = p;
        c.bytes = need;
    }
    *out = c.ptr;
    return MOE_OK;
}

// The no-allocation entry point's scratch: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (in host code it is only a stand-in): each
// device's address is looked up once with hipGetSymbolAddress, with that
// device current, and kept here.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

moe_status_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d >= 64", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return fail(MOE_ERR_HIP, "hipGetSymbolAddress of the scratch array: %s", hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// Stage-boundary events of profiled calls (moe_ffn_profile_begin/end).
struct Profiler {
    bool active = false;
    int max_calls = 0;
    int calls = 0;
    uint32_t mask = 0;         // stages timed
    hipEvent_t* ev = nullptr;  // [max_calls][MOE_NUM_STAGES + 1]
    uint32_t* skipped = nullptr;  // [max_calls]: stages that launched nothing
};
std::mutex g_prof_mu;
Profiler g_prof;

// Events for the next profiled call (nullptr if none), the stage mask and
// the call's record of skipped stages.
hipEvent_t* profile_slot(uint32_t* mask, uint32_t** skipped) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof.active || g_prof.calls >= g_prof.max_calls) return nullptr;
    *mask = g_prof.mask;
    *skipped = g_prof.skipped + g_prof.calls;
    **skipped = 0;
    return g_prof.ev + (size_t)(g_prof.calls++) * (MOE_NUM_STAGES + 1);
}

// Boundary i (the start of stage i, the end of stage i - 1) is recorded when
// either neighbouring stage is timed.
bool boundary_needed(uint32_t mask, int i) {
    const bool after = i < MOE_NUM_STAGES && ((mask >> i) & 1u);
    const bool before = i > 0 && ((mask >> (i - 1)) & 1u);
    return after || before;
}

#define LAUNCH(call, name)                                   \
    do {                                                     \
        hipError_t e_ = (call);                              \
        if (e_ != hipSuccess) return hip_fail(e_, name);     \
    } while (0)

moe_status_t forward_impl(const void* x, const void* w_router, const void* w1, const void* w3,
                          const void* w2, int64_t T, int64_t d, int64_t f, int64_t E, int64_t k,
                          void* out, void* stream_ptr, const moe_ffn_opts_t* opts, int dtype) {
    moe_status_t st = check_sizes(T, d, f, E, k, dtype);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !w1 || !w3 || !w2 || !out)
        return fail(MOE_ERR_INVALID_ARG, "a tensor pointer is NULL");
    const bool norm_in = opts && opts->rmsnorm_input != 0;
    const void* must_align[] = {x, w_router, w1, w3, w2, out,
                                opts ? opts->residual : nullptr,
                                opts ? opts->h_out : nullptr,
                                opts ? (const void*)opts->y_out : nullptr,
                                opts ? opts->workspace : nullptr,
                                norm_in ? opts->x_norm_out : nullptr};
    for (const void* p : must_align)
        if (p && !aligned16(p)) return fail(MOE_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
    if (norm_in) {
        const float eps = opts->rmsnorm_eps;
        if (!(eps >= 0.0f) || eps > 3.0e38f)
            return fail(MOE_ERR_INVALID_ARG, "rmsnorm_eps must be finite and >= 0");
        const void* xn = opts->x_norm_out;
        if (xn && (xn == x || xn == out || xn == opts->residual))
            return fail(MOE_ERR_INVALID_ARG, "x_norm_out must not overlap x, out or residual");
    }

    const Plan plan = make_plan(T, d, f, E, k, dtype);
    char* ws = nullptr;
    if (opts && opts->workspace) {
        if (opts->workspace_bytes < plan.total)
            return fail(MOE_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu needed",
                        opts->workspace_bytes, plan.total);
        ws = static_cast<char*>(opts->workspace);
    } else {
        void* p = nullptr;
        st = cached_workspace(plan.total, &p);
        if (st != MOE_OK) return st;
        ws = static_cast<char*>(p);
    }

    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    const int Ti = (int)T, di = (int)d, fi = (int)f, Ei = (int)E, ki = (int)k;
    const int R = Ti * ki;
    int32_t* ids = (opts && opts->topk_ids) ? opts->topk_ids : reinterpret_cast<int32_t*>(ws + plan.ids);
    float* gates = (opts && opts->topk_weights) ? opts->topk_weights : reinterpret_cast<float*>(ws + plan.gates);
    int32_t* counts = (opts && opts->expert_counts) ? opts->expert_counts : reinterpret_cast<int32_t*>(ws + plan.counts);
    int32_t* offsets = (opts && opts->expert_offsets) ? opts->expert_offsets : reinterpret_cast<int32_t*>(ws + plan.offsets);
    int32_t* slot_row = (opts && opts->slot_row) ? opts->slot_row : reinterpret_cast<int32_t*>(ws + plan.slot_row);
    int32_t* row_token = (opts && opts->row_token) ? opts->row_token : reinterpret_cast<int32_t*>(ws + plan.row_token);
    void* x_perm = ws + plan.x_perm;
    void* h = (opts && opts->h_out) ? opts->h_out : (void*)(ws + plan.h);
    float* y = reinterpret_cast<float*>(ws + plan.y);
    const float* bias = opts ? opts->router_bias : nullptr;
    const void* residual = opts ? opts->residual : nullptr;

    uint32_t prof_mask = 0;
    uint32_t* prof_skipped = nullptr;
    hipEvent_t* ev = profile_slot(&prof_mask, &prof_skipped);
    auto mark = [&](int i) {
        if (ev && boundary_needed(prof_mask, i)) (void)hipEventRecord(ev[i], stream);
    };
    // a stage that launches nothing reports no time (its two boundary events
    // still bracket an empty interval of event overhead)
    auto skip = [&](int s) {
        if (ev) *prof_skipped |= 1u << s;
    };
    // With rmsnorm_input the router writes x = RMSNorm(h) and the later
    // steps read that.  Without x_norm_out it goes to the y region, which is
    // free until GEMM 2 (by then every reader of x has run) and holds at
    // least T*d fp32 values.
    void* x_norm = nullptr;
    if (norm_in) x_norm = opts->x_norm_out ? opts->x_norm_out : (void*)y;
    mark(0);
    LAUNCH(launch_router_topk(dtype, x, w_router, bias, Ti, di, Ei, ki, ids, gates, x_norm,
                              norm_in ? opts->rmsnorm_eps : 0.0f, stream),
           "router_topk");
    if (norm_in) x = x_norm;
    mark(1);
    LAUNCH(launch_route_scan(ids, Ti, ki, Ei, counts, offsets, slot_row, row_token,
                             reinterpret_cast<int32_t*>(ws + plan.scan), stream),
           "route_scan");
    mark(2);
    // The 256-row tile GEMMs read x_perm and h in a K-blocked layout (see
    // tile_gemm.h); a caller asking for h gets it row-major instead.
    const int kb = (dtype == MOE_DTYPE_BF16 && plan.variant == GEMM_TILE256 && !(opts && opts->h_out)) ? 1 : 0;
    // The streamed GEMM 1 reads x through row_token itself.
    const bool gather = !(dtype == MOE_DTYPE_BF16 && plan.variant == GEMM_STREAM);
    if (gather) LAUNCH(launch_gather_rows(dtype, x, row_token, R, di, kb, x_perm, stream), "gather_rows");
    else skip(2);
    mark(3);
    if (dtype == MOE_DTYPE_BF16 && plan.variant == GEMM_STREAM) {
        LAUNCH(launch_gemm1_swiglu_stream(x, row_token, w1, w3, offsets, R, Ei, di, fi,
                                          plan.g1_k_waves, h, stream),
               "gemm1_swiglu");
        mark(4);
        LAUNCH(launch_gemm2_stream(h, w2, offsets, R, Ei, fi, di, plan.splits, y, stream), "gemm2");
    } else if (dtype == MOE_DTYPE_BF16 && plan.variant == GEMM_TILE256) {
        float* partials = reinterpret_cast<float*>(ws + plan.partials);
        LAUNCH(launch_gemm1_swiglu_tile(x_perm, w1, w3, offsets, R, Ei, di, fi, kb, partials,
                                        R < kNtWeightRows * Ei, h, stream),
               "gemm1_swiglu");
        mark(4);
        LAUNCH(launch_gemm2_tile(h, w2, offsets, R, Ei, fi, di, kb, partials, y, stream), "gemm2");
    } else if (dtype == MOE_DTYPE_BF16) {
        LAUNCH(launch_gemm1_swiglu_bf16(plan.variant, x_perm, w1, w3, offsets, R, Ei, di, fi, h, stream), "gemm1_swiglu");
        mark(4);
        LAUNCH(launch_gemm2_bf16(plan.variant, h, w2, offsets, R, Ei, fi, di, plan.splits, y, stream), "gemm2");
    } else {
        LAUNCH(launch_gemm1_swiglu_f32(x_perm, w1, w3, offsets, R, Ei, di, fi, h, stream), "gemm1_swiglu");
        mark(4);
        LAUNCH(launch_gemm2_f32(h, w2, offsets, R, Ei, fi, di, y, stream), "gemm2");
    }
    mark(5);
    if (opts && opts->y_out)
        LAUNCH(launch_sum_splits(y, plan.splits, R, di, opts->y_out, stream), "sum_splits");
    else
        skip(5);
    mark(6);
    LAUNCH(launch_combine(dtype, y, plan.splits, gates, slot_row, residual, Ti, di, ki, R, out, stream), "combine");
    mark(7);
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_ffn_forward(const void* x, const void* w_router, const void* w1, const void* w3,
                             const void* w2, int64_t T, int64_t d, int64_t f, int64_t E, int64_t k,
                             void* out, void* stream) {
    return forward_impl(x, w_router, w1, w3, w2, T, d, f, E, k, out, stream, nullptr, MOE_DTYPE_BF16);
}

moe_status_t moe_ffn_forward_f32(const float* x, const float* w_router, const float* w1,
                                 const float* w3, const float* w2, int64_t T, int64_t d, int64_t f,
                                 int64_t E, int64_t k, float* out, void* stream) {
    return forward_impl(x, w_router, w1, w3, w2, T, d, f, E, k, out, stream, nullptr, MOE_DTYPE_F32);
}

moe_status_t moe_ffn_forward_ex(const void* x, const void* w_router, const void* w1,
                                const void* w3, const void* w2, int64_t T, int64_t d, int64_t f,
                                int64_t E, int64_t k, void* out, void* stream,
                                const moe_ffn_opts_t* opts) {
    const int dtype = opts ? opts->dtype : MOE_DTYPE_BF16;
    return forward_impl(x, w_router, w1, w3, w2, T, d, f, E, k, out, stream, opts, dtype);
}

moe_status_t moe_ffn_forward_noalloc(const void* x, const void* w_router, const void* w1,
                                     const void* w3, const void* w2, int64_t T, int64_t d,
                                     int64_t f, int64_t E, int64_t k, void* out, void* stream,
                                     const moe_ffn_opts_t* opts) {
    const int dtype = opts ? opts->dtype : MOE_DTYPE_BF16;
    moe_status_t st = check_sizes(T, d, f, E, k, dtype);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (opts && opts->workspace)
        return fail(MOE_ERR_INVALID_ARG,
                    "moe_ffn_forward_noalloc uses the library's static scratch; opts->workspace must be NULL");
    const size_t need = make_plan(T, d, f, E, k, dtype).total;
    if (need > kNoAllocScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED,
                    "these sizes need %zu bytes of scratch, above the %zu bytes the no-allocation entry "
                    "point holds (pass a workspace to moe_ffn_forward_ex instead)",
                    need, kNoAllocScratchBytes);
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != MOE_OK) return st;
    moe_ffn_opts_t o;
    if (opts) o = *opts;
    else memset(&o, 0, sizeof o);
    o.dtype = dtype;
    o.workspace = ws;
    o.workspace_bytes = kNoAllocScratchBytes;
    return forward_impl(x, w_router, w1, w3, w2, T, d, f, E, k, out, stream, &o, dtype);
}

size_t moe_ffn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

size_t moe_ffn_workspace_bytes(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k, moe_dtype_t dtype) {
    char saved[sizeof g_err];
    memcpy(saved, g_err, sizeof g_err);
    const moe_status_t st = check_sizes(T, d, f, E, k, dtype);
    memcpy(g_err, saved, sizeof g_err);
    if (st != MOE_OK) return 0;
    return make_plan(T, d, f, E, k, dtype).total;
}

moe_status_t moe_rmsnorm(const void* h, void* x, int64_t T, int64_t d, float eps, moe_dtype_t dtype,
                         void* stream) {
    if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_F32)
        return fail(MOE_ERR_INVALID_ARG, "dtype %d is neither MOE_DTYPE_BF16 nor MOE_DTYPE_F32", dtype);
    if (T < 0 || d < 1 || !(eps >= 0.0f))
        return fail(MOE_ERR_INVALID_ARG, "need T >= 0, d >= 1, eps >= 0");
    const int64_t mult = dtype == MOE_DTYPE_BF16 ? 8 : 4;
    if (d % mult != 0)
        return fail(MOE_ERR_UNSUPPORTED, "d=%lld must be a multiple of %lld", (long long)d, (long long)mult);
    if (T >= ((int64_t)1 << 30) || d >= ((int64_t)1 << 30))
        return fail(MOE_ERR_UNSUPPORTED, "T and d must be below 2^30");
    if (T == 0) return MOE_OK;
    if (!h || !x) return fail(MOE_ERR_INVALID_ARG, "a tensor pointer is NULL");
    if (!aligned16(h) || !aligned16(x)) return fail(MOE_ERR_UNSUPPORTED, "a tensor pointer is not 16-byte aligned");
    LAUNCH(launch_rmsnorm(dtype, h, x, (int)T, (int)d, eps, reinterpret_cast<hipStream_t>(stream)), "rmsnorm");
    return MOE_OK;
}

moe_status_t moe_ffn_profile_begin(int32_t max_calls, uint32_t stage_mask) {
    if (max_calls < 1 || max_calls > 1000000)
        return fail(MOE_ERR_INVALID_ARG, "max_calls must be in [1, 1e6]");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof.active) return fail(MOE_ERR_INVALID_ARG, "profiling already active");
    const size_t n = (size_t)max_calls * (MOE_NUM_STAGES + 1);
    hipEvent_t* ev = new hipEvent_t[n];
    // Timing-only events: a device-scope release when recorded, so a record
    // between two kernels does not write the L2 back to memory first (the
    // default system-scope release would, adding that time to the stream).
    for (size_t i = 0; i < n; ++i) {
        const hipError_t e = hipEventCreateWithFlags(&ev[i], hipEventReleaseToDevice);
        if (e != hipSuccess) {
            for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
            delete[] ev;
            return hip_fail(e, "hipEventCreateWithFlags");
        }
    }
    g_prof.ev = ev;
    g_prof.skipped = new uint32_t[max_calls]();
    g_prof.max_calls = max_calls;
    g_prof.calls = 0;
    g_prof.mask = stage_mask == 0 ? (1u << MOE_NUM_STAGES) - 1 : stage_mask & ((1u << MOE_NUM_STAGES) - 1);
    g_prof.active = true;
    return MOE_OK;
}

moe_status_t moe_ffn_profile_end(float* stage_ms, int32_t* calls) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof.active) return fail(MOE_ERR_INVALID_ARG, "profiling is not active");
    moe_status_t st = MOE_OK;
    float sums[MOE_NUM_STAGES] = {0};
    for (int c = 0; c < g_prof.calls && st == MOE_OK; ++c) {
        hipEvent_t* e = g_prof.ev + (size_t)c * (MOE_NUM_STAGES + 1);
        for (int s = 0; s < MOE_NUM_STAGES; ++s) {
            if (!((g_prof.mask >> s) & 1u) || ((g_prof.skipped[c] >> s) & 1u)) continue;
            hipError_t r = hipEventSynchronize(e[s + 1]);
            if (r != hipSuccess) { st = hip_fail(r, "hipEventSynchronize"); break; }
            float ms = 0.0f;
            r = hipEventElapsedTime(&ms, e[s], e[s + 1]);
            if (r != hipSuccess) { st = hip_fail(r, "hipEventElapsedTime"); break; }
            sums[s] += ms;
        }
    }
    const size_t n = (size_t)g_prof.max_calls * (MOE_NUM_STAGES + 1);
    for (size_t i = 0; i < n; ++i) (void)hipEventDestroy(g_prof.ev[i]);
    delete[] g_prof.ev;
    delete[] g_prof.skipped;
    const int recorded = g_prof.calls;
    const uint32_t mask = g_prof.mask;
    g_prof = Profiler();
    if (st != MOE_OK) return st;
    if (stage_ms)
        for (int s = 0; s < MOE_NUM_STAGES; ++s) stage_ms[s] = ((mask >> s) & 1u) ? sums[s] : -1.0f;
    if (calls) *calls = recorded;
    return MOE_OK;
}

const char* moe_ffn_stage_name(int32_t stage) {
    static const char* names[MOE_NUM_STAGES] = {"router_topk", "route_scan", "gather_rows",
                                                "gemm1_swiglu", "gemm2", "sum_splits", "combine"};
    return (stage >= 0 && stage < MOE_NUM_STAGES) ? names[stage] : "";
}

const char* moe_ffn_last_error(void) { return g_err; }

void moe_ffn_release_workspace(void) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (int dev = 0; dev < 64; ++dev) {
        WorkspaceCache& c = g_ws[dev];
        if (c.ptr == nullptr) continue;
        if (hipSetDevice(dev) == hipSuccess) {
            (void)hipDeviceSynchronize();
            (void)hipFree(c.ptr);
        }
        c.ptr = nullptr;
        c.bytes = 0;
    }
    if (have_cur) (void)hipSetDevice(cur);
}

moe_status_t moe_hbm_read_probe(const void* buf, size_t bytes, int32_t blocks, uint32_t* sink,
                                void* stream) {
    if (bytes == 0) return MOE_OK;
    if (!buf || !sink) return fail(MOE_ERR_INVALID_ARG, "a pointer is NULL");
    if (!aligned16(buf) || bytes % 16 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "buf must be 16-byte aligned and bytes a multiple of 16");
    if (blocks < 1 || blocks > 65536) return fail(MOE_ERR_INVALID_ARG, "blocks must be in [1, 65536]");
    LAUNCH(launch_read_probe(buf, bytes, blocks, sink, reinterpret_cast<hipStream_t>(stream)),
           "read_probe");
    return MOE_OK;
}

moe_status_t moe_mfma_probe(const void* operands, size_t operand_bytes, int32_t iters,
                            int32_t blocks, uint32_t* sink, uint64_t* clocks, void* stream) {
    if (!operands || !sink) return fail(MOE_ERR_INVALID_ARG, "a pointer is NULL");
    if (!aligned16(operands) || operand_bytes % 16 != 0 || operand_bytes < 16 * 1024)
        return fail(MOE_ERR_UNSUPPORTED,
                    "operands must be 16-byte aligned, at least 16 KiB and a multiple of 16 bytes");
    if (iters < 1 || iters > (1 << 24)) return fail(MOE_ERR_INVALID_ARG, "iters must be in [1, 2^24]");
    if (blocks < 1 || blocks > 65536) return fail(MOE_ERR_INVALID_ARG, "blocks must be in [1, 65536]");
    LAUNCH(launch_mfma_probe(operands, operand_bytes, iters, blocks, sink,
                             reinterpret_cast<unsigned long long*>(clocks),
                             reinterpret_cast<hipStream_t>(stream)),
           "mfma_probe");
    return MOE_OK;
}

const char* moe_ffn_version(void) { return "0.2.0"; }

}  // extern "C"

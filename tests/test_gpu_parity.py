"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases compare every output element; the full-size workloads check
routing on every token and outputs (plus the SwiGLU activations h and the
expert outputs y) on sampled tokens, in the same launch configuration the
benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import parity as PT
from sparse_mixture_experts_select_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def case(T, d, f, E, dtype, seed, x_dist="rms", bias=None, label="case"):
    inp = inputs.make_weights(d, f, E, dtype, DEV, seed, label)
    inp["x"] = inputs.make_x(T, d, dtype, DEV, x_dist, seed, label)
    inp["bias"] = None if bias is None else torch.tensor(bias, dtype=torch.float32, device=DEV)
    return inp


def banner(msg):
    print("\n[case] " + msg, flush=True)


def test_tiny_fp32_workload():
    banner("tiny fp32 T=64 d=128 f=256 E=8 k=2")
    inp = inputs.workload_inputs("tiny", DEV)
    r = PT.full_check(inp, 2, label="tiny")
    print(r["label"], "near ties", r["near_ties"], "err", r["err_out"], r["err_h"], r["err_y"])


SMALL = [
    # T, d, f, E, k, dtype
    (300, 192, 320, 8, 2, torch.bfloat16),    # 256-row tiles: tail tiles only (~75 rows per expert), ragged
    (40, 256, 384, 8, 2, torch.bfloat16),     # streamed, one-fragment tiles
    (1, 128, 128, 8, 2, torch.bfloat16),      # one token
    (257, 512, 640, 6, 3, torch.bfloat16),
    (100, 128, 192, 4, 1, torch.bfloat16),    # k = 1
    (64, 128, 128, 4, 4, torch.bfloat16),     # k = E: dense softmax mixture
    (33, 64, 128, 1, 1, torch.bfloat16),      # E = 1: plain SwiGLU
    (100, 128, 128, 64, 8, torch.bfloat16),   # widest routing
    (700, 256, 256, 8, 2, torch.bfloat16),    # 256-row tiles: one partial row tile per expert (~175 rows)
    # 256x256 macro tiles (at least 128 rows per expert on average)
    (1100, 256, 384, 8, 2, torch.bfloat16),   # partial last row tiles, K split 2 in GEMM 2
    (600, 192, 320, 4, 2, torch.bfloat16),    # ragged columns in both GEMMs
    (2000, 128, 256, 8, 1, torch.bfloat16),   # k = 1, 250 rows per expert
    (2101, 128, 256, 8, 2, torch.bfloat16),   # router with 8 tokens per workgroup, ragged last group
    # streamed-weight path (about a dozen rows or fewer per expert)
    (48, 192, 320, 8, 2, torch.bfloat16),     # ragged slabs, experts above 16 rows, K split 2
    (20, 256, 1024, 8, 2, torch.bfloat16),    # K split 8, one step per wave
    (5, 128, 128, 64, 8, torch.bfloat16),     # E = 64, most experts empty
    (2, 256, 1024, 8, 2, torch.bfloat16),     # GEMM 1 with K split over the waves
    (2, 256, 4032, 64, 8, torch.bfloat16),    # GEMM 1 with K split over 2 waves per slab, partial last slab
    (110, 192, 320, 8, 2, torch.bfloat16),    # streamed, 2 row fragments per tile, ragged slabs
    (150, 256, 512, 8, 2, torch.bfloat16),    # streamed, 4 row fragments per tile
    (240, 256, 512, 8, 2, torch.bfloat16),    # 256-row tiles: tail tiles only (~60 rows per expert)
    (600, 512, 1024, 8, 2, torch.bfloat16),   # GEMM 2's last round cut into 4 K pieces (fixup sums them)
    (1500, 1024, 2048, 8, 2, torch.bfloat16), # GEMM 2 tiles cut into 3 K pieces, several per XCD
    (2600, 768, 704, 2, 2, torch.bfloat16),   # 10 row tiles + a tail per expert: a partial block of
                                              # row tiles, partial column-tile groups in both GEMMs
    (1100, 320, 384, 8, 2, torch.bfloat16),   # GEMM 2: a whole column tile + one of 64 columns
    (2000, 704, 256, 8, 2, torch.bfloat16),   # GEMM 2: two whole column tiles + one of 192 columns
    (1300, 1152, 512, 4, 2, torch.bfloat16),  # partial last row tiles of ~138 rows (6 fragments per wave row)
    (50, 100, 60, 5, 2, torch.float32),
    (200, 64, 96, 16, 4, torch.float32),
    # multi-workgroup route scan (over 4096 assignments) with wide routing
    (700, 128, 128, 64, 8, torch.bfloat16),
    (1100, 64, 96, 8, 4, torch.float32),      # and fp32 router with 4 tokens per workgroup
    # k above 8, up to k = E = 64 (the dense softmax-gated mixture)
    (90, 128, 128, 16, 16, torch.bfloat16),   # k = E = 16
    (70, 128, 128, 64, 64, torch.bfloat16),   # k = E = 64: every token reaches every expert
    (130, 128, 192, 32, 17, torch.bfloat16),  # k = 17 of 32 (picks in three batches of 8)
    (40, 64, 96, 24, 12, torch.float32),      # fp32, k = 12 of 24
    (3, 256, 512, 64, 40, torch.bfloat16),    # streamed path, k = 40 of 64
    # streamed GEMM 2 with the most K slices the plans use, summed by the combine
    (1, 4096, 2048, 8, 2, torch.bfloat16),    # 13 slices
    (1, 512, 2048, 8, 2, torch.bfloat16),     # 16 slices
]


@pytest.mark.parametrize("T,d,f,E,k,dtype", SMALL)
def test_small_shapes(T, d, f, E, k, dtype):
    from sparse_mixture_experts_select_amd import binding
    banner("small T=%d d=%d f=%d E=%d k=%d %s" % (T, d, f, E, k, dtype))
    inp = case(T, d, f, E, dtype, seed=T + d + f + E + k, label="small")
    r = PT.full_check(inp, k)
    print("near ties", r["near_ties"], "err", r["err_out"], r["err_h"], r["err_y"])
    # Without the debug outputs the 256-row tile path keeps x_perm and h in
    # its K-blocked layout; the arithmetic is the same, so out must match the
    # checked run bit for bit.
    fwd = binding.moe_ffn_forward if dtype == torch.bfloat16 else binding.moe_ffn_forward_f32
    plain = fwd(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], k)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       r["gpu"]["out"].view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


CUT_CASES = [
    # T, d, f, E, k, piece counts GEMM 2's schedule cuts tiles into (E = 1 or
    # k = E: every expert's row count is known, so the tile plan is)
    (256, 256, 512, 1, 1, {2}),
    (256, 2048, 2048, 1, 1, {8}),
    (256, 2048, 1536, 1, 1, {6}),
    (256, 2048, 1280, 1, 1, {5}),
    (512, 1024, 2048, 2, 2, {5}),       # two cut tiles on every XCD
    (768, 1536, 2048, 2, 2, {8, 4}),    # one cut tile on some XCDs, five on others
]


@pytest.mark.parametrize("T,d,f,E,k,pieces", CUT_CASES)
def test_gemm2_tiles_cut_into_k_pieces(T, d, f, E, k, pieces):
    """GEMM 2's last round cut into 2, 4, 5, 6 or 8 K pieces (5, 6 and 8 are
    the counts the full-size workloads use), the fixup summing them: every
    row of out, h and y against the oracle."""
    import tile_plan
    cpx = torch.cuda.get_device_properties(0).multi_processor_count // 8
    assert tile_plan.gemm2_pieces([T * k // E] * E, d, f, cpx) == pieces
    banner("GEMM 2 cut into %s K pieces: T=%d d=%d f=%d E=%d k=%d" % (sorted(pieces), T, d, f, E, k))
    inp = case(T, d, f, E, torch.bfloat16, seed=T + d + f, label="cut")
    r = PT.full_check(inp, k)
    np.testing.assert_array_equal(PT.to_np(r["gpu"]["counts"]), [T * k // E] * E)
    print("near ties", r["near_ties"], "err", r["err_out"], r["err_h"], r["err_y"])



FRAGMENT_CASES = [
    # T, d, f, E, k, GEMM 2's piece counts (E = 1 or k = E: every expert
    # holds T*k/E rows, so which K loop each tile runs is known)
    (276, 2048, 2048, 1, 1, {5}),   # a full tile + 20-row tails (2 fragments), all cut
    (300, 1024, 2048, 2, 2, {5}),   # full tiles + 44-row tails (4 fragments)
    (60, 2048, 2048, 1, 1, {8}),    # tail tiles only, 60 rows (4 fragments), cut into 8
    (80, 2048, 2048, 1, 1, {8}),    # tail tiles only, 80 rows (6 fragments)
    (90, 1024, 2048, 2, 2, {8}),    # tail tiles only, 90 rows (6 fragments)
    (150, 2048, 2048, 1, 1, {8}),   # one full tile of 150 rows (6 fragments per wave row)
    (230, 1024, 2048, 2, 2, {8}),   # one full tile of 230 rows (all 8, alternate fragments part empty)
    (420, 2048, 2048, 1, 1, {5}),   # a whole tile + a full tile of 164 rows (6 per wave row)
]


@pytest.mark.parametrize("T,d,f,E,k,pieces", FRAGMENT_CASES)
def test_tiles_by_row_fragments(T, d, f, E, k, pieces):
    """The 256-row tile kernels multiply only the 16-row fragments that hold
    some of a tile's rows: a tail tile (an expert's last 1..128 rows over two
    column tiles, the same rows in every wave) 2, 4, 6 or 8 of them, a full
    tile with at most 192 rows 6 per wave row (the wave rows take alternate
    fragments).  Each class in both GEMMs and in GEMM 2 tiles cut into K
    pieces: every row of out, h and y against the oracle."""
    import tile_plan
    rows = T * k // E
    cpx = torch.cuda.get_device_properties(0).multi_processor_count // 8
    assert tile_plan.gemm2_pieces([rows] * E, d, f, cpx) == pieces
    banner("tiles of %d rows per expert: T=%d d=%d f=%d E=%d k=%d" % (rows, T, d, f, E, k))
    inp = case(T, d, f, E, torch.bfloat16, seed=T + d + f + 1, label="frag")
    r = PT.full_check(inp, k)
    np.testing.assert_array_equal(PT.to_np(r["gpu"]["counts"]), [rows] * E)
    print("near ties", r["near_ties"], "err", r["err_out"], r["err_h"], r["err_y"])


MODEL_SHAPES = [
    # label, T, d, f, E, k, tokens checked: all, or those reaching every
    # 128-row block of every expert's rows
    ("d6144 f16384 E8 k2 streamed", 16, 6144, 16384, 8, 2, "all"),     # router with d > 4096
    ("d6144 f16384 E8 k2 tiles", 1024, 6144, 16384, 8, 2, "blocks"),
    ("d2048 f1408 E64 k6 streamed", 256, 2048, 1408, 64, 6, "all"),    # fine-grained experts
    ("d2048 f1408 E64 k6 tiles", 2048, 2048, 1408, 64, 6, "blocks"),
    ("d3584 f2560 E64 k8 streamed", 128, 3584, 2560, 64, 8, "all"),    # d, f not powers of 2
    ("d3584 f2560 E64 k8 tiles", 1024, 3584, 2560, 64, 8, "blocks"),
]


@pytest.mark.parametrize("label,T,d,f,E,k,which", MODEL_SHAPES, ids=[m[0] for m in MODEL_SHAPES])
def test_other_model_shapes(label, T, d, f, E, k, which):
    """Published MoE configurations other than the Mixtral 8x7B one: a
    larger hidden size (the router's general kernel, d > 4096), 64
    fine-grained experts with k = 6 and 8, and hidden / expert sizes that
    are not powers of two, each on the few-rows-per-expert path and on the
    256-row tile path (by T)."""
    banner("%s: T=%d d=%d f=%d E=%d k=%d" % (label, T, d, f, E, k))
    inp = case(T, d, f, E, torch.bfloat16, seed=d + f + E + k, label="model")
    tokens = None if which == "all" else (lambda g: PT.segment_sample_tokens(g, 5))
    r = PT.full_check(inp, k, tokens=tokens, label=label)
    R = T * k
    streamed = R < 52 * E
    assert streamed == ("streamed" in label)
    print("near ties", r["near_ties"], "tokens checked", len(r["tokens"]), "err", r["err_out"],
          r["err_h"], r["err_y"])
    del inp, r
    torch.cuda.empty_cache()

def test_batch_with_h_past_2gib():
    """h = 65600 x 16384 bf16 is past 2 GiB: the GEMMs fall back from the
    256-row tile kernels (32-bit buffer offsets) to the 128-row grouped ones."""
    banner("T=32800 d=128 f=16384 E=8 k=2 (h > 2 GiB)")
    inp = case(32800, 128, 16384, 8, torch.bfloat16, seed=12, label="huge")
    r = PT.full_check(inp, 2, tokens=np.arange(0, 32800, 2050), want_h=False, want_y=False,
                      label="huge")
    print("near ties", r["near_ties"], "err", r["err_out"])


def test_all_logits_tied():
    banner("w_router = 0")
    inp = case(70, 128, 128, 8, torch.bfloat16, seed=5, label="ties")
    inp["w_router"].zero_()
    g = PT.run_gpu(inp, 2)
    ids = PT.to_np(g["ids"])
    assert np.all(ids[:, 0] == 0) and np.all(ids[:, 1] == 1)
    assert np.all(PT.to_np(g["gates"]) == 0.5)
    np.testing.assert_array_equal(PT.to_np(g["counts"]), [70, 70, 0, 0, 0, 0, 0, 0])
    host = PT.host_inputs(inp)
    logits, _, _ = oracle.route(host["x"], host["w_router"], 2)
    assert np.all(logits == 0.0)
    # every pair of experts is a correct top-2 here (28 of them)
    assert len(PT.valid_topk_sets(logits[0], 2)) == 28
    PT.check_outputs(g, host, np.arange(70), logits, 2, torch.bfloat16)


def test_imbalanced_and_empty_experts():
    banner("bias: expert 3 takes every token, experts 5-7 get none")
    bias = [0.0, 0.0, 0.0, 40.0, 0.0, -40.0, -40.0, -40.0]
    inp = case(300, 256, 256, 8, torch.bfloat16, seed=6, bias=bias, label="skew")
    r = PT.full_check(inp, 2)
    counts = PT.to_np(r["gpu"]["counts"])
    assert counts[3] == 300 and counts[5:].sum() == 0


@pytest.mark.parametrize("T", [40, 70, 100, 150])
def test_streamed_path_with_one_heavy_expert(T):
    # expert 2 takes every token (one of each token's two picks), so its
    # row tiles are: T = 40: one tile of 40 rows (4 fragments, the last
    # partial); 70: 64 + 6 rows (4 fragments, then 1); 100: 64 + 36 (4 and a
    # partial 4); 150: 64 + 64 + 22 (4, 4, then 2).  The other experts share
    # the second picks: one-fragment tiles, and two-fragment ones at T = 150.
    banner("streamed path, expert 2 takes all %d tokens" % T)
    bias = [0.0, 0.0, 40.0, 0.0, 0.0, 0.0, 0.0, 0.0]
    inp = case(T, 128, 256, 8, torch.bfloat16, seed=11 + T, bias=bias, label="heavy")
    r = PT.full_check(inp, 2)
    assert PT.to_np(r["gpu"]["counts"])[2] == T


@pytest.mark.parametrize("T,d,f,E,k,dtype", [
    (40, 256, 384, 8, 2, torch.bfloat16),    # streamed GEMMs
    (600, 192, 320, 8, 2, torch.bfloat16),   # 256-row tiles
    (50, 128, 96, 8, 2, torch.float32),      # fp32 GEMMs
])
def test_saturated_silu(T, d, f, E, k, dtype):
    """w1 scaled by 200, so its pre-activations reach the hundreds while the
    router's logits keep their scale: SiLU's exp(-z) overflows fp32 for z
    below about -88 (its sigmoid factor then has to come out as 0, h as -0)
    and underflows for large z (factor 1, h = z * b).  Every element of out,
    h and y against the oracle."""
    banner("saturated SiLU T=%d d=%d f=%d E=%d k=%d %s" % (T, d, f, E, k, dtype))
    inp = case(T, d, f, E, dtype, seed=T + d + f + 7, label="saturated")
    inp["w1"] = (inp["w1"].float() * 200.0).to(dtype)
    r = PT.full_check(inp, k)
    h = PT.out_f64(r["gpu"]["h"])
    assert np.all(np.isfinite(h)) and np.abs(h).max() > 100
    print("near ties", r["near_ties"], "err", r["err_out"], r["err_h"], r["err_y"])


def test_zero_tokens_leaves_out_untouched():
    from sparse_mixture_experts_select_amd import binding
    inp = case(0, 128, 128, 8, torch.bfloat16, seed=1, label="empty")
    # T = 0 with out (and the residual) pointing at a sentinel-filled
    # buffer, through the C ABI: a call that wrote anything there would
    # change the buffer
    import ctypes
    buf = torch.full((4, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    w = [p(inp[n]) for n in ("w_router", "w1", "w3", "w2")]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = binding.lib.moe_ffn_forward(p(buf), *w, 0, 128, 128, 8, 2, p(buf), stream)
    assert st == binding.MOE_OK
    opts = binding.MoeFfnOpts()
    opts.residual = p(buf)
    opts.rmsnorm_input = 1
    opts.rmsnorm_eps = 1e-5
    st = binding.lib.moe_ffn_forward_ex(p(buf), *w, 0, 128, 128, 8, 2, p(buf), stream,
                                        ctypes.byref(opts))
    assert st == binding.MOE_OK
    torch.cuda.synchronize()
    assert torch.all(buf == 3.0)


def test_forward_entry_points_agree_and_are_deterministic():
    from sparse_mixture_experts_select_amd import binding
    banner("determinism T=1000 d=256 f=512")
    inp = case(1000, 256, 512, 8, torch.bfloat16, seed=7, label="det")
    a = binding.moe_ffn_forward(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2)
    b = binding.moe_ffn_forward(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2)
    c = binding.moe_ffn_forward_ex(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2)
    nbytes = binding.moe_ffn_workspace_bytes(1000, 256, 512, 8, 2)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    dws = binding.moe_ffn_forward_ex(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2,
                                     workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(a.view(torch.int16), dws.view(torch.int16))


def test_residual_and_in_place():
    from sparse_mixture_experts_select_amd import binding
    banner("residual")
    inp = case(150, 128, 256, 8, torch.bfloat16, seed=8, label="res")
    resid = inputs.make_x(150, 128, torch.bfloat16, DEV, "normal", 9, "resid")
    plain = binding.moe_ffn_forward(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2)
    out = resid.clone()
    binding.moe_ffn_forward_ex(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2,
                               out=out, residual=out)
    torch.cuda.synchronize()
    want = (resid.float() + plain.float())
    # residual + layer is rounded once; layer alone is rounded once too, so the
    # two paths differ by at most one bf16 rounding of the layer output.
    err = (out.float() - want).abs().max().item()
    assert err <= 2 ** -7 * want.abs().max().item()
    g = PT.run_gpu(inp, 2, residual=resid)
    host = PT.host_inputs(inp)
    logits, o_ids, _ = oracle.route(host["x"], host["w_router"], 2)
    PT.check_routing(g, logits, o_ids, 2)
    PT.check_outputs(g, host, np.arange(150), logits, 2, torch.bfloat16,
                     residual=PT.out_f64(resid))
    # out == x is allowed
    x2 = inp["x"].clone()
    binding.moe_ffn_forward(x2, inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2, out=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2.view(torch.int16), plain.view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rmsnorm(dtype):
    from sparse_mixture_experts_select_amd import binding
    h = inputs.make_x(333, 4096 if dtype == torch.bfloat16 else 200, dtype, DEV, "normal", 3, "rms") * 3
    x = binding.moe_rmsnorm(h, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(inputs.host_array(h), 1e-5)
    got = PT.out_f64(x)
    tol = 2 ** -8 if dtype == torch.bfloat16 else 1e-6
    assert np.abs(got - ref).max() <= tol * np.abs(ref).max()


FUSED_NORM = [
    # T, d, f, E, k, dtype: router tokens per workgroup 1, 2, 4, 8 (ragged last
    # group), streamed and 256-row tile GEMM paths, general E, fp32
    (20, 256, 512, 8, 2, torch.bfloat16),
    (401, 256, 256, 8, 2, torch.bfloat16),
    (1000, 256, 384, 8, 2, torch.bfloat16),
    (2101, 128, 256, 8, 2, torch.bfloat16),
    (300, 192, 320, 16, 4, torch.bfloat16),
    (90, 200, 96, 8, 2, torch.float32),
]


@pytest.mark.parametrize("T,d,f,E,k,dtype", FUSED_NORM)
def test_rmsnorm_fused_into_router(T, d, f, E, k, dtype):
    """The block h + MoE(RMSNorm(h)) as one call (the router forms RMSNorm(h))
    gives the same bits as moe_rmsnorm followed by the layer, also in place."""
    from sparse_mixture_experts_select_amd import binding
    banner("fused rmsnorm T=%d d=%d f=%d E=%d k=%d %s" % (T, d, f, E, k, dtype))
    inp = case(T, d, f, E, dtype, seed=31, label="fnorm")
    h = inputs.make_x(T, d, dtype, DEV, "normal", 32, "fnorm_h") * 3
    eps = 1e-5
    x_ref = binding.moe_rmsnorm(h, eps=eps)
    w = (inp["w_router"], inp["w1"], inp["w3"], inp["w2"])
    ids_a = torch.empty((T, k), dtype=torch.int32, device=DEV)
    ids_b = torch.empty_like(ids_a)
    want = binding.moe_ffn_forward_ex(x_ref, *w, k, residual=h, topk_ids=ids_a)
    xn = torch.full_like(h, float("nan"))
    got = binding.moe_ffn_forward_ex(h, *w, k, residual=h, topk_ids=ids_b, rmsnorm_eps=eps,
                                     x_norm_out=xn)
    h2 = h.clone()
    binding.moe_ffn_forward_ex(h2, *w, k, out=h2, residual=h2, rmsnorm_eps=eps)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(xn.view(bits), x_ref.view(bits))
    assert torch.equal(ids_b, ids_a)
    assert torch.equal(got.view(bits), want.view(bits))
    assert torch.equal(h2.view(bits), want.view(bits))
    # and RMSNorm itself against the oracle
    ref = oracle.rmsnorm(inputs.host_array(h), eps)
    tol = 2 ** -8 if dtype == torch.bfloat16 else 1e-6
    assert np.abs(PT.out_f64(xn) - ref).max() <= tol * np.abs(ref).max()


# ---------------------------------------------------------------- workloads


def sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=min(n, T), replace=False))


def test_decode_workload():
    banner("decode bf16 T=32 d=4096 f=14336 E=8 k=2 (all tokens)")
    inp = inputs.workload_inputs("decode", DEV)
    r = PT.full_check(inp, 2, label="decode")
    print("near ties", r["near_ties"], "err", r["err_out"], r["err_h"], r["err_y"])


def test_prefill_workload():
    banner("prefill bf16 T=4096 (routing, outputs, h and y on all tokens)")
    inp = inputs.workload_inputs("prefill", DEV)
    r = PT.full_check(inp, 2, label="prefill")
    print("near ties", r["near_ties"], "err", r["err_out"], r["err_h"], r["err_y"])
    # the benchmark's call (no debug outputs: K-blocked x_perm and h)
    from sparse_mixture_experts_select_amd import binding
    plain = binding.moe_ffn_forward(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), r["gpu"]["out"].view(torch.int16))


def test_skewed_workload():
    banner("skewed bf16 T=16384 (routing on all tokens; outputs, h and y on tokens reaching "
           "every 128-row block of every expert)")
    inp = inputs.workload_inputs("skewed", DEV)
    r = PT.full_check(inp, 2, tokens=lambda g: PT.segment_sample_tokens(g, 2), label="skewed")
    counts = PT.to_np(r["gpu"]["counts"])
    share = counts / counts.sum()
    print("near ties", r["near_ties"], "tokens checked", len(r["tokens"]), "err", r["err_out"],
          r["err_h"], r["err_y"], "shares", np.round(share, 3))
    # the workload's definition: the heaviest expert takes roughly 40%
    assert 0.35 < share[0] < 0.45
    from sparse_mixture_experts_select_amd import binding
    plain = binding.moe_ffn_forward_ex(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2,
                                       router_bias=inp["bias"])
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), r["gpu"]["out"].view(torch.int16))


@pytest.fixture(scope="module")
def mixtral_weights():
    wl = inputs.WORKLOADS["prefill"]
    w = inputs.make_weights(wl.d, wl.f, wl.E, torch.bfloat16, DEV, 0, "small-batch")
    host = {kk: inputs.host_array(v) for kk, v in w.items() if kk in ("w_router", "w1", "w3", "w2")}
    yield w, host
    del w, host
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 2, 3, 4, 8, 16, 64, 128, 207])
def test_mixtral_shape_small_batches(T, mixtral_weights):
    """The batch sizes at the HBM-bound end of the batch sweep, at d=4096,
    f=14336, E=8, k=2, every token: the streamed kernels with GEMM 1's K
    split over the waves (T <= 2), GEMM 2 cut into up to 13 K slices (T = 1),
    and row tiles of 1, 2 and 4 fragments over the full K loops (about 16,
    32 and 52 rows per expert at T = 64, 128 and 207, the largest batch on
    the streamed path, where experts past 64 rows take a second tile)."""
    w, host_w = mixtral_weights
    banner("Mixtral shape T=%d (all tokens)" % T)
    inp = dict(w)
    inp["x"] = inputs.make_x(T, 4096, torch.bfloat16, DEV, "rms", T, "small-batch")
    inp["bias"] = None
    g = PT.run_gpu(inp, 2, want_h=True, want_y=True)
    host = dict(host_w)
    host["x"] = inputs.host_array(inp["x"])
    logits, o_ids, _ = oracle.route(host["x"], host["w_router"], 2)
    exempt = PT.check_routing(g, logits, o_ids, 2)
    errs = PT.check_outputs(g, host, np.arange(T), logits, 2, torch.bfloat16)
    print("near ties", int(exempt.sum()), "err", errs)


def test_stack_workload_teacher_forced():
    """32 blocks h <- h + MoE(RMSNorm(h)), T=2048, each with its own weights.
    Every layer is checked on the GPU's own bf16 input of that layer: RMSNorm
    and the output on sampled tokens, routing on every token.  Beside that,
    8 tokens are carried through the blocks by the oracle alone (its own h
    from h0, no GPU value as input), and the GPU's h after every block is
    compared with that chain on the tokens whose routing has not differed."""
    from sparse_mixture_experts_select_amd import binding
    wl = inputs.WORKLOADS["stack"]
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.k
    banner("stack bf16 T=%d, %d layers (teacher-forced per layer)" % (T, wl.layers))
    h = inputs.make_x(T, d, torch.bfloat16, DEV, wl.x_dist, 0, "stack")
    x = torch.empty_like(h)
    rng = np.random.default_rng(3)
    total_ties = 0
    # Free-running tokens: the oracle carries them through all the layers on
    # its own, with the same bf16 storage of x and h as the GPU, and their
    # final h is compared with the GPU's where their routing never differed.
    free_tok = np.sort(rng.choice(T, size=8, replace=False))
    free_idx = torch.as_tensor(free_tok, device=DEV)
    h_free = inputs.host_array(h[free_idx])  # bf16 bits
    diverged = np.zeros(len(free_tok), bool)

    def bf16_bits(a):
        return inputs.host_array(torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16))

    for layer in range(wl.layers):
        inp = inputs.make_weights(d, f, E, torch.bfloat16, DEV, 0, "stack", layer)
        # the benchmark's block: one call, RMSNorm formed by the router
        inp["x"] = h
        g = PT.run_gpu(inp, k, residual=h, rmsnorm_eps=wl.rms_eps, x_norm_out=x)
        assert torch.equal(x.view(torch.int16), binding.moe_rmsnorm(h, eps=wl.rms_eps).view(torch.int16))
        inp["x"] = x
        host = PT.host_inputs(inp)
        # free-running tokens: oracle layer on the oracle's own h
        x_free = bf16_bits(oracle.rmsnorm(h_free, wl.rms_eps))
        fr = oracle.moe_tokens(x_free, host["w_router"], host["w1"], host["w3"], host["w2"], k)
        gpu_ids = PT.to_np(g["ids"])[free_tok]
        diverged |= np.any(np.sort(fr["ids"], axis=1) != np.sort(gpu_ids, axis=1), axis=1)
        h_free = bf16_bits(inputs.bf16_bits_to_f64(h_free) + fr["out"])
        keep = ~diverged
        if keep.any():
            # the oracle-only chain against the GPU after this block: both
            # sides round h to bf16 after every block from slightly different
            # sums, so they may drift apart by up to one bf16 unit (2^-8 of
            # |h|) per block
            got_f = PT.out_f64(g["out"][free_idx])[keep]
            want_f = inputs.bf16_bits_to_f64(h_free)[keep]
            rel_f = np.abs(got_f - want_f).max() / np.abs(want_f).max()
            assert rel_f <= (layer + 1) * 2.0 ** -8, "layer %d free-running drift %g" % (layer, rel_f)
        # tokens reaching every 128-row block of every expert's rows
        tok = PT.segment_sample_tokens(g, layer)
        # RMSNorm of this layer's input, against the oracle
        h_tok = inputs.host_array(h[torch.as_tensor(tok, device=DEV)])
        x_ref = oracle.rmsnorm(h_tok, wl.rms_eps)
        x_err = np.abs(PT.out_f64(x[torch.as_tensor(tok, device=DEV)]) - x_ref).max()
        assert x_err <= 2 ** -8 * np.abs(x_ref).max(), "layer %d rmsnorm error %g" % (layer, x_err)
        # routing on every token
        logits, o_ids, _ = oracle.route(host["x"], host["w_router"], k)
        exempt = PT.check_routing(g, logits, o_ids, k)
        total_ties += int(exempt.sum())
        # h + MoE(x) on the sampled tokens: the MoE part to the bf16 bar, plus
        # one bf16 rounding of the residual sum
        ref_ids, ref_gates = PT.reference_selection(logits, PT.to_np(g["ids"]), tok, k)
        ref = oracle.moe_tokens(host["x"], None, host["w1"], host["w3"], host["w2"], k, tokens=tok,
                                forced_ids=ref_ids, forced_gates=ref_gates)
        moe_ref = ref["out"]
        want = PT.out_f64(h[torch.as_tensor(tok, device=DEV)]) + moe_ref
        got = PT.out_f64(g["out"][torch.as_tensor(tok, device=DEV)])
        bound = PT.TOL[torch.bfloat16] * np.abs(moe_ref).max() + 2.0 ** -8 * np.abs(want)
        worst = (np.abs(got - want) - bound).max()
        assert worst <= 0, "layer %d output outside the bar by %g" % (layer, worst)
        rel = np.abs(got - want).max() / np.abs(moe_ref).max()
        print("layer %2d: near ties %d, rmsnorm err %.2e, out err %.2e of max|moe|, max|h| %.2f"
              % (layer, int(exempt.sum()), x_err, rel, np.abs(want).max()), flush=True)
        h = g["out"]
        del inp, host, g
    print("stack: %d near-tie tokens over %d layers" % (total_ties, wl.layers))
    got = PT.out_f64(h[free_idx])
    want = inputs.bf16_bits_to_f64(h_free)
    keep = ~diverged
    print("free-running: %d of %d tokens kept their routing through %d layers"
          % (int(keep.sum()), len(free_tok), wl.layers))
    if keep.any():
        # Both sides round h to bf16 after every layer from slightly different
        # sums, so the two h may drift apart by up to one bf16 unit (2^-8 of
        # |h|) per layer; this reports the drift and bounds it linearly.
        rel = np.abs(got[keep] - want[keep]).max() / np.abs(want[keep]).max()
        print("free-running h_%d error on those tokens: %.2e of max|h|" % (wl.layers, rel))
        assert rel <= wl.layers * 2.0 ** -8, rel

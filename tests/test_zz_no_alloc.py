"""moe_ffn_forward_noalloc, called through the C ABI: the same results as
moe_ffn_forward_ex with the library's own workspace, bit for bit, on calls
in a row whose inputs shrink (the scratch array keeps the previous call's
contents), and refusal of sizes beyond its scratch."""
import ctypes

import pytest
import torch

from sparse_mixture_experts_select_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(T, d, f, E, dtype, seed):
    inp = inputs.make_weights(d, f, E, dtype, DEV, seed, "noalloc")
    inp["x"] = inputs.make_x(T, d, dtype, DEV, "rms", seed, "noalloc")
    return inp


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(inp, k, out, opts=None):
    x = inp["x"]
    T, d = x.shape
    E, _, f = inp["w1"].shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = binding.lib.moe_ffn_forward_noalloc(
        _p(x), _p(inp["w_router"]), _p(inp["w1"]), _p(inp["w3"]), _p(inp["w2"]), T, d, f, E, k,
        _p(out), stream, ctypes.byref(opts) if opts is not None else None)
    return st


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def test_noalloc_matches_forward_ex_on_shrinking_calls():
    # (T, d, f, E, k, dtype): 256-row tiles with GEMM 2's last round cut into
    # K pieces, then a smaller streamed-weight batch, then fp32 with a
    # residual added and RMSNorm formed in the router
    cases = [(600, 512, 1024, 8, 2, torch.bfloat16), (40, 256, 384, 8, 2, torch.bfloat16),
             (64, 128, 256, 8, 2, torch.float32)]
    for i, (T, d, f, E, k, dtype) in enumerate(cases):
        print("\n[case] no-alloc call %d: T=%d d=%d f=%d E=%d k=%d %s" % (i, T, d, f, E, k, dtype),
              flush=True)
        inp = _case(T, d, f, E, dtype, seed=i + 1)
        assert binding.moe_ffn_workspace_bytes(
            T, d, f, E, k, binding.MOE_DTYPE_BF16 if dtype == torch.bfloat16 else binding.MOE_DTYPE_F32
        ) <= binding.moe_ffn_noalloc_scratch_bytes()
        out = torch.full_like(inp["x"], float("nan"))
        if i < 2:
            ref = binding.moe_ffn_forward_ex(inp["x"], inp["w_router"], inp["w1"], inp["w3"],
                                             inp["w2"], k)
            st = _noalloc(inp, k, out)
        else:
            resid = inputs.make_x(T, d, dtype, DEV, "normal", 77, "noalloc-resid")
            ref = binding.moe_ffn_forward_ex(inp["x"], inp["w_router"], inp["w1"], inp["w3"],
                                             inp["w2"], k, residual=resid, rmsnorm_eps=1e-5)
            opts = binding.MoeFfnOpts()
            opts.dtype = binding.MOE_DTYPE_F32
            opts.residual = resid.data_ptr()
            opts.rmsnorm_input = 1
            opts.rmsnorm_eps = 1e-5
            st = _noalloc(inp, k, out, opts)
        torch.cuda.synchronize()
        assert st == binding.MOE_OK, binding.moe_ffn_last_error()
        assert torch.equal(_bits(out), _bits(ref))


def test_noalloc_mixtral_decode_batch():
    """The serving case it is for: a decode batch at Mixtral shapes (T = 32,
    d = 4096, f = 14336, E = 8, k = 2), then one token."""
    wl = inputs.WORKLOADS["decode"]
    w = inputs.make_weights(wl.d, wl.f, wl.E, torch.bfloat16, DEV, 0, "noalloc-decode")
    for T in (32, 1):
        print("\n[case] no-alloc Mixtral shape T=%d" % T, flush=True)
        inp = dict(w)
        inp["x"] = inputs.make_x(T, wl.d, torch.bfloat16, DEV, "rms", T, "noalloc-decode")
        ref = binding.moe_ffn_forward(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"], 2)
        out = torch.empty_like(inp["x"])
        assert _noalloc(inp, 2, out) == binding.MOE_OK, binding.moe_ffn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref))


def test_noalloc_refuses_sizes_beyond_its_scratch():
    inp = _case(16, 128, 128, 8, torch.bfloat16, seed=9)
    out = torch.full_like(inp["x"], 3.0)
    # a workspace given in opts is refused: the scratch is the library's
    opts = binding.MoeFfnOpts()
    opts.workspace = out.data_ptr()
    opts.workspace_bytes = out.numel() * 2
    assert _noalloc(inp, 2, out, opts) == binding.MOE_ERR_INVALID_ARG
    # T = 4096 at d = 4096, f = 14336 needs about 544 MiB of workspace: refused
    # before any launch (the sizes alone decide; the pointers are never read)
    assert binding.moe_ffn_workspace_bytes(4096, 4096, 14336, 8, 2) > binding.moe_ffn_noalloc_scratch_bytes()
    p = _p(out)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = binding.lib.moe_ffn_forward_noalloc(p, p, p, p, p, 4096, 4096, 14336, 8, 2, p, stream, None)
    assert st == binding.MOE_ERR_UNSUPPORTED
    assert "scratch" in binding.moe_ffn_last_error()
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)

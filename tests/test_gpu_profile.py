"""Measurement aids: per-stage timing through moe_ffn_profile_begin/end (call
count, stage mask, stages a call skips reporting no time) and the streaming
read probe."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_select_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("T,f,skipped", [(24, 1024, {"gather_rows", "sum_splits"}),  # streamed weights
                                         (300, 512, {"sum_splits"})])               # 256-row tiles
def test_profile_stages(T, f, skipped):
    print("\n[case] profile T=%d f=%d" % (T, f), flush=True)
    d, E, k = 256, 8, 2
    w = inputs.make_weights(d, f, E, torch.bfloat16, DEV, 0, "profile", 0)
    x = inputs.make_x(T, d, torch.bfloat16, DEV, "normal", 0, "profile")
    out = torch.empty_like(x)
    args = (x, w["w_router"], w["w1"], w["w3"], w["w2"], k)

    binding.moe_ffn_profile_begin(3)
    for _ in range(5):  # only the first 3 are recorded
        binding.moe_ffn_forward(*args, out=out)
    torch.cuda.synchronize()
    ms, calls = binding.moe_ffn_profile_end()
    assert calls == 3
    assert set(ms) == {binding.moe_ffn_stage_name(i) for i in range(binding.MOE_NUM_STAGES)}
    for name, v in ms.items():
        if name in skipped:
            assert v == 0.0, name
        else:
            assert v > 0.0, name

    # with y_out, sum_splits runs
    y_out = torch.empty(T * k, d, dtype=torch.float32, device=DEV)
    binding.moe_ffn_profile_begin(1, ["sum_splits", "gemm2"])
    binding.moe_ffn_forward_ex(*args, out=out, y_out=y_out)
    torch.cuda.synchronize()
    ms, calls = binding.moe_ffn_profile_end()
    assert calls == 1 and set(ms) == {"sum_splits", "gemm2"}
    assert ms["sum_splits"] > 0.0 and ms["gemm2"] > 0.0

    # nested begin is refused and leaves the first session intact
    binding.moe_ffn_profile_begin(1)
    with pytest.raises(binding.MoeError):
        binding.moe_ffn_profile_begin(1)
    binding.moe_ffn_forward(*args, out=out)
    torch.cuda.synchronize()
    _, calls = binding.moe_ffn_profile_end()
    assert calls == 1


@pytest.mark.parametrize("n_words,blocks", [(4, 1), (1 << 18, 64), ((1 << 20) + 12, 1000)])
def test_read_probe_reads_every_word(n_words, blocks):
    """The streaming-read probe folds every 32-bit word of the buffer exactly
    once (XOR of all words), for grids smaller and larger than the data."""
    from sparse_mixture_experts_select_amd import binding
    print("\n[case] read probe %d words, %d workgroups" % (n_words, blocks), flush=True)
    g = torch.Generator().manual_seed(n_words)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_words,), dtype=torch.int64, generator=g)
    host = host.to(torch.int32)
    buf = host.cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.moe_hbm_read_probe(buf, blocks, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert sink.cpu().numpy().view(np.uint32)[0] == want

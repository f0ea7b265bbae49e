"""Per-stage timing through moe_ffn_profile_begin/end: call count, stage mask,
and stages a call skips reporting no time."""
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

"""A stack of RMSNorm + MoE blocks captured in one HIP graph (through
torch.cuda.CUDAGraph) replays to the same bits as the eager calls, with
RMSNorm as its own call or formed by the router inside the layer call."""
import pytest
import torch

from sparse_mixture_experts_select_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def make_stack(layers, T, d, f, E, k):
    ws_bytes = binding.moe_ffn_workspace_bytes(T, d, f, E, k)
    return {
        "w": [inputs.make_weights(d, f, E, torch.bfloat16, DEV, 0, "graph", i) for i in range(layers)],
        "h0": inputs.make_x(T, d, torch.bfloat16, DEV, "normal", 0, "graph"),
        # graph users pass their own workspace: the library's cached one may
        # be reallocated by a later call with a larger shape
        "ws": torch.empty(ws_bytes, dtype=torch.uint8, device=DEV),
    }


def run_stack(st, h, x, k, fused=False):
    h.copy_(st["h0"])
    for w in st["w"]:
        if fused:
            binding.moe_ffn_forward_ex(h, w["w_router"], w["w1"], w["w3"], w["w2"], k, out=h,
                                       residual=h, rmsnorm_eps=1e-5, workspace=st["ws"])
        else:
            binding.moe_rmsnorm(h, x, eps=1e-5)
            binding.moe_ffn_forward_ex(x, w["w_router"], w["w1"], w["w3"], w["w2"], k, out=h,
                                       residual=h, workspace=st["ws"])


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("T,d,f", [(300, 256, 512),    # 256-row tile path
                                   (768, 1024, 2048),  # tiles, GEMM 2's last round cut into K pieces
                                   (24, 256, 1024),    # streamed-weight path
                                   (2, 256, 8448)])    # streamed, GEMM 1 with 2 waves per slab
def test_graph_replay_matches_eager(T, d, f, fused):
    print("\n[case] graph of 4 blocks T=%d d=%d f=%d fused=%s" % (T, d, f, fused), flush=True)
    E, k = 8, 2
    st = make_stack(4, T, d, f, E, k)
    h = torch.empty_like(st["h0"])
    x = torch.empty_like(st["h0"])
    run_stack(st, h, x, k)
    torch.cuda.synchronize()
    ref = h.clone()
    if fused:
        # the fused block gives the same bits as RMSNorm then the layer
        run_stack(st, h, x, k, fused=True)
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), ref.view(torch.int16))

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_stack(st, h, x, k, fused)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_stack(st, h, x, k, fused)
    torch.cuda.synchronize()

    for rep in range(4):
        h.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), ref.view(torch.int16)), "replay %d differs" % rep
        # eager work between replays, on the same buffers
        run_stack(st, h, x, k, fused)
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), ref.view(torch.int16))

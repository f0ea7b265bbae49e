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


def _probe_fold_reference(ops16, blocks, iters):
    """What the MFMA probe's sink must hold, computed on the CPU from the
    16x16x32 bf16 MFMA's operand and result layout: lane (c, g) = (lane % 16,
    lane // 16) supplies row c (A) or column c (B) at k = 8g .. 8g + 7, and
    receives rows 4g .. 4g + 3 of column c of the product.  The operands are
    small integers, so every sum is exact in fp32 and the order of the
    hardware's additions cannot matter."""
    n16 = ops16.size // 8
    vec = ops16.reshape(n16, 8).astype(np.float64)
    fold = np.uint32(0)
    for blk in range(blocks):
        for w in range(4):
            lanes = np.arange(64)
            base = ((blk * 256 + w * 64 + lanes) * 16)
            a = np.stack([vec[(base + i) % n16] for i in range(8)])      # [8 frag][64 lane][8]
            b = np.stack([vec[(base + 8 + i) % n16] for i in range(8)])
            # A_i[r][k] = a[i][r + 16 (k // 8)][k % 8]; B_j[k][c] = b[j][c + 16 (k // 8)][k % 8]
            A = np.zeros((8, 16, 32))
            B = np.zeros((8, 32, 16))
            for kg in range(4):
                A[:, :, 8 * kg:8 * kg + 8] = a[:, 16 * kg:16 * kg + 16, :]
                B[:, 8 * kg:8 * kg + 8, :] = b[:, 16 * kg:16 * kg + 16, :].transpose(0, 2, 1)
            f = np.zeros(64, np.uint32)
            for m in range(8):
                for n in range(8):
                    C = sum(A[(m + h) & 7] @ B[(n + 3 * h) & 7] for h in range(2)) * iters
                    # lane (c, g): C[4g][c] + C[4g+1][c] + C[4g+2][c] + C[4g+3][c]
                    s = C.reshape(4, 4, 16).sum(axis=1)  # [g][c]
                    vals = np.array([s[l // 16][l % 16] for l in range(64)], np.float32)
                    f ^= vals.view(np.uint32)
            fold ^= np.bitwise_xor.reduce(f)
    return fold


@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 5)])
def test_mfma_probe_products_are_exact(blocks, iters):
    """The MFMA probe computes what the matrix-core layout says: with
    small-integer bf16 operands (exact sums), its XOR fold equals the CPU's,
    and its clock record is positive."""
    from sparse_mixture_experts_select_amd import binding
    print("\n[case] mfma probe %d workgroups x %d iterations" % (blocks, iters), flush=True)
    g = torch.Generator().manual_seed(blocks * 100 + iters)
    ops = torch.randint(-2, 3, (8192,), generator=g).to(torch.bfloat16)   # 16 KiB
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    binding.moe_mfma_probe(ops.cuda(), iters, blocks, sink, clocks)
    torch.cuda.synchronize()
    want = _probe_fold_reference(ops.float().numpy(), blocks, iters)
    assert sink.cpu().numpy().view(np.uint32)[0] == want
    ck = clocks.cpu().numpy().reshape(blocks, 2)
    assert np.all(ck > 0)

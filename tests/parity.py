"""GPU-vs-oracle comparison helpers for the parity tests.

Acceptance rule (per layer):
  - expert ids and per-expert counts bit-exact, except for tokens whose
    oracle k-th / (k+1)-th logit gap is at most 1e-3 ("near ties"); for
    those the GPU's pick must still be a valid top-k within that gap;
  - the grouping (offsets, row_token, slot_row) bit-exact against the stable
    expert-major order of the GPU's own ids;
  - gates within 1e-6 of the fp64 softmax over the chosen logits;
  - outputs within max|err| <= tol * max|ref| with tol = 1e-4 (fp32) or
    2e-2 (bf16 storage, fp32 accumulation), against the oracle run with a
    selection the oracle itself names: its own top-k off near ties; at a near
    tie, whichever of the top-k sets it enumerates as correct within the gap
    the GPU took (the GPU's choice only picks among the oracle's answers).
"""
from __future__ import annotations

import itertools

import numpy as np
import scipy.special
import torch

import oracle
from sparse_mixture_experts_select_amd import binding, inputs

GAP = 1e-3
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def run_gpu(inp, k, want_h=False, want_y=False, residual=None, **extra):
    """One forward through moe_ffn_forward_ex with every debug output (extra:
    further options of the binding, passed through)."""
    x, wr, w1, w3, w2 = inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"]
    T, d = x.shape
    E, _, f = w1.shape
    R = T * k
    dev = x.device
    i32 = dict(dtype=torch.int32, device=dev)
    res = {
        "ids": torch.full((T, k), -7, **i32),
        "gates": torch.full((T, k), -7.0, dtype=torch.float32, device=dev),
        "counts": torch.full((E,), -7, **i32),
        "offsets": torch.full((E + 1,), -7, **i32),
        "row_token": torch.full((R,), -7, **i32),
        "slot_row": torch.full((R,), -7, **i32),
    }
    h = torch.full((R, f), float("nan"), dtype=x.dtype, device=dev) if want_h else None
    y = torch.full((R, d), float("nan"), dtype=torch.float32, device=dev) if want_y else None
    out = binding.moe_ffn_forward_ex(
        x, wr, w1, w3, w2, k, router_bias=inp.get("bias"), topk_ids=res["ids"],
        topk_weights=res["gates"], expert_counts=res["counts"], expert_offsets=res["offsets"],
        row_token=res["row_token"], slot_row=res["slot_row"], h_out=h, y_out=y, residual=residual,
        **extra)
    torch.cuda.synchronize()
    res["out"] = out
    res["h"] = h
    res["y"] = y
    return res


def to_np(t):
    return t.detach().cpu().numpy()


def out_f64(t):
    """GPU output tensor -> float64 numpy (exact widening)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_routing(g, logits, o_ids, k):
    """Routing checks; returns the near-tie mask [T]."""
    ids = to_np(g["ids"])
    gates = to_np(g["gates"]).astype(np.float64)
    counts = to_np(g["counts"])
    offsets = to_np(g["offsets"])
    row_token = to_np(g["row_token"])
    slot_row = to_np(g["slot_row"])
    T, E = logits.shape
    R = T * k
    srt = -np.sort(-logits, axis=1)
    if k < E:
        exempt = (srt[:, k - 1] - srt[:, k]) <= GAP
    else:
        exempt = np.zeros(T, bool)
    assert ids.min() >= 0 and ids.max() < E, "ids out of range"
    for t in range(T):
        assert len(set(ids[t].tolist())) == k, "repeated expert for token %d" % t
    keep = ~exempt
    np.testing.assert_array_equal(np.sort(ids[keep], 1), np.sort(o_ids[keep], 1),
                                  err_msg="expert sets differ off near ties")
    clear = keep.copy()
    for j in range(k - 1):
        clear &= (srt[:, j] - srt[:, j + 1]) > GAP
    np.testing.assert_array_equal(ids[clear], o_ids[clear], err_msg="pick order differs")
    for t in np.nonzero(exempt)[0]:
        chosen = logits[t, ids[t]]
        others = np.delete(logits[t], ids[t])
        assert chosen.min() >= others.max() - GAP, "invalid pick at near tie, token %d" % t
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    mixed = np.where(exempt[:, None], ids, o_ids)
    np.testing.assert_array_equal(counts, np.bincount(mixed.ravel(), minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    order = np.argsort(ids.ravel(), kind="stable")
    np.testing.assert_array_equal(row_token, order // k)
    exp_slot = np.empty(R, np.int64)
    exp_slot[order] = np.arange(R)
    np.testing.assert_array_equal(slot_row, exp_slot)
    ref_ids, ref_gates = reference_selection(logits, ids, np.arange(T), k)
    # the oracle's gate for the expert in each of the GPU's slots
    ref_g = np.array([[ref_gates[t, list(ref_ids[t]).index(e)] for e in ids[t]] for t in range(T)],
                     np.float64).reshape(T, k)
    gerr = np.abs(gates - ref_g).max() if T else 0.0
    assert gerr <= 1e-6, "gate error %g" % gerr
    assert np.all(gates[:, :-1] >= gates[:, 1:] - 1e-7)
    return exempt


def valid_topk_sets(row, k):
    """Every k-subset of experts that is a correct top-k of one token's
    logits within GAP: its smallest logit is at least the largest logit left
    out minus GAP.  Each set is a tuple in descending-logit order (ties by
    index).  Off near ties this is the one true top-k set.  Every member of
    such a set has a logit of at least the k-th largest minus GAP, so only
    those experts are enumerated."""
    E = row.shape[0]
    key = lambda e: (-row[e], e)
    if k >= E:
        return [tuple(sorted(range(E), key=key))]
    kth = np.sort(row)[::-1][k - 1]
    pool = [e for e in range(E) if row[e] >= kth - GAP]
    sets = []
    for s in itertools.combinations(pool, k):
        rest = np.delete(row, list(s))
        if row[list(s)].min() >= rest.max() - GAP:
            sets.append(tuple(sorted(s, key=key)))
    return sets


def reference_selection(logits, gpu_ids, tokens, k):
    """The selection each sampled token's output is checked against: among
    the oracle's correct top-k sets (valid_topk_sets of the oracle's logits),
    the one the GPU took; it is the oracle's own top-k off near ties.  Fails
    if the GPU's set is not one of them.  Returns (ids [n,k] in
    descending-logit order, gates [n,k]: fp64 softmax over those logits)."""
    n = len(tokens)
    ids = np.empty((n, k), np.int32)
    for i, t in enumerate(tokens):
        mine = tuple(sorted(int(e) for e in gpu_ids[t]))
        match = [s for s in valid_topk_sets(logits[t], k) if tuple(sorted(s)) == mine]
        assert match, "token %d: GPU experts %s are not a correct top-%d" % (t, mine, k)
        ids[i] = match[0]
    gates = scipy.special.softmax(logits[np.asarray(tokens)[:, None], ids], axis=1)
    return ids, gates


def check_outputs(g, host, tokens, logits, k, dtype, check_h=True, check_y=True,
                  residual=None):
    """Sampled tokens' outputs (and their h / y rows) against the oracle run
    with reference_selection's ids and gates.  ``logits`` are the oracle's
    [T,E] (bias included).  Returns (rel_err_out, rel_err_h, rel_err_y)."""
    tol = TOL[dtype]
    gpu_ids = to_np(g["ids"])
    tok = np.asarray(tokens, np.int64)
    ref_ids, ref_gates = reference_selection(logits, gpu_ids, tok, k)
    ref = oracle.moe_tokens(host["x"], None, host["w1"], host["w3"], host["w2"], k, tokens=tok,
                            forced_ids=ref_ids, forced_gates=ref_gates,
                            want_y=check_y and g["y"] is not None, want_h=check_h and g["h"] is not None)
    got = out_f64(g["out"][torch.as_tensor(tok, device=g["out"].device)])
    want = ref["out"]
    if residual is not None:
        want = want + residual[tok]
    scale = np.abs(want).max()
    err_out = np.abs(got - want).max() / scale
    assert err_out <= tol, "output error %g > %g" % (err_out, tol)
    slot = to_np(g["slot_row"]).reshape(-1, k)
    rows = torch.as_tensor(slot[tok].ravel(), device=g["out"].device, dtype=torch.long)
    # the GPU's j-th row of a token belongs to its j-th expert: line each up
    # with the oracle's row for the same expert
    perm = np.array([[list(ref_ids[i]).index(e) for e in gpu_ids[t]] for i, t in enumerate(tok)],
                    np.int64).reshape(len(tok), k)
    pick = (np.arange(len(tok))[:, None], perm)
    err_h = err_y = None
    if "h" in ref:
        gh = out_f64(g["h"][rows]).reshape(len(tok), k, -1)
        rh = ref["h"][pick]
        err_h = np.abs(gh - rh).max() / np.abs(rh).max()
        assert err_h <= tol, "h error %g" % err_h
    if "y" in ref:
        gy = out_f64(g["y"][rows]).reshape(len(tok), k, -1)
        ry = ref["y"][pick]
        err_y = np.abs(gy - ry).max() / np.abs(ry).max()
        assert err_y <= tol, "y error %g" % err_y
    return err_out, err_h, err_y


def host_inputs(inp):
    return {kk: inputs.host_array(v) for kk, v in inp.items()
            if kk in ("x", "w_router", "w1", "w3", "w2")}


def segment_sample_tokens(g, seed, step=128):
    """Tokens whose grouped rows reach every row block of every expert
    segment: each expert's rows [offsets[e], offsets[e+1]) are cut into
    blocks of ``step`` rows from the segment's start, and each block gives
    its first row, its last row and one random row.  With step dividing the
    GEMM tiles' row heights, every row tile of every expert (full, partial,
    tail) holds checked rows, and a checked row is compared over all its
    columns, so every tile the GEMMs run -- whole, cut into K pieces or a
    tail -- is covered.  Picked from the GPU's own offsets and row_token."""
    offsets = to_np(g["offsets"])
    row_token = to_np(g["row_token"])
    rng = np.random.default_rng(seed)
    rows = []
    for e in range(len(offsets) - 1):
        o0, o1 = int(offsets[e]), int(offsets[e + 1])
        for b in range(o0, o1, step):
            hi = min(b + step, o1)
            rows += [b, hi - 1, int(rng.integers(b, hi))]
    if not rows:
        return np.zeros(0, np.int64)
    return np.unique(row_token[np.asarray(rows, np.int64)]).astype(np.int64)


def full_check(inp, k, tokens=None, want_h=True, want_y=True, label=""):
    """Run the GPU layer and check routing on every token and outputs on
    ``tokens`` (all tokens when None; a callable is given the GPU results
    and returns the tokens).  Returns a summary dict."""
    x = inp["x"]
    g = run_gpu(inp, k, want_h=want_h, want_y=want_y)
    host = host_inputs(inp)
    bias = None if inp.get("bias") is None else to_np(inp["bias"])
    logits, o_ids, _ = oracle.route(host["x"], host["w_router"], k, bias=bias)
    exempt = check_routing(g, logits, o_ids, k)
    T = x.shape[0]
    if tokens is None:
        tok = np.arange(T)
    elif callable(tokens):
        tok = np.asarray(tokens(g))
    else:
        tok = np.asarray(tokens)
    errs = check_outputs(g, host, tok, logits, k, x.dtype)
    return {"label": label, "near_ties": int(exempt.sum()), "err_out": errs[0],
            "err_h": errs[1], "err_y": errs[2], "gpu": g, "tokens": tok}

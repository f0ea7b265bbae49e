"""The parity tests' acceptance rules on the CPU: the enumeration of correct
top-k sets at near ties, and the selection the GPU's outputs are checked
against, both checked by brute force over every k-subset."""
import itertools

import numpy as np
import pytest

import parity as PT


def brute_sets(row, k):
    E = len(row)
    out = set()
    for s in itertools.combinations(range(E), k):
        rest = [row[e] for e in range(E) if e not in s]
        if not rest or min(row[e] for e in s) >= max(rest) - PT.GAP:
            out.add(frozenset(s))
    return out


@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (8, 4), (16, 4), (4, 4), (6, 5)])
def test_valid_sets_equal_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for trial in range(300):
        row = rng.normal(size=E)
        # plant ties and near ties at and around the k-th place
        if trial % 3:
            order = np.argsort(-row)
            a, b = order[k - 1], order[min(k, E - 1)]
            row[b] = row[a] - rng.choice([0.0, 0.5e-3, 1e-3, 2e-3])
        if trial % 7 == 0:
            row[:] = np.round(row, 0)
        got = PT.valid_topk_sets(row, k)
        assert {frozenset(s) for s in got} == brute_sets(row, k)
        assert len(got) == len(set(got))
        for s in got:
            assert list(s) == sorted(s, key=lambda e: (-row[e], e))


def test_clear_gap_gives_the_one_top_k():
    row = np.array([0.1, 2.0, -1.0, 1.5, 0.3, 0.2, -0.5, 0.0])
    assert PT.valid_topk_sets(row, 2) == [(1, 3)]
    assert len(PT.valid_topk_sets(np.zeros(8), 2)) == 28


def test_reference_selection_picks_among_the_oracles_sets():
    logits = np.array([[0.0, 1.0, 1.0005, -2.0],     # clear set, near tie in its order
                       [3.0, 1.0, 1.0, 0.0],         # tie for the 2nd place
                       [0.0, 0.0, 0.0, 0.0]])
    gpu = np.array([[1, 2], [0, 2], [3, 1]])
    ids, gates = PT.reference_selection(logits, gpu, np.arange(3), 2)
    assert ids.tolist() == [[2, 1], [0, 2], [1, 3]]
    assert np.allclose(gates.sum(1), 1.0)
    assert np.allclose(gates[1], np.exp([3.0, 1.0]) / np.exp([3.0, 1.0]).sum())
    with pytest.raises(AssertionError, match="not a correct top-2"):
        PT.reference_selection(logits, np.array([[0, 1], [0, 1], [0, 1]]), np.arange(1), 2)

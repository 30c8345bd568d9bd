"""Pins of the oracle's best-first draft-tree construction (CPU only).

Closed forms and brute force, independent of the heap the oracle uses:
- equal candidates at every depth give breadth-first order with children in
  candidate order (ties go to the earlier push);
- one dominant candidate gives a chain first;
- on a tiny implicit tree, the popped set is exactly the T best paths by
  score, in descending order (brute-force enumeration of every path);
- structural invariants: a parent precedes its child, scores never increase
  in pop order, and each score is its parent's plus one log-probability.
"""
import itertools

import numpy as np
import pytest

import oracle


def logsoftmax(z):
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=-1, keepdims=True)
    return (z - m - np.log(np.exp(z - m).sum(axis=-1, keepdims=True))).astype(np.float32)


@pytest.mark.parametrize("K,T", [(3, 12), (8, 100), (2, 30)])
def test_equal_candidates_give_breadth_first_order(K, T):
    lp = np.full((2, 16, K), np.float32(np.log(np.float32(1.0 / K))), dtype=np.float32)
    parent, choice, _ = oracle.build_tree(lp, T)
    for b in range(2):
        for i in range(T):
            assert parent[b, i] == (-1 if i < K else (i - K) // K)
            assert choice[b, i] == i % K


def test_dominant_candidate_gives_a_chain():
    K, Dmax = 8, 16
    z = np.full((1, Dmax, K), -30.0)
    z[:, :, 5] = 0.0
    lp = logsoftmax(z)
    parent, choice, _ = oracle.build_tree(lp, Dmax)
    assert parent[0].tolist() == [-1] + list(range(Dmax - 1))
    assert choice[0].tolist() == [5] * Dmax


def enumerate_paths(lp, Dmax, K):
    """Every node of the implicit tree as (score, path), score summed in fp32
    in depth order."""
    out = []
    for d in range(1, Dmax + 1):
        for path in itertools.product(range(K), repeat=d):
            s = np.float32(0.0)
            for depth, k in enumerate(path):
                s = np.float32(s + lp[depth, k]) if depth else lp[0, k]
            out.append((float(s), path))
    return out


@pytest.mark.parametrize("seed", range(4))
def test_top_t_by_brute_force(seed):
    K, Dmax = 3, 4
    rng = np.random.default_rng(seed)
    lp = logsoftmax(rng.normal(0, 2, size=(1, Dmax, K)))
    allp = enumerate_paths(lp[0], Dmax, K)
    scores = sorted(s for s, _ in allp)
    assert len(set(scores)) == len(scores)      # no exact ties in this data
    for T in (1, 5, 17, 60, 120):
        parent, choice, score = oracle.build_tree(lp, T)
        best = sorted(allp, key=lambda x: -x[0])[:T]
        # rebuild each node's path from parent / choice
        paths = []
        for i in range(T):
            p = parent[0, i]
            paths.append((paths[p] if p >= 0 else ()) + (int(choice[0, i]),))
        assert paths == [path for _, path in best]
        assert np.array_equal(score[0], np.array([s for s, _ in best], dtype=np.float32))


def test_structure_invariants():
    rng = np.random.default_rng(5)
    K, Dmax, T = 8, 16, 256
    lp = logsoftmax(rng.normal(0, 2, size=(3, Dmax, K)))
    parent, choice, score = oracle.build_tree(lp, T)
    for b in range(3):
        depth = np.zeros(T, dtype=np.int64)
        for i in range(T):
            p = parent[b, i]
            assert -1 <= p < i
            depth[i] = 1 if p < 0 else depth[p] + 1
            assert depth[i] <= Dmax
            base = np.float32(0.0) if p < 0 else score[b, p]
            expect = lp[b, 0, choice[b, i]] if p < 0 else np.float32(base + lp[b, depth[i] - 1, choice[b, i]])
            assert score[b, i] == expect
            if i:
                assert score[b, i] <= score[b, i - 1]


def test_rejects_a_budget_larger_than_the_tree():
    lp = np.zeros((1, 2, 2), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.build_tree(lp, 7)        # the implicit tree has 2 + 4 = 6 nodes
    oracle.build_tree(lp, 6)

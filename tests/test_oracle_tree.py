"""Pins of the oracle's best-first draft-tree construction (CPU only).

Closed forms and brute force, independent of the heap the oracle uses:
- equal candidates at every depth give breadth-first order with children in
  candidate order (ties go to the earlier push);
- one dominant candidate gives a chain first;
- on a tiny implicit tree, the popped set is exactly the T best paths by
  score, in descending order (brute-force enumeration of every path);
- structural invariants: a parent precedes its child, scores never increase
  in pop order, and each score is its parent's plus one log-probability;
- NaN log-probabilities (which the pages' ranking of real scores leaves
  open) mean "no candidate": brute force over the paths whose fp32 score is
  not NaN gives the popped set, and nodes beyond the finite candidates are
  written as missing (parent -1, choice -1, NaN score).
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


def paths_of(parent, choice, n):
    paths = []
    for i in range(n):
        p = parent[i]
        paths.append((paths[p] if p >= 0 else ()) + (int(choice[i]),))
    return paths


@pytest.mark.parametrize("seed", range(6))
def test_nan_candidates_by_brute_force(seed):
    K, Dmax = 3, 4
    rng = np.random.default_rng(100 + seed)
    lp = logsoftmax(rng.normal(0, 2, size=(1, Dmax, K)))
    # NaN at a few (depth, candidate) places, the first at depth 0 so that a
    # NaN would sit among the earliest candidates of the pool
    lp[0, 0, rng.integers(K)] = np.nan
    for _ in range(2):
        lp[0, rng.integers(1, Dmax), rng.integers(K)] = np.nan
    allp = [(s, path) for s, path in enumerate_paths(lp[0], Dmax, K) if s == s]
    assert len(set(s for s, _ in allp)) == len(allp)
    best = sorted(allp, key=lambda x: -x[0])
    for T in (1, 4, 9, len(best), len(best) + 7, 120):
        parent, choice, score = oracle.build_tree(lp, T)
        m = min(T, len(best))
        assert paths_of(parent[0], choice[0], m) == [path for _, path in best[:m]]
        assert np.array_equal(score[0, :m], np.array([s for s, _ in best[:m]], dtype=np.float32))
        assert (parent[0, m:] == -1).all() and (choice[0, m:] == -1).all()
        assert np.isnan(score[0, m:]).all()


def test_chain_cut_by_a_nan_log_probability():
    # one candidate per depth, NaN at depth 3: the first three nodes form a
    # chain and every later node is missing
    Dmax, T = 8, 8
    lp = np.full((2, Dmax, 1), -0.5, dtype=np.float32)
    lp[1, 3, 0] = np.nan
    parent, choice, score = oracle.build_tree(lp, T)
    assert parent[0].tolist() == [-1] + list(range(T - 1))
    assert parent[1].tolist() == [-1, 0, 1] + [-1] * 5
    assert choice[1].tolist() == [0, 0, 0] + [-1] * 5
    assert score[1, :3].tolist() == [-0.5, -1.0, -1.5]
    assert np.isnan(score[1, 3:]).all()

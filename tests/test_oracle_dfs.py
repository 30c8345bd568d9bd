"""Pins of the oracle's depth-first relabelling (CPU only).

Each pin is independent of the stack walk the oracle uses:
- the preorder of a forest whose roots and children are taken in increasing
  index is the lexicographic order of the root-to-node index paths (every
  path is increasing, since parents precede children): sorting nodes by
  their path reproduces the permutation;
- a small tree whose preorder is written out by hand;
- closed forms: a chain and a forest of roots keep their labels;
- structure: parents precede children after relabelling, and every subtree
  occupies a contiguous range starting at its root;
- the attention output is invariant: the oracle run on relabelled inputs
  gives the original outputs, moved to the new rows (fp64, only the order of
  the tree-key sums differs);
- the plan's status codes for bad trees.
"""
import numpy as np
import torch
import pytest

import oracle
from tree_masked_attention_plan_amd import workloads as W


def paths(parent):
    """Root-to-node path of every node, as a tuple of local indices."""
    out = []
    for i in range(len(parent)):
        p, j = [], i
        while j != -1:
            p.append(j)
            j = int(parent[j])
        out.append(tuple(reversed(p)))
    return out


def forest(trees):
    parent = np.concatenate([np.asarray(t, np.int32) for t in trees]) if trees else np.zeros(0, np.int32)
    off = np.zeros(len(trees) + 1, np.int32)
    off[1:] = np.cumsum([len(t) for t in trees])
    return parent, off, np.zeros(len(trees), np.int32)


def sample_trees(seed):
    rng = W.rng_for(seed, 7)
    return [W.random_tree(int(rng.integers(1, 60)), 8, rng),
            W.best_first_tree(64, rng),
            W.best_first_tree(256, rng, per_node_logits=True),
            W.chain(9),
            np.full(5, -1, np.int32)]


@pytest.mark.parametrize("seed", range(4))
def test_permutation_is_the_lexicographic_order_of_paths(seed):
    trees = sample_trees(seed)
    parent, off, L = forest(trees)
    perm, inv, parent_new, status = oracle.dfs_order(parent, off, L, 256)
    assert (status == 0).all()
    for b, t in enumerate(trees):
        o = int(off[b])
        P = paths(t)
        expect = sorted(range(len(t)), key=lambda i: P[i])
        assert (perm[o:o + len(t)] - o).tolist() == expect
        assert (inv[perm[o:o + len(t)]] == np.arange(o, o + len(t))).all()


def test_hand_written_preorder():
    #        0        1           roots 0 and 1
    #       / \\       |
    #      2   4      3
    #      |
    #      5
    parent = np.array([-1, -1, 0, 1, 0, 2], np.int32)
    perm, inv, parent_new, status = oracle.dfs_order(parent, [0, 6], [3], 256)
    assert status.tolist() == [0]
    assert perm.tolist() == [0, 2, 5, 4, 1, 3]
    assert inv.tolist() == [0, 4, 1, 5, 3, 2]
    assert parent_new.tolist() == [-1, 0, 1, 0, -1, 4]


@pytest.mark.parametrize("T", [1, 7, 256])
def test_chain_and_roots_keep_their_labels(T):
    for tree in (W.chain(T), np.full(T, -1, np.int32)):
        perm, inv, parent_new, status = oracle.dfs_order(tree, [0, T], [0], 256)
        assert perm.tolist() == list(range(T))
        assert inv.tolist() == list(range(T))
        assert parent_new.tolist() == tree.tolist()


@pytest.mark.parametrize("seed", range(4))
def test_relabelled_tree_is_topological_with_contiguous_subtrees(seed):
    trees = sample_trees(seed)
    parent, off, L = forest(trees)
    perm, inv, parent_new, status = oracle.dfs_order(parent, off, L, 256)
    for b, t in enumerate(trees):
        o, T = int(off[b]), len(t)
        pn = parent_new[o:o + T]
        assert all(pn[i] < i for i in range(T))
        # the relabelled tree is the old one under the permutation
        for i_new in range(T):
            i_old = perm[o + i_new] - o
            p_old = t[i_old]
            assert pn[i_new] == (-1 if p_old == -1 else inv[o + p_old] - o)
        # subtree of node v = v and every node whose path passes through v
        P = paths(pn)
        for v in range(T):
            members = sorted(i for i in range(T) if v in P[i])
            assert members == list(range(v, v + len(members)))


def test_relabelled_attention_is_the_permuted_output():
    rng = W.rng_for(11, 3)
    trees = [W.best_first_tree(40, rng), W.random_tree(25, 6, rng)]
    w = W.make_workload("dfs-pin", [37, 80], trees, Hq=4, Hkv=2, D=16, dtype=torch.float32, seed=5)
    out, lse = oracle.tree_attn_workload(w)
    perm, inv, parent_new, status = oracle.dfs_order(w.parent, w.tree_off, w.prefix_len, w.max_tree)
    q = w.q.numpy()[perm]
    kt = w.k_tree.numpy()[perm]
    vt = w.v_tree.numpy()[perm]
    out2, lse2 = oracle.tree_attn(q, kt, vt, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                  w.tree_off, parent_new)
    np.testing.assert_allclose(out2, out[perm], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse[perm], rtol=0, atol=1e-12)
    # and the plan of the relabelled tree is the old plan with bits moved
    m0, d0, p0, _ = oracle.plan(w.parent, w.tree_off, w.prefix_len, w.max_tree)
    m1, d1, p1, _ = oracle.plan(parent_new, w.tree_off, w.prefix_len, w.max_tree)
    assert (d1 == d0[perm]).all() and (p1 == p0[perm]).all()


@pytest.mark.parametrize("parent,expect", [
    ([-1, 0, 2, 1], 3),     # node 2's parent is itself
    ([-1, -2, 0], 2),       # below -1
    ([0, -1], 1),           # the first node cannot have a parent
])
def test_bad_trees_report_the_plan_status(parent, expect):
    parent = np.asarray(parent, np.int32)
    _, _, _, status = oracle.dfs_order(parent, [0, len(parent)], [4], 256)
    assert status.tolist() == [expect]
    _, _, _, st_plan = oracle.plan(parent, [0, len(parent)], [4], 256)
    assert status.tolist() == st_plan.tolist()


def test_depth_first_order_skips_more_tree_tiles():
    """The reason for the relabelling: at budget 256 a best-first tree in
    depth-first order leaves fewer non-empty 32 x 32 blocks in the lower
    triangle of its ancestor matrix (mean over seeds)."""
    before, after = [], []
    for seed in range(6):
        t = W.best_first_tree(256, W.rng_for(seed, 9))
        _, _, pn, _ = oracle.dfs_order(t, [0, 256], [0], 256)
        for par, acc in ((t, before), (pn, after)):
            m, _, _, _ = oracle.plan(par, [0, 256], [0], 256)
            bits = np.unpackbits(m.view(np.uint8), bitorder="little").reshape(256, 256)
            blocks = bits.reshape(8, 32, 8, 32).any(axis=(1, 3))
            acc.append(int(np.tril(blocks).sum()))
    assert np.mean(after) < np.mean(before)

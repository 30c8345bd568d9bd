"""Pins of the oracle's accepted-path commit (CPU only).

The commit appends the K/V rows of the accepted node's root path, root
first, to the request's paged prefix.  Nothing printed on the pages fixes
values, so the pins are closed forms and independent facts:
- a chain accepting node a commits nodes 0..a in order;
- against the (separately pinned) plan oracle, the row at position L + d - 1
  is the ancestor of the accepted node whose depth is d;
- every byte outside the committed slots is untouched;
- two successive commits equal one flat append of both paths;
- the status codes.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_masked_attention_plan_amd import workloads as W


def rows_bytes(t):
    """uint8 view [.., Hkv, D * elem] of a K/V tensor."""
    return t.contiguous().view(torch.uint8).numpy()


def build(trees, lens, reserve, dtype=torch.bfloat16, page_size=16, Hkv=2, D=64, seed=7):
    return W.make_workload("commit", lens, trees, Hkv * 2, Hkv, D, dtype, seed,
                           page_size=page_size, reserve_tokens=reserve)


def slot_of(w, b, t):
    page = int(w.block_table[b, t // w.page_size])
    return page, t % w.page_size


def test_chain_commits_nodes_in_order():
    for a in (0, 4, 15):
        w = build([W.chain(16)], [21], reserve=16)
        kc, vc, new_len, st = oracle.commit(w.parent, w.tree_off, w.prefix_len, [a], w.k_tree, w.v_tree,
                                            w.k_cache, w.v_cache, w.block_table, max_tree=16)
        assert st.tolist() == [0] and new_len.tolist() == [21 + a + 1]
        kt, vt = rows_bytes(w.k_tree), rows_bytes(w.v_tree)
        for d in range(a + 1):
            pg, sl = slot_of(w, 0, 21 + d)
            assert np.array_equal(kc[pg, sl], kt[d]) and np.array_equal(vc[pg, sl], vt[d])


@pytest.mark.parametrize("dtype,page_size", [(torch.bfloat16, 16), (torch.float32, 16), (torch.bfloat16, 1),
                                             (torch.bfloat16, 64)])
def test_rows_are_the_accepted_nodes_ancestors_by_depth(dtype, page_size):
    rng = W.rng_for(11, 0)
    trees = [W.best_first_tree(40, rng), W.random_tree(30, 9, rng), W.chain(7), W.best_first_tree(64, rng)]
    lens = [0, 33, 100, 17]
    w = build(trees, lens, reserve=64, dtype=dtype, page_size=page_size)
    acc = np.array([39, 17, 6, 50], dtype=np.int32)
    kc, vc, new_len, st = oracle.commit(w.parent, w.tree_off, w.prefix_len, acc, w.k_tree, w.v_tree,
                                        w.k_cache, w.v_cache, w.block_table, max_tree=64)
    assert st.tolist() == [0, 0, 0, 0]
    mask, depth, _, pst = oracle.plan(w.parent, w.tree_off, w.prefix_len, max_tree=64)
    assert pst.tolist() == [0, 0, 0, 0]
    kt, vt = rows_bytes(w.k_tree), rows_bytes(w.v_tree)
    off = w.tree_off.numpy()
    written = set()
    for b in range(4):
        a = int(off[b] + acc[b])
        da = int(depth[a])
        assert new_len[b] == lens[b] + da
        anc = [int(off[b]) + j for j in range(trees[b].size) if (int(mask[a, j // 64]) >> (j % 64)) & 1]
        assert len(anc) == da
        for d in range(1, da + 1):
            (node,) = [n for n in anc if depth[n] == d]
            pg, sl = slot_of(w, b, lens[b] + d - 1)
            assert np.array_equal(kc[pg, sl], kt[node]) and np.array_equal(vc[pg, sl], vt[node])
            written.add((pg, sl))
    # everything else is byte-identical (NaN sentinels included)
    k0, v0 = rows_bytes(w.k_cache), rows_bytes(w.v_cache)
    for pg in range(w.num_pages):
        for sl in range(w.page_size):
            if (pg, sl) not in written:
                assert np.array_equal(kc[pg, sl], k0[pg, sl]) and np.array_equal(vc[pg, sl], v0[pg, sl])


def test_nothing_accepted_changes_nothing():
    w = build([W.chain(5), W.chain(3)], [10, 0], reserve=8)
    kc, vc, new_len, st = oracle.commit(w.parent, w.tree_off, w.prefix_len, [-1, -1], w.k_tree, w.v_tree,
                                        w.k_cache, w.v_cache, w.block_table, max_tree=5)
    assert st.tolist() == [0, 0] and new_len.tolist() == [10, 0]
    assert np.array_equal(kc, rows_bytes(w.k_cache)) and np.array_equal(vc, rows_bytes(w.v_cache))


def test_two_commits_equal_one_flat_append():
    # commit node 2 of a chain, then (the next step's tree being the chain's
    # continuation) commit 3 more: the cache then holds all 6 rows in order
    w = build([W.chain(6)], [9], reserve=16)
    kc, vc, n1, _ = oracle.commit(w.parent, w.tree_off, w.prefix_len, [2], w.k_tree, w.v_tree,
                                  w.k_cache, w.v_cache, w.block_table, max_tree=6)
    assert n1.tolist() == [12]
    tail = W.chain(3)
    kt2 = w.k_tree[3:].clone()
    vt2 = w.v_tree[3:].clone()
    kc_t = torch.from_numpy(kc).view(w.k_cache.dtype).view(w.k_cache.shape)
    vc_t = torch.from_numpy(vc).view(w.v_cache.dtype).view(w.v_cache.shape)
    kc2, vc2, n2, st = oracle.commit(torch.from_numpy(tail), torch.tensor([0, 3], dtype=torch.int32),
                                     torch.from_numpy(n1), [2], kt2, vt2, kc_t, vc_t, w.block_table, max_tree=3)
    assert st.tolist() == [0] and n2.tolist() == [15]
    kt = rows_bytes(w.k_tree)
    for d in range(6):
        pg, sl = slot_of(w, 0, 9 + d)
        assert np.array_equal(kc2[pg, sl], kt[d])


def test_error_statuses_write_nothing_for_that_request():
    trees = [W.chain(4), np.array([-1, 0, 2, 1], np.int32), W.chain(4), W.chain(4), W.chain(4)]
    lens = [5, 5, 5, -1, 60]
    w = build(trees, [max(x, 0) for x in lens], reserve=8)
    prefix = torch.tensor(lens, dtype=torch.int32)
    bt = w.block_table.clone()
    bt[4, :] = -1                         # request 4's pages are gone
    acc = [4, 3, 2, 0, 1]                 # 4 is out of range for request 0
    kc, vc, new_len, st = oracle.commit(w.parent, w.tree_off, prefix, acc, w.k_tree, w.v_tree,
                                        w.k_cache, w.v_cache, bt, max_tree=4)
    # request 1: node 3's parent 1 is fine, node 1's parent 0 fine... node 3 -> 1 -> 0: valid;
    # node 2 (parent 2 >= 2) is not on that path, so request 1 commits
    assert st.tolist() == [-3, 0, 0, -2, -4]
    assert new_len.tolist() == [5, 5 + 3, 5 + 3, -1, 60]
    # a path through a bad parent is reported with the node's one-based id
    _, _, _, st2 = oracle.commit(w.parent, w.tree_off, w.prefix_len, [0, 2, 0, 0, 0], w.k_tree, w.v_tree,
                                 w.k_cache, w.v_cache, w.block_table, max_tree=4)
    assert st2[1] == 3
    # a broken offsets array
    off = w.tree_off.clone()
    off[0] = 1
    _, _, _, st3 = oracle.commit(w.parent, off, w.prefix_len, acc, w.k_tree, w.v_tree, w.k_cache,
                                 w.v_cache, w.block_table, max_tree=4)
    assert st3[0] == -1
    # only request 1 and 2 wrote anything
    k0 = rows_bytes(w.k_cache)
    changed = {(pg, sl) for pg in range(w.num_pages) for sl in range(w.page_size)
               if not np.array_equal(kc[pg, sl], k0[pg, sl])}
    expect = {slot_of(w, 1, 5 + d) for d in range(3)} | {slot_of(w, 2, 5 + d) for d in range(3)}
    assert changed == expect

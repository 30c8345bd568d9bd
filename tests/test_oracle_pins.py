"""Pins of the fp64 oracle against facts that do not come from the oracle.

Every check here compares the oracle with something independent of its code:
closed forms, a hand-derived fixture, torch's fp64 scaled_dot_product_attention
(a library routine) on the cases where tree attention reduces to ordinary
causal attention, a separate brute force, and exact invariances of the
definition.  CPU only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tree_masked_attention_plan_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_workload(prefix_lens, trees, Hq=4, Hkv=2, D=16, page_size=16, seed=7,
                   dtype=torch.float64):
    return W.make_workload("small", prefix_lens, trees, Hq, Hkv, D, dtype, seed,
                           page_size=page_size)


def logical_prefix(w, b):
    """[L, Hkv, D] prefix K and V of request b gathered through its block table."""
    L = int(w.prefix_len[b])
    t = torch.arange(L)
    pages = w.block_table[b, t // w.page_size].long()
    k = w.k_cache[pages, t % w.page_size].double()
    v = w.v_cache[pages, t % w.page_size].double()
    return k, v


def root_path(parent, off, i):
    path = []
    j = i
    while j != -1:
        path.append(j)
        j = int(parent[off + j])
    return path[::-1]


# ---------------------------------------------------------------- plan pins

def test_plan_hand_fixture():
    g = json.load(open(os.path.join(GOLDEN, "hand_forest.json")))
    mask, depth, pos, status = oracle.plan(np.array(g["parent"], np.int32),
                                           np.array(g["tree_off"], np.int32),
                                           np.array(g["prefix_len"], np.int32), 6)
    assert status.tolist() == [0, 0]
    off = g["tree_off"]
    for n, anc in enumerate(g["expected_ancestors"]):
        bits = {j for j in range(256) if (int(mask[n, j // 64]) >> (j % 64)) & 1}
        assert bits == set(anc), n
    assert depth.tolist() == g["expected_depth"]
    assert pos.tolist() == g["expected_pos_id"]
    assert off[-1] == len(g["parent"])


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 200, 256])
def test_plan_chain_closed_form(T):
    L = 37
    mask, depth, pos, status = oracle.plan(W.chain(T), np.array([0, T], np.int32),
                                           np.array([L], np.int32), 256)
    assert status.tolist() == [0]
    for i in range(T):
        want = (1 << (i + 1)) - 1          # lower-triangular row of ones
        got = sum(int(mask[i, w]) << (64 * w) for w in range(4))
        assert got == want
    assert depth.tolist() == list(range(1, T + 1))
    assert pos.tolist() == [L + i for i in range(T)]


def test_plan_recurrence_and_popcount():
    rng = W.rng_for(3, 0)
    trees = [W.random_tree(40, 9, rng), W.best_first_tree(256, rng), W.chain(5),
             W.best_first_tree(17, rng, per_node_logits=True)]
    off = np.concatenate([[0], np.cumsum([len(t) for t in trees])]).astype(np.int32)
    L = np.array([0, 5, 100, 16], np.int32)
    parent = np.concatenate(trees)
    mask, depth, pos, status = oracle.plan(parent, off, L, 256)
    assert status.tolist() == [0, 0, 0, 0]
    for b in range(4):
        for i in range(off[b + 1] - off[b]):
            n = off[b] + i
            row = sum(int(mask[n, w]) << (64 * w) for w in range(4))
            p = parent[n]
            prow = 0 if p < 0 else sum(int(mask[off[b] + p, w]) << (64 * w) for w in range(4))
            assert row == prow | (1 << i)                  # A(i) = {i} U A(parent(i))
            assert bin(row).count("1") == depth[n]         # depth = |A(i)|
            assert pos[n] == L[b] + depth[n] - 1
            assert row >> (i + 1) == 0                     # no descendants / later nodes


def test_plan_relabel_invariance():
    rng = W.rng_for(11, 0)
    par = W.best_first_tree(150, rng)
    newp, sigma = W.topo_relabel(par, rng)
    off = np.array([0, 150], np.int32)
    L = np.array([3], np.int32)
    m1, d1, p1, _ = oracle.plan(par, off, L, 256)
    m2, d2, p2, _ = oracle.plan(newp, off, L, 256)

    def bits(m, n):
        return {j for j in range(256) if (int(m[n, j // 64]) >> (j % 64)) & 1}
    for i in range(150):
        assert {int(sigma[j]) for j in bits(m1, i)} == bits(m2, int(sigma[i]))
        assert d1[i] == d2[sigma[i]] and p1[i] == p2[sigma[i]]


def test_plan_error_statuses():
    # request 0 fine; request 1 has parent[2] = 2 (not earlier); request 2 has
    # parent[1] = -2; request 3 has a negative prefix length.
    parent = np.array([-1, 0, -1, 0, 2, -1, -2, 0, 0, -1], np.int32)
    off = np.array([0, 2, 5, 8, 10], np.int32)
    L = np.array([4, 4, 4, -1], np.int32)
    _, _, _, status = oracle.plan(parent, off, L, 256)
    assert status.tolist() == [0, 3, 2, -2]
    # tree larger than max_tree, and inconsistent offsets
    _, _, _, status = oracle.plan(np.array([-1, 0, 1], np.int32), np.array([0, 3], np.int32),
                                  np.array([0], np.int32), 2)
    assert status.tolist() == [-1]
    _, _, _, status = oracle.plan(np.array([-1, 0, 1], np.int32), np.array([0, 2], np.int32),
                                  np.array([0], np.int32), 8)
    assert status.tolist() == [-1]
    _, _, _, status = oracle.plan(np.array([-1, 0, 1], np.int32), np.array([0, 1, 0], np.int32),
                                  np.array([0, 0], np.int32), 8)
    assert status.tolist()[1] == -1


# ----------------------------------------------------------- attention pins

def test_attn_hand_fixture():
    g = json.load(open(os.path.join(GOLDEN, "hand_forest.json")))
    N, D = len(g["parent"]), g["D"]
    ps, P = g["page_size"], g["num_pages"]
    k_cache = np.full((P, ps, 1, D), np.nan)
    v_cache = np.full((P, ps, 1, D), np.nan)
    pk = g["prefix_k"]
    k_cache[pk["page"], pk["slot"], 0] = pk["k"]
    v_cache[pk["page"], pk["slot"], 0] = pk["v"]
    k_tree = np.zeros((N, 1, D))
    k_tree[:, 0, 0] = [math.log(float(Fraction(a))) for a in g["tree_weight"]]
    v_tree = np.array(g["tree_v"], np.float64).reshape(N, 1, D)
    q = np.zeros((N, 1, D))
    q[:, 0, 0] = 1.0
    out, lse = oracle.tree_attn(q, k_tree, v_tree, k_cache, v_cache,
                                np.array(g["block_table"], np.int32),
                                np.array(g["prefix_len"], np.int32),
                                np.array(g["tree_off"], np.int32),
                                np.array(g["parent"], np.int32), scale=g["scale"])
    want_o = np.array([[float(Fraction(x)) for x in row] for row in g["expected_out"]])
    want_l = np.array([math.log(float(Fraction(x))) for x in g["expected_lse_exp"]])
    np.testing.assert_allclose(out[:, 0], want_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[:, 0], want_l, rtol=0, atol=1e-14)


def _sdpa_flat(q_rows, k_seq, v_seq, q_pos, scale):
    """fp64 SDPA: query r sits at flat position q_pos[r] and sees keys 0..q_pos[r].

    q_rows [R,Hq,D], k_seq/v_seq [S,Hq,D] (already expanded to q heads).
    The causal mask is given explicitly (bottom-right aligned), not through
    is_causal, which aligns top-left when there are fewer queries than keys."""
    S = k_seq.shape[0]
    mask = torch.arange(S)[None, :] <= torch.as_tensor(q_pos)[:, None]
    qh = q_rows.permute(1, 0, 2).double()
    kh = k_seq.permute(1, 0, 2).double()
    vh = v_seq.permute(1, 0, 2).double()
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)
    s = torch.matmul(qh, kh.transpose(1, 2).contiguous()) * scale
    s = s.masked_fill(~mask, float("-inf"))
    return o.permute(1, 0, 2), torch.logsumexp(s, dim=-1).T


@pytest.mark.parametrize("L,T,ps", [(0, 1, 16), (0, 9, 16), (45, 16, 16), (128, 16, 4),
                                    (77, 33, 1), (300, 64, 16)])
def test_chain_equals_causal_sdpa(L, T, ps):
    Hq, Hkv, D = 6, 2, 8
    w = small_workload([L], [W.chain(T)], Hq, Hkv, D, page_size=ps, seed=L * 31 + T)
    out, lse = oracle.tree_attn_workload(w)
    kp, vp = logical_prefix(w, 0)
    G = Hq // Hkv
    k_seq = torch.cat([kp, w.k_tree.double()]).repeat_interleave(G, dim=1)
    v_seq = torch.cat([vp, w.v_tree.double()]).repeat_interleave(G, dim=1)
    o_ref, l_ref = _sdpa_flat(w.q, k_seq, v_seq, L + torch.arange(T), w.scale)
    np.testing.assert_allclose(out, o_ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_ref.numpy(), rtol=0, atol=1e-12)


def _trees_for_brute(seed):
    rng = W.rng_for(seed, 0)
    return [W.random_tree(12, 5, rng), W.best_first_tree(10, rng, max_depth=4, children=3),
            np.array([-1, -1, 0, 1, 0, 2, -1], np.int32), W.chain(1)]


@pytest.mark.parametrize("seed,ps", [(1, 16), (2, 4), (3, 1)])
def test_path_as_flat_sequence(seed, ps):
    """Each node's row equals causal attention over prefix ++ (root..node) run
    as one flat sequence (the branch factorisation); every path node's query
    is placed at its own position, so all rows along the path are checked."""
    trees = _trees_for_brute(seed)
    prefix = [37, 0, 16, 5]
    Hq, Hkv, D = 4, 2, 8
    G = Hq // Hkv
    w = small_workload(prefix, trees, Hq, Hkv, D, page_size=ps, seed=seed)
    out, lse = oracle.tree_attn_workload(w)
    off = w.tree_off.numpy()
    par = w.parent.numpy()
    for b in range(w.B):
        kp, vp = logical_prefix(w, b)
        L = int(w.prefix_len[b])
        for i in range(off[b + 1] - off[b]):
            path = root_path(par, off[b], i)
            nodes = [off[b] + j for j in path]
            k_seq = torch.cat([kp, w.k_tree[nodes].double()]).repeat_interleave(G, dim=1)
            v_seq = torch.cat([vp, w.v_tree[nodes].double()]).repeat_interleave(G, dim=1)
            o_ref, l_ref = _sdpa_flat(w.q[nodes], k_seq, v_seq, L + torch.arange(len(path)), w.scale)
            np.testing.assert_allclose(out[nodes], o_ref.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[nodes], l_ref.numpy(), rtol=0, atol=1e-12)
            # separate numpy brute force of the last row (no torch)
            n = off[b] + i
            for h in range(Hq):
                c = h // G
                ks = np.concatenate([kp[:, c].numpy(), w.k_tree[nodes, c].double().numpy()])
                vs = np.concatenate([vp[:, c].numpy(), w.v_tree[nodes, c].double().numpy()])
                s = ks @ w.q[n, h].double().numpy() * w.scale
                e = np.exp(s - s.max())
                np.testing.assert_allclose(out[n, h], e @ vs / e.sum(), rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse[n, h], s.max() + np.log(e.sum()), rtol=0, atol=1e-12)


def test_relabel_invariance_exact():
    rng = W.rng_for(5, 0)
    par = W.best_first_tree(90, rng)
    newp, sigma = W.topo_relabel(par, rng)
    w1 = small_workload([50], [par], seed=5)
    inv = np.argsort(sigma)               # inv[new] = old
    w2 = small_workload([50], [newp], seed=5)
    w2.q = w1.q[inv]
    w2.k_tree = w1.k_tree[inv]
    w2.v_tree = w1.v_tree[inv]
    o1, l1 = oracle.tree_attn_workload(w1)
    o2, l2 = oracle.tree_attn_workload(w2)
    assert np.array_equal(o2[sigma], o1) and np.array_equal(l2[sigma], l1)


def test_page_permutation_and_page_size_invariance():
    rng = W.rng_for(9, 0)
    trees = [W.best_first_tree(20, rng), W.chain(3)]
    w1 = small_workload([70, 33], trees, page_size=16, seed=9)
    o1, l1 = oracle.tree_attn_workload(w1)
    # a fresh physical permutation of the same logical prefix
    w2 = small_workload([70, 33], trees, page_size=16, seed=9)
    P = w2.num_pages
    perm = torch.from_numpy(W.rng_for(99, 0).permutation(P))
    k2 = torch.empty_like(w2.k_cache)
    v2 = torch.empty_like(w2.v_cache)
    k2[perm] = w2.k_cache
    v2[perm] = w2.v_cache
    bt = w2.block_table.clone()
    bt[bt >= 0] = perm[bt[bt >= 0].long()].int()
    w2.k_cache, w2.v_cache, w2.block_table = k2, v2, bt
    o2, l2 = oracle.tree_attn_workload(w2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # contiguous, unpaged layout: one token per page in logical order
    pre = [logical_prefix(w1, b) for b in range(2)]
    k_flat = torch.cat([k for k, _ in pre])[:, None]
    v_flat = torch.cat([v for _, v in pre])[:, None]
    bt = torch.full((2, 70), -1, dtype=torch.int32)
    bt[0, :70] = torch.arange(70)
    bt[1, :33] = 70 + torch.arange(33)
    o3, l3 = oracle.tree_attn(w1.q, w1.k_tree, w1.v_tree, k_flat, v_flat, bt, w1.prefix_len,
                              w1.tree_off, w1.parent, scale=w1.scale)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


def test_non_ancestors_do_not_leak():
    rng = W.rng_for(13, 0)
    par = W.best_first_tree(40, rng)
    w = small_workload([25], [par], seed=13)
    o1, l1 = oracle.tree_attn_workload(w)
    for i in (0, 7, 21, 39):
        anc = set(root_path(par, 0, i))
        others = [j for j in range(40) if j not in anc]
        w2 = small_workload([25], [par], seed=13)
        w2.k_tree[others] = torch.randn(len(others), w.Hkv, w.D, dtype=w.k_tree.dtype) * 5
        w2.v_tree[others] = torch.randn(len(others), w.Hkv, w.D, dtype=w.v_tree.dtype) * 5
        o2, l2 = oracle.tree_attn_workload(w2)
        assert np.array_equal(o1[i], o2[i]) and np.array_equal(l1[i], l2[i])
        # and every ancestor (self included) does matter
        for a in anc:
            w3 = small_workload([25], [par], seed=13)
            w3.v_tree[a] += 1.0
            o3, _ = oracle.tree_attn_workload(w3)
            assert not np.array_equal(o1[i], o3[i])


def test_lse_merge_of_prefix_halves():
    """The split-K merge rule on oracle outputs.  Every row sees its root
    path, so runs over the first half of the prefix (A) and the second half
    (B) both hold the tree; a run with no prefix (C) removes the double count:
    e^lse = e^lse_A + e^lse_B - e^lse_C and O e^lse = O_A e^lse_A +
    O_B e^lse_B - O_C e^lse_C, to fp64 rounding.  This pins lse as the natural
    log of the row's exp-sum and O as the normalised weighted sum."""
    rng = W.rng_for(29, 0)
    trees = [W.best_first_tree(24, rng), W.random_tree(17, 5, rng)]
    w = small_workload([200, 75], trees, seed=29)
    ps = w.page_size
    o_f, l_f = oracle.tree_attn_workload(w)
    half = torch.tensor([(int(L) // (2 * ps)) * ps for L in w.prefix_len], dtype=torch.int32)
    bt_b = torch.full_like(w.block_table, -1)
    for b in range(w.B):
        skip = int(half[b]) // ps
        bt_b[b, :w.max_pages - skip] = w.block_table[b, skip:]
    run = lambda bt, L: oracle.tree_attn(w.q, w.k_tree, w.v_tree, w.k_cache, w.v_cache, bt, L,
                                        w.tree_off, w.parent, scale=w.scale)
    o_a, l_a = run(w.block_table, half)
    o_b, l_b = run(bt_b, w.prefix_len - half)
    o_c, l_c = run(w.block_table, torch.zeros_like(w.prefix_len))
    m = np.maximum(np.maximum(l_a, l_b), l_c)
    ea, eb, ec = np.exp(l_a - m), np.exp(l_b - m), np.exp(l_c - m)
    tot = ea + eb - ec
    np.testing.assert_allclose(np.log(tot) + m, l_f, rtol=0, atol=1e-12)
    merged = (o_a * ea[..., None] + o_b * eb[..., None] - o_c * ec[..., None]) / tot[..., None]
    np.testing.assert_allclose(merged, o_f, rtol=0, atol=1e-11)


def test_zero_keys_closed_form():
    rng = W.rng_for(17, 0)
    trees = [W.random_tree(30, 6, rng), W.chain(4)]
    w = small_workload([19, 0], trees, seed=17)
    w.k_cache.zero_()
    w.k_tree.zero_()
    out, lse = oracle.tree_attn_workload(w)
    off = w.tree_off.numpy()
    par = w.parent.numpy()
    G = w.Hq // w.Hkv
    for b in range(2):
        kp, vp = logical_prefix(w, b)
        L = int(w.prefix_len[b])
        for i in range(off[b + 1] - off[b]):
            nodes = [off[b] + j for j in root_path(par, off[b], i)]
            vis = torch.cat([vp, w.v_tree[nodes].double()])        # all scores are 0
            for h in range(w.Hq):
                np.testing.assert_allclose(out[off[b] + i, h], vis[:, h // G].mean(0).numpy(),
                                           rtol=0, atol=1e-13)
                assert abs(lse[off[b] + i, h] - math.log(L + len(nodes))) < 1e-13


def test_one_visible_key():
    # no prefix, single root: the only visible key is the node's own
    w = small_workload([0, 0], [W.chain(1), np.array([-1, -1], np.int32)], seed=21)
    out, lse = oracle.tree_attn_workload(w)
    G = w.Hq // w.Hkv
    for n in range(3):
        for h in range(w.Hq):
            np.testing.assert_array_equal(out[n, h], w.v_tree[n, h // G].double().numpy())
            s = w.scale * float(w.q[n, h].double() @ w.k_tree[n, h // G].double())
            assert abs(lse[n, h] - s) < 1e-13


def test_gqa_equals_repeat_interleave_mha():
    rng = W.rng_for(23, 0)
    trees = [W.best_first_tree(24, rng), W.random_tree(9, 4, rng)]
    w = small_workload([40, 17], trees, Hq=8, Hkv=2, seed=23)
    o1, l1 = oracle.tree_attn_workload(w)
    G = 4
    o2, l2 = oracle.tree_attn(w.q, w.k_tree.repeat_interleave(G, 1), w.v_tree.repeat_interleave(G, 1),
                              w.k_cache.repeat_interleave(G, 2), w.v_cache.repeat_interleave(G, 2),
                              w.block_table, w.prefix_len, w.tree_off, w.parent, scale=w.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_row_subset_matches_full():
    rng = W.rng_for(29, 0)
    w = small_workload([33, 64], [W.best_first_tree(30, rng), W.chain(7)], seed=29)
    out, lse = oracle.tree_attn_workload(w)
    rows = np.array([0, 5, 30 * 4 + 1, w.N * w.Hq - 1])
    o2, l2 = oracle.tree_attn_workload(w, rows=rows)
    assert np.array_equal(o2, out.reshape(-1, w.D)[rows]) and np.array_equal(l2, lse.reshape(-1)[rows])


def test_threads_do_not_change_results():
    w = small_workload([100], [W.best_first_tree(50, W.rng_for(31, 0))], seed=31)
    o1, l1 = oracle.tree_attn_workload(w, threads=1)
    o2, l2 = oracle.tree_attn_workload(w, threads=7)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_oracle_rejects_cyclic_or_forward_parents():
    w = small_workload([4], [np.array([-1, 0, 3, 1], np.int32)], seed=3)
    with pytest.raises(ValueError):
        oracle.tree_attn_workload(w)

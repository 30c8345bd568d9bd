"""GPU parity of the depth-first relabelling (tree_attn_plan_dfs) and the row
gather (tree_attn_gather_rows) against the oracle.

- permutation, inverse and relabelled parents: bit-exact against
  oracle.dfs_order on forests, best-first trees, chains and the named
  workloads' trees;
- the relabelled plan (mask, depth, position id): bit-exact against the
  oracle's plan of the oracle's relabelled parents;
- status codes for bad trees: those of the oracle;
- gather: bit-exact against indexing, with out-of-range indices giving zero
  rows;
- end to end: attention run in the depth-first order (inputs gathered with
  perm, outputs gathered back with inv_perm) meets the parity bars against
  the oracle in the old order.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_masked_attention_plan_amd as ta
from tree_masked_attention_plan_amd import workloads as W
from tests.test_gpu_parity import assert_close

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP device")
    ta.load_library()
    return torch.device("cuda:0")


def forest(trees, L=None):
    parent = np.concatenate([np.asarray(t, np.int32) for t in trees])
    off = np.zeros(len(trees) + 1, np.int32)
    off[1:] = np.cumsum([len(t) for t in trees])
    L = np.zeros(len(trees), np.int32) if L is None else np.asarray(L, np.int32)
    return parent, off, L


def run_dfs(dev, parent, off, L, max_tree):
    t = lambda a: torch.as_tensor(np.asarray(a, np.int32)).to(dev)
    r = ta.plan_dfs(t(parent), t(off), t(L), max_tree=max_tree)
    torch.cuda.synchronize()
    return r


def check_against_oracle(r, parent, off, L, max_tree, what):
    perm, inv, pn, st = oracle.dfs_order(parent, off, L, max_tree)
    g_st = r.plan.status.cpu().numpy()
    say(f"  {what}: status {g_st.tolist()[:8]}")
    assert g_st.tolist() == st.tolist()
    ok = np.zeros(len(parent), bool)
    for b in range(len(L)):
        if st[b] == 0:
            ok[off[b]:off[b + 1]] = True
    assert np.array_equal(r.perm.cpu().numpy()[ok], perm[ok]), what
    assert np.array_equal(r.inv_perm.cpu().numpy()[ok], inv[ok]), what
    assert np.array_equal(r.parent_new.cpu().numpy()[ok], pn[ok]), what
    # the plan of the relabelled trees, from the oracle's relabelled parents
    pn_fixed = np.where(ok, pn, -1).astype(np.int32)
    m, d, p, _ = oracle.plan(pn_fixed, off, np.maximum(L, 0), max_tree)
    assert np.array_equal(r.plan.anc_mask.cpu().numpy().view(np.uint64)[ok], m[ok]), what
    assert np.array_equal(r.plan.depth.cpu().numpy()[ok], d[ok]), what
    assert np.array_equal(r.plan.pos_id.cpu().numpy()[ok], p[ok]), what


def test_forests_bit_exact(dev):
    rng = W.rng_for(5, 1)
    trees = [W.best_first_tree(256, rng), W.random_tree(100, 12, rng), W.chain(256),
             np.full(37, -1, np.int32), np.array([-1, -1, 0, 1, 0, 2], np.int32), W.chain(1),
             np.zeros(0, np.int32), W.best_first_tree(64, rng, per_node_logits=True),
             W.random_tree(256, 3, rng)]
    parent, off, _ = forest(trees)
    L = np.array([0, 7, 2048, 1, 3, 0, 5, 100, 9], np.int32)
    say(f"plan_dfs forests: B={len(trees)} N={len(parent)}")
    check_against_oracle(run_dfs(dev, parent, off, L, 256), parent, off, L, 256, "forests")


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_named_workload_trees_bit_exact(dev, name):
    w = W.make_config(name)
    say(f"plan_dfs {name}: B={w.B} N={w.N}")
    parent, off, L = (w.parent.numpy(), w.tree_off.numpy(), w.prefix_len.numpy())
    check_against_oracle(run_dfs(dev, parent, off, L, w.max_tree), parent, off, L, w.max_tree, name)


def test_bad_trees_report_the_oracle_status(dev):
    # request 0 fine, 1 with a self parent, 2 with parent < -1, 3 with a
    # negative prefix, 4 fine
    parent = np.array([-1, 0, -1, 0, 2, 1, -1, -2, 0, -1, 0, -1, 0, 1], np.int32)
    off = np.array([0, 2, 6, 9, 11, 14], np.int32)
    L = np.array([4, 4, 4, -1, 0], np.int32)
    say("plan_dfs error statuses")
    r = run_dfs(dev, parent, off, L, 4)
    check_against_oracle(r, parent, off, L, 4, "bad trees")
    assert r.plan.status.cpu().numpy().tolist() == [0, 3, 2, -2, 0]


@pytest.mark.parametrize("dtype,shape", [(torch.bfloat16, (300, 32, 128)), (torch.float32, (77, 32)),
                                         (torch.int32, (50, 3)), (torch.float32, (1, 4))])
def test_gather_rows_bit_exact(dev, dtype, shape):
    g = torch.Generator().manual_seed(3)
    src = torch.randn(shape, generator=g).to(dtype) if dtype != torch.int32 else \
        torch.randint(-9, 9, shape, generator=g, dtype=torch.int32)
    n = shape[0]
    idx = torch.randint(0, n, (n + 5,), generator=g, dtype=torch.int32)
    idx[3] = -1
    idx[-1] = n          # out of range: zero rows
    say(f"gather {dtype} {tuple(shape)}")
    out = ta.gather_rows(src.to(dev), idx.to(dev))
    torch.cuda.synchronize()
    ref = torch.zeros((n + 5,) + tuple(shape[1:]), dtype=src.dtype)
    okm = (idx >= 0) & (idx < n)
    ref[okm] = src[idx[okm].long()]
    assert torch.equal(out.cpu(), ref)


@pytest.mark.parametrize("name", ["dfs-mixed", "tree256-short"])
def test_attention_in_depth_first_order(dev, name):
    rng = W.rng_for(17, 2)
    if name == "dfs-mixed":
        trees = [W.best_first_tree(64, rng), W.best_first_tree(200, rng), W.random_tree(40, 8, rng)]
        w = W.make_workload(name, [300, 1000, 64], trees, 32, 8, 128, torch.bfloat16, 17)
    else:
        w = W.make_workload(name, [256], [W.best_first_tree(256, rng)], 32, 8, 128, torch.bfloat16, 18)
    say(f"fwd in depth-first order {name}: B={w.B} N={w.N}")
    wd = w.to(dev)
    r = ta.plan_dfs(wd.parent, wd.tree_off, wd.prefix_len, max_tree=w.max_tree)
    ta.check_status(r.plan.status)
    q = ta.gather_rows(wd.q, r.perm)
    kt = ta.gather_rows(wd.k_tree, r.perm)
    vt = ta.gather_rows(wd.v_tree, r.perm)
    out_n, lse_n = ta.fwd(q, kt, vt, wd.k_cache, wd.v_cache, wd.block_table, wd.prefix_len, wd.tree_off,
                          r.plan.anc_mask, max_tree=w.max_tree, max_prefix=w.max_prefix)
    out = ta.gather_rows(out_n, r.inv_perm)
    lse = ta.gather_rows(lse_n, r.inv_perm)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.tree_attn_workload(w)
    assert_close(w, out.float().cpu().double(), lse.cpu().double(), o_ref, l_ref, what=name)

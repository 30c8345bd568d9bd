"""GPU parity of tree_attn_plan_fwd: the plan built inside the attention
kernel, from the parent array, in the same call as the attention.

- out / lse meet the parity bars against the oracle (the same bars as
  tree_attn_fwd) on the five named workloads and on the small cases, over
  several split counts;
- the plan outputs (mask, depth, position id, status) are bit-exact against
  the oracle's plan, bad trees included; the rows of a batch's valid
  requests are unaffected by its bad ones;
- with bf16 the one-call result equals plan + fwd bit for bit (the attention
  arithmetic is the same, only the mask's source differs);
- a captured HIP graph of the call replays to the eager result.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_masked_attention_plan_amd as ta
from tree_masked_attention_plan_amd import workloads as W
from tests.test_gpu_parity import CASES, assert_close, random_config, small

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP device")
    ta.load_library()
    return torch.device("cuda:0")


def run(w, dev, num_splits=0, parent=None, prefix_len=None, tree_off=None):
    say(f"plan_fwd {w.name}: B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} dtype={w.dtype} "
        f"max_prefix={w.max_prefix} max_tree={w.max_tree} splits={num_splits}")
    wd = w.to(dev)
    t = lambda a, d: d if a is None else torch.as_tensor(np.asarray(a, np.int32)).to(dev)
    plan, out, lse = ta.plan_fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                                 t(prefix_len, wd.prefix_len), t(tree_off, wd.tree_off),
                                 t(parent, wd.parent), max_tree=w.max_tree, max_prefix=w.max_prefix,
                                 num_splits=num_splits)
    torch.cuda.synchronize()
    return plan, out.float().cpu().double(), lse.cpu().double()


def check_plan(plan, parent, tree_off, prefix_len, max_tree, what=""):
    """Status of every request as the oracle's; mask, depth and position ids
    of the valid requests' nodes bit-exact.  Returns the valid-node mask."""
    parent, tree_off, prefix_len = (np.asarray(a, np.int32) for a in (parent, tree_off, prefix_len))
    m, d, p, s = oracle.plan(parent, tree_off, prefix_len, max_tree)
    st = plan.status.cpu().numpy()
    say(f"  {what}: status {st.tolist()[:8]}")
    assert st.tolist() == s.tolist(), what
    ok = np.zeros(len(parent), bool)
    for b in range(len(prefix_len)):
        if s[b] == 0:
            ok[tree_off[b]:tree_off[b + 1]] = True
    assert np.array_equal(plan.anc_mask.cpu().numpy().view(np.uint64)[ok], m[ok]), what
    assert np.array_equal(plan.depth.cpu().numpy()[ok], d[ok]), what
    assert np.array_equal(plan.pos_id.cpu().numpy()[ok], p[ok]), what
    return ok


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_named_workload(dev, name, named_reference):
    """Every (node, head) row of each named workload against the oracle, and
    the plan bit-exact."""
    w, o_ref, l_ref = named_reference(name)
    plan, out, lse = run(w, dev)
    check_plan(plan, w.parent, w.tree_off, w.prefix_len, w.max_tree, name)
    assert_close(w, out, lse, o_ref, l_ref, f"{name} (all {w.N * w.Hq} rows)", raw=True)


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_small_cases(dev, idx):
    name, prefix, trees, kw = CASES[idx]
    w = small(name, prefix, trees, seed=100 + idx, **kw)
    o_ref, l_ref = oracle.tree_attn_workload(w)
    splits = (0, 1, 3, 64) if w.dtype == torch.bfloat16 and w.max_prefix > 0 else (0,)
    for ns in splits:
        plan, out, lse = run(w, dev, num_splits=ns)
        check_plan(plan, w.parent, w.tree_off, w.prefix_len, w.max_tree, f"{name} splits={ns}")
        assert_close(w, out, lse, o_ref, l_ref, f"{name} splits={ns}")


@pytest.mark.parametrize("i", range(200))
def test_random_configurations(dev, i):
    """The seeded random shapes of the forward tests, through the one call."""
    name, prefix, trees, kw, splits = random_config(i)
    w = small(name, prefix, trees, seed=700 + i, **kw)
    o_ref, l_ref = oracle.tree_attn_workload(w)
    plan, out, lse = run(w, dev, num_splits=splits)
    check_plan(plan, w.parent, w.tree_off, w.prefix_len, w.max_tree, name)
    assert_close(w, out, lse, o_ref, l_ref, f"{name} one call, splits={splits}")


@pytest.mark.parametrize("num_splits", [1, 4])
def test_bad_trees_leave_valid_requests_exact(dev, num_splits):
    """Requests 1 (a self parent), 3 (a parent below -1) and 4 (a negative
    prefix) are bad; 0, 2 and 5 keep the oracle's outputs."""
    rng = W.rng_for(23, 0)
    trees = [W.best_first_tree(40, rng), W.chain(9), W.best_first_tree(70, rng),
             W.random_tree(30, 5, rng), W.chain(4), W.best_first_tree(64, rng)]
    w = small("bad-trees", [300, 64, 1000, 17, 80, 129], trees, seed=23)
    o_ref, l_ref = oracle.tree_attn_workload(w)
    off = w.tree_off.numpy()
    parent = w.parent.numpy().copy()
    parent[off[1] + 5] = 5
    parent[off[3] + 7] = -2
    prefix = w.prefix_len.numpy().copy()
    prefix[4] = -1
    plan, out, lse = run(w, dev, num_splits=num_splits, parent=parent, prefix_len=prefix)
    check_plan(plan, parent, off, prefix, w.max_tree, "bad trees")
    assert plan.status.cpu().tolist() == [0, 6, 0, 8, -2, 0]
    ok = np.zeros(w.N, bool)
    for b in (0, 2, 5):
        ok[off[b]:off[b + 1]] = True
    ok_t = torch.from_numpy(ok)
    o_ref = torch.as_tensor(o_ref).reshape(out.shape)[ok_t]
    l_ref = torch.as_tensor(l_ref).reshape(lse.shape)[ok_t]
    assert_close(w, out[ok_t], lse[ok_t], o_ref, l_ref, "valid requests beside bad ones")


def test_bad_offsets_and_empty_trees(dev):
    # request 0's tree is larger than max_tree; request 1 is fine
    w = small("bad-offsets", [20, 40], [W.chain(2), W.chain(2)], seed=3)
    plan, _, _ = run(w, dev, parent=[-1, 0, 1, -1], tree_off=[0, 3, 4])
    assert plan.status.cpu().tolist() == [-1, 0]
    # empty trees beside a non-empty one still get their status
    w = small("empty-trees", [10, 30, 5], [np.zeros(0, np.int32), W.chain(3), np.zeros(0, np.int32)],
              seed=4)
    for ns in (1, 3):
        plan, out, lse = run(w, dev, num_splits=ns)
        check_plan(plan, w.parent, w.tree_off, w.prefix_len, w.max_tree, f"empty trees splits={ns}")
        o_ref, l_ref = oracle.tree_attn_workload(w)
        assert_close(w, out, lse, o_ref, l_ref, f"empty trees splits={ns}")


@pytest.mark.parametrize("name", ["chain16", "tree256"])
def test_equals_plan_then_fwd(dev, name):
    w = W.make_config(name)
    wd = w.to(dev)
    say(f"plan_fwd vs plan + fwd {name}")
    res = ta.plan(wd.parent, wd.tree_off, wd.prefix_len, max_tree=w.max_tree)
    o2, l2 = ta.fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table, wd.prefix_len,
                    wd.tree_off, res.anc_mask, max_tree=w.max_tree, max_prefix=w.max_prefix)
    plan, o1, l1 = ta.plan_fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                               wd.prefix_len, wd.tree_off, wd.parent, max_tree=w.max_tree,
                               max_prefix=w.max_prefix)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(plan, res):
        assert torch.equal(a, b)
    # the two stages of the call give the same result
    call = ta.prepare_plan_fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                               wd.prefix_len, wd.tree_off, wd.parent, max_tree=w.max_tree,
                               max_prefix=w.max_prefix)
    call.partial().merge()
    torch.cuda.synchronize()
    assert torch.equal(call.out, o1) and torch.equal(call.lse, l1)
    for a, b in zip(call.plan, res):
        assert torch.equal(a, b)


def test_graph_replay(dev):
    """The call captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, gives the eager result."""
    w = W.make_config("chain16")
    wd = w.to(dev)
    call = ta.prepare_plan_fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                               wd.prefix_len, wd.tree_off, wd.parent, max_tree=w.max_tree,
                               max_prefix=w.max_prefix)
    call.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (call.out, call.lse) + tuple(call.plan)]
    say("plan_fwd graph capture")
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call.run()
    torch.cuda.synchronize()
    for i in range(3):
        for t in (call.out, call.lse) + tuple(call.plan):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [call.out, call.lse] + list(call.plan)
        say(f"  replay {i}")
        for a, b in zip(got, ref):
            assert torch.equal(a, b)

"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Bars (written here, from the required tolerances): bf16 inputs -- max abs
error <= 1e-2 and mean abs error <= 1e-3 on both ``out`` and ``lse``; fp32
inputs -- both <= 1e-4.  Plan outputs are integers and must match exactly.
The page pool's spare pages, tail slots and unused table entries hold NaN, so
any read of a key that is not visible poisons the output and fails the test.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_masked_attention_plan_amd as ta
from tree_masked_attention_plan_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (1e-2, 1e-3), torch.float32: (1e-4, 1e-4)}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    ta.load_library()
    return torch.device("cuda:0")


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def gpu_plan(w, dev):
    wd_parent = w.parent.to(dev)
    res = ta.plan(wd_parent, w.tree_off.to(dev), w.prefix_len.to(dev), max_tree=w.max_tree)
    torch.cuda.synchronize()
    return res


def gpu_fwd(w, dev, num_splits=0, scale=None, stream=None):
    say(f"fwd {w.name}: B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} ps={w.page_size} "
        f"dtype={w.dtype} max_prefix={w.max_prefix} max_tree={w.max_tree} splits={num_splits}")
    wd = w.to(dev)
    res = ta.plan(wd.parent, wd.tree_off, wd.prefix_len, max_tree=w.max_tree, stream=stream)
    ta.check_status(res.status)
    out, lse = ta.fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                      wd.prefix_len, wd.tree_off, res.anc_mask, max_tree=w.max_tree,
                      max_prefix=w.max_prefix, scale=scale, num_splits=num_splits, stream=stream)
    torch.cuda.synchronize()
    return out.float().cpu().double(), lse.cpu().double()


def bf16_round(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.float32).to(torch.bfloat16).double()


def bf16_ulp(x: torch.Tensor) -> torch.Tensor:
    """Spacing of bf16 values (8 significant bits) at |x|."""
    e = torch.floor(torch.log2(x.abs().clamp_min(2.0 ** -126)))
    return torch.pow(2.0, e - 7)


def assert_close(w, out, lse, o_ref, l_ref, what="", raw=False):
    """Compare with the oracle.

    fp32: max and mean abs error <= 1e-4 against the exact result.
    bf16: ``out`` is compared with the exact result rounded to bf16 (the
    closest value the output can hold); the max bar is 1e-2, widened to one
    bf16 step of the exact value where that step is larger (|O| >= 2, only on
    rows with a handful of visible keys), and the mean bar is 1e-3.  ``lse``
    (fp32) always meets 1e-2 / 1e-3.  ``raw=True`` additionally requires the
    plain bars against the unrounded exact result, as on the five named
    workloads."""
    tmax, tmean = TOL[w.dtype]
    o_ref = torch.as_tensor(o_ref).reshape(out.shape).double()
    l_ref = torch.as_tensor(l_ref).reshape(lse.shape).double()
    assert torch.isfinite(out).all(), f"{what}: non-finite output"
    assert torch.isfinite(lse).all(), f"{what}: non-finite lse"
    el = (lse - l_ref).abs()
    eo_raw = (out - o_ref).abs()
    if w.dtype == torch.bfloat16:
        eo = (out - bf16_round(o_ref)).abs()
        bound = torch.clamp(bf16_ulp(o_ref), min=tmax)
    else:
        eo = eo_raw
        bound = torch.full_like(eo, tmax)
    say(f"  {what}: out max {eo.max():.3e} mean {eo.mean():.3e} (raw max {eo_raw.max():.3e} "
        f"mean {eo_raw.mean():.3e}) | lse max {el.max():.3e} mean {el.mean():.3e}")
    assert (eo <= bound).all() and eo.mean() <= tmean, \
        f"{what}: out err max {eo.max()} (bound {bound.flatten()[eo.argmax()]}) mean {eo.mean()}"
    assert el.max() <= tmax and el.mean() <= tmean, f"{what}: lse err max {el.max()} mean {el.mean()}"
    if raw:
        assert eo_raw.max() <= tmax and eo_raw.mean() <= tmean, \
            f"{what}: raw out err max {eo_raw.max()} mean {eo_raw.mean()}"


# ------------------------------------------------------------------- plan

def _forest_batch():
    rng = W.rng_for(41, 0)
    trees = [W.best_first_tree(256, rng), W.chain(64), W.chain(65), W.random_tree(100, 12, rng),
             np.array([-1, -1, 0, 1, 2, -1], np.int32), W.chain(1),
             W.best_first_tree(200, rng, per_node_logits=True), W.chain(256)]
    return W.make_workload("forests", [0, 5, 16, 300, 1, 64, 9, 2048], trees, 8, 2, 64,
                           torch.bfloat16, 41)


@pytest.mark.parametrize("name", W.CONFIG_NAMES + ("forests",))
def test_plan_bit_exact(dev, name):
    w = _forest_batch() if name == "forests" else W.make_config(name)
    say(f"plan {name}: B={w.B} N={w.N}")
    res = gpu_plan(w, dev)
    m, d, p, s = oracle.plan(w.parent, w.tree_off, w.prefix_len, w.max_tree)
    assert res.status.cpu().numpy().tolist() == s.tolist() == [0] * w.B
    assert np.array_equal(res.anc_mask.cpu().numpy().view(np.uint64), m)
    assert np.array_equal(res.depth.cpu().numpy(), d)
    assert np.array_equal(res.pos_id.cpu().numpy(), p)


def test_plan_error_statuses(dev):
    parent = np.array([-1, 0, -1, 0, 2, -1, -2, 0, 0, -1, -1, 0, 1], np.int32)
    off = np.array([0, 2, 5, 8, 10, 13], np.int32)
    L = np.array([4, 4, 4, -1, 0], np.int32)
    say("plan error statuses")
    res = ta.plan(torch.from_numpy(parent).to(dev), torch.from_numpy(off).to(dev),
                  torch.from_numpy(L).to(dev), max_tree=3)
    torch.cuda.synchronize()
    _, _, _, s = oracle.plan(parent, off, L, 3)
    assert res.status.cpu().numpy().tolist() == s.tolist() == [0, 3, 2, -2, 0]
    with pytest.raises(ta.TreeAttnError):
        ta.check_status(res.status)
    # a tree larger than max_tree (N itself is within B * max_tree), and
    # offsets that do not end at N
    par = torch.tensor([-1, 0, 1, -1], dtype=torch.int32, device=dev)
    res = ta.plan(par, torch.tensor([0, 3, 4], dtype=torch.int32, device=dev),
                  torch.tensor([0, 0], dtype=torch.int32, device=dev), max_tree=2)
    torch.cuda.synchronize()
    assert res.status.cpu().tolist() == [-1, 0]
    res = ta.plan(par, torch.tensor([0, 1, 3], dtype=torch.int32, device=dev),
                  torch.tensor([0, 0], dtype=torch.int32, device=dev), max_tree=3)
    torch.cuda.synchronize()
    assert res.status.cpu().tolist() == [0, -1]


# ------------------------------------------------------------- forward

def small(name, prefix, trees, Hq=8, Hkv=2, D=128, dtype=torch.bfloat16, ps=16, seed=0):
    return W.make_workload(name, prefix, trees, Hq, Hkv, D, dtype, seed, page_size=ps)


def small_cases():
    rng = W.rng_for(5, 0)
    cases = [
        ("chain-L0", [0], [W.chain(16)], {}),
        ("single-node", [1], [W.chain(1)], {}),
        ("ragged-prefix", [77], [W.best_first_tree(37, rng)], {}),
        ("multi-request", [0, 15, 300, 1000],
         [W.chain(5), W.best_first_tree(64, rng), W.best_first_tree(65, rng), W.random_tree(130, 9, rng)], {}),
        ("empty-tree-in-batch", [100, 40, 0], [W.chain(3), np.zeros(0, np.int32), W.chain(2)], {}),
        ("tree256-short-prefix", [33], [W.best_first_tree(256, rng)], {}),
        ("gqa1", [200], [W.best_first_tree(40, rng)], dict(Hq=4, Hkv=4)),
        ("gqa8", [129], [W.best_first_tree(50, rng)], dict(Hq=16, Hkv=2)),
        ("gqa5", [64], [W.random_tree(23, 6, rng)], dict(Hq=10, Hkv=2)),
        ("d64", [311], [W.best_first_tree(90, rng)], dict(D=64)),
        ("page1", [150], [W.best_first_tree(20, rng)], dict(ps=1)),
        ("page64", [1000], [W.best_first_tree(40, rng)], dict(ps=64)),
        ("forest-rows", [17], [np.array([-1, -1, -1, 0, 1, 2, 3, -1], np.int32)], dict(Hq=2, Hkv=1)),
        ("fp32-d64", [128], [W.random_tree(16, 8, rng)], dict(Hq=4, Hkv=1, D=64, dtype=torch.float32)),
        ("fp32-d128", [45, 0], [W.best_first_tree(70, rng), W.chain(3)],
         dict(Hq=8, Hkv=2, D=128, dtype=torch.float32)),
        ("fp32-page4", [99], [W.best_first_tree(33, rng)], dict(D=64, dtype=torch.float32, ps=4)),
        # enough (request, kv head, 128-row) units for the 4-wave workgroups
        ("wide-batch", [int(x) for x in rng.integers(1, 400, 16)],
         [W.best_first_tree(64, rng) for _ in range(16)], dict(Hq=32, Hkv=8)),
        # at least 4096 (node, head) rows: the merge takes lanes per row for
        # up to 16 splits (head_dim 64: 8 lanes per row)
        ("many-rows-d64", [900, 2100], [W.best_first_tree(128, rng), W.best_first_tree(100, rng)],
         dict(Hq=32, Hkv=8, D=64)),
        # the largest page size: a 64-key block inside one page, three pages
        # for the longest prefix
        ("page1024", [3000, 500], [W.best_first_tree(30, rng), W.chain(8)], dict(ps=1024)),
        ("page256-d64", [700, 1], [W.random_tree(50, 10, rng), W.chain(2)], dict(ps=256, D=64)),
        ("fp32-page1024", [1500], [W.best_first_tree(20, rng)], dict(dtype=torch.float32, ps=1024)),
        # many small requests: hundreds of work units of one row tile each
        ("many-small-requests", [int(x) for x in rng.integers(0, 41, 300)],
         [W.random_tree(int(t), 3, rng) for t in rng.integers(1, 5, 300)], {}),
        # <= 32 rows per kv head with long prefixes: one row tile, so a wave's
        # copy rows of a full prefix block span two 16-row page groups
        # (head_dim 128: four key slices; head_dim 64: two)
        ("few-rows-long-prefix", [1000, 613], [W.chain(5), W.best_first_tree(7, rng)], {}),
        ("d64-few-rows-long-prefix", [1500], [W.chain(6)], dict(D=64)),
        # pages of 32 tokens: two 16-row groups per page
        ("page32-long-prefix", [2000, 77], [W.best_first_tree(64, rng), W.chain(4)], dict(ps=32)),
        # 8-wave units (more than 128 rows per kv head) that fill the GPU
        # without splits, over prefixes of at least 1024 keys: four K/V
        # stages, copies three steps ahead; ragged prefixes and tree blocks
        # make the last steps issue fewer copies
        ("four-stages", [int(x) for x in rng.integers(1024, 1401, 32)],
         [W.best_first_tree(int(t), rng) for t in rng.integers(129, 201, 32)], dict(Hq=8, Hkv=8)),
        # the same with units of 0 to 4 steps beside long ones, and pages of
        # 8 tokens (page ids loaded per lane)
        ("four-stages-short-units", [0, 5, 70, 130, 200, 1100] + [int(x) for x in rng.integers(0, 1500, 26)],
         [W.best_first_tree(int(t), rng) for t in rng.integers(129, 257, 32)], dict(Hq=8, Hkv=8, ps=8)),
        ("four-stages-page256", [int(x) for x in rng.integers(900, 1300, 32)],
         [W.random_tree(int(t), 12, rng) for t in rng.integers(129, 180, 32)], dict(Hq=8, Hkv=8, ps=256)),
        # one request of 8-wave units with a prefix of at least 4096 keys: the
        # tree rides with the last prefix chunk (8 keys of prefix, then the
        # tree's two blocks) instead of taking a slot of its own
        ("tree-rides-long-prefix", [5000], [W.best_first_tree(100, rng)], {}),
    ]
    return cases


CASES = small_cases()


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_fwd_small_cases(dev, idx):
    name, prefix, trees, kw = CASES[idx]
    w = small(name, prefix, trees, seed=100 + idx, **kw)
    o_ref, l_ref = oracle.tree_attn_workload(w)
    splits = (0, 1, 3, 12, 64) if w.dtype == torch.bfloat16 and w.max_prefix > 0 else (0,)
    for ns in splits:
        out, lse = gpu_fwd(w, dev, num_splits=ns)
        assert_close(w, out, lse, o_ref, l_ref, f"{name} splits={ns}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_large_and_jumping_scores(dev, dtype):
    """Scores with a wide range whose running max jumps by far more than the
    lazy-rescale slack from block to block: Q scaled by 4 and every physical
    page's keys by its own factor in [0.1, 4] (the block table scatters
    pages, so the magnitude jumps along each prefix and between splits)."""
    rng = W.rng_for(21, 0)
    w = small("rescale", [700, 129, 64], [W.best_first_tree(64, rng), W.chain(20), W.random_tree(30, 5, rng)],
              D=64 if dtype == torch.float32 else 128, dtype=dtype, seed=21)
    g = torch.Generator().manual_seed(21)
    fac = (0.1 + 3.9 * torch.rand(w.k_cache.shape[0], generator=g)).view(-1, 1, 1, 1)
    w.k_cache = (w.k_cache.float() * fac).to(dtype)    # sentinel NaN slots stay NaN
    w.k_tree = (w.k_tree.float() * 2.5).to(dtype)
    w.q = (w.q.float() * 4.0).to(dtype)
    o_ref, l_ref = oracle.tree_attn_workload(w)
    splits = (0, 1, 5, 64) if dtype == torch.bfloat16 else (0,)
    for ns in splits:
        out, lse = gpu_fwd(w, dev, num_splits=ns)
        assert_close(w, out, lse, o_ref, l_ref, f"rescale {dtype} splits={ns}")


@pytest.mark.parametrize("rows", ["few", "many"])
@pytest.mark.parametrize("log2_scale", [13, 17, 60, -60])
def test_large_values_through_fp16_partials(dev, log2_scale, rows):
    """Split calls keep each split's normalised partial output in fp16, each
    row scaled by a power of two so that its largest magnitude is in [2^14,
    2^15).  V scaled by 2^13 (|V| up to about 4e4), 2^17 (about 6e5, beyond
    the fp16 range), 2^60 (about 1e19) and 2^-60 (below the smallest fp16
    subnormal) -- all exact in bf16 -- must still match the oracle through
    splits 5, 12, 17 and 64, compared in units of the scale; with few rows
    (one wave per row in the merge) and with many (lanes per row up to 16
    splits)."""
    rng = W.rng_for(23, 0)
    if rows == "few":
        w = small("large-v", [1500, 300], [W.chain(16), W.best_first_tree(40, rng)], seed=23)
    else:
        w = small("large-v-rows", [1500, 300], [W.best_first_tree(100, rng), W.best_first_tree(60, rng)],
                  Hq=32, Hkv=8, seed=23)
        assert w.N * w.Hq >= 4096
    scale = 2.0 ** log2_scale
    w.v_cache = (w.v_cache.float() * scale).to(torch.bfloat16)    # sentinel NaN slots stay NaN
    w.v_tree = (w.v_tree.float() * scale).to(torch.bfloat16)
    vmax = max(torch.nan_to_num(w.v_cache.float()).abs().max().item(), w.v_tree.float().abs().max().item())
    assert 2.0 ** (log2_scale + 1) < vmax < 2.0 ** (log2_scale + 4)
    o_ref, l_ref = oracle.tree_attn_workload(w)
    for ns in (0, 5, 12, 17, 64):
        out, lse = gpu_fwd(w, dev, num_splits=ns)
        assert_close(w, out / scale, lse, np.asarray(o_ref) / scale, l_ref,
                     f"V * 2^{log2_scale} splits={ns}")


def random_config(i):
    """A seeded random shape: batch, tree kinds and sizes, prefix lengths,
    GQA ratio, head dim, page size, dtype and a forced split count, sized so
    that the oracle finishes in about a second."""
    rng = np.random.default_rng(5000 + i)
    B = int(rng.integers(1, 7))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 5, 8]))
    D = int(rng.choice([64, 128]))
    ps = int(rng.choice([1, 4, 16, 32, 64, 256, 1024]))
    dtype = torch.float32 if rng.random() < 0.2 else torch.bfloat16
    trees, prefix = [], []
    for _ in range(B):
        T = int(rng.integers(0, 257)) if rng.random() < 0.3 else int(rng.integers(1, 65))
        kind = rng.integers(0, 3) if T > 0 else 0
        trees.append(W.chain(T) if kind == 0 else
                     (W.random_tree(T, int(rng.integers(2, 17)), rng) if kind == 1 else W.best_first_tree(T, rng)))
        prefix.append(int(rng.integers(0, 3000)) if rng.random() < 0.85 else 0)
    splits = int(rng.choice([0, 0, 1, 2, 7, 64])) if dtype == torch.bfloat16 else 0
    return f"random-{i}", prefix, trees, dict(Hq=G * Hkv, Hkv=Hkv, D=D, dtype=dtype, ps=ps), splits


@pytest.mark.parametrize("i", range(200))
def test_random_configurations(dev, i):
    name, prefix, trees, kw, splits = random_config(i)
    w = small(name, prefix, trees, seed=700 + i, **kw)
    o_ref, l_ref = oracle.tree_attn_workload(w)
    out, lse = gpu_fwd(w, dev, num_splits=splits)
    assert_close(w, out, lse, o_ref, l_ref, f"{name} splits={splits}")


def test_invisible_tree_keys_get_exact_zero_weight(dev):
    """A tree node's K and V reach only its own rows and its descendants'
    (JetFlow technical summary, section 2, the tree-causal mask).  Giving a
    leaf huge but finite K and V (V = 1e30) must leave every other row's
    output and LSE bit-identical, with and without splits: inside a computed
    tile an invisible key's weight is an exact zero.  The leaf's own rows
    still meet the per-element bar against the oracle (one bf16 step of the
    exact value, or 1e-2)."""
    import dataclasses
    rng = W.rng_for(21, 0)
    w = small("invisible-huge", [300, 1000], [W.best_first_tree(100, rng), W.best_first_tree(64, rng)],
              Hq=8, Hkv=2, seed=21)
    par = w.parent.numpy()[:100]
    has_child = np.zeros(100, bool)
    has_child[par[par >= 0]] = True
    leaves = [j for j in range(100) if not has_child[j] and j % 64 not in (0, 63)]
    j = leaves[len(leaves) // 2]
    w2 = dataclasses.replace(w, k_tree=w.k_tree.clone(), v_tree=w.v_tree.clone())
    w2.k_tree[j] = (w.k_tree[j].float() * 40).to(w.k_tree.dtype)
    w2.v_tree[j] = torch.full_like(w.v_tree[j], 1e30)
    others = torch.ones(w.N, dtype=torch.bool)
    others[j] = False
    o_ref, l_ref = oracle.tree_attn_workload(w2)
    o_ref = torch.as_tensor(o_ref).reshape(w.N, w.Hq, w.D).double()
    l_ref = torch.as_tensor(l_ref).reshape(w.N, w.Hq).double()
    for ns in (0, 1, 5):
        o1, l1 = gpu_fwd(w, dev, num_splits=ns)
        o2, l2 = gpu_fwd(w2, dev, num_splits=ns)
        say(f"  leaf {j}: splits {ns}, leaf rows max |O| {o2[j].abs().max():.3e}")
        assert torch.equal(o1[others], o2[others]) and torch.equal(l1[others], l2[others]), \
            f"splits={ns}: rows that cannot see node {j} changed"
        assert torch.isfinite(o2[j]).all()
        eo = (o2[j] - bf16_round(o_ref[j])).abs()
        assert (eo <= torch.clamp(bf16_ulp(o_ref[j]), min=1e-2)).all(), f"splits={ns}: leaf rows {eo.max()}"
        assert (l2[j] - l_ref[j]).abs().max() <= 1e-2, f"splits={ns}: leaf lse"


def test_softmax_scale_override(dev):
    rng = W.rng_for(8, 0)
    w = small("scale", [90], [W.best_first_tree(30, rng)], seed=8)
    o_ref, l_ref = oracle.tree_attn_workload(w, scale=0.05)
    out, lse = gpu_fwd(w, dev, scale=0.05)
    assert_close(w, out, lse, o_ref, l_ref, "scale=0.05")


def test_relabelled_tree_permutes_outputs(dev):
    rng = W.rng_for(12, 0)
    par = W.best_first_tree(120, rng)
    newp, sigma = W.topo_relabel(par, rng)
    w1 = small("relabel-a", [500], [par], seed=12)
    w2 = small("relabel-b", [500], [newp], seed=12)
    inv = torch.from_numpy(np.argsort(sigma))
    w2.q, w2.k_tree, w2.v_tree = w1.q[inv], w1.k_tree[inv], w1.v_tree[inv]
    o1, l1 = gpu_fwd(w1, dev)
    o2, l2 = gpu_fwd(w2, dev)
    sig = torch.from_numpy(sigma)
    assert (o2[sig] - o1).abs().max() <= 1e-2
    assert (l2[sig] - l1).abs().max() <= 1e-3


def test_non_default_stream_and_determinism(dev):
    rng = W.rng_for(13, 0)
    w = small("stream", [700, 33], [W.best_first_tree(80, rng), W.chain(9)], seed=13)
    s = torch.cuda.Stream(dev)
    with torch.cuda.stream(s):
        o1, l1 = gpu_fwd(w, dev, stream=s)
    o2, l2 = gpu_fwd(w, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_concurrent_host_threads(dev):
    """The library keeps no state, so calls are reentrant: two host threads,
    each on its own stream with its own workload and split workspace, issue
    calls at the same time; every result equals the same call made alone,
    bit for bit."""
    import threading
    rng = W.rng_for(17, 0)
    ws = [small("threads-a", [1800, 60], [W.chain(16), W.best_first_tree(50, rng)], seed=17),
          small("threads-b", [900], [W.best_first_tree(120, rng)], D=64, seed=18)]
    ref = []
    for w in ws:
        o, l = gpu_fwd(w, dev, num_splits=5)
        torch.cuda.synchronize()
        ref.append((o.clone(), l.clone()))
    wds = [w.to(dev) for w in ws]
    plans = [ta.plan(wd.parent, wd.tree_off, wd.prefix_len, max_tree=w.max_tree) for w, wd in zip(ws, wds)]
    torch.cuda.synchronize()
    results = [[None] * 8 for _ in ws]
    errors = []
    start = threading.Barrier(len(ws))

    def worker(i):
        try:
            w, wd, res = ws[i], wds[i], plans[i]
            st = torch.cuda.Stream(dev)
            start.wait()
            with torch.cuda.stream(st):
                for r in range(8):
                    results[i][r] = ta.fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                                           wd.prefix_len, wd.tree_off, res.anc_mask, max_tree=w.max_tree,
                                           max_prefix=w.max_prefix, num_splits=5, stream=st)
            st.synchronize()
        except Exception as e:   # reported below, on the test's thread
            errors.append(e)

    say("two host threads, one stream each, 8 calls each")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(ws))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for i, (o_ref, l_ref) in enumerate(ref):
        for o, l in results[i]:
            assert torch.equal(o.float().cpu().double(), o_ref) and torch.equal(l.cpu().double(), l_ref)


def test_side_stream_keeps_workspace_alive(dev):
    """A forward call enqueued on a side stream from outside that stream's
    context, with the library-allocated split workspace: once the call
    returns, the workspace's memory must not be handed to an allocation on
    the current stream before the side stream has passed the call, and the
    results must match the oracle.  The side stream is held busy first
    (a bounded spin kernel), so the attention has not run when the
    allocation and the fill on the current stream happen."""
    rng = W.rng_for(15, 0)
    w = small("side-stream", [1500, 90], [W.chain(16), W.best_first_tree(40, rng)], seed=15)
    o_ref, l_ref = oracle.tree_attn_workload(w)
    wd = w.to(dev)
    res = ta.plan(wd.parent, wd.tree_off, wd.prefix_len, max_tree=w.max_tree)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    say("side stream: forced 9 splits, workspace allocated by the binding")
    if hasattr(torch.cuda, "_sleep"):
        with torch.cuda.stream(s):
            torch.cuda._sleep(20_000_000)
    call = ta.prepare_fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                          wd.prefix_len, wd.tree_off, res.anc_mask, max_tree=w.max_tree,
                          max_prefix=w.max_prefix, num_splits=9)
    assert call.workspace is not None
    call.run(stream=s)
    ws_ptr, ws_n = call.workspace.data_ptr(), call.workspace.numel()
    out, lse = call.out, call.lse
    del call
    junk = torch.full((ws_n,), 0xFF, dtype=torch.uint8, device=dev)   # NaN bytes for fp16 / fp32
    assert junk.data_ptr() != ws_ptr, "the workspace was reused while the side stream still needs it"
    torch.cuda.synchronize()
    assert_close(w, out.float().cpu().double(), lse.cpu().double(), o_ref, l_ref, "side stream")


def test_partial_then_merge_equals_fwd(dev):
    rng = W.rng_for(14, 0)
    w = small("stages", [900, 64], [W.best_first_tree(100, rng), W.chain(12)], seed=14)
    wd = w.to(dev)
    res = ta.plan(wd.parent, wd.tree_off, wd.prefix_len, max_tree=w.max_tree)
    for ns in (1, 5):
        say(f"stages splits={ns}")
        call = ta.prepare_fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                              wd.prefix_len, wd.tree_off, res.anc_mask, max_tree=w.max_tree,
                              max_prefix=w.max_prefix, num_splits=ns)
        call.run()
        torch.cuda.synchronize()
        o1, l1 = call.out.clone(), call.lse.clone()
        call.out.zero_()
        call.lse.zero_()
        call.partial().merge()
        torch.cuda.synchronize()
        assert torch.equal(o1, call.out) and torch.equal(l1, call.lse)


def test_one_workspace_across_split_counts(dev):
    """One caller-owned workspace, filled with NaN bytes (fp16 and fp32) before
    the first call, serves calls whose split counts and shapes go down and up
    again.  Slots a call does not write keep what an earlier call, or the
    fill, left there; the merge must read only what the current call wrote
    (partial rows of zero-weight slots are excluded by a select, not a
    multiplication)."""
    rng = W.rng_for(33, 0)
    wa = small("ws-a", [900, 300, 0], [W.best_first_tree(40, rng), W.chain(7), W.chain(3)], seed=33)
    wb = small("ws-b", [250], [W.random_tree(30, 5, rng)], seed=34)
    refs = {w.name: oracle.tree_attn_workload(w) for w in (wa, wb)}
    dws = {w.name: w.to(dev) for w in (wa, wb)}
    plans = {}
    for w in (wa, wb):
        wd = dws[w.name]
        plans[w.name] = ta.plan(wd.parent, wd.tree_off, wd.prefix_len, max_tree=w.max_tree).anc_mask
    need = max(ta.workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.max_tree, w.max_prefix, num_splits=ns)
               for w in (wa, wb) for ns in (3, 5, 12))
    ws = torch.full((need + 256,), 0xFF, dtype=torch.uint8, device=dev)
    for w, ns in ((wa, 12), (wb, 3), (wa, 5), (wb, 12), (wa, 3)):
        say(f"shared workspace: {w.name} splits={ns}")
        wd = dws[w.name]
        out, lse = ta.fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                          wd.prefix_len, wd.tree_off, plans[w.name], max_tree=w.max_tree,
                          max_prefix=w.max_prefix, num_splits=ns, workspace=ws)
        torch.cuda.synchronize()
        o_ref, l_ref = refs[w.name]
        assert_close(w, out.float().cpu().double(), lse.cpu().double(), o_ref, l_ref,
                     f"{w.name} splits={ns}, shared workspace")


def test_empty_batch_is_noop(dev):
    say("empty batch")
    e = torch.zeros(0, dtype=torch.int32, device=dev)
    res = ta.plan(e, torch.zeros(1, dtype=torch.int32, device=dev), e, max_tree=0)
    assert res.anc_mask.shape == (0, 4)
    w = small("empty", [10, 20], [np.zeros(0, np.int32), np.zeros(0, np.int32)])
    wd = w.to(dev)
    out, lse = ta.fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                      wd.prefix_len, wd.tree_off, torch.zeros((0, 4), dtype=torch.int64, device=dev),
                      max_tree=0, max_prefix=20)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 128) and lse.shape == (0, 8)


# ------------------------------------------------- the five named workloads

@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_named_workload(dev, name, named_reference):
    """Every (node, head) row of each named workload against the oracle."""
    w, o_ref, l_ref = named_reference(name)
    out, lse = gpu_fwd(w, dev)
    assert_close(w, out, lse, o_ref, l_ref, f"{name} (all {w.N * w.Hq} rows)", raw=True)

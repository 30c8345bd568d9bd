"""GPU parity of tree_attn_build_tree against the oracle's sequential
best-first expansion: parent ids and candidate choices must be identical and
scores bit-identical (both sides add the same fp32 values in the same
order), including exact ties, zero-probability candidates, NaN
candidates (never chosen; nodes beyond the finite candidates are missing)
and budgets up to the implicit tree's size."""
import numpy as np
import pytest
import torch

import oracle
import tree_masked_attention_plan_amd as ta
from tree_masked_attention_plan_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP device")
    ta.load_library()
    return torch.device("cuda:0")


def logsoftmax(z):
    return torch.log_softmax(torch.as_tensor(z, dtype=torch.float64), dim=-1).float().numpy()


def check(lp, T, dev, what):
    p_ref, c_ref, s_ref = oracle.build_tree(lp, T)
    p, c, s = ta.build_tree(torch.from_numpy(np.ascontiguousarray(lp)).to(dev), T)
    torch.cuda.synchronize()
    p, c, s = p.cpu().numpy(), c.cpu().numpy(), s.cpu().numpy()
    say(f"  {what}: B={lp.shape[0]} depth={lp.shape[1]} K={lp.shape[2]} T={T}")
    assert np.array_equal(p, p_ref), f"{what}: parents differ at {np.argwhere(p != p_ref)[:4].tolist()}"
    assert np.array_equal(c, c_ref), f"{what}: choices differ"
    nan = np.isnan(s_ref)
    assert np.array_equal(np.isnan(s), nan), f"{what}: missing nodes differ"
    assert np.array_equal(s[~nan].view(np.int32), s_ref[~nan].view(np.int32)), f"{what}: scores differ"


@pytest.mark.parametrize("K,Dmax,T", [(8, 16, 256), (8, 16, 16), (2, 16, 200), (3, 4, 120), (16, 8, 256),
                                      (64, 4, 256), (8, 1, 8), (1, 64, 64),
                                      # the limits: K * max_depth = 4096, K * (T + 1) = 16448
                                      (64, 64, 256), (16, 64, 256)])
def test_random_candidates(dev, K, Dmax, T):
    rng = np.random.default_rng(K * 1000 + Dmax * 10 + T)
    lp = logsoftmax(rng.normal(0, 2, size=(6, Dmax, K)))
    check(lp, T, dev, "random")


def test_many_requests(dev):
    """300 requests in one launch (one workgroup each)."""
    rng = np.random.default_rng(31)
    lp = logsoftmax(rng.normal(0, 2, size=(300, 16, 8)))
    check(lp, 64, dev, "many requests")


def test_ties_give_breadth_first_order(dev):
    for K in (2, 3, 8):
        lp = np.full((3, 16, K), np.float32(np.log(np.float32(1.0 / K))), dtype=np.float32)
        check(lp, 200 if K > 2 else 120, dev, f"ties K={K}")


def test_zero_probability_candidates(dev):
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2, size=(4, 16, 8))
    z[:, :, 5:] = -np.inf            # three candidates with probability 0 at every depth
    lp = logsoftmax(z)
    check(lp, 256, dev, "zero-probability candidates")


def test_gpu_trees_feed_the_plan(dev):
    rng = np.random.default_rng(9)
    B, T = 4, 256
    lp = logsoftmax(rng.normal(0, 2, size=(B, 16, 8)))
    p, _, _ = ta.build_tree(torch.from_numpy(lp).to(dev), T)
    parent = p.flatten().contiguous()
    tree_off = torch.arange(0, (B + 1) * T, T, dtype=torch.int32, device=dev)
    prefix = torch.full((B,), 100, dtype=torch.int32, device=dev)
    res = ta.plan(parent, tree_off, prefix, max_tree=T)
    mask, depth, pos, st = oracle.plan(parent.cpu(), tree_off.cpu(), prefix.cpu(), max_tree=T)
    assert st.tolist() == [0] * B and res.status.cpu().tolist() == [0] * B
    assert np.array_equal(res.depth.cpu().numpy(), depth)
    assert int(depth.max()) <= 16


def test_nan_candidates_are_never_chosen(dev):
    """NaN log-probabilities are never popped.  With enough finite candidates
    left, the trees equal the oracle's on the same inputs with NaN replaced by
    -inf (every pop is then finite, and -inf candidates are never reached)."""
    rng = np.random.default_rng(17)
    lp = logsoftmax(rng.normal(0, 2, size=(4, 16, 8)))
    nan_at = rng.random(size=lp.shape) < 0.4
    nan_at[..., 0] = False                     # every depth keeps finite candidates
    lp_nan = np.where(nan_at, np.float32(np.nan), lp).astype(np.float32)
    lp_inf = np.where(nan_at, np.float32(-np.inf), lp).astype(np.float32)
    p_ref, c_ref, s_ref = oracle.build_tree(lp_inf, 256)
    assert np.isfinite(s_ref).all()
    p, c, s = ta.build_tree(torch.from_numpy(lp_nan).to(dev), 256)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), p_ref)
    assert np.array_equal(c.cpu().numpy(), c_ref)
    assert np.array_equal(s.cpu().numpy().view(np.int32), s_ref.view(np.int32))


@pytest.mark.parametrize("frac,K,Dmax,T", [(0.1, 8, 16, 256), (0.5, 8, 16, 256), (0.85, 8, 16, 256),
                                           (0.6, 3, 6, 120), (0.3, 1, 64, 64), (0.7, 64, 4, 256)])
def test_nan_candidates_against_the_oracle(dev, frac, K, Dmax, T):
    """NaN log-probabilities at random places, compared with the oracle run
    on the same inputs: the denser cases leave requests with fewer finite
    candidates than the budget, so missing nodes are covered too."""
    rng = np.random.default_rng(int(frac * 100) * 7 + K + Dmax + T)
    lp = logsoftmax(rng.normal(0, 2, size=(6, Dmax, K)))
    lp = np.where(rng.random(size=lp.shape) < frac, np.float32(np.nan), lp).astype(np.float32)
    check(lp, T, dev, f"NaN fraction {frac}")


def test_nan_candidates_can_leave_nodes_missing(dev):
    """One finite candidate per depth and three depths: a chain of three
    nodes, then no candidate is left; the rest are written as missing."""
    K, Dmax, T = 4, 3, 10
    lp = np.full((2, Dmax, K), np.float32(np.nan), dtype=np.float32)
    lp[0, :, 2] = np.float32(-0.5)
    lp[1, :, 0] = np.float32(-1.0)
    p, c, s = ta.build_tree(torch.from_numpy(lp).to(dev), T)
    torch.cuda.synchronize()
    p, c, s = p.cpu().numpy(), c.cpu().numpy(), s.cpu().numpy()
    assert p[:, :3].tolist() == [[-1, 0, 1], [-1, 0, 1]]
    assert c[:, :3].tolist() == [[2, 2, 2], [0, 0, 0]]
    np.testing.assert_array_equal(s[0, :3], np.float32([-0.5, -1.0, -1.5]))
    np.testing.assert_array_equal(s[1, :3], np.float32([-1.0, -2.0, -3.0]))
    assert (p[:, 3:] == -1).all() and (c[:, 3:] == -1).all() and np.isnan(s[:, 3:]).all()

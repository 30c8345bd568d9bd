"""GPU parity of tree_attn_build_tree against the oracle's sequential
best-first expansion: parent ids and candidate choices must be identical and
scores bit-identical (both sides add the same fp32 values in the same
order), including exact ties, zero-probability candidates and budgets up to
the implicit tree's size."""
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
    assert np.array_equal(s.view(np.int32), s_ref.view(np.int32)), f"{what}: scores differ"


@pytest.mark.parametrize("K,Dmax,T", [(8, 16, 256), (8, 16, 16), (2, 16, 200), (3, 4, 120), (16, 8, 256),
                                      (64, 4, 256), (8, 1, 8), (1, 64, 64)])
def test_random_candidates(dev, K, Dmax, T):
    rng = np.random.default_rng(K * 1000 + Dmax * 10 + T)
    lp = logsoftmax(rng.normal(0, 2, size=(6, Dmax, K)))
    check(lp, T, dev, "random")


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

"""GPU test of tree_attn_fwd_noalloc, the forward entry point that allocates
nothing (its split workspace is the library's fixed per-device array).

Two calls in a row through the C ABI, the second on a smaller input, each
compared with tree_attn_fwd on the same inputs (which uses a caller-owned
workspace): the kernels and the arithmetic are the same, so the outputs must
be equal bit for bit (a stricter bar than the oracle tolerances, which the
tree_attn_fwd outputs are checked against too).  A call that needs more
workspace than the array holds is refused before any launch.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_masked_attention_plan_amd as ta
from tree_masked_attention_plan_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (1e-2, 1e-3), torch.float32: (1e-4, 1e-4)}


def say(*a):
    print("[gpu]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP device")
    ta.load_library()
    return torch.device("cuda:0")


def both(w, dev, num_splits=0):
    """tree_attn_fwd and tree_attn_fwd_noalloc on the same inputs."""
    wd = w.to(dev)
    res = ta.plan(wd.parent, wd.tree_off, wd.prefix_len, max_tree=w.max_tree)
    ref_out, ref_lse = ta.fwd(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table,
                              wd.prefix_len, wd.tree_off, res.anc_mask, max_tree=w.max_tree,
                              max_prefix=w.max_prefix, num_splits=num_splits)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    ta.fwd_noalloc(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table, wd.prefix_len,
                   wd.tree_off, res.anc_mask, out=out, lse=lse, max_tree=w.max_tree,
                   max_prefix=w.max_prefix, num_splits=num_splits)
    torch.cuda.synchronize()
    ta.check_status(res.status)
    return ref_out, ref_lse, out, lse


def test_noalloc_matches_fwd_twice_second_smaller(dev):
    """tree256 (8 splits: about 17 MB of split workspace), then chain16 (17
    splits over 16 nodes: about 2 MB) on the same array."""
    for name in ("tree256", "chain16"):
        w = W.make_config(name)
        need = ta.workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.max_tree, w.max_prefix)
        say(f"noalloc {name}: N={w.N} workspace {need} bytes")
        assert 0 < need <= ta.NOALLOC_SCRATCH_BYTES
        ref_out, ref_lse, out, lse = both(w, dev)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), name
        assert torch.equal(lse, ref_lse), name
        # and the shared outputs meet the oracle bars
        o_ref, l_ref = oracle.tree_attn_workload(w)
        eo = np.abs(out.float().cpu().double().numpy() - o_ref)
        el = np.abs(lse.cpu().double().numpy() - l_ref)
        tmax, tmean = TOL[w.dtype]
        say(f"  {name}: out max {eo.max():.2e} mean {eo.mean():.2e}; lse max {el.max():.2e}")
        assert eo.max() <= tmax and eo.mean() <= tmean and el.max() <= tmax and el.mean() <= tmean


def test_noalloc_forced_splits_and_no_split(dev):
    """A forced split count (5) on a two-request batch, then a call with one
    split (no workspace at all), in a row."""
    rng = W.rng_for(31, 0)
    w = W.make_workload("noalloc-small", [1200, 77], [W.best_first_tree(60, rng), W.chain(9)], 8, 2, 128,
                        torch.bfloat16, 31)
    for ns in (5, 1):
        say(f"noalloc small batch splits={ns}")
        ref_out, ref_lse, out, lse = both(w, dev, num_splits=ns)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)


def test_noalloc_refuses_a_call_beyond_its_array(dev):
    """64 forced splits of a 256-node tree need about 135 MB of workspace:
    refused with TA_ERR_SCRATCH_LIMIT before anything is launched, and the
    outputs are left untouched."""
    w = W.make_config("tree256")
    need = ta.workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.max_tree, w.max_prefix, num_splits=64)
    assert need > ta.NOALLOC_SCRATCH_BYTES
    wd = w.to(dev)
    res = ta.plan(wd.parent, wd.tree_off, wd.prefix_len, max_tree=w.max_tree)
    out = torch.zeros((w.N, w.Hq, w.D), dtype=w.dtype, device=dev)
    lse = torch.zeros((w.N, w.Hq), dtype=torch.float32, device=dev)
    with pytest.raises(ta.TreeAttnError, match="status 6"):
        ta.fwd_noalloc(wd.q, wd.k_tree, wd.v_tree, wd.k_cache, wd.v_cache, wd.block_table, wd.prefix_len,
                       wd.tree_off, res.anc_mask, out=out, lse=lse, max_tree=w.max_tree,
                       max_prefix=w.max_prefix, num_splits=64)
    torch.cuda.synchronize()
    assert not out.float().abs().sum().item() and not lse.abs().sum().item()

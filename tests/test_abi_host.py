"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library is loaded and every function declared in include/tree_attn.h must
be exported; the argument checks of tree_attn_fwd / tree_attn_plan return
their documented codes before touching the device; the split choice and the
workspace size are pure functions with the documented properties.
"""
import ctypes
import os
import re
import subprocess

import pytest

import tree_masked_attention_plan_amd as ta
from tree_masked_attention_plan_amd import build as ta_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_attn.h")

TA_OK, TA_ERR_NULL_PTR, TA_ERR_BAD_SHAPE, TA_ERR_UNSUPPORTED, TA_ERR_WORKSPACE, TA_ERR_HIP, \
    TA_ERR_SCRATCH_LIMIT = range(7)
BF16, FP32 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ta.library_path()):
        ta_build.build()
    return ta.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tree_attn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("tree_attn_plan", "tree_attn_plan_dfs", "tree_attn_gather_rows", "tree_attn_fwd",
                     "tree_attn_plan_fwd",
                     "tree_attn_workspace_bytes",
                     "tree_attn_num_splits", "tree_attn_fwd_check", "tree_attn_status_str",
                     "tree_attn_abi_version", "tree_attn_fwd_noalloc"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ta.library_path()],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tree_attn_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "tree_attn.h"\nint main(void){return tree_attn_abi_version()==0;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I",
                    os.path.join(ROOT, "include"), str(src)], check=True)


def test_version_and_strings(lib):
    assert ta.abi_version() == 1
    for code in range(7):
        assert lib.tree_attn_status_str(code) != b"unknown status"
    assert lib.tree_attn_status_str(99) == b"unknown status"


FAKE = 0x10000   # a non-null, 256-byte aligned address that is never dereferenced


def fwd_args(**over):
    a = dict(q=FAKE, k_tree=FAKE, v_tree=FAKE, k_cache=FAKE, v_cache=FAKE, block_table=FAKE,
             prefix_len=FAKE, tree_off=FAKE, anc_mask=FAKE, B=1, N=16, Hq=32, Hkv=8, D=128,
             page_size=16, num_pages=141, max_pages=128, max_tree=16, max_prefix=2048, scale=0.0,
             dtype=BF16, num_splits=0, out=FAKE, lse=FAKE, workspace=FAKE, ws_bytes=1 << 30)
    a.update(over)
    return a


def check(lib, **over):
    a = fwd_args(**over)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.tree_attn_fwd_check(P(a["q"]), P(a["k_tree"]), P(a["v_tree"]), P(a["k_cache"]),
                                   P(a["v_cache"]), P(a["block_table"]), P(a["prefix_len"]),
                                   P(a["tree_off"]), P(a["anc_mask"]), a["B"], a["N"], a["Hq"],
                                   a["Hkv"], a["D"], a["page_size"], a["num_pages"], a["max_pages"],
                                   a["max_tree"], a["max_prefix"], a["scale"], a["dtype"],
                                   a["num_splits"], P(a["out"]), P(a["lse"]), P(a["workspace"]),
                                   a["ws_bytes"])


def call_fwd(lib, **over):
    a = fwd_args(**over)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.tree_attn_fwd(P(a["q"]), P(a["k_tree"]), P(a["v_tree"]), P(a["k_cache"]),
                             P(a["v_cache"]), P(a["block_table"]), P(a["prefix_len"]),
                             P(a["tree_off"]), P(a["anc_mask"]), a["B"], a["N"], a["Hq"], a["Hkv"],
                             a["D"], a["page_size"], a["num_pages"], a["max_pages"], a["max_tree"],
                             a["max_prefix"], a["scale"], a["dtype"], a["num_splits"], P(a["out"]),
                             P(a["lse"]), P(a["workspace"]), a["ws_bytes"], None)


def test_fwd_check_accepts_valid_arguments(lib):
    assert check(lib) == TA_OK
    assert check(lib, dtype=FP32, D=64, Hq=4, Hkv=1, workspace=None, ws_bytes=0) == TA_OK
    assert check(lib, page_size=1, max_pages=2048) == TA_OK
    assert check(lib, page_size=1024, max_pages=2) == TA_OK


@pytest.mark.parametrize("over,code", [
    (dict(dtype=7), TA_ERR_UNSUPPORTED),
    (dict(D=96), TA_ERR_UNSUPPORTED),
    (dict(D=256), TA_ERR_UNSUPPORTED),
    (dict(max_tree=257, N=16), TA_ERR_UNSUPPORTED),
    (dict(page_size=24), TA_ERR_UNSUPPORTED),
    (dict(page_size=0), TA_ERR_UNSUPPORTED),
    (dict(page_size=2048, max_pages=1), TA_ERR_UNSUPPORTED),
    (dict(Hq=30), TA_ERR_BAD_SHAPE),
    (dict(Hkv=0), TA_ERR_BAD_SHAPE),
    (dict(B=-1), TA_ERR_BAD_SHAPE),
    (dict(N=17), TA_ERR_BAD_SHAPE),           # N > B * max_tree
    (dict(max_prefix=2049), TA_ERR_BAD_SHAPE),  # beyond the block table
    (dict(num_pages=0), TA_ERR_BAD_SHAPE),
    (dict(num_splits=65), TA_ERR_BAD_SHAPE),
    (dict(num_splits=-1), TA_ERR_BAD_SHAPE),
    (dict(scale=float("nan")), TA_ERR_BAD_SHAPE),
    (dict(scale=float("inf")), TA_ERR_BAD_SHAPE),
    (dict(q=None), TA_ERR_NULL_PTR),
    (dict(anc_mask=None), TA_ERR_NULL_PTR),
    (dict(lse=None), TA_ERR_NULL_PTR),
    (dict(k_cache=None), TA_ERR_NULL_PTR),
    (dict(block_table=None), TA_ERR_NULL_PTR),
    (dict(workspace=None), TA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), TA_ERR_WORKSPACE),
    (dict(workspace=FAKE + 4), TA_ERR_WORKSPACE),
    # rows move as 16-byte vectors, mask words as u64, the rest as 32-bit words
    (dict(q=FAKE + 4), TA_ERR_BAD_SHAPE),
    (dict(k_cache=FAKE + 8), TA_ERR_BAD_SHAPE),
    (dict(v_tree=FAKE + 2), TA_ERR_BAD_SHAPE),
    (dict(out=FAKE + 12), TA_ERR_BAD_SHAPE),
    (dict(anc_mask=FAKE + 4), TA_ERR_BAD_SHAPE),
    (dict(lse=FAKE + 2), TA_ERR_BAD_SHAPE),
])
def test_fwd_check_rejects(lib, over, code):
    assert check(lib, **over) == code
    # the full entry points return the same code before any launch
    assert call_fwd(lib, **over) == code
    assert call_plan_fwd(lib, **over) == code


def call_plan_fwd(lib, **over):
    a = fwd_args(**over)
    for k in ("parent", "depth", "pos_id", "status"):
        a.setdefault(k, FAKE)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.tree_attn_plan_fwd(P(a["q"]), P(a["k_tree"]), P(a["v_tree"]), P(a["k_cache"]),
                                  P(a["v_cache"]), P(a["block_table"]), P(a["prefix_len"]),
                                  P(a["tree_off"]), P(a["parent"]), a["B"], a["N"], a["Hq"], a["Hkv"],
                                  a["D"], a["page_size"], a["num_pages"], a["max_pages"], a["max_tree"],
                                  a["max_prefix"], a["scale"], a["dtype"], a["num_splits"],
                                  P(a["anc_mask"]), P(a["depth"]), P(a["pos_id"]), P(a["status"]),
                                  P(a["out"]), P(a["lse"]), P(a["workspace"]), a["ws_bytes"], None)


@pytest.mark.parametrize("over", [dict(parent=None), dict(depth=None), dict(pos_id=None),
                                  dict(status=None), dict(status=None, dtype=FP32, D=64, Hq=4, Hkv=1)])
def test_plan_fwd_pointer_rules(lib, over):
    # the plan's pointers are checked after the forward's, before any launch
    assert call_plan_fwd(lib, **over) == TA_ERR_NULL_PTR


def test_plan_fwd_empty_batch_is_noop(lib):
    assert call_plan_fwd(lib, B=0, N=0, q=None, out=None, lse=None, workspace=None, parent=None,
                         anc_mask=None, depth=None, pos_id=None, status=None) == TA_OK


def test_no_prefix_needs_no_cache_pointers(lib):
    assert check(lib, k_cache=None, v_cache=None, block_table=None, max_prefix=0,
                 workspace=None, ws_bytes=0) == TA_OK


def test_empty_calls_are_noops(lib):
    # nothing to do: valid even with null buffers, and nothing is launched
    assert call_fwd(lib, N=0, q=None, out=None, lse=None, workspace=None) == TA_OK
    assert call_fwd(lib, B=0, N=0, q=None, out=None, lse=None, workspace=None) == TA_OK
    assert lib.tree_attn_plan(None, None, None, 0, 0, 16, None, None, None, None, None) == TA_OK


def test_plan_argument_checks(lib):
    P = ctypes.c_void_p
    f = P(FAKE)
    assert lib.tree_attn_plan(f, f, f, 1, 16, 300, f, f, f, f, None) == TA_ERR_UNSUPPORTED
    assert lib.tree_attn_plan(f, f, f, -1, 16, 16, f, f, f, f, None) == TA_ERR_BAD_SHAPE
    assert lib.tree_attn_plan(f, f, f, 1, 17, 16, f, f, f, f, None) == TA_ERR_BAD_SHAPE
    assert lib.tree_attn_plan(f, None, f, 1, 16, 16, f, f, f, f, None) == TA_ERR_NULL_PTR
    assert lib.tree_attn_plan(f, f, f, 1, 16, 16, f, f, None, f, None) == TA_ERR_NULL_PTR
    assert lib.tree_attn_plan(f, f, f, 1, 16, 16, f, f, f, None, None) == TA_ERR_NULL_PTR


def test_split_choice_for_the_named_workloads():
    # (B, Hq, Hkv, D, max_tree, max_prefix, dtype) -> splits
    assert ta.num_splits(1, 4, 1, 64, 16, 128, __import__("torch").float32) == 1    # tiny (fp32)
    assert ta.num_splits(1, 32, 8, 128, 16, 2048) == 17                                # chain16
    assert ta.num_splits(1, 32, 8, 128, 256, 2048) == 6                                # tree256
    assert ta.num_splits(1, 32, 8, 128, 256, 8192) == 8    # one request, long prefix: no tree slot
    assert ta.num_splits(8, 32, 8, 128, 64, 8192) == 5                                 # mixed
    assert ta.num_splits(32, 32, 4, 128, 256, 4096) == 1                               # moe


def test_split_choice_properties():
    for B in (1, 2, 5, 40):
        for T in (1, 16, 100, 256):
            for L in (0, 1, 63, 64, 65, 1000, 8192, 100000):
                s = ta.num_splits(B, 16, 4, 128, T, L)
                assert 1 <= s <= 64
                if L == 0:
                    assert s == 1
                elif s > 1:
                    # each prefix slot keeps >= 1 key block; a single request
                    # has one more slot, for its tree
                    assert s - (1 if B == 1 else 0) <= -(-L // 64)
                ws = ta.workspace_bytes(B, B * T, 16, 4, 128, T, L)
                if s == 1:
                    assert ws == 0
                else:
                    # fp16 partial outputs and fp32 (lse, scale exponent) pairs per split
                    assert ws >= s * B * T * 16 * (128 * 2 + 8)
    # forcing a split count, and no workspace without a prefix
    assert ta.workspace_bytes(1, 16, 32, 8, 128, 16, 2048, num_splits=3) > 0
    assert ta.workspace_bytes(1, 16, 32, 8, 128, 16, 0) == 0
    assert ta.workspace_bytes(1, 16, 32, 8, 128, 16, 2048, num_splits=1) == 0


def commit_call(lib, **over):
    a = dict(anc=FAKE, depth=FAKE, tree_off=FAKE, prefix_len=FAKE, accepted=FAKE, k_tree=FAKE,
             v_tree=FAKE, k_cache=FAKE, v_cache=FAKE, block_table=FAKE, B=2, N=10, Hkv=8, D=128,
             page_size=16, num_pages=100, max_pages=8, max_tree=8, dtype=BF16, new_len=FAKE,
             status=FAKE)
    a.update(over)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.tree_attn_commit(P(a["anc"]), P(a["depth"]), P(a["tree_off"]), P(a["prefix_len"]),
                                P(a["accepted"]), P(a["k_tree"]), P(a["v_tree"]), P(a["k_cache"]),
                                P(a["v_cache"]), P(a["block_table"]), a["B"], a["N"], a["Hkv"], a["D"],
                                a["page_size"], a["num_pages"], a["max_pages"], a["max_tree"], a["dtype"],
                                P(a["new_len"]), P(a["status"]), None)


@pytest.mark.parametrize("over,code", [
    (dict(dtype=7), TA_ERR_UNSUPPORTED),
    (dict(max_tree=257, N=10), TA_ERR_UNSUPPORTED),
    (dict(page_size=24), TA_ERR_UNSUPPORTED),
    (dict(Hkv=1, D=4), TA_ERR_UNSUPPORTED),        # 8-byte rows cannot move 16 bytes at a time
    (dict(N=17), TA_ERR_BAD_SHAPE),                # N > B * max_tree
    (dict(B=-1), TA_ERR_BAD_SHAPE),
    (dict(Hkv=0), TA_ERR_BAD_SHAPE),
    (dict(accepted=None), TA_ERR_NULL_PTR),
    (dict(block_table=None), TA_ERR_NULL_PTR),
    (dict(status=None), TA_ERR_NULL_PTR),
    (dict(anc=None), TA_ERR_NULL_PTR),
    (dict(k_cache=FAKE + 8), TA_ERR_BAD_SHAPE),     # rows are copied 16 bytes at a time
])
def test_commit_rejects_before_launch(lib, over, code):
    assert commit_call(lib, **over) == code


def test_commit_empty_batch_is_noop(lib):
    assert commit_call(lib, B=0, N=0, anc=None, depth=None, tree_off=None, prefix_len=None,
                       accepted=None, k_tree=None, v_tree=None, k_cache=None, v_cache=None,
                       block_table=None, new_len=None, status=None) == TA_OK


@pytest.mark.parametrize("args,code", [
    ((2, 16, 65, 16), TA_ERR_UNSUPPORTED),   # K > 64
    ((2, 65, 8, 16), TA_ERR_UNSUPPORTED),    # depth > 64
    ((2, 16, 8, 257), TA_ERR_UNSUPPORTED),   # budget > 256
    ((2, 2, 2, 7), TA_ERR_BAD_SHAPE),        # the implicit tree has 6 nodes
    ((-1, 16, 8, 16), TA_ERR_BAD_SHAPE),
    ((2, 16, 0, 16), TA_ERR_BAD_SHAPE),
])
def test_build_tree_rejects_before_launch(lib, args, code):
    B, Dmax, K, T = args
    f = ctypes.c_void_p(FAKE)
    assert lib.tree_attn_build_tree(f, B, Dmax, K, T, f, f, f, None) == code


def test_build_tree_null_and_empty(lib):
    f = ctypes.c_void_p(FAKE)
    assert lib.tree_attn_build_tree(None, 2, 16, 8, 16, f, f, f, None) == TA_ERR_NULL_PTR
    assert lib.tree_attn_build_tree(None, 0, 16, 8, 16, None, None, None, None) == TA_OK
    assert lib.tree_attn_build_tree(None, 2, 16, 8, 0, None, None, None, None) == TA_OK


def plan_dfs_call(lib, **over):
    a = dict(parent=FAKE, tree_off=FAKE, prefix_len=FAKE, B=2, N=300, max_tree=256, perm=FAKE,
             inv=FAKE, parent_new=FAKE, anc=FAKE, depth=FAKE, pos=FAKE, status=FAKE)
    a.update(over)
    P = ctypes.c_void_p
    return lib.tree_attn_plan_dfs(P(a["parent"]), P(a["tree_off"]), P(a["prefix_len"]), a["B"], a["N"],
                                  a["max_tree"], P(a["perm"]), P(a["inv"]), P(a["parent_new"]),
                                  P(a["anc"]), P(a["depth"]), P(a["pos"]), P(a["status"]), None)


def test_plan_dfs_argument_checks(lib):
    assert plan_dfs_call(lib, max_tree=257) == TA_ERR_UNSUPPORTED
    assert plan_dfs_call(lib, N=513) == TA_ERR_BAD_SHAPE          # more nodes than B * max_tree
    assert plan_dfs_call(lib, B=-1) == TA_ERR_BAD_SHAPE
    assert plan_dfs_call(lib, B=0, N=0) == TA_OK                    # nothing to do, nothing launched
    for name in ("tree_off", "prefix_len", "status", "parent", "perm", "inv", "parent_new", "anc",
                 "depth", "pos"):
        assert plan_dfs_call(lib, **{name: 0}) == TA_ERR_NULL_PTR, name


def gather_call(lib, **over):
    a = dict(src=FAKE, n_src=10, index=FAKE, dst=FAKE, n_rows=10, row_bytes=256)
    a.update(over)
    P = ctypes.c_void_p
    return lib.tree_attn_gather_rows(P(a["src"]), a["n_src"], P(a["index"]), P(a["dst"]), a["n_rows"],
                                     a["row_bytes"], None)


def test_gather_rows_argument_checks(lib):
    assert gather_call(lib, row_bytes=6) == TA_ERR_BAD_SHAPE        # not a multiple of 4
    assert gather_call(lib, n_rows=-1) == TA_ERR_BAD_SHAPE
    assert gather_call(lib, n_src=1 << 40) == TA_ERR_BAD_SHAPE      # indices are int32
    assert gather_call(lib, n_rows=0) == TA_OK                       # nothing to do, nothing launched
    assert gather_call(lib, index=0) == TA_ERR_NULL_PTR
    assert gather_call(lib, dst=0) == TA_ERR_NULL_PTR
    assert gather_call(lib, src=0) == TA_ERR_NULL_PTR
    assert gather_call(lib, src=FAKE + 2) == TA_ERR_UNSUPPORTED       # not 4-byte aligned


def call_noalloc(lib, **over):
    a = fwd_args(**over)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.tree_attn_fwd_noalloc(P(a["q"]), P(a["k_tree"]), P(a["v_tree"]), P(a["k_cache"]),
                                     P(a["v_cache"]), P(a["block_table"]), P(a["prefix_len"]),
                                     P(a["tree_off"]), P(a["anc_mask"]), a["B"], a["N"], a["Hq"], a["Hkv"],
                                     a["D"], a["page_size"], a["num_pages"], a["max_pages"], a["max_tree"],
                                     a["max_prefix"], a["scale"], a["dtype"], a["num_splits"], P(a["out"]),
                                     P(a["lse"]), None)


def test_noalloc_refuses_beyond_its_array_before_launching(lib):
    """The no-allocation forward computes its workspace need on the host and
    refuses a call that needs more than its fixed array, before any HIP call
    (this runs without a GPU)."""
    limit = ta.NOALLOC_SCRATCH_BYTES
    big = dict(B=1, N=256, max_tree=256, num_splits=64)
    assert ta.workspace_bytes(1, 256, 32, 8, 128, 256, 2048, num_splits=64) > limit
    assert call_noalloc(lib, **big) == TA_ERR_SCRATCH_LIMIT
    assert lib.tree_attn_status_str(TA_ERR_SCRATCH_LIMIT).startswith(b"the call needs more split workspace")
    # host argument errors come first when the workspace fits (or is not needed)
    assert call_noalloc(lib, D=96) == TA_ERR_UNSUPPORTED
    assert call_noalloc(lib, B=0, N=0, q=None, out=None, lse=None) == TA_OK


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define TREE_ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ta.NOALLOC_SCRATCH_BYTES

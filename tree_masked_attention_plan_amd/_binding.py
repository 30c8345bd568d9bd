"""ctypes marshalling for libtree_attn.so; see include/tree_attn.h for the
contract of every call (layouts, ownership, error codes)."""
from __future__ import annotations

import ctypes
import math
import os
from typing import NamedTuple, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libtree_attn.so"

MASK_WORDS = 4
MAX_TREE = 256
NOALLOC_SCRATCH_BYTES = 32 << 20   # TREE_ATTN_NOALLOC_SCRATCH_BYTES
TA_DTYPE = {torch.bfloat16: 0, torch.float32: 1}

_lib = None


class TreeAttnError(RuntimeError):
    pass


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build the HIP library first "
                          f"(python -m tree_masked_attention_plan_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.tree_attn_abi_version.restype = ctypes.c_int
    lib.tree_attn_abi_version.argtypes = []
    lib.tree_attn_status_str.restype = ctypes.c_char_p
    lib.tree_attn_status_str.argtypes = [ctypes.c_int]
    lib.tree_attn_plan.restype = ctypes.c_int
    lib.tree_attn_plan.argtypes = [P, P, P, i32, i32, i32, P, P, P, P, P]
    lib.tree_attn_num_splits.restype = i32
    lib.tree_attn_num_splits.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int]
    lib.tree_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.tree_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.c_int, i32]
    fwd_args = [P, P, P, P, P, P, P, P, P,
                i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                ctypes.c_float, ctypes.c_int, i32, P, P, P, ctypes.c_size_t]
    for name in ("tree_attn_fwd", "tree_attn_fwd_partial", "tree_attn_merge"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = fwd_args + [P]
    for name in ("tree_attn_plan_fwd", "tree_attn_plan_fwd_partial"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = fwd_args[:9] + fwd_args[9:22] + [P, P, P, P] + fwd_args[22:] + [P]
    lib.tree_attn_fwd_check.restype = ctypes.c_int
    lib.tree_attn_fwd_check.argtypes = fwd_args
    lib.tree_attn_fwd_noalloc.restype = ctypes.c_int
    lib.tree_attn_fwd_noalloc.argtypes = fwd_args[:24] + [P]
    lib.tree_attn_build_tree.restype = ctypes.c_int
    lib.tree_attn_build_tree.argtypes = [P, i32, i32, i32, i32, P, P, P, P]
    lib.tree_attn_plan_dfs.restype = ctypes.c_int
    lib.tree_attn_plan_dfs.argtypes = [P, P, P, i32, i32, i32, P, P, P, P, P, P, P, P]
    lib.tree_attn_gather_rows.restype = ctypes.c_int
    lib.tree_attn_gather_rows.argtypes = [P, ctypes.c_int64, P, P, ctypes.c_int64, ctypes.c_int64, P]
    lib.tree_attn_commit.restype = ctypes.c_int
    lib.tree_attn_commit.argtypes = [P, P, P, P, P, P, P, P, P, P,
                                     i32, i32, i32, i32, i32, i32, i32, i32, ctypes.c_int, P, P, P]
    _lib = lib
    return lib


def abi_version() -> int:
    return load_library().tree_attn_abi_version()


def _raise(rc: int, what: str):
    if rc != 0:
        msg = load_library().tree_attn_status_str(rc).decode()
        raise TreeAttnError(f"{what}: {msg} (status {rc})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _after_current(stream, device) -> None:
    """A call enqueued on another stream than the current one first waits
    for the current stream, on which its inputs were produced and its
    buffers allocated."""
    if stream is not None and stream != torch.cuda.current_stream(device):
        stream.wait_stream(torch.cuda.current_stream(device))


def _keep_for(stream, *tensors) -> None:
    """Tie tensors allocated on the current stream to ``stream`` as well when
    the kernels run on another one: the caching allocator then does not hand
    their memory to a later allocation until ``stream`` has passed this
    point (the workspace in particular, whose only reference is dropped when
    a one-shot call returns)."""
    if stream is None:
        return
    for t in tensors:
        if t is not None and t.numel() > 0 and stream != torch.cuda.current_stream(t.device):
            t.record_stream(stream)


def _dev_tensor(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class PlanResult(NamedTuple):
    anc_mask: torch.Tensor   # [N, 4] int64 bit patterns of u64 words
    depth: torch.Tensor      # [N] int32
    pos_id: torch.Tensor     # [N] int32
    status: torch.Tensor     # [B] int32


def _max_tree_of(tree_off: torch.Tensor) -> int:
    if tree_off.numel() <= 1:
        return 0
    return int((tree_off[1:] - tree_off[:-1]).max().item())   # synchronises


def plan(parent: torch.Tensor, tree_off: torch.Tensor, prefix_len: torch.Tensor,
         max_tree: Optional[int] = None, *, out: Optional[PlanResult] = None,
         stream=None) -> PlanResult:
    """Ancestor bitmask, depth and position ids of every tree node.

    ``max_tree`` (a host bound on every tree size) avoids a device sync when
    given.  ``status`` is written on the device; :func:`check_status` reads it.
    """
    _dev_tensor(parent, "parent", torch.int32)
    _dev_tensor(tree_off, "tree_off", torch.int32)
    _dev_tensor(prefix_len, "prefix_len", torch.int32)
    dev = parent.device
    B = prefix_len.numel()
    N = parent.numel()
    if tree_off.numel() != B + 1:
        raise ValueError("tree_off must have B+1 entries")
    if max_tree is None:
        max_tree = _max_tree_of(tree_off)
    if out is None:
        out = PlanResult(torch.empty((N, MASK_WORDS), dtype=torch.int64, device=dev),
                         torch.empty(N, dtype=torch.int32, device=dev),
                         torch.empty(N, dtype=torch.int32, device=dev),
                         torch.empty(B, dtype=torch.int32, device=dev))
    rc = load_library().tree_attn_plan(_ptr(parent), _ptr(tree_off), _ptr(prefix_len), B, N,
                                       int(max_tree), _ptr(out.anc_mask), _ptr(out.depth),
                                       _ptr(out.pos_id), _ptr(out.status), _stream(dev, stream))
    _raise(rc, "tree_attn_plan")
    _keep_for(stream, *out)
    return out


class PlanDfsResult(NamedTuple):
    perm: torch.Tensor        # [N] int32: new global index -> old global index
    inv_perm: torch.Tensor    # [N] int32: old -> new
    parent_new: torch.Tensor  # [N] int32: local parents in the new labelling
    plan: PlanResult          # the plan of the relabelled trees (rows in the new order)


def plan_dfs(parent: torch.Tensor, tree_off: torch.Tensor, prefix_len: torch.Tensor,
             max_tree: Optional[int] = None, *, stream=None) -> PlanDfsResult:
    """The plan of every tree in a depth-first relabelling (preorder, roots
    and children in increasing index), with the permutation that maps it to
    the old labels.  Gather the rows of q / k_tree / v_tree with ``perm``
    (:func:`gather_rows`) to run :func:`fwd` in the new order, and the rows
    of its outputs with ``inv_perm`` to return to the old order."""
    _dev_tensor(parent, "parent", torch.int32)
    _dev_tensor(tree_off, "tree_off", torch.int32)
    _dev_tensor(prefix_len, "prefix_len", torch.int32)
    dev = parent.device
    B = prefix_len.numel()
    N = parent.numel()
    if tree_off.numel() != B + 1:
        raise ValueError("tree_off must have B+1 entries")
    if max_tree is None:
        max_tree = _max_tree_of(tree_off)
    res = PlanDfsResult(torch.empty(N, dtype=torch.int32, device=dev),
                        torch.empty(N, dtype=torch.int32, device=dev),
                        torch.empty(N, dtype=torch.int32, device=dev),
                        PlanResult(torch.empty((N, MASK_WORDS), dtype=torch.int64, device=dev),
                                   torch.empty(N, dtype=torch.int32, device=dev),
                                   torch.empty(N, dtype=torch.int32, device=dev),
                                   torch.empty(B, dtype=torch.int32, device=dev)))
    rc = load_library().tree_attn_plan_dfs(
        _ptr(parent), _ptr(tree_off), _ptr(prefix_len), B, N, int(max_tree), _ptr(res.perm),
        _ptr(res.inv_perm), _ptr(res.parent_new), _ptr(res.plan.anc_mask), _ptr(res.plan.depth),
        _ptr(res.plan.pos_id), _ptr(res.plan.status), _stream(dev, stream))
    _raise(rc, "tree_attn_plan_dfs")
    _keep_for(stream, res.perm, res.inv_perm, res.parent_new, *res.plan)
    return res


def gather_rows(src: torch.Tensor, index: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """``out[i] = src[index[i]]`` along the first dimension (rows of any
    contiguous device tensor; an index out of range gives a zero row)."""
    _dev_tensor(index, "index", torch.int32)
    if src.device != index.device or not src.is_contiguous():
        raise ValueError("src must be a contiguous tensor on the index's device")
    n_src = src.shape[0] if src.dim() > 0 else 0
    row_bytes = src[0].numel() * src.element_size() if n_src > 0 else 0
    if out is None:
        out = torch.empty((index.numel(),) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    rc = load_library().tree_attn_gather_rows(_ptr(src), int(n_src), _ptr(index), _ptr(out),
                                              int(index.numel()), int(row_bytes),
                                              _stream(src.device, stream))
    _raise(rc, "tree_attn_gather_rows")
    _keep_for(stream, out)
    return out


def build_tree(logp: torch.Tensor, T: int, *, stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Best-first draft trees of budget ``T`` from per-depth candidate
    log-probabilities ``logp`` [B, max_depth, K] (fp32).  Returns ``(parent,
    choice, score)``, each [B, T], nodes in pop order (``parent[b, i] < i``;
    -1 hangs off the prefix)."""
    _dev_tensor(logp, "logp", torch.float32)
    if logp.dim() != 3:
        raise ValueError("logp must be [B, max_depth, K]")
    B, Dmax, K = logp.shape
    dev = logp.device
    parent = torch.empty((B, T), dtype=torch.int32, device=dev)
    choice = torch.empty((B, T), dtype=torch.int32, device=dev)
    score = torch.empty((B, T), dtype=torch.float32, device=dev)
    rc = load_library().tree_attn_build_tree(_ptr(logp), B, Dmax, K, int(T), _ptr(parent), _ptr(choice),
                                             _ptr(score), _stream(dev, stream))
    _raise(rc, "tree_attn_build_tree")
    _keep_for(stream, parent, choice, score)
    return parent, choice, score


def commit(anc_mask: torch.Tensor, depth: torch.Tensor, tree_off: torch.Tensor,
           prefix_len: torch.Tensor, accepted: torch.Tensor, k_tree: torch.Tensor,
           v_tree: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_table: torch.Tensor, max_tree: Optional[int] = None, *,
           new_prefix_len: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Append each request's accepted path (node ``accepted[b]`` and its
    ancestors, from :func:`plan`'s ``anc_mask`` / ``depth``) to its paged
    K/V cache, in place.  Returns ``(new_prefix_len, status)`` (device)."""
    if k_cache.dtype not in TA_DTYPE:
        raise ValueError(f"unsupported dtype {k_cache.dtype}")
    dt = k_cache.dtype
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name, dt)
    _dev_tensor(anc_mask, "anc_mask", torch.int64)
    for name, t in (("depth", depth), ("tree_off", tree_off), ("prefix_len", prefix_len),
                    ("accepted", accepted), ("block_table", block_table)):
        _dev_tensor(t, name, torch.int32)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_tree.dim() != 3 or v_tree.shape != k_tree.shape:
        raise ValueError("k_cache/v_cache must be [num_pages,page_size,Hkv,D] and k_tree/v_tree [N,Hkv,D]")
    num_pages, page_size, Hkv, D = k_cache.shape
    N = k_tree.shape[0]
    B = prefix_len.numel()
    if k_tree.shape[1:] != (Hkv, D) or tree_off.numel() != B + 1 or accepted.numel() != B:
        raise ValueError("inconsistent shapes")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    if anc_mask.shape != (N, MASK_WORDS) or depth.numel() != N:
        raise ValueError("anc_mask / depth must come from a plan of these trees")
    if max_tree is None:
        max_tree = _max_tree_of(tree_off)
    dev = k_cache.device
    if new_prefix_len is None:
        new_prefix_len = torch.empty(B, dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=dev)
    rc = load_library().tree_attn_commit(
        _ptr(anc_mask), _ptr(depth), _ptr(tree_off), _ptr(prefix_len), _ptr(accepted), _ptr(k_tree),
        _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), B, N, Hkv, D, page_size,
        num_pages, block_table.shape[1], int(max_tree), TA_DTYPE[dt], _ptr(new_prefix_len),
        _ptr(status), _stream(dev, stream))
    _raise(rc, "tree_attn_commit")
    _keep_for(stream, new_prefix_len, status)
    return new_prefix_len, status


def check_status(status: torch.Tensor) -> None:
    """Raise if any request's plan status is non-zero (synchronises)."""
    s = status.cpu()
    bad = torch.nonzero(s).flatten().tolist()
    if bad:
        b = bad[0]
        code = int(s[b])
        if code == -1:
            why = "inconsistent tree offsets or a tree larger than max_tree"
        elif code == -2:
            why = "negative prefix length"
        else:
            why = f"node {code - 1} has a parent that does not precede it"
        raise TreeAttnError(f"request {b}: {why} (status {code}); bad requests: {bad}")


def num_splits(B: int, Hq: int, Hkv: int, D: int, max_tree: int, max_prefix: int,
               dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load_library().tree_attn_num_splits(B, Hq, Hkv, D, max_tree, max_prefix, TA_DTYPE[dtype]))


def workspace_bytes(B: int, N: int, Hq: int, Hkv: int, D: int, max_tree: int, max_prefix: int,
                    dtype: torch.dtype = torch.bfloat16, num_splits: int = 0) -> int:
    return int(load_library().tree_attn_workspace_bytes(B, N, Hq, Hkv, D, max_tree, max_prefix,
                                                        TA_DTYPE[dtype], num_splits))


_NO_WORKSPACE = object()   # prepare_fwd: marshal without a workspace (the no-allocation entry)


class FwdCall:
    """One forward call with its arguments marshalled once.

    ``run()`` enqueues the whole operation, ``partial()`` / ``merge()`` its two
    stages (see tree_attn_fwd_partial / tree_attn_merge); all on ``stream``
    (default: the current stream at call time).  ``out`` / ``lse`` hold the
    results once the stream reaches that point.
    """

    def __init__(self, args, out, lse, workspace, nsplit):
        self._args = args
        self.out = out
        self.lse = lse
        self.workspace = workspace
        self.num_splits = nsplit
        self._lib = load_library()

    def _call(self, fn, name, stream):
        _after_current(stream, self.out.device)
        rc = fn(*self._args, _stream(self.out.device, stream))
        _raise(rc, name)
        _keep_for(stream, self.workspace, self.out, self.lse)
        return self

    def run(self, stream=None):
        return self._call(self._lib.tree_attn_fwd, "tree_attn_fwd", stream)

    def partial(self, stream=None):
        return self._call(self._lib.tree_attn_fwd_partial, "tree_attn_fwd_partial", stream)

    def merge(self, stream=None):
        return self._call(self._lib.tree_attn_merge, "tree_attn_merge", stream)


def prepare_fwd(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor, k_cache: torch.Tensor,
                v_cache: torch.Tensor, block_table: torch.Tensor, prefix_len: torch.Tensor,
                tree_off: torch.Tensor, anc_mask: torch.Tensor, *, max_tree: Optional[int] = None,
                max_prefix: Optional[int] = None, scale: Optional[float] = None, num_splits: int = 0,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> FwdCall:
    """Check and marshal the arguments of a forward call; see :func:`fwd`."""
    if q.dtype not in TA_DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dt = q.dtype
    for name, t in (("q", q), ("k_tree", k_tree), ("v_tree", v_tree), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _dev_tensor(t, name, dt)
    _dev_tensor(block_table, "block_table", torch.int32)
    _dev_tensor(prefix_len, "prefix_len", torch.int32)
    _dev_tensor(tree_off, "tree_off", torch.int32)
    _dev_tensor(anc_mask, "anc_mask", torch.int64)
    if q.dim() != 3 or k_tree.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q/k_tree must be [N,H,D] and k_cache [pages,page_size,Hkv,D]")
    N, Hq, D = q.shape
    Hkv = k_tree.shape[1]
    if k_tree.shape != (N, Hkv, D) or v_tree.shape != k_tree.shape:
        raise ValueError("k_tree/v_tree must be [N,Hkv,D]")
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    if k_cache.shape[2:] != (Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [num_pages,page_size,Hkv,D]")
    B = prefix_len.numel()
    if tree_off.numel() != B + 1 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("tree_off must be [B+1] and block_table [B, max_pages]")
    if anc_mask.shape != (N, MASK_WORDS):
        raise ValueError(f"anc_mask must be [N,{MASK_WORDS}]")
    max_pages = block_table.shape[1]
    dev = q.device
    if max_tree is None:
        max_tree = _max_tree_of(tree_off)
    if max_prefix is None:
        max_prefix = int(prefix_len.max().item()) if B else 0
    if out is None:
        out = torch.empty((N, Hq, D), dtype=dt, device=dev)
    else:
        _dev_tensor(out, "out", dt)
        if out.shape != (N, Hq, D):
            raise ValueError("out must be [N,Hq,D]")
    if lse is None:
        lse = torch.empty((N, Hq), dtype=torch.float32, device=dev)
    else:
        _dev_tensor(lse, "lse", torch.float32)
        if lse.shape != (N, Hq):
            raise ValueError("lse must be [N,Hq]")
    lib = load_library()
    need = lib.tree_attn_workspace_bytes(B, N, Hq, Hkv, D, max_tree, max_prefix, TA_DTYPE[dt], num_splits)
    no_ws = workspace is _NO_WORKSPACE
    if no_ws:
        workspace = None
    elif workspace is None and need > 0:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev_tensor(workspace, "workspace", torch.uint8)
        base = workspace.data_ptr()
        pad = (-base) % 256
        ws_ptr = ctypes.c_void_p(base + pad)
        ws_bytes = max(0, workspace.numel() - pad)
    sc = 0.0 if scale is None else float(scale)
    if not math.isfinite(sc):
        raise ValueError("scale must be finite")
    args = (_ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(prefix_len), _ptr(tree_off), _ptr(anc_mask), B, N, Hq, Hkv, D, page_size, num_pages,
            max_pages, int(max_tree), int(max_prefix), sc, TA_DTYPE[dt], int(num_splits), _ptr(out),
            _ptr(lse), ws_ptr, ws_bytes)
    if not no_ws:
        rc = lib.tree_attn_fwd_check(*args)
        _raise(rc, "tree_attn_fwd")
    nsplit = lib.tree_attn_num_splits(B, Hq, Hkv, D, int(max_tree), int(max_prefix), TA_DTYPE[dt]) \
        if num_splits == 0 else num_splits
    return FwdCall(args, out, lse, workspace, nsplit)


def fwd(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor, k_cache: torch.Tensor,
        v_cache: torch.Tensor, block_table: torch.Tensor, prefix_len: torch.Tensor,
        tree_off: torch.Tensor, anc_mask: torch.Tensor, *, max_tree: Optional[int] = None,
        max_prefix: Optional[int] = None, scale: Optional[float] = None, num_splits: int = 0,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, stream=None):
    """Tree-causal attention; returns ``(out [N,Hq,D], lse [N,Hq] fp32)``.

    ``max_tree`` / ``max_prefix`` are host bounds; when omitted they are read
    from the device (a synchronisation).  ``workspace`` (a uint8 tensor of at
    least :func:`workspace_bytes` bytes) is allocated here when not given.
    ``num_splits`` = 0 lets the library choose the prefix split count.
    """
    call = prepare_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off,
                       anc_mask, max_tree=max_tree, max_prefix=max_prefix, scale=scale,
                       num_splits=num_splits, out=out, lse=lse, workspace=workspace)
    call.run(stream)
    return call.out, call.lse


class PlanFwdCall:
    """One tree_attn_plan_fwd call with its arguments marshalled once.

    ``run()`` enqueues the plan and the attention in one call on ``stream``
    (default: the current stream at call time); ``partial()`` / ``merge()``
    its two stages (tree_attn_plan_fwd_partial, then tree_attn_merge).
    ``plan`` (a PlanResult), ``out`` and ``lse`` hold the results once the
    stream reaches that point.
    """

    def __init__(self, args, fwd_args, plan_res, out, lse, workspace, nsplit):
        self._args = args
        self._fwd_args = fwd_args
        self.plan = plan_res
        self.out = out
        self.lse = lse
        self.workspace = workspace
        self.num_splits = nsplit
        self._lib = load_library()

    def _kept(self, stream):
        _keep_for(stream, self.workspace, self.out, self.lse, *self.plan)
        return self

    def run(self, stream=None):
        _after_current(stream, self.out.device)
        rc = self._lib.tree_attn_plan_fwd(*self._args, _stream(self.out.device, stream))
        _raise(rc, "tree_attn_plan_fwd")
        return self._kept(stream)

    def partial(self, stream=None):
        _after_current(stream, self.out.device)
        rc = self._lib.tree_attn_plan_fwd_partial(*self._args, _stream(self.out.device, stream))
        _raise(rc, "tree_attn_plan_fwd_partial")
        return self._kept(stream)

    def merge(self, stream=None):
        _after_current(stream, self.out.device)
        rc = self._lib.tree_attn_merge(*self._fwd_args, _stream(self.out.device, stream))
        _raise(rc, "tree_attn_merge")
        return self._kept(stream)


def prepare_plan_fwd(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor, k_cache: torch.Tensor,
                     v_cache: torch.Tensor, block_table: torch.Tensor, prefix_len: torch.Tensor,
                     tree_off: torch.Tensor, parent: torch.Tensor, *, max_tree: Optional[int] = None,
                     max_prefix: Optional[int] = None, scale: Optional[float] = None, num_splits: int = 0,
                     plan_out: Optional[PlanResult] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> PlanFwdCall:
    """Check and marshal the arguments of a plan + forward call; see :func:`plan_fwd`."""
    _dev_tensor(parent, "parent", torch.int32)
    N, B = q.shape[0], prefix_len.numel()
    if parent.numel() != N:
        raise ValueError("parent must have N entries")
    dev = q.device
    if plan_out is None:
        plan_out = PlanResult(torch.empty((N, MASK_WORDS), dtype=torch.int64, device=dev),
                              torch.empty(N, dtype=torch.int32, device=dev),
                              torch.empty(N, dtype=torch.int32, device=dev),
                              torch.empty(B, dtype=torch.int32, device=dev))
    else:
        _dev_tensor(plan_out.depth, "depth", torch.int32)
        _dev_tensor(plan_out.pos_id, "pos_id", torch.int32)
        _dev_tensor(plan_out.status, "status", torch.int32)
        if plan_out.depth.numel() != N or plan_out.pos_id.numel() != N or plan_out.status.numel() != B:
            raise ValueError("plan_out must hold [N] depth / pos_id and [B] status")
    # the forward's own checks and marshalling, with the plan's mask output in
    # place of the mask input
    call = prepare_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off,
                       plan_out.anc_mask, max_tree=max_tree, max_prefix=max_prefix, scale=scale,
                       num_splits=num_splits, out=out, lse=lse, workspace=workspace)
    a = call._args
    args = (a[:8] + (_ptr(parent),) + a[9:22] +
            (_ptr(plan_out.anc_mask), _ptr(plan_out.depth), _ptr(plan_out.pos_id), _ptr(plan_out.status)) +
            a[22:])
    return PlanFwdCall(args, a, plan_out, call.out, call.lse, call.workspace, call.num_splits)


def plan_fwd(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor, k_cache: torch.Tensor,
             v_cache: torch.Tensor, block_table: torch.Tensor, prefix_len: torch.Tensor,
             tree_off: torch.Tensor, parent: torch.Tensor, *, max_tree: Optional[int] = None,
             max_prefix: Optional[int] = None, scale: Optional[float] = None, num_splits: int = 0,
             stream=None) -> Tuple[PlanResult, torch.Tensor, torch.Tensor]:
    """:func:`plan` and :func:`fwd` in one call (tree_attn_plan_fwd): returns
    ``(plan, out, lse)``, the plan exactly as :func:`plan` writes it."""
    call = prepare_plan_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off, parent,
                            max_tree=max_tree, max_prefix=max_prefix, scale=scale, num_splits=num_splits)
    call.run(stream)
    return call.plan, call.out, call.lse


def fwd_noalloc(q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor, k_cache: torch.Tensor,
                v_cache: torch.Tensor, block_table: torch.Tensor, prefix_len: torch.Tensor,
                tree_off: torch.Tensor, anc_mask: torch.Tensor, *, out: torch.Tensor, lse: torch.Tensor,
                max_tree: int, max_prefix: int, scale: Optional[float] = None, num_splits: int = 0,
                stream=None):
    """:func:`fwd` through tree_attn_fwd_noalloc: the split workspace comes
    from the library's fixed per-device array, and nothing is allocated here
    either (``out``, ``lse``, ``max_tree`` and ``max_prefix`` are the
    caller's).  Raises TreeAttnError with TA_ERR_SCRATCH_LIMIT when the call
    needs more than NOALLOC_SCRATCH_BYTES of workspace."""
    call = prepare_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off, anc_mask,
                       max_tree=max_tree, max_prefix=max_prefix, scale=scale, num_splits=num_splits,
                       out=out, lse=lse, workspace=_NO_WORKSPACE)
    a = call._args
    _after_current(stream, out.device)
    rc = load_library().tree_attn_fwd_noalloc(*a[:24], _stream(out.device, stream))
    _raise(rc, "tree_attn_fwd_noalloc")
    return out, lse

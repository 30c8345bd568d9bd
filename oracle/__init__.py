"""fp64 CPU oracle for tree-causal paged attention -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it.

``oracle_tree_attn`` / ``oracle_plan`` / ``oracle_dfs_order`` (and the
adjacent steps) live in ``tree_attn_oracle.c`` (plain
C, built with gcc by :func:`build`); this module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tree_attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

MASK_WORDS = 4


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (never with hipcc)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _declare(lib):
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.oracle_plan.restype = ctypes.c_int
    lib.oracle_plan.argtypes = [P, P, P, i32, i32, i32, P, P, P, P]
    lib.oracle_tree_attn.restype = ctypes.c_int
    lib.oracle_tree_attn.argtypes = [P, P, P, P, P, P, P, P, P,
                                     i32, i32, i32, i32, i32, i32, i32, i32, ctypes.c_double,
                                     P, ctypes.c_int64, P, P, i32]
    lib.oracle_dfs_order.restype = ctypes.c_int
    lib.oracle_dfs_order.argtypes = [P, P, P, i32, i32, i32, P, P, P, P]
    lib.oracle_build_tree.restype = ctypes.c_int
    lib.oracle_build_tree.argtypes = [P, i32, i32, i32, i32, P, P, P]
    lib.oracle_commit.restype = ctypes.c_int
    lib.oracle_commit.argtypes = [P, P, P, P, P, P, P, P, P,
                                  i32, i32, i32, i32, i32, i32, i32, i32, i32, P, P]
    return lib


def load_library(path: str):
    """Load an oracle build from ``path`` (used to load planted-mistake builds
    in the pin-strength test)."""
    return _declare(ctypes.CDLL(path))


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = load_library(_LIB_PATH)
    return _lib


def _np(x, dtype) -> np.ndarray:
    """numpy copy/view of a numpy array or a (CPU) torch tensor, contiguous."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if dtype == np.float64:
            x = x.double()
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def plan(parent, tree_off, prefix_len, max_tree: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(anc_mask [N,4] uint64, depth [N] int32, pos_id [N] int32, status [B] int32)."""
    lib = _load()
    parent = _np(parent, np.int32)
    tree_off = _np(tree_off, np.int32)
    prefix_len = _np(prefix_len, np.int32)
    B = len(prefix_len)
    N = len(parent)
    mask = np.zeros((N, MASK_WORDS), dtype=np.uint64)
    depth = np.zeros(N, dtype=np.int32)
    pos = np.zeros(N, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    rc = lib.oracle_plan(_ptr(parent), _ptr(tree_off), _ptr(prefix_len), B, N, int(max_tree),
                         _ptr(mask), _ptr(depth), _ptr(pos), _ptr(status))
    if rc != 0:
        raise ValueError(f"oracle_plan: error {rc}")
    return mask, depth, pos, status


def dfs_order(parent, tree_off, prefix_len, max_tree: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Depth-first relabelling of every request's tree (``oracle_dfs_order``):
    (perm [N] new -> old, inv [N] old -> new, both global node indices;
    parent_new [N] local parents in the new labelling; status [B])."""
    lib = _load()
    parent = _np(parent, np.int32)
    tree_off = _np(tree_off, np.int32)
    prefix_len = _np(prefix_len, np.int32)
    B = len(prefix_len)
    N = len(parent)
    perm = np.zeros(N, dtype=np.int32)
    inv = np.zeros(N, dtype=np.int32)
    parent_new = np.zeros(N, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    rc = lib.oracle_dfs_order(_ptr(parent), _ptr(tree_off), _ptr(prefix_len), B, N, int(max_tree),
                              _ptr(perm), _ptr(inv), _ptr(parent_new), _ptr(status))
    if rc != 0:
        raise ValueError(f"oracle_dfs_order: error {rc}")
    return perm, inv, parent_new, status


def tree_attn(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, tree_off, parent,
              scale: Optional[float] = None, rows=None, threads: Optional[int] = None):
    """fp64 tree attention.  Returns ``(out, lse)``: ``out`` is [N,Hq,D] and
    ``lse`` [N,Hq] (natural log), or [R,D] / [R] for an explicit list of rows
    ``row = node * Hq + h``.  Float inputs are widened exactly to fp64."""
    lib = _load()
    q = _np(q, np.float64)
    k_tree = _np(k_tree, np.float64)
    v_tree = _np(v_tree, np.float64)
    k_cache = _np(k_cache, np.float64)
    v_cache = _np(v_cache, np.float64)
    block_table = _np(block_table, np.int32)
    prefix_len = _np(prefix_len, np.int32)
    tree_off = _np(tree_off, np.int32)
    parent = _np(parent, np.int32)
    N, Hq, D = q.shape
    Hkv = k_tree.shape[1]
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    B = len(prefix_len)
    if block_table.ndim != 2:
        block_table = block_table.reshape(B, -1)
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        rows_arr = None
        R = N * Hq
    else:
        rows_arr = _np(rows, np.int64)
        R = len(rows_arr)
    out = np.zeros((R, D), dtype=np.float64)
    lse = np.zeros(R, dtype=np.float64)
    nt = default_threads() if threads is None else int(threads)
    rc = lib.oracle_tree_attn(_ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_table), _ptr(prefix_len), _ptr(tree_off), _ptr(parent),
                              B, N, Hq, Hkv, D, page_size, max_pages, num_pages, float(scale),
                              None if rows_arr is None else _ptr(rows_arr), R,
                              _ptr(out), _ptr(lse), nt)
    if rc != 0:
        raise ValueError(f"oracle_tree_attn: error {rc}")
    if rows is None:
        return out.reshape(N, Hq, D), lse.reshape(N, Hq)
    return out, lse


def tree_attn_workload(w, rows=None, threads=None, scale=None):
    """Convenience: run :func:`tree_attn` on a ``workloads.Workload``."""
    return tree_attn(w.q, w.k_tree, w.v_tree, w.k_cache, w.v_cache, w.block_table,
                     w.prefix_len, w.tree_off, w.parent,
                     scale=w.scale if scale is None else scale, rows=rows, threads=threads)


def commit(parent, tree_off, prefix_len, accepted, k_tree, v_tree, k_cache, v_cache, block_table,
           max_tree: int):
    """Copy of the accepted paths' K/V rows into the paged caches.

    Works on raw bytes, so any element type is fine.  Returns
    ``(k_cache', v_cache', new_prefix_len [B] int32, status [B] int32)``;
    the caches come back as uint8 arrays [num_pages, page_size, Hkv,
    D * element size] holding the committed bytes (the inputs are not
    modified)."""
    lib = _load()
    parent = _np(parent, np.int32)
    tree_off = _np(tree_off, np.int32)
    prefix_len = _np(prefix_len, np.int32)
    accepted = _np(accepted, np.int32)
    bt = _np(block_table, np.int32)

    def raw(x):
        """The tensor's bytes as a fresh uint8 array (last axis = D * element size)."""
        if hasattr(x, "detach"):
            return x.detach().cpu().contiguous().view(__import__("torch").uint8).numpy().copy()
        x = np.ascontiguousarray(x)
        return x.view(np.uint8).reshape(x.shape[:-1] + (-1,)).copy()

    def elem(x):
        return x.element_size() if hasattr(x, "element_size") else np.asarray(x).itemsize

    e = elem(k_cache)
    kt, vt, kc, vc = raw(k_tree), raw(v_tree), raw(k_cache), raw(v_cache)
    shape = tuple(k_cache.shape)
    num_pages, page_size, Hkv, D = shape
    B = len(prefix_len)
    N = len(parent)
    new_len = np.zeros(B, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    rc = lib.oracle_commit(_ptr(parent), _ptr(tree_off), _ptr(prefix_len), _ptr(accepted), _ptr(kt),
                           _ptr(vt), _ptr(kc), _ptr(vc), _ptr(bt), B, N, Hkv, D, e, page_size,
                           num_pages, bt.shape[1] if bt.ndim == 2 else 0, int(max_tree),
                           _ptr(new_len), _ptr(status))
    if rc != 0:
        raise ValueError(f"oracle_commit: error {rc}")
    return kc, vc, new_len, status


def build_tree(logp, T: int):
    """Best-first draft trees from per-depth candidate log-probabilities
    ``logp`` [B, Dmax, K] (fp32).  Returns ``(parent, choice, score)``, each
    [B, T] (int32, int32, float32), nodes in pop order."""
    lib = _load()
    lp = _np(logp, np.float32)
    B, Dmax, K = lp.shape
    parent = np.zeros((B, T), dtype=np.int32)
    choice = np.zeros((B, T), dtype=np.int32)
    score = np.zeros((B, T), dtype=np.float32)
    rc = lib.oracle_build_tree(_ptr(lp), B, Dmax, K, int(T), _ptr(parent), _ptr(choice), _ptr(score))
    if rc != 0:
        raise ValueError(f"oracle_build_tree: error {rc}")
    return parent, choice, score

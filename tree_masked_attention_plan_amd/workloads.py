"""Seeded synthetic inputs for tree-causal paged attention.

This module only *generates inputs*: token trees (as parent arrays), prefix
lengths, a shuffled page pool with block tables, and Q/K/V values.  It holds
none of the attention arithmetic and none of the mask construction; the HIP
library and the fp64 oracle both consume what it produces.

Shapes follow the five workloads of the method's evaluation, re-created
synthetically because the models (Qwen3-8B dense, Qwen3-30B-A3B MoE) and the
benchmark suites named on the pages are not available:

* ``tiny``    -- 1 request, prefix 128, random 16-node tree (depth <= 8),
                 4 q-heads / 1 kv-head, head_dim 64, fp32.
* ``chain16`` -- 1 request, prefix 2048, a 16-node chain (budget 16 is the
                 "short linear draft" regime), 32/8 heads, head_dim 128, bf16.
* ``tree256`` -- 1 request, prefix 2048, best-first tree of 256 nodes.
* ``mixed``   -- 8 requests, prefix lengths uniform in [512, 8192], best-first
                 trees of 64 nodes, one shared shuffled page pool.
* ``moe``     -- 32 requests, prefix 4096, best-first trees of 256 nodes,
                 32/4 heads (GQA group 8).

Tree construction for the synthetic trees follows the pages' description of
drafting (JetFlow technical summary, section 2, "tree construction"): logits
for every depth come from one pass, a branch is scored by its cumulative draft
log-probability, and best-first expansion grows the tree up to the budget.
The logits themselves are random: one vector of 8 candidate logits
``z_d ~ N(0, 2^2)`` per depth ``d``, shared by every node at depth ``d - 1``.

Seeds: workload ``i`` of the table above uses base seed ``1000 + i``; each
kind of random draw has its own independent stream (tree, prefix lengths,
page permutation, cache values, query/tree values).
"""
from __future__ import annotations

import dataclasses
import heapq
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

PAGE_SIZE = 16
MASK_WORDS = 4          # u64 words per node row of the ancestor bitmask
MAX_TREE = 64 * MASK_WORDS

# independent random streams per kind of draw
_STREAM_TREE, _STREAM_PREFIX, _STREAM_PERM, _STREAM_CACHE, _STREAM_QKV = range(5)

CONFIG_NAMES = ("tiny", "chain16", "tree256", "mixed", "moe")


def rng_for(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(stream)]))


# --------------------------------------------------------------------------
# token trees (parent arrays, topologically ordered: parent[i] < i, -1 = hangs
# directly off the prefix)
# --------------------------------------------------------------------------

def chain(T: int) -> np.ndarray:
    """Linear draft of T tokens: node i's parent is node i-1."""
    return np.arange(-1, T - 1, dtype=np.int32)


def random_tree(T: int, max_depth: int, rng: np.random.Generator) -> np.ndarray:
    """Single-root random tree: parent[i] uniform over earlier nodes whose
    depth (path length including the node) is below ``max_depth``."""
    if T == 0:
        return np.zeros(0, dtype=np.int32)
    parent = np.empty(T, dtype=np.int32)
    depth = np.empty(T, dtype=np.int64)
    parent[0] = -1
    depth[0] = 1
    for i in range(1, T):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        p = int(cand[rng.integers(len(cand))])
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def best_first_tree(T: int, rng: np.random.Generator, max_depth: int = 16,
                    children: int = 8, sigma: float = 2.0,
                    per_node_logits: bool = False) -> np.ndarray:
    """Best-first candidate tree over synthetic draft log-probabilities.

    A virtual root (the last context token, already in the prefix) has score
    0.  A node at depth d has ``children`` candidate continuations whose
    log-probabilities are ``log_softmax(z)`` with ``z ~ N(0, sigma^2)``; a
    child's score is its parent's score plus its own log-probability.  The
    highest-scoring candidate is popped, given the next node id (so ids are in
    pop order, which is topological), and its children are pushed unless it is
    at ``max_depth``.  Ties go to the earlier push.  With
    ``per_node_logits=False`` one logit vector per depth is shared by all
    nodes of that depth; otherwise each popped node draws its own.
    """
    if T == 0:
        return np.zeros(0, dtype=np.int32)

    def logprobs() -> np.ndarray:
        z = rng.normal(0.0, sigma, size=children)
        zmax = z.max()
        return z - (zmax + math.log(np.exp(z - zmax).sum()))

    depth_lp = None if per_node_logits else [logprobs() for _ in range(max_depth)]
    heap: List[tuple] = []
    seq = 0
    lp1 = depth_lp[0] if depth_lp is not None else logprobs()
    for k in range(children):
        heapq.heappush(heap, (-float(lp1[k]), seq, -1, 1))
        seq += 1
    parent: List[int] = []
    while len(parent) < T and heap:
        neg, _, par, d = heapq.heappop(heap)
        nid = len(parent)
        parent.append(par)
        if d < max_depth:
            lp = depth_lp[d] if depth_lp is not None else logprobs()
            for k in range(children):
                heapq.heappush(heap, (neg - float(lp[k]), seq, nid, d + 1))
                seq += 1
    return np.asarray(parent, dtype=np.int32)


def topo_relabel(parent: np.ndarray, rng: np.random.Generator):
    """Random topological relabelling sigma of a tree.

    Returns ``(new_parent, sigma)`` with ``sigma[old] = new`` such that every
    parent still precedes its child."""
    T = len(parent)
    children: Dict[int, List[int]] = {}
    for i, p in enumerate(parent):
        children.setdefault(int(p), []).append(i)
    ready = list(children.get(-1, []))
    sigma = np.full(T, -1, dtype=np.int64)
    nxt = 0
    while ready:
        k = int(rng.integers(len(ready)))
        node = ready.pop(k)
        sigma[node] = nxt
        nxt += 1
        ready.extend(children.get(node, []))
    assert nxt == T
    new_parent = np.empty(T, dtype=np.int32)
    for old in range(T):
        p = int(parent[old])
        new_parent[sigma[old]] = -1 if p < 0 else sigma[p]
    return new_parent, sigma


# --------------------------------------------------------------------------
# a batch of requests with a shared shuffled page pool
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    dtype: torch.dtype
    parent: torch.Tensor        # [N] int32, local parent ids
    tree_off: torch.Tensor      # [B+1] int32
    prefix_len: torch.Tensor    # [B] int32
    block_table: torch.Tensor   # [B, max_pages] int32, -1 = unused
    q: torch.Tensor             # [N, Hq, D]
    k_tree: torch.Tensor        # [N, Hkv, D]
    v_tree: torch.Tensor        # [N, Hkv, D]
    k_cache: torch.Tensor       # [num_pages, page_size, Hkv, D]
    v_cache: torch.Tensor
    seed: int

    @property
    def N(self) -> int:
        return int(self.tree_off[-1])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def tree_sizes(self) -> np.ndarray:
        off = self.tree_off.numpy().astype(np.int64)
        return off[1:] - off[:-1]

    @property
    def max_tree(self) -> int:
        return int(self.tree_sizes.max()) if self.B else 0

    @property
    def max_prefix(self) -> int:
        return int(self.prefix_len.max()) if self.B else 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def to(self, device) -> "Workload":
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**kw)


def _normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(dtype)


def make_workload(name: str, prefix_lens: Sequence[int], trees: Sequence[np.ndarray],
                  Hq: int, Hkv: int, D: int, dtype: torch.dtype, seed: int,
                  page_size: int = PAGE_SIZE, spare_frac: float = 0.10,
                  sentinel: float = float("nan"),
                  perm_rng: Optional[np.random.Generator] = None,
                  reserve_tokens: int = 0) -> Workload:
    """Assemble a batch: paged prefix K/V in one shuffled pool, tree K/V, Q.

    The pool holds exactly the live pages plus ``spare_frac`` spare pages; the
    physical id of every live page comes from a seeded permutation, so each
    request's pages are scattered and interleaved with the others.  Spare
    pages, slots past a request's prefix length in its last page, and unused
    block-table entries (-1) are filled with ``sentinel`` (NaN by default) so
    that any read of them poisons the output.  ``reserve_tokens`` extra
    token slots per request get live pages too (room for committing accepted
    tree tokens after the prefix); their slots hold the sentinel.
    """
    B = len(prefix_lens)
    assert len(trees) == B
    prefix_lens = [int(x) for x in prefix_lens]
    sizes = [len(t) for t in trees]
    tree_off = np.zeros(B + 1, dtype=np.int32)
    tree_off[1:] = np.cumsum(sizes)
    N = int(tree_off[-1])
    parent = np.concatenate([np.asarray(t, dtype=np.int32) for t in trees]) if N else np.zeros(0, np.int32)

    pages_per = [(L + reserve_tokens + page_size - 1) // page_size for L in prefix_lens]
    live = int(sum(pages_per))
    num_pages = max(1, live + int(math.ceil(spare_frac * live)))
    prng = perm_rng if perm_rng is not None else rng_for(seed, _STREAM_PERM)
    perm = prng.permutation(num_pages).astype(np.int32)
    max_pages = max(1, max(pages_per) if B else 1)
    block_table = np.full((B, max_pages), -1, dtype=np.int32)
    cur = 0
    for b in range(B):
        block_table[b, :pages_per[b]] = perm[cur:cur + pages_per[b]]
        cur += pages_per[b]

    crng = rng_for(seed, _STREAM_CACHE)
    k_cache = torch.full((num_pages, page_size, Hkv, D), sentinel, dtype=torch.float32).to(dtype)
    v_cache = torch.full((num_pages, page_size, Hkv, D), sentinel, dtype=torch.float32).to(dtype)
    kf = k_cache.view(num_pages * page_size, Hkv, D)
    vf = v_cache.view(num_pages * page_size, Hkv, D)
    for b in range(B):
        L = prefix_lens[b]
        if L == 0:
            continue
        kb = _normal(crng, (L, Hkv, D), dtype)
        vb = _normal(crng, (L, Hkv, D), dtype)
        t = np.arange(L)
        slots = torch.from_numpy(block_table[b, t // page_size].astype(np.int64) * page_size + t % page_size)
        kf[slots] = kb
        vf[slots] = vb

    qrng = rng_for(seed, _STREAM_QKV)
    q = _normal(qrng, (N, Hq, D), dtype)
    k_tree = _normal(qrng, (N, Hkv, D), dtype)
    v_tree = _normal(qrng, (N, Hkv, D), dtype)
    return Workload(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, page_size=page_size, dtype=dtype,
                    parent=torch.from_numpy(parent), tree_off=torch.from_numpy(tree_off),
                    prefix_len=torch.tensor(prefix_lens, dtype=torch.int32),
                    block_table=torch.from_numpy(block_table),
                    q=q, k_tree=k_tree, v_tree=v_tree, k_cache=k_cache, v_cache=v_cache,
                    seed=seed)


def make_config(name: str, seed: Optional[int] = None) -> Workload:
    """One of the five named workloads, from its default seed unless given."""
    idx = CONFIG_NAMES.index(name)
    seed = 1000 + idx if seed is None else int(seed)
    trng = rng_for(seed, _STREAM_TREE)
    if name == "tiny":
        return make_workload(name, [128], [random_tree(16, 8, trng)], 4, 1, 64, torch.float32, seed)
    if name == "chain16":
        return make_workload(name, [2048], [chain(16)], 32, 8, 128, torch.bfloat16, seed)
    if name == "tree256":
        return make_workload(name, [2048], [best_first_tree(256, trng)], 32, 8, 128, torch.bfloat16, seed)
    if name == "mixed":
        prng = rng_for(seed, _STREAM_PREFIX)
        lens = [int(x) for x in prng.integers(512, 8192, size=8, endpoint=True)]
        trees = [best_first_tree(64, trng) for _ in range(8)]
        return make_workload(name, lens, trees, 32, 8, 128, torch.bfloat16, seed)
    if name == "moe":
        trees = [best_first_tree(256, trng) for _ in range(32)]
        return make_workload(name, [4096] * 32, trees, 32, 4, 128, torch.bfloat16, seed)
    raise ValueError(name)


def random_accepted(trees: Sequence[np.ndarray], rng: np.random.Generator,
                    p_none: float = 0.1) -> np.ndarray:
    """One accepted node per tree (local id), uniform over its nodes, or -1
    (nothing accepted) with probability ``p_none`` or for an empty tree."""
    out = np.full(len(trees), -1, dtype=np.int32)
    for b, t in enumerate(trees):
        if len(t) and rng.random() >= p_none:
            out[b] = int(rng.integers(0, len(t)))
    return out

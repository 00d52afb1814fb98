"""Seeded synthetic workloads shaped like the verify step of tree speculative
decoding over a paged MLA latent KV cache.

Shapes follow the pages "The Custom sm_120 Verify Kernel: From 0.7 tok/s to
3-6x Decode Speedup on Blackwell Consumer GPUs" (Part I: one MLA latent row per
token in a pool of 195,011 slots; Part VI: page size 1 because accepted tree
nodes are scattered; Part VII: about 9 verify queries, 8 heads per rank,
NSPLIT 64) and "One Blocking Memcpy Per Verify Step" (a draft block of B = 12
verified as one causal chain; pages of 64 tokens).

Every array is a plain NumPy array. bf16 tensors are carried as their uint16
bit patterns. No attention arithmetic lives here: only random draws, the
round-to-nearest-even cast of the draws to bf16, tree shapes and page tables.

Layouts (the C-ABI uses the same ones):
  q           uint16 [B, T, H, 576]   absorbed query per (request, node, head)
  kv          uint16 [num_slots, 576] latent pool; V is the first 512 dims
  page_table  int32  [B, max_pages]   physical page ids, row b for request b
  seq_lens    int32  [B]              keys per request, tree rows included
  tree_parent int32  [B, T]           -1 for a root, else an index < i
Logical key p of request b lives in slot page_table[b, p // ps] * ps + p % ps.
The last T logical keys hold the tree nodes' own latent rows, in node order.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

HEAD_DIM_QK = 576  # 512 latent + 64 rope
HEAD_DIM_V = 512  # V is the leading 512 dims of the same latent row
SM_SCALE = 1.0 / math.sqrt(192.0)  # 128 nope + 64 rope query dims
POOL_SLOTS_PAGES = 195_011  # the KV pool size the first page reports


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and return
    the uint16 bit patterns. Inputs are finite draws, so NaN handling is moot."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16 bit patterns."""
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


# ---------------------------------------------------------------- draft trees

def tree_chain(t: int) -> np.ndarray:
    """A chain of t nodes: node i's parent is i-1 (a causal block)."""
    return np.arange(-1, t - 1, dtype=np.int32)


def tree_uniform(t: int, rng: np.random.Generator) -> np.ndarray:
    """Node 0 is the root; node i's parent is uniform over 0..i-1."""
    p = np.empty(t, dtype=np.int32)
    p[0] = -1
    for i in range(1, t):
        p[i] = rng.integers(0, i)
    return p


def tree_depth_capped(t: int, max_depth: int, rng: np.random.Generator) -> np.ndarray:
    """Node 0 is the root (depth 0); node i's parent is uniform over the earlier
    nodes whose depth is below max_depth, so no node is deeper than max_depth."""
    p = np.empty(t, dtype=np.int32)
    depth = np.zeros(t, dtype=np.int64)
    p[0] = -1
    for i in range(1, t):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        j = int(cand[rng.integers(0, len(cand))])
        p[i] = j
        depth[i] = depth[j] + 1
    return p


# ---------------------------------------------------------------- case record

@dataclass
class Case:
    name: str
    q: np.ndarray
    kv: np.ndarray
    page_table: np.ndarray
    seq_lens: np.ndarray
    tree_parent: np.ndarray
    page_size: int
    sm_scale: float = SM_SCALE
    nsplit: int = 1
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_nodes(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_slots(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def with_(self, **kw) -> "Case":
        return replace(self, **kw)

    def kv_bytes(self) -> int:
        """Latent bytes the step must read: one 576-wide bf16 row per key."""
        return int(np.sum(self.seq_lens.astype(np.int64))) * HEAD_DIM_QK * 2


def _scattered_single(name, seed, context, t, heads, pool_slots, tree, nsplit,
                      contiguous=False) -> Case:
    """One request, page size 1, its n = context + t keys on distinct slots of
    a pool: a random permutation prefix, or slots 0..n-1 when contiguous."""
    rng = np.random.default_rng(seed)
    n = context + t
    if n > pool_slots:
        raise ValueError("pool too small")
    q = normal_bf16(rng, (1, t, heads, HEAD_DIM_QK))
    kv = normal_bf16(rng, (pool_slots, HEAD_DIM_QK))
    slots = rng.permutation(pool_slots)[:n].astype(np.int32)
    if contiguous:
        # Same logical rows, laid out in ascending slots (a defragmented pool).
        logical = kv[slots].copy()
        kv = kv.copy()
        kv[:n] = logical
        slots = np.arange(n, dtype=np.int32)
    return Case(name=name, q=q, kv=kv, page_table=slots[None, :].copy(),
                seq_lens=np.array([n], dtype=np.int32),
                tree_parent=tree[None, :].astype(np.int32), page_size=1,
                nsplit=nsplit, meta=dict(seed=seed, context=[context]))


def _c1(seed=1, nsplit=4):
    rng = np.random.default_rng(seed)
    t, h, c = 4, 8, 256
    n = c + t
    q = normal_bf16(rng, (1, t, h, HEAD_DIM_QK))
    kv = normal_bf16(rng, (n, HEAD_DIM_QK))
    pt = rng.permutation(n).astype(np.int32)[None, :]
    return Case("C1", q, kv, pt, np.array([n], np.int32), tree_chain(t)[None, :],
                page_size=1, nsplit=nsplit, meta=dict(seed=seed, context=[c]))


def _c2(seed=2, nsplit=64):
    rng = np.random.default_rng(seed + 1000)
    tree = tree_uniform(16, rng)
    return _scattered_single("C2", seed, 4096, 16, 8, 200_000, tree, nsplit)


def _c3(seed=3, nsplit=128):
    rng = np.random.default_rng(seed + 1000)
    tree = tree_depth_capped(32, 8, rng)
    return _scattered_single("C3", seed, 65_536, 32, 8, POOL_SLOTS_PAGES, tree, nsplit)


def _c4(seed=4, nsplit=128, contiguous=False):
    rng = np.random.default_rng(seed + 1000)
    tree = tree_uniform(32, rng)
    return _scattered_single("C4b" if contiguous else "C4a", seed, 184_728, 32, 8,
                             POOL_SLOTS_PAGES, tree, nsplit, contiguous=contiguous)


def _c5(seed=5, nsplit=32, batch=8, t=12, heads=8, ps=64, lo=1024, hi=131_072):
    rng = np.random.default_rng(seed)
    ctx = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch))).astype(np.int64)
    n = ctx + t
    pages_needed = (n + ps - 1) // ps
    pool_pages = int(math.ceil(1.25 * int(pages_needed.sum())))
    max_pages = int(pages_needed.max())
    q = normal_bf16(rng, (batch, t, heads, HEAD_DIM_QK))
    kv = normal_bf16(rng, (pool_pages * ps, HEAD_DIM_QK))
    perm = rng.permutation(pool_pages).astype(np.int32)
    # Rows past a request's last page are never read; -1 marks them.
    pt = np.full((batch, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        k = int(pages_needed[b])
        pt[b, :k] = perm[off:off + k]
        off += k
    tree = np.stack([tree_chain(t)] * batch)
    return Case("C5", q, kv, pt, n.astype(np.int32), tree, page_size=ps,
                nsplit=nsplit, meta=dict(seed=seed, context=ctx.tolist()))


CONFIGS = {
    "C1": _c1,
    "C2": _c2,
    "C3": _c3,
    "C4a": lambda seed=4, nsplit=128: _c4(seed, nsplit, contiguous=False),
    "C4b": lambda seed=4, nsplit=128: _c4(seed, nsplit, contiguous=True),
    "C5": _c5,
}

SWEEP_CONTEXTS = (1024, 2048, 4096, 8192, 16_384, 32_768, 65_536, 131_072, 184_728)
SWEEP_NODES = (9, 16, 32)


def sweep_case(context: int, t: int, seed: int = 6, nsplit: int = 64) -> Case:
    """One point of the context sweep: page size 1 on a 195,011-slot pool, uniform
    parents (depth capped at 8 when t = 32)."""
    rng = np.random.default_rng(seed * 1_000_003 + context * 67 + t)
    tree = tree_depth_capped(t, 8, rng) if t == 32 else tree_uniform(t, rng)
    return _scattered_single(f"S{context}_T{t}", seed * 7919 + context + t, context, t, 8,
                             max(POOL_SLOTS_PAGES, context + t), tree, nsplit)


def make_case(name: str, seed: int | None = None, nsplit: int | None = None) -> Case:
    """Build one named configuration (C1, C2, C3, C4a, C4b, C5) with its default
    seed and NSPLIT unless overridden."""
    fn = CONFIGS[name]
    kw = {}
    if seed is not None:
        kw["seed"] = seed
    if nsplit is not None:
        kw["nsplit"] = nsplit
    return fn(**kw)


def small_case(seed: int, batch: int, nodes: int, heads: int, contexts, page_size: int = 1,
               tree: str = "uniform", nsplit: int = 4, pool_extra: int = 7,
               max_pages_extra: int = 0) -> Case:
    """A small random case for parity and property tests: given per-request
    contexts, a tree kind ('uniform', 'chain', 'depth8', 'star') and page size.
    Pages are drawn from a shuffled pool with some spare pages."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(contexts, dtype=np.int64)
    assert ctx.shape == (batch,)
    n = ctx + nodes
    pages = (n + page_size - 1) // page_size
    pool_pages = int(pages.sum()) + pool_extra
    max_pages = int(pages.max()) + max_pages_extra
    q = normal_bf16(rng, (batch, nodes, heads, HEAD_DIM_QK))
    kv = normal_bf16(rng, (pool_pages * page_size, HEAD_DIM_QK))
    perm = rng.permutation(pool_pages).astype(np.int32)
    pt = np.full((batch, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        pt[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])
    trees = []
    for _ in range(batch):
        if tree == "uniform":
            trees.append(tree_uniform(nodes, rng))
        elif tree == "chain":
            trees.append(tree_chain(nodes))
        elif tree == "depth8":
            trees.append(tree_depth_capped(nodes, 8, rng))
        elif tree == "star":
            p = np.zeros(nodes, dtype=np.int32)
            p[0] = -1
            trees.append(p)
        elif tree == "forest":
            p = tree_uniform(nodes, rng)
            roots = rng.random(nodes) < 0.3
            p[roots] = -1
            trees.append(p)
        else:
            raise ValueError(tree)
    return Case(f"small{seed}", q, kv, pt, n.astype(np.int32), np.stack(trees).astype(np.int32),
                page_size=page_size, nsplit=nsplit, meta=dict(seed=seed, context=ctx.tolist()))

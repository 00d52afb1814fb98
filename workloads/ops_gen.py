"""Seeded synthetic inputs for the steps next to the verify attention: sparse
top-k decode, the draft-tree accept and commit, the KV append, the sliding-window
gather and the fp8 indexer.

Shapes follow the pages: "The 24% Ceiling..." (sparse MLA decode of one token
over 512 top-k tokens with 64 heads, a split of 8 over the tokens; concurrency
up to 16), "The Custom sm_120 Verify Kernel..." (draft trees of about 9 nodes,
commit lengths of 7-8 on easy text, page size 1, a 195,011-slot pool), "One
Blocking Memcpy Per Verify Step" (window W = 4096, pages of P = 64, batch 8,
blocks of 12 tokens) and "The Indexer Breakthrough..." (64 positions of 128 fp8
values plus 64 fp32 scales per 8,448-byte block, a 4,097-entry page table,
262,208 positions).

No arithmetic of the methods lives here: only random draws, the RNE cast of
draws to bf16 bit patterns, and random fp8 codes drawn field by field.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .gen import HEAD_DIM_QK, SM_SCALE, normal_bf16, tree_chain, tree_depth_capped, tree_uniform

IDX_DIM = 128
IDX_PAGE = 64
IDX_BLOCK_BYTES = 8448
POOL_SLOTS = 195_011


# ---------------------------------------------------------------- sparse top-k decode

@dataclass
class SparseCase:
    q: np.ndarray         # uint16 [B, H, 576]
    kv: np.ndarray        # uint16 [slots, 576]
    indices: np.ndarray   # int32 [B, K], -1 = unused
    lens: np.ndarray      # int32 [B], entries of the list in use
    sm_scale: float = SM_SCALE
    nsplit: int = 16
    meta: dict = field(default_factory=dict)


def sparse_case(seed: int, batch: int = 1, heads: int = 64, topk: int = 512, pool: int = POOL_SLOTS,
                lens=None, holes: float = 0.0, nsplit: int = 16) -> SparseCase:
    """q and the pool are N(0,1) rounded to bf16; each request lists `topk`
    distinct random slots of the pool (its selected tokens); entries at or past
    lens[b] are -1, and a fraction `holes` of the others is set to -1 too."""
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (batch, heads, HEAD_DIM_QK))
    kv = normal_bf16(rng, (pool, HEAD_DIM_QK))
    idx = np.stack([rng.choice(pool, size=topk, replace=False) for _ in range(batch)]).astype(np.int32)
    ln = np.full(batch, topk, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
    for b in range(batch):
        idx[b, ln[b]:] = -1
        if holes > 0:
            idx[b, :ln[b]][rng.random(ln[b]) < holes] = -1
    return SparseCase(q, kv, idx, ln, nsplit=nsplit, meta=dict(seed=seed))


# ---------------------------------------------------------------- tree accept / commit / append

@dataclass
class AcceptCase:
    tree_parent: np.ndarray    # int32 [B, T]
    draft_tokens: np.ndarray   # int32 [B, T]
    target_tokens: np.ndarray  # int32 [B, T]
    page_table: np.ndarray     # int32 [B, max_pages] (page size 1)
    seq_lens: np.ndarray       # int32 [B], context + T
    num_slots: int
    meta: dict = field(default_factory=dict)


def accept_case(seed: int, batch: int = 1, nodes: int = 16, tree: str = "uniform", match: float = 0.8,
                vocab: int = 151_936, contexts=None, pool: int = POOL_SLOTS) -> AcceptCase:
    """Random draft trees; the target's greedy choices are random tokens; a
    node's draft token copies the target's choice after its parent with
    probability `match`, else it is another random token. Each request's keys
    (context + tree rows) sit on distinct random slots of the pool."""
    rng = np.random.default_rng(seed)
    trees = []
    for _ in range(batch):
        if tree == "uniform":
            trees.append(tree_uniform(nodes, rng))
        elif tree == "chain":
            trees.append(tree_chain(nodes))
        elif tree == "depth8":
            trees.append(tree_depth_capped(nodes, 8, rng))
        elif tree == "forest":
            p = tree_uniform(nodes, rng)
            p[rng.random(nodes) < 0.25] = -1
            p[0] = -1
            trees.append(p)
        else:
            raise ValueError(tree)
    par = np.stack(trees).astype(np.int32)
    tgt = rng.integers(0, vocab, size=(batch, nodes), dtype=np.int64)
    drf = rng.integers(0, vocab, size=(batch, nodes), dtype=np.int64)
    for b in range(batch):
        for i in range(nodes):
            p = par[b, i]
            if p >= 0:
                if rng.random() < match:
                    drf[b, i] = tgt[b, p]
                elif drf[b, i] == tgt[b, p]:
                    drf[b, i] = (drf[b, i] + 1) % vocab
    ctx = np.asarray(contexts if contexts is not None else rng.integers(10, 5000, size=batch), dtype=np.int64)
    n = ctx + nodes
    maxp = int(n.max()) + 3
    pt = np.full((batch, maxp), -1, dtype=np.int32)
    if int(n.sum()) > pool:
        raise ValueError("pool too small for the requests' keys")
    perm = rng.permutation(pool)[:int(n.sum())].astype(np.int32)
    off = 0
    for b in range(batch):
        pt[b, :n[b]] = perm[off:off + n[b]]
        off += int(n[b])
    return AcceptCase(par, drf.astype(np.int32), tgt.astype(np.int32), pt, n.astype(np.int32), pool,
                      meta=dict(seed=seed, context=ctx.tolist()))


# ---------------------------------------------------------------- sliding-window gather

def window_case(seed: int, batch: int = 8, width: int = 200_000, lens=None, lo: int = 1, hi: int = 131_072):
    """target_map [B, width]: random slot ids (distinct per row); lens [B]
    log-uniform in [lo, hi] unless given."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = np.rint(np.exp(rng.uniform(np.log(lo), np.log(hi), size=batch))).astype(np.int64)
    lens = np.minimum(np.asarray(lens, dtype=np.int64), width)
    tm = np.stack([rng.permutation(10 * width)[:width] for _ in range(batch)]).astype(np.int32)
    return tm, lens.astype(np.int32)


# ---------------------------------------------------------------- fp8 indexer

def e4m3_codes(rng: np.random.Generator, shape, spread: float = 2.0) -> np.ndarray:
    """Random finite fp8 E4M3 codes drawn field by field: a uniform sign, an
    exponent field 7 + round(N(0, spread)) clipped to [0, 15], a uniform
    mantissa; the NaN code S.1111.111 is replaced by S.1111.110."""
    sign = rng.integers(0, 2, size=shape).astype(np.uint8) << 7
    e = np.clip(7 + np.rint(rng.normal(0.0, spread, size=shape)), 0, 15).astype(np.uint8)
    m = rng.integers(0, 8, size=shape).astype(np.uint8)
    m = np.where((e == 15) & (m == 7), 6, m).astype(np.uint8)
    return (sign | (e << 3) | m).astype(np.uint8)


@dataclass
class IndexerCase:
    q: np.ndarray            # uint8 [B, H, 128] e4m3 codes
    weights: np.ndarray      # float32 [B, H]
    blocks: np.ndarray       # uint8 [num_blocks, 8448]
    block_table: np.ndarray  # int32 [B, max_blocks]
    seq_lens: np.ndarray     # int32 [B] positions
    meta: dict = field(default_factory=dict)


def indexer_case(seed: int, batch: int = 1, heads: int = 64, max_blocks: int = 4097, seq_lens=None,
                 spare_blocks: int = 5) -> IndexerCase:
    """Blocks hold random e4m3 codes and positive fp32 scales exp(N(0,1)) / 64;
    weights are N(0,1) / sqrt(H); each request's pages are distinct random
    blocks of the cache, -1 past its last page."""
    rng = np.random.default_rng(seed)
    sl = np.full(batch, max_blocks * IDX_PAGE, dtype=np.int64) if seq_lens is None else np.asarray(seq_lens, np.int64)
    pages = -(-sl // IDX_PAGE)
    nb = int(pages.sum()) + spare_blocks
    codes = e4m3_codes(rng, (nb, IDX_PAGE * IDX_DIM))
    scales = (np.exp(rng.standard_normal((nb, IDX_PAGE))) / 64.0).astype(np.float32)
    blocks = np.concatenate([codes, scales.view(np.uint8).reshape(nb, IDX_PAGE * 4)], axis=1)
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])
    q = e4m3_codes(rng, (batch, heads, IDX_DIM))
    w = (rng.standard_normal((batch, heads)) / np.sqrt(heads)).astype(np.float32)
    return IndexerCase(q, w, np.ascontiguousarray(blocks), bt, sl.astype(np.int32), meta=dict(seed=seed))

"""Validity of the seeded input generators (workloads/): both the oracles and the
GPU tests consume them, so a generator bug would pass silently through both.

Checks: draft trees are topological (parent < child) with the depth cap held;
page tables name distinct in-range pages; seq_lens count the tree rows; the
C4a/C4b layouts hold the same logical rows; C5's page counts and ragged
lengths; the bf16 rounding agrees with torch's cast (round to nearest even);
the same seed gives the same arrays; the next-row generators keep their stated
shapes and ranges."""

import math

import numpy as np
import pytest
import torch

from workloads import make_case, sweep_case
from workloads.gen import (POOL_SLOTS_PAGES, f32_to_bf16_bits, small_case, tree_chain, tree_depth_capped,
                           tree_uniform)
from workloads.ops_gen import accept_case, e4m3_codes, indexer_case, sparse_case, window_case


def _depths(par):
    d = np.zeros(len(par), dtype=np.int64)
    for i, p in enumerate(par):
        d[i] = 0 if p < 0 else d[p] + 1
    return d


def _topological(par):
    return all(p == -1 or 0 <= p < i for i, p in enumerate(par.tolist()))


# ------------------------------------------------------------------ trees

def test_chain_tree():
    for t in (1, 2, 12, 64):
        par = tree_chain(t)
        assert par.dtype == np.int32 and len(par) == t
        assert par[0] == -1 and all(par[i] == i - 1 for i in range(1, t))


def test_uniform_tree_is_topological_with_one_root():
    rng = np.random.default_rng(0)
    seen_parents = set()
    for t in (1, 2, 9, 16, 32, 64):
        for _ in range(20):
            par = tree_uniform(t, rng)
            assert par[0] == -1 and _topological(par)
            assert np.count_nonzero(par == -1) == 1
            seen_parents |= {(i, int(p)) for i, p in enumerate(par) if i == 5}
    # node 5's parent ranges over all of 0..4 (uniform over the earlier nodes)
    assert {p for _, p in seen_parents} == {0, 1, 2, 3, 4}


@pytest.mark.parametrize("cap", [1, 3, 8])
def test_depth_capped_tree(cap):
    rng = np.random.default_rng(cap)
    reached = False
    for _ in range(30):
        par = tree_depth_capped(32, cap, rng)
        assert par[0] == -1 and _topological(par)
        d = _depths(par)
        assert d.max() <= cap
        reached |= d.max() == cap
    # a uniform 32-node tree is about ln 32 deep, so only the small caps bind
    assert reached or cap == 8


# ------------------------------------------------------------------ the named configurations

def _slots_of(case, b):
    n = int(case.seq_lens[b])
    p = np.arange(n)
    pages = case.page_table[b][p // case.page_size].astype(np.int64)
    return pages * case.page_size + p % case.page_size


@pytest.mark.parametrize("name,context,nodes,pool", [("C1", 256, 4, 260), ("C2", 4096, 16, 200_000),
                                                     ("C3", 65_536, 32, POOL_SLOTS_PAGES)])
def test_single_request_configs(name, context, nodes, pool):
    c = make_case(name)
    assert c.q.shape == (1, nodes, 8, 576) and c.q.dtype == np.uint16
    assert c.kv.shape == (pool, 576) and c.page_size == 1
    assert int(c.seq_lens[0]) == context + nodes and c.meta["context"] == [context]
    s = _slots_of(c, 0)
    assert len(np.unique(s)) == len(s) and s.min() >= 0 and s.max() < pool
    assert _topological(c.tree_parent[0])
    if name == "C1":
        assert np.array_equal(c.tree_parent[0], tree_chain(4))
    if name == "C3":
        assert _depths(c.tree_parent[0]).max() <= 8


def test_185k_layouts_hold_the_same_logical_rows():
    a, b = make_case("C4a"), make_case("C4b")
    n = 184_728 + 32
    assert int(a.seq_lens[0]) == n == int(b.seq_lens[0])
    sa, sb = _slots_of(a, 0), _slots_of(b, 0)
    assert len(np.unique(sa)) == n and sa.max() < POOL_SLOTS_PAGES
    assert np.array_equal(sb, np.arange(n))  # contiguous
    assert not np.array_equal(sa, sb)        # fragmented
    assert np.array_equal(a.kv[sa], b.kv[sb])
    assert np.array_equal(a.q, b.q) and np.array_equal(a.tree_parent, b.tree_parent)


def test_batched_block_verify_config():
    c = make_case("C5")
    ctx = np.asarray(c.meta["context"])
    assert c.batch == 8 and c.page_size == 64 and c.num_nodes == 12
    assert np.all(ctx >= 1024) and np.all(ctx <= 131_072)
    assert len(set(ctx.tolist())) > 1  # ragged
    n = ctx + 12
    assert np.array_equal(c.seq_lens, n)
    pages = -(-n // 64)
    assert c.max_pages == pages.max()
    assert c.kv.shape[0] == 64 * math.ceil(1.25 * int(pages.sum()))
    used = []
    for b in range(8):
        row = c.page_table[b]
        assert np.all(row[:pages[b]] >= 0) and np.all(row[pages[b]:] == -1)
        used += row[:pages[b]].tolist()
        assert np.array_equal(c.tree_parent[b], tree_chain(12))
    assert len(used) == len(set(used)) and max(used) < c.kv.shape[0] // 64


def test_sweep_case():
    c = sweep_case(4096, 9, nsplit=32)
    assert c.q.shape == (1, 9, 8, 576) and int(c.seq_lens[0]) == 4096 + 9 and c.nsplit == 32
    s = _slots_of(c, 0)
    assert len(np.unique(s)) == len(s) and s.max() < c.kv.shape[0]
    c32 = sweep_case(2048, 32)
    assert _depths(c32.tree_parent[0]).max() <= 8


@pytest.mark.parametrize("ps", [1, 4, 64])
def test_small_case(ps):
    c = small_case(seed=9, batch=3, nodes=7, heads=2, contexts=[0, 65, 300], page_size=ps, tree="forest",
                   max_pages_extra=2)
    assert np.array_equal(c.seq_lens, np.array([7, 72, 307]))
    used = []
    for b in range(3):
        k = -(-int(c.seq_lens[b]) // ps)
        row = c.page_table[b]
        assert np.all(row[:k] >= 0) and np.all(row[k:] == -1)
        used += row[:k].tolist()
        assert _topological(c.tree_parent[b])
    assert len(used) == len(set(used)) and max(used) < c.kv.shape[0] // ps


def test_same_seed_same_arrays():
    a, b = make_case("C2"), make_case("C2")
    for f in ("q", "kv", "page_table", "seq_lens", "tree_parent"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = make_case("C2", seed=99)
    assert not np.array_equal(a.q, c.q)


# ------------------------------------------------------------------ bf16 rounding

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200_000).astype(np.float32)
    # ties: the low 16 bits exactly 0x8000, with even and odd upper halves
    ties = (np.arange(1000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32)
    edge = np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, 65504.0], dtype=np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)], edge])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), want)


# ------------------------------------------------------------------ generators of the next rows

def test_sparse_case():
    c = sparse_case(3, batch=4, heads=16, topk=64, pool=5000, lens=[64, 10, 0, 33], holes=0.2)
    assert c.q.shape == (4, 16, 576) and c.indices.shape == (4, 64)
    for b, n in enumerate([64, 10, 0, 33]):
        live = c.indices[b, :n]
        assert np.all(c.indices[b, n:] == -1)
        assert np.all(live >= -1) and np.all(live < 5000)
        kept = live[live >= 0]
        assert len(np.unique(kept)) == len(kept)


def test_accept_case():
    c = accept_case(4, batch=5, nodes=12, tree="depth8", contexts=[3, 100, 7, 1000, 50], pool=3000)
    assert np.array_equal(c.seq_lens, np.array([15, 112, 19, 1012, 62]))
    used = []
    for b in range(5):
        assert _topological(c.tree_parent[b]) and _depths(c.tree_parent[b]).max() <= 8
        n = int(c.seq_lens[b])
        assert np.all(c.page_table[b, :n] >= 0) and np.all(c.page_table[b, n:] == -1)
        used += c.page_table[b, :n].tolist()
    assert len(used) == len(set(used)) and max(used) < 3000
    assert c.draft_tokens.min() >= 0 and c.target_tokens.max() < 151_936


def test_window_case():
    tm, lens = window_case(2, batch=6, width=3000, lo=1, hi=3000)
    assert tm.shape == (6, 3000) and lens.shape == (6,)
    assert np.all(lens >= 1) and np.all(lens <= 3000)
    for row in tm:
        assert len(np.unique(row)) == len(row)


def test_indexer_case_and_codes():
    rng = np.random.default_rng(1)
    codes = e4m3_codes(rng, (100_000,))
    assert not np.any((codes & 0x7F) == 0x7F)  # no NaN code
    c = indexer_case(6, batch=3, heads=8, max_blocks=5, seq_lens=[320, 1, 0], spare_blocks=2)
    assert c.blocks.shape == (5 + 1 + 0 + 2, 8448) and c.q.shape == (3, 8, 128)
    scales = np.ascontiguousarray(c.blocks[:, 8192:]).view(np.float32)
    assert np.all(scales > 0)
    for b, k in enumerate([5, 1, 0]):
        assert np.all(c.block_table[b, :k] >= 0) and np.all(c.block_table[b, k:] == -1)
    used = c.block_table[c.block_table >= 0]
    assert len(np.unique(used)) == len(used) and used.max() < c.blocks.shape[0]

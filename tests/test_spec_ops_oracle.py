"""Pins for the oracles of the steps next to the verify attention, each tied to
something other than the oracle itself: the verify oracle and its brute force
(already pinned), library decoders and attention routines, closed forms, the
pages' own claims and printed numbers, hand-worked examples, independent
enumerations and invariants. The planted-mistake tests at the end check that the
pins fail when an oracle is wrong in a plausible way."""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.spec_ops_oracle as so
from oracle import bf16_bits_to_f64, brute_force_verify, oracle_verify
from workloads.gen import f32_to_bf16_bits
from workloads.ops_gen import (IDX_BLOCK_BYTES, IDX_DIM, IDX_PAGE, accept_case, e4m3_codes, indexer_case,
                               sparse_case, window_case)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "next_rows_arithmetic.json")
G = {e["name"]: e for e in json.load(open(GOLDEN))["entries"]}


# ================================================================== golden numbers

def test_printed_sparse_decode_grid():
    e = G["sparse_decode_grid_without_split"]
    assert e["inputs"]["batch"] * e["inputs"]["heads"] == e["printed"]
    e = G["sparse_decode_grid_with_split"]
    assert e["inputs"]["batch"] * e["inputs"]["heads"] * e["inputs"]["split"] == e["printed"]
    assert sparse_case(1, pool=2000).indices.shape[1] == G["sparse_decode_topk"]["printed"]


def test_printed_indexer_block_layout():
    e = G["indexer_block_bytes"]["inputs"]
    assert e["positions"] * (e["fp8_values_per_position"] + e["scale_bytes"]) == G["indexer_block_bytes"]["printed"]
    assert IDX_BLOCK_BYTES == so.IDX_BLOCK_BYTES == G["indexer_block_bytes"]["printed"]
    assert IDX_PAGE * IDX_DIM == so.IDX_PAGE * so.IDX_DIM == G["indexer_fp8_part_bytes"]["printed"]
    e = G["indexer_positions_of_full_table"]
    assert e["inputs"]["page_table_entries"] * e["inputs"]["positions_per_block"] == e["printed"]


def test_printed_window_width_and_block():
    e = G["window_rectangle_width"]
    w, p = e["inputs"]["window"], e["inputs"]["page"]
    tm, lens = window_case(1, batch=1, width=20_000, lens=[10_000])
    dm, _ = so.window_map(tm, lens, w, p)
    assert dm.shape[1] == e["printed"] == w + p - 1
    e = G["block_verify_tokens"]
    assert e["inputs"]["batch"] * e["inputs"]["block"] == e["printed"]


# ================================================================== sparse top-k decode

def test_sparse_equals_verify_with_one_node():
    """With one node, the verify definition over a page-size-1 table sees every
    key (the context and the node's own row): the listed slots."""
    c = sparse_case(11, batch=3, heads=4, topk=40, pool=500)
    out, lse = so.sparse_decode(c.q, c.kv, c.indices, c.lens, c.sm_scale)
    ro, rl = oracle_verify(c.q[:, None], c.kv, c.indices, c.lens, np.full((3, 1), -1, np.int32), 1, c.sm_scale)
    assert np.allclose(out, ro[:, 0], atol=1e-12) and np.allclose(lse, rl[:, 0], atol=1e-12)


def test_sparse_matches_brute_force():
    c = sparse_case(12, batch=2, heads=2, topk=9, pool=60)
    out, lse = so.sparse_decode(c.q, c.kv, c.indices, c.lens, c.sm_scale)
    bo, bl = brute_force_verify(c.q[:, None], c.kv, c.indices, c.lens, np.full((2, 1), -1, np.int32), 1, c.sm_scale)
    assert np.allclose(out, np.array(bo)[:, 0], atol=1e-12) and np.allclose(lse, np.array(bl)[:, 0], atol=1e-12)


def test_sparse_matches_torch_sdpa():
    c = sparse_case(13, batch=2, heads=8, topk=64, pool=900, lens=[64, 37], holes=0.2)
    out, lse = so.sparse_decode(c.q, c.kv, c.indices, c.lens, c.sm_scale)
    for b in range(2):
        keys = c.indices[b, :c.lens[b]]
        keys = keys[keys >= 0]
        k = torch.from_numpy(bf16_bits_to_f64(c.kv[keys]))
        q = torch.from_numpy(bf16_bits_to_f64(c.q[b]))[:, None, :]  # [H, 1, 576]
        o = F.scaled_dot_product_attention(q, k[None].expand(8, -1, -1), k[None, :, :512].expand(8, -1, -1),
                                           scale=c.sm_scale)
        l = torch.logsumexp(c.sm_scale * (q[:, 0] @ k.T), dim=1)
        assert np.allclose(out[b], o[:, 0].numpy(), atol=1e-12) and np.allclose(lse[b], l.numpy(), atol=1e-12)


def test_sparse_zero_query_is_mean_of_listed_rows():
    c = sparse_case(14, batch=2, heads=3, topk=50, pool=400, lens=[50, 20], holes=0.3)
    z = np.zeros_like(c.q)
    out, lse = so.sparse_decode(z, c.kv, c.indices, c.lens, c.sm_scale)
    for b in range(2):
        keys = c.indices[b, :c.lens[b]]
        keys = keys[keys >= 0]
        mean = bf16_bits_to_f64(c.kv[keys, :512]).mean(axis=0)
        assert np.allclose(out[b], mean[None], atol=1e-12)
        assert np.allclose(lse[b], math.log(len(keys)), atol=1e-12)


def test_sparse_unused_entries_and_order_do_not_matter():
    c = sparse_case(15, batch=1, heads=4, topk=64, pool=700, holes=0.25)
    out, lse = so.sparse_decode(c.q, c.kv, c.indices, c.lens, c.sm_scale)
    keys = c.indices[0][c.indices[0] >= 0]
    rng = np.random.default_rng(0)
    packed = np.full((1, 64), -1, np.int32)
    packed[0, :len(keys)] = rng.permutation(keys)
    o2, l2 = so.sparse_decode(c.q, c.kv, packed, np.array([len(keys)], np.int32), c.sm_scale)
    assert np.allclose(out, o2, atol=1e-12) and np.allclose(lse, l2, atol=1e-12)


def test_sparse_empty_list():
    c = sparse_case(16, batch=2, heads=2, topk=8, pool=50, lens=[0, 8])
    out, lse = so.sparse_decode(c.q, c.kv, c.indices, c.lens, c.sm_scale)
    assert np.all(lse[0] == -np.inf) and np.all(out[0] == 0) and np.all(np.isfinite(lse[1]))


# ================================================================== greedy tree accept

def _accept_by_enumeration(par, drf, tgt):
    """Every root-to-node path, from children lists by depth-first search; a
    path is accepted iff each non-root node's draft equals the target's choice
    after the node before it. Longest path wins, then the smaller end node."""
    t = len(par)
    kids = [[] for _ in range(t)]
    for i, p in enumerate(par):
        if p >= 0:
            kids[p].append(i)
    best = None
    stack = [[r] for r in range(t) if par[r] == -1]
    while stack:
        path = stack.pop()
        if best is None or len(path) > len(best) or (len(path) == len(best) and path[-1] < best[-1]):
            best = path
        for c in kids[path[-1]]:
            if drf[c] == tgt[path[-1]]:
                stack.append(path + [c])
    return best


def test_accept_matches_enumeration():
    for seed in range(30):
        for tree in ("uniform", "chain", "depth8", "forest"):
            c = accept_case(seed, batch=2, nodes=[1, 5, 12, 33, 64][seed % 5], tree=tree, match=[0.0, 0.5, 0.9][seed % 3])
            n, path, com = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
            for b in range(2):
                ref = _accept_by_enumeration(c.tree_parent[b], c.draft_tokens[b], c.target_tokens[b])
                assert list(path[b, :n[b]]) == ref, (seed, tree, b)
                assert np.all(path[b, n[b]:] == -1)
                toks = [int(c.draft_tokens[b, j]) for j in ref[1:]] + [int(c.target_tokens[b, ref[-1]])]
                assert list(com[b, :n[b]]) == toks and np.all(com[b, n[b]:] == -1)


def test_accept_hand_worked():
    # root 0 -> 1 -> 3, root 0 -> 2 -> 4 -> 5; target after node i is 100 + i
    par = np.array([[-1, 0, 0, 1, 2, 4]], np.int32)
    tgt = np.array([[100, 101, 102, 103, 104, 105]], np.int32)
    # node 1 matches (100), node 3 matches (101), node 2 matches (100), node 4 fails (7 != 102)
    drf = np.array([[9, 100, 100, 101, 7, 104]], np.int32)
    n, path, com = so.tree_accept(par, drf, tgt)
    assert n[0] == 3 and list(path[0, :3]) == [0, 1, 3] and list(com[0, :3]) == [100, 101, 103]
    # make node 4 match too: the branch 0-2-4-5 (depth 3) wins
    drf[0, 4] = 102
    n, path, com = so.tree_accept(par, drf, tgt)
    assert n[0] == 4 and list(path[0, :4]) == [0, 2, 4, 5] and list(com[0, :4]) == [100, 102, 104, 105]
    # equal depths: the smaller end node wins (0-1 vs 0-2 when neither goes deeper)
    drf = np.array([[9, 100, 100, 7, 7, 7]], np.int32)
    n, path, _ = so.tree_accept(par, drf, tgt)
    assert n[0] == 2 and list(path[0, :2]) == [0, 1]


def test_accept_nothing_matches_commits_one_token():
    # verify-kernel page, Part II: avg_commit_len = 1.00 is one token per step
    e = G["avg_commit_len_no_speedup"]
    c = accept_case(3, batch=6, nodes=16, match=0.0)
    n, path, com = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
    assert np.all(n == e["printed"]) and np.all(path[:, 0] == 0)
    assert np.array_equal(com[:, 0], c.target_tokens[:, 0])


def test_accept_chain_stops_at_first_mismatch():
    t = 12
    par = np.arange(-1, t - 1, dtype=np.int32)[None]
    tgt = np.arange(t, dtype=np.int32)[None] + 500
    for k in range(1, t + 1):
        drf = np.concatenate([[0], tgt[0, :-1]])[None].astype(np.int32)  # node i copies target after i-1
        if k < t:
            drf[0, k] = 1  # first mismatch at node k
        n, _, _ = so.tree_accept(par, drf, tgt)
        assert n[0] == k


# ================================================================== KV append and commit

def test_kv_append_writes_exactly_the_named_rows():
    rng = np.random.default_rng(1)
    kv = rng.integers(0, 65535, size=(300, 576), dtype=np.uint16)
    rows = rng.integers(0, 65535, size=(17, 576), dtype=np.uint16)
    loc = rng.choice(300, 17, replace=False).astype(np.int32)
    out = so.kv_append(kv, rows, loc)
    assert np.array_equal(out[loc], rows)
    others = np.setdiff1d(np.arange(300), loc)
    assert np.array_equal(out[others], kv[others])
    with pytest.raises(ValueError):
        so.kv_append(kv, rows[:2], np.array([5, 5], np.int32))


def test_commit_page_table_and_release():
    c = accept_case(5, batch=3, nodes=16, match=0.8, pool=5000, contexts=[1000, 3, 1500])
    n, path, _ = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
    pt, ctx, freed, kv2 = so.commit_accepted(c.page_table, c.seq_lens, 16, n, path)
    assert kv2 is None
    for b in range(3):
        cb = int(c.seq_lens[b]) - 16
        assert ctx[b] == cb + n[b]
        assert np.array_equal(pt[b, :cb], c.page_table[b, :cb])  # the committed prefix is untouched
        tree = c.page_table[b, cb:cb + 16]
        assert list(pt[b, cb:cb + n[b]]) == [int(tree[j]) for j in path[b, :n[b]]]
        rel = freed[b][freed[b] >= 0]
        assert len(rel) == 16 - n[b]
        assert sorted(rel.tolist() + pt[b, cb:cb + n[b]].tolist()) == sorted(tree.tolist())


def test_commit_relocation_moves_rows():
    c = accept_case(6, batch=2, nodes=9, match=0.9, pool=3000, contexts=[100, 57])
    rng = np.random.default_rng(2)
    kv = rng.integers(0, 65535, size=(3000, 576), dtype=np.uint16)
    n, path, _ = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
    used = set(c.page_table[c.page_table >= 0].tolist())
    free = np.array(sorted(set(range(3000)) - used), np.int32)
    dest = np.stack([free[:9], free[9:18]])  # contiguous fresh runs
    pt, ctx, _, kv2 = so.commit_accepted(c.page_table, c.seq_lens, 9, n, path, dest_slots=dest, kv_bits=kv)
    for b in range(2):
        cb = int(c.seq_lens[b]) - 9
        for k in range(n[b]):
            src = int(c.page_table[b, cb + path[b, k]])
            assert pt[b, cb + k] == dest[b, k] and np.array_equal(kv2[dest[b, k]], kv[src])
    touched = set(dest[0, :n[0]].tolist()) | set(dest[1, :n[1]].tolist())
    untouched = np.array(sorted(set(range(3000)) - touched))
    assert np.array_equal(kv2[untouched], kv[untouched])


# ================================================================== sliding-window gather

@pytest.mark.parametrize("w,p", [(4096, 64), (2048, 64), (7, 3), (1, 1), (5, 8), (64, 64)])
def test_window_bound_exhaustive(w, p):
    """The page's claim c(L) <= min(L, W + P - 1), checked over every L up to
    four windows, with the floor identity behind its proof."""
    prev = None
    saw_drop = False
    top = 0
    for length in range(0, 4 * (w + p) + 1):
        s, c = so.window_start(length, w, p), so.compact_len(length, w, p)
        assert s % p == 0 and 0 <= s
        u = length - min(length, w)  # unaligned start
        assert s <= u < s + p
        assert c <= min(length, w + p - 1)
        if length <= w:
            assert s == 0 and c == length
        if prev is not None and c < prev:
            saw_drop = True
        prev = c
        top = max(top, c)
    assert top == (w + p - 1 if p > 1 else w)  # the bound is reached
    if p > 1:
        assert saw_drop  # not monotone: it sawtooths when the aligned start jumps a page


def test_window_map_holds_the_last_tokens():
    tm, lens = window_case(3, batch=8, width=50_000, lo=1, hi=50_000)
    lens[0], lens[1] = 0, 4096 + 63
    w, p = 4096, 64
    dm, cl = so.window_map(tm, lens, w, p)
    for i in range(8):
        c = int(cl[i])
        assert np.array_equal(dm[i, :c], tm[i, lens[i] - c:lens[i]])  # the window is the last c tokens
        assert np.all(dm[i, c:] == -1)
        assert (lens[i] - c) % p == 0
        assert c >= min(lens[i], w)  # the most recent W tokens are all resident


# ================================================================== fp8 decode and indexer logits

def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = so.e4m3_to_f64(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert np.all(same)


def test_e4m3_textbook_values():
    d = so.e4m3_to_f64(np.array([0x38, 0x7E, 0x08, 0x01, 0x07, 0x80, 0xB8, 0x40], np.uint8))
    assert list(d[:5]) == [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9]
    assert d[5] == 0.0 and math.copysign(1, d[5]) < 0 and d[6] == -1.0 and d[7] == 2.0
    assert np.isnan(so.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def test_generated_codes_are_finite():
    codes = e4m3_codes(np.random.default_rng(0), (100_000,))
    assert np.all(np.isfinite(so.e4m3_to_f64(codes)))


def test_indexer_matches_brute_force():
    c = indexer_case(21, batch=2, heads=3, max_blocks=3, seq_lens=[130, 64])
    got = so.indexer_logits(c.q, c.weights, c.blocks, c.block_table, c.seq_lens)
    ref = np.array(so.brute_force_indexer(c.q, c.weights, c.blocks, c.block_table, c.seq_lens))
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


def _indexer_torch(c):
    """The same logits with torch's float8_e4m3fn decoder and library matrix
    products: relu(K Q^T) w * s, per request and page."""
    out = np.full((c.q.shape[0], c.block_table.shape[1] * 64), -np.inf)
    q = torch.from_numpy(c.q.copy()).view(torch.float8_e4m3fn).to(torch.float64)
    for b in range(c.q.shape[0]):
        n = int(c.seq_lens[b])
        for pg in range(-(-n // 64)):
            blk = c.blocks[c.block_table[b, pg]]
            k = torch.from_numpy(blk[:8192].copy()).view(torch.float8_e4m3fn).to(torch.float64).reshape(64, 128)
            s = torch.from_numpy(blk[8192:].copy().view(np.float32).astype(np.float64))
            w = torch.from_numpy(c.weights[b].astype(np.float64))
            v = (torch.relu(k @ q[b].T) @ w) * s
            lo, hi = pg * 64, min(n, pg * 64 + 64)
            out[b, lo:hi] = v[:hi - lo].numpy()
    return out


def test_indexer_matches_torch_decode_and_matmul():
    c = indexer_case(22, batch=3, heads=64, max_blocks=9, seq_lens=[576, 1, 300])
    got = so.indexer_logits(c.q, c.weights, c.blocks, c.block_table, c.seq_lens)
    ref = _indexer_torch(c)
    assert np.array_equal(np.isfinite(got), np.isfinite(ref))
    fin = np.isfinite(ref)
    assert np.allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)
    assert np.all(got[1, 1:] == -np.inf) and np.all(got[2, 300:] == -np.inf)


def test_indexer_zero_query_and_scale_linearity():
    c = indexer_case(23, batch=1, heads=8, max_blocks=4, seq_lens=[200])
    z = so.indexer_logits(np.zeros_like(c.q), c.weights, c.blocks, c.block_table, c.seq_lens)
    assert np.all(z[0, :200] == 0) and np.all(z[0, 200:] == -np.inf)
    blocks2 = c.blocks.copy()
    sc = blocks2[:, 8192:].copy().view(np.float32) * 2
    blocks2[:, 8192:] = sc.view(np.uint8)
    a = so.indexer_logits(c.q, c.weights, c.blocks, c.block_table, c.seq_lens)
    b = so.indexer_logits(c.q, c.weights, blocks2, c.block_table, c.seq_lens)
    assert np.array_equal(b[0, :200], 2 * a[0, :200])


def test_indexer_joint_block_permutation():
    c = indexer_case(24, batch=2, heads=4, max_blocks=5, seq_lens=[320, 129])
    a = so.indexer_logits(c.q, c.weights, c.blocks, c.block_table, c.seq_lens)
    pi = np.random.default_rng(1).permutation(c.blocks.shape[0])
    blocks2 = np.empty_like(c.blocks)
    blocks2[pi] = c.blocks
    bt2 = np.where(c.block_table >= 0, pi[np.maximum(c.block_table, 0)], -1).astype(np.int32)
    b = so.indexer_logits(c.q, c.weights, blocks2, bt2, c.seq_lens)
    assert np.array_equal(a, b)


def test_indexer_magnitude_bounds_every_logit():
    """The error scale the GPU indexer check is measured against,
    sum_h |w_h| sum_d |q_hd k_pd| s_p, must never fall below |logit|: a
    magnitude that came out too small would tighten that check, one that came
    out too large would loosen it. Pinned three ways: it bounds |logit| at every
    position (the triangle inequality through the ReLU); it equals the logit
    when every q, k and w is non-negative (no cancellation, the ReLU passes all);
    and it equals the scalar brute force run on the absolute values (codes with
    the sign bit cleared, |w|), which decodes each byte from its bit fields."""
    c = indexer_case(25, batch=2, heads=6, max_blocks=3, seq_lens=[150, 64])
    args = (c.weights, c.blocks, c.block_table, c.seq_lens)
    lg = so.indexer_logits(c.q, *args)
    mag = so.indexer_magnitude(c.q, *args)
    fin = np.isfinite(lg)
    assert np.all(mag[fin] >= np.abs(lg[fin]) * (1 - 1e-12))
    assert np.any(mag[fin] > 2 * np.abs(lg[fin]))  # cancellation does occur in the signed case
    assert np.all(mag[~fin] == 0)
    # non-negative inputs: the magnitude is the logit itself
    blocks_pos = c.blocks.copy()
    blocks_pos[:, :8192] &= 0x7F
    q_pos, w_pos = c.q & 0x7F, np.abs(c.weights)
    lg_pos = so.indexer_logits(q_pos, w_pos, blocks_pos, c.block_table, c.seq_lens)
    mag_pos = so.indexer_magnitude(q_pos, w_pos, blocks_pos, c.block_table, c.seq_lens)
    assert np.allclose(mag_pos[fin], lg_pos[fin], rtol=1e-12, atol=0)
    # and the scalar brute force on the absolute values
    small = indexer_case(26, batch=1, heads=3, max_blocks=2, seq_lens=[70])
    sb = small.blocks.copy()
    sb[:, :8192] &= 0x7F
    ref = np.array(so.brute_force_indexer(small.q & 0x7F, np.abs(small.weights), sb, small.block_table,
                                          small.seq_lens))
    got = so.indexer_magnitude(small.q, small.weights, small.blocks, small.block_table, small.seq_lens)
    assert np.allclose(got[0, :70], ref[0, :70], rtol=1e-12, atol=0)


def test_commit_freed_slots_hand_worked():
    """The release list of the commit, worked by hand: the tree slots of the
    nodes off the accepted path, in node order, then -1 (with or without
    relocation, which moves the accepted rows and leaves their old slots to the
    caller, who named the destinations)."""
    # context slots 10, 11, 12; tree nodes 0..4 on slots 20..24; parents -1, 0, 0, 1, 3
    pt = np.array([[10, 11, 12, 20, 21, 22, 23, 24, -1]], np.int32)
    sl = np.array([8], np.int32)
    cases = [
        (3, [0, 1, 3], [20, 21, 23], [22, 24, -1, -1, -1]),
        (2, [0, 2], [20, 22], [21, 23, 24, -1, -1]),
        (1, [0], [20], [21, 22, 23, 24, -1]),
        (4, [0, 1, 3, 4], [20, 21, 23, 24], [22, -1, -1, -1, -1]),
    ]
    for n_acc, chain, new_slots, freed_want in cases:
        path = np.array([chain + [-1] * (5 - n_acc)], np.int32)
        out_pt, ctx, freed, kv2 = so.commit_accepted(pt, sl, 5, np.array([n_acc], np.int32), path)
        assert ctx[0] == 3 + n_acc and kv2 is None
        assert out_pt[0, :3].tolist() == [10, 11, 12]
        assert out_pt[0, 3:3 + n_acc].tolist() == new_slots
        assert freed[0].tolist() == freed_want
        kv = np.arange(60 * 576, dtype=np.uint16).reshape(60, 576)
        dest = np.array([[40, 41, 42, 43, 44]], np.int32)
        out_pt, _, freed_r, kv_r = so.commit_accepted(pt, sl, 5, np.array([n_acc], np.int32), path,
                                                      dest_slots=dest, kv_bits=kv)
        assert out_pt[0, 3:3 + n_acc].tolist() == [40 + k for k in range(n_acc)]
        assert freed_r[0].tolist() == freed_want
        for k, s in enumerate(new_slots):
            assert np.array_equal(kv_r[40 + k], kv[s])


# ================================================================== planted mistakes

def _plant_decode_bias(monkeypatch):
    orig = so.e4m3_to_f64
    monkeypatch.setattr(so, "e4m3_to_f64", lambda codes: orig(codes) * 0.5)  # exponent bias 8


def _plant_no_relu(monkeypatch):
    def mutant(q_codes, weights, blocks, block_table, seq_lens):
        # the definition with the ReLU left out
        q = so.e4m3_to_f64(q_codes)
        out = np.full((q.shape[0], block_table.shape[1] * 64), -np.inf)
        for b in range(q.shape[0]):
            n = int(seq_lens[b])
            for pg in range(-(-n // 64)):
                codes, scales = so.indexer_block_fields(blocks[int(block_table[b, pg])])
                val = (so.e4m3_to_f64(codes) @ q[b].T) @ np.asarray(weights[b], np.float64) * scales
                lo, hi = pg * 64, min(n, pg * 64 + 64)
                out[b, lo:hi] = val[:hi - lo]
        return out
    monkeypatch.setattr(so, "indexer_logits", mutant)


def _plant_accept_own_target(monkeypatch):
    def wrong(tree_parent, draft_tokens, target_tokens):
        # compares a node's draft with the target's choice after the node itself
        par = np.asarray(tree_parent)
        shifted = np.array(target_tokens, copy=True)
        for b in range(par.shape[0]):
            for i in range(par.shape[1]):
                if par[b, i] >= 0:
                    shifted[b, par[b, i]] = target_tokens[b, i]
        return ORIG_ACCEPT(tree_parent, draft_tokens, shifted)
    monkeypatch.setattr(so, "tree_accept", wrong)


def _plant_magnitude_signed_weights(monkeypatch):
    monkeypatch.setattr(so, "indexer_magnitude", _magnitude_signed)


def _magnitude_signed(q_codes, weights, blocks, block_table, seq_lens):
    # the magnitude with the weights' signs kept (|q k| summed, w signed)
    q = np.abs(so.e4m3_to_f64(q_codes))
    w = np.asarray(weights, dtype=np.float64)
    out = np.zeros((q.shape[0], block_table.shape[1] * 64))
    for b in range(q.shape[0]):
        n = int(seq_lens[b])
        for pg in range(-(-n // 64)):
            codes, scales = so.indexer_block_fields(blocks[int(block_table[b, pg])])
            mag = (np.abs(so.e4m3_to_f64(codes)) @ q[b].T) @ w[b] * np.abs(scales)
            lo, hi = pg * 64, min(n, pg * 64 + 64)
            out[b, lo:hi] = mag[:hi - lo]
    return out


def _plant_window_ceil(monkeypatch):
    monkeypatch.setattr(so, "window_start",
                        lambda length, w, p: -(-(length - min(length, w)) // p) * p)


ORIG_ACCEPT = so.tree_accept
PINS = {
    _plant_decode_bias: [test_e4m3_decode_matches_torch_for_every_code, test_e4m3_textbook_values],
    _plant_no_relu: [test_indexer_matches_torch_decode_and_matmul],
    _plant_accept_own_target: [test_accept_matches_enumeration, test_accept_hand_worked],
    _plant_window_ceil: [lambda: test_window_bound_exhaustive(4096, 64), test_window_map_holds_the_last_tokens],
    _plant_magnitude_signed_weights: [test_indexer_magnitude_bounds_every_logit],
}


@pytest.mark.parametrize("plant", list(PINS), ids=lambda f: f.__name__)
def test_pins_detect_planted_mistakes(plant, monkeypatch):
    plant(monkeypatch)
    for pin in PINS[plant]:
        with pytest.raises(AssertionError):
            pin()

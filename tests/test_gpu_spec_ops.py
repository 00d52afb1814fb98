"""GPU parity of the steps next to the verify attention, through the C ABI,
against the CPU oracle (oracle/spec_ops_oracle.py).

Integer and byte work (append, accept, commit, window map) must match bit for
bit. Sparse decode: out max-abs <= 1e-2, lse max-abs <= 1e-3 (the verify
tolerances; one bf16 ulp where |out| >= 4). Indexer logits: fp32 accumulation
of exact fp8 products; the tolerance is derived from the terms' magnitude
(2e-6 x sum_h |w_h| sum_d |q_hd k_pd| s_p, about 32 fp32 roundings of the
largest term), and -inf positions must be -inf exactly."""

import numpy as np
import pytest
import torch

import oracle.spec_ops_oracle as so
import speculative_decoding_mla_amd as mv
from oracle import bf16_bits_to_f64
from workloads.gen import f32_to_bf16_bits
from workloads.ops_gen import IndexerCase, accept_case, indexer_case, sparse_case, window_case
from tests.gpu_util import LSE_TOL, OUT_TOL, bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mv.load_library()


def _t(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda() if dtype is None else \
        torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def _err():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


# ================================================================== sparse top-k decode

def run_sparse(c, nsplit=None, use_lens=True):
    q, kv = bf16(c.q).cuda(), bf16(c.kv).cuda()
    idx = _t(c.indices.astype(np.int32))
    lens = _t(c.lens.astype(np.int32)) if use_lens else None
    b, h, _ = c.q.shape
    out = torch.empty((b, h, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, h), dtype=torch.float32, device="cuda")
    ns = nsplit or c.nsplit
    ws = mv.alloc_sparse_workspace(mv.sparse_desc(q, kv, idx, nsplit=ns, sm_scale=c.sm_scale))
    mv.sparse_decode(q, kv, idx, lens, out, lse, ws, nsplit=ns, sm_scale=c.sm_scale)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy(), mv.device_error(ws)


def check_sparse(c, out_bits, lse, label):
    ro, rl = so.sparse_decode(c.q, c.kv, c.indices, c.lens, c.sm_scale)
    o = bf16_bits_to_f64(out_bits)
    ulp = np.where(np.abs(ro) >= 4, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ro), 1e-30))) - 7), 0)
    assert np.all(np.abs(o - ro) <= np.maximum(OUT_TOL, ulp)), (label, float(np.abs(o - ro).max()))
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse)), label
    assert np.all(np.abs(lse[fin] - rl[fin]) <= LSE_TOL), (label, float(np.abs(lse[fin] - rl[fin]).max()))
    assert np.all(o[~fin] == 0), label


SPARSE = [
    dict(seed=601, batch=1, heads=64, topk=512, nsplit=16),           # the page's shape
    dict(seed=602, batch=16, heads=64, topk=512, nsplit=8),           # concurrency 16, split 8
    dict(seed=603, batch=3, heads=64, topk=512, nsplit=7, lens=[512, 100, 1], holes=0.1),
    dict(seed=604, batch=2, heads=5, topk=97, nsplit=3, lens=[97, 0]),  # ragged heads, an empty list
    dict(seed=605, batch=1, heads=128, topk=2048, nsplit=64, holes=0.5),
]


@pytest.mark.parametrize("spec", SPARSE, ids=lambda s: f"seed{s['seed']}")
def test_sparse_decode_parity(spec):
    spec = dict(spec)
    spec.setdefault("pool", 60_000)
    c = sparse_case(**spec)
    say(f"sparse decode {spec}")
    out, lse, err = run_sparse(c)
    assert err == 0  # -1 entries are unused, not errors
    check_sparse(c, out, lse, str(spec))


def test_sparse_decode_nsplit_and_no_lens():
    c = sparse_case(606, batch=2, heads=64, topk=512, pool=30_000)
    for ns in (1, 8, 32, 512, 600):
        out, lse, err = run_sparse(c, nsplit=ns, use_lens=ns % 2 == 0)
        assert err == 0
        check_sparse(c, out, lse, f"nsplit {ns}")


def test_sparse_decode_hot_key_exact():
    """Integer-valued inputs: one listed slot's score exceeds every other by a
    margin that makes all other weights underflow: out is exactly its V row."""
    c = sparse_case(607, batch=1, heads=64, topk=512, pool=4000)
    kv = np.zeros((4000, 576), np.float32)
    kv[:, 0] = np.arange(4000) % 256 + 1
    kv[:, 1] = np.arange(4000) // 256 + 1
    hot = int(c.indices[0, 333])
    kv[hot, 512:] = 16.0
    q = np.zeros(c.q.shape, np.float32)
    q[..., 512:] = 1.0
    c2 = c.__class__(f32_to_bf16_bits(q), f32_to_bf16_bits(kv), c.indices, c.lens, c.sm_scale, c.nsplit)
    out, lse, err = run_sparse(c2)
    o = bf16_bits_to_f64(out)
    assert np.all(o[..., 0] == hot % 256 + 1) and np.all(o[..., 1] == hot // 256 + 1) and np.all(o[..., 2:] == 0)


def test_sparse_decode_unused_entries_are_inert():
    """Unused (-1) entries and the padding past each list's length enter the
    products as exact zeros: with slot 0 and every row no list names set to
    NaN or an infinity, the output is finite and equals the oracle's."""
    c = sparse_case(611, batch=3, heads=64, topk=256, pool=4000, lens=[256, 77, 5], holes=0.3, nsplit=8)
    named = set(c.indices[c.indices >= 0].tolist())
    if 0 in named:  # keep slot 0 unnamed
        free = min(set(range(4000)) - named)
        c.kv[free] = c.kv[0]
        c.indices[c.indices == 0] = free
        named = set(c.indices[c.indices >= 0].tolist())
    poison = np.array([0x7FC0, 0x7F80, 0xFF80], np.uint16)
    for i, r in enumerate(sorted(set(range(4000)) - named)):
        c.kv[r] = poison[i % 3]
    say("sparse decode with non-finite unnamed rows")
    out, lse, err = run_sparse(c)
    assert err == 0
    assert np.all(np.isfinite(bf16_bits_to_f64(out))) and np.all(np.isfinite(lse))
    check_sparse(c, out, lse, "inert unused entries")


def test_sparse_decode_out_of_pool_slot_flagged():
    c = sparse_case(608, batch=1, heads=64, topk=64, pool=1000)
    bad = c.indices.copy()
    bad[0, 5] = 1000 + 7
    out, lse, err = run_sparse(c.__class__(c.q, c.kv, bad, c.lens, c.sm_scale, 4))
    assert err & mv.DEVERR_SLOT_RANGE
    ref = c.indices.copy()
    ref[0, 5] = -1
    check_sparse(c.__class__(c.q, c.kv, ref, c.lens, c.sm_scale, 4), out, lse, "masked slot")


# ================================================================== KV append

def test_kv_append_bit_exact():
    rng = np.random.default_rng(11)
    for n, slots, stride in [(1, 50, 576), (12 * 8, 5000, 576), (64, 3000, 640), (1000, 200_000, 576)]:
        kv = rng.integers(0, 65535, size=(slots, stride), dtype=np.uint16)
        rows = rng.integers(0, 65535, size=(n, 576), dtype=np.uint16)
        loc = rng.choice(slots, n, replace=False).astype(np.int32)
        kv_t = bf16(kv).cuda()
        err = _err()
        mv.kv_append(kv_t, bf16(rows).cuda(), _t(loc), err)
        torch.cuda.synchronize()
        got = kv_t.view(torch.int16).cpu().numpy().view(np.uint16)
        want = kv.copy()
        want[:, :576] = so.kv_append(kv[:, :576], rows, loc)
        assert np.array_equal(got, want) and int(err.item()) == 0, (n, slots, stride)


def test_kv_append_bad_slot_skipped_and_flagged():
    rng = np.random.default_rng(12)
    kv = rng.integers(0, 65535, size=(100, 576), dtype=np.uint16)
    rows = rng.integers(0, 65535, size=(3, 576), dtype=np.uint16)
    loc = np.array([4, 100, -2], np.int32)
    kv_t = bf16(kv).cuda()
    err = _err()
    mv.kv_append(kv_t, bf16(rows).cuda(), _t(loc), err)
    torch.cuda.synchronize()
    want = kv.copy()
    want[4] = rows[0]
    assert np.array_equal(kv_t.view(torch.int16).cpu().numpy().view(np.uint16), want)
    assert int(err.item()) & mv.DEVERR_SLOT_RANGE


# ================================================================== tree accept

def run_accept(c):
    b, t = c.tree_parent.shape
    n = torch.empty(b, dtype=torch.int32, device="cuda")
    path = torch.empty((b, t), dtype=torch.int32, device="cuda")
    com = torch.empty((b, t), dtype=torch.int32, device="cuda")
    err = _err()
    mv.tree_accept(_t(c.tree_parent), _t(c.draft_tokens), _t(c.target_tokens), n, path, com, err)
    torch.cuda.synchronize()
    return n.cpu().numpy(), path.cpu().numpy(), com.cpu().numpy(), int(err.item())


@pytest.mark.parametrize("tree", ["uniform", "chain", "depth8", "forest"])
def test_tree_accept_bit_exact(tree):
    for seed, t, match in [(1, 1, 0.5), (2, 9, 0.9), (3, 12, 1.0), (4, 16, 0.0), (5, 32, 0.85), (6, 63, 0.7),
                           (7, 64, 0.95), (8, 64, 1.0)]:
        c = accept_case(seed * 13, batch=8, nodes=t, tree=tree, match=match, pool=60_000)
        n, path, com, err = run_accept(c)
        rn, rp, rc = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
        assert err == 0
        assert np.array_equal(n, rn) and np.array_equal(path, rp) and np.array_equal(com, rc), (tree, seed, t)


def test_tree_accept_bad_parent_is_root():
    c = accept_case(77, batch=2, nodes=10, match=1.0, pool=20_000)
    par = c.tree_parent.copy()
    par[1, 6] = 8  # not an earlier node
    c2 = c.__class__(par, c.draft_tokens, c.target_tokens, c.page_table, c.seq_lens, c.num_slots)
    n, path, com, err = run_accept(c2)
    assert err & mv.DEVERR_BAD_PARENT
    par[1, 6] = -1
    rn, rp, rc = so.tree_accept(par, c.draft_tokens, c.target_tokens)
    assert np.array_equal(n, rn) and np.array_equal(path, rp) and np.array_equal(com, rc)


# ================================================================== commit (and relocation)

def run_commit(c, n, path, dest=None, kv=None):
    b, t = c.tree_parent.shape
    pt = _t(c.page_table)
    ctx = torch.empty(b, dtype=torch.int32, device="cuda")
    freed = torch.empty((b, t), dtype=torch.int32, device="cuda")
    kv_t = None if kv is None else bf16(kv).cuda()
    err = _err()
    mv.commit_accepted(pt, _t(c.seq_lens), t, _t(n), _t(path), ctx, freed, kv_t,
                       None if dest is None else _t(dest), err)
    torch.cuda.synchronize()
    kv_out = None if kv is None else kv_t.view(torch.int16).cpu().numpy().view(np.uint16)
    return pt.cpu().numpy(), ctx.cpu().numpy(), freed.cpu().numpy(), kv_out, int(err.item())


def test_commit_bit_exact():
    for seed, t in [(1, 1), (2, 9), (3, 16), (4, 32), (5, 64)]:
        c = accept_case(seed * 7, batch=6, nodes=t, match=0.8, pool=100_000)
        n, path, _ = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
        pt, ctx, freed, _, err = run_commit(c, n, path)
        rpt, rctx, rfreed, _ = so.commit_accepted(c.page_table, c.seq_lens, t, n, path)
        assert err == 0
        assert np.array_equal(pt, rpt) and np.array_equal(ctx, rctx) and np.array_equal(freed, rfreed), (seed, t)


def test_commit_relocation_bit_exact():
    rng = np.random.default_rng(5)
    for seed, t, overlap in [(1, 9, False), (2, 32, False), (3, 64, True), (4, 16, True)]:
        c = accept_case(seed * 31, batch=4, nodes=t, match=0.9, pool=30_000, contexts=[500, 9, 1200, 77])
        kv = rng.integers(0, 65535, size=(30_000, 576), dtype=np.uint16)
        n, path, _ = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
        if overlap:
            # compact in place: the request's own tree slots, sorted, are the destinations
            dest = np.stack([np.sort(c.page_table[b, c.seq_lens[b] - t:c.seq_lens[b]]) for b in range(4)]).astype(np.int32)
        else:
            used = set(c.page_table[c.page_table >= 0].tolist())
            free = np.array(sorted(set(range(30_000)) - used), np.int32)
            dest = free[:4 * t].reshape(4, t)
        pt, ctx, freed, kv_out, err = run_commit(c, n, path, dest, kv)
        rpt, rctx, rfreed, rkv = so.commit_accepted(c.page_table, c.seq_lens, t, n, path, dest_slots=dest, kv_bits=kv)
        assert err == 0
        assert np.array_equal(pt, rpt) and np.array_equal(ctx, rctx) and np.array_equal(freed, rfreed)
        assert np.array_equal(kv_out, rkv), (seed, t, overlap)


def test_commit_clamps_and_flags():
    c = accept_case(91, batch=2, nodes=8, match=0.9, pool=20_000, contexts=[40, 50])
    n, path, _ = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
    bad_n = n.copy()
    bad_n[0] = 99  # clamped to T
    bad_path = path.copy()
    bad_path[0, :] = np.arange(8)
    bad_path[0, 0] = 0
    pt, ctx, freed, _, err = run_commit(c, bad_n, bad_path)
    assert err & mv.DEVERR_INDEX_RANGE
    assert ctx[0] == c.seq_lens[0] - 8 + 8 and ctx[1] == c.seq_lens[1] - 8 + n[1]


# ================================================================== accept and commit in one launch

def run_accept_commit(c, dest=None, kv=None, with_commit=True, seq_lens=None, parents=None):
    b, t = c.tree_parent.shape
    pt = _t(c.page_table)
    n = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    path = torch.full((b, t), -7, dtype=torch.int32, device="cuda")
    com = torch.full((b, t), -7, dtype=torch.int32, device="cuda") if with_commit else None
    ctx = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    freed = torch.full((b, t), -7, dtype=torch.int32, device="cuda")
    kv_t = None if kv is None else bf16(kv).cuda()
    err = _err()
    mv.accept_commit(_t(c.tree_parent if parents is None else parents), _t(c.draft_tokens), _t(c.target_tokens), pt,
                     _t(c.seq_lens if seq_lens is None else seq_lens), n, path, ctx, com, freed, kv_t,
                     None if dest is None else _t(dest), err)
    torch.cuda.synchronize()
    kv_out = None if kv is None else kv_t.view(torch.int16).cpu().numpy().view(np.uint16)
    return (n.cpu().numpy(), path.cpu().numpy(), None if com is None else com.cpu().numpy(), pt.cpu().numpy(),
            ctx.cpu().numpy(), freed.cpu().numpy(), kv_out, int(err.item()))


@pytest.mark.parametrize("tree", ["uniform", "chain", "depth8", "forest"])
def test_accept_commit_matches_oracle(tree):
    """One launch equals the oracle's accept followed by its commit."""
    for seed, t, match in [(1, 1, 0.5), (2, 9, 0.9), (3, 16, 0.0), (4, 32, 0.85), (5, 63, 0.7), (6, 64, 1.0)]:
        c = accept_case(seed * 17, batch=6, nodes=t, tree=tree, match=match, pool=100_000)
        say(f"accept_commit tree={tree} seed={seed} T={t}")
        n, path, com, pt, ctx, freed, _, err = run_accept_commit(c)
        rn, rp, rc = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
        rpt, rctx, rfreed, _ = so.commit_accepted(c.page_table, c.seq_lens, t, rn, rp)
        assert err == 0
        assert np.array_equal(n, rn) and np.array_equal(path, rp) and np.array_equal(com, rc), (tree, seed, t)
        assert np.array_equal(pt, rpt) and np.array_equal(ctx, rctx) and np.array_equal(freed, rfreed), (tree, seed, t)


def test_accept_commit_relocation_matches_oracle():
    rng = np.random.default_rng(9)
    for seed, t, overlap in [(1, 9, False), (2, 64, True), (3, 32, False), (4, 16, True)]:
        c = accept_case(seed * 29, batch=4, nodes=t, match=0.9, pool=30_000, contexts=[500, 9, 1200, 77])
        kv = rng.integers(0, 65535, size=(30_000, 576), dtype=np.uint16)
        if overlap:
            dest = np.stack([np.sort(c.page_table[b, c.seq_lens[b] - t:c.seq_lens[b]]) for b in range(4)]).astype(np.int32)
        else:
            used = set(c.page_table[c.page_table >= 0].tolist())
            free = np.array(sorted(set(range(30_000)) - used), np.int32)
            dest = free[:4 * t].reshape(4, t)
        say(f"accept_commit relocation seed={seed} T={t} overlap={overlap}")
        n, path, com, pt, ctx, freed, kv_out, err = run_accept_commit(c, dest, kv, with_commit=False)
        rn, rp, _ = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
        rpt, rctx, rfreed, rkv = so.commit_accepted(c.page_table, c.seq_lens, t, rn, rp, dest_slots=dest, kv_bits=kv)
        assert err == 0
        assert np.array_equal(n, rn) and np.array_equal(path, rp)
        assert np.array_equal(pt, rpt) and np.array_equal(ctx, rctx) and np.array_equal(freed, rfreed)
        assert np.array_equal(kv_out, rkv), (seed, t, overlap)


def test_accept_commit_flags():
    c = accept_case(92, batch=2, nodes=10, match=1.0, pool=20_000, contexts=[40, 50])
    # a parent that is not an earlier node is read as a root
    par = c.tree_parent.copy()
    par[1, 6] = 8
    n, path, com, pt, ctx, freed, _, err = run_accept_commit(c, parents=par)
    assert err & mv.DEVERR_BAD_PARENT
    par[1, 6] = -1
    rn, rp, rc = so.tree_accept(par, c.draft_tokens, c.target_tokens)
    rpt, rctx, rfreed, _ = so.commit_accepted(c.page_table, c.seq_lens, 10, rn, rp)
    assert np.array_equal(n, rn) and np.array_equal(path, rp) and np.array_equal(com, rc)
    assert np.array_equal(pt, rpt) and np.array_equal(ctx, rctx) and np.array_equal(freed, rfreed)
    # a length below T is clamped to T (first committed position 0)
    sl = c.seq_lens.copy()
    sl[0] = 3
    n, path, com, pt, ctx, freed, _, err = run_accept_commit(c, seq_lens=sl)
    assert err & mv.DEVERR_INDEX_RANGE
    assert ctx[0] == n[0] and ctx[1] == c.seq_lens[1] - 10 + n[1]


# ================================================================== sliding-window map

def test_window_map_bit_exact():
    for seed, (w, p) in enumerate([(4096, 64), (2048, 64), (512, 16), (7, 3), (1, 1)]):
        tm, lens = window_case(seed, batch=8, width=20_000, lo=1, hi=20_000)
        edge = [0, w, w + p - 1, w + p, min(20_000, 3 * w + 1)]
        lens[:len(edge)] = edge
        dm = torch.full((8, w + p - 1), 7, dtype=torch.int32, device="cuda")
        cl = torch.empty(8, dtype=torch.int32, device="cuda")
        err = _err()
        mv.window_map(_t(tm), _t(lens), w, p, dm, cl, err)
        torch.cuda.synchronize()
        rdm, rcl = so.window_map(tm, lens, w, p)
        assert np.array_equal(dm.cpu().numpy(), rdm) and np.array_equal(cl.cpu().numpy(), rcl), (w, p)
        assert int(err.item()) == 0
        assert np.all(rcl <= np.minimum(lens, w + p - 1))


def test_window_map_clamps_long_length():
    tm, lens = window_case(9, batch=2, width=5000, lens=[100, 100])
    lens = np.array([6000, -3], np.int32)  # past the map, negative
    dm = torch.empty((2, 4096 + 63), dtype=torch.int32, device="cuda")
    err = _err()
    mv.window_map(_t(tm), _t(lens), 4096, 64, dm, None, err)
    torch.cuda.synchronize()
    rdm, _ = so.window_map(tm, np.array([5000, 0], np.int32), 4096, 64)
    assert np.array_equal(dm.cpu().numpy(), rdm) and int(err.item()) & mv.DEVERR_SEQ_LEN


# ================================================================== fp8 indexer logits

def run_indexer(c):
    b = c.q.shape[0]
    m = c.block_table.shape[1]
    logits = torch.full((b, m * 64), 12345.0, dtype=torch.float32, device="cuda")
    err = _err()
    mv.indexer_logits(_t(c.q), _t(c.weights), _t(c.blocks), _t(c.block_table), _t(c.seq_lens), logits, err)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), int(err.item())


def check_indexer(c, got, label):
    ref = so.indexer_logits(c.q, c.weights, c.blocks, c.block_table, c.seq_lens)
    mag = so.indexer_magnitude(c.q, c.weights, c.blocks, c.block_table, c.seq_lens)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)) and np.all(got[~fin] == -np.inf), label
    err = np.abs(got[fin] - ref[fin])
    assert np.all(err <= 2e-6 * mag[fin] + 1e-30), (label, float((err / np.maximum(mag[fin], 1e-30)).max()))


INDEXER = [
    dict(seed=701, batch=1, heads=64, max_blocks=16, seq_lens=[1000]),
    dict(seed=702, batch=4, heads=64, max_blocks=40, seq_lens=[2560, 1, 0, 1777]),
    dict(seed=703, batch=2, heads=7, max_blocks=3, seq_lens=[130, 64]),
    dict(seed=704, batch=3, heads=33, max_blocks=9, seq_lens=[576, 575, 65]),
]


@pytest.mark.parametrize("spec", INDEXER, ids=lambda s: f"seed{s['seed']}")
def test_indexer_parity(spec):
    c = indexer_case(**spec)
    say(f"indexer {spec}")
    got, err = run_indexer(c)
    assert err == 0
    check_indexer(c, got, str(spec))


def test_indexer_widens_every_e4m3_code_exactly():
    """gfx950's fp8 -> bf16 widening inside the indexer, over all 256 E4M3 codes
    against torch's float8_e4m3fn decoder. Code c sits at position c of a
    256-position request (block c // 64, row c % 64), dimension 0, all other
    dimensions +0; head 0's query is +1 there with weight +1, head 1's is -1
    with weight -1, every scale is 1. Every product and sum is then exact in
    fp32 and logit = relu(d) - relu(-d) = d for each finite code d. The two NaN
    codes are outside the workloads' domain (the generator never draws them):
    they must not come out as finite values other than 0."""
    codes = np.arange(256, dtype=np.uint8)
    pos = np.arange(256, dtype=np.int64)  # (index arithmetic in uint8 would wrap)
    blocks = np.zeros((4, 8448), np.uint8)
    blocks[pos // 64, (pos % 64) * 128] = codes
    blocks[:, 8192:] = np.ones((4, 64), np.float32).view(np.uint8)
    q = np.zeros((1, 2, 128), np.uint8)
    q[0, 0, 0], q[0, 1, 0] = 0x38, 0xB8  # +1.0, -1.0
    c = IndexerCase(q=q, weights=np.array([[1.0, -1.0]], np.float32), blocks=blocks,
                    block_table=np.array([[0, 1, 2, 3]], np.int32), seq_lens=np.array([256], np.int32))
    say("indexer: all 256 e4m3 codes")
    got, err = run_indexer(c)
    assert err == 0
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    assert fin.sum() == 254
    assert np.array_equal(got[0, fin], ref[fin]), np.nonzero(got[0, fin] != ref[fin])
    assert np.all(np.isnan(got[0, ~fin]) | (got[0, ~fin] == 0))


def test_indexer_full_table():
    """The page's whole table: 4,097 blocks = 262,208 positions for one request,
    and a request at 32,768 positions (128K tokens at four per position)."""
    c = indexer_case(705, batch=2, heads=64, max_blocks=4097, seq_lens=[262_208, 32_768])
    say("indexer full table")
    got, err = run_indexer(c)
    assert err == 0
    check_indexer(c, got, "full table")


def test_indexer_runs_cross_requests():
    """Persistent waves take runs of consecutive half-blocks (at least 1,024
    waves): 3 x 701 blocks = 4,206 half-blocks give runs of 5 that start and
    end inside requests (1,402 and 2,804 are not multiples of 5), so a wave
    switches requests mid-run, after half-blocks past a length, and with
    48 heads (rows past the count are zero)."""
    c = indexer_case(707, batch=3, heads=48, max_blocks=701, seq_lens=[44_800, 44_864, 3_001])
    units = 3 * 701 * 2
    per = -(-units // 1024)
    assert per > 3 and (701 * 2) % per != 0 and (2 * 701 * 2) % per != 0
    say("indexer runs across requests")
    got, err = run_indexer(c)
    assert err == 0
    check_indexer(c, got, "runs across requests")


def test_indexer_bad_block_flagged():
    c = indexer_case(706, batch=1, heads=64, max_blocks=4, seq_lens=[256])
    bt = c.block_table.copy()
    bt[0, 2] = c.blocks.shape[0] + 3
    c2 = c.__class__(c.q, c.weights, c.blocks, bt, c.seq_lens)
    got, err = run_indexer(c2)
    assert err & mv.DEVERR_SLOT_RANGE
    assert np.all(got[0, 128:192] == -np.inf)
    ref = so.indexer_logits(c.q, c.weights, c.blocks, c.block_table, c.seq_lens)
    keep = np.r_[0:128, 192:256]
    mag = so.indexer_magnitude(c.q, c.weights, c.blocks, c.block_table, c.seq_lens)
    assert np.all(np.abs(got[0, keep] - ref[0, keep]) <= 2e-6 * mag[0, keep] + 1e-30)


# ================================================================== capture of the step around verify

@pytest.mark.parametrize("fused", [False, True])
def test_append_accept_commit_graph_replays(fused):
    """KV append -> tree accept -> commit (two launches, or one with fused)
    captured in one hipGraph; every replay (fresh inputs copied in by kernels
    inside the graph, eager work and synchronisations between replays) matches
    the oracle bit for bit."""
    t, b = 16, 4
    c = accept_case(808, batch=b, nodes=t, match=0.85, pool=40_000, contexts=[300, 4000, 17, 999])
    rng = np.random.default_rng(8)
    kv0 = rng.integers(0, 65535, size=(40_000, 576), dtype=np.uint16)
    rows = rng.integers(0, 65535, size=(b * t, 576), dtype=np.uint16)
    loc = np.concatenate([c.page_table[i, c.seq_lens[i] - t:c.seq_lens[i]] for i in range(b)]).astype(np.int32)
    pt0 = _t(c.page_table)
    kv0_t = bf16(kv0).cuda()
    kv = kv0_t.clone()
    pt = pt0.clone()
    rows_t, loc_t = bf16(rows).cuda(), _t(loc)
    par, drf, tgt, sl = _t(c.tree_parent), _t(c.draft_tokens), _t(c.target_tokens), _t(c.seq_lens)
    n = torch.empty(b, dtype=torch.int32, device="cuda")
    path = torch.empty((b, t), dtype=torch.int32, device="cuda")
    ctx = torch.empty(b, dtype=torch.int32, device="cuda")
    freed = torch.empty((b, t), dtype=torch.int32, device="cuda")

    def step():
        kv.copy_(kv0_t)
        pt.copy_(pt0)
        mv.kv_append(kv, rows_t, loc_t)
        if fused:
            mv.accept_commit(par, drf, tgt, pt, sl, n, path, ctx, None, freed)
        else:
            mv.tree_accept(par, drf, tgt, n, path)
            mv.commit_accepted(pt, sl, t, n, path, ctx, freed)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="global"):
        step()
    kv_ref = kv0.copy()
    kv_ref[loc] = rows
    rn, rp, _ = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
    rpt, rctx, rfreed, _ = so.commit_accepted(c.page_table, c.seq_lens, t, rn, rp)
    for r in range(3):
        pt.fill_(-5)
        n.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(kv.view(torch.int16).cpu().numpy().view(np.uint16), kv_ref), r
        assert np.array_equal(n.cpu().numpy(), rn) and np.array_equal(path.cpu().numpy(), rp), r
        assert np.array_equal(pt.cpu().numpy(), rpt) and np.array_equal(ctx.cpu().numpy(), rctx), r
        assert np.array_equal(freed.cpu().numpy(), rfreed), r

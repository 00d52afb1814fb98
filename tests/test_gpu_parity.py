"""GPU parity of the HIP verify path against the CPU oracle, through the C ABI.

Tolerances: out max-abs <= 1e-2 (one bf16 ulp where |out| >= 4), lse max-abs
<= 1e-3; mask bits and index probes bit-exact."""

import numpy as np
import pytest
import torch

import speculative_decoding_mla_amd as mv
from oracle import ancestor_mask, ancestor_sets, bf16_bits_to_f64, oracle_case
from workloads import make_case
from workloads.gen import f32_to_bf16_bits, small_case, tree_chain, tree_uniform
from tests.gpu_util import check_parity, device_case, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mv.load_library()


# ------------------------------------------------------------------ mask builder (bit-exact)

def _trees(rng):
    out = []
    for t in [1, 2, 3, 7, 12, 16, 31, 32, 33, 48, 63, 64]:
        out.append(tree_chain(t))
        out.append(tree_uniform(t, rng))
        star = np.zeros(t, np.int32)
        star[0] = -1
        out.append(star)
        forest = tree_uniform(t, rng)
        forest[rng.random(t) < 0.25] = -1
        forest[0] = -1
        out.append(forest)
    return out


def test_tree_mask_bit_exact():
    rng = np.random.default_rng(101)
    for par in _trees(rng):
        t = len(par)
        batch = np.stack([par, par[::-1] * 0 + par])  # two requests with the same tree
        tp = torch.from_numpy(batch.astype(np.int32)).cuda()
        anc = torch.full((2, t), -7, dtype=torch.int64, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        say(f"tree mask T={t}")
        mv.build_tree_mask(tp, anc, err)
        torch.cuda.synchronize()
        got = anc.cpu().numpy().view(np.uint64)
        want = ancestor_mask(par)
        assert np.array_equal(got[0], want) and np.array_equal(got[1], want), par
        assert int(err.item()) == 0


def test_tree_mask_bad_parent_flagged():
    par = np.array([[-1, 0, 5, 1, -3, 2]], dtype=np.int32)  # nodes 2 and 4 are invalid
    tp = torch.from_numpy(par).cuda()
    anc = torch.zeros((1, 6), dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    mv.build_tree_mask(tp, anc, err)
    torch.cuda.synchronize()
    fixed = np.array([-1, 0, -1, 1, -1, 2], dtype=np.int32)
    assert np.array_equal(anc.cpu().numpy().view(np.uint64)[0], ancestor_mask(fixed))
    assert int(err.item()) & mv.DEVERR_BAD_PARENT


# ------------------------------------------------------------------ small cases: tiles, ragged tails

SMALL = [
    dict(seed=201, batch=1, nodes=1, heads=1, contexts=[0], page_size=1, tree="chain", nsplit=1),
    dict(seed=202, batch=1, nodes=4, heads=8, contexts=[31], page_size=1, tree="chain", nsplit=1),
    dict(seed=203, batch=2, nodes=9, heads=8, contexts=[100, 517], page_size=1, tree="uniform", nsplit=3),
    dict(seed=204, batch=3, nodes=16, heads=5, contexts=[1000, 33, 2], page_size=4, tree="forest", nsplit=7),
    dict(seed=205, batch=1, nodes=64, heads=2, contexts=[300], page_size=16, tree="uniform", nsplit=2),
    dict(seed=206, batch=1, nodes=32, heads=8, contexts=[2500], page_size=1, tree="depth8", nsplit=1),
    dict(seed=207, batch=2, nodes=12, heads=8, contexts=[130, 4000], page_size=64, tree="chain", nsplit=5),
    dict(seed=208, batch=1, nodes=3, heads=3, contexts=[5000], page_size=1, tree="uniform", nsplit=64),
    dict(seed=209, batch=1, nodes=8, heads=16, contexts=[70], page_size=2, tree="star", nsplit=100),
    dict(seed=210, batch=2, nodes=20, heads=8, contexts=[4500, 61], page_size=8, tree="uniform", nsplit=2),
    # the largest tree (64 nodes) with many heads: 1,024 rows in 8 row blocks over two requests, and 4,096 rows
    # (64 heads, no tensor parallelism) in 32 row blocks
    dict(seed=212, batch=2, nodes=64, heads=16, contexts=[700, 2049], page_size=1, tree="uniform", nsplit=3),
    dict(seed=213, batch=1, nodes=64, heads=64, contexts=[300], page_size=8, tree="depth8", nsplit=2),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: f"seed{s['seed']}")
def test_parity_small(spec):
    case = small_case(**spec)
    say(f"small case {spec}")
    out, lse, err = run_gpu(case)
    assert err == 0
    check_parity(case, out, lse, label=str(spec))


@pytest.mark.parametrize("nsplit", [1, 3, 8, 64])
def test_skewed_batch_split_plan(nsplit):
    """One long request beside short ones: the split slots follow the key
    counts (the short requests keep one slot at least) and every request's
    result still matches the oracle."""
    spec = dict(seed=211, batch=5, nodes=6, heads=8, contexts=[9000, 3, 40, 2100, 700], page_size=4,
                tree="uniform", nsplit=nsplit)
    case = small_case(**spec)
    say(f"skewed batch {spec}")
    out, lse, err = run_gpu(case)
    assert err == 0
    check_parity(case, out, lse, label=f"skewed nsplit={nsplit}")


# ------------------------------------------------------------------ the named workloads

@pytest.mark.parametrize("nsplit", [1, 4, 64])
def test_parity_tiny_config(nsplit):
    case = make_case("C1")
    say(f"C1 nsplit={nsplit}")
    out, lse, err = run_gpu(case, nsplit=nsplit)
    assert err == 0
    check_parity(case, out, lse, label=f"C1/{nsplit}")


def test_parity_4k_config_nsplit_sweep():
    # One request of 128 rows (one row block): NSPLIT 64, 1, 7 and 16 give
    # grids of at most a quarter of the CUs (four column parts), 128 half of
    # them (two), 257 more (one), so every column-part mode meets the oracle
    # here. The combine's workgroup sizes follow NSPLIT: 1 wave (1, 7), 2 (16),
    # 8 (64) and 16 (128, 257).
    case = make_case("C2")
    ref = oracle_case(case)
    dc = device_case(case)
    outs = {}
    for ns in [64, 1, 7, 16, 128, 257]:
        say(f"C2 nsplit={ns}")
        out, lse, err = run_gpu(case, nsplit=ns, dc=dc)
        assert err == 0
        e_out, e_lse = check_parity(case, out, lse, ref=ref, label=f"C2/{ns}")
        say(f"  out max-abs {e_out:.2e}  lse max-abs {e_lse:.2e}")
        outs[ns] = (bf16_bits_to_f64(out), lse)
    # Results do not depend on NSPLIT beyond rounding noise. Each split picks
    # its own softmax reference, so a key's weight is rounded to bf16 at a
    # different scale per NSPLIT (relative 2^-9 per weight) and two results
    # carry independent errors of ~1e-3 each (the oracle check above bounds
    # both); their difference stays at that noise level everywhere and is
    # far smaller on average.
    base_o, base_l = outs[64]
    for ns, (o, l) in outs.items():
        d = np.abs(o - base_o)
        assert d.max() <= 5e-3 and d.mean() <= 2e-4, (ns, float(d.max()), float(d.mean()))
        assert np.abs(l - base_l).max() <= 1e-5, ns


def test_parity_64k_config():
    case = make_case("C3")
    say("C3 (context 65,536, 32-node depth<=8 tree)")
    out, lse, err = run_gpu(case)
    assert err == 0
    check_parity(case, out, lse, label="C3")


def test_parity_185k_fragmented_equals_contiguous():
    a = make_case("C4a")
    say("C4a (context 184,728, fragmented)")
    out_a, lse_a, err_a = run_gpu(a)
    ref = oracle_case(a)
    check_parity(a, out_a, lse_a, ref=ref, label="C4a")
    del a
    b = make_case("C4b")
    say("C4b (context 184,728, contiguous)")
    out_b, lse_b, err_b = run_gpu(b)
    assert err_a == 0 and err_b == 0
    # same logical rows in the same order: bitwise identical results
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


def test_parity_batched_block_verify():
    case = make_case("C5")
    say(f"C5 contexts={case.meta['context']}")
    out, lse, err = run_gpu(case)
    assert err == 0
    check_parity(case, out, lse, label="C5")


# ------------------------------------------------------------------ bit-exact index probes

def _probe(hot_pos, *, ctx=300, nodes=8, gap_rope=16.0, seed=301, page_size=1, nsplit=2):
    """Integer-valued inputs: every query is 1 on the 64 rope dims; every key row
    is 0 there except the row at logical key hot_pos (gap_rope), whose score then
    exceeds all others by 64*gap_rope*scale. Value dims 0 and 1 encode the slot
    as (slot % 256 + 1, slot // 256 + 1)."""
    case = small_case(seed=seed, batch=1, nodes=nodes, heads=2, contexts=[ctx], page_size=page_size,
                      tree="uniform", nsplit=nsplit, pool_extra=700)
    nslots = case.kv.shape[0]
    kv = np.zeros((nslots, 576), dtype=np.float32)
    slots = np.arange(nslots)
    kv[:, 0] = slots % 256 + 1
    kv[:, 1] = slots // 256 + 1
    hot_slot = int(case.page_table[0][hot_pos // page_size]) * page_size + hot_pos % page_size
    kv[hot_slot, 512:] = gap_rope
    q = np.zeros(case.q.shape, dtype=np.float32)
    q[..., 512:] = 1.0
    return case.with_(kv=f32_to_bf16_bits(kv), q=f32_to_bf16_bits(q)), hot_slot


@pytest.mark.parametrize("gap_rope", [16.0, 32.0])  # 32 forces the recompute path (gap > 128 in log2 units)
@pytest.mark.parametrize("hot_pos", [0, 37, 150, 299])
def test_hot_context_key_exact(hot_pos, gap_rope):
    case, hot_slot = _probe(hot_pos, gap_rope=gap_rope)
    say(f"hot context key {hot_pos} gap {gap_rope}")
    out, lse, err = run_gpu(case)
    o = bf16_bits_to_f64(out)
    assert err == 0
    assert np.all(o[..., 0] == hot_slot % 256 + 1) and np.all(o[..., 1] == hot_slot // 256 + 1)
    assert np.all(o[..., 2:] == 0)


@pytest.mark.parametrize("page_size,gap_rope", [(1, 16.0), (4, 16.0), (1, 32.0)])
def test_hot_tree_key_follows_ancestors(page_size, gap_rope):
    """A hot tree key reaches exactly the nodes it is an ancestor of. With gap
    32 only those rows take the recompute path's trigger (their score is more
    than 128 above the reference in log2 units) while the others, row 0
    among them for j > 0, do not: the workgroup's vote must hear every row."""
    ctx, nodes = 300, 8
    for j in range(nodes):
        case, hot_slot = _probe(ctx + j, ctx=ctx, nodes=nodes, page_size=page_size, gap_rope=gap_rope)
        say(f"hot tree key j={j} ps={page_size} gap={gap_rope}")
        out, lse, err = run_gpu(case)
        assert err == 0
        o = bf16_bits_to_f64(out)
        anc = ancestor_sets(case.tree_parent[0])
        ref = oracle_case(case)
        for i in range(nodes):
            hit = bool(np.all(o[0, i, :, 0] == hot_slot % 256 + 1) and np.all(o[0, i, :, 1] == hot_slot // 256 + 1))
            assert hit == (j in anc[i]), (i, j)
        check_parity(case, out, lse, ref=ref, label=f"probe j={j}")


def test_joint_permutation_bitwise():
    case = small_case(seed=401, batch=2, nodes=16, heads=8, contexts=[3000, 777], page_size=4, nsplit=9)
    out1, lse1, _ = run_gpu(case)
    rng = np.random.default_rng(3)
    pages = case.kv.shape[0] // 4
    pi = rng.permutation(pages)
    kv2 = np.empty_like(case.kv)
    for p in range(pages):
        kv2[pi[p] * 4:(pi[p] + 1) * 4] = case.kv[p * 4:(p + 1) * 4]
    pt2 = np.where(case.page_table >= 0, pi[np.maximum(case.page_table, 0)], -1).astype(np.int32)
    out2, lse2, _ = run_gpu(case.with_(kv=kv2, page_table=pt2))
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_chain_equals_causal_block():
    """A chain tree is a causal block: the oracle's chain result (itself pinned
    to a causal-mask library routine on the CPU) is matched."""
    case = small_case(seed=402, batch=2, nodes=12, heads=8, contexts=[999, 64], page_size=64, tree="chain",
                      nsplit=4)
    out, lse, err = run_gpu(case)
    check_parity(case, out, lse, label="chain")


def test_deterministic():
    case = make_case("C2")
    dc = device_case(case)
    a = run_gpu(case, dc=dc)
    b = run_gpu(case, dc=dc)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_head_permutation_permutes_outputs():
    case = small_case(seed=403, batch=1, nodes=9, heads=8, contexts=[1500], page_size=1, nsplit=5)
    out1, lse1, _ = run_gpu(case)
    perm = np.array([3, 1, 7, 0, 2, 6, 4, 5])
    out2, lse2, _ = run_gpu(case.with_(q=case.q[:, :, perm].copy()))
    assert np.array_equal(out2, out1[:, :, perm]) and np.array_equal(lse2, lse1[:, :, perm])


# ------------------------------------------------------------------ capture safety

def test_graph_capture_replays_match_eager():
    case = make_case("C2")
    dc = device_case(case)
    b, t, h, _ = case.q.shape
    desc = mv.desc_for(dc["q"], dc["kv"], dc["page_table"], page_size=1, nsplit=64, sm_scale=case.sm_scale)
    ws = mv.alloc_workspace(desc)
    out = torch.empty((b, t, h, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, t, h), dtype=torch.float32, device="cuda")
    eager_out, eager_lse, _ = run_gpu(case, dc=dc)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        mv.verify_attention(dc["q"], dc["kv"], dc["page_table"], dc["seq_lens"], dc["tree_parent"], out, lse, ws,
                            page_size=1, nsplit=64, sm_scale=case.sm_scale)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("capturing")
    with torch.cuda.graph(g, capture_error_mode="global"):
        mv.verify_attention(dc["q"], dc["kv"], dc["page_table"], dc["seq_lens"], dc["tree_parent"], out, lse, ws,
                            page_size=1, nsplit=64, sm_scale=case.sm_scale)
    for r in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(o, eager_out), r
        assert np.array_equal(lse.cpu().numpy(), eager_lse), r


# ------------------------------------------------------------------ data errors: flags, no faults

def test_seq_len_clamped_and_flagged():
    case = small_case(seed=501, batch=2, nodes=6, heads=8, contexts=[400, 50], page_size=4, nsplit=3)
    bad = case.with_(seq_lens=np.array([10_000, 3], dtype=np.int32))  # above capacity / below T
    out, lse, err = run_gpu(bad)
    assert err & mv.DEVERR_SEQ_LEN
    cap = case.page_table.shape[1] * 4
    fixed = case.with_(seq_lens=np.array([cap, 6], dtype=np.int32))
    # the clamped request 0 reads pages up to capacity: give it valid ones
    pt = fixed.page_table.copy()
    pt[0, pt[0] < 0] = pt[1, 0]
    out2, lse2, err2 = run_gpu(fixed.with_(page_table=pt))
    o1, o2 = bf16_bits_to_f64(out), bf16_bits_to_f64(out2)
    assert np.array_equal(o1[1], o2[1])  # request 1 clamped to T = 6 keys
    check_parity(fixed.with_(page_table=pt), out2, lse2, label="clamped reference")
    check_parity(fixed.with_(page_table=pt, seq_lens=np.array([cap, 6], np.int32)), out, lse, label="clamped")


def test_out_of_range_slot_is_masked_and_flagged():
    case = small_case(seed=502, batch=1, nodes=8, heads=8, contexts=[260], page_size=1, nsplit=4)
    pt = case.page_table.copy()
    pt[0, 77] = case.kv.shape[0] + 5  # past the pool
    out, lse, err = run_gpu(case.with_(page_table=pt))
    assert err & mv.DEVERR_SLOT_RANGE
    # reference: the same request with logical key 77 removed
    keep = np.r_[0:77, 78:pt.shape[1]]
    ref_case = case.with_(page_table=np.ascontiguousarray(case.page_table[:, keep]),
                          seq_lens=case.seq_lens - 1)
    check_parity(ref_case, out, lse, label="masked slot")


def test_bad_parent_treated_as_root_and_flagged():
    case = small_case(seed=503, batch=1, nodes=10, heads=8, contexts=[123], page_size=1, nsplit=2)
    tp = case.tree_parent.copy()
    tp[0, 4] = 7  # not an earlier node
    out, lse, err = run_gpu(case.with_(tree_parent=tp))
    assert err & mv.DEVERR_BAD_PARENT
    tp[0, 4] = -1
    check_parity(case.with_(tree_parent=tp), out, lse, label="bad parent")


BF16_NAN, BF16_POS_INF, BF16_NEG_INF = 0x7FC0, 0x7F80, 0xFF80


def _referenced_slots(case):
    used = set()
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        p = np.arange(n)
        pages = case.page_table[b][p // case.page_size].astype(np.int64)
        used |= set((pages * case.page_size + p % case.page_size).tolist())
    return used


def test_masked_keys_are_inert_with_non_finite_pool_rows():
    """Keys that no row may see (an out-of-range page, the padding past each
    request's last key in its last tile) must enter the products as exact
    zeros: 0 x NaN would be NaN. Every pool row that no key names, slot 0
    among them, holds NaN or an infinity; the output must be finite and equal
    the oracle's on the same request with the masked page removed."""
    ps = 4
    case = small_case(seed=504, batch=2, nodes=9, heads=8, contexts=[700, 45], page_size=ps, nsplit=5,
                      pool_extra=30)
    pt = case.page_table.copy()
    num_pages = case.kv.shape[0] // ps
    if 0 in pt[pt >= 0]:  # make page 0 (slot 0) a page no request names
        spare = sorted(set(range(num_pages)) - set(pt[pt >= 0].tolist()))[0]
        kv = case.kv.copy()
        kv[spare * ps:(spare + 1) * ps] = case.kv[0:ps]
        pt[pt == 0] = spare
        case = case.with_(kv=kv, page_table=pt)
    kv = case.kv.copy()
    unused = sorted(set(range(kv.shape[0])) - _referenced_slots(case))
    assert 0 in unused
    poison = np.array([BF16_NAN, BF16_POS_INF, BF16_NEG_INF], np.uint16)
    for i, r in enumerate(unused):
        kv[r] = poison[i % 3]
    bad_pt = case.page_table.copy()
    bad_pt[0, 10] = num_pages + 3  # keys 40..43 of request 0: out of range, masked and flagged
    poisoned = case.with_(kv=kv, page_table=bad_pt)
    say("masked keys with non-finite unused rows")
    out, lse, err = run_gpu(poisoned)
    assert err & mv.DEVERR_SLOT_RANGE
    o = bf16_bits_to_f64(out)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    # reference: request 0 without its page 10 (keys 40..43), the rest unchanged
    keep = np.r_[0:10, 11:bad_pt.shape[1]]
    ref_pt = np.full_like(bad_pt, -1)
    ref_pt[0, :len(keep)] = case.page_table[0, keep]
    ref_pt[1] = case.page_table[1]
    ref_case = case.with_(kv=kv, page_table=ref_pt, seq_lens=case.seq_lens - np.array([4, 0], np.int32))
    check_parity(ref_case, out, lse, label="inert masked keys")

"""Pins for the CPU oracle, each tied to something other than the oracle itself:
a scalar brute force, a library attention routine fed an independently built
mask, closed forms, softmax invariants, the split/combine identity, exact
integer probes and relabelling symmetries. The planted-mistake tests at the end
check that these pins do fail when the oracle is wrong in a plausible way."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (ancestor_mask, ancestor_sets, bf16_bits_to_f64, brute_force_verify,
                    oracle_case, oracle_split_combine, oracle_verify)
from workloads import make_case
from workloads.gen import f32_to_bf16_bits, small_case, tree_chain

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def run(case, **kw):
    return oracle_verify(case.q, case.kv, case.page_table, case.seq_lens, case.tree_parent,
                         case.page_size, case.sm_scale, **kw)


def closure_mask(parents):
    """Reachability through parent links by boolean matrix powers: R = I + A +
    A^2 + ... with A[i, j] = 1 iff parent(i) = j. Written independently of the
    oracle's recursive ancestor sets."""
    t = len(parents)
    a = np.zeros((t, t), dtype=np.int64)
    for i, p in enumerate(parents):
        if p >= 0:
            a[i, p] = 1
    r = np.eye(t, dtype=np.int64)
    power = np.eye(t, dtype=np.int64)
    for _ in range(t):
        power = (power @ a > 0).astype(np.int64)
        r = ((r + power) > 0).astype(np.int64)
    return r.astype(bool)


def sdpa_reference(case):
    """torch's scaled_dot_product_attention in float64 on the CPU, with the
    boolean mask built by closure_mask; lse from torch.logsumexp."""
    outs, lses = [], []
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        t = case.num_nodes
        c = n - t
        p = np.arange(n)
        slots = case.page_table[b][p // case.page_size].astype(np.int64) * case.page_size + p % case.page_size
        k = torch.from_numpy(bf16_bits_to_f64(case.kv[slots]))
        q = torch.from_numpy(bf16_bits_to_f64(case.q[b])).permute(1, 0, 2)  # [H, T, 576]
        mask = torch.ones((t, n), dtype=torch.bool)
        mask[:, c:] = torch.from_numpy(closure_mask(case.tree_parent[b]))
        kk = k[None].expand(case.num_heads, n, 576)
        vv = k[None, :, :512].expand(case.num_heads, n, 512)
        o = F.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, scale=case.sm_scale)
        sc = case.sm_scale * (q @ kk.transpose(1, 2))
        sc = sc.masked_fill(~mask, float("-inf"))
        lse = torch.logsumexp(sc, dim=-1)
        outs.append(o.permute(1, 0, 2).numpy())
        lses.append(lse.permute(1, 0).numpy())
    return np.stack(outs), np.stack(lses)


TINY = [
    dict(seed=11, batch=1, nodes=4, heads=2, contexts=[9], page_size=1, tree="chain"),
    dict(seed=12, batch=2, nodes=6, heads=1, contexts=[17, 3], page_size=4, tree="uniform"),
    dict(seed=13, batch=1, nodes=8, heads=2, contexts=[30], page_size=4, tree="forest"),
    dict(seed=14, batch=1, nodes=5, heads=1, contexts=[0], page_size=1, tree="star"),
]


# ------------------------------------------------------------------ P1: brute force

@pytest.mark.parametrize("spec", TINY, ids=lambda s: f"seed{s['seed']}")
def test_brute_force_matches_oracle(spec):
    case = small_case(**spec)
    out, lse = run(case)
    bo, bl = brute_force_verify(case.q, case.kv, case.page_table, case.seq_lens,
                                case.tree_parent, case.page_size, case.sm_scale)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ library routine

@pytest.mark.parametrize("spec", [
    dict(seed=21, batch=2, nodes=16, heads=4, contexts=[200, 57], page_size=1, tree="uniform"),
    dict(seed=22, batch=3, nodes=12, heads=3, contexts=[130, 0, 64], page_size=64, tree="chain"),
    dict(seed=23, batch=1, nodes=32, heads=2, contexts=[333], page_size=16, tree="depth8"),
    dict(seed=24, batch=1, nodes=64, heads=2, contexts=[100], page_size=1, tree="forest"),
], ids=lambda s: f"seed{s['seed']}")
def test_oracle_matches_torch_sdpa(spec):
    case = small_case(**spec)
    out, lse = run(case)
    ro, rl = sdpa_reference(case)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_oracle_matches_sdpa_on_tiny_config():
    case = make_case("C1")
    out, lse = oracle_case(case)
    ro, rl = sdpa_reference(case)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ P2: closed forms

def _depths(parents):
    d = []
    for i, p in enumerate(parents):
        d.append(0 if p < 0 else d[p] + 1)
    return np.array(d)


def test_zero_query_gives_uniform_average():
    case = small_case(seed=31, batch=2, nodes=8, heads=2, contexts=[40, 11], page_size=4)
    case = case.with_(q=np.zeros_like(case.q))
    out, lse = run(case)
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        c = n - case.num_nodes
        p = np.arange(n)
        slots = case.page_table[b][p // 4].astype(np.int64) * 4 + p % 4
        v = bf16_bits_to_f64(case.kv[slots])[:, :512]
        dep = _depths(case.tree_parent[b])
        for i in range(case.num_nodes):
            cnt = c + dep[i] + 1  # |Visible(i)| = C + depth(i) + 1
            # closed form lse = ln |Visible(i)|
            np.testing.assert_allclose(lse[b, i], math.log(cnt), rtol=0, atol=1e-12)
            # closed form out = mean of the visible values: rebuild the visible
            # set from the chain of parents by hand
            vis = list(range(c))
            j = i
            while j >= 0:
                vis.append(c + j)
                j = int(case.tree_parent[b][j])
            assert len(vis) == cnt
            np.testing.assert_allclose(out[b, i], np.broadcast_to(v[vis].mean(axis=0), out[b, i].shape),
                                       rtol=0, atol=1e-12)


def test_equal_keys_give_that_value():
    case = small_case(seed=32, batch=1, nodes=6, heads=2, contexts=[25], page_size=1)
    row = case.kv[0].copy()
    kv = np.broadcast_to(row, case.kv.shape).copy()
    case = case.with_(kv=kv)
    out, lse = run(case)
    k = bf16_bits_to_f64(row)
    dep = _depths(case.tree_parent[0])
    for i in range(case.num_nodes):
        for h in range(case.num_heads):
            s = case.sm_scale * float(bf16_bits_to_f64(case.q[0, i, h]) @ k)
            np.testing.assert_allclose(out[0, i, h], k[:512], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[0, i, h], s + math.log(25 + dep[i] + 1), rtol=0, atol=1e-11)


# ------------------------------------------------------------------ P3: invariants

def test_weights_sum_to_one_and_convexity():
    case = small_case(seed=33, batch=2, nodes=12, heads=2, contexts=[77, 5], page_size=4, tree="forest")
    kv = case.kv.copy()
    kv[:, 7] = f32_to_bf16_bits(np.ones(1, np.float32))[0]  # a constant-1 value channel
    case = case.with_(kv=kv)
    out, _ = run(case)
    np.testing.assert_allclose(out[..., 7], 1.0, rtol=0, atol=1e-12)  # sum of weights
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        p = np.arange(n)
        slots = case.page_table[b][p // 4].astype(np.int64) * 4 + p % 4
        v = bf16_bits_to_f64(case.kv[slots])[:, :512]
        assert np.all(out[b] <= v.max(axis=0) + 1e-12)
        assert np.all(out[b] >= v.min(axis=0) - 1e-12)


# ------------------------------------------------------------------ P4: chain == causal block

def test_chain_equals_causal_block():
    case = small_case(seed=34, batch=2, nodes=9, heads=3, contexts=[50, 13], page_size=1, tree="chain")
    out, lse = run(case)
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        c = n - case.num_nodes
        k = torch.from_numpy(bf16_bits_to_f64(case.kv[case.page_table[b][:n]]))
        q = torch.from_numpy(bf16_bits_to_f64(case.q[b])).permute(1, 0, 2)
        # causal-extend rule: query i sees keys p <= c + i
        mask = torch.arange(n)[None, :] <= (c + torch.arange(case.num_nodes))[:, None]
        kk = k[None].expand(case.num_heads, n, 576)
        o = F.scaled_dot_product_attention(q, kk, kk[..., :512], attn_mask=mask, scale=case.sm_scale)
        np.testing.assert_allclose(out[b], o.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ P5: split independence

@pytest.mark.parametrize("nsplit", [1, 3, 7, 64, "N", "N+5"])
def test_split_combine_equals_unsplit(nsplit):
    case = small_case(seed=35, batch=2, nodes=8, heads=2, contexts=[90, 20], page_size=4, tree="uniform")
    out, lse = run(case)
    n = int(case.seq_lens.max())
    s = {"N": n, "N+5": n + 5}.get(nsplit, nsplit)
    so, sl = oracle_split_combine(case.q, case.kv, case.page_table, case.seq_lens, case.tree_parent,
                                  case.page_size, case.sm_scale, nsplit=s)
    np.testing.assert_allclose(so, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sl, lse, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ P6: joint permutation

def test_joint_permutation_of_pool_and_page_table():
    case = small_case(seed=36, batch=2, nodes=10, heads=2, contexts=[61, 33], page_size=4)
    out, lse = run(case)
    rng = np.random.default_rng(5)
    pages = case.kv.shape[0] // case.page_size
    pi = rng.permutation(pages)  # page p moves to pi[p]
    kv2 = np.empty_like(case.kv)
    for p in range(pages):
        kv2[pi[p] * 4:(pi[p] + 1) * 4] = case.kv[p * 4:(p + 1) * 4]
    pt2 = np.where(case.page_table >= 0, pi[np.maximum(case.page_table, 0)], -1).astype(np.int32)
    out2, lse2 = run(case.with_(kv=kv2, page_table=pt2))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# ------------------------------------------------------------------ P7: hot-key probes

def _probe_case(hot_pos, seed=37, nodes=8, ctx=20):
    """Integer-valued bf16 inputs. Every key row is zero except: the row at
    logical key hot_pos carries 16 in dims 512..575 (rope part), and every
    query carries 1 there, so its score is 16*64*scale ~ 73.9 above all others
    and every other weight underflows below 2^-106. The value part of each row
    encodes the row's slot as exact integers (slot % 256, slot // 256)."""
    case = small_case(seed=seed, batch=1, nodes=nodes, heads=2, contexts=[ctx], page_size=1, tree="uniform")
    kv = np.zeros((case.kv.shape[0], 576), dtype=np.float32)
    slots = np.arange(kv.shape[0])
    kv[:, 0] = slots % 256
    kv[:, 1] = slots // 256
    hot_slot = int(case.page_table[0][hot_pos])
    kv[hot_slot, 512:] = 16.0
    q = np.zeros(case.q.shape, dtype=np.float32)
    q[..., 512:] = 1.0
    return case.with_(kv=f32_to_bf16_bits(kv), q=f32_to_bf16_bits(q)), hot_slot


def test_hot_context_key_is_exact():
    case, hot_slot = _probe_case(hot_pos=7)
    out, _ = run(case)
    assert np.all(out[..., 0] == hot_slot % 256)
    assert np.all(out[..., 1] == hot_slot // 256)


def test_hot_tree_key_follows_ancestors():
    ctx, nodes = 20, 8
    for j in range(nodes):
        case, hot_slot = _probe_case(hot_pos=ctx + j, ctx=ctx, nodes=nodes)
        out, _ = run(case)
        anc = ancestor_sets(case.tree_parent[0])
        for i in range(nodes):
            hit = bool(np.all(out[0, i, :, 0] == hot_slot % 256) and np.all(out[0, i, :, 1] == hot_slot // 256))
            assert hit == (j in anc[i]), (i, j)


# ------------------------------------------------------------------ P8 (oracle side): mask

def test_ancestor_mask_matches_closure_and_walk():
    rng = np.random.default_rng(9)
    for t in [1, 2, 5, 31, 32, 33, 63, 64]:
        for kind in range(4):
            if kind == 0:
                par = tree_chain(t)
            elif kind == 1:
                par = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, t)], np.int32)
            elif kind == 2:
                par = np.array([-1] + [0] * (t - 1), np.int32)
            else:
                par = np.array([-1 if rng.random() < 0.3 else int(rng.integers(0, max(i, 1))) for i in range(t)],
                               np.int32)
                par[0] = -1
            m = ancestor_mask(par)
            r = closure_mask(par)
            for i in range(t):
                bits = [(int(m[i]) >> j) & 1 for j in range(64)]
                assert bits[:t] == [int(x) for x in r[i]]
                assert not any(bits[t:])


def test_bad_parent_rejected():
    with pytest.raises(ValueError):
        ancestor_sets([-1, 1])
    with pytest.raises(ValueError):
        ancestor_sets([-1, 0, -2])


# ------------------------------------------------------------------ P9: relabelling

def test_head_permutation_permutes_outputs():
    case = small_case(seed=38, batch=1, nodes=6, heads=4, contexts=[40], page_size=1)
    out, lse = run(case)
    perm = np.array([2, 0, 3, 1])
    out2, lse2 = run(case.with_(q=case.q[:, :, perm].copy()))
    assert np.array_equal(out2, out[:, :, perm]) and np.array_equal(lse2, lse[:, :, perm])


def test_topological_relabel_permutes_outputs():
    """Swap two sibling leaves' labels (keeps parent < child) and move their
    queries and tree rows to match: outputs swap the same way."""
    case = small_case(seed=39, batch=1, nodes=3, heads=2, contexts=[30], page_size=1, tree="star")
    # star: nodes 1 and 2 are both children of 0; swap them
    out, lse = run(case)
    n = int(case.seq_lens[0])
    c = n - 3
    q2 = case.q[:, [0, 2, 1]].copy()
    pt2 = case.page_table.copy()
    pt2[0, c + 1], pt2[0, c + 2] = case.page_table[0, c + 2], case.page_table[0, c + 1]
    out2, lse2 = run(case.with_(q=q2, page_table=pt2))
    assert np.array_equal(out2, out[:, [0, 2, 1]]) and np.array_equal(lse2, lse[:, [0, 2, 1]])


# ------------------------------------------------------------------ planted mistakes
# Each mutant plants a plausible mistake inside the oracle module (on the CPU)
# and checks that the library-routine pin above would catch it.

import oracle.mla_oracle as om  # noqa: E402


def _plant_no_self(monkeypatch):
    orig = om.ancestor_sets
    monkeypatch.setattr(om, "ancestor_sets", lambda par: [s - {i} for i, s in enumerate(orig(par))])


def _plant_one_level(monkeypatch):
    def one_level(par):
        return [{i} | ({int(p)} if p >= 0 else set()) for i, p in enumerate(par)]
    monkeypatch.setattr(om, "ancestor_sets", one_level)


def _plant_drop_rope(monkeypatch):
    orig = om._gather_rows

    def no_rope(kv, slots, num_slots):
        r = orig(kv, slots, num_slots).copy()
        r[:, 512:] = 0.0
        return r
    monkeypatch.setattr(om, "_gather_rows", no_rope)


def _plant_page_offset(monkeypatch):
    def shifted(page_row, n_keys, page_size):
        p = np.arange(n_keys, dtype=np.int64)
        pages = np.asarray(page_row, dtype=np.int64)[p // page_size]
        return pages * page_size + (page_size - 1 - p % page_size)  # reversed within a page
    monkeypatch.setattr(om, "request_slots", shifted)


@pytest.mark.parametrize("plant", [_plant_no_self, _plant_one_level, _plant_drop_rope, _plant_page_offset])
def test_pins_detect_planted_mistakes(plant, monkeypatch):
    case = small_case(seed=23, batch=1, nodes=12, heads=2, contexts=[33], page_size=4, tree="depth8")
    ro, rl = sdpa_reference(case)
    plant(monkeypatch)
    try:
        mo, ml = run(case)
    except Exception:
        return  # a crash is also a detection
    assert not (np.allclose(mo, ro, rtol=0, atol=1e-9) and np.allclose(ml, rl, rtol=0, atol=1e-9))

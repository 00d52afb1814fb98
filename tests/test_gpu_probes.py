"""Bit-exact index probes and full-size parity in the launch configurations the
performance figures rest on (one request, page size 1, 9 or 16 nodes x 8 heads,
NSPLIT 128/256; one split over windows of 2,048 keys; pages of 64 in a ragged
batch of 8), through the C ABI.

A probe makes one logical key "hot": every query is 1 on the 64 rope dims and
every key row 0 there except the hot one, whose score then exceeds all others by
64 * gap * scale (gap 16: 74 in natural units; gap 32 forces the exact
recompute path). Value dims 0-2 encode each slot's id in base 128 (integers up
to 128 are exact in bf16), so a row that sees the hot key must return exactly
that slot's code, and one that does not see it must not. Dropping, doubling or
misplacing one key at a split, window, tile or page edge therefore shows up as
a wrong integer rather than as noise far below the tolerance."""

import math

import numpy as np
import pytest
import torch

import speculative_decoding_mla_amd as mv
from oracle import ancestor_sets, bf16_bits_to_f64, oracle_case
from workloads import sweep_case
from workloads.gen import f32_to_bf16_bits, small_case
from tests.gpu_util import check_parity, device_case, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mv.load_library()


def _encode(slots):
    s = np.asarray(slots, dtype=np.int64)
    return np.stack([s % 128 + 1, (s // 128) % 128 + 1, s // 16384 + 1], axis=-1).astype(np.float64)


def _probe_base(case):
    """The probe's integer inputs for a case's shapes and page table (no hot key yet)."""
    nslots = case.kv.shape[0]
    kv = np.zeros((nslots, 576), dtype=np.float32)
    kv[:, 0:3] = _encode(np.arange(nslots))
    q = np.zeros(case.q.shape, dtype=np.float32)
    q[..., 512:] = 1.0
    return case.with_(kv=f32_to_bf16_bits(kv), q=f32_to_bf16_bits(q))


def _slot(case, b, p):
    ps = case.page_size
    return int(case.page_table[b][p // ps]) * ps + p % ps


class Prober:
    """One probe case resident on the GPU; hot keys are set and cleared in place."""

    def __init__(self, case, nsplit):
        self.case = _probe_base(case)
        self.dc = device_case(self.case)
        self.nsplit = nsplit
        desc = mv.desc_for(self.dc["q"], self.dc["kv"], self.dc["page_table"], page_size=case.page_size,
                           nsplit=nsplit, sm_scale=case.sm_scale)
        self.ws = mv.alloc_workspace(desc)
        self.anc = [ancestor_sets(case.tree_parent[b]) for b in range(case.batch)]

    def run(self, hot, gap):
        """hot: {request: logical key}. Returns out as float64 [B, T, H, 512]."""
        kv = self.dc["kv"]
        slots = {b: _slot(self.case, b, p) for b, p in hot.items()}
        for s in slots.values():
            kv[s, 512:] = gap
        self.ws[:4].zero_()
        out, lse, err = run_gpu(self.case, nsplit=self.nsplit, dc=self.dc, workspace=self.ws)
        for s in slots.values():
            kv[s, 512:] = 0
        assert err == 0
        assert np.all(np.isfinite(lse))
        return bf16_bits_to_f64(out), slots

    def check(self, hot, gap, label=""):
        o, slots = self.run(hot, gap)
        t = self.case.num_nodes
        for b, p in hot.items():
            ctx = int(self.case.seq_lens[b]) - t
            want = _encode(slots[b])
            for i in range(t):
                sees = p < ctx or (p - ctx) in self.anc[b][i]
                hit = np.all(o[b, i, :, 0:3] == want) and np.all(o[b, i, :, 3:] == 0)
                assert bool(hit) == sees, f"{label} request {b} key {p} node {i}: sees={sees} hit={bool(hit)}"
        return o


def _edges(n, ns):
    """First and last keys of a few adjacent splits of n keys cut into ns chunks."""
    chunk = -(-n // ns)
    out = {0, n - 1}
    for s in (1, 2, ns // 2, ns - 1):
        if 0 < s * chunk < n:
            out |= {s * chunk - 1, s * chunk}
    return sorted(out)


# ------------------------------------------------------------------ split edges at 64k, NSPLIT 128 / 256

@pytest.mark.parametrize("nsplit", [128, 256])
def test_hot_keys_at_split_edges_64k(nsplit):
    """One request of 65,536 context keys and a 9-node tree x 8 heads (72 rows,
    three waves per workgroup), page size 1: the hot key sits on the first and
    last key of adjacent splits, on the last context key and on tree keys.
    NSPLIT 128 runs two column parts per split, 256 one."""
    case = small_case(seed=601, batch=1, nodes=9, heads=8, contexts=[65_536], page_size=1, tree="uniform",
                      nsplit=nsplit, pool_extra=1000)
    pr = Prober(case, nsplit)
    n = int(case.seq_lens[0])
    pos = sorted(set(_edges(n, nsplit)) | {65_535, 65_536, 65_538, n - 1})
    for gap in (16.0, 32.0):
        for p in pos:
            say(f"64k T9 nsplit {nsplit} hot key {p} gap {gap}")
            pr.check({0: p}, gap, label=f"nsplit {nsplit}")


@pytest.mark.parametrize("nodes", [9, 16])
def test_hot_keys_at_window_edges_one_split(nodes):
    """NSPLIT 1 over 6,000 context keys: the split crosses the 2,048-key slot
    windows at keys 2,048 and 4,096. Hot keys on both sides of each window
    edge, on tile edges, and (gap 32) with the exact recompute pass, which
    walks the windows again."""
    case = small_case(seed=602, batch=1, nodes=nodes, heads=8, contexts=[6000], page_size=1, tree="uniform",
                      nsplit=1, pool_extra=500)
    pr = Prober(case, 1)
    n = int(case.seq_lens[0])
    for gap in (16.0, 32.0):
        for p in [0, 31, 32, 2046, 2047, 2048, 2049, 4095, 4096, 4097, 5999, 6000, n - 1]:
            say(f"one split T{nodes} hot key {p} gap {gap}")
            pr.check({0: p}, gap, label=f"one split T{nodes}")


def _plan_chunks(seq_lens, nsplit):
    """Keys per split of each request under the plan the ABI documents: the
    B*nsplit split slots shared out in proportion to the key counts, one at
    least each."""
    n = np.asarray(seq_lens, dtype=np.int64)
    b = len(n)
    if b == 1:
        return [-(-int(n[0]) // nsplit)]
    spare = b * nsplit - b
    per = [1 + (spare * int(x)) // int(n.sum()) for x in n]
    return [-(-int(x) // k) for x, k in zip(n, per)]


def test_hot_keys_at_page_edges_ragged_batch():
    """Eight requests, pages of 64, a 12-node chain each, ragged lengths (whole
    pages, one key on the last page, shorter than a page, long): one hot key
    per request per round, on page edges, the first and last key of a split,
    the last context key and the last tree key (seen by the last node only)."""
    contexts = [1000, 4084, 4085, 40, 53, 20_000, 7777, 131_000]
    nsplit = 32
    case = small_case(seed=603, batch=8, nodes=12, heads=8, contexts=contexts, page_size=64, tree="chain",
                      nsplit=nsplit, pool_extra=40)
    pr = Prober(case, nsplit)
    chunks = _plan_chunks(case.seq_lens, nsplit)
    cand = []
    for b in range(8):
        n = int(case.seq_lens[b])
        ctx = n - 12
        last_page = (n - 1) // 64 * 64
        c = [0, 63, 64, 127, 128, last_page - 1, last_page, chunks[b] - 1, chunks[b], ctx - 1, ctx, n - 1]
        cand.append(sorted({p for p in c if 0 <= p < n}))
    rounds = max(len(c) for c in cand)
    for gap in (16.0, 32.0):
        for r in range(rounds):
            hot = {b: cand[b][r % len(cand[b])] for b in range(8)}
            say(f"ragged batch round {r} gap {gap}: {hot}")
            pr.check(hot, gap, label=f"ragged round {r}")


def test_nsplit_independence_exact():
    """The split/merge algebra without rounding in the way: with a hot key on
    each split edge of several NSPLIT, every NSPLIT returns exactly the hot
    slot's value, so the outputs agree bitwise across NSPLIT."""
    case = small_case(seed=604, batch=1, nodes=16, heads=8, contexts=[4096], page_size=1, tree="uniform",
                      nsplit=1, pool_extra=300)
    n = int(case.seq_lens[0])
    splits = [1, 7, 16, 64, 128, 257]
    probers = {ns: Prober(case, ns) for ns in splits}
    pos = sorted(set().union(*[_edges(n, ns) for ns in splits]))
    ctx = n - 16
    anc = ancestor_sets(case.tree_parent[0])
    for p in pos:
        # the rows that see the hot key: all of them for a context key, the
        # tree key's descendants (and itself) for a tree key; the other rows
        # average ordinary keys and round differently per NSPLIT
        seeing = [i for i in range(16) if p < ctx or (p - ctx) in anc[i]]
        outs = {}
        for ns in splits:
            say(f"nsplit independence: key {p} nsplit {ns}")
            outs[ns] = probers[ns].check({0: p}, 16.0, label=f"nsplit {ns}")[0, seeing]
        for ns in splits[1:]:
            assert np.array_equal(outs[ns], outs[splits[0]]), (p, ns)


# ------------------------------------------------------------------ full size, the swept launch shapes

@pytest.mark.parametrize("context,nodes", [(184_728, 9), (65_536, 16), (65_536, 9)])
def test_parity_full_size_nsplit256(context, nodes):
    """The launch behind the HBM-bound figures: one request, page size 1, KV
    rows scattered over a 195,011-slot pool, NSPLIT 256, against the oracle
    over the whole output."""
    case = sweep_case(context, nodes, nsplit=256)
    say(f"full size: context {context}, {nodes} nodes, nsplit 256")
    out, lse, err = run_gpu(case)
    assert err == 0
    e_out, e_lse = check_parity(case, out, lse, label=f"S{context}_T{nodes}")
    say(f"  out max-abs {e_out:.2e}  lse max-abs {e_lse:.2e}")

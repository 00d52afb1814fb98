#!/usr/bin/env python3
"""Verify-attention benchmark on one MI355X: verify-step latency and effective
KV bandwidth (fraction of the HBM roofline) against context length.

A step is one verify call: the split-KV partial attention (which builds the
ancestor masks in registers) and the log-sum-exp merge, over one batch of
synthetic input. Inputs are in HBM before the timed region starts. To measure
HBM rather than the 256 MB Infinity Cache, the steps cycle over R replicas of
the workload whose KV rows sit in disjoint regions of one pool (R x KV bytes >=
1 GiB); every replica holds the same logical rows, so every step computes the
same result. Whole cycles of calls are captured in hipGraphs; the warmup
replays whole cycles and the timed calls start right after one, so each timed
call reads a replica last touched R-1 calls earlier.

The default workload is C4a (context 184,728, 32-node tree, 8 heads, page size
1, fragmented), the largest single-GPU configuration.

Prints one JSON line. Options: --workload (C1, C2, C3, C4a, C4b, C5, a sweep
point S<context>_T<nodes>[_contig], or one of the rows next to verify, F1_* to
F4_*), --nsplit, --steps, --warmup, --no-sweep, --full-sweep, --no-cpu,
--cpu-seconds, --no-next.

The default line also carries next_rows: the steps next to verify (sparse
top-k decode, KV append + tree accept + commit, the sliding-window slot map,
the fp8 indexer), each timed from graph replays, with its parity against the
oracle and the oracle's host time.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify-step latency (µs) + effective KV GB/s (% HBM roofline) vs context length"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
# LDS: 256 CUs x 128 B/clk (what 128-bit LDS reads deliver per CU) at 2.4 GHz
LDS_PEAK_TBS = 256 * 128 * 2.4e9 / 1e12
QK_DIM, V_DIM = 576, 512
KV_ROW_BYTES = QK_DIM * 2  # one bf16 latent row per key
ROTATE_BYTES = 1 << 30     # >= 4 x the 256 MB Infinity Cache
KERNEL_SOURCE = os.path.join(ROOT, "speculative_decoding_mla_amd", "csrc", "mla_verify_kernels.hip")

def traffic_profile(workload: str) -> str:
    """The committed counter summary of the partial kernel on a workload."""
    return os.path.join(ROOT, "profiles", f"verify_partial_{workload}_hbm_traffic.md")

OPS_SOURCE = os.path.join(ROOT, "speculative_decoding_mla_amd", "csrc", "mla_spec_ops.hip")
INDEXER_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "indexer_F3_B1_262208_hbm_traffic.md")
# Context-sweep grid (contexts x tree sizes); --full-sweep adds the short contexts.
SWEEP = [(c, t) for c in (4_096, 16_384, 65_536, 131_072, 184_728) for t in (9, 16, 32)]
FULL_SWEEP = [(c, t) for c in (1_024, 2_048, 4_096, 8_192, 16_384, 32_768, 65_536, 131_072, 184_728)
              for t in (9, 16, 32)]

WORKLOAD_TEXT = {
    "C1": "1 request, context 256, 4-node chain, 8 heads, page size 1",
    "C2": "1 request, context 4,096, 16-node random tree, 8 heads, page size 1 scattered in a 200k-slot pool",
    "C3": "1 request, context 65,536, 32-node tree (depth <= 8), 8 heads, page size 1 scattered",
    "C4a": "1 request, context 184,728, 32-node tree, 8 heads, page size 1, fragmented page table",
    "C4b": "1 request, context 184,728, 32-node tree, 8 heads, page size 1, contiguous slots",
    "C5": "8 requests, contexts log-uniform in [1k, 128k], 12-node chain, 8 heads, page size 64",
}


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- accounting

def kv_bytes(seq_lens) -> int:
    """Latent bytes a verify call must read: one 1,152-byte row per key."""
    return int(np.sum(np.asarray(seq_lens, dtype=np.int64))) * KV_ROW_BYTES


def effective_kv_gbs(seq_lens, seconds: float) -> float:
    """The metric's effective KV bandwidth: latent bytes a step must read over
    the step time, in GB/s."""
    return kv_bytes(seq_lens) / seconds / 1e9


def partial_algorithmic_bytes(seq_lens, nodes, heads, page_size) -> int:
    """Bytes the split-partial kernel must move by the method's definition: KV
    rows, page-table entries, queries, tree parents and sequence lengths.
    Split partials are implementation traffic and are not counted."""
    keys = int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
    b = len(seq_lens)
    pages = int(sum(math.ceil(int(n) / page_size) for n in seq_lens))
    return keys * KV_ROW_BYTES + pages * 4 + b * nodes * heads * KV_ROW_BYTES + b * nodes * 4 + b * 4


def step_algorithmic_bytes(seq_lens, nodes, heads, page_size) -> int:
    b = len(seq_lens)
    return partial_algorithmic_bytes(seq_lens, nodes, heads, page_size) + b * nodes * heads * (V_DIM * 2 + 4)


def algorithmic_flops(seq_lens, nodes, heads) -> int:
    """QK^T (2 x 576) and PV (2 x 512) multiply-adds per (row, key)."""
    keys = int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
    return keys * nodes * heads * 2 * (QK_DIM + V_DIM)


def roof_bound(nodes, heads) -> str:
    intensity = nodes * heads * 2 * (QK_DIM + V_DIM) / KV_ROW_BYTES  # flop per KV byte
    return "mfma" if intensity > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"


def default_nsplit(batch, nodes, heads, max_keys) -> int:
    """NSPLIT for a sweep point: about sqrt(keys) / row blocks, as a power of
    two, and no more split workgroups than CUs. A split's tiles run one after
    another (time ~ keys / NSPLIT) while the combine merges NSPLIT partials per
    row (time ~ NSPLIT x rows); on this GPU the best of {16, ..., 256} at 4k,
    16k and 64k keys for 9, 16 and 32 nodes follows this rule."""
    rows = nodes * heads
    waves = -(-rows // 32)
    row_blocks = -(-waves // 4)
    cap = max(1, 256 // max(1, batch * row_blocks))
    root = 1 << max(0, int(math.isqrt(max(1, max_keys))).bit_length() - 1)
    return int(max(1, min(cap, root // row_blocks)))


def kernel_source_digest(path: str = KERNEL_SOURCE) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str, profile: str | None = None, source: str = KERNEL_SOURCE):
    """HBM bytes per launch of a kernel from a committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the copy-kernel calibration).
    Returns None unless the summary was taken on this workload from the kernel
    source as it is now."""
    profile = profile or traffic_profile(workload)
    try:
        with open(profile) as f:
            fields = dict(ln.split(":", 1) for ln in f if ln.startswith(("traffic_", "kernel_source_sha256", "workload")))
    except OSError:
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("kernel_source_sha256") != kernel_source_digest(source) or fields.get("workload") != workload:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- inputs on the GPU

class Replicated:
    """R replicas of one logical workload in one pool of R x (pages per
    replica) pages. "scattered": one random permutation of all the pool's
    pages, so every replica's pages lie all over the pool (page size 1 is a
    KV row per page, the fragmented layout). "contiguous": replica r owns a
    run of consecutive pages, in logical order (a defragmented pool)."""

    def __init__(self, torch, logical_rows, q_bits, seq_lens, tree_parent, page_size, replicas, seed,
                 layout="scattered"):
        self.torch = torch
        dev = "cuda"
        b = len(seq_lens)
        ps = page_size
        pages = [math.ceil(int(n) / ps) for n in seq_lens]
        ptot = sum(pages)
        self.max_pages = max(pages)
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        # logical rows of every request, each padded to whole pages
        padded = torch.zeros((ptot * ps, QK_DIM), dtype=torch.bfloat16, device=dev)
        off_rows, off = 0, 0
        for i in range(b):
            n = int(seq_lens[i])
            padded[off_rows:off_rows + n] = logical_rows[off:off + n]
            off_rows += pages[i] * ps
            off += n
        self.pool = torch.empty((replicas * ptot * ps, QK_DIM), dtype=torch.bfloat16, device=dev)
        pool_pages = self.pool.view(replicas * ptot, ps, QK_DIM)
        if layout == "contiguous":
            order = torch.arange(replicas * ptot, device=dev)
        elif layout == "scattered":
            order = torch.randperm(replicas * ptot, generator=gen, device=dev)
        else:
            raise ValueError(f"unknown layout {layout}")
        self.page_tables = []
        for r in range(replicas):
            perm = order[r * ptot:(r + 1) * ptot]
            pool_pages[perm] = padded.view(ptot, ps, QK_DIM)
            pt = torch.full((b, self.max_pages), -1, dtype=torch.int32, device=dev)
            o = 0
            for i in range(b):
                pt[i, :pages[i]] = perm[o:o + pages[i]].to(torch.int32)
                o += pages[i]
            self.page_tables.append(pt)
        del padded
        self.q = q_bits
        self.seq_lens = torch.tensor(np.asarray(seq_lens, dtype=np.int32), device=dev)
        self.tree_parent = torch.tensor(np.asarray(tree_parent, dtype=np.int32), device=dev)
        self.page_size = ps
        self.replicas = replicas
        self.layout = layout


def case_layout(case) -> str:
    """'contiguous' when every request's pages are consecutive ascending ids."""
    for b in range(case.batch):
        n_pages = math.ceil(int(case.seq_lens[b]) / case.page_size)
        row = case.page_table[b, :n_pages].astype(np.int64)
        if n_pages > 1 and not np.all(np.diff(row) == 1):
            return "scattered"
    return "contiguous"


def bf16_from_bits(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def logical_rows_of_case(case):
    rows = []
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        p = np.arange(n)
        slots = case.page_table[b][p // case.page_size].astype(np.int64) * case.page_size + p % case.page_size
        rows.append(case.kv[slots])
    return np.concatenate(rows)


# ---------------------------------------------------------------- timing

def capture(torch, fns):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def cycle_calls(replicas: int) -> int:
    """Calls per captured graph: whole cycles over the replicas, at least 64
    calls, so that a small replica count does not add a graph launch per call."""
    return replicas * max(1, -(-64 // replicas))


def time_rotating(torch, make_call, replicas, steps, warmup):
    """Device time of exactly `steps` calls that cycle over the replicas
    (call i reads replica i mod R), as ms per call.

    Every graph is captured first (capture runs each call once, eagerly) and
    replayed once before the timed window, so that no graph is launched for
    the first time inside it (a first launch also uploads the graph). The
    warmup then replays whole cycles (at least `warmup` calls, ending on
    replica R-1), and the timed calls start at replica 0. So every timed call,
    however few there are, reads a replica last touched R-1 calls earlier: R-1
    other replicas (>= 1 GiB - one replica's KV) went through the 256 MB
    Infinity Cache in between, and its rows come from HBM."""
    per = cycle_calls(replicas)
    g_cycle = capture(torch, [make_call(i % replicas) for i in range(per)])
    rem = steps % per
    g_rem = capture(torch, [make_call(i % replicas) for i in range(rem)]) if rem else None
    if g_rem is not None:
        g_rem.replay()
    warm_cycles = max(1, -(-warmup // per))
    for _ in range(warm_cycles):
        g_cycle.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps // per):
        g_cycle.replay()
    if g_rem is not None:
        g_rem.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, warm_cycles * per + rem


def time_workload(torch, mv, rep: Replicated, nodes, heads, nsplit, sm_scale, steps, warmup):
    """Returns (ms per step over exactly `steps` steps, partial-kernel us per
    launch, out, lse, workspace, warmup calls run)."""
    b = rep.q.shape[0]
    out = torch.empty((b, nodes, heads, V_DIM), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, nodes, heads), dtype=torch.float32, device="cuda")
    desc = mv.desc_for(rep.q, rep.pool, rep.page_tables[0], page_size=rep.page_size, nsplit=nsplit,
                       sm_scale=sm_scale)
    ws = mv.alloc_workspace(desc)

    def full_call(r):
        return lambda: mv.verify_attention(rep.q, rep.pool, rep.page_tables[r], rep.seq_lens, rep.tree_parent,
                                           out, lse, ws, page_size=rep.page_size, nsplit=nsplit,
                                           sm_scale=sm_scale)

    def partial_call(r):
        return lambda: mv.verify_partial(desc, rep.q, rep.pool, rep.page_tables[r], rep.seq_lens, rep.tree_parent,
                                         ws)

    R = rep.replicas
    ms_per_step, warm_calls = time_rotating(torch, full_call, R, steps, warmup)
    # the dominant kernel alone, timed the same way with events on the stream
    # it runs on (at least one whole cycle of calls)
    p_steps = max(steps, cycle_calls(R))
    ms_partial, _ = time_rotating(torch, partial_call, R, p_steps, warmup)
    # leave the full result of replica 0 in out/lse
    full_call(0)()
    torch.cuda.synchronize()
    return ms_per_step, ms_partial * 1e3, out, lse, ws, warm_calls


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(case, budget_s=10.0, max_reps=20):
    """Time the oracle (as it stands) on this host's cores on the same workload."""
    from oracle import oracle_case  # the checker's leg of the benchmark only

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    times, ref = [], None
    t_start = time.perf_counter()
    while len(times) < max_reps:
        t = time.perf_counter()
        ref = oracle_case(case)
        times.append(time.perf_counter() - t)
        if time.perf_counter() - t_start > budget_s:
            break
    med = statistics.median(times)
    return med, len(times), threads, ref


def cpu_baseline_one_thread(case, budget_s=10.0, max_reps=5):
    """The same oracle timing with the BLAS pool limited to one thread."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        med, reps, _, _ = cpu_baseline(case, budget_s=budget_s, max_reps=max_reps)
    return med, reps


def measured_peaks():
    """The achievable peaks of this GPU, measured in this run by the mla_peaks
    program (streaming read, copy, bf16 MFMA), as a child process."""
    import subprocess
    exe = os.path.join(ROOT, "speculative_decoding_mla_amd", "lib", "mla_peaks")
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        return json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else None
    except (OSError, ValueError, IndexError, subprocess.TimeoutExpired):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- the steps next to verify

def graph_us_per_call(torch, calls, reps=4, batches=5):
    """Per-call device time of `calls`, captured in one hipGraph: the median
    over `batches` windows of `reps` replays, each between two events (one
    host stall between two replays, which leaves the GPU idle inside a window,
    then moves one window rather than the figure)."""
    g = capture(torch, calls)
    g.replay()
    torch.cuda.synchronize()
    per_call = []
    for _ in range(batches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) * 1e3 / (reps * len(calls)))
    return statistics.median(per_call)


def _cpu_time(fn, budget_s=5.0, max_reps=5):
    times, out = [], None
    t_start = time.perf_counter()
    while len(times) < max_reps:
        t = time.perf_counter()
        out = fn()
        times.append(time.perf_counter() - t)
        if time.perf_counter() - t_start > budget_s:
            break
    return statistics.median(times), out


def next_sparse_decode(torch, mv, batch, nsplit=16, heads=64, topk=512, replicas=64, seed=31, with_cpu=True):
    """Sparse top-k MLA decode (one query token, 64 heads, 512 selected latent
    rows per request) over a 2 GiB pool; each replica selects its own random
    slots, so most rows come from HBM rather than the 256 MB Infinity Cache."""
    import oracle.spec_ops_oracle as so

    pool_rows = (2 << 30) // KV_ROW_BYTES
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    pool = torch.randn((pool_rows, QK_DIM), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    q = torch.randn((batch, heads, QK_DIM), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    idx = [torch.randperm(pool_rows, generator=gen, device="cuda")[:batch * topk].view(batch, topk).to(torch.int32)
           for _ in range(replicas)]
    out = torch.empty((batch, heads, V_DIM), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((batch, heads), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(192.0)
    ws = mv.alloc_sparse_workspace(mv.sparse_desc(q, pool, idx[0], nsplit=nsplit, sm_scale=scale))
    us = graph_us_per_call(torch, [lambda r=r: mv.sparse_decode(q, pool, idx[r], None, out, lse, ws, nsplit=nsplit,
                                                                 sm_scale=scale) for r in range(replicas)])
    mv.sparse_decode(q, pool, idx[0], None, out, lse, ws, nsplit=nsplit, sm_scale=scale)
    torch.cuda.synchronize()
    # parity of replica 0 on its gathered rows (the same definition, rows renumbered)
    rows = pool[idx[0].long().flatten()].view(torch.int16).cpu().numpy().view(np.uint16)
    local = np.arange(batch * topk, dtype=np.int32).reshape(batch, topk)
    qb = q.view(torch.int16).cpu().numpy().view(np.uint16)
    keys = batch * topk
    alg = keys * KV_ROW_BYTES + keys * 4 + batch * heads * (KV_ROW_BYTES + V_DIM * 2 + 4)
    e = dict(row="sparse top-k decode", workload=f"{batch} request(s), 1 query token, {heads} heads, top-k {topk}, "
                                                   f"page size 1 over a 2 GiB pool, NSPLIT {nsplit}",
             latency_us=round(us, 3), bytes_per_call=alg, achieved_gbs=round(alg / (us * 1e-6) / 1e9, 1),
             bound="hbm", hbm_frac=round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
    if with_cpu:
        t, (ro, rl) = _cpu_time(lambda: so.sparse_decode(qb, rows, local, None, scale))
        o = bf16_from_bits(torch, out.view(torch.int16).cpu().numpy().view(np.uint16)).float().numpy()
        e["parity_vs_oracle"] = dict(out_max_abs=float(np.abs(o - ro).max()),
                                     lse_max_abs=float(np.abs(lse.cpu().numpy() - rl).max()))
        e["cpu_oracle_us"] = round(t * 1e6, 1)
    del pool, idx
    torch.cuda.empty_cache()
    return e


def next_indexer(torch, mv, batch, positions, heads=64, seed=41, with_cpu=True):
    """fp8 indexer logits over a paged cache of 8,448-byte blocks; R replicas of
    the blocks (R x bytes >= 1 GiB), each with its own block table."""
    import oracle.spec_ops_oracle as so
    from workloads.ops_gen import indexer_case

    max_blocks = -(-positions // 64)
    c = indexer_case(seed, batch=batch, heads=heads, max_blocks=max_blocks, seq_lens=[positions] * batch,
                     spare_blocks=0)
    nb = c.blocks.shape[0]
    reps_data = max(1, math.ceil(ROTATE_BYTES / c.blocks.nbytes))
    blocks = torch.from_numpy(c.blocks).cuda().repeat(reps_data, 1)
    bts = [torch.from_numpy(np.where(c.block_table >= 0, c.block_table + r * nb, -1).astype(np.int32)).cuda()
           for r in range(reps_data)]
    q = torch.from_numpy(c.q).cuda()
    w = torch.from_numpy(c.weights).cuda()
    sl = torch.from_numpy(c.seq_lens).cuda()
    logits = torch.empty((batch, max_blocks * 64), dtype=torch.float32, device="cuda")
    us = graph_us_per_call(torch, [lambda r=r: mv.indexer_logits(q, w, blocks, bts[r], sl, logits)
                                   for r in range(reps_data)])
    mv.indexer_logits(q, w, blocks, bts[0], sl, logits)
    torch.cuda.synchronize()
    pages = batch * max_blocks
    alg = pages * (8448 + 4) + batch * max_blocks * 64 * 4 + batch * heads * (128 + 4) + batch * 4
    flops = batch * positions * heads * 128 * 2
    e = dict(row="fp8 indexer logits", workload=f"{batch} request(s) x {positions} positions, {heads} heads x 128 "
                                                 f"e4m3, 8,448-byte blocks",
             latency_us=round(us, 3), bytes_per_call=alg, achieved_gbs=round(alg / (us * 1e-6) / 1e9, 1),
             bound="hbm", hbm_frac=round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
             mfma_frac=round(flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 5),
             traffic=measured_traffic(f"F3_indexer_B{batch}_{positions}", INDEXER_TRAFFIC_PROFILE, OPS_SOURCE))
    if with_cpu:
        t, ref = _cpu_time(lambda: so.indexer_logits(c.q, c.weights, c.blocks, c.block_table, c.seq_lens), max_reps=1)
        mag = so.indexer_magnitude(c.q, c.weights, c.blocks, c.block_table, c.seq_lens)
        got = logits.cpu().numpy()
        fin = np.isfinite(ref)
        # error over the fp32 terms' magnitude sum_h |w_h| sum_d |q k| s (the tests allow 2e-6)
        e["parity_vs_oracle"] = dict(max_err_over_term_magnitude=float(np.max(np.abs(got[fin] - ref[fin]) /
                                                                               np.maximum(mag[fin], 1e-30))),
                                     neg_inf_positions_match=bool(np.array_equal(np.isfinite(got), fin)))
        e["cpu_oracle_us"] = round(t * 1e6, 1)
    del blocks
    torch.cuda.empty_cache()
    return e


def next_accept_commit(torch, mv, batch, nodes, tree, seed=51, with_cpu=True):
    """The step around verify: the draft rows' KV append, then the greedy tree
    accept and the commit of the accepted path in one launch, as one captured
    sequence (the accept and the commit as two launches timed beside it)."""
    import oracle.spec_ops_oracle as so
    from workloads.ops_gen import accept_case

    c = accept_case(seed, batch=batch, nodes=nodes, tree=tree, match=0.85)
    rng = np.random.default_rng(seed)
    kv = torch.randn((c.num_slots, QK_DIM), device="cuda", dtype=torch.float32).to(torch.bfloat16)
    rows_np = rng.integers(0, 65535, size=(batch * nodes, QK_DIM), dtype=np.uint16)
    rows = bf16_from_bits(torch, rows_np).cuda()
    loc_np = np.concatenate([c.page_table[b, c.seq_lens[b] - nodes:c.seq_lens[b]] for b in range(batch)])
    loc = torch.from_numpy(loc_np.astype(np.int32)).cuda()
    pt0 = torch.from_numpy(c.page_table).cuda()
    pt = pt0.clone()
    par, drf, tgt = (torch.from_numpy(x).cuda() for x in (c.tree_parent, c.draft_tokens, c.target_tokens))
    sl = torch.from_numpy(c.seq_lens).cuda()
    n = torch.empty(batch, dtype=torch.int32, device="cuda")
    path = torch.empty((batch, nodes), dtype=torch.int32, device="cuda")
    com = torch.empty((batch, nodes), dtype=torch.int32, device="cuda")
    ctx = torch.empty(batch, dtype=torch.int32, device="cuda")
    freed = torch.empty((batch, nodes), dtype=torch.int32, device="cuda")

    def step_separate():
        pt.copy_(pt0)
        mv.kv_append(kv, rows, loc)
        mv.tree_accept(par, drf, tgt, n, path, com)
        mv.commit_accepted(pt, sl, nodes, n, path, ctx, freed)

    def step():
        pt.copy_(pt0)
        mv.kv_append(kv, rows, loc)
        mv.accept_commit(par, drf, tgt, pt, sl, n, path, ctx, com, freed)

    us_sep = graph_us_per_call(torch, [step_separate] * 16)
    us = graph_us_per_call(torch, [step] * 16)
    step()
    torch.cuda.synchronize()
    alg = batch * nodes * (2 * KV_ROW_BYTES + 4) + batch * nodes * 4 * 6 + batch * 4 * 3
    e = dict(row="KV append + tree accept + commit", workload=f"{batch} request(s), {nodes}-node {tree} trees, "
                                                                 f"page size 1",
             latency_us=round(us, 3), latency_us_accept_and_commit_as_two_launches=round(us_sep, 3),
             bytes_per_call=alg, achieved_gbs=round(alg / (us * 1e-6) / 1e9, 2), bound="latency")
    if with_cpu:
        def cpu():
            rn, rp, rc = so.tree_accept(c.tree_parent, c.draft_tokens, c.target_tokens)
            return rn, rp, rc, so.commit_accepted(c.page_table, c.seq_lens, nodes, rn, rp)
        t, (rn, rp, rc, (rpt, rctx, rfreed, _)) = _cpu_time(cpu)
        e["parity_vs_oracle"] = dict(bit_exact=bool(
            np.array_equal(n.cpu().numpy(), rn) and np.array_equal(path.cpu().numpy(), rp) and
            np.array_equal(com.cpu().numpy(), rc) and np.array_equal(pt.cpu().numpy(), rpt) and
            np.array_equal(ctx.cpu().numpy(), rctx) and np.array_equal(freed.cpu().numpy(), rfreed)))
        e["mean_commit_len"] = float(rn.mean())
        e["cpu_oracle_us"] = round(t * 1e6, 1)
    return e


def next_window_map(torch, mv, batch=8, window=4096, page=64, seed=61, with_cpu=True):
    """The page-aligned sliding-window slot map of a draft cache (W = 4096,
    P = 64), lengths log-uniform in [1k, 128k]."""
    import oracle.spec_ops_oracle as so
    from workloads.ops_gen import window_case

    tm_np, lens_np = window_case(seed, batch=batch, width=131_072, lo=1024, hi=131_072)
    tm = torch.from_numpy(tm_np).cuda()
    lens = torch.from_numpy(lens_np).cuda()
    dm = torch.empty((batch, window + page - 1), dtype=torch.int32, device="cuda")
    cl = torch.empty(batch, dtype=torch.int32, device="cuda")
    us = graph_us_per_call(torch, [lambda: mv.window_map(tm, lens, window, page, dm, cl)] * 64)
    mv.window_map(tm, lens, window, page, dm, cl)
    torch.cuda.synchronize()
    alg = int(sum(so.compact_len(int(x), window, page) for x in lens_np)) * 4 + batch * (window + page - 1) * 4 + batch * 8
    e = dict(row="sliding-window slot map", workload=f"{batch} requests, W {window}, P {page}, lengths log-uniform "
                                                       f"in [1k, 128k]",
             latency_us=round(us, 3), bytes_per_call=alg, achieved_gbs=round(alg / (us * 1e-6) / 1e9, 2),
             bound="latency")
    if with_cpu:
        t, (rdm, rcl) = _cpu_time(lambda: so.window_map(tm_np, lens_np, window, page))
        e["parity_vs_oracle"] = dict(bit_exact=bool(np.array_equal(dm.cpu().numpy(), rdm) and
                                                     np.array_equal(cl.cpu().numpy(), rcl)))
        e["cpu_oracle_us"] = round(t * 1e6, 1)
    return e


NEXT_ROWS = {
    "F1_sparse_B1": (next_sparse_decode, dict(batch=1, nsplit=16)),
    "F1_sparse_B16": (next_sparse_decode, dict(batch=16, nsplit=8)),
    "F2_accept_B8_chain12": (next_accept_commit, dict(batch=8, nodes=12, tree="chain")),
    "F2_accept_B1_tree32": (next_accept_commit, dict(batch=1, nodes=32, tree="depth8")),
    "F4_window_B8": (next_window_map, dict()),
    "F3_indexer_B1_262208": (next_indexer, dict(batch=1, positions=262_208)),
    "F3_indexer_B16_32768": (next_indexer, dict(batch=16, positions=32_768)),
}


def measure_next_rows(torch, mv, with_cpu=True, only=None):
    rows = []
    for name, (fn, kw) in NEXT_ROWS.items():
        if only is not None and name != only:
            continue
        e = fn(torch, mv, with_cpu=with_cpu, **kw)
        e["name"] = name
        log(f"next row {name}: {e['workload']}: {e['latency_us']} us")
        rows.append(e)
    return rows


# ---------------------------------------------------------------- main

def measure_case(torch, mv, case, nsplit, steps, warmup, seed, replicas=None):
    rows = logical_rows_of_case(case)
    lr = bf16_from_bits(torch, rows).cuda()
    q = bf16_from_bits(torch, case.q).cuda()
    kvb = kv_bytes(case.seq_lens)
    if replicas is None:
        replicas = max(1, math.ceil(ROTATE_BYTES / max(kvb, 1)))
    rep = Replicated(torch, lr, q, case.seq_lens, case.tree_parent, case.page_size, replicas, seed,
                     layout=case_layout(case))
    del lr
    res = time_workload(torch, mv, rep, case.num_nodes, case.num_heads, nsplit, case.sm_scale, steps, warmup)
    return res, rep


def parity_of(case, out_bits, lse, ref=None):
    """Max-abs error of the GPU result against the oracle (the checker's leg)."""
    from oracle import bf16_bits_to_f64, oracle_case
    ref_out, ref_lse = oracle_case(case) if ref is None else ref
    return dict(out_max_abs=float(np.abs(bf16_bits_to_f64(out_bits) - ref_out).max()),
                lse_max_abs=float(np.abs(lse.astype(np.float64) - ref_lse).max()),
                within_tolerance=bool(np.abs(bf16_bits_to_f64(out_bits) - ref_out).max() <= 1e-2 and
                                      np.abs(lse.astype(np.float64) - ref_lse).max() <= 1e-3))


def partial_lds_bytes(seq_lens, nodes, heads, nsplit) -> int:
    """LDS bytes the partial kernel's dataflow moves per launch (not a property
    of the method, of this kernel): for every 32-key tile of a request, every
    row block and every column part, each computing wave reads the K tile
    (36,864 B) and the V^T columns of its part (32,768 / parts B), and the
    tile's 36,864 B arrive in LDS once per workgroup. The column-part rule is
    the library's: 4 parts while the grid fills at most a quarter of the 256
    CUs, 2 up to half."""
    rows = nodes * heads
    waves = -(-rows // 32)
    nwq = min(waves, 4)
    row_blocks = -(-waves // nwq)
    wgs = len(seq_lens) * nsplit * row_blocks
    ncp = 4 if wgs * 4 <= 256 else (2 if wgs * 2 <= 256 else 1)
    tiles = sum(-(-int(n) // 32) for n in seq_lens)
    tile_bytes = 32 * KV_ROW_BYTES
    return tiles * row_blocks * ncp * (nwq * (tile_bytes + 32 * V_DIM * 2 // ncp) + tile_bytes)


def roofline_fields(seq_lens, nodes, heads, page_size, partial_us, nsplit):
    """The partial kernel against both roofs: algorithmic bytes and flops per
    launch over its measured launch time. `bound` names the roof its
    arithmetic intensity puts it under. Beside them, the LDS bytes of this
    kernel's dataflow against the LDS peak, the resource its tile loop is
    actually bound by."""
    pbytes = partial_algorithmic_bytes(seq_lens, nodes, heads, page_size)
    pflops = algorithmic_flops(seq_lens, nodes, heads)
    lbytes = partial_lds_bytes(seq_lens, nodes, heads, nsplit)
    gbs = pbytes / (partial_us * 1e-6) / 1e9
    tflops = pflops / (partial_us * 1e-6) / 1e12
    ltbs = lbytes / (partial_us * 1e-6) / 1e12
    return dict(bound=roof_bound(nodes, heads), bytes_per_launch=pbytes, flops_per_launch=pflops,
                achieved_gbs=gbs, achieved_tflops=tflops, hbm_frac=gbs / HBM_PEAK_GBS,
                mfma_frac=tflops / BF16_PEAK_TFLOPS, lds_bytes_per_launch=lbytes, lds_tbs=ltbs,
                lds_frac=ltbs / LDS_PEAK_TBS)


def sweep_point(torch, mv, context, nodes, heads=8, nsplit=None, layout="scattered", with_parity=True):
    """A context-sweep point: the seeded sweep case (N(0,1) bf16 rows and
    queries, uniform-parent tree, depth <= 8 for 32 nodes, page size 1), its
    logical rows replicated over a >= 1 GiB pool, scattered or contiguous;
    parity of the result against the oracle."""
    from workloads import sweep_case

    n = context + nodes
    nsplit = nsplit or default_nsplit(1, nodes, heads, n)
    case = sweep_case(context, nodes, nsplit=nsplit)
    rows = bf16_from_bits(torch, logical_rows_of_case(case)).cuda()
    q = bf16_from_bits(torch, case.q).cuda()
    replicas = max(1, math.ceil(ROTATE_BYTES / kv_bytes([n])))
    rep = Replicated(torch, rows, q, case.seq_lens, case.tree_parent, 1, replicas, 7, layout=layout)
    del rows
    steps = cycle_calls(replicas) * 2
    ms, partial_us, out, lse, *_ = time_workload(torch, mv, rep, nodes, heads, nsplit, case.sm_scale, steps,
                                                 replicas)
    lat_us = ms * 1e3
    eff = effective_kv_gbs([n], lat_us * 1e-6)
    rf = roofline_fields([n], nodes, heads, 1, partial_us, nsplit)
    entry = dict(workload=f"context {context}, {nodes}-node tree, {heads} heads, page size 1, {layout} KV rows",
                 layout=layout, context=context, nodes=nodes, rows=nodes * heads, nsplit=nsplit, replicas=replicas,
                 latency_us=round(lat_us, 2), eff_kv_gbs=round(eff, 1), eff_kv_hbm_frac=round(eff / HBM_PEAK_GBS, 4),
                 partial_us=round(partial_us, 2), partial_hbm_frac=round(rf["hbm_frac"], 4),
                 partial_mfma_frac=round(rf["mfma_frac"], 4), partial_lds_frac=round(rf["lds_frac"], 4),
                 bound=rf["bound"])
    if with_parity:
        entry["parity_vs_oracle"] = parity_of(case, out.view(torch.int16).cpu().numpy().view(np.uint16),
                                              lse.cpu().numpy())
    del rep, out, lse
    torch.cuda.empty_cache()
    return entry


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="C4a",
                    help="C1, C2, C3, C4a, C4b, C5, a context-sweep point S<context>_T<nodes>[_contig], or one "
                         "row next to verify: " + ", ".join(NEXT_ROWS))
    ap.add_argument("--nsplit", type=int, default=None)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--full-sweep", action="store_true", help="contexts from 1k to 184,728 (27 points)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="host time budget of the oracle baseline")
    ap.add_argument("--no-next", action="store_true", help="skip the rows next to verify (sparse decode, accept/"
                                                            "commit, window map, fp8 indexer)")
    ap.add_argument("--seed", type=int, default=1234)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the verify kernel works on one GPU's "
                                   "share (8 heads of a tensor-parallel rank) and no multi-GPU path is built",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import speculative_decoding_mla_amd as mv
    from workloads import make_case

    mv.load_library()
    if args.workload in NEXT_ROWS:
        e = measure_next_rows(torch, mv, with_cpu=not args.no_cpu, only=args.workload)[0]
        print(json.dumps(dict(metric=METRIC, n_gpus=1, next_rows=[e])), flush=True)
        return
    if args.workload.startswith("S"):
        spec = args.workload[1:].split("_")
        ctx, nodes = int(spec[0]), int(spec[1][1:])
        layout = "contiguous" if spec[2:] == ["contig"] else "scattered"
        e = sweep_point(torch, mv, ctx, nodes, nsplit=args.nsplit, layout=layout, with_parity=not args.no_cpu)
        log(json.dumps(e))
        print(json.dumps(dict(metric=METRIC, value=e["eff_kv_gbs"], unit="GB/s", n_gpus=1, latency_us=e["latency_us"],
                              config=dict(workload=e["workload"]), sweep=[e])), flush=True)
        return
    if args.workload not in WORKLOAD_TEXT:
        ap.error(f"unknown workload {args.workload}")
    log(f"generating {args.workload}")
    case = make_case(args.workload, nsplit=args.nsplit)
    log(f"timing {args.workload}: {args.steps} steps after {args.warmup} warmup")
    nsplit = case.nsplit
    (ms, partial_us, out, lse, ws, warm_calls), rep = measure_case(torch, mv, case, nsplit, args.steps,
                                                                    args.warmup, args.seed)
    dev_err = mv.device_error(ws)
    lat_us = ms * 1e3
    kvb = kv_bytes(case.seq_lens)
    eff = effective_kv_gbs(case.seq_lens, lat_us * 1e-6)
    rf = roofline_fields(case.seq_lens, case.num_nodes, case.num_heads, case.page_size, partial_us, nsplit)
    traffic = measured_traffic(args.workload)
    if rf["bound"] == "hbm":
        roof = dict(bound="hbm", achieved=round(rf["achieved_gbs"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(rf["hbm_frac"], 4), traffic=traffic)
    else:
        roof = dict(bound="mfma", achieved=round(rf["achieved_tflops"], 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(rf["mfma_frac"], 4), traffic=traffic)
    # both roofs side by side, whichever binds
    roof.update(kernel="verify_partial_kernel", kernel_us=round(partial_us, 3), bytes_per_launch=rf["bytes_per_launch"],
                flops_per_launch=rf["flops_per_launch"], hbm_gbs=round(rf["achieved_gbs"], 1),
                hbm_frac=round(rf["hbm_frac"], 4), mfma_tflops=round(rf["achieved_tflops"], 1),
                mfma_frac=round(rf["mfma_frac"], 4), lds_bytes_per_launch=rf["lds_bytes_per_launch"],
                lds_tbs=round(rf["lds_tbs"], 2), lds_peak_tbs=round(LDS_PEAK_TBS, 1), lds_frac=round(rf["lds_frac"], 4))
    if traffic:
        roof["traffic_over_algorithmic"] = round(traffic / rf["bytes_per_launch"], 3)
    gpu_out = out.view(torch.int16).cpu().numpy().view(np.uint16)
    gpu_lse = lse.cpu().numpy()
    layout = rep.layout
    replicas = rep.replicas
    del rep, out, lse, ws
    torch.cuda.empty_cache()

    line = dict(metric=METRIC, value=round(eff, 2), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=round(ms, 6), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
                data="synthetic",
                config=dict(workload=f"{args.workload}: {WORKLOAD_TEXT[args.workload]}",
                            context=case.meta["context"], nodes=case.num_nodes, heads=case.num_heads,
                            page_size=case.page_size, nsplit=nsplit, rows=case.num_nodes * case.num_heads,
                            replicas=replicas, layout=layout, parallelism="none (1 GPU)"),
                latency_us=round(lat_us, 3), eff_kv_hbm_frac=round(eff / HBM_PEAK_GBS, 4),
                roofline=roof, device_error=dev_err,
                timing=dict(warmup_calls_run=warm_calls,
                            rotation=f"{replicas} replicas of the workload's KV (>= 1 GiB together); timed calls "
                                     "cycle over them starting right after a whole warmup cycle, so each reads "
                                     "a replica last touched R-1 calls earlier"))

    log(f"{args.workload}: {lat_us:.2f} us/step, partial kernel {partial_us:.2f} us")
    # The same workload from one replica: its KV stays in the 256 MB Infinity
    # Cache between steps. Reported beside the rotating-replica number, which
    # is the measurement; this one is labelled cache-resident.
    (w_ms, w_partial_us, *_), w_rep = measure_case(torch, mv, case, nsplit, 256, 64, args.seed, replicas=1)
    del w_rep
    torch.cuda.empty_cache()
    line["warm_cache_resident"] = dict(latency_us=round(w_ms * 1e3, 3), partial_us=round(w_partial_us, 3),
                                       eff_kv_gbs=round(effective_kv_gbs(case.seq_lens, w_ms * 1e-3), 1),
                                       note="one replica, KV resident in the Infinity Cache across steps")
    peaks = measured_peaks()
    if peaks:
        line["measured_peaks"] = dict(hbm_read_gbs=peaks.get("hbm_read_gbs"),
                                      mfma_bf16_tflops=peaks.get("mfma_bf16_tflops"),
                                      source="mla_peaks, run by this benchmark on this GPU")
        den = peaks.get("hbm_read_gbs") if roof["bound"] == "hbm" else peaks.get("mfma_bf16_tflops")
        if den:
            roof["frac_of_measured_peak"] = round(roof["achieved"] / den, 4)
        if peaks.get("hbm_read_gbs"):
            line["eff_kv_frac_of_measured_read"] = round(eff / peaks["hbm_read_gbs"], 4)
    if not args.no_cpu:
        log("timing the CPU oracle")
        budget = args.cpu_seconds
        med, reps, threads, ref = cpu_baseline(case, budget_s=budget)
        line["cpu_baseline"] = dict(value=round(kvb / med / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
                                    sample=f"the whole {args.workload} verify call (all {kvb // KV_ROW_BYTES} keys), "
                                           f"{reps} timed run(s) in a {budget:.0f} s budget, median "
                                           f"{med * 1e6:.0f} us; CPU {cpu_model()}")
        med1, reps1 = cpu_baseline_one_thread(case, budget_s=budget, max_reps=3)
        line["cpu_baseline_1thread"] = dict(value=round(kvb / med1 / 1e9, 4), unit="GB/s", cores=1,
                                            kind="oracle", sample=f"the same call, {reps1} timed run(s), median "
                                                                  f"{med1 * 1e6:.0f} us, BLAS limited to 1 thread")
        line["parity_vs_oracle"] = parity_of(case, gpu_out, gpu_lse, ref=ref)

    if not args.no_next:
        line["next_rows"] = measure_next_rows(torch, mv, with_cpu=not args.no_cpu)

    if not args.no_sweep:
        sweep = []
        for ctx, t in (FULL_SWEEP if args.full_sweep else SWEEP):
            sweep.append(sweep_point(torch, mv, ctx, t, with_parity=not args.no_cpu))
            log(f"sweep context {ctx} nodes {t}: {sweep[-1]['latency_us']} us, {sweep[-1]['eff_kv_gbs']} GB/s")
        line["sweep"] = sweep
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

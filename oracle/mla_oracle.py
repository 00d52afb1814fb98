"""Plain fp64 oracle for the verify attention of tree speculative decoding over a
paged MLA latent KV cache.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. Nothing on the product path imports it.

What it computes, and where the pages say so. Page "The Custom sm_120 Verify
Kernel: From 0.7 tok/s to 3-6x Decode Speedup on Blackwell Consumer GPUs":
  * Part VI: the verify step evaluates every draft-tree node of a request as a
    query against the request's KV, with a custom tree attention mask, over a
    page-size-1 latent pool.
  * Part VII: the committed prefix needs no mask; only the small tree block
    carries the custom mask.
  * Part IX, "The Debugging Gauntlet", Bug 2: the keys are the prefix slots
    followed by the draft tokens' own slots (combined indices), and the mask
    stride is prefix + q_len, so a draft node sees the whole prefix plus part
    of the draft block.
  * Part VII: the kernel splits the KV into NSPLIT chunks, computes partial
    results per chunk and reduces them (partial + reduce).
Shapes: the query is the absorbed 576-wide vector (512 latent + 64 rope) per
(node, head); the key is the whole 576-wide latent row; the value is its first
512 entries; the softmax scale is a caller parameter (1/sqrt(192) in every
workload here).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * a node sees its ancestors and itself (a chain then equals a causal block);
  * seq_lens counts the tree rows: context C = seq_len - T, tree node j's own
    latent row is logical key C + j;
  * node order is topological (parent < child); anything else is an error here;
  * lse is the natural log of the sum of exp(scale * q.k) over visible keys.

Definition used by oracle_verify, for request b, node i, head h:
  N = seq_lens[b], C = N - T,
  slot(p) = page_table[b, p // ps] * ps + p % ps,
  k_p = kv[slot(p), 0:576],  v_p = kv[slot(p), 0:512],
  Anc*(i) = {i} u Anc*(parent(i)) (just {i} for a root),
  Visible(i) = {p < C} u {C + j : j in Anc*(i)},
  s_p = scale * q[b,i,h,:] . k_p  for p in Visible(i),
  m = max s_p, Z = sum exp(s_p - m), lse = m + ln Z,
  out[b,i,h,:] = sum_p exp(s_p - lse) v_p.
Everything is float64; bf16 inputs are decoded exactly.
"""

from __future__ import annotations

import math

import numpy as np

QK_DIM = 576
V_DIM = 512


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly: a bf16 value is the float32
    whose upper 16 bits are the pattern and whose lower 16 bits are zero."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def ancestor_sets(parents) -> list:
    """Anc*(i) for every node of one request: node i together with every node
    reached by following parent links. Raises on a parent that is not an
    earlier node (the order must be topological)."""
    parents = [int(x) for x in parents]
    out = []
    for i, p in enumerate(parents):
        if p < -1 or p >= i:
            raise ValueError(f"node {i} has parent {p}; parents must be -1 or < {i}")
        s = {i}
        if p >= 0:
            s |= out[p]
        out.append(s)
    return out


def ancestor_mask(parents) -> np.ndarray:
    """The same sets as 64-bit masks: bit j of entry i is set iff j is in
    Anc*(i). Requires at most 64 nodes."""
    sets = ancestor_sets(parents)
    if len(sets) > 64:
        raise ValueError("at most 64 tree nodes fit a 64-bit mask")
    masks = []
    for s in sets:
        m = 0
        for j in s:
            m |= 1 << j
        masks.append(m)
    return np.array(masks, dtype=np.uint64)


def request_slots(page_row, n_keys: int, page_size: int) -> np.ndarray:
    """Physical pool slot of each logical key 0..n_keys-1 of one request."""
    p = np.arange(n_keys, dtype=np.int64)
    pages = np.asarray(page_row, dtype=np.int64)[p // page_size]
    if n_keys and pages.min() < 0:
        raise ValueError("page table row holds a negative page id inside seq_len")
    return pages * page_size + p % page_size


def visible_positions(n_keys: int, parents) -> list:
    """Visible(i) as sorted arrays of logical key positions."""
    t = len(parents)
    c = n_keys - t
    if c < 0:
        raise ValueError("seq_len must count the tree rows (seq_len >= T)")
    sets = ancestor_sets(parents)
    ctx = np.arange(c, dtype=np.int64)
    return [np.concatenate([ctx, c + np.array(sorted(s), dtype=np.int64)]) for s in sets]


def _gather_rows(kv_bits, slots, num_slots):
    if slots.size and (slots.min() < 0 or slots.max() >= num_slots):
        raise ValueError("slot outside the KV pool")
    return bf16_bits_to_f64(kv_bits[slots])


def oracle_verify(q_bits, kv_bits, page_table, seq_lens, tree_parent, page_size: int,
                  sm_scale: float):
    """Masked MLA verify attention by its definition (module docstring).

    Returns (out, lse): float64 [B, T, H, 512] and float64 [B, T, H]."""
    q_bits = np.asarray(q_bits)
    b_n, t_n, h_n, d = q_bits.shape
    if d != QK_DIM:
        raise ValueError("query width must be 576")
    out = np.zeros((b_n, t_n, h_n, V_DIM), dtype=np.float64)
    lse = np.zeros((b_n, t_n, h_n), dtype=np.float64)
    num_slots = kv_bits.shape[0]
    for b in range(b_n):
        n = int(seq_lens[b])
        slots = request_slots(page_table[b], n, page_size)
        k = _gather_rows(kv_bits, slots, num_slots)  # [N, 576]
        v = k[:, :V_DIM]  # the value is the leading 512 entries of the same row
        visible = np.zeros((t_n, n), dtype=bool)
        for i, pos in enumerate(visible_positions(n, tree_parent[b])):
            visible[i, pos] = True
        qb = bf16_bits_to_f64(q_bits[b])  # [T, H, 576]
        s = sm_scale * (qb.reshape(t_n * h_n, QK_DIM) @ k.T).reshape(t_n, h_n, n)
        s = np.where(visible[:, None, :], s, -np.inf)
        m = s.max(axis=2, keepdims=True)
        z = np.exp(s - m).sum(axis=2, keepdims=True)
        l_row = m + np.log(z)
        w = np.exp(s - l_row)  # exp(-inf) = 0 for keys a node does not see
        out[b] = (w.reshape(t_n * h_n, n) @ v).reshape(t_n, h_n, V_DIM)
        lse[b] = l_row[..., 0]
    return out, lse


def oracle_split_combine(q_bits, kv_bits, page_table, seq_lens, tree_parent, page_size: int,
                         sm_scale: float, nsplit: int):
    """The split-KV form: each request's keys 0..N-1 are cut into nsplit chunks
    of ceil(N / nsplit) keys (trailing chunks may be empty); each chunk yields a
    normalised partial output and the log-sum-exp of its visible scores; the
    partials are merged with weights exp(lse_s - lse). Equal to oracle_verify in
    exact arithmetic; used only to check that identity."""
    b_n, t_n, h_n, _ = q_bits.shape
    out = np.zeros((b_n, t_n, h_n, V_DIM), dtype=np.float64)
    lse = np.zeros((b_n, t_n, h_n), dtype=np.float64)
    for b in range(b_n):
        n = int(seq_lens[b])
        slots = request_slots(page_table[b], n, page_size)
        k = _gather_rows(kv_bits, slots, kv_bits.shape[0])
        v = k[:, :V_DIM]
        vis = visible_positions(n, tree_parent[b])
        qb = bf16_bits_to_f64(q_bits[b])
        chunk = -(-n // nsplit)
        for i in range(t_n):
            parts = []
            for s_idx in range(nsplit):
                lo, hi = s_idx * chunk, min(n, (s_idx + 1) * chunk)
                sel = vis[i][(vis[i] >= lo) & (vis[i] < hi)]
                if sel.size == 0:
                    continue  # an empty chunk contributes nothing
                sc = sm_scale * (qb[i] @ k[sel].T)
                m = sc.max(axis=1, keepdims=True)
                z = np.exp(sc - m).sum(axis=1, keepdims=True)
                l_s = m + np.log(z)
                o_s = np.exp(sc - l_s) @ v[sel]
                parts.append((o_s, l_s[:, 0]))
            lses = np.stack([p[1] for p in parts])  # [S, H]
            big = lses.max(axis=0)
            wts = np.exp(lses - big)
            tot = wts.sum(axis=0)
            lse[b, i] = big + np.log(tot)
            out[b, i] = sum(wts[s][:, None] * parts[s][0] for s in range(len(parts))) / tot[:, None]
    return out, lse


def brute_force_verify(q_bits, kv_bits, page_table, seq_lens, tree_parent, page_size: int,
                       sm_scale: float):
    """Scalar pure-Python rendering of the same definition, for tiny inputs:
    a dense boolean visibility matrix is built by walking parent links one step
    at a time, and every dot product, exponential and sum is a Python float
    loop. Returns nested lists out[b][i][h][c] and lse[b][i][h]."""
    b_n, t_n, h_n, _ = np.asarray(q_bits).shape

    def dec(x):
        bits = int(x) << 16
        return float(np.array([bits], dtype=np.uint32).view(np.float32)[0])

    out, lse = [], []
    for b in range(b_n):
        n = int(seq_lens[b])
        c = n - t_n
        rows = []
        for p in range(n):
            page = int(page_table[b][p // page_size])
            rows.append(page * page_size + p % page_size)
        # dense visibility: visible[i][p]
        visible = [[False] * n for _ in range(t_n)]
        for i in range(t_n):
            for p in range(c):
                visible[i][p] = True
            j = i
            while j != -1:
                visible[i][c + j] = True
                j = int(tree_parent[b][j])
        ob, lb = [], []
        for i in range(t_n):
            oi, li = [], []
            for h in range(h_n):
                qv = [dec(x) for x in q_bits[b][i][h]]
                scores = []
                for p in range(n):
                    if not visible[i][p]:
                        continue
                    kr = kv_bits[rows[p]]
                    acc = 0.0
                    for dd in range(QK_DIM):
                        acc += qv[dd] * dec(kr[dd])
                    scores.append((p, sm_scale * acc))
                mx = max(sv for _, sv in scores)
                z = 0.0
                for _, sv in scores:
                    z += math.exp(sv - mx)
                l_val = mx + math.log(z)
                o = [0.0] * V_DIM
                for p, sv in scores:
                    w = math.exp(sv - l_val)
                    kr = kv_bits[rows[p]]
                    for cc in range(V_DIM):
                        o[cc] += w * dec(kr[cc])
                oi.append(o)
                li.append(l_val)
            ob.append(oi)
            lb.append(li)
        out.append(ob)
        lse.append(lb)
    return out, lse


def oracle_case(case, split: int | None = None):
    """Run the oracle on a workloads Case (split=None: the plain definition;
    split=S: the split-KV form with S chunks)."""
    args = (case.q, case.kv, case.page_table, case.seq_lens, case.tree_parent,
            case.page_size, case.sm_scale)
    if split is None:
        return oracle_verify(*args)
    return oracle_split_combine(*args, nsplit=split)

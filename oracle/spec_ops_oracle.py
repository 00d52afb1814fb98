"""Plain CPU oracles for the steps that sit next to the verify attention of tree
speculative decoding: sparse top-k MLA decode, the greedy tree accept, the KV
append before verify and the commit (with optional relocation) after it, the
sliding-window page-aligned gather of a draft cache, and the fp8 indexer
logits over a paged cache.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. Nothing on the product path imports it,
and it shares no code with the HIP path. Integers are exact; floating point is
float64 with exact decoding of the bf16 / e4m3 inputs.

Sources, by function (the readings taken where a page is silent are stated in
each docstring and collected in the repository's design notes):
  * sparse_decode: page "The 24% Ceiling: When Configuration Tuning Meets the
    sm_120 Kernel Wall", section "The Decisive Profile: 63% in One Kernel": a sparse MLA decode attends each head of one query token to a
    request's 512 top-k selected tokens; the fix it proposes adds a split over
    the selected tokens to the grid. This is the plain definition: softmax
    attention over the listed latent rows, all heads sharing them (MLA).
  * tree_accept, kv_append, commit_accepted: page "The Custom sm_120 Verify
    Kernel: From 0.7 tok/s to 3-6x Decode Speedup on Blackwell Consumer GPUs",
    Part II (avg_commit_len = 1.00 means one token per step), Part IV (commit
    lengths of 7-8 with draft depth 6-7), Part IX Bug 2 (the draft tokens' KV is
    written to its own pool slots, out_cache_loc, before attention), Part VIII
    and the capstone report's section 3 (tier-1 live relocation of scattered
    slots).
  * window_start, compact_len, window_map: page "One Blocking Memcpy Per Verify
    Step", section "The sync, and the bound that replaced it".
  * e4m3_to_f64, indexer_logits: page "The Indexer Breakthrough: Implementing a
    Capture-Safe Triton Kernel for O(actual_seq) Inference", sections
    "The Technical Context" and "Design Decisions and Assumptions".
"""

from __future__ import annotations

import math

import numpy as np

QK_DIM = 576
V_DIM = 512
IDX_DIM = 128          # fp8 values per cached indexer position
IDX_PAGE = 64          # positions per cache block
IDX_BLOCK_BYTES = 8448  # 64 x 128 fp8 values, then 64 fp32 scales


def _bf16_to_f64(bits) -> np.ndarray:
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- sparse top-k decode

def sparse_keys(indices_row, length: int | None) -> np.ndarray:
    """The key slots of one request: the first `length` entries of its index
    list (all of them when length is None) that are not -1. An entry of -1
    marks an unused place in the list; any other negative entry is an error."""
    row = np.asarray(indices_row, dtype=np.int64)
    if length is not None:
        row = row[:max(0, int(length))]
    if np.any(row < -1):
        raise ValueError("index below -1")
    return row[row >= 0]


def sparse_decode(q_bits, kv_bits, indices, lens, sm_scale: float):
    """Sparse MLA decode by its definition. q_bits uint16 [B, H, 576] (one
    query token per request, H heads), kv_bits uint16 [slots, 576], indices
    int32 [B, K] (pool slots, -1 = unused), lens int32 [B] or None (entries of
    the list in use). For request b, head h, with keys S_b = sparse_keys(...):
      s_j = sm_scale * q[b,h,:] . kv[j, 0:576]   for each listed slot j,
      lse = ln sum_j exp(s_j),  out = sum_j exp(s_j - lse) kv[j, 0:512].
    A slot listed twice counts twice (the list is a multiset). A request with no
    key gets lse = -inf and out = 0. Returns float64 (out [B,H,512], lse [B,H])."""
    q_bits = np.asarray(q_bits)
    b_n, h_n, d = q_bits.shape
    if d != QK_DIM:
        raise ValueError("query width must be 576")
    out = np.zeros((b_n, h_n, V_DIM))
    lse = np.full((b_n, h_n), -np.inf)
    for b in range(b_n):
        keys = sparse_keys(indices[b], None if lens is None else lens[b])
        if keys.size == 0:
            continue
        if keys.max() >= kv_bits.shape[0]:
            raise ValueError("slot outside the KV pool")
        k = _bf16_to_f64(kv_bits[keys])
        s = sm_scale * (_bf16_to_f64(q_bits[b]) @ k.T)  # [H, n]
        m = s.max(axis=1, keepdims=True)
        lrow = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
        out[b] = np.exp(s - lrow) @ k[:, :V_DIM]
        lse[b] = lrow[:, 0]
    return out, lse


# ---------------------------------------------------------------- greedy tree accept

def tree_accept(tree_parent, draft_tokens, target_tokens):
    """Greedy acceptance of a draft tree after the verify forward.

    Reading taken (the pages give the outcome, not the rule): node i carries
    the draft token draft_tokens[i]; target_tokens[i] is the target model's
    greedy choice for the token that follows node i. A root (parent -1) holds
    the token fixed by the previous step and is accepted as it stands. Any
    other node is accepted iff its parent is accepted and its draft token equals
    the target's choice after its parent. The step keeps the deepest accepted
    node (the smallest index among equally deep ones), commits the draft tokens
    on the path below the root and then the target's choice after that node:
    depth + 1 tokens, so a step where no draft matches commits exactly one token
    (avg_commit_len = 1.00 on the verify-kernel page, Part II).

    Returns int32 arrays: accept_len [B]; path [B, T], the node indices from
    the root to the kept node then -1; commit_tokens [B, T], the committed
    tokens then -1. Raises on a parent that is not an earlier node."""
    par = np.asarray(tree_parent, dtype=np.int64)
    drf = np.asarray(draft_tokens, dtype=np.int64)
    tgt = np.asarray(target_tokens, dtype=np.int64)
    b_n, t_n = par.shape
    accept_len = np.zeros(b_n, dtype=np.int32)
    path = np.full((b_n, t_n), -1, dtype=np.int32)
    commit = np.full((b_n, t_n), -1, dtype=np.int32)
    for b in range(b_n):
        accepted = [False] * t_n
        depth = [0] * t_n
        for i in range(t_n):
            p = int(par[b, i])
            if p < -1 or p >= i:
                raise ValueError(f"node {i} has parent {p}")
            if p == -1:
                accepted[i], depth[i] = True, 0
            else:
                accepted[i] = accepted[p] and int(drf[b, i]) == int(tgt[b, p])
                depth[i] = depth[p] + 1
        best = None
        for i in range(t_n):
            if accepted[i] and (best is None or depth[i] > depth[best]):
                best = i
        chain = []
        j = best
        while j != -1:
            chain.append(j)
            j = int(par[b, j])
        chain.reverse()
        accept_len[b] = len(chain)
        path[b, :len(chain)] = chain
        toks = [int(drf[b, j]) for j in chain[1:]] + [int(tgt[b, best])]
        commit[b, :len(toks)] = toks
    return accept_len, path, commit


# ---------------------------------------------------------------- KV append and commit

def kv_append(kv_bits, new_rows, out_cache_loc):
    """The draft tokens' latent rows written to their own pool slots before the
    verify attention (verify-kernel page, Part IX, Bug 2): row r of new_rows goes
    to slot out_cache_loc[r]. Returns a new pool; raises on a slot outside it or
    on a slot named twice."""
    loc = np.asarray(out_cache_loc, dtype=np.int64)
    if loc.size and (loc.min() < 0 or loc.max() >= kv_bits.shape[0]):
        raise ValueError("slot outside the pool")
    if len(set(loc.tolist())) != loc.size:
        raise ValueError("slot named twice")
    out = np.array(kv_bits, copy=True)
    for r, s in enumerate(loc.tolist()):
        out[s] = new_rows[r]
    return out


def commit_accepted(page_table, seq_lens, num_nodes: int, accept_len, path, dest_slots=None, kv_bits=None):
    """The commit after an accept, for a page-size-1 pool (the tree's rows sit
    at logical keys C..C+T-1 of the request, C = seq_lens - T). The rows of the
    accepted path become the next committed keys C..C+accept_len-1, in path
    order; the other tree rows' slots are released. With dest_slots [B, T] the
    accepted rows are also moved: row k of the path is copied to dest_slots[b][k]
    and the page table names the new slot (live relocation of scattered slots,
    verify-kernel page Part VIII; capstone report section 3).

    Returns (page_table', context_lens', freed [B, T] (released slots in node
    order, then -1), kv') where kv' is None unless dest_slots is given."""
    pt = np.array(page_table, dtype=np.int64, copy=True)
    b_n = pt.shape[0]
    t = int(num_nodes)
    ctx_out = np.zeros(b_n, dtype=np.int32)
    freed = np.full((b_n, t), -1, dtype=np.int32)
    kv_out = None if dest_slots is None else np.array(kv_bits, copy=True)
    for b in range(b_n):
        c = int(seq_lens[b]) - t
        tree_slots = [int(pt[b, c + j]) for j in range(t)]
        n_acc = int(accept_len[b])
        chain = [int(path[b, k]) for k in range(n_acc)]
        for k, j in enumerate(chain):
            src = tree_slots[j]
            if dest_slots is None:
                pt[b, c + k] = src
            else:
                dst = int(dest_slots[b][k])
                kv_out[dst] = kv_bits[src]
                pt[b, c + k] = dst
        keep = set(chain)
        rel = [tree_slots[j] for j in range(t) if j not in keep]
        freed[b, :len(rel)] = rel
        ctx_out[b] = c + n_acc
    return pt.astype(np.int32), ctx_out, freed, kv_out


# ---------------------------------------------------------------- sliding-window gather

def window_start(length: int, window: int, page: int) -> int:
    """s(L) = floor((L - min(L, W)) / P) * P, the page-aligned start of the
    window ("One Blocking Memcpy Per Verify Step", section "The sync, and the
    bound that replaced it")."""
    return ((length - min(length, window)) // page) * page


def compact_len(length: int, window: int, page: int) -> int:
    """c(L) = L - s(L), the compact length resident in the draft cache."""
    return length - window_start(length, window, page)


def window_map(target_map, lens, window: int, page: int):
    """The fixed-shape rectangle of the same section: width W + P - 1; for
    request i and column j, draft_map[i][j] = target_map[i][s(L_i) + j] when
    j < c(L_i). The page leaves the other columns unspecified; here they are -1.
    Returns (draft_map int32 [B, W + P - 1], compact lengths int32 [B])."""
    tm = np.asarray(target_map)
    b_n = tm.shape[0]
    width = window + page - 1
    out = np.full((b_n, width), -1, dtype=np.int32)
    cl = np.zeros(b_n, dtype=np.int32)
    for i in range(b_n):
        length = int(lens[i])
        if length < 0 or length > tm.shape[1]:
            raise ValueError("length outside the target map")
        s, c = window_start(length, window, page), compact_len(length, window, page)
        for j in range(c):
            out[i, j] = tm[i, s + j]
        cl[i] = c
    return out, cl


# ---------------------------------------------------------------- fp8 indexer logits

def e4m3_to_f64(codes) -> np.ndarray:
    """Decode fp8 E4M3 codes (the OCP "FN" form: 1 sign, 4 exponent bits with
    bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest 448):
    exponent field 0 is subnormal, value (m / 8) * 2^-6; otherwise
    (1 + m / 8) * 2^(e - 7)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def indexer_block_fields(block_bytes):
    """Split one 8,448-byte cache block into its 64 x 128 fp8 codes and its 64
    fp32 scales (the layout the indexer page states)."""
    blk = np.asarray(block_bytes, dtype=np.uint8)
    if blk.shape[-1] != IDX_BLOCK_BYTES:
        raise ValueError("a block holds 8,448 bytes")
    codes = blk[..., :IDX_PAGE * IDX_DIM].reshape(blk.shape[:-1] + (IDX_PAGE, IDX_DIM))
    scales = np.ascontiguousarray(blk[..., IDX_PAGE * IDX_DIM:]).view(np.float32)
    return codes, scales.astype(np.float64)


def indexer_logits(q_codes, weights, blocks, block_table, seq_lens):
    """DSA indexer logits by the definition on the indexer page: for request b
    and cached position p < seq_lens[b], with block = block_table[b][p // 64],
    k = e4m3(codes of row p % 64 of that block), s = its fp32 scale,
      logits[b, p] = ( sum_h weights[b, h] * max(0, q[b, h, :] . k) ) * s
    (query vectors are the raw e4m3 values, no separate scale); positions p >=
    seq_lens[b], up to the width max_blocks * 64, are -inf. Returns float64
    [B, max_blocks * 64]."""
    q = e4m3_to_f64(q_codes)                         # [B, H, 128]
    w = np.asarray(weights, dtype=np.float64)        # [B, H]
    bt = np.asarray(block_table, dtype=np.int64)
    b_n, max_blocks = bt.shape
    out = np.full((b_n, max_blocks * IDX_PAGE), -np.inf)
    for b in range(b_n):
        n = int(seq_lens[b])
        if n < 0 or n > max_blocks * IDX_PAGE:
            raise ValueError("seq_len outside the block table")
        for pg in range(-(-n // IDX_PAGE)):
            blk = int(bt[b, pg])
            if blk < 0 or blk >= blocks.shape[0]:
                raise ValueError("block id outside the cache")
            codes, scales = indexer_block_fields(blocks[blk])
            k = e4m3_to_f64(codes)                   # [64, 128]
            dots = k @ q[b].T                        # [64 positions, H]
            val = (np.maximum(dots, 0.0) * w[b][None, :]).sum(axis=1) * scales
            lo = pg * IDX_PAGE
            hi = min(n, lo + IDX_PAGE)
            out[b, lo:hi] = val[:hi - lo]
    return out


def indexer_magnitude(q_codes, weights, blocks, block_table, seq_lens):
    """sum_h |w_h| * sum_d |q_hd * k_pd| * |s_p| per position (0 past seq_len):
    the scale of the terms an fp32 evaluation of indexer_logits adds, which
    bounds its rounding error."""
    q = np.abs(e4m3_to_f64(q_codes))
    w = np.abs(np.asarray(weights, dtype=np.float64))
    bt = np.asarray(block_table, dtype=np.int64)
    b_n, max_blocks = bt.shape
    out = np.zeros((b_n, max_blocks * IDX_PAGE))
    for b in range(b_n):
        n = int(seq_lens[b])
        for pg in range(-(-n // IDX_PAGE)):
            codes, scales = indexer_block_fields(blocks[int(bt[b, pg])])
            mag = (np.abs(e4m3_to_f64(codes)) @ q[b].T) @ w[b] * np.abs(scales)
            lo = pg * IDX_PAGE
            hi = min(n, lo + IDX_PAGE)
            out[b, lo:hi] = mag[:hi - lo]
    return out


def brute_force_indexer(q_codes, weights, blocks, block_table, seq_lens):
    """The same definition as scalar loops over heads, dimensions and bytes,
    decoding each e4m3 byte from its bit fields one at a time; for tiny inputs."""
    def dec(x):
        x = int(x)
        s = -1.0 if x & 0x80 else 1.0
        e, m = (x >> 3) & 15, x & 7
        return s * (m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))

    b_n, max_blocks = np.asarray(block_table).shape
    h_n = np.asarray(q_codes).shape[1]
    out = [[-math.inf] * (max_blocks * IDX_PAGE) for _ in range(b_n)]
    for b in range(b_n):
        for p in range(int(seq_lens[b])):
            blk = blocks[int(block_table[b][p // IDX_PAGE])]
            r = p % IDX_PAGE
            scale = float(np.frombuffer(bytes(blk[IDX_PAGE * IDX_DIM + 4 * r:IDX_PAGE * IDX_DIM + 4 * r + 4]),
                                        dtype=np.float32)[0])
            tot = 0.0
            for h in range(h_n):
                dot = 0.0
                for d in range(IDX_DIM):
                    dot += dec(q_codes[b][h][d]) * dec(blk[r * IDX_DIM + d])
                tot += float(weights[b][h]) * max(0.0, dot)
            out[b][p] = tot * scale
    return out

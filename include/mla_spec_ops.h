/*
 * mla_spec_ops.h - C ABI of the MI355X (gfx950) kernels for the steps next to
 * the verify attention in tree speculative decoding: sparse top-k MLA decode,
 * the draft rows' KV append, the greedy tree accept, the commit of the
 * accepted path (with optional relocation of its rows), the page-aligned
 * sliding-window gather of a draft cache and the fp8 indexer logits.
 *
 * Conventions are those of mla_verify.h: every pointer is device memory owned
 * by the caller; nothing here allocates, synchronises, copies to the host or
 * reads the environment, so every call may be captured into a hipGraph; the
 * launch shape depends only on the host-side arguments; a negative status
 * means nothing was enqueued (MLA_ERR_HIP: a launch failed); bad data only
 * sets sticky bits in a caller-provided uint32 device error word (nullable
 * where noted) and gets the stated fallback.
 */
#ifndef MLA_SPEC_OPS_H
#define MLA_SPEC_OPS_H

#include "mla_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Sticky bits used only by these entry points (the verify bits keep their
 * meaning). */
#define MLA_DEVERR_INDEX_RANGE 8u /* an accept length, path entry or length outside its range: clamped */

/* ------------------------------------------------------------------ sparse top-k decode
 * Page "The 24% Ceiling: When Configuration Tuning Meets the sm_120 Kernel
 * Wall", sections "The Decisive Profile" and "The
 * Path Forward": a sparse MLA decode attends each head of one query token to
 * the request's 512 selected (top-k) latent rows; the remedy the page names is
 * a split of the selected tokens across the grid. Definition, per request b
 * and head h, over the listed slots S_b = {indices[b][j] : j < lens[b],
 * indices[b][j] != -1}:
 *   s_j = sm_scale * <q[b,h,:], kv_cache[j, 0:576]>,
 *   lse[b,h] = ln sum_j exp(s_j),  out[b,h,:] = sum_j exp(s_j - lse) kv_cache[j, 0:512].
 * A slot listed twice counts twice. A request with no listed slot gets
 * lse = -inf and out = 0. All heads read the same rows (one latent per token). */
typedef struct {
  int32_t batch;         /* B >= 1 requests, one query token each */
  int32_t num_heads;     /* H >= 1 query heads */
  int32_t head_dim_qk;   /* must be 576 */
  int32_t head_dim_v;    /* must be 512 */
  int32_t topk;          /* K >= 1: width of a row of `indices` */
  int32_t nsplit;        /* >= 1: splits of each index list (results do not depend on it beyond rounding) */
  int64_t num_kv_slots;  /* rows in kv_cache */
  int64_t kv_row_stride; /* elements between kv_cache rows: >= 576, multiple of 8, <= 2^30 */
  float sm_scale;
} mla_sparse_desc;

/* Workspace bytes for mla_sparse_decode (0 for a descriptor it would reject).
 * The first 4 bytes are the sticky device error word. */
MLA_API size_t mla_sparse_decode_workspace_bytes(const mla_sparse_desc* d);

/*   q:        bf16 [B, H, 576], 16-byte aligned.
 *   kv_cache: bf16 [num_kv_slots, kv_row_stride], 16-byte aligned.
 *   indices:  int32 [B, topk]: pool slots; -1 marks an unused entry (skipped,
 *             no error); a slot < -1 or >= num_kv_slots is skipped and sets
 *             MLA_DEVERR_SLOT_RANGE.
 *   lens:     int32 [B] entries of each row in use, or NULL for all topk; a
 *             value outside [0, topk] is clamped and sets MLA_DEVERR_SEQ_LEN.
 *   out:      bf16 [B, H, 512] (fp32 accumulation, one rounding); lse: fp32 [B, H].
 *   workspace: >= mla_sparse_decode_workspace_bytes(d), 16-byte aligned.
 * Errors as for mla_verify_attention. */
MLA_API mla_status mla_sparse_decode(const mla_sparse_desc* d, const void* q, const void* kv_cache,
                                     const int32_t* indices, const int32_t* lens, void* out, float* lse,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ KV append before verify
 * Page "The Custom sm_120 Verify Kernel: From 0.7 tok/s to 3-6x Decode Speedup
 * on Blackwell Consumer GPUs", Part IX, Bug 2: the draft tokens' latent rows
 * are computed fresh and written to their own pool slots (out_cache_loc)
 * before the verify attention reads them as the last T keys of each request.
 *   kv_cache[out_cache_loc[r], 0:576] = new_rows[r, 0:576] for r < n.
 *   kv_cache:      bf16 [num_kv_slots, kv_row_stride], written; 16-byte aligned.
 *   new_rows:      bf16 [n, 576] row-contiguous, 16-byte aligned.
 *   out_cache_loc: int32 [n]; a slot outside [0, num_kv_slots) is skipped and
 *                  sets MLA_DEVERR_SLOT_RANGE. Two rows naming one slot race.
 *   dev_err:       nullable.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (n < 0, bad stride), MLA_ERR_ALIGN, MLA_ERR_HIP.
 * n = 0 enqueues nothing. */
MLA_API mla_status mla_kv_append(void* kv_cache, int64_t num_kv_slots, int64_t kv_row_stride, const void* new_rows,
                                 const int32_t* out_cache_loc, int32_t n, uint32_t* dev_err, hipStream_t stream);

/* ------------------------------------------------------------------ greedy tree accept
 * The verify-kernel page, Part II (avg_commit_len = 1.00: one token per step
 * when no draft is accepted) and Part IV (commit lengths of 7-8 tokens with
 * draft depth 6-7). Rule (the pages give outcomes, not the rule; this is the
 * plain greedy reading): node i carries draft_tokens[i]; target_tokens[i] is
 * the target model's greedy choice for the token after node i. A root
 * (tree_parent = -1) holds the token fixed by the previous step and is
 * accepted. Another node is accepted iff its parent is accepted and
 * draft_tokens[i] == target_tokens[parent(i)]. The deepest accepted node is
 * kept (the smallest index among equally deep ones); the step commits the
 * draft tokens of the path below the root, then the target's choice after the
 * kept node: depth + 1 tokens.
 *   tree_parent, draft_tokens, target_tokens: int32 [B, T], T in [1, 64].
 *   accept_len:    int32 [B], written: depth + 1.
 *   accept_path:   int32 [B, T], written: node indices root..kept node, then -1.
 *   commit_tokens: int32 [B, T], written: committed tokens, then -1 (nullable).
 *   dev_err:       nullable; a parent outside [-1, i) sets MLA_DEVERR_BAD_PARENT
 *                  and the node is read as a root.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_HIP. */
MLA_API mla_status mla_tree_accept(const int32_t* tree_parent, const int32_t* draft_tokens,
                                   const int32_t* target_tokens, int32_t batch, int32_t num_nodes,
                                   int32_t* accept_len, int32_t* accept_path, int32_t* commit_tokens,
                                   uint32_t* dev_err, hipStream_t stream);

/* ------------------------------------------------------------------ commit of the accepted path
 * After the accept, on a page-size-1 pool (the verify-kernel page, Part VI:
 * accepted nodes sit on scattered slots): the tree rows of request b are its
 * logical keys C..C+T-1 (C = seq_lens[b] - T); the rows of the accepted path
 * become its next committed keys C..C+accept_len-1 in path order, the page
 * table names their slots and the other tree slots are released. With
 * dest_slots the accepted rows are also moved, row k of the path to
 * dest_slots[b][k], and the page table names the new slots: the live
 * relocation of scattered slots (the verify-kernel page, Part VIII, tier 1;
 * "The Capstone Report: When Kernel Engineering Meets Honest Bottleneck
 * Analysis", section 3). Source and destination rows of one request may
 * overlap (all are read before any is written); different requests must not
 * share slots.
 *   page_table:   int32 [B, max_pages], entries C..C+accept_len-1 rewritten.
 *   seq_lens:     int32 [B], the verify call's lengths (tree rows included).
 *   accept_len, accept_path: as written by mla_tree_accept.
 *   context_lens: int32 [B], written: C + accept_len.
 *   freed_slots:  int32 [B, T], written: released slots in node order, then -1 (nullable).
 *   kv_cache, dest_slots: both NULL (no move) or both set; kv_cache bf16
 *                 [num_kv_slots, kv_row_stride], dest_slots int32 [B, T].
 *   dev_err:      nullable. A seq_len outside [T, max_pages], an accept_len
 *                 outside [1, T] or a path entry outside [0, T) sets
 *                 MLA_DEVERR_INDEX_RANGE and is clamped; a slot outside the
 *                 pool sets MLA_DEVERR_SLOT_RANGE and that row is not moved.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ALIGN, MLA_ERR_HIP. */
MLA_API mla_status mla_commit_accepted(int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                                       int32_t batch, int32_t num_nodes, const int32_t* accept_len,
                                       const int32_t* accept_path, int32_t* context_lens, int32_t* freed_slots,
                                       void* kv_cache, int64_t num_kv_slots, int64_t kv_row_stride,
                                       const int32_t* dest_slots, uint32_t* dev_err, hipStream_t stream);

/* ------------------------------------------------------------------ accept and commit in one launch
 * mla_tree_accept followed by mla_commit_accepted (the verify-kernel page,
 * Part II and Part IV for the accept, Part VI and Part VIII for the commit),
 * one workgroup per request: the accept's outputs are written exactly as
 * mla_tree_accept writes them, and the commit takes the path from on-chip
 * memory rather than reading accept_len / accept_path back. The results equal
 * those of the two calls in sequence.
 *   tree_parent, draft_tokens, target_tokens, accept_len, accept_path,
 *   commit_tokens: as for mla_tree_accept (accept_len and accept_path are
 *                  written; commit_tokens nullable).
 *   page_table, max_pages, seq_lens, context_lens, freed_slots, kv_cache,
 *   num_kv_slots, kv_row_stride, dest_slots: as for mla_commit_accepted.
 *   dev_err:       nullable; MLA_DEVERR_BAD_PARENT as for mla_tree_accept,
 *                  MLA_DEVERR_INDEX_RANGE for a seq_len outside [T, max_pages]
 *                  (clamped), MLA_DEVERR_SLOT_RANGE as for mla_commit_accepted.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ALIGN, MLA_ERR_HIP. */
MLA_API mla_status mla_accept_commit(const int32_t* tree_parent, const int32_t* draft_tokens,
                                     const int32_t* target_tokens, int32_t batch, int32_t num_nodes,
                                     int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                                     int32_t* accept_len, int32_t* accept_path, int32_t* commit_tokens,
                                     int32_t* context_lens, int32_t* freed_slots, void* kv_cache,
                                     int64_t num_kv_slots, int64_t kv_row_stride, const int32_t* dest_slots,
                                     uint32_t* dev_err, hipStream_t stream);

/* ------------------------------------------------------------------ sliding-window gather
 * Page "One Blocking Memcpy Per Verify Step", section "The sync, and the bound
 * that replaced it": a draft model keeps the most recent W tokens in a cache
 * of P-token pages; the window's start is page-aligned,
 *   s(L) = floor((L - min(L, W)) / P) * P,  c(L) = L - s(L) <= min(L, W + P - 1),
 * and its slot map is a fixed-shape rectangle of width W + P - 1 computed on
 * the device from the exact lengths:
 *   draft_map[i][j] = target_map[i][s(L_i) + j] for j < c(L_i), else -1.
 *   target_map:   int32 [B, map_stride] per-token slot map of each request.
 *   lens:         int32 [B] exact lengths L_i; outside [0, map_stride] they are
 *                 clamped and set MLA_DEVERR_SEQ_LEN.
 *   draft_map:    int32 [B, W + P - 1], written.
 *   compact_lens: int32 [B], written c(L_i) (nullable).
 *   dev_err:      nullable.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (B < 1, W < 1, P < 1, map_stride < 1), MLA_ERR_HIP. */
MLA_API mla_status mla_window_map(const int32_t* target_map, int32_t map_stride, const int32_t* lens, int32_t batch,
                                  int32_t window, int32_t page, int32_t* draft_map, int32_t* compact_lens,
                                  uint32_t* dev_err, hipStream_t stream);

/* ------------------------------------------------------------------ fp8 indexer logits
 * Page "The Indexer Breakthrough: Implementing a Capture-Safe Triton Kernel
 * for O(actual_seq) Inference", sections "The Technical Context" and
 * "Design Decisions and Assumptions": the DSA indexer scores every cached
 * position of a request: q . k per head, ReLU, times a per-head weight, summed
 * over heads, times the position's scale. The cache is paged in blocks of
 * 8,448 bytes: 64 positions x 128 fp8 E4M3 values, then 64 fp32 scales. A
 * fixed grid of persistent waves streams runs of half-blocks; blocks past a
 * request's length are not read and only get -inf.
 *   logits[b][p] = ( sum_h weights[b][h] * max(0, q[b,h,:] . k_p) ) * scale_p
 * for p < seq_lens[b], with k_p row p % 64 of block block_table[b][p / 64]
 * (E4M3, OCP form, no separate query scale); -inf for p in [seq_lens[b],
 * max_blocks * 64). fp32 accumulation. */
typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t num_heads;   /* H in [1, 64] */
  int32_t head_dim;    /* must be 128 */
  int32_t max_blocks;  /* columns of block_table; logits rows hold max_blocks * 64 */
  int64_t num_blocks;  /* blocks in kv_blocks */
} mla_indexer_desc;

/*   q:           uint8 [B, H, 128] E4M3 codes, 16-byte aligned.
 *   weights:     fp32 [B, H].
 *   kv_blocks:   uint8 [num_blocks, 8448], 16-byte aligned.
 *   block_table: int32 [B, max_blocks]; entries past ceil(seq_lens[b] / 64)
 *                are never read; an out-of-range block id sets
 *                MLA_DEVERR_SLOT_RANGE and its positions get -inf.
 *   seq_lens:    int32 [B] positions; outside [0, max_blocks * 64] clamped
 *                with MLA_DEVERR_SEQ_LEN.
 *   logits:      fp32 [B, max_blocks * 64], written.
 *   dev_err:     nullable.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED (head_dim != 128,
 * H > 64), MLA_ERR_ALIGN, MLA_ERR_HIP. */
MLA_API mla_status mla_indexer_logits(const mla_indexer_desc* d, const uint8_t* q, const float* weights,
                                      const uint8_t* kv_blocks, const int32_t* block_table,
                                      const int32_t* seq_lens, float* logits, uint32_t* dev_err,
                                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_SPEC_OPS_H */

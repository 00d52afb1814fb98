// C ABI of the steps next to the verify attention (mla_spec_ops.h): argument
// checks and launches. Nothing here reads device memory, synchronises or
// allocates, so every entry point may be captured into a hipGraph.

#include <stdint.h>

#include <cmath>
#include <limits>

#include "mla_spec_ops.h"
#include "mla_spec_ops_internal.h"
#include "mla_verify_internal.h"

namespace {

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

mla_status launched(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

mla_status check_sparse(const mla_sparse_desc* d) {
  if (d == nullptr) return MLA_ERR_NULL;
  if (d->head_dim_qk != mlav::kQkDim || d->head_dim_v != mlav::kVDim) return MLA_ERR_UNSUPPORTED;
  if (d->batch < 1 || d->num_heads < 1 || d->topk < 1 || d->nsplit < 1 || d->num_kv_slots < 1) return MLA_ERR_SHAPE;
  if (d->kv_row_stride < mlav::kQkDim || (d->kv_row_stride % 8) != 0) return MLA_ERR_SHAPE;
  if (d->kv_row_stride > mlav::kMaxRowStride) return MLA_ERR_SHAPE;
  if (!std::isfinite(d->sm_scale)) return MLA_ERR_SHAPE;
  if (d->num_kv_slots > std::numeric_limits<int32_t>::max() || d->num_heads > (1 << 20)) return MLA_ERR_SHAPE;
  const mlav::RowPlan rp = mlav::plan_rows(1, d->num_heads);
  if (static_cast<int64_t>(d->batch) * d->nsplit * rp.row_blocks > (1LL << 30)) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(d->batch) * (rp.rows_pad / 32) * 64 > (1LL << 30)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

// Checks shared by the two commit entry points; fills every field of C but
// accept_len and path.
mla_status commit_launch(int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                         int32_t num_nodes, int32_t* context_lens, int32_t* freed_slots, void* kv_cache,
                         int64_t num_kv_slots, int64_t kv_row_stride, const int32_t* dest_slots, uint32_t* dev_err,
                         mlav::CommitLaunch& C) {
  if (page_table == nullptr || seq_lens == nullptr || context_lens == nullptr) return MLA_ERR_NULL;
  if ((kv_cache == nullptr) != (dest_slots == nullptr)) return MLA_ERR_NULL;
  if (batch < 1 || num_nodes < 1 || num_nodes > mlav::kMaxTreeNodes || max_pages < num_nodes) return MLA_ERR_SHAPE;
  if (kv_cache != nullptr) {
    if (num_kv_slots < 1 || num_kv_slots > std::numeric_limits<int32_t>::max() || kv_row_stride < mlav::kQkDim ||
        (kv_row_stride % 8) != 0)
      return MLA_ERR_SHAPE;
    if (misaligned(kv_cache, 16)) return MLA_ERR_ALIGN;
  }
  C.page_table = page_table;
  C.seq_lens = seq_lens;
  C.accept_len = nullptr;
  C.path = nullptr;
  C.context_lens = context_lens;
  C.freed = freed_slots;
  C.kv = static_cast<uint8_t*>(kv_cache);
  C.dest = dest_slots;
  C.err = dev_err;
  C.num_slots = num_kv_slots;
  C.row_bytes = kv_row_stride * 2;
  C.batch = batch;
  C.nodes = num_nodes;
  C.max_pages = max_pages;
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_sparse_decode_workspace_bytes(const mla_sparse_desc* d) {
  if (check_sparse(d) != MLA_OK) return 0;
  const mlav::RowPlan rp = mlav::plan_rows(1, d->num_heads);
  return mlav::workspace_bytes(d->batch, d->nsplit, rp.rows_pad);
}

mla_status mla_sparse_decode(const mla_sparse_desc* d, const void* q, const void* kv_cache, const int32_t* indices,
                             const int32_t* lens, void* out, float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  const mla_status st = check_sparse(d);
  if (st != MLA_OK) return st;
  if (q == nullptr || kv_cache == nullptr || indices == nullptr || out == nullptr || lse == nullptr ||
      workspace == nullptr)
    return MLA_ERR_NULL;
  if (misaligned(q, 16) || misaligned(kv_cache, 16) || misaligned(out, 16) || misaligned(workspace, 16) ||
      misaligned(indices, 4) || misaligned(lens, 4) || misaligned(lse, 4))
    return MLA_ERR_ALIGN;
  const mlav::RowPlan rp = mlav::plan_rows(1, d->num_heads);
  if (workspace_bytes < mlav::workspace_bytes(d->batch, d->nsplit, rp.rows_pad)) return MLA_ERR_WORKSPACE;
  // One query token per request is a verify call with one tree node whose
  // visible keys are the whole list: the index list is a page-size-1 table.
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  mlav::VerifyLaunch L;
  L.q = static_cast<const uint16_t*>(q);
  L.kv = static_cast<const uint8_t*>(kv_cache);
  L.page_table = indices;
  L.seq_lens = lens;
  L.tree_parent = nullptr;
  L.out = static_cast<uint16_t*>(out);
  L.lse = lse;
  L.err = reinterpret_cast<uint32_t*>(ws);
  L.part_lse = reinterpret_cast<float*>(ws + mlav::part_lse_offset());
  L.part_o = reinterpret_cast<uint16_t*>(ws + mlav::part_o_offset(d->batch, d->nsplit, rp.rows_pad));
  L.kv_row_bytes = d->kv_row_stride * 2;
  L.num_slots = d->num_kv_slots;
  L.batch = d->batch;
  L.nodes = 1;
  L.heads = d->num_heads;
  L.rows = rp.rows;
  L.rows_pad = rp.rows_pad;
  L.waves_per_wg = rp.waves_per_wg;
  L.row_blocks = rp.row_blocks;
  L.nsplit = d->nsplit;
  L.page_shift = 0;
  L.max_pages = d->topk;
  L.capacity = d->topk;
  L.min_len = 0;
  L.quiet_unused = 1;
  L.col_parts = mlav::col_parts_for(d->batch, d->nsplit, rp.row_blocks);
  L.scale_log2 = d->sm_scale * 1.4426950408889634f;
  if (mlav::launch_partial(L, stream) != hipSuccess) return MLA_ERR_HIP;
  return launched(mlav::launch_combine(L, stream));
}

mla_status mla_kv_append(void* kv_cache, int64_t num_kv_slots, int64_t kv_row_stride, const void* new_rows,
                         const int32_t* out_cache_loc, int32_t n, uint32_t* dev_err, hipStream_t stream) {
  if (n < 0 || num_kv_slots < 1 || kv_row_stride < mlav::kQkDim || (kv_row_stride % 8) != 0) return MLA_ERR_SHAPE;
  if (num_kv_slots > std::numeric_limits<int32_t>::max()) return MLA_ERR_SHAPE;
  if (kv_cache == nullptr || new_rows == nullptr || out_cache_loc == nullptr) return MLA_ERR_NULL;
  if (misaligned(kv_cache, 16) || misaligned(new_rows, 16) || misaligned(out_cache_loc, 4) || misaligned(dev_err, 4))
    return MLA_ERR_ALIGN;
  if (n == 0) return MLA_OK;
  return launched(mlav::launch_kv_append(static_cast<uint8_t*>(kv_cache), num_kv_slots, kv_row_stride * 2,
                                         static_cast<const uint8_t*>(new_rows), out_cache_loc, n, dev_err, stream));
}

mla_status mla_tree_accept(const int32_t* tree_parent, const int32_t* draft_tokens, const int32_t* target_tokens,
                           int32_t batch, int32_t num_nodes, int32_t* accept_len, int32_t* accept_path,
                           int32_t* commit_tokens, uint32_t* dev_err, hipStream_t stream) {
  if (tree_parent == nullptr || draft_tokens == nullptr || target_tokens == nullptr || accept_len == nullptr ||
      accept_path == nullptr)
    return MLA_ERR_NULL;
  if (batch < 1 || num_nodes < 1 || num_nodes > mlav::kMaxTreeNodes) return MLA_ERR_SHAPE;
  const mlav::AcceptLaunch A{tree_parent, draft_tokens, target_tokens, accept_len, accept_path, commit_tokens, dev_err};
  return launched(mlav::launch_tree_accept(A, batch, num_nodes, stream));
}

mla_status mla_commit_accepted(int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                               int32_t num_nodes, const int32_t* accept_len, const int32_t* accept_path,
                               int32_t* context_lens, int32_t* freed_slots, void* kv_cache, int64_t num_kv_slots,
                               int64_t kv_row_stride, const int32_t* dest_slots, uint32_t* dev_err,
                               hipStream_t stream) {
  if (accept_len == nullptr || accept_path == nullptr) return MLA_ERR_NULL;
  mlav::CommitLaunch C;
  const mla_status st = commit_launch(page_table, max_pages, seq_lens, batch, num_nodes, context_lens, freed_slots,
                                      kv_cache, num_kv_slots, kv_row_stride, dest_slots, dev_err, C);
  if (st != MLA_OK) return st;
  C.accept_len = accept_len;
  C.path = accept_path;
  return launched(mlav::launch_commit(C, stream));
}

mla_status mla_accept_commit(const int32_t* tree_parent, const int32_t* draft_tokens, const int32_t* target_tokens,
                             int32_t batch, int32_t num_nodes, int32_t* page_table, int32_t max_pages,
                             const int32_t* seq_lens, int32_t* accept_len, int32_t* accept_path,
                             int32_t* commit_tokens, int32_t* context_lens, int32_t* freed_slots, void* kv_cache,
                             int64_t num_kv_slots, int64_t kv_row_stride, const int32_t* dest_slots,
                             uint32_t* dev_err, hipStream_t stream) {
  if (tree_parent == nullptr || draft_tokens == nullptr || target_tokens == nullptr || accept_len == nullptr ||
      accept_path == nullptr)
    return MLA_ERR_NULL;
  mlav::CommitLaunch C;
  const mla_status st = commit_launch(page_table, max_pages, seq_lens, batch, num_nodes, context_lens, freed_slots,
                                      kv_cache, num_kv_slots, kv_row_stride, dest_slots, dev_err, C);
  if (st != MLA_OK) return st;
  const mlav::AcceptLaunch A{tree_parent, draft_tokens, target_tokens, accept_len, accept_path, commit_tokens, dev_err};
  return launched(mlav::launch_accept_commit(A, C, stream));
}

mla_status mla_window_map(const int32_t* target_map, int32_t map_stride, const int32_t* lens, int32_t batch,
                          int32_t window, int32_t page, int32_t* draft_map, int32_t* compact_lens, uint32_t* dev_err,
                          hipStream_t stream) {
  if (target_map == nullptr || lens == nullptr || draft_map == nullptr) return MLA_ERR_NULL;
  if (batch < 1 || window < 1 || page < 1 || map_stride < 1) return MLA_ERR_SHAPE;
  if (static_cast<int64_t>(window) + page - 1 > std::numeric_limits<int32_t>::max() / 2 || batch > 65535)
    return MLA_ERR_SHAPE;
  return launched(mlav::launch_window_map(target_map, map_stride, lens, batch, window, page, draft_map, compact_lens,
                                          dev_err, stream));
}

mla_status mla_indexer_logits(const mla_indexer_desc* d, const uint8_t* q, const float* weights,
                              const uint8_t* kv_blocks, const int32_t* block_table, const int32_t* seq_lens,
                              float* logits, uint32_t* dev_err, hipStream_t stream) {
  if (d == nullptr || q == nullptr || weights == nullptr || kv_blocks == nullptr || block_table == nullptr ||
      seq_lens == nullptr || logits == nullptr)
    return MLA_ERR_NULL;
  if (d->head_dim != 128 || d->num_heads > 64) return MLA_ERR_UNSUPPORTED;
  if (d->batch < 1 || d->num_heads < 1 || d->max_blocks < 1 || d->num_blocks < 1 || d->batch > 65535 ||
      d->max_blocks > (1 << 24) || d->num_blocks > std::numeric_limits<int32_t>::max())
    return MLA_ERR_SHAPE;
  if (misaligned(q, 16) || misaligned(kv_blocks, 16) || misaligned(weights, 4) || misaligned(block_table, 4) ||
      misaligned(seq_lens, 4) || misaligned(logits, 4))
    return MLA_ERR_ALIGN;
  mlav::IndexerLaunch I;
  I.q = q;
  I.weights = weights;
  I.kv_blocks = kv_blocks;
  I.block_table = block_table;
  I.seq_lens = seq_lens;
  I.logits = logits;
  I.err = dev_err;
  I.num_blocks = d->num_blocks;
  I.batch = d->batch;
  I.heads = d->num_heads;
  I.max_blocks = d->max_blocks;
  return launched(mlav::launch_indexer(I, stream));
}

}  // extern "C"

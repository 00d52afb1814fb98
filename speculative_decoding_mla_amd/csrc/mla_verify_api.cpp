// C ABI of the verify-attention library: descriptor checks, workspace sizing
// and launches. Nothing here reads device memory, synchronises or allocates,
// so every entry point may be captured into a hipGraph.

#include <stdint.h>

#include <cmath>
#include <limits>

#include "mla_verify.h"
#include "mla_verify_internal.h"

namespace {

bool is_pow2(int32_t v) { return v > 0 && (v & (v - 1)) == 0; }

int log2i(int32_t v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

}  // namespace

namespace mlav {

// Shape checks shared by sizing and launching. Returns MLA_OK or the reason.
mla_status check_desc(const mla_verify_desc* d) {
  if (d == nullptr) return MLA_ERR_NULL;
  if (d->head_dim_qk != mlav::kQkDim || d->head_dim_v != mlav::kVDim) return MLA_ERR_UNSUPPORTED;
  if (!is_pow2(d->page_size)) return MLA_ERR_UNSUPPORTED;
  if (d->batch < 1 || d->num_nodes < 1 || d->num_nodes > mlav::kMaxNodes || d->num_heads < 1 ||
      d->max_pages < 1 || d->nsplit < 1 || d->num_kv_slots < 1)
    return MLA_ERR_SHAPE;
  if (d->kv_row_stride < mlav::kQkDim || (d->kv_row_stride % 8) != 0) return MLA_ERR_SHAPE;
  if (d->kv_row_stride > mlav::kMaxRowStride) return MLA_ERR_SHAPE;
  if (!std::isfinite(d->sm_scale)) return MLA_ERR_SHAPE;
  // Keys, slots and launch sizes are indexed with 32-bit integers on the device.
  const int64_t capacity = static_cast<int64_t>(d->max_pages) * d->page_size;
  if (capacity > std::numeric_limits<int32_t>::max()) return MLA_ERR_SHAPE;
  if (capacity < d->num_nodes) return MLA_ERR_SHAPE;
  if (d->num_kv_slots > std::numeric_limits<int32_t>::max()) return MLA_ERR_SHAPE;
  const int64_t rows = static_cast<int64_t>(d->num_nodes) * d->num_heads;
  if (rows > (1 << 20)) return MLA_ERR_SHAPE;
  const mlav::RowPlan rp = mlav::plan_rows(d->num_nodes, d->num_heads);
  const int64_t wgs = static_cast<int64_t>(d->batch) * d->nsplit * rp.row_blocks;
  if (wgs > (1LL << 30)) return MLA_ERR_SHAPE;
  const int64_t combine_wgs = static_cast<int64_t>(d->batch) * (rp.rows_pad / 32) * 64;
  if (combine_wgs > (1LL << 30)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

}  // namespace mlav

using mlav::check_desc;

extern "C" {

size_t mla_verify_workspace_bytes(const mla_verify_desc* d) {
  if (check_desc(d) != MLA_OK) return 0;
  const mlav::RowPlan rp = mlav::plan_rows(d->num_nodes, d->num_heads);
  return mlav::workspace_bytes(d->batch, d->nsplit, rp.rows_pad);
}

mla_status mla_build_tree_mask(const int32_t* tree_parent, uint64_t* anc_mask, int32_t batch,
                               int32_t num_nodes, uint32_t* dev_err, hipStream_t stream) {
  if (tree_parent == nullptr || anc_mask == nullptr) return MLA_ERR_NULL;
  if (batch < 1 || num_nodes < 1 || num_nodes > mlav::kMaxNodes) return MLA_ERR_SHAPE;
  const hipError_t e = mlav::launch_tree_mask(tree_parent, anc_mask, batch, num_nodes, dev_err, stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"

namespace mlav {

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// Checks the descriptor, the workspace and whichever pointers the stage uses
// (null entries are not used), then fills the launch record.
mla_status prepare(const mla_verify_desc* d, const void* q, const void* kv_cache, const int32_t* page_table,
                   const int32_t* seq_lens, const int32_t* tree_parent, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, bool partial, bool combine, mlav::VerifyLaunch* L) {
  const mla_status st = check_desc(d);
  if (st != MLA_OK) return st;
  if (workspace == nullptr) return MLA_ERR_NULL;
  if (partial && (q == nullptr || kv_cache == nullptr || page_table == nullptr || seq_lens == nullptr ||
                  tree_parent == nullptr))
    return MLA_ERR_NULL;
  if (combine && (out == nullptr || lse == nullptr)) return MLA_ERR_NULL;
  if (misaligned(workspace, 16)) return MLA_ERR_ALIGN;
  if (partial && (misaligned(q, 16) || misaligned(kv_cache, 16) || misaligned(page_table, 4) ||
                  misaligned(seq_lens, 4) || misaligned(tree_parent, 4)))
    return MLA_ERR_ALIGN;
  if (combine && (misaligned(out, 16) || misaligned(lse, 4))) return MLA_ERR_ALIGN;
  const mlav::RowPlan rp = mlav::plan_rows(d->num_nodes, d->num_heads);
  if (workspace_bytes < mlav::workspace_bytes(d->batch, d->nsplit, rp.rows_pad)) return MLA_ERR_WORKSPACE;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  L->q = static_cast<const uint16_t*>(q);
  L->kv = static_cast<const uint8_t*>(kv_cache);
  L->page_table = page_table;
  L->seq_lens = seq_lens;
  L->tree_parent = tree_parent;
  L->out = static_cast<uint16_t*>(out);
  L->lse = lse;
  L->err = reinterpret_cast<uint32_t*>(ws);
  L->part_lse = reinterpret_cast<float*>(ws + mlav::part_lse_offset());
  L->part_o = reinterpret_cast<uint16_t*>(ws + mlav::part_o_offset(d->batch, d->nsplit, rp.rows_pad));
  L->kv_row_bytes = d->kv_row_stride * 2;
  L->num_slots = d->num_kv_slots;
  L->batch = d->batch;
  L->nodes = d->num_nodes;
  L->heads = d->num_heads;
  L->rows = rp.rows;
  L->rows_pad = rp.rows_pad;
  L->waves_per_wg = rp.waves_per_wg;
  L->row_blocks = rp.row_blocks;
  L->nsplit = d->nsplit;
  L->page_shift = log2i(d->page_size);
  L->max_pages = d->max_pages;
  L->capacity = static_cast<int32_t>(static_cast<int64_t>(d->max_pages) * d->page_size);
  L->min_len = d->num_nodes;
  L->quiet_unused = 0;
  L->col_parts = mlav::col_parts_for(d->batch, d->nsplit, rp.row_blocks);
  L->scale_log2 = d->sm_scale * 1.4426950408889634f;
  return MLA_OK;
}

}  // namespace mlav

using mlav::prepare;

extern "C" {

mla_status mla_verify_attention(const mla_verify_desc* d, const void* q, const void* kv_cache,
                                const int32_t* page_table, const int32_t* seq_lens,
                                const int32_t* tree_parent, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  mlav::VerifyLaunch L;
  const mla_status st = prepare(d, q, kv_cache, page_table, seq_lens, tree_parent, out, lse, workspace,
                                workspace_bytes, true, true, &L);
  if (st != MLA_OK) return st;
  if (mlav::launch_partial(L, stream) != hipSuccess) return MLA_ERR_HIP;
  return mlav::launch_combine(L, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_verify_partial(const mla_verify_desc* d, const void* q, const void* kv_cache,
                              const int32_t* page_table, const int32_t* seq_lens, const int32_t* tree_parent,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  mlav::VerifyLaunch L;
  const mla_status st = prepare(d, q, kv_cache, page_table, seq_lens, tree_parent, nullptr, nullptr, workspace,
                                workspace_bytes, true, false, &L);
  if (st != MLA_OK) return st;
  return mlav::launch_partial(L, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_verify_combine(const mla_verify_desc* d, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  mlav::VerifyLaunch L;
  const mla_status st = prepare(d, nullptr, nullptr, nullptr, nullptr, nullptr, out, lse, workspace,
                                workspace_bytes, false, true, &L);
  if (st != MLA_OK) return st;
  return mlav::launch_combine(L, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "null pointer";
    case MLA_ERR_SHAPE: return "dimension out of range";
    case MLA_ERR_UNSUPPORTED: return "unsupported head dims or page size";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_ALIGN: return "misaligned pointer";
    case MLA_ERR_HIP: return "kernel launch failed";
    case MLA_ERR_SCRATCH: return "problem needs more than the no-allocation scratch (MLA_VERIFY_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int32_t mla_verify_abi_version(void) { return MLA_VERIFY_ABI_VERSION; }

}  // extern "C"

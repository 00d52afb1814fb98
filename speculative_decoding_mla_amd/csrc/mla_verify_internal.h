// Internal launch interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "mla_verify.h"

namespace mlav {

constexpr int kQkDim = 576;       // 512 latent + 64 rope
constexpr int kVDim = 512;        // V = leading 512 entries of the latent row
constexpr int kMaxNodes = 64;     // ancestor sets are 64-bit masks
constexpr int kCusPerDevice = 256;  // MI355X
constexpr int kMaxColParts = 4;     // partial-lse records per (split, row): one per column part
constexpr int64_t kMaxRowStride = int64_t{1} << 30;  // bf16 entries: row bytes stay below 2^31
constexpr int kRowsPerWave = 32;  // one 32x32 MFMA column block of (node, head) rows per wave
constexpr int kHeaderBytes = 256; // workspace header; word 0 is the device error word

// Everything one verify call needs, resolved on the host from the descriptor.
struct VerifyLaunch {
  const uint16_t* q;           // bf16 [B, T, H, 576]
  const uint8_t* kv;           // bf16 rows, byte pointer
  const int32_t* page_table;   // [B, max_pages]
  const int32_t* seq_lens;     // [B]; null: every request holds capacity keys
  const int32_t* tree_parent;  // [B, T]; null: every node is a root
  uint16_t* out;               // bf16 [B, T, H, 512]
  float* lse;                  // [B, T, H]
  uint32_t* err;               // device error word (workspace head)
  float* part_lse;             // [B*nsplit slots][kMaxColParts][rows_pad] pairs {partial lse (log2 units), scale exponent}
  uint16_t* part_o;            // fragment-ordered partial outputs, fp16, scaled by 2^-exponent
  int64_t kv_row_bytes;        // bytes between kv rows
  int64_t num_slots;
  int32_t batch, nodes, heads, rows, rows_pad, waves_per_wg, row_blocks;
  int32_t nsplit, page_shift, max_pages;
  int32_t capacity;            // max_pages * page_size (clamp bound for seq_lens)
  int32_t min_len;             // lower clamp bound for seq_lens: T (verify) or 0 (sparse decode)
  int32_t quiet_unused;        // 1: a page id of -1 is an unused entry, masked without an error bit
  int32_t col_parts;           // 1, 2 or 4 workgroups per (split, row block), each over 512/col_parts columns
  float scale_log2;            // sm_scale * log2(e)
};

// Rows (node, head) are grouped in waves of 32; a workgroup holds 1..4 waves.
struct RowPlan {
  int rows, waves_per_wg, row_blocks, rows_pad;
};
RowPlan plan_rows(int nodes, int heads);
// Column parts for a grid of batch * nsplit * row_blocks workgroups.
int col_parts_for(int batch, int nsplit, int row_blocks);

size_t workspace_bytes(int batch, int nsplit, int rows_pad);
size_t part_lse_offset();
size_t part_o_offset(int batch, int nsplit, int rows_pad);

// Host-side checks and the launch record (mla_verify_api.cpp); the
// no-allocation entry point runs the same ones on its static scratch.
mla_status check_desc(const mla_verify_desc* d);
bool misaligned(const void* p, uintptr_t a);
mla_status prepare(const mla_verify_desc* d, const void* q, const void* kv_cache, const int32_t* page_table,
                   const int32_t* seq_lens, const int32_t* tree_parent, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, bool partial, bool combine, VerifyLaunch* L);

hipError_t launch_tree_mask(const int32_t* tree_parent, uint64_t* anc, int batch, int nodes,
                            uint32_t* err, hipStream_t stream);
hipError_t launch_partial(const VerifyLaunch& L, hipStream_t stream);
hipError_t launch_combine(const VerifyLaunch& L, hipStream_t stream);

}  // namespace mlav

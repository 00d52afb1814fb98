// Internal launch interface between the C-ABI host code of mla_spec_ops.h and
// its gfx950 kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mlav {

constexpr int kMaxTreeNodes = 64;  // draft trees are handled one node per lane of a wave

struct AcceptLaunch {
  const int32_t* parents;  // [B, T]
  const int32_t* draft;    // [B, T]
  const int32_t* target;   // [B, T]
  int32_t* accept_len;     // [B] out
  int32_t* path;           // [B, T] out
  int32_t* commit;         // [B, T] out, nullable
  uint32_t* err;           // nullable
};

struct CommitLaunch {
  int32_t* page_table;        // [B, max_pages], page size 1
  const int32_t* seq_lens;    // [B] verify lengths (tree rows included)
  const int32_t* accept_len;  // [B]
  const int32_t* path;        // [B, T]
  int32_t* context_lens;      // [B] out
  int32_t* freed;             // [B, T] out, nullable
  uint8_t* kv;                // pool bytes (relocation only)
  const int32_t* dest;        // [B, T] destination slots, nullable (no relocation)
  uint32_t* err;              // nullable
  int64_t num_slots, row_bytes;
  int32_t batch, nodes, max_pages;
};

struct IndexerLaunch {
  const uint8_t* q;            // [B, H, 128] e4m3
  const float* weights;        // [B, H]
  const uint8_t* kv_blocks;    // [num_blocks, 8448]
  const int32_t* block_table;  // [B, max_blocks]
  const int32_t* seq_lens;     // [B]
  float* logits;               // [B, max_blocks * 64]
  uint32_t* err;               // nullable
  int64_t num_blocks;
  int32_t batch, heads, max_blocks;
};

hipError_t launch_kv_append(uint8_t* kv, int64_t num_slots, int64_t row_bytes, const uint8_t* rows,
                            const int32_t* loc, int n, uint32_t* err, hipStream_t stream);
hipError_t launch_tree_accept(const AcceptLaunch& A, int batch, int T, hipStream_t stream);
hipError_t launch_commit(const CommitLaunch& C, hipStream_t stream);
hipError_t launch_accept_commit(const AcceptLaunch& A, const CommitLaunch& C, hipStream_t stream);
hipError_t launch_window_map(const int32_t* target_map, int map_stride, const int32_t* lens, int batch, int W,
                             int P, int32_t* draft_map, int32_t* compact_lens, uint32_t* err, hipStream_t stream);
hipError_t launch_indexer(const IndexerLaunch& I, hipStream_t stream);

}  // namespace mlav

// gfx950 (MI355X) kernels for the steps next to the verify attention: the
// draft rows' KV append, the greedy tree accept, the commit (and optional
// relocation) of the accepted path, the page-aligned sliding-window map of a
// draft cache, and the DSA indexer logits over an fp8 paged cache.
//
// The first four are integer and byte work: each is laid out for coalesced
// 16-byte (rows) or 4-byte (maps) accesses, with the per-request logic of a
// draft tree (at most 64 nodes) done inside one wave by pointer jumping. The
// indexer is a small dense contraction per cache block (64 positions x 64
// heads x 128 dims): its fp8 operands are widened exactly to bf16 and fed to
// v_mfma_f32_32x32x16_bf16 straight from global memory by persistent
// workgroups, and the ReLU / weight / head-sum / scale epilogue stays in
// registers. Every grid is fixed by host-known sizes; blocks past a request's
// length are written -inf without being read.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "mla_spec_ops.h"
#include "mla_spec_ops_internal.h"

namespace mlav {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowChunks = 72;  // 16-byte chunks of a 1,152-byte latent row
// Persistent indexer workgroups: one per CU, one wave per SIMD. Measured
// against two per CU (two waves per SIMD fit the registers): fewer, longer
// runs are faster, as each run pays two dependent round trips (block table,
// then keys) before its stream starts.
constexpr int kIndexerGrid = 256;

__device__ __forceinline__ void flag(uint32_t* err, uint32_t bit) {
  if (err != nullptr) atomicOr(err, bit);
}

// ---------------------------------------------------------------- KV append

__global__ __launch_bounds__(256) void kv_append_kernel(uint8_t* __restrict__ kv, int64_t num_slots,
                                                        int64_t row_bytes, const uint8_t* __restrict__ rows,
                                                        const int32_t* __restrict__ loc, int n, uint32_t* err) {
  const int64_t total = static_cast<int64_t>(n) * kRowChunks;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = t / kRowChunks;
    const int c = static_cast<int>(t - r * kRowChunks);
    const int32_t slot = loc[r];
    if (slot < 0 || slot >= num_slots) {
      if (c == 0) flag(err, MLA_DEVERR_SLOT_RANGE);
      continue;
    }
    const u32x4 v = *reinterpret_cast<const u32x4*>(rows + r * (kRowChunks * 16) + c * 16);
    *reinterpret_cast<u32x4*>(kv + slot * row_bytes + c * 16) = v;
  }
}

// ---------------------------------------------------------------- tree helpers (one wave, lane = node)

// Parent of node `lane` (-1 for lanes >= T); a parent outside [-1, lane) is
// reported and read as -1 (a root).
__device__ __forceinline__ int checked_parent(const int32_t* parents, int T, int lane, uint32_t* err) {
  int p = lane < T ? parents[lane] : -1;
  const bool bad = lane < T && (p < -1 || p >= lane);
  if (bad) p = -1;
  if (__any(bad) && lane == 0) flag(err, MLA_DEVERR_BAD_PARENT);
  return p;
}

// Pointer jumping over parent links (six rounds cover 64 nodes): `all` becomes
// the AND of `f` over the node and its ancestors, `anc` the ancestor-or-self
// bitmask and `depth` the number of links to the root.
__device__ __forceinline__ void climb(int parent, bool f, int lane, int T, bool& all, uint64_t& anc, int& depth) {
  int p = parent;
  all = lane < T && f;
  anc = lane < T ? 1ull << lane : 0ull;
  depth = p >= 0 ? 1 : 0;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = p >= 0 ? p : lane;
    const bool all_p = __shfl(static_cast<int>(all), src) != 0;
    const uint32_t lo = __shfl(static_cast<uint32_t>(anc), src);
    const uint32_t hi = __shfl(static_cast<uint32_t>(anc >> 32), src);
    const int depth_p = __shfl(depth, src);
    const int p2 = __shfl(p, src);
    if (p >= 0) {
      all = all && all_p;
      anc |= (static_cast<uint64_t>(hi) << 32) | lo;
      depth += depth_p;
      p = p2;
    }
  }
}

// ---------------------------------------------------------------- greedy tree accept (one wave per request)

struct Accepted {
  uint64_t on_path;  // nodes of the kept path, root..kept node
  int n_acc;         // committed tokens: depth of the kept node + 1
};

// The accept of request b by one wave (lane = node); writes accept_len, path
// and (when set) commit as mla_tree_accept documents them.
__device__ __forceinline__ Accepted accept_one(const AcceptLaunch& A, int T, int b, int lane) {
  const size_t base = static_cast<size_t>(b) * T;
  const int p = checked_parent(A.parents + base, T, lane, A.err);
  const int d = lane < T ? A.draft[base + lane] : 0;
  const int tg = lane < T ? A.target[base + lane] : 0;
  // a root is accepted; another node iff its draft equals the target's choice after its parent
  const int tg_parent = __shfl(tg, p >= 0 ? p : lane);
  const bool match = p < 0 || d == tg_parent;
  bool acc;
  uint64_t anc;
  int depth;
  climb(p, match, lane, T, acc, anc, depth);
  // deepest accepted node, the smaller index among equals: max of depth * 64 + (63 - lane)
  int key = acc ? depth * 64 + (63 - lane) : -1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) key = max(key, __shfl_xor(key, o));
  const int best = 63 - (key & 63);  // node 0 is a root (parent -1), so key >= 0
  const int best_depth = key >> 6;
  const uint32_t blo = __shfl(static_cast<uint32_t>(anc), best);
  const uint32_t bhi = __shfl(static_cast<uint32_t>(anc >> 32), best);
  const uint64_t on_path = (static_cast<uint64_t>(bhi) << 32) | blo;
  const int n_acc = best_depth + 1;
  if (lane == 0) A.accept_len[b] = n_acc;
  if (lane < T) {
    const bool mine = (on_path >> lane) & 1ull;
    const int pos = __popcll(on_path & ((1ull << lane) - 1ull));  // place on the path (root = 0)
    if (mine) A.path[base + pos] = lane;
    if (lane >= n_acc) A.path[base + lane] = -1;
    if (A.commit != nullptr) {
      if (mine && pos >= 1) A.commit[base + pos - 1] = d;
      if (lane == best) A.commit[base + best_depth] = tg;
      if (lane > best_depth) A.commit[base + lane] = -1;
    }
  }
  return {on_path, n_acc};
}

__global__ __launch_bounds__(64) void tree_accept_kernel(AcceptLaunch A, int T) {
  accept_one(A, T, blockIdx.x, threadIdx.x);
}

// ---------------------------------------------------------------- commit of the accepted path (one workgroup per request)

constexpr int kCommitThreads = 256;

struct CommitLds {
  int32_t tree_slot[kMaxTreeNodes];  // slots of the request's tree rows, node order
  int32_t path[kMaxTreeNodes];       // accepted nodes, root first
  uint64_t on_path;
  int32_t n_acc, c0;
  u32x4 rows[kMaxTreeNodes * kRowChunks];  // accepted rows in flight during a relocation
};

// One wave: the first committed position c0 = seq_len - T and the tree rows'
// slots from the page table.
__device__ __forceinline__ void load_tree_slots(const CommitLaunch& C, CommitLds& S, int b, int lane) {
  const int T = C.nodes;
  const int sl = C.seq_lens[b];
  const int sl_c = min(max(sl, T), C.max_pages);
  if (sl != sl_c && lane == 0) flag(C.err, MLA_DEVERR_INDEX_RANGE);
  const int c0 = sl_c - T;
  if (lane == 0) S.c0 = c0;
  if (lane < T) S.tree_slot[lane] = C.page_table[static_cast<size_t>(b) * C.max_pages + c0 + lane];
}

// The whole workgroup, after S is filled and a barrier: relocation (every
// accepted row is read into LDS before any is written), page-table entries,
// released slots and the new context length.
__device__ __forceinline__ void commit_rows(const CommitLaunch& C, CommitLds& S, int b, int tid) {
  const int T = C.nodes;
  const size_t tb = static_cast<size_t>(b) * T;
  const int c0 = S.c0, n_acc = S.n_acc;
  int32_t* row = C.page_table + static_cast<size_t>(b) * C.max_pages;
  if (C.dest != nullptr) {
    for (int t = tid; t < n_acc * kRowChunks; t += kCommitThreads) {
      const int k = t / kRowChunks, c = t - k * kRowChunks;
      const int32_t src = S.tree_slot[S.path[k]];
      u32x4 v = {0u, 0u, 0u, 0u};
      if (src >= 0 && src < C.num_slots) v = *reinterpret_cast<const u32x4*>(C.kv + src * C.row_bytes + c * 16);
      S.rows[t] = v;
    }
    __syncthreads();
    for (int t = tid; t < n_acc * kRowChunks; t += kCommitThreads) {
      const int k = t / kRowChunks, c = t - k * kRowChunks;
      const int32_t src = S.tree_slot[S.path[k]];
      const int32_t dst = C.dest[tb + k];
      const bool ok = src >= 0 && src < C.num_slots && dst >= 0 && dst < C.num_slots;
      if (!ok) {
        if (c == 0) flag(C.err, MLA_DEVERR_SLOT_RANGE);
        continue;
      }
      *reinterpret_cast<u32x4*>(C.kv + dst * C.row_bytes + c * 16) = S.rows[t];
    }
  }
  if (tid < n_acc) row[c0 + tid] = C.dest != nullptr ? C.dest[tb + tid] : S.tree_slot[S.path[tid]];
  if (tid < T && C.freed != nullptr) {
    const uint64_t on_path = S.on_path;
    const bool kept = (on_path >> tid) & 1ull;
    const uint64_t below = (tid == 0 ? 0ull : (~0ull >> (64 - tid)));
    const int pos = tid - __popcll(on_path & below);  // released nodes before this one
    if (!kept) C.freed[tb + pos] = S.tree_slot[tid];
    if (tid >= T - n_acc) C.freed[tb + tid] = -1;
  }
  if (tid == 0) C.context_lens[b] = c0 + n_acc;
}

// Commit of a path written earlier (accept_len, path in global memory, range
// checked): wave 0 reads the page table, wave 1 the path.
__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitLaunch C) {
  __shared__ CommitLds S;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int T = C.nodes;
  if (wave == 0) {
    load_tree_slots(C, S, b, lane);
  } else if (wave == 1) {
    const int na = C.accept_len[b];
    const int n_acc = min(max(na, 1), T);
    int j = lane < n_acc ? C.path[static_cast<size_t>(b) * T + lane] : 0;
    const bool bad = na != n_acc || j < 0 || j >= T;
    if (__any(bad) && lane == 0) flag(C.err, MLA_DEVERR_INDEX_RANGE);
    j = min(max(j, 0), T - 1);
    uint64_t bit = lane < n_acc ? 1ull << j : 0ull;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t lo = __shfl_xor(static_cast<uint32_t>(bit), o);
      const uint32_t hi = __shfl_xor(static_cast<uint32_t>(bit >> 32), o);
      bit |= (static_cast<uint64_t>(hi) << 32) | lo;
    }
    if (lane < n_acc) S.path[lane] = j;
    if (lane == 0) {
      S.n_acc = n_acc;
      S.on_path = bit;
    }
  }
  __syncthreads();
  commit_rows(C, S, b, tid);
}

// Accept and commit in one launch: wave 0 runs the accept while wave 1 reads
// the page table; the commit takes the path from LDS.
__global__ __launch_bounds__(kCommitThreads) void accept_commit_kernel(AcceptLaunch A, CommitLaunch C) {
  __shared__ CommitLds S;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int T = C.nodes;
  if (wave == 0) {
    const Accepted a = accept_one(A, T, b, lane);
    if (lane < T && ((a.on_path >> lane) & 1ull)) S.path[__popcll(a.on_path & ((1ull << lane) - 1ull))] = lane;
    if (lane == 0) {
      S.n_acc = a.n_acc;
      S.on_path = a.on_path;
    }
  } else if (wave == 1) {
    load_tree_slots(C, S, b, lane);
  }
  __syncthreads();
  commit_rows(C, S, b, tid);
}

// ---------------------------------------------------------------- sliding-window map

__global__ __launch_bounds__(256) void window_map_kernel(const int32_t* __restrict__ target_map, int map_stride,
                                                         const int32_t* __restrict__ lens, int W, int P,
                                                         int32_t* __restrict__ draft_map,
                                                         int32_t* __restrict__ compact_lens, uint32_t* err) {
  const int b = blockIdx.y;
  const int width = W + P - 1;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int raw = lens[b];
  const int L = min(max(raw, 0), map_stride);
  const int start = ((L - min(L, W)) / P) * P;  // page-aligned window start s(L)
  const int c = L - start;                       // compact length c(L)
  if (j == 0) {
    if (raw != L) flag(err, MLA_DEVERR_SEQ_LEN);
    if (compact_lens != nullptr) compact_lens[b] = c;
  }
  if (j < width)
    draft_map[static_cast<size_t>(b) * width + j] =
        j < c ? target_map[static_cast<size_t>(b) * map_stride + start + j] : -1;
}

// ---------------------------------------------------------------- fp8 indexer logits

// Eight E4M3 codes (two dwords) widened exactly to bf16 (four significant
// bits fit bf16's eight, and the exponent range is wider): one gfx950
// conversion per pair of codes, with scale 1. The order of the eight values is
// that of the bytes; any fixed order serves, as queries and keys are widened
// alike.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// max(x, 0) on the bit pattern: a negative float is a negative int32
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

constexpr int kIdxPage = 64, kIdxDim = 128, kIdxBlockBytes = 8448, kIdxScaleOff = kIdxPage * kIdxDim;

// Persistent waves, independent of each other (no barrier, no LDS): the
// work unit is half a block, 32 positions x all 64 heads. Wave g of the grid
// streams a contiguous run of units of the flattened (request, block, half)
// space: the run's block ids, lengths and requests are read once (one lane per
// unit), the request's queries are widened to bf16 once and stay in
// registers, and the 4 KiB of the next two units are in flight while the
// current one is multiplied. A unit is two 32 x 32 tiles of Q K^T (head halves) over the same
// K fragments: 16 MFMAs. The contraction index is permuted the same way on
// both sides (k-step ks and lane half hs cover dims 64 hs + 8 ks + 0..7), so a
// lane's operand bytes are 64 contiguous bytes of its row. Heads are the rows
// of the product and positions its columns, so each lane ends with 32 heads
// of one position: the ReLU, the head weights and the sum over heads are done
// in its registers, and one exchange between the lane halves completes it.
__global__ __launch_bounds__(256) void indexer_kernel(IndexerLaunch I) {
  const int lane = threadIdx.x & 63;
  const int hs = lane >> 5;
  const int cap = I.max_blocks * kIdxPage;
  const int units = I.batch * I.max_blocks * 2;
  const int waves = static_cast<int>(gridDim.x) * (blockDim.x >> 6);
  const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int per = (units + waves - 1) / waves;  // <= 64 (host)
  const int first = gw * per;
  const int cnt = min(units, first + per) - first;
  if (cnt <= 0) return;

  const int hd = lane & 31;  // this lane's query row in each head half, and its key row

  // The product's rows held by this lane: heads 32 h2 + wrow(j), j = 0..15.
  auto wrow = [&](int j) { return 8 * (j >> 2) + 4 * hs + (j & 3); };
  // The queries of a request, as stored (widened later), and the weights of
  // the heads this lane sums: lane (hs, hd) holds bytes 64 hs .. 64 hs + 63
  // of head hd and of head 32 + hd. Heads past the count are read as head 0
  // and zeroed at widening.
  u32x4 qraw[2][4];
  float wv[2][16];
  auto load_q = [&](int b) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int head = h2 * 32 + hd < I.heads ? h2 * 32 + hd : 0;
      const u32x4* qrow =
          reinterpret_cast<const u32x4*>(I.q + (static_cast<size_t>(b) * I.heads + head) * kIdxDim + hs * 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) qraw[h2][i] = qrow[i];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int hw = h2 * 32 + wrow(j);
        wv[h2][j] = I.weights[static_cast<size_t>(b) * I.heads + (hw < I.heads ? hw : 0)];
      }
    }
  };
  // The run's first request is known from the unit index alone: its queries
  // are requested before anything else, so they arrive first.
  load_q(first / (2 * I.max_blocks));

  // lane k < cnt describes unit `first + k`: request, clamped length, block id
  // (-1 past the length, -2 out of range); lanes past the run repeat the last
  // unit's reads (every lane loads, so the number of loads in flight is fixed)
  // and describe nothing. The table entry is read together with the length
  // (the table is in bounds whatever the length; an entry past it is never
  // used), so the block ids are one round trip away, not two.
  int my_b, my_n, my_blk = -1;
  {
    const int u = first + min(lane, cnt - 1);
    my_b = u / (2 * I.max_blocks);
    const int page = (u >> 1) - my_b * I.max_blocks;
    int raw = I.seq_lens[my_b];
    int entry = I.block_table[u >> 1];
    asm volatile("" : "+v"(raw), "+v"(entry));  // both reads issued before either is waited for
    my_n = min(max(raw, 0), cap);
    if (lane < cnt) {
      if (raw != my_n && page == 0 && (u & 1) == 0) flag(I.err, MLA_DEVERR_SEQ_LEN);
      if (page * kIdxPage + (u & 1) * 32 < my_n) {
        my_blk = entry;
        if (my_blk < 0 || my_blk >= I.num_blocks) {
          flag(I.err, MLA_DEVERR_SLOT_RANGE);
          my_blk = -2;
        }
      }
    }
  }

  // A unit's bytes (this lane's 64 bytes of the K tile, and the scale of the
  // position it will hold) are loaded kAhead units before they are used;
  // loads retire in issue order, so nothing that waits on a unit's bytes also
  // waits on a later unit's. The loads are issued for every unit, also past
  // the run or the length (then from a block that exists, and never used):
  // with a load count that does not depend on the data, each wait
  // counts exactly the loads issued after its unit. Loads under a condition
  // make every later wait assume the fewest loads, which drains the prefetch.
  constexpr int kAhead = 2;
  struct UnitBytes {
    u32x4 k[4];
    float scale;
  };
  // Units past the run or the length read the run's last block instead (in
  // this wave's cache already; one block shared by every wave would be a hot
  // spot), or block 0 when that one is past the length too.
  const int spare_blk = max(__shfl(my_blk, cnt - 1), 0);
  auto load_unit = [&](int kk, UnitBytes& dst) {
    const int blk = __shfl(my_blk, kk & 63);
    const int use = kk < cnt && blk >= 0 ? blk : spare_blk;
    const uint8_t* block = I.kv_blocks + static_cast<size_t>(use) * kIdxBlockBytes;
    const int half = (first + kk) & 1;
    dst.scale = reinterpret_cast<const float*>(block + kIdxScaleOff)[half * 32 + hd];
    const u32x4* a = reinterpret_cast<const u32x4*>(block + (half * 32 + hd) * kIdxDim + hs * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst.k[i] = a[i];
  };

  bf16x8 q0[8], q1[8];
  auto widen_q = [&]() {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const bool ok = h2 * 32 + hd < I.heads;
      bf16x8(&qd)[8] = h2 == 0 ? q0 : q1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 qq = ok ? qraw[h2][i] : u32x4{0u, 0u, 0u, 0u};
        qd[2 * i] = e4m3x8_to_bf16(qq[0], qq[1]);
        qd[2 * i + 1] = e4m3x8_to_bf16(qq[2], qq[3]);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (h2 * 32 + wrow(j) >= I.heads) wv[h2][j] = 0.f;
    }
  };
  int cur_b = first / (2 * I.max_blocks);
  auto process = [&](int kk, const UnitBytes& ub) {
    const int u = first + kk;
    const int b = __shfl(my_b, kk & 63);
    const int n = __shfl(my_n, kk & 63);
    const int blk = __shfl(my_blk, kk & 63);
    const int page = (u >> 1) - b * I.max_blocks;
    const int pos0 = page * kIdxPage + (u & 1) * 32;
    float* out = I.logits + static_cast<size_t>(b) * cap + pos0;
    if (kk >= cnt || blk < 0) {
      // Past the run (nothing to write), past the length or an out-of-range
      // block (-inf): the unit's bytes are not used, but are waited for here as
      // on the other path, so that no later wait has to allow for them.
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(ub.k[i]));
      asm volatile("" ::"v"(ub.scale));
      if (kk < cnt && lane < 32) out[lane] = -INFINITY;
      return;
    }
    if (b != cur_b) {  // a new request within the run: its queries and head weights
      cur_b = b;
      load_q(b);
      widen_q();
    }
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4& a = ub.k[ks >> 1];
      const int o = (ks & 1) * 2;
      const bf16x8 kb = e4m3x8_to_bf16(a[o], a[o + 1]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q0[ks], kb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q1[ks], kb, acc1, 0, 0, 0);
    }
    // lane holds the products of position hd with heads wrow(j) (acc0) and
    // 32 + wrow(j) (acc1); four partial sums keep the chain of adds short
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      part[j & 3] = fmaf(wv[0][j], relu_bits(acc0[j]), part[j & 3]);
      part[j & 3] = fmaf(wv[1][j], relu_bits(acc1[j]), part[j & 3]);
    }
    float sum = (part[0] + part[1]) + (part[2] + part[3]);
    sum += __shfl_xor(sum, 32);  // the other lane half's 32 heads
    if (lane < 32) out[hd] = pos0 + hd < n ? sum * ub.scale : -INFINITY;
  };

  // ring of kAhead + 1 units, unrolled so that every ring index is a constant
  UnitBytes ring[kAhead + 1];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) load_unit(i, ring[i]);
  // the first request's queries are widened while the first units are in
  // flight (the empty statements keep the widening after the loads' issue)
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(qraw[h2][i])::"memory");
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(wv[h2][j])::"memory");
  }
  widen_q();
  for (int k = 0; k < cnt; k += kAhead + 1) {
#pragma unroll
    for (int slot = 0; slot <= kAhead; ++slot) {
      load_unit(k + slot + kAhead, ring[(slot + kAhead) % (kAhead + 1)]);
      process(k + slot, ring[slot]);
    }
  }
}

}  // namespace

hipError_t launch_kv_append(uint8_t* kv, int64_t num_slots, int64_t row_bytes, const uint8_t* rows,
                            const int32_t* loc, int n, uint32_t* err, hipStream_t stream) {
  const int64_t chunks = static_cast<int64_t>(n) * kRowChunks;
  const int64_t want = (chunks + 255) / 256;
  const int grid = static_cast<int>(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(256), 0, stream, kv, num_slots, row_bytes, rows, loc, n, err);
  return hipGetLastError();
}

hipError_t launch_tree_accept(const AcceptLaunch& A, int batch, int T, hipStream_t stream) {
  hipLaunchKernelGGL(tree_accept_kernel, dim3(batch), dim3(64), 0, stream, A, T);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitLaunch& C, hipStream_t stream) {
  hipLaunchKernelGGL(commit_kernel, dim3(C.batch), dim3(kCommitThreads), 0, stream, C);
  return hipGetLastError();
}

hipError_t launch_accept_commit(const AcceptLaunch& A, const CommitLaunch& C, hipStream_t stream) {
  hipLaunchKernelGGL(accept_commit_kernel, dim3(C.batch), dim3(kCommitThreads), 0, stream, A, C);
  return hipGetLastError();
}

hipError_t launch_window_map(const int32_t* target_map, int map_stride, const int32_t* lens, int batch, int W,
                             int P, int32_t* draft_map, int32_t* compact_lens, uint32_t* err, hipStream_t stream) {
  const int width = W + P - 1;
  hipLaunchKernelGGL(window_map_kernel, dim3((width + 255) / 256, batch), dim3(256), 0, stream, target_map,
                     map_stride, lens, W, P, draft_map, compact_lens, err);
  return hipGetLastError();
}

hipError_t launch_indexer(const IndexerLaunch& I, hipStream_t stream) {
  // persistent waves (four per workgroup, all resident), each over at most 64 consecutive half-blocks
  const int64_t units = static_cast<int64_t>(I.batch) * I.max_blocks * 2;
  int64_t waves = (units + 63) / 64;
  if (waves < 4 * kIndexerGrid) waves = 4 * kIndexerGrid;
  if (waves > units) waves = units;
  const int64_t grid = (waves + 3) / 4;
  hipLaunchKernelGGL(indexer_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, I);
  return hipGetLastError();
}

}  // namespace mlav

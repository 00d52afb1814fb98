// gfx950 (MI355X) kernels for tree-masked MLA verify attention over a paged
// latent KV pool.
//
// The method (page "The Custom sm_120 Verify Kernel: From 0.7 tok/s to 3-6x
// Decode Speedup on Blackwell Consumer GPUs", Part VII): split each request's
// keys into NSPLIT chunks, compute a partial attention per chunk, merge the
// partials; only the tree block carries a mask (prefix keys are visible to all
// nodes); KV rows are read with 128-bit loads. Everything below is laid out for
// CDNA4 rather than taken from that design:
//
//  * One workgroup per (request, split, block of up to 128 query rows). A query
//    row is a (node, head) pair; all rows of a request read the same latent
//    row (MLA), so a key tile staged once in LDS feeds every row of the block.
//  * Key tiles of 32 rows x 1152 B move HBM -> LDS with gfx950's 128-bit
//    global_load_lds (no VGPR staging), kStages deep, one s_barrier per tile.
//    A tile holds the 32 latent parts (1 KiB each, one wave-wide load per key
//    whose row address is wave-uniform) followed by the 32 rope parts (128 B,
//    eight keys per load). Each 16-byte chunk lands at chunk ^ swz(key)
//    inside its 128-byte group, which spreads the fragment reads below over
//    the LDS banks with addresses that are a per-lane base plus an immediate.
//  * The loop over tiles is straight-line code: the loads of tile t+3 are
//    issued between the MFMAs of tile t+1 with no branch (the last two steps,
//    which issue none, are a loop of their own).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    K fragments come from LDS, the wave's 32 query rows stay in VGPRs for the
//    whole kernel. In the S^T accumulator every lane owns one query row, so the
//    row max needs one cross-lane step and P^T is already in the B-operand
//    layout of the next product.
//  * O^T += V^T P^T on the same MFMA; the V^T operand is read straight from the
//    row-major tile with ds_read_b64_tr_b16 (no transposed copy).
//  * Softmax in log2 units against a fixed per-row reference, set from the
//    split's first tile (its max + kRefLift) and folded into the scaling of
//    the scores, so a weight is one exp2. Weights exp2(s - ref)
//    are accumulated without ever rescaling the accumulator, which therefore
//    only sees MFMA writes and stays in AGPRs. fp32 and bf16 share an 8-bit
//    exponent, so scores from ~94 below to kRefHead above the reference are
//    exact in relative terms; anything lower is negligible next to the row
//    max. Should a score rise beyond the reference + kRefHead (a gap of over
//    128 in log2 units, ~89 in natural units: not seen with attention scores
//    of ordinary range), or should a row that the first tile showed no key
//    see one later, the workgroup recomputes its split: one pass for the
//    exact row max, one accumulating against it. P is rounded to bf16 for the
//    MFMA; the output normaliser sums those rounded weights (a convex
//    combination) while the lse sums the fp32 weights.
//  * Partials are written in the accumulator's own fragment order (each store
//    instruction writes 1 KiB contiguous) and merged by a second kernel.
//  * Workgroup ids are remapped so the row blocks of one split run on one XCD
//    back to back and share its L2 for the key rows.
// Every path is capture-safe: fixed grid from host-known sizes, early exit for
// empty splits, no device-to-host traffic, no allocation.

#include <hip/hip_runtime.h>

#include <utility>
#include <math.h>
#include <stdint.h>

#include "mla_verify.h"
#include "mla_verify_internal.h"

namespace mlav {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kKeysPerTile = 32;
constexpr int kRowBytes = kQkDim * 2;                              // 1152 per key in HBM
constexpr int kLatentBytes = kVDim * 2;                            // 1024: one wave-wide load
constexpr int kRopeBytes = kRowBytes - kLatentBytes;               // 128
constexpr int kRopeBase = kKeysPerTile * kLatentBytes;             // rope part of a tile in LDS
constexpr int kTileBytes = kKeysPerTile * kRowBytes;               // 36864
constexpr int kRopeInstr = kKeysPerTile * kRopeBytes / 1024;       // 4 loads of 8 keys' rope
constexpr int kTileInstr = kKeysPerTile + kRopeInstr;              // 36 wave-wide 1 KiB loads
constexpr int kStages = 4;
constexpr int kWaves = 4;  // per partial workgroup: one per SIMD
constexpr int kQSteps = kQkDim / 16;                               // 36 k-steps of 16
constexpr int kColBlocks = kVDim / 32;                             // 16
constexpr float kRefLift = 32.0f;  // log2 units: reference above the max of the split's first tile
constexpr float kRefHead = 96.0f;  // log2 units: largest weight kept is 2^kRefHead
constexpr float kHeadWeight = 0x1p96f;  // 2^kRefHead
static_assert(kRefHead == 96.0f, "kHeadWeight must stay 2^kRefHead");

// Source of the keys that no row may see (an out-of-range or unused slot, the
// padding past a request's last key): a row of zeros, so that such keys enter
// both products as exact zeros whatever the pool holds (a weight of 0 times a
// non-finite value is not 0). Never written.
__device__ __align__(256) uint8_t kZeroRow[kRowBytes];

// 16-byte chunk permutation inside a 128-byte group, keyed by the key's index
// in the tile: 8 consecutive keys hit 8 distinct slots (K reads), and the
// 32-byte pairs of 4 consecutive keys hit 4 distinct pairs (V^T reads). A
// 256-byte permutation measures faster for the V^T reads alone (gfx950 LDS
// serves ds_read_b64_tr_b16 256 bytes wide) but its fragment addresses cost
// a VALU operation per read, which costs more in this loop than it saves.
__device__ __forceinline__ int swz(int key) { return ((key & 3) << 1) | ((key >> 2) & 1); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const LDS_AS void*)p));
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16*lane.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

// 4 bytes per lane from global memory straight into LDS at m0 + 4*lane (lanes
// outside exec write nothing).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

// A key row's 1 KiB latent part: 16 bytes per lane from the wave-uniform row
// address plus the lane offset lane16 ^ x into LDS at lds_base + lds_off +
// 16*lane. The xor sits between the M0 write and the load, which needs one
// wait state after it. The row address may come straight from v_readlane (a
// VALU write of an SGPR), which a VMEM instruction may read only 5 wait states
// later: the compiler does not see inside this asm, so the block supplies them
// itself (s_nop 2, the M0 write and the xor).
__device__ __forceinline__ void dma16_row(const void* row, uint32_t lane16, uint32_t x, uint32_t lds_base,
                                          uint32_t lds_off) {
  uint32_t voff;
  asm volatile("s_nop 2\n\ts_add_u32 m0, %2, %3\n\tv_xor_b32 %0, %4, %5\n\tglobal_load_lds_dwordx4 %0, %1"
               : "=&v"(voff)
               : "s"(row), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "s"(__builtin_amdgcn_readfirstlane(lds_off)),
                 "s"(__builtin_amdgcn_readfirstlane(x)), "v"(lane16)
               : "memory", "m0", "scc");
}

// Same, from a wave-uniform base address plus a per-lane 32-bit offset (5
// wait states after the asm starts, for a base an earlier VALU wrote).
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_nop 3\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

// 8-byte store at device (agent) scope: written through to the device's point
// of coherence rather than left dirty in this XCD's L2, so the release at the
// end of the kernel has nothing to write back and the next kernel, on any
// XCD, reads the value from the memory-side cache.
template <typename T>
__device__ __forceinline__ void store_agent8(T* p, const T& v) {
  static_assert(sizeof(T) == 8, "8-byte values");
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// v, opaque to the compiler from here on: lane-derived addresses computed
// from it are rebuilt where they are used (one VALU operation) rather than
// hoisted to the kernel's start and spilled to scratch across the tile loop
// (each reload would put a memory round trip into the next window's setup).
__device__ __forceinline__ int fresh(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// f(integral_constant<int, 0>{}), ..., f(integral_constant<int, N-1>{}): a
// loop whose index is a compile-time constant in every copy of the body.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N < 63 ? N : 63) : "memory");
}

// Workgroup barrier that does not drain outstanding global->LDS loads.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl(static_cast<uint32_t>(v), src);
  const uint32_t hi = __shfl(static_cast<uint32_t>(v >> 32), src);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Value of lane l ^ 32 (the other half of the wave) without going through LDS.
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Keys of request b as given (all of the table's capacity when no lengths
// are passed), and after the clamp to [min_len, capacity] (the device-side
// guard for seq_lens; min_len is T for verify, 0 for sparse decode).
__device__ __forceinline__ int raw_len(const VerifyLaunch& L, int b) {
  return L.seq_lens != nullptr ? L.seq_lens[b] : L.capacity;
}
__device__ __forceinline__ int clamped_len(const VerifyLaunch& L, int b) {
  return min(max(raw_len(L, b), L.min_len), L.capacity);
}

// Wave-wide inclusive prefix sum of v (64 lanes).
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t lo = __shfl_up(static_cast<uint32_t>(v), d);
    const uint32_t hi = __shfl_up(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32), d);
    const int64_t o = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    if (lane >= d) v += o;
  }
  return v;
}

// Split plan: the grid's B*NSPLIT split slots are shared out over the
// requests in proportion to their key counts, one slot at least each:
// request b owns nsplit_b = 1 + floor((B*NSPLIT - B) * n_b / sum n) consecutive
// slots from first_b = sum_{b' < b} nsplit_b'. Equal lengths give every request
// NSPLIT slots at b*NSPLIT (the plain split of the method); ragged batches get
// chunks of about the same size, so no request's keys set the step alone.
// Slots past the last owned one stay idle. Computed by every wave from
// seq_lens alone (no host data), identically in both kernels.
struct SplitRange {
  int b;      // owning request, -1 for an idle slot
  int first;  // first slot of the request
  int count;  // slots of the request
};
// by_slot: find the owner of slot `key`; otherwise the range of request `key`.
__device__ SplitRange split_plan(const VerifyLaunch& L, int key, bool by_slot, int lane) {
  const int B = L.batch;
  if (B == 1) return SplitRange{by_slot ? (key < L.nsplit ? 0 : -1) : 0, 0, L.nsplit};
  int64_t total = 0;
  for (int base = 0; base < B; base += 64) {
    const int i = base + lane;
    const int64_t n = i < B ? clamped_len(L, i) : 0;
    const int64_t sum = wave_incl_scan(n, lane);
    total += static_cast<int64_t>(__shfl(static_cast<uint32_t>(sum), 63)) |
             (static_cast<int64_t>(__shfl(static_cast<uint32_t>(static_cast<uint64_t>(sum) >> 32), 63)) << 32);
  }
  const int64_t spare = static_cast<int64_t>(B) * L.nsplit - B;
  int64_t run = 0;
  for (int base = 0; base < B; base += 64) {
    const int i = base + lane;
    const int64_t n = i < B ? clamped_len(L, i) : 0;
    const int64_t ns = i < B ? 1 + (total > 0 ? (spare * n) / total : 0) : 0;
    const int64_t incl = wave_incl_scan(ns, lane);
    const int64_t excl = incl - ns;
    const bool own = i < B && (by_slot ? (key >= run + excl && key < run + incl) : i == key);
    const uint64_t m = __ballot(own);
    if (m != 0) {
      const int src = __builtin_ctzll(m);
      return SplitRange{base + src,
                        __builtin_amdgcn_readfirstlane(static_cast<int>(run) + __shfl(static_cast<int>(excl), src)),
                        __builtin_amdgcn_readfirstlane(__shfl(static_cast<int>(ns), src))};
    }
    run += static_cast<int64_t>(__shfl(static_cast<uint32_t>(incl), 63)) |
           (static_cast<int64_t>(__shfl(static_cast<uint32_t>(static_cast<uint64_t>(incl) >> 32), 63)) << 32);
  }
  return SplitRange{-1, 0, 0};
}

// Ancestor-or-self bitmask of node `lane` (lanes >= T get 0) by pointer
// jumping: after round r a node's mask covers ancestors closer than 2^r and its
// pointer names the ancestor 2^r up. Six rounds cover 64 nodes. The whole wave
// must call it. A parent outside [-1, lane) is reported and replaced by -1.
// `parent` is parents[lane] for lane < T (ignored above).
__device__ uint64_t ancestor_bits_of(int parent, int T, int lane, uint32_t* err) {
  int p = -1;
  bool bad = false;
  if (lane < T) {
    p = parent;
    if (p < -1 || p >= lane) {
      bad = true;
      p = -1;
    }
  }
  uint64_t anc = lane < T ? (1ull << lane) : 0ull;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = p < 0 ? lane : p;
    const uint64_t a2 = shfl_u64(anc, src);
    const int p2 = __shfl(p, src);
    if (p >= 0) {
      anc |= a2;
      p = p2;
    }
  }
  if (__any(bad) && lane == 0 && err != nullptr) atomicOr(err, MLA_DEVERR_BAD_PARENT);
  return anc;
}
__device__ uint64_t ancestor_bits(const int32_t* parents, int T, int lane, uint32_t* err) {
  return ancestor_bits_of(lane < T ? parents[lane] : -1, T, lane, err);
}

__global__ __launch_bounds__(64) void tree_mask_kernel(const int32_t* __restrict__ parents,
                                                       uint64_t* __restrict__ anc, int T,
                                                       uint32_t* err) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const uint64_t a = ancestor_bits(parents + static_cast<size_t>(b) * T, T, lane, err);
  if (lane < T) anc[static_cast<size_t>(b) * T + lane] = a;
}

template <int V>
struct PassMode {
  static constexpr int value = V;
};
constexpr int kPassAdaptive = 0;  // accumulate; reference = the split's first tile max + kRefLift
constexpr int kPassMaxOnly = 1;   // scores only: exact row max over the split
constexpr int kPassFixed = 2;     // accumulate against a given reference

// kSparse: one query token per request over an index list (sparse top-k
// decode): lengths may be absent, an entry of -1 is unused, every node is a
// root. A compile-time switch, so the verify instantiations carry none of it.
// NWQ: waves that own query rows (32 each). Every workgroup runs kWaves waves:
// all of them stream key tiles (wave w loads keys 8w..8w+7 of each tile), the
// first NWQ also compute.
// NCP: column parts. With NCP > 1, NCP workgroups share a (split, row block):
// each computes the same scores and weights but only its 512/NCP output
// columns (kCB column blocks), so a grid that would leave CUs idle spreads the
// PV products, the normalisation and the partial stores over NCP CUs.
//
// Split s of a request that owns nsb split slots takes the request's key tiles
// s, s + nsb, s + 2 nsb, ... (tile g = keys 32g .. 32g + 31). The keys of a
// split are a subset like any other for the merge; taken this way, the first
// tiles of a split do not depend on the request's length, so for one request
// their page-table entries are requested together with the length.
template <int NWQ, bool kSparse, int NCP>
__global__ __launch_bounds__(kWaves * 64, 1) void verify_partial_kernel(VerifyLaunch L) {
  constexpr int kCB = kColBlocks / NCP;
  constexpr int kLoadsPerTile = kTileInstr / kWaves;  // 8 latent rows + the rope parts of those 8 keys
  constexpr int kLoadsPerStep = kLoadsPerTile + 1;    // + the page-table entries of a later tile
  static_assert(kLoadsPerTile == 9 && kKeysPerTile == 8 * kWaves, "a wave streams 8 keys of every tile");
  constexpr int kPeRing = 4;   // page-table entries of tiles k .. k+3 (one slot per lane and wave)
  constexpr int kBadRing = 8;  // bad-key bits of recent tiles

  __shared__ __attribute__((aligned(1024))) uint8_t kv_s[kStages * kTileBytes];
  __shared__ int32_t pe_s[kPeRing][kWaves][64];
  __shared__ uint32_t bad_s[kBadRing];  // byte w of entry k % kBadRing: keys 8w..8w+7 of tile k on a bad slot
  __shared__ uint64_t anc_s[kMaxNodes];
  __shared__ int32_t over_s[kWaves];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int hsel = lane >> 5;
  const bool qk_wave = wid < NWQ;

  // XCD-aware order: workgroup i runs on XCD i % 8, so consecutive logical ids
  // (the column parts and row blocks of one split) are placed on one XCD in
  // dispatch order and share its L2 for the key rows.
  const int total = L.batch * L.nsplit * L.row_blocks * NCP;
  const int per_xcd = gridDim.x >> 3;
  const int logical_cp = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical_cp >= total) return;
  const int cp = logical_cp % NCP;  // column part: blocks cp*kCB .. cp*kCB + kCB - 1
  const int logical = logical_cp / NCP;
  const int rb = logical % L.row_blocks;
  const int slot = logical / L.row_blocks;  // split slot in [0, B*NSPLIT)
  const SplitRange sr = split_plan(L, slot, true, lane);
  if (sr.b < 0) return;  // idle slot: no request owns it and the combine never reads it
  const int b = __builtin_amdgcn_readfirstlane(sr.b);
  const int s = slot - __builtin_amdgcn_readfirstlane(sr.first);
  const int nsb = __builtin_amdgcn_readfirstlane(sr.count);

  const int T = L.nodes;
  const int row = rb * (NWQ * 32) + wid * 32 + (lane & 31);
  const bool row_ok = qk_wave && row < L.rows;

  const uint32_t lds_kv = lds_addr(kv_s);
  const uint32_t lane16 = lane * 16;
  const uint64_t row_bytes = static_cast<uint64_t>(L.kv_row_bytes);

  // This lane's key in every tile: the wave streams keys 8 wid .. 8 wid + 7
  // (a 1 KiB latent load per key, one load for the rope parts of all eight),
  // and lane l's key, page-table entry and rope chunks are key 8 wid + l / 8.
  const int lkey = 8 * wid + (lane >> 3);
  const int32_t* pt_row = L.page_table + static_cast<size_t>(b) * L.max_pages;
  const uint32_t lds_pe = lds_addr(&pe_s[0][wid][0]);
  // Page-table entry of this lane's key in local tile k of the split (global
  // tile s + k nsb), into ring slot k % kPeRing. Positions past the table
  // read its last entry (such a key lies past the length and is never used).
  auto issue_pe = [&](int k) {
    // (64-bit: k runs up to five tiles past the split's last one)
    const int64_t p = (static_cast<int64_t>(s) + static_cast<int64_t>(k) * nsb) * kKeysPerTile + lkey;
    const int pc = static_cast<int>(min(p, static_cast<int64_t>(L.capacity - 1)));
    dma4(pt_row + (pc >> L.page_shift), lds_pe + (k % kPeRing) * (kWaves * 256));
  };

  // The length (scalar load) and the tree parents (wave 0); the page-table
  // entries of the split's first three tiles, which do not depend on the
  // length; then the query rows of the computing waves. For one request
  // nothing here waits for anything else.
  const int n_raw = kSparse ? raw_len(L, b) : L.seq_lens[b];
  int parent = -1;
  if (!kSparse && wid == 0 && lane < T) parent = L.tree_parent[static_cast<size_t>(b) * T + lane];
  issue_pe(0);
  issue_pe(1);
  issue_pe(2);
  // A computing wave's 32 query rows go to KV stage `wid` in the layout of a
  // key tile (row k of the wave in the place of key k), with the same
  // line-coalesced global->LDS loads; each lane then reads its B operands of
  // S^T = K Q^T from there exactly as it reads K fragments. (Loaded straight
  // into registers, every load instruction would gather 32 bytes from each
  // of 32 rows, and the rows of four waves do not fit the L1: each line came
  // from L2 four times over.) Padding rows load row 0 of the request; their
  // results are never stored.
  if (qk_wave) {
    const int r0 = rb * (NWQ * 32) + wid * 32;  // wave-uniform
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(L.q) + static_cast<size_t>(b) * L.rows * kRowBytes;
    const uint32_t stage = lds_kv + wid * kTileBytes;
#pragma unroll 4
    for (int k = 0; k < kKeysPerTile; ++k) {
      const int r = r0 + k < L.rows ? r0 + k : 0;
      dma16_sbase(qb + static_cast<size_t>(r) * kRowBytes, lane16 ^ (swz(k) << 4), stage + k * kLatentBytes);
    }
#pragma unroll
    for (int g = 0; g < kRopeInstr; ++g) {
      const int k = 8 * g + (lane >> 3);
      const int r = r0 + k < L.rows ? r0 + k : 0;
      dma16(qb + static_cast<size_t>(r) * kRowBytes + ((kVDim / 8 + ((lane & 7) ^ swz(k))) << 4),
            stage + kRopeBase + g * 1024);
    }
  }
  wait_vmcnt<0>();

  const int n = min(max(n_raw, kSparse ? 0 : T), L.capacity);
  if (n != n_raw && threadIdx.x == 0 && s == 0 && rb == 0 && cp == 0) atomicOr(L.err, MLA_DEVERR_SEQ_LEN);
  const int ctx = n - T;
  const int ntot = (n + kKeysPerTile - 1) / kKeysPerTile;  // key tiles of the request
  const int ntiles = s < ntot ? (ntot - 1 - s) / nsb + 1 : 0;

  f32x2* lse_dst =
      reinterpret_cast<f32x2*>(L.part_lse) + (static_cast<size_t>(slot) * kMaxColParts + cp) * L.rows_pad + row;
  if (ntiles == 0) {  // empty split: contributes nothing (every load above has landed)
    if (qk_wave && lane < 32) store_agent8(lse_dst, f32x2{-INFINITY, 0.f});
    return;
  }

  // Ancestor-or-self masks of the request's nodes (wave 0), read by every
  // row's lane after the barrier; sparse decode: every node is a root.
  if (wid == 0) {
    const int ln = fresh(lane);
    anc_s[ln] = kSparse ? (ln < T ? 1ull << ln : 0ull) : ancestor_bits_of(parent, T, ln, L.err);
  }
  lds_barrier();

  bf16x8 qf[kQSteps];  // lane: dims 16ks + 8*hsel + 0..7 of row lane%32
  uint64_t my_anc = 0;

  // Per-lane LDS offsets that do not change from tile to tile.
  const int kkey = lane & 31;
  const int kswz = swz(kkey);
  int koff[4];  // latent chunks; the rope chunks sit at koff + krope
#pragma unroll
  for (int r = 0; r < 4; ++r) koff[r] = kkey * kLatentBytes + (((2 * r + hsel) ^ kswz) << 4);
  const int krope = kRopeBase - kkey * (kLatentBytes - kRopeBytes);
  const int tg = lane >> 4, tj = lane & 15;
  const int vkey = 4 * hsel + (tj >> 2);  // + 16*kk + 8*u
  const int vy = (2 * (tg & 1) + ((tj & 3) >> 1)) ^ swz(vkey);
  const int voff_even = vkey * kLatentBytes + (tj & 1) * 8 + (vy << 4);
  const int voff_odd = vkey * kLatentBytes + (tj & 1) * 8 + ((vy ^ 4) << 4);

  f32x16 o[kCB];
  float m_ref = -INFINITY;  // reference max (log2 units) of this lane's row
  float m_max = -INFINITY;  // exact row max (pass B)
  float l_sum = 0.f;        // sum of fp32 weights (this lane's half of the keys)
  float l_pb = 0.f;         // sum of bf16-rounded weights
  bool overflow = false;    // a score left the range the reference can absorb
  float mu = 0.f;           // shift folded into the scaled scores: the reference once set, else 0
  bool unset = false;       // no reference after the split's first tile (set only in the adaptive pass)

  // ---- building blocks of the tile pipeline
  // K fragment of k-step ks (dims 16ks..16ks+15 of key lane%32).
  auto ld_k = [&](const uint8_t* st, int ks) {
    if (ks < kVDim / 16) return *reinterpret_cast<const bf16x8*>(st + koff[ks & 3] + (ks >> 2) * 128);
    return *reinterpret_cast<const bf16x8*>(st + koff[ks & 3] + krope);
  };

  // One MFMA step of S^T = K Q^T. The accumulator lives in VGPRs (the AGPR
  // file holds the whole O^T accumulator), so the step is issued as inline
  // asm with a VGPR destination: back-to-back accumulation into the same
  // registers needs no wait states; qk_done() adds the 20 wait states an XDL
  // result needs before a VALU instruction may read it.
  auto qk_step = [&](f32x16& acc, const bf16x8& a, const bf16x8& q, bool first) {
    if (first)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(q));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(q));
  };
  auto qk_done = [&](f32x16& acc) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc)); };
  auto qk = [&](const uint8_t* st) {  // S^T of a whole tile, not interleaved
    f32x16 acc;
    bf16x8 kf[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) kf[p] = ld_k(st, p);
    static_for<kQSteps>([&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      qk_step(acc, kf[ks & 3], qf[ks], ks == 0);
      if constexpr (ks + 4 < kQSteps) kf[ks & 3] = ld_k(st, ks + 4);
    });
    qk_done(acc);
    return acc;
  };

  // Row address of this lane's key in local tile k, from its page-table entry
  // in the ring: keys past the length, on an out-of-range slot or on an unused
  // (-1) index entry read the zero row instead, so that they enter both
  // products as exact zeros. Records the tile's bad-key bits (keys inside the
  // length that cannot be loaded) for the mask, and flags the bad ones.
  auto tile_addr = [&](int k) -> uint64_t {
    const int p = (s + k * nsb) * kKeysPerTile + lkey;
    const int32_t page = pe_s[k % kPeRing][wid][lane];
    const int64_t slot_id = (static_cast<int64_t>(page) << L.page_shift) + (p & ((1 << L.page_shift) - 1));
    const bool in_len = p < n;
    const bool ok = in_len && page >= 0 && slot_id < L.num_slots;
    const uint64_t addr = ok ? reinterpret_cast<uint64_t>(L.kv) + static_cast<uint64_t>(slot_id) * row_bytes
                             : reinterpret_cast<uint64_t>(kZeroRow);
    const uint64_t badm = __ballot(in_len && !ok);
    uint32_t byte = 0;
    if (badm != 0) {  // rare: one bit per key (lanes 8j hold key 8 wid + j)
      const uint64_t errm = kSparse ? __ballot(in_len && !ok && page != -1) : badm;
      if (errm != 0 && lane == 0) atomicOr(L.err, MLA_DEVERR_SLOT_RANGE);
#pragma unroll
      for (int j = 0; j < 8; ++j) byte |= static_cast<uint32_t>((badm >> (8 * j)) & 1u) << j;
    }
    if (lane == 0) reinterpret_cast<uint8_t*>(bad_s)[(k % kBadRing) * kWaves + wid] = static_cast<uint8_t>(byte);
    return addr;
  };
  // Load i of this wave for a tile whose key addresses are `addr`: the 1 KiB
  // latent part of key 8 wid + i (i < 8; its row address is wave-uniform), or
  // the rope parts of all eight keys (i = 8; a row address per lane).
  auto issue_one = [&](int k, int i, uint64_t addr) {
    const uint32_t stage = lds_kv + (k % kStages) * kTileBytes;
    if (i < 8) {
      const int key = 8 * wid + i;
      const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(addr), 8 * i);
      const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(addr >> 32), 8 * i);
      const void* rowp = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
      dma16_row(rowp, lane16, swz(key) << 4, stage, key * kLatentBytes);
    } else {
      const uint32_t chunk = (kVDim / 8 + ((lane & 7) ^ swz(lkey))) << 4;
      dma16(reinterpret_cast<const uint8_t*>(addr) + chunk, stage + kRopeBase + wid * 1024);
    }
  };
  auto issue_tile = [&](int k, uint64_t addr) {
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i) issue_one(k, i, addr);
  };

  // Visibility of the tile's 32 keys for this lane's row: context keys are
  // visible to every node, a tree key C + j only to the nodes with j in their
  // ancestor set, keys past the length or on a bad slot to nobody.
  auto visible_bits = [&](int k) -> uint32_t {
    const int p0 = (s + k * nsb) * kKeysPerTile;
    const int a = p0 - ctx;  // key k of the tile is tree node a + k when a + k >= 0
    const int left = n - p0;
    uint32_t bits = left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
    bits &= ~bad_s[k % kBadRing];
    // Keys before the tree (a + k < 0) are visible; node j = a + k is visible
    // when bit j of the ancestor mask is set. Selects, not branches: the
    // shifts are clamped to [0, 63] and the out-of-range cases chosen after.
    const uint64_t ctx_then_anc = (my_anc << 32) | 0xffffffffull;
    const uint32_t v_lo = static_cast<uint32_t>(ctx_then_anc >> min(max(a + 32, 0), 63));
    const uint32_t v_hi = static_cast<uint32_t>(my_anc >> min(max(a, 0), 63));
    const uint32_t vis = a < 0 ? (a <= -32 ? 0xffffffffu : v_lo) : (a < 64 ? v_hi : 0u);
    return bits & vis;
  };

  // Element j of a score tile is key 8*(j/4) + 4*hsel + j%4 of the tile.
  auto scale_mask = [&](const f32x16& acc, uint32_t vis, float (&tsc)[16]) {
    const uint32_t vsh = vis >> (4 * hsel);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      tsc[j] = ((vsh >> (8 * (j >> 2) + (j & 3))) & 1u) ? fmaf(acc[j], L.scale_log2, -mu) : -INFINITY;
    return (vsh & 0x0f0f0f0fu) != 0u;  // this lane sees a key of the tile
  };

  // Softmax of one tile, cut into pieces so that it can be spread between the
  // MFMAs of the next tile's scores. The scores arrive already shifted by the
  // row's reference (mu), so a weight is a single exp2.
  // Exact-max pass (kPassMaxOnly): pieces 0-8 row max, 9 running max.
  // Accumulating passes: pieces 0-7 weights of two elements each, 8 sums, the
  // P^T B operands of the two 16-key halves and the overflow check.
  struct SoftmaxState {
    float mx, ts, tb;
    bf16x2 pb2[8];
  };
  auto softmax_pieces = [](auto mode_tag) { return decltype(mode_tag)::value == kPassMaxOnly ? 10 : 9; };
  auto softmax_piece = [&](auto mode_tag, int piece, SoftmaxState& sm, const float (&tsc)[16], bf16x8 (&pf)[2]) {
    constexpr int kMode = decltype(mode_tag)::value;
    if constexpr (kMode == kPassMaxOnly) {
      if (piece == 0) {
        sm.mx = fmaxf(tsc[0], tsc[1]);
      } else if (piece < 8) {
        sm.mx = fmaxf(sm.mx, fmaxf(tsc[2 * piece], tsc[2 * piece + 1]));
      } else if (piece == 8) {
        sm.mx = fmaxf(sm.mx, xor32(sm.mx));
      } else if (piece == 9) {
        m_max = fmaxf(m_max, sm.mx);
      }
    } else {
      if (piece < 8) {
        const float p0 = __builtin_amdgcn_exp2f(tsc[2 * piece]);
        const float p1 = __builtin_amdgcn_exp2f(tsc[2 * piece + 1]);
        sm.ts = piece == 0 ? p0 + p1 : sm.ts + (p0 + p1);
        sm.pb2[piece] = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
        // the rounded pair summed in one bf16 dot product with (1, 1)
        sm.tb = __builtin_amdgcn_fdot2_f32_bf16(sm.pb2[piece],
                                                bf16x2{static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)},
                                                piece == 0 ? 0.f : sm.tb, false);
      } else if (piece == 8) {
        l_sum += sm.ts;
        l_pb += sm.tb;
        // A weight beyond 2^kRefHead (the lane's tile sum is a bound from
        // above) means a score the reference cannot absorb.
        if constexpr (kMode == kPassAdaptive) overflow |= !(sm.ts <= kHeadWeight);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          pf[kk] = bf16x8{sm.pb2[4 * kk][0], sm.pb2[4 * kk][1], sm.pb2[4 * kk + 1][0], sm.pb2[4 * kk + 1][1],
                          sm.pb2[4 * kk + 2][0], sm.pb2[4 * kk + 2][1], sm.pb2[4 * kk + 3][0], sm.pb2[4 * kk + 3][1]};
      }
    }
  };
  // Pins the values a piece produced at this point of the instruction stream
  // (the compiler may not sink the piece past the MFMA that follows).
  auto anchor = [&](auto mode_tag, int piece, SoftmaxState& sm, bf16x8 (&pf)[2]) {
    constexpr int kMode = decltype(mode_tag)::value;
    if constexpr (kMode == kPassMaxOnly) {
      asm volatile("" : "+v"(sm.mx));
    } else if (piece < 8) {
      asm volatile("" : "+v"(sm.ts), "+v"(sm.tb), "+v"(sm.pb2[piece]));
    } else if (piece == 8) {
      asm volatile("" : "+v"(pf[0]), "+v"(pf[1]));
    }
  };
  auto softmax = [&](auto mode_tag, const float (&tsc)[16], bf16x8 (&pf)[2]) {
    SoftmaxState sm;
#pragma unroll
    for (int piece = 0; piece < 10; ++piece)
      if (piece < softmax_pieces(mode_tag)) softmax_piece(mode_tag, piece, sm, tsc, pf);
  };

  // V^T fragment of PV step i (column block cp*kCB + i%kCB, keys
  // 16*(i/kCB)..+15); kCB is even, so the block's parity is i's.
  auto ld_v = [&](const uint8_t* st, int i, i16x4 (&v)[2]) {
    const int cb = i % kCB, kk = i / kCB;
    const uint8_t* vb = st + cp * (kCB / 2) * 128 + (cb & 1 ? voff_odd : voff_even) + (cb >> 1) * 128;
    v[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vb + (16 * kk) * kLatentBytes));
    v[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vb + (16 * kk + 8) * kLatentBytes));
  };
  // O^T += V^T P^T: 2*kCB MFMA steps into the AGPR-resident accumulator, V^T
  // reads three steps ahead. Keys 0-15 of the tile go into all kCB column
  // blocks before keys 16-31, so no MFMA waits for the one before it (a
  // dependent MFMA issues only after its predecessor has finished). Issued as
  // inline asm so that the order of loads, MFMAs and the interleaved VALU work
  // (between(i) after step i) is kept.
  auto pv = [&](const uint8_t* st, const bf16x8 (&pf)[2], auto&& between) {
    i16x4 vr[4][2];
#pragma unroll
    for (int i = 0; i < 3; ++i) ld_v(st, i, vr[i]);
#pragma unroll
    for (int i = 0; i < 2 * kCB; ++i) {
      if (i + 3 < 2 * kCB) ld_v(st, i + 3, vr[(i + 3) & 3]);
      const i16x8 v = __builtin_shufflevector(vr[i & 3][0], vr[i & 3][1], 0, 1, 2, 3, 4, 5, 6, 7);
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+a"(o[i % kCB])
                   : "v"(__builtin_bit_cast(bf16x8, v)), "v"(pf[i / kCB]));
      between(i);
    }
  };
  auto nothing = [](int) {};

  // One pass over the split's tiles, streamed through kStages LDS buffers.
  // Step t overlaps the scores of tile t+1 (MFMA) with the softmax of tile t
  // (VALU), then the PV product of tile t (MFMA) with the masking of tile
  // t+1's scores (VALU); every wave issues its loads of tile t+3 in between
  // and requests the page-table entries of tile t+5.
  // kCompute: the wave owns query rows. A wave without rows runs the same
  // pass with the same waits and barriers but only streams its keys: the two
  // kinds of wave never share a code path while the accumulator is live, so
  // it stays in the AGPRs.
  auto run_pass = [&](auto mode_tag, auto compute_tag) {
    constexpr int kMode = decltype(mode_tag)::value;
    constexpr bool kCompute = decltype(compute_tag)::value;
    constexpr bool kAccum = kMode != kPassMaxOnly && kCompute;
    if constexpr (kAccum) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) o[cb] = f32x16{};
      l_sum = 0.f;
      l_pb = 0.f;
    }
    mu = kMode == kPassFixed && m_ref != -INFINITY ? m_ref : 0.f;
    // The first pass's first page-table entries were requested in the
    // prologue; another pass requests them again once every wave is done with
    // the stages of the previous one.
    if constexpr (kMode != kPassAdaptive) {
      lds_barrier();
      issue_pe(0);
      issue_pe(1);
      issue_pe(2);
      wait_vmcnt<0>();
    }
    // Tiles 0-2, with the entries of tiles 3 and 4 requested between them in
    // the order the steps keep: entries of tile k + 2, then the loads of k.
    issue_tile(0, tile_addr(0));
    if (ntiles > 1) {
      issue_pe(3);
      issue_tile(1, tile_addr(1));
    }
    if (ntiles > 2) {
      issue_pe(4);
      issue_tile(2, tile_addr(2));
    }

    // Scores of tile 0 (loads complete in issue order: tiles 1 and 2 may
    // still be in flight).
    if (ntiles >= 3) wait_vmcnt<2 * kLoadsPerStep>();
    else if (ntiles == 2) wait_vmcnt<kLoadsPerStep>();
    else wait_vmcnt<0>();
    lds_barrier();
    float tsc[16];
    if constexpr (kCompute) scale_mask(qk(kv_s), visible_bits(0), tsc);
    if constexpr (kCompute && kMode == kPassAdaptive) {
      // The split's first tile fixes each row's reference: its max +
      // kRefLift (room for scores up to kRefLift + kRefHead above it). A row
      // it shows no key to keeps none; should a later tile show it one, the
      // split takes the exact path.
      float mx = tsc[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, tsc[j]);
      mx = fmaxf(mx, xor32(mx));
      m_ref = mx + kRefLift;  // -inf stays -inf
      mu = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
      for (int j = 0; j < 16; ++j) tsc[j] -= mu;  // these scores were taken unshifted
      unset = m_ref == -INFINITY;
    }

    // Step t: scores of tile t+1, softmax and PV of tile t, loads of tile
    // t+3. The steps that issue loads and the last two (which issue none)
    // are separate loops, so the steady state has no branches.
    auto step = [&](auto dma_tag, int t) {
      constexpr bool dma_next = decltype(dma_tag)::value;
      // Tile t+1 has landed (this wave's part, and with it the page-table
      // entries of tile t+3) once only the loads of the last step are
      // outstanding; the barrier also retires PV(t-1), freeing the stage that
      // tile t+3 loads into.
      if (dma_next || t + 2 < ntiles) wait_vmcnt<kLoadsPerStep>();
      else wait_vmcnt<0>();
      lds_barrier();
      uint64_t a3 = 0;
      if constexpr (dma_next) {
        a3 = tile_addr(t + 3);
        issue_pe(t + 5);
      }
      if constexpr (!kCompute) {  // a wave without query rows only streams its keys
        if constexpr (dma_next) issue_tile(t + 3, a3);
        return;
      }
      const uint8_t* st = kv_s + (t % kStages) * kTileBytes;
      const uint8_t* st1 = kv_s + ((t + 1) % kStages) * kTileBytes;

      // phase 1: the 36 MFMAs of QK(t+1) with K fragments prefetched four
      // steps ahead; between them the softmax of tile t (VALU) and the loads
      // of tile t+3 (one after every fourth MFMA).
      bf16x8 pf[2];
      {
        f32x16 acc;
        bf16x8 kf[4];
        SoftmaxState sm;
        constexpr int kDmaEvery = kQSteps / kLoadsPerTile;
#pragma unroll
        for (int p = 0; p < 4; ++p) kf[p] = ld_k(st1, p);
        static_for<kQSteps>([&](auto ks_c) {
          constexpr int ks = decltype(ks_c)::value;
          qk_step(acc, kf[ks & 3], qf[ks], ks == 0);
          if constexpr (ks + 4 < kQSteps) kf[ks & 3] = ld_k(st1, ks + 4);
          if constexpr (ks % 2 == 0 && ks / 2 < (kMode == kPassMaxOnly ? 10 : 9)) {
            softmax_piece(mode_tag, ks / 2, sm, tsc, pf);
            anchor(mode_tag, ks / 2, sm, pf);
          }
          if constexpr (dma_next && ks % kDmaEvery == kDmaEvery - 1) issue_one(t + 3, ks / kDmaEvery, a3);
        });
        qk_done(acc);

        // phase 2: PV(t) on the matrix cores; the masking of tile t+1's
        // scores (one element per step) on the VALU in between.
        const uint32_t vsh = visible_bits(t + 1) >> (4 * hsel);
        // (16 elements over 2*kCB steps: one per step, or 16/(2*kCB))
        constexpr int kMaskPer = 2 * kCB >= 16 ? 1 : 16 / (2 * kCB);
        // Scale on the VALU between the MFMAs; the mask after them, and only
        // for a tile that is not wholly visible (tree keys, the end of the
        // request, bad slots): a tile of context keys needs none.
        auto scale_step = [&](int i) {
#pragma unroll
          for (int k = 0; k < kMaskPer; ++k) {
            const int m = i * kMaskPer + k;
            if (m < 16) {
              tsc[m] = fmaf(acc[m], L.scale_log2, -mu);
              asm volatile("" : "+v"(tsc[m]));
            }
          }
        };
        if constexpr (kAccum) {
          pv(st, pf, scale_step);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) scale_step(i);
        }
        const int p1 = (s + (t + 1) * nsb) * kKeysPerTile;
        const bool all_visible =
            p1 + kKeysPerTile <= ctx && __builtin_amdgcn_readfirstlane(bad_s[(t + 1) % kBadRing]) == 0u;
        if (!all_visible) {
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            tsc[m] = ((vsh >> (8 * (m >> 2) + (m & 3))) & 1u) ? tsc[m] : -INFINITY;
            asm volatile("" : "+v"(tsc[m]));  // (keeps the branch: no speculative selects)
          }
          if constexpr (kMode == kPassAdaptive) overflow |= unset && (vsh & 0x0f0f0f0fu) != 0u;
        } else {
          if constexpr (kMode == kPassAdaptive) overflow |= unset;
        }
      }
    };
    int t = 0;
    for (; t + 3 < ntiles; ++t) step(BoolTag<true>{}, t);
    for (; t + 1 < ntiles; ++t) step(BoolTag<false>{}, t);
    // the split's last tile
    if constexpr (kCompute) {
      bf16x8 pf[2];
      softmax(mode_tag, tsc, pf);
      if constexpr (kAccum) pv(kv_s + ((ntiles - 1) % kStages) * kTileBytes, pf, nothing);
    }
  };

  // Workgroup-wide vote: did any row see a score the reference cannot absorb?
  // (the vote is taken by the whole wave: inside `lane == 0` it would see only
  // that lane's row)
  auto vote = [&]() {
    const bool wave_over = __any(overflow);
    if (lane == 0) over_s[wid] = wave_over;
    lds_barrier();
    bool any_over = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any_over |= over_s[w] != 0;
    return any_over;
  };
  if (!qk_wave) {
    lds_barrier();  // (the computing waves' query read-out)
    run_pass(PassMode<kPassAdaptive>{}, BoolTag<false>{});
    if (vote()) {
      run_pass(PassMode<kPassMaxOnly>{}, BoolTag<false>{});
      run_pass(PassMode<kPassFixed>{}, BoolTag<false>{});
    }
    return;
  }
  {  // the wave's query rows, from its own stage, into registers
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) qf[ks] = ld_k(kv_s + wid * kTileBytes, ks);
    const int r = rb * (NWQ * 32) + wid * 32 + (fresh(lane) & 31);
    my_anc = anc_s[(r < L.rows ? r : 0) / fresh(L.heads)];  // this lane's node (divisor rebuilt here too)
  }
  lds_barrier();  // the query rows are out of the stages before key tiles land there
  run_pass(PassMode<kPassAdaptive>{}, BoolTag<true>{});
  if (vote()) {  // rare: exact row max first, then accumulate against it
    run_pass(PassMode<kPassMaxOnly>{}, BoolTag<true>{});
    m_ref = m_max;
    run_pass(PassMode<kPassFixed>{}, BoolTag<true>{});
  }

  // ---- partial result of this split: O / l in fp16 and lse in log2 units,
  // stored at device scope (see store_agent8).
  // O / l is a convex combination of V rows; it is stored as fp16 scaled by
  // 2^-e, with e = 0 unless the largest |O / l| of the row's columns in this
  // part reaches 2^15 (then the smallest e that brings it below), and e is
  // kept beside the lse in the part's own record. fp16 adds at most 2^-12
  // relative to each stored value, well inside one bf16 rounding of the final
  // output.
  // (wait states between the last XDL write of O and the reads below)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
  const float l_sum_t = l_sum + __shfl_xor(l_sum, 32);
  const float l_pb_t = l_pb + __shfl_xor(l_pb, 32);
  const float inv = l_pb_t > 0.f ? 1.f / l_pb_t : 0.f;
  float amax = 0.f;
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(o[cb][j]));
  amax = fmaxf(amax, xor32(amax)) * inv;  // the row's values sit on lanes l and l ^ 32
  const int e = max(0, __builtin_amdgcn_frexp_expf(amax) - 15);
  if (lane < 32)
    store_agent8(lse_dst, f32x2{l_sum_t > 0.f ? m_ref + __builtin_amdgcn_logf(l_sum_t) : -INFINITY, static_cast<float>(e)});
  if (!row_ok) return;  // padding rows are never read
  const float sc = __builtin_ldexpf(inv, -e);
  f16x4* dst = reinterpret_cast<f16x4*>(L.part_o) + (static_cast<size_t>(slot) * (L.rows_pad / 32) + row / 32) * 4096 + lane;
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = f32x4{o[cb][4 * q], o[cb][4 * q + 1], o[cb][4 * q + 2], o[cb][4 * q + 3]} * sc;
      store_agent8(&dst[((cp * kCB + cb) * 4 + q) * 64], __builtin_convertvector(v, f16x4));
      if (q == 3) __builtin_amdgcn_sched_barrier(0);
    }
}

// Merge of the split partials of one fragment slot (32 rows x 8 columns). The
// kCombineWaves waves of the workgroup take every kCombineWaves-th split and
// keep a running merge per lane (its row, four columns): M = largest lse so
// far, acc = sum 2^(lse_s - M) O_s, w = sum 2^(lse_s - M), rescaled when M
// grows (O_s = stored fp16 x 2^e_s); empty splits (lse = -inf) are skipped. The
// waves' states are merged the same way in LDS. out = acc / w rounded to bf16
// once; lse = M + log2 w in natural-log units.
// The waves per workgroup follow NSPLIT (one round of 8 loads per wave where
// 16 waves allow it), so that a small NSPLIT does not spread one split per
// wave over workgroups that then wait on a cross-wave merge.
template <int kCombineWaves>
__global__ __launch_bounds__(kCombineWaves * 64, 4) void verify_combine_kernel(VerifyLaunch L) {
  __shared__ f32x4 red_acc[kCombineWaves][64];
  __shared__ float red_w[kCombineWaves][64];
  __shared__ float red_m[kCombineWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nwb = L.rows_pad / 32;
  const int frag = blockIdx.x & 63;
  const int wb = (blockIdx.x >> 6) % nwb;
  const int b = (blockIdx.x >> 6) / nwb;
  const int row = wb * 32 + (lane & 31);  // < rows_pad: its partial lse is always written
  const bool row_ok = row < L.rows;       // partial outputs exist for real rows only

  const SplitRange sr = split_plan(L, b, false, lane);  // this request's split slots
  const int first = __builtin_amdgcn_readfirstlane(sr.first);
  const int count = __builtin_amdgcn_readfirstlane(sr.count);
  // the record {lse, e} of the column part that wrote this fragment
  const int part = (frag >> 2) * L.col_parts / kColBlocks;
  const f32x2* pl =
      reinterpret_cast<const f32x2*>(L.part_lse) + (static_cast<size_t>(first) * kMaxColParts + part) * L.rows_pad + row;
  const size_t split_stride = static_cast<size_t>(nwb) * 4096;
  const f16x4* po = reinterpret_cast<const f16x4*>(L.part_o) + static_cast<size_t>(first) * split_stride +
                    static_cast<size_t>(wb) * 4096 + frag * 64 + lane;
  float mx = -INFINITY, wsum = 0.f;
  f32x4 acc = {};
  // Rounds of R splits per wave: all loads of a round go out before any is
  // used (indices past the request's last split repeat it and are masked;
  // padding rows load slots that lie inside the workspace and are discarded
  // by the select), so a wave waits for one round trip per round, not per
  // split. R is the wave's share of the splits rounded up to a power of two,
  // at most 8 (so that four waves fit per SIMD without spills), and few loads
  // are spent on repeats.
  auto rounds = [&](auto r_tag) {
    constexpr int R = decltype(r_tag)::value;
    for (int s0 = w; s0 < count; s0 += kCombineWaves * R) {
      f32x2 le[R];
      f16x4 vh[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int s = min(s0 + i * kCombineWaves, count - 1);
        le[i] = pl[static_cast<size_t>(s) * kMaxColParts * L.rows_pad];
        vh[i] = po[s * split_stride];
      }
      // (the values are taken here, unconditionally, so that no load is moved
      // under the branch of a masked split)
#pragma unroll
      for (int i = 0; i < R; ++i) asm volatile("" : "+v"(le[i]), "+v"(vh[i]));
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const f32x4 vi = __builtin_convertvector(vh[i], f32x4);
        const float l2 = le[i][0];
        const bool live = s0 + i * kCombineWaves < count && row_ok && l2 > -INFINITY;
        const float nm = live ? fmaxf(mx, l2) : mx;
        const float sc = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - nm);
        const float wt = live ? __builtin_amdgcn_exp2f(l2 - nm) : 0.f;
        acc = acc * sc + __builtin_ldexpf(wt, static_cast<int>(le[i][1])) * (live ? vi : f32x4{});
        wsum = wsum * sc + wt;
        mx = nm;
      }
    }
  };
  const int per_wave = (count + kCombineWaves - 1) / kCombineWaves;
  if (per_wave > 4) rounds(std::integral_constant<int, 8>{});
  else if (per_wave > 2) rounds(std::integral_constant<int, 4>{});
  else if (per_wave > 1) rounds(std::integral_constant<int, 2>{});
  else rounds(std::integral_constant<int, 1>{});
  red_acc[w][lane] = acc;
  red_w[w][lane] = wsum;
  red_m[w][lane] = mx;
  __syncthreads();
  if (w != 0 || !row_ok) return;
  float m_all = red_m[0][lane];
#pragma unroll
  for (int i = 1; i < kCombineWaves; ++i) m_all = fmaxf(m_all, red_m[i][lane]);
  acc = f32x4{};
  wsum = 0.f;
  if (m_all > -INFINITY) {
#pragma unroll
    for (int i = 0; i < kCombineWaves; ++i) {
      const float mi = red_m[i][lane];
      const float sc = mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - m_all);
      acc += sc * red_acc[i][lane];
      wsum += sc * red_w[i][lane];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const f32x4 r = acc * inv;
  const int col = (frag >> 2) * 32 + (frag & 3) * 8 + (lane >> 5) * 4;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<bf16x4*>(L.out + (static_cast<size_t>(b) * L.rows + row) * kVDim + col) =
      __builtin_convertvector(r, bf16x4);
  if (frag == 0 && lane < 32)
    L.lse[static_cast<size_t>(b) * L.rows + row] =
        wsum > 0.f ? (m_all + __builtin_amdgcn_logf(wsum)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

RowPlan plan_rows(int nodes, int heads) {
  RowPlan p;
  p.rows = nodes * heads;
  const int waves = (p.rows + kRowsPerWave - 1) / kRowsPerWave;
  p.waves_per_wg = waves < 4 ? waves : 4;
  p.row_blocks = (waves + p.waves_per_wg - 1) / p.waves_per_wg;
  p.rows_pad = p.row_blocks * p.waves_per_wg * kRowsPerWave;
  return p;
}

size_t part_lse_offset() { return kHeaderBytes; }

size_t part_o_offset(int batch, int nsplit, int rows_pad) {
  const size_t lse_bytes = static_cast<size_t>(batch) * nsplit * rows_pad * kMaxColParts * 2 * sizeof(float);
  return (part_lse_offset() + lse_bytes + 255) & ~static_cast<size_t>(255);
}

size_t workspace_bytes(int batch, int nsplit, int rows_pad) {
  return part_o_offset(batch, nsplit, rows_pad) +
         static_cast<size_t>(batch) * nsplit * rows_pad * kVDim * sizeof(uint16_t);
}

hipError_t launch_tree_mask(const int32_t* tree_parent, uint64_t* anc, int batch, int nodes,
                            uint32_t* err, hipStream_t stream) {
  hipLaunchKernelGGL(tree_mask_kernel, dim3(batch), dim3(64), 0, stream, tree_parent, anc, nodes, err);
  return hipGetLastError();
}

template <bool kSparse, int NCP>
void launch_partial_t(const VerifyLaunch& L, hipStream_t stream) {
  const int total = L.batch * L.nsplit * L.row_blocks * NCP;
  const int grid = (total + 7) / 8 * 8;
  const dim3 block(kWaves * 64);
  switch (L.waves_per_wg) {
    case 1: hipLaunchKernelGGL((verify_partial_kernel<1, kSparse, NCP>), dim3(grid), block, 0, stream, L); break;
    case 2: hipLaunchKernelGGL((verify_partial_kernel<2, kSparse, NCP>), dim3(grid), block, 0, stream, L); break;
    case 3: hipLaunchKernelGGL((verify_partial_kernel<3, kSparse, NCP>), dim3(grid), block, 0, stream, L); break;
    default: hipLaunchKernelGGL((verify_partial_kernel<4, kSparse, NCP>), dim3(grid), block, 0, stream, L); break;
  }
}

template <bool kSparse>
void launch_partial_s(const VerifyLaunch& L, hipStream_t stream) {
  if (L.col_parts == 4)
    launch_partial_t<kSparse, 4>(L, stream);
  else if (L.col_parts == 2)
    launch_partial_t<kSparse, 2>(L, stream);
  else
    launch_partial_t<kSparse, 1>(L, stream);
}

int col_parts_for(int batch, int nsplit, int row_blocks) {
  // Column parts while the (split, row block) workgroups would fill at most a
  // quarter (4 parts) or half (2 parts) of the CUs.
  const int64_t wgs = static_cast<int64_t>(batch) * nsplit * row_blocks;
  return wgs * 4 <= kCusPerDevice ? 4 : (wgs * 2 <= kCusPerDevice ? 2 : 1);
}

hipError_t launch_partial(const VerifyLaunch& L, hipStream_t stream) {
  if (L.quiet_unused)
    launch_partial_s<true>(L, stream);
  else
    launch_partial_s<false>(L, stream);
  return hipGetLastError();
}

hipError_t launch_combine(const VerifyLaunch& L, hipStream_t stream) {
  const int cgrid = L.batch * (L.rows_pad / 32) * 64;
  // Waves per workgroup: enough that a request's NSPLIT splits take one round
  // of 8 loads per wave (at most 16 waves), and no more: a small NSPLIT gets
  // small workgroups instead of waves that hold one split each.
  const int want = (L.nsplit + 7) / 8;
  if (want > 8)
    hipLaunchKernelGGL(verify_combine_kernel<16>, dim3(cgrid), dim3(16 * 64), 0, stream, L);
  else if (want > 4)
    hipLaunchKernelGGL(verify_combine_kernel<8>, dim3(cgrid), dim3(8 * 64), 0, stream, L);
  else if (want > 2)
    hipLaunchKernelGGL(verify_combine_kernel<4>, dim3(cgrid), dim3(4 * 64), 0, stream, L);
  else if (want > 1)
    hipLaunchKernelGGL(verify_combine_kernel<2>, dim3(cgrid), dim3(2 * 64), 0, stream, L);
  else
    hipLaunchKernelGGL(verify_combine_kernel<1>, dim3(cgrid), dim3(64), 0, stream, L);
  return hipGetLastError();
}

}  // namespace mlav

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
//    Each 16-byte chunk of a row lands at chunk ^ swz(key) inside its 128-byte
//    group so both LDS read patterns below are free of bank conflicts.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    K fragments come from LDS, the wave's 32 query rows stay in VGPRs for the
//    whole kernel. In the S^T accumulator every lane owns one query row, so the
//    row max needs one cross-lane step and P^T is already in the B-operand
//    layout of the next product.
//  * O^T += V^T P^T on the same MFMA; the V^T operand is read straight from the
//    row-major tile with ds_read_b64_tr_b16 (no transposed copy).
//  * Softmax in log2 units against a fixed per-row reference, set from the
//    first tile with a visible key (its max + kRefLift). Weights exp2(s - ref)
//    are accumulated without ever rescaling the accumulator, which therefore
//    only sees MFMA writes and stays in AGPRs. fp32 and bf16 share an 8-bit
//    exponent, so scores from ~94 below to kRefHead above the reference are
//    exact in relative terms; anything lower is negligible next to the row
//    max. Should a score rise beyond the reference + kRefHead (a gap of over
//    128 in log2 units, ~89 in natural units: not seen with attention scores
//    of ordinary range), the workgroup recomputes its split: one pass for the
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

#define LDS_AS __attribute__((address_space(3)))

constexpr int kKeysPerTile = 32;
constexpr int kRowBytes = kQkDim * 2;                              // 1152
constexpr int kChunksPerRow = kRowBytes / 16;                      // 72
constexpr int kTileBytes = kKeysPerTile * kRowBytes;               // 36864
constexpr int kTileInstr = kKeysPerTile * kChunksPerRow / 64;      // 36 wave-wide 1 KiB loads
constexpr int kStages = 4;
constexpr int kSlotCap = 2048;
constexpr int kQSteps = kQkDim / 16;                               // 36 k-steps of 16
constexpr int kColBlocks = kVDim / 32;                             // 16
constexpr float kRefLift = 32.0f;  // log2 units: reference above the first visible tile max
constexpr float kRefHead = 96.0f;  // log2 units: largest weight kept is 2^kRefHead

// Chunk permutation inside a 128-byte group, keyed by the key's index in the
// tile: 8 consecutive keys hit 8 distinct 16-byte slots (K reads), and the
// 32-byte pairs of 4 consecutive keys hit 4 distinct pairs (V^T reads).
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

// Ancestor-or-self bitmask of node `lane` (lanes >= T get 0) by pointer
// jumping: after round r a node's mask covers ancestors closer than 2^r and its
// pointer names the ancestor 2^r up. Six rounds cover 64 nodes. The whole wave
// must call it. A parent outside [-1, lane) is reported and replaced by -1.
__device__ uint64_t ancestor_bits(const int32_t* parents, int T, int lane, uint32_t* err) {
  int p = -1;
  bool bad = false;
  if (lane < T) {
    p = parents[lane];
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
constexpr int kPassAdaptive = 0;  // accumulate; reference = first visible tile max + kRefLift
constexpr int kPassMaxOnly = 1;   // scores only: exact row max over the split
constexpr int kPassFixed = 2;     // accumulate against a given reference

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void verify_partial_kernel(VerifyLaunch L) {
  constexpr int kInstrPerWave = kTileInstr / NW;
  static_assert(kTileInstr % NW == 0, "tile loads must split evenly over the waves");

  __shared__ __attribute__((aligned(1024))) uint8_t kv_s[kStages * kTileBytes];
  __shared__ int32_t slot_s[kSlotCap];
  __shared__ uint64_t anc_s[kMaxNodes];
  __shared__ int32_t badw_s[NW];
  __shared__ int32_t over_s[NW];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int hsel = lane >> 5;

  // XCD-aware order: workgroup i runs on XCD i % 8, so consecutive logical ids
  // (the row blocks of one split) are placed on one XCD in dispatch order.
  const int total = L.batch * L.nsplit * L.row_blocks;
  const int per_xcd = gridDim.x >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= total) return;
  const int rb = logical % L.row_blocks;
  const int bs = logical / L.row_blocks;
  const int s = bs % L.nsplit;
  const int b = bs / L.nsplit;

  const int T = L.nodes;
  const int n_raw = L.seq_lens[b];
  const int n = min(max(n_raw, T), L.capacity);
  if (n != n_raw && threadIdx.x == 0 && s == 0 && rb == 0) atomicOr(L.err, MLA_DEVERR_SEQ_LEN);
  const int ctx = n - T;
  const int chunk = (n + L.nsplit - 1) / L.nsplit;
  const int k0 = s * chunk;
  const int k1 = min(n, k0 + chunk);

  const int row = rb * (NW * 32) + wid * 32 + (lane & 31);
  const bool row_ok = row < L.rows;
  float* lse_dst = L.part_lse + (static_cast<size_t>(b) * L.nsplit + s) * L.rows_pad + row;
  if (k0 >= k1) {  // empty split: contributes nothing
    if (lane < 32) *lse_dst = -INFINITY;
    return;
  }

  // This wave's 32 query rows as B operands of S^T = K Q^T (k-step ks covers
  // dims 16ks..16ks+15; lane holds dims 16ks + 8*hsel + 0..7 of row lane%32).
  bf16x8 qf[kQSteps];
  {
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(L.q) +
                         (static_cast<size_t>(b) * L.rows + (row_ok ? row : 0)) * (kQkDim / 8);
    const bf16x8 zero = {};
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      const bf16x8 v = qrow[2 * ks + hsel];
      qf[ks] = row_ok ? v : zero;
    }
  }
  const int node = row_ok ? row / L.heads : 0;
  const bool need_mask = k1 > ctx;
  uint64_t my_anc = 0;
  bool win_bad = false;

  const uint32_t lds_kv = lds_addr(kv_s);

  // Per-lane LDS offsets that do not change from tile to tile.
  const int kkey = lane & 31;
  const int kswz = swz(kkey);
  int koff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) koff[r] = kkey * kRowBytes + (((2 * r + hsel) ^ kswz) << 4);
  const int tg = lane >> 4, tj = lane & 15;
  const int vkey = 4 * hsel + (tj >> 2);  // + 16*kk + 8*u
  const int vy = (2 * (tg & 1) + ((tj & 3) >> 1)) ^ swz(vkey);
  const int voff_even = vkey * kRowBytes + (tj & 1) * 8 + (vy << 4);
  const int voff_odd = vkey * kRowBytes + (tj & 1) * 8 + ((vy ^ 4) << 4);

  f32x16 o[kColBlocks];
  float m_ref = -INFINITY;  // reference max (log2 units) of this lane's row
  float m_max = -INFINITY;  // exact row max (pass B)
  float l_sum = 0.f;        // sum of fp32 weights (this lane's half of the keys)
  float l_pb = 0.f;         // sum of bf16-rounded weights
  bool overflow = false;    // a score left the range the reference can absorb

  // One pass over the split's keys: windows of up to kSlotCap keys, tiles of
  // 32 keys streamed through kStages LDS buffers.
  auto run_pass = [&](auto mode_tag) {
    constexpr int kMode = decltype(mode_tag)::value;
    constexpr bool kAccum = kMode != kPassMaxOnly;
    if constexpr (kAccum) {
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) o[cb] = f32x16{};
      l_sum = 0.f;
      l_pb = 0.f;
    }
    for (int w0 = k0; w0 < k1; w0 += kSlotCap) {
      const int wn = min(k1 - w0, kSlotCap);
      lds_barrier();  // everyone is done with the previous window or pass

      // Physical slot of every key in this window; -1 marks an out-of-range slot.
      int bad = 0;
      for (int i = threadIdx.x; i < wn; i += NW * 64) {
        const int p = w0 + i;
        const int page = L.page_table[static_cast<size_t>(b) * L.max_pages + (p >> L.page_shift)];
        const int64_t slot = (static_cast<int64_t>(page) << L.page_shift) + (p & ((1 << L.page_shift) - 1));
        const bool ok = page >= 0 && slot < L.num_slots;
        slot_s[i] = ok ? static_cast<int32_t>(slot) : -1;
        bad |= !ok;
      }
      const int wave_bad = __any(bad);
      if (lane == 0) badw_s[wid] = wave_bad;
      if (kMode == kPassAdaptive && need_mask && w0 == k0 && wid == 0) {
        const uint64_t a = ancestor_bits(L.tree_parent + static_cast<size_t>(b) * T, T, lane, L.err);
        anc_s[lane] = a;
      }
      lds_barrier();
      win_bad = false;
#pragma unroll
      for (int w = 0; w < NW; ++w) win_bad |= badw_s[w] != 0;
      if (kMode == kPassAdaptive) {
        if (win_bad && threadIdx.x == 0) atomicOr(L.err, MLA_DEVERR_SLOT_RANGE);
        if (need_mask && w0 == k0) my_anc = anc_s[node];
      }

      const int ntiles = (wn + kKeysPerTile - 1) / kKeysPerTile;

      auto issue_tile = [&](int t) {
        const int tk0 = t * kKeysPerTile;
        const uint32_t base = lds_kv + (t % kStages) * kTileBytes;
#pragma unroll 3
        for (int i = 0; i < kInstrPerWave; ++i) {
          const int ins = wid + i * NW;
          const int pos = ins * 64 + lane;  // 16-byte chunk position inside the tile
          const int key = pos / kChunksPerRow;
          const int c = (pos - key * kChunksPerRow) ^ swz(key);
          const int kk = min(tk0 + key, wn - 1);  // keys past the window reload a real row
          int slot = slot_s[kk];
          slot = slot < 0 ? 0 : slot;
          const uint8_t* g = L.kv + static_cast<size_t>(slot) * L.kv_row_bytes + c * 16;
          dma16(g, base + ins * 1024);
        }
      };

#pragma unroll
      for (int t = 0; t < kStages - 1; ++t)
        if (t < ntiles) issue_tile(t);

      for (int t = 0; t < ntiles; ++t) {
        const int ahead = min(kStages - 2, ntiles - 1 - t);
        if (ahead >= 2) wait_vmcnt<2 * kInstrPerWave>();
        else if (ahead == 1) wait_vmcnt<kInstrPerWave>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (t + kStages - 1 < ntiles) issue_tile(t + kStages - 1);

        const uint8_t* st = kv_s + (t % kStages) * kTileBytes;
        const int tk0 = t * kKeysPerTile;

        // ---- S^T = K Q^T for 32 keys x this wave's 32 rows
        f32x16 sacc = {};
#pragma unroll
        for (int ks = 0; ks < kQSteps; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + koff[ks & 3] + (ks >> 2) * 128);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc, 0, 0, 0);
          if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }

        // Element j of sacc is key tk0 + 8*(j/4) + 4*hsel + j%4 of row lane%32.
        float tsc[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) tsc[j] = sacc[j] * L.scale_log2;
        const bool special = (w0 + tk0 + kKeysPerTile > ctx) || (tk0 + kKeysPerTile > wn) || win_bad;
        if (special) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = tk0 + 8 * (j >> 2) + 4 * hsel + (j & 3);
            bool vis = key < wn;
            if (vis) {
              vis = slot_s[key] >= 0;
              const int p = w0 + key;
              if (p >= ctx) vis = vis && ((my_anc >> (p - ctx)) & 1ull);
            }
            tsc[j] = vis ? tsc[j] : -INFINITY;
          }
        }
        float mt = tsc[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mt = fmaxf(mt, tsc[j]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        if constexpr (kMode == kPassMaxOnly) {
          m_max = fmaxf(m_max, mt);
        } else {
          if constexpr (kMode == kPassAdaptive) {
            // The first visible tile fixes the reference. Lifting it by
            // kRefLift leaves room for scores up to kRefLift + kRefHead above
            // that tile's max before a weight could overflow.
            if (m_ref == -INFINITY && mt > -INFINITY) m_ref = mt + kRefLift;
            overflow |= mt > m_ref + kRefHead;
          }
          const float mu = m_ref == -INFINITY ? 0.f : m_ref;
          float ps[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) ps[j] = __builtin_amdgcn_exp2f(tsc[j] - mu);

          bf16x2 pb2[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) pb2[k] = __builtin_convertvector(f32x2{ps[2 * k], ps[2 * k + 1]}, bf16x2);
          float ts = 0.f, tb = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) ts += ps[j];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const f32x2 back = __builtin_convertvector(pb2[k], f32x2);
            tb += back[0] + back[1];
          }
          l_sum += ts;
          l_pb += tb;
          bf16x8 pf[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            pf[kk] = bf16x8{pb2[4 * kk][0], pb2[4 * kk][1], pb2[4 * kk + 1][0], pb2[4 * kk + 1][1],
                            pb2[4 * kk + 2][0], pb2[4 * kk + 2][1], pb2[4 * kk + 3][0], pb2[4 * kk + 3][1]};

          // ---- O^T += V^T P^T; V^T fragments via transposing LDS reads
#pragma unroll
          for (int cb = 0; cb < kColBlocks; ++cb) {
            const uint8_t* vb = st + (cb & 1 ? voff_odd : voff_even) + (cb >> 1) * 128;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vb + (16 * kk) * kRowBytes));
              const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vb + (16 * kk + 8) * kRowBytes));
              const i16x8 v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
              o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), pf[kk], o[cb], 0, 0, 0);
            }
            if (cb & 1) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  };

  run_pass(PassMode<kPassAdaptive>{});
  // Workgroup-wide vote: did any row see a score the reference cannot absorb?
  if (lane == 0) over_s[wid] = __any(overflow);
  lds_barrier();
  bool any_over = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) any_over |= over_s[w] != 0;
  if (any_over) {  // rare: exact row max first, then accumulate against it
    run_pass(PassMode<kPassMaxOnly>{});
    m_ref = m_max;
    run_pass(PassMode<kPassFixed>{});
  }

  // ---- partial result of this split: O / l (fp32) and lse in log2 units
  const float l_sum_t = l_sum + __shfl_xor(l_sum, 32);
  const float l_pb_t = l_pb + __shfl_xor(l_pb, 32);
  if (lane < 32) *lse_dst = l_sum_t > 0.f ? m_ref + __builtin_amdgcn_logf(l_sum_t) : -INFINITY;
  const float inv = l_pb_t > 0.f ? 1.f / l_pb_t : 0.f;
  f32x4* dst = reinterpret_cast<f32x4*>(L.part_o) +
               ((static_cast<size_t>(b) * L.nsplit + s) * (L.rows_pad / 32) + row / 32) * 4096 + lane;
#pragma unroll
  for (int cb = 0; cb < kColBlocks; ++cb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
    {
      dst[(cb * 4 + q) * 64] = f32x4{o[cb][4 * q] * inv, o[cb][4 * q + 1] * inv, o[cb][4 * q + 2] * inv,
                                     o[cb][4 * q + 3] * inv};
      if (q == 3) __builtin_amdgcn_sched_barrier(0);
    }
}

// Merge of the split partials of one fragment slot (32 rows x 8 columns): the
// four waves of the workgroup take every fourth split, so a slot's partials
// are read with four waves' worth of loads in flight. Pass 1 finds each row's
// largest partial lse M; pass 2 accumulates w_s = 2^(lse_s - M) and w_s * O_s
// (empty splits have lse = -inf and are skipped); the waves' sums are added in
// LDS. out = sum w_s O_s / sum w_s rounded to bf16 once; lse = M + log2 sum w_s,
// converted to natural-log units.
constexpr int kCombineWaves = 4;

__global__ __launch_bounds__(kCombineWaves * 64) void verify_combine_kernel(VerifyLaunch L) {
  __shared__ float red_m[kCombineWaves][32];
  __shared__ f32x4 red_acc[kCombineWaves][64];
  __shared__ float red_w[kCombineWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nwb = L.rows_pad / 32;
  const int frag = blockIdx.x & 63;
  const int wb = (blockIdx.x >> 6) % nwb;
  const int b = (blockIdx.x >> 6) / nwb;
  const int row = wb * 32 + (lane & 31);  // < rows_pad: its partial lse is always written

  const float* pl = L.part_lse + static_cast<size_t>(b) * L.nsplit * L.rows_pad + row;
  float mx = -INFINITY;
#pragma unroll 8
  for (int s = w; s < L.nsplit; s += kCombineWaves) mx = fmaxf(mx, pl[static_cast<size_t>(s) * L.rows_pad]);
  if (lane < 32) red_m[w][lane] = mx;
  __syncthreads();
  mx = red_m[0][lane & 31];
#pragma unroll
  for (int i = 1; i < kCombineWaves; ++i) mx = fmaxf(mx, red_m[i][lane & 31]);

  f32x4 acc = {};
  float wsum = 0.f;
  if (mx > -INFINITY) {
    const size_t split_stride = static_cast<size_t>(nwb) * 4096;
    const f32x4* po = reinterpret_cast<const f32x4*>(L.part_o) +
                      static_cast<size_t>(b) * L.nsplit * split_stride + static_cast<size_t>(wb) * 4096 +
                      frag * 64 + lane;
#pragma unroll 8
    for (int s = w; s < L.nsplit; s += kCombineWaves) {
      const float l2 = pl[static_cast<size_t>(s) * L.rows_pad];
      const f32x4 v = po[s * split_stride];
      const bool live = l2 > -INFINITY;
      const float wt = live ? __builtin_amdgcn_exp2f(l2 - mx) : 0.f;
      acc += wt * (live ? v : f32x4{});
      wsum += wt;
    }
  }
  red_acc[w][lane] = acc;
  red_w[w][lane] = wsum;
  __syncthreads();
  if (w != 0 || row >= L.rows) return;
#pragma unroll
  for (int i = 1; i < kCombineWaves; ++i) {
    acc += red_acc[i][lane];
    wsum += red_w[i][lane];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const f32x4 r = acc * inv;
  const int col = (frag >> 2) * 32 + (frag & 3) * 8 + (lane >> 5) * 4;
  const bf16x2 lo = __builtin_convertvector(f32x2{r[0], r[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector(f32x2{r[2], r[3]}, bf16x2);
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4* dst = reinterpret_cast<bf16x4*>(L.out + (static_cast<size_t>(b) * L.rows + row) * kVDim + col);
  *dst = bf16x4{lo[0], lo[1], hi[0], hi[1]};
  if (frag == 0 && lane < 32)
    L.lse[static_cast<size_t>(b) * L.rows + row] =
        wsum > 0.f ? (mx + __builtin_amdgcn_logf(wsum)) * 0.69314718055994530942f : -INFINITY;
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
  const size_t lse_bytes = static_cast<size_t>(batch) * nsplit * rows_pad * sizeof(float);
  return (part_lse_offset() + lse_bytes + 255) & ~static_cast<size_t>(255);
}

size_t workspace_bytes(int batch, int nsplit, int rows_pad) {
  return part_o_offset(batch, nsplit, rows_pad) +
         static_cast<size_t>(batch) * nsplit * rows_pad * kVDim * sizeof(float);
}

hipError_t launch_tree_mask(const int32_t* tree_parent, uint64_t* anc, int batch, int nodes,
                            uint32_t* err, hipStream_t stream) {
  hipLaunchKernelGGL(tree_mask_kernel, dim3(batch), dim3(64), 0, stream, tree_parent, anc, nodes, err);
  return hipGetLastError();
}

hipError_t launch_partial(const VerifyLaunch& L, hipStream_t stream) {
  const int total = L.batch * L.nsplit * L.row_blocks;
  const int grid = (total + 7) / 8 * 8;
  switch (L.waves_per_wg) {
    case 1: hipLaunchKernelGGL(verify_partial_kernel<1>, dim3(grid), dim3(64), 0, stream, L); break;
    case 2: hipLaunchKernelGGL(verify_partial_kernel<2>, dim3(grid), dim3(128), 0, stream, L); break;
    case 3: hipLaunchKernelGGL(verify_partial_kernel<3>, dim3(grid), dim3(192), 0, stream, L); break;
    default: hipLaunchKernelGGL(verify_partial_kernel<4>, dim3(grid), dim3(256), 0, stream, L); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const VerifyLaunch& L, hipStream_t stream) {
  const int cgrid = L.batch * (L.rows_pad / 32) * 64;
  hipLaunchKernelGGL(verify_combine_kernel, dim3(cgrid), dim3(kCombineWaves * 64), 0, stream, L);
  return hipGetLastError();
}

}  // namespace mlav

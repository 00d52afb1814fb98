/*
 * mla_verify.h - C ABI of the MI355X (gfx950) verify attention for tree
 * speculative decoding over a paged MLA latent KV cache.
 *
 * The operation. Page "The Custom sm_120 Verify Kernel: From 0.7 tok/s to 3-6x
 * Decode Speedup on Blackwell Consumer GPUs":
 *   - Part VI: in the verify step every draft-tree node of a request is a
 *     query against the request's latent KV, under a custom tree mask, with a
 *     page size of 1 because accepted tree nodes sit on scattered slots.
 *   - Part VII: the committed prefix is visible to every node without a mask;
 *     only the small tree block is masked. The KV is split into NSPLIT chunks
 *     that each yield a partial result, and a reduce merges the partials.
 *   - Part VII, "Making the Kernel CUDA Graph Capture-Safe": static buffers, a
 *     fixed NSPLIT, a caller-allocated workspace, no host synchronisation and
 *     no allocation on the call path.
 *   - Part IX, "The Debugging Gauntlet", Bug 2: the keys of a request are its
 *     prefix slots followed by the draft tokens' own slots, and the mask stride
 *     is prefix + q_len.
 *
 * Definition computed, for request b, node i, head h:
 *   N = seq_lens[b] (tree rows included), C = N - T,
 *   slot(p) = page_table[b*max_pages + p/page_size]*page_size + p%page_size,
 *   k_p = kv_cache[slot(p), 0:576], v_p = kv_cache[slot(p), 0:512],
 *   Anc*(i) = {i} u Anc*(tree_parent[b][i]) ({i} for a root),
 *   visible keys: every p < C, and C + j for each j in Anc*(i),
 *   s_p = sm_scale * <q[b,i,h,:], k_p>,
 *   lse[b,i,h] = ln sum_p exp(s_p),  out[b,i,h,:] = sum_p exp(s_p - lse) v_p.
 * A node sees itself, so a chain tree is a causal block. lse is in natural-log
 * units and includes sm_scale.
 *
 * Conventions for every entry point:
 *   - Every pointer argument is device memory owned by the caller. The library
 *     allocates nothing, keeps no pointer after returning, holds no global
 *     mutable state and reads no environment variables. Distinct workspaces
 *     make concurrent calls safe.
 *   - Work is enqueued on `stream`; the call never synchronises, never copies
 *     device data to the host and never allocates, so it may be captured into a
 *     hipGraph (global capture mode). The grid depends only on the descriptor.
 *   - A negative status means nothing was enqueued (bad descriptor, null or
 *     misaligned pointer, small workspace), except MLA_ERR_HIP, which reports
 *     a failed launch.
 *   - Bad data is only visible on the device. It never traps; it sets sticky
 *     bits in a device error word and gets a defined fallback (see
 *     MLA_DEVERR_*).
 */
#ifndef MLA_VERIFY_H
#define MLA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_VERIFY_ABI_VERSION 1

#ifndef MLA_API
#define MLA_API __attribute__((visibility("default")))
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is null */
  MLA_ERR_SHAPE = -2,       /* a dimension is out of its range */
  MLA_ERR_UNSUPPORTED = -3, /* head dims other than 576/512, page size not a power of two */
  MLA_ERR_WORKSPACE = -4,   /* workspace smaller than mla_verify_workspace_bytes() */
  MLA_ERR_ALIGN = -5,       /* q, kv_cache, out or workspace not 16-byte aligned */
  MLA_ERR_HIP = -6,         /* a kernel launch failed (hipGetLastError) */
  MLA_ERR_SCRATCH = -7      /* mla_verify_attention_noalloc: the problem needs more than
                               MLA_VERIFY_NOALLOC_SCRATCH_BYTES of scratch */
} mla_status;

/* Sticky bits of the device error word (uint32). */
#define MLA_DEVERR_BAD_PARENT 1u /* tree_parent[i] not in [-1, i): node treated as a root */
#define MLA_DEVERR_SEQ_LEN 2u    /* seq_lens[b] outside [T, max_pages*page_size]: clamped */
#define MLA_DEVERR_SLOT_RANGE 4u /* a page id < 0 or a slot >= num_kv_slots: that key is masked */

/* Shapes and scalars of one call. All of it is known on the host; none of it
 * is read from device memory, so it fixes the launch shape for a capture. The
 * eight int32 fields come first and the two int64 fields after them, so the
 * struct has no padding hole for a foreign-function mirror to get wrong
 * (8 x 4 + 2 x 8 + 4 = 52 bytes, 56 with the tail padding). */
typedef struct {
  int32_t batch;         /* B >= 1 requests */
  int32_t num_nodes;     /* T in [1, 64]: draft-tree nodes = verify queries per request */
  int32_t num_heads;     /* H >= 1 query heads; all read the one latent row (MLA) */
  int32_t head_dim_qk;   /* must be 576 (512 latent + 64 rope) */
  int32_t head_dim_v;    /* must be 512: V is kv_cache[slot, 0:512] */
  int32_t page_size;     /* power of two >= 1 (1 for scattered tree slots, 64 for block pages) */
  int32_t max_pages;     /* row stride of page_table; a request holds <= max_pages*page_size keys */
  int32_t nsplit;        /* >= 1: KV chunks per request on average. The B*nsplit chunk slots are
                            shared out over the requests in proportion to their key counts
                            (one at least each; equal lengths give nsplit each). Results do not
                            depend on it beyond rounding. */
  int64_t num_kv_slots;  /* rows in kv_cache; slots >= this are out of range */
  int64_t kv_row_stride; /* elements between consecutive kv_cache rows: >= 576, multiple of 8, <= 2^30 */
  float sm_scale;        /* softmax scale applied to q.k (1/sqrt(192) for 128 nope + 64 rope) */
} mla_verify_desc;

/* Bytes of workspace mla_verify_attention needs for this descriptor (page "The
 * Custom sm_120 Verify Kernel ...", Part VII, "Making the Kernel CUDA Graph
 * Capture-Safe": the split partials live in a workspace the caller allocates
 * once, outside the captured region, so the call itself allocates nothing).
 * Layout: a 256-byte header whose first 4 bytes are the device error word (the
 * rest of the header is reserved), then per-split partial log-sum-exps and
 * partial outputs (fp16). Returns 0 for a descriptor that mla_verify_attention
 * would reject. Pure host arithmetic: no device access. */
MLA_API size_t mla_verify_workspace_bytes(const mla_verify_desc* d);

/* Ancestor bitmask of each request's draft tree (page "The Capstone Report:
 * When Kernel Engineering Meets Honest Bottleneck Analysis", section 2: the
 * reference builds this mask on the host each step; here it is built on the
 * device). anc_mask[b*T + i] has bit j set iff node j is node i or one of its
 * ancestors.
 *   tree_parent: int32 [batch, num_nodes], -1 for a root, else an index < i.
 *   anc_mask:    uint64 [batch, num_nodes], written.
 *   dev_err:     uint32 error word, may be null; MLA_DEVERR_BAD_PARENT is OR-ed
 *                in for a parent outside [-1, i), and that node is a root.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (batch < 1 or num_nodes not in [1, 64]),
 * MLA_ERR_HIP. */
MLA_API mla_status mla_build_tree_mask(const int32_t* tree_parent, uint64_t* anc_mask, int32_t batch,
                               int32_t num_nodes, uint32_t* dev_err, hipStream_t stream);

/* Tree-masked MLA verify attention over a paged latent KV pool, split into
 * d->nsplit chunks per request with a log-sum-exp merge (the definition at the
 * top of this header).
 *   q:           bf16 [B, T, H, 576], row-contiguous, 16-byte aligned.
 *   kv_cache:    bf16 [num_kv_slots, kv_row_stride]; the first 576 entries of a
 *                row are the latent (512) and rope (64) parts. 16-byte aligned.
 *   page_table:  int32 [B, max_pages]: physical page ids. Entries past
 *                ceil(seq_lens[b]/page_size) are never read.
 *   seq_lens:    int32 [B]: keys of request b including its T tree rows. The
 *                tree node j's latent row is logical key seq_lens[b] - T + j.
 *   tree_parent: int32 [B, T]: -1 for a root, else an earlier node.
 *   out:         bf16 [B, T, H, 512], written (fp32 accumulation, one rounding).
 *   lse:         fp32 [B, T, H], written (natural log).
 *   workspace:   >= mla_verify_workspace_bytes(d) bytes, 16-byte aligned. Its
 *                first 4 bytes are the sticky device error word (MLA_DEVERR_*);
 *                the caller zeroes it when it wants to start afresh and reads
 *                it whenever it chooses. The rest is scratch.
 *   workspace_bytes: size of `workspace`; MLA_ERR_WORKSPACE if below
 *                mla_verify_workspace_bytes(d). (An argument beyond the
 *                problem's own list: it lets the host reject a short
 *                workspace before anything is enqueued.)
 *   stream:      HIP stream to enqueue on (0 = the null stream).
 * Fallbacks for bad data (with the matching error bit): a bad parent makes that
 * node a root; seq_len is clamped to [T, max_pages*page_size]; a key on an
 * out-of-range slot is masked out. A row left with no visible key gets lse =
 * -inf and out = 0. */
MLA_API mla_status mla_verify_attention(const mla_verify_desc* d, const void* q, const void* kv_cache,
                                const int32_t* page_table, const int32_t* seq_lens,
                                const int32_t* tree_parent, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The two stages of mla_verify_attention, for callers that schedule or time
 * them separately (page "The Custom sm_120 Verify Kernel ...", Part VII: a
 * partial kernel per KV split, then a reduce). mla_verify_partial writes the
 * per-split partial outputs and log-sum-exps into the workspace;
 * mla_verify_combine merges them into out and lse. Called back to back on one
 * stream with the same descriptor and workspace they equal one
 * mla_verify_attention call. Arguments, checks and errors as above. */
MLA_API mla_status mla_verify_partial(const mla_verify_desc* d, const void* q, const void* kv_cache,
                                      const int32_t* page_table, const int32_t* seq_lens,
                                      const int32_t* tree_parent, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);
MLA_API mla_status mla_verify_combine(const mla_verify_desc* d, void* out, float* lse, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code (the mla_status values above; no page
 * defines them). Never null; unknown codes give "unknown status". */
MLA_API const char* mla_status_string(mla_status s);

/* Largest scratch mla_verify_attention_noalloc can use on one GPU: calls whose
 * mla_verify_workspace_bytes(d) exceeds it are rejected with MLA_ERR_SCRATCH. */
#define MLA_VERIFY_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* mla_verify_attention for callers that cannot allocate device memory at all:
 * code under hipGraph capture that must not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation. Instead of a caller-provided workspace, the
 * split partials live in a static scratch array of
 * MLA_VERIFY_NOALLOC_SCRATCH_BYTES in the library's device code: every GPU the
 * library runs on holds one copy of it until the process ends, and its device
 * address is looked up once per device, on the first call made with that
 * device current (that first call is the only one that touches the HIP
 * runtime beyond enqueuing the two kernels; it allocates nothing).
 *   q, kv_cache, page_table, seq_lens, tree_parent, out, lse: as for
 *                mla_verify_attention.
 *   dev_err:     uint32 sticky device error word (MLA_DEVERR_*), caller-owned
 *                and caller-cleared, 4-byte aligned; may be null, then data
 *                errors still get their fallbacks but are not reported.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents: calls that overlap in time on one GPU (concurrent streams, or
 * threads without ordering) race and must not be made. Nothing in the scratch
 * has to start at zero: each call writes every partial it reads back.
 * Errors: as mla_verify_attention (no MLA_ERR_WORKSPACE), plus MLA_ERR_SCRATCH
 * when mla_verify_workspace_bytes(d) > MLA_VERIFY_NOALLOC_SCRATCH_BYTES, and
 * MLA_ERR_HIP when the scratch address cannot be looked up; nothing is
 * enqueued in either case. Results are bitwise those of mla_verify_attention
 * (the same kernels). */
MLA_API mla_status mla_verify_attention_noalloc(const mla_verify_desc* d, const void* q, const void* kv_cache,
                                                const int32_t* page_table, const int32_t* seq_lens,
                                                const int32_t* tree_parent, void* out, float* lse,
                                                uint32_t* dev_err, hipStream_t stream);

/* MLA_VERIFY_ABI_VERSION of the built library. */
MLA_API int32_t mla_verify_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H */

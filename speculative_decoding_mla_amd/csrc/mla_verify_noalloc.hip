// The verify call for callers that cannot allocate: the split partials live in
// a file-scope device array instead of a caller-provided workspace. The kernels
// are the ones mla_verify_attention launches; only the buffer differs.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>

#include "mla_verify.h"
#include "mla_verify_internal.h"

namespace {

constexpr size_t kScratchBytes = MLA_VERIFY_NOALLOC_SCRATCH_BYTES;

// One copy per GPU, at that GPU's own address. In host code the name is only
// a handle for the runtime: kernels get the device address looked up below.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_lookup;

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" mla_status mla_verify_attention_noalloc(const mla_verify_desc* d, const void* q, const void* kv_cache,
                                                   const int32_t* page_table, const int32_t* seq_lens,
                                                   const int32_t* tree_parent, void* out, float* lse,
                                                   uint32_t* dev_err, hipStream_t stream) {
  const mla_status st = mlav::check_desc(d);
  if (st != MLA_OK) return st;
  if (mla_verify_workspace_bytes(d) > kScratchBytes) return MLA_ERR_SCRATCH;
  if (dev_err != nullptr && mlav::misaligned(dev_err, 4)) return MLA_ERR_ALIGN;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return MLA_ERR_HIP;
  mlav::VerifyLaunch L;
  const mla_status pst =
      mlav::prepare(d, q, kv_cache, page_table, seq_lens, tree_parent, out, lse, ws, kScratchBytes, true, true, &L);
  if (pst != MLA_OK) return pst;
  // Data errors go to the caller's word; without one, to the scratch header
  // (written, never read).
  if (dev_err != nullptr) L.err = dev_err;
  if (mlav::launch_partial(L, stream) != hipSuccess) return MLA_ERR_HIP;
  return mlav::launch_combine(L, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

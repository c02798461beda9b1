// Decode attention for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the per-split partial results
// live in a fixed array of this library's device code instead of a caller workspace.
//
// Each GPU the library runs on holds its own copy of `scratch` at its own address, found once
// per device with hipGetSymbolAddress; host code passes only that address to kernels (the
// array's name on the host is a stand-in, not a device address). Every call on one GPU shares
// that GPU's copy, so calls that overlap on one GPU race; nothing in it has to start at zero
// (every split writes all of its partial results before the merge reads them).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "qwen3_prefill.h"

namespace q3 {
int set_error(int status, const char* msg);  // capi.hip: the text qwen3_last_error() returns
}

namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;  // QWEN3_NOALLOC_SCRATCH_BYTES in the header
static_assert(kScratchBytes == QWEN3_NOALLOC_SCRATCH_BYTES, "header and library disagree");

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this GPU's `scratch` (looked up on the first call on each device, with that
// device current), or nullptr with the error text set.
void* scratch_ptr() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    q3::set_error(QWEN3_ERR_HIP, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    q3::set_error(QWEN3_ERR_UNSUPPORTED, "device index beyond the no-allocation table");
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      q3::set_error(QWEN3_ERR_HIP, e != hipSuccess ? hipGetErrorString(e) : "scratch symbol has no address");
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int gqa_decode_attention_noalloc(const float* q, const void* k_cache, const void* v_cache,
                                            int32_t capacity, int32_t len, int32_t n_heads, int32_t n_kv_heads,
                                            int32_t head_dim, float scale, qwen3_dtype cache_dtype, float* out,
                                            void* stream) {
  const size_t need = gqa_decode_attention_workspace_bytes(n_heads, n_kv_heads, head_dim, len);
  if (need > kScratchBytes)
    return q3::set_error(QWEN3_ERR_UNSUPPORTED,
                         "gqa_decode_attention_noalloc: these heads and length need more partial-result "
                         "memory than the fixed 8 MiB (use gqa_decode_attention with a workspace)");
  void* ws = scratch_ptr();
  if (!ws) return QWEN3_ERR_HIP;
  // the same checks and kernels as the workspace form, on this device's fixed array; a zero
  // `need` (invalid heads or length) is rejected there with its own message
  return gqa_decode_attention(q, k_cache, v_cache, capacity, len, n_heads, n_kv_heads, head_dim, scale,
                              cache_dtype, out, ws, kScratchBytes, stream);
}

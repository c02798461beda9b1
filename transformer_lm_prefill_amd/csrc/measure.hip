// Measurement aid: an MFMA throughput probe. Each wave issues `iters` rounds of 8 independent
// v_mfma_f32_32x32x16_f16 (no memory traffic, operands that differ per lane and per round), so
// the launch runs at the matrix cores' issue rate for the clock the chip holds under that load.
// Lane 0 of workgroup 0 reads the shader clock counter (s_memtime) and the fixed 100 MHz real-
// time counter (s_memrealtime) before and after its loop, giving the clock during the probe.
#include <hip/hip_runtime.h>

#include "common.h"
#include "qwen3_prefill.h"

namespace q3 {
int set_error(int status, const char* msg);  // capi.hip
}

namespace {

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink, unsigned long long* clocks) {
  const int lane = threadIdx.x & 63;
  u32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = 0x3c003c00u ^ (static_cast<uint32_t>(lane * 2654435761u + e * 40503u) & 0x03ff03ffu);
    b[e] = 0x3c003c00u ^ (static_cast<uint32_t>((lane + 17) * 2246822519u + e * 12289u) & 0x03ff03ffu);
  }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long c0 = 0, r0 = 0;
  if (timer) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = q3::Fmt<q3::OP_F16>::mfma(a, b, acc[i]);
    // new operand bits every round (one VALU op per 8 MFMAs)
    a[it & 3] ^= 0x00010001u;
  }
  if (timer) {
    clocks[0] = __builtin_amdgcn_s_memtime() - c0;
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][lane & 15];
  if (s == 1234.5f) sink[0] = s;  // keeps the products alive; never true for these operands
}

}  // namespace

extern "C" int qwen3_mfma_probe(int32_t workgroups, int32_t iters, float* sink, unsigned long long* clocks,
                                void* stream) {
  if (workgroups < 1 || iters < 1) return q3::set_error(QWEN3_ERR_INVALID_ARG, "workgroups and iters must be >= 1");
  if (!sink || !clocks) return q3::set_error(QWEN3_ERR_INVALID_ARG, "sink / clocks is NULL");
  mfma_probe_kernel<<<workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink, clocks);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? QWEN3_OK : q3::set_error(QWEN3_ERR_HIP, hipGetErrorString(e));
}

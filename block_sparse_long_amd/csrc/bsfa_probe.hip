// Sustained bf16 MFMA rate of the device: every wave runs four independent chains of
// v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic in the loop), so the time
// of a launch is the matrix cores' own rate at the clock they hold under full load. The
// operands depend on the lane and the accumulators are written out, so nothing is folded away.
#include "bsfa_internal.h"

namespace bsfa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)(lane + e));
    b[e] = (__bf16)(1e-3f * (float)(lane - e));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int t = 0; t < iters; ++t) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_rate(int workgroups, int iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace bsfa

// Calibration kernel for the roofline denominator: the bf16 MFMA rate this
// chip sustains in a loop with no memory traffic, measured beside the
// vendor's dense peak.  Not part of the attention method.
//
// Each wave runs four independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 (32768 flops each) on register operands, so the
// matrix cores never wait on a dependence or on memory; eight waves per
// workgroup and four workgroups per compute unit.
#include "basa_common.h"
#include "basa_internal.h"

namespace basa {

namespace {

__global__ void __launch_bounds__(512) mfma_rate_kernel(float* sink, int iters, float seed) {
  bf16x8 a0, a1, a2, a3, b;
  const float t = (float)threadIdx.x * 1e-3f + seed;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a0[j] = (__bf16)(t + j);
    a1[j] = (__bf16)(2.0f * t + j);
    a2[j] = (__bf16)(3.0f * t + j);
    a3[j] = (__bf16)(4.0f * t + j);
    b[j] = (__bf16)(0.5f * j - t);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  // one store per workgroup keeps the chains live without measurable traffic
  if (s == 12345.678f || threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

int launch_mfma_rate(float* sink, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(512), 0, stream, sink, iters, 0.25f);
  return hipGetLastError() == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

}  // namespace basa

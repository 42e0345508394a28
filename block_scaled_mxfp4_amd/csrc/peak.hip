// The matrix cores' sustained rate for the block-scaled MFMA of the w4a8
// GEMMs (v_mfma_scale_f32_16x16x128_f8f6f4, E2M1 x E4M3, 65536 flops per
// instruction): a measured reference for their roofline beside the published
// FP8 peak.  Each wave keeps 8 independent accumulators on register operands
// and issues `iters` rounds of 8 MFMAs; 4 waves per SIMD keep every matrix
// core's issue slots full.  The operands are small finite codes derived from
// the thread index, so nothing folds at compile time.
#include "common.hpp"
#include "internal.hpp"

namespace situ {

// External linkage, so that the compiler cannot prove the store below dead.
__device__ float g_peak_sink;

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters) {
  const uint32_t t = threadIdx.x * 2654435761u + blockIdx.x;
  uint32_t a[4], b[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = (t >> i) & 0x33333333u;   // E2M1 codes of magnitude <= 1.5
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (t >> i) & 0x33333333u;   // E4M3 codes of small magnitude
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = mfma_scale_fp4_fp8(a, b, 127u, 127u, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  // a store no input reaches (the sum is finite), which keeps the MFMAs
  if (s != s) g_peak_sink = s;
}

hipError_t launch_mfma_peak(int iters, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, s, iters);
  return hipGetLastError();
}

}  // namespace situ

// Top-k weighted combine into the shard's partial output.
//
// out[t, :] = sum over slots s = 0..k-1 whose pair is local, in slot order,
// of weight[t, s] * y[inv[t*k + s], :], accumulated in fp32 (the golden
// skeleton's `out += weight * (h @ w2.T)` in the review of
// test_kimi_k3_situ_moe.py, pull request 17865).  A token with no local slot
// gets an exact zero row ("TokenSpeed SiTU", "Supported contract": the
// output is a partial sum the caller all-reduces, so nothing is
// renormalized).  One workgroup per token, four columns per lane.
#include "common.hpp"
#include "internal.hpp"

namespace situ {

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  for (int64_t t = blockIdx.x; t < a.T; t += gridDim.x) {
    const int32_t* inv = a.inv + t * a.k;
    for (int c = threadIdx.x * 4; c < a.H; c += blockDim.x * 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < a.k; ++s) {
        const int p = inv[s];
        if (p < 0) continue;
        const uint32_t wb = a.packed ? ((uint32_t)a.packed[t * a.k + s] >> 16) : a.weights[t * a.k + s];
        const float wgt = bf16_to_f32(wb);
        const f32x4 yv = *reinterpret_cast<const f32x4*>(a.y + (int64_t)p * a.H + c);
        acc[0] = __builtin_fmaf(wgt, yv[0], acc[0]);
        acc[1] = __builtin_fmaf(wgt, yv[1], acc[1]);
        acc[2] = __builtin_fmaf(wgt, yv[2], acc[2]);
        acc[3] = __builtin_fmaf(wgt, yv[3], acc[3]);
      }
      if (a.out_bf16) {
        const uint32_t lo = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + t * a.H + c) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + t * a.H + c) = acc;
      }
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t grid = a.T < 65536 ? a.T : 65536;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace situ

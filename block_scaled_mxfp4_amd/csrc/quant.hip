// Per-token MXFP8 quantization of bf16 activations (the w4a8 FC1 input).
//
// "TokenSpeed SiTU", "Supported contract": w4a8 takes MXFP8 activations with
// a per-token block-scale tensor.  Rule (OCP MX v1.0, conversion to MX):
// per row and per 32 consecutive columns, scale code = floor(log2(amax)) - 8
// + 127 clamped to [0, 254]; each element is the E4M3 round-to-nearest-even
// of x / 2^(code - 127), saturating to +-448.
//
// Layout: four consecutive lanes share one 32-element block, each lane
// loading 8 bf16 (16 bytes), so a wave covers 512 contiguous bytes of a row;
// the block max is combined across the four lanes with two shuffles.
#include "common.hpp"
#include "internal.hpp"

namespace situ {

__global__ __launch_bounds__(256) void quant_mxfp8_kernel(QuantArgs a) {
  const int64_t n8 = a.rows * (int64_t)(a.cols / 8);
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool in = c < n8;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (in) v = reinterpret_cast<const uint4*>(a.x)[c];
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  if (!in) return;
  const uint32_t code = e8m0_code_for_e4m3(amax);
  const int sh = 127 - (int)code;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= e4m3_encode(__builtin_ldexpf(f[i], sh)) << (8 * i);
    hi |= e4m3_encode(__builtin_ldexpf(f[4 + i], sh)) << (8 * i);
  }
  reinterpret_cast<uint2*>(a.codes)[c] = make_uint2(lo, hi);
  if ((c & 3) == 0) a.scales[c >> 2] = (uint8_t)code;
}

hipError_t launch_quant_mxfp8(const QuantArgs& a, hipStream_t s) {
  const int64_t n8 = a.rows * (int64_t)(a.cols / 8);
  if (n8 == 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(quant_mxfp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace situ

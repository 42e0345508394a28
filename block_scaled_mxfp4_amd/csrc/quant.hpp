// The per-token MXFP8 quantization of bf16 activations, one 8-element piece
// per thread, shared by the quantize kernel and the routing launch that
// quantizes beside the router (quant.hip, route.hip).
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
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace situ {

// Piece c (elements 8c .. 8c + 7 of the row-major matrix).  Every lane of
// the wave calls it (the shuffles need all four lanes of a block), with c
// consecutive across lanes from a multiple of 4; pieces past the matrix
// write nothing.
__device__ __forceinline__ void quant_mxfp8_piece(const QuantArgs& a, int64_t c) {
  const bool in = c < quant_pieces(a);
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

}  // namespace situ

// Device helpers shared by the gfx950 kernels of the MXFP4 + SiTU MoE layer.
//
// Formats (OCP Microscaling Formats v1.0, "Scale data type" and "Element
// data types"): E2M1 elements packed two per byte with the low nibble the
// even element; E8M0 scales 2^(c-127); E4M3 (FN) elements with bias 7,
// max 448; bf16 is the upper half of an IEEE binary32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace situ {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round a float to the nearest bf16, ties to even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// E8M0 scale code of an MXFP8 (E4M3) block from the block's |max|:
// floor(log2(amax)) - 8 + 127, clamped at 0 (an all-zero or tiny block).
// The exponent field of a float is floor(log2) + 127 for normal values, and
// every block with a subnormal amax clamps to 0 as well.
__device__ __forceinline__ uint32_t e8m0_code_for_e4m3(float amax) {
  int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
  int c = ef - 8;
  return (uint32_t)(c < 0 ? 0 : c);
}

// E4M3 code of v (finite, already divided by the block scale), nearest
// value with ties to even, saturating to +-448; -0 and values that round
// to zero give +0.  Exact: every step below is exact in binary32.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of step 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);    // 0..8; 8 is the smallest normal, code 0x08
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;   // -6..8
    float m = __builtin_ldexpf(a, 3 - e);                     // [8, 16)
    uint32_t q = (uint32_t)__builtin_rintf(m);                // 8..16
    if (q == 16u) { q = 8u; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | (q - 8u);
  }
  return code == 0u ? 0u : (code | sign);
}

// 2^(c-127) as a float for an E8M0 code c in [1, 254]; c = 0 gives 2^-127
// (a binary32 subnormal) and is built exactly as well.
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  return c == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(c << 23);
}

// Eight E2M1 values (one dword, low nibble first) times 2^(c-127) as eight
// bf16 in four dwords (element 2i in the low half of dword i).  The scaled
// convert multiplies each E2M1 value by the float scale; the product is
// exact in bf16 for every scale code the layer's weights carry.
__device__ __forceinline__ void fp4x8_to_bf16x8(uint32_t w, float scale, uint32_t out[4]) {
  bf16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  out[0] = __builtin_bit_cast(uint32_t, r0);
  out[1] = __builtin_bit_cast(uint32_t, r1);
  out[2] = __builtin_bit_cast(uint32_t, r2);
  out[3] = __builtin_bit_cast(uint32_t, r3);
}

// Eight E2M1 values (one dword, low nibble first) times an arbitrary fp32
// scale s as eight bf16 in four dwords.  The scaled convert applies only the
// exponent of its scale operand (measured on gfx950: a scale of 0.7 acts as
// 0.5), so an NVFP4 block's E4M3 scale is applied by a multiply: E2M1 values
// have at most two significant bits and E4M3 values four, so every product
// is exact in fp32 and in bf16, whose upper halves are kept.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fp4x8_to_bf16x8_mul(uint32_t w, float s, uint32_t out[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x2 v;
    switch (i) {
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
    out[i] = __builtin_amdgcn_perm(__float_as_uint(v.y * s), __float_as_uint(v.x * s), 0x07060302u);
  }
}

// Value of an E4M3 code (OCP FN variant: bias 7, 0x7F / 0xFF NaN) by the hardware decode.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) { return __builtin_amdgcn_cvt_f32_fp8((int)code, 0); }

// One lane's 32 E2M1 weights of a K block (16 bytes) as 16 dwords of bf16:
// MXFP4 with the block's E8M0 code in s, or (NV) NVFP4 with the two E4M3
// scales of its 16-element halves in the two low bytes of s.
template <bool NV>
__device__ __forceinline__ void dequant_w4a16(const uint4& w, uint32_t s, uint32_t wb[16]) {
  if constexpr (NV) {
    const float s0 = e4m3_to_f32(s & 0xffu), s1 = e4m3_to_f32((s >> 8) & 0xffu);
    fp4x8_to_bf16x8_mul(w.x, s0, wb + 0);
    fp4x8_to_bf16x8_mul(w.y, s0, wb + 4);
    fp4x8_to_bf16x8_mul(w.z, s1, wb + 8);
    fp4x8_to_bf16x8_mul(w.w, s1, wb + 12);
  } else {
    const float sc = e8m0_to_f32(s);
    fp4x8_to_bf16x8(w.x, sc, wb + 0);
    fp4x8_to_bf16x8(w.y, sc, wb + 4);
    fp4x8_to_bf16x8(w.z, sc, wb + 8);
    fp4x8_to_bf16x8(w.w, sc, wb + 12);
  }
}

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l holds A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16];
// the result D[4*(l/16) + i][l%16] sits in element i of lane l.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const uint32_t a[4], const uint32_t b[4], f32x4 c) {
  bf16x8 av = __builtin_bit_cast(bf16x8, i32x4{(int)a[0], (int)a[1], (int)a[2], (int)a[3]});
  bf16x8 bv = __builtin_bit_cast(bf16x8, i32x4{(int)b[0], (int)b[1], (int)b[2], (int)b[3]});
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

// D(16x16) += (A * 2^sa) (16x128, E2M1) * (B * 2^sb) (128x16, E4M3), fp32 accumulate.
// Operand layouts, measured on gfx950 with one-hot operands and scales:
//  - A (E2M1, 4 dwords): lane l holds row l%16, K = 32*(l/16) + e for nibble
//    e = 0..31, low nibble first;
//  - B (E4M3, 8 dwords): lane l holds column l%16, K = 16*(l/16) + e in bytes
//    e = 0..15 and K = 64 + 16*(l/16) + (e - 16) in bytes e = 16..31;
//  - the E8M0 scale of lane l applies, for both operands, to the K block
//    32*(l/16) .. +31 of its row (A) or column (B).
__device__ __forceinline__ f32x4 mfma_scale_fp4_fp8(const uint32_t a[4], const uint32_t b[8], uint32_t sa,
                                                     uint32_t sb, f32x4 c) {
  i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], (int)b[4], (int)b[5], (int)b[6], (int)b[7]};
  // format codes: 4 = FP4 E2M1 (A), 0 = FP8 E4M3 (B)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 0, 0, (int)sa, 0, (int)sb);
}

// tanh(x) as a quotient n / d of fp32 values: x clamped to [-9, 9] (tanh(9)
// is 1 in fp32), n = x P(x^2), d = Q(x^2) with P, Q of degree 4, fitted on
// [0, 9] for the smallest largest relative error (reweighted least squares
// on the linearized residual x P - tanh(x) Q): 3.5e-7 relative when evaluated
// in fp32 by Horner's rule.  All coefficients are positive, so d >= 1.
__device__ __forceinline__ void tanh_nd(float x, float& n, float& d) {
  const float c = __builtin_amdgcn_fmed3f(x, -9.0f, 9.0f);
  const float s = c * c;
  float p = 1.3419761e-08f, q = 7.80470088e-07f;
  p = fmaf(p, s, 2.06612074e-05f); q = fmaf(q, s, 0.000329103255f);
  p = fmaf(p, s, 0.00349899239f);  q = fmaf(q, s, 0.0258901921f);
  p = fmaf(p, s, 0.133839771f);    q = fmaf(q, s, 0.467172986f);
  p = fmaf(p, s, 1.0f);            q = fmaf(q, s, 1.0f);
  n = c * p;
  d = q;
}

// SiTU(g, u) = [b*tanh(g/b)*sigmoid(g)] * [lb*tanh(u/lb)] of the alpha-scaled
// accumulators g = ag*acc_g, u = au*acc_u, in fp32.  The per-expert constants
// fold alpha, 1/beta and log2(e) into one multiplier per use, and the two
// tanh quotients and sigmoid = 1 / (1 + e^-g) share a single reciprocal (one
// exponential and one reciprocal per element).  situ_q leaves out the factor
// b*lb (applied by situ_h, or folded into the MXFP8 block scale).  Relative
// error below ~4e-6 over every input range (host emulation of these fp32
// steps against float64: under 1e-6 for inputs of unit scale, 3.8e-6 at scale
// 30-100, where the rounding of the exponent's argument dominates): h feeds a
// rounding point (bf16, or MXFP8 whose E4M3 steps are 6-12 % apart), and an h
// this close to the exact value flips a rounding decision only for elements
// within ~2^-18 of a rounding boundary.  For g below about -76 the
// denominator overflows and h is 0 (the exact value is below 1e-33).
struct SituK {
  float kg, ke, ku, blb;   // ag/b, -ag*log2(e), au/lb, b*lb
};
__device__ __forceinline__ SituK situ_consts(float ag, float au, float b, float lb) {
  constexpr float kL2e = 1.44269502162933349609375f;     // log2(e) rounded to fp32
  return SituK{ag * (1.0f / b), -(ag * kL2e), au * (1.0f / lb), b * lb};
}
__device__ __forceinline__ float situ_q(float acc_g, float acc_u, const SituK& k) {
  float n1, d1, n3, d3;
  tanh_nd(acc_g * k.kg, n1, d1);
  tanh_nd(acc_u * k.ku, n3, d3);
  const float e = __builtin_amdgcn_exp2f(acc_g * k.ke);   // e^-g (hardware 2^y, ~1 ulp)
  const float t = d1 * d3;
  return (n1 * n3) * __builtin_amdgcn_rcpf(__builtin_fmaf(t, e, t));
}
__device__ __forceinline__ float situ_h(float acc_g, float acc_u, const SituK& k) {
  return situ_q(acc_g, acc_u, k) * k.blb;
}

// The gated activation of the FC1 epilogues, h = q * blb with q = act_q:
//  kind 0, SiTU: as situ_q above (blb = b*lb);
//  kind 1, SwiGLU, g * sigmoid(g) * u, the fused SwiGLU the pages compare SiTU
//          against (pull request 17865, review of test_kimi_k3_situ_moe.py);
//  kind 2, SwigluBias, g * sigmoid(g * sa) * (u + sb) with per-expert sa, sb
//          (CUTLASS SwigluBias, the same review's _swiglu_bias_act);
// for kinds 1 and 2, q = (kg*x_g) * (ku*x_u + kb) / (1 + 2^(ke*x_g)) with one
// exponential and one reciprocal, blb = 1.  The inputs x_g, x_u are the
// accumulators (alpha folded into the constants; a LoRA delta enters divided
// by alpha).
enum : int { kActSitu = 0, kActSwiglu = 1, kActSwigluBias = 2 };
struct ActK {
  int kind;
  SituK s;       // SiTU
  float kg, ke, ku, kb;
};
__device__ __forceinline__ ActK act_consts(int kind, float ag, float au, float p0, float p1) {
  constexpr float kL2e = 1.44269502162933349609375f;
  ActK k;
  k.kind = kind;
  if (kind == kActSitu) {
    k.s = situ_consts(ag, au, p0, p1);
    k.kg = k.ke = k.ku = k.kb = 0.0f;
  } else {
    const float sa = kind == kActSwigluBias ? p0 : 1.0f;
    k.s = SituK{0.0f, 0.0f, 0.0f, 1.0f};
    k.kg = ag;
    k.ke = -(sa * ag * kL2e);
    k.ku = au;
    k.kb = kind == kActSwigluBias ? p1 : 0.0f;
  }
  return k;
}
__device__ __forceinline__ float act_blb(const ActK& k) { return k.s.blb; }
__device__ __forceinline__ float act_q(float xg, float xu, const ActK& k) {
  if (k.kind == kActSitu) return situ_q(xg, xu, k.s);
  const float e = __builtin_amdgcn_exp2f(xg * k.ke);
  return (xg * k.kg) * __builtin_fmaf(xu, k.ku, k.kb) * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float act_h(float xg, float xu, const ActK& k) { return act_q(xg, xu, k) * k.s.blb; }

// Per-expert activation constants of one FC1 work item and its LoRA mode:
// `lora` set when a delta is added (the inputs are then acc + d / alpha, with
// rag = 1 / alpha_g and rau = 1 / alpha_u).
struct ActItem {
  ActK k;
  float ag, au, rag, rau;
  bool lora;
};

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

}  // namespace situ

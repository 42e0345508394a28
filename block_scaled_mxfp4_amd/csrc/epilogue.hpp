// FC1 epilogue pieces shared by the grouped-GEMM kernels: the per-expert
// activation constants of a work item, the LoRA delta of one lane's columns
// and the bf16 rows handed to the down LoRA.
//
// The LoRA bridges follow the decomposed MoE-LoRA op of the xorl-wheels
// release notes ("Changes since 875b7d7"): a gate_up LoRA delta is added to
// the FC1 output before the activation, the activation's output is handed
// back as the down LoRA's input, and with no bridges the op is the plain
// pipeline.  The delta is in the layer's real-valued domain, so it is added
// after the alpha scaling: g = alpha_g * acc_g + d_g, u = alpha_u * acc_u + d_u.
// The activation constants fold alpha in (act_consts), so the delta enters
// as acc_g + d_g / alpha_g; a zero delta element leaves the accumulator
// untouched, so an all-zero delta gives the plain pipeline bit for bit (the
// release notes' zero-B adapters equal to the base output).  With a delta,
// alpha_gate and alpha_up must be nonzero.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace situ {

// Activation constants of expert l (scalar loads of the per-expert arrays).
__device__ __forceinline__ ActItem act_item(const GemmArgs& a, int l) {
  typedef const int32_t __attribute__((address_space(4)))* cp;
  ActItem it;
  it.ag = a.alpha_g ? __builtin_bit_cast(float, ((cp)a.alpha_g)[l]) : 1.0f;
  it.au = a.alpha_u ? __builtin_bit_cast(float, ((cp)a.alpha_u)[l]) : 1.0f;
  const float p0 = a.beta ? __builtin_bit_cast(float, ((cp)a.beta)[l]) : 0.0f;
  const float p1 = a.lbeta ? __builtin_bit_cast(float, ((cp)a.lbeta)[l]) : 0.0f;
  it.lora = a.lora_delta != nullptr;
  it.k = act_consts(a.act_kind, it.ag, it.au, p0, p1);
  it.rag = 1.0f / it.ag;
  it.rau = 1.0f / it.au;
  return it;
}

// SiTU constants of expert l for the plain epilogue (no LoRA bridges).
__device__ __forceinline__ SituK situ_item(const GemmArgs& a, int l) {
  typedef const int32_t __attribute__((address_space(4)))* cp;
  const float ag = a.alpha_g ? __builtin_bit_cast(float, ((cp)a.alpha_g)[l]) : 1.0f;
  const float au = a.alpha_u ? __builtin_bit_cast(float, ((cp)a.alpha_u)[l]) : 1.0f;
  return situ_consts(ag, au, __builtin_bit_cast(float, ((cp)a.beta)[l]), __builtin_bit_cast(float, ((cp)a.lbeta)[l]));
}

// A pair's LoRA delta at four gate columns and the matching four up columns
// (I further), as bf16 bits.
struct DeltaPiece {
  uint2 g, u;
};
__device__ __forceinline__ DeltaPiece load_delta(const uint16_t* drow, int I) {
  return DeltaPiece{*reinterpret_cast<const uint2*>(drow), *reinterpret_cast<const uint2*>(drow + I)};
}

// The activation inputs of four gate/up column pairs: the accumulators, plus
// with a LoRA delta the delta piece divided by alpha.
__device__ __forceinline__ void act_inputs_of(const ActItem& it, const DeltaPiece& d, const float ag4[4],
                                              const float au4[4], float xg[4], float xu[4]) {
  if (it.lora) {
    const float dg[4] = {bf16_to_f32(d.g.x & 0xffffu), bf16_to_f32(d.g.x >> 16), bf16_to_f32(d.g.y & 0xffffu),
                         bf16_to_f32(d.g.y >> 16)};
    const float du[4] = {bf16_to_f32(d.u.x & 0xffffu), bf16_to_f32(d.u.x >> 16), bf16_to_f32(d.u.y & 0xffffu),
                         bf16_to_f32(d.u.y >> 16)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xg[e] = dg[e] != 0.0f ? __builtin_fmaf(dg[e], it.rag, ag4[e]) : ag4[e];
      xu[e] = du[e] != 0.0f ? __builtin_fmaf(du[e], it.rau, au4[e]) : au4[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xg[e] = ag4[e];
      xu[e] = au4[e];
    }
  }
}

// The same with the delta read here (drow = the pair's delta row at the first
// gate column).
__device__ __forceinline__ void act_inputs(const ActItem& it, const uint16_t* drow, int I, const float ag4[4],
                                           const float au4[4], float xg[4], float xu[4]) {
  act_inputs_of(it, it.lora ? load_delta(drow, I) : DeltaPiece{}, ag4, au4, xg, xu);
}

// E4M3 code (one byte of `codes`, hardware decode, exact) times 2^(sc - 127), as bf16 bits.
__device__ __forceinline__ uint32_t e4m3_scaled_bf16(uint32_t codes, int byte, int sc) {
  float v;
  switch (byte) {
    case 0: v = __builtin_amdgcn_cvt_f32_fp8((int)codes, 0); break;
    case 1: v = __builtin_amdgcn_cvt_f32_fp8((int)codes, 1); break;
    case 2: v = __builtin_amdgcn_cvt_f32_fp8((int)codes, 2); break;
    default: v = __builtin_amdgcn_cvt_f32_fp8((int)codes, 3); break;
  }
  return f32_to_bf16_rne(__builtin_ldexpf(v, sc - 127));
}

// Four E4M3 codes (one dword) under scale code sc as four bf16 (two dwords).
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t codes, int sc) {
  return make_uint2(e4m3_scaled_bf16(codes, 0, sc) | (e4m3_scaled_bf16(codes, 1, sc) << 16),
                    e4m3_scaled_bf16(codes, 2, sc) | (e4m3_scaled_bf16(codes, 3, sc) << 16));
}

}  // namespace situ

#include "../../include/situ_moe.h"
static_assert(situ::kActSitu == SITU_ACTIVATION_SITU && situ::kActSwiglu == SITU_ACTIVATION_SWIGLU &&
                  situ::kActSwigluBias == SITU_ACTIVATION_SWIGLU_BIAS,
              "the planner passes the ABI's activation values as the kernels' kinds");

// Grouped GEMMs of the routed MoE layer on gfx950 matrix cores.
//
// FC1: for every local expert l and every pair p of its group,
//   acc[p, n] = sum_k x[t(p), k] * W1[l, n, k]          n < 2I (gate rows, then up rows)
//   h[p, n]   = SiTU(alpha_g[l] * acc[p, n], alpha_u[l] * acc[p, I + n])   n < I
// with the SiTU of the golden reference in the review of
// test_kimi_k3_situ_moe.py (TensorRT-LLM pull request 17865) and the alpha
// rescale of the up half from the xorl-wheels release notes ("Changes since
// 875b7d7").  h is stored bf16 (w4a16) or as MXFP8 per 32 along I (w4a8;
// "TokenSpeed SiTU", "Activation precision": the FC1 fp8 output is
// dequantized before FC2).
// FC2: y[p, n] = sum_i h[p, i] * W2[l, n, i], n < H, stored fp32.
//
// Mapping.  The weights sit on the 16-row side of each MFMA and the tokens
// on the 16-column side ("swap-AB"): the weight stream is the large operand
// in every configuration of this layer, and a decode group holds only a few
// rows.  Lane l of a wave owns weight row l%16 of each 16-row tile and token
// l%16 of each 16-token tile, and the weight K block 32*(l/16) of every
// 128-wide K step, which is exactly one E8M0 scale block per lane: a lane
// reads 16 contiguous bytes of its weight row and one scale byte per step.
// (E4M3 activations follow the block-scaled MFMA's own split K layout: two
// 16-byte pieces per lane, 64 apart.)
//   w4a16: the 32 E2M1 values are converted to bf16 with their scale by the
//          gfx950 scaled convert, then fed to four 16x16x32 bf16 MFMAs.
//   w4a8:  one 16x16x128 block-scaled MFMA takes the E2M1 weights and the
//          E4M3 activations with both E8M0 scales directly.
// K need not be a multiple of 128 (H = 3584 is 28 steps, I = 64 half a
// step): lanes whose K block lies past the end feed zeros.
//
// Scheduling.  A persistent grid walks work items (m-tile, column tile); the
// m-tiles and their experts come from the router's tile list on the device,
// so no group size is ever read back to the host.
#include "common.hpp"
#include "internal.hpp"

namespace situ {

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <bool FP8, int TOKT>
__global__ __launch_bounds__(kGemmThreads) void fc1_kernel(GemmArgs a) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int I = a.N, K = a.K;
  const int nkb = K / 32, steps = (nkb + 3) / 4;
  const int units = I / kFc1ColsPerWave;
  const int n_wgn = (units + 3) / 4;
  const int total = a.mtiles[a.E_l] * n_wgn;
  const int64_t xrow_bytes = FP8 ? (int64_t)K : (int64_t)K * 2;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int mt = w / n_wgn;
    const int unit = (w % n_wgn) * 4 + wave;
    if (unit >= units) continue;
    const int l = a.tile_expert[mt];
    const int p0 = a.offsets[l] + (mt - a.mtiles[l]) * (16 * TOKT);
    const int p1 = min(a.offsets[l + 1], p0 + 16 * TOKT);
    const int n0 = unit * kFc1ColsPerWave;

    const uint8_t* xrow[TOKT];
    const uint8_t* xsrow[TOKT];
    bool valid[TOKT];
#pragma unroll
    for (int tt = 0; tt < TOKT; ++tt) {
      const int p = p0 + 16 * tt + r;
      valid[tt] = p < p1;
      const int64_t t = valid[tt] ? (int64_t)(a.perm[p] / a.top_k) : 0;
      xrow[tt] = static_cast<const uint8_t*>(a.act) + t * xrow_bytes;
      xsrow[tt] = FP8 ? a.act_scale + t * nkb : nullptr;
    }
    const uint8_t* wrow[4];
    const uint8_t* srow[4];
    {
      const int64_t ebase = (int64_t)l * (2 * I);
      const int rows[4] = {n0 + r, n0 + 16 + r, I + n0 + r, I + n0 + 16 + r};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wrow[q] = a.w + (ebase + rows[q]) * (int64_t)(K / 2);
        srow[q] = a.ws + (ebase + rows[q]) * (int64_t)nkb;
      }
    }

    f32x4 acc[4][TOKT];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int tt = 0; tt < TOKT; ++tt) acc[q][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j < steps; ++j) {
      const int kb = 4 * j + g;
      const bool kin = kb < nkb;
      uint4 wv[4];
      uint32_t sv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wv[q] = kin ? ld16(wrow[q] + kb * 16) : make_uint4(0, 0, 0, 0);
        sv[q] = kin ? srow[q][kb] : 127u;
      }
      if constexpr (!FP8) {
        uint4 xv[TOKT][4];
#pragma unroll
        for (int tt = 0; tt < TOKT; ++tt)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            xv[tt][c] = (kin && valid[tt]) ? ld16(xrow[tt] + kb * 64 + 16 * c) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sc = e8m0_to_f32(sv[q]);
          uint32_t wb[16];
          fp4x8_to_bf16x8(wv[q].x, sc, wb + 0);
          fp4x8_to_bf16x8(wv[q].y, sc, wb + 4);
          fp4x8_to_bf16x8(wv[q].z, sc, wb + 8);
          fp4x8_to_bf16x8(wv[q].w, sc, wb + 12);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int tt = 0; tt < TOKT; ++tt) {
              const uint32_t b[4] = {xv[tt][qq].x, xv[tt][qq].y, xv[tt][qq].z, xv[tt][qq].w};
              acc[q][tt] = mfma_bf16_16x16x32(wb + 4 * qq, b, acc[q][tt]);
            }
        }
      } else {
        // E4M3 operand: this lane's bytes 0..15 are K 128j + 16g .. +15 (block 4j + g/2),
        // bytes 16..31 are K 128j + 64 + 16g .. +15 (block 4j + 2 + g/2); see mfma_scale_fp4_fp8
        const int kb_lo = 4 * j + (g >> 1);
        const int kb_hi = 4 * j + 2 + (g >> 1);
        uint32_t xv[TOKT][8];
        uint32_t xs[TOKT];
#pragma unroll
        for (int tt = 0; tt < TOKT; ++tt) {
          const bool ok = kin && valid[tt];
          const uint4 v0 = (valid[tt] && kb_lo < nkb) ? ld16(xrow[tt] + 128 * j + 16 * g) : make_uint4(0, 0, 0, 0);
          const uint4 v1 = (valid[tt] && kb_hi < nkb) ? ld16(xrow[tt] + 128 * j + 64 + 16 * g) : make_uint4(0, 0, 0, 0);
          xv[tt][0] = v0.x; xv[tt][1] = v0.y; xv[tt][2] = v0.z; xv[tt][3] = v0.w;
          xv[tt][4] = v1.x; xv[tt][5] = v1.y; xv[tt][6] = v1.z; xv[tt][7] = v1.w;
          xs[tt] = ok ? xsrow[tt][kb] : 127u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t av[4] = {wv[q].x, wv[q].y, wv[q].z, wv[q].w};
#pragma unroll
          for (int tt = 0; tt < TOKT; ++tt) acc[q][tt] = mfma_scale_fp4_fp8(av, xv[tt], sv[q], xs[tt], acc[q][tt]);
        }
      }
    }

    // epilogue: alpha, SiTU, rounding point R1, store h in perm order
    const float ag = a.alpha_g ? a.alpha_g[l] : 1.0f;
    const float au = a.alpha_u ? a.alpha_u[l] : 1.0f;
    const float b = a.beta[l], lb = a.lbeta[l];
    const float inv_b = 1.0f / b, inv_lb = 1.0f / lb;
#pragma unroll
    for (int tt = 0; tt < TOKT; ++tt) {
      const int64_t p = p0 + 16 * tt + r;
      float hv[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hv[half][i] = situ_act(ag * acc[half][tt][i], au * acc[2 + half][tt][i], b, lb, inv_b, inv_lb);
      if constexpr (!FP8) {
        if (valid[tt]) {
          uint16_t* hrow = static_cast<uint16_t*>(a.out) + p * I + n0 + 4 * g;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t lo = f32_to_bf16_rne(hv[half][0]) | (f32_to_bf16_rne(hv[half][1]) << 16);
            const uint32_t hi = f32_to_bf16_rne(hv[half][2]) | (f32_to_bf16_rne(hv[half][3]) << 16);
            *reinterpret_cast<uint2*>(hrow + 16 * half) = make_uint2(lo, hi);
          }
        }
      } else {
        float amax = 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(hv[half][i]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        if (valid[tt]) {
          const uint32_t code = e8m0_code_for_e4m3(amax);
          const int sh = 127 - (int)code;
          uint8_t* hrow = static_cast<uint8_t*>(a.out) + p * I + n0 + 4 * g;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            uint32_t packed = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) packed |= e4m3_encode(__builtin_ldexpf(hv[half][i], sh)) << (8 * i);
            *reinterpret_cast<uint32_t*>(hrow + 16 * half) = packed;
          }
          if (g == 0) a.out_scale[p * (I / 32) + n0 / 32] = (uint8_t)code;
        }
      }
    }
  }
}

template <bool FP8, int TOKT>
__global__ __launch_bounds__(kGemmThreads) void fc2_kernel(GemmArgs a) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.N, K = a.K;
  const int nkb = K / 32, steps = (nkb + 3) / 4;
  const int wg_rows = 4 * kFc2RowsPerWave;
  const int n_wgn = (H + wg_rows - 1) / wg_rows;
  const int total = a.mtiles[a.E_l] * n_wgn;
  const int64_t hrow_bytes = FP8 ? (int64_t)K : (int64_t)K * 2;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int mt = w / n_wgn;
    const int n0 = (w % n_wgn) * wg_rows + wave * kFc2RowsPerWave;
    if (n0 >= H) continue;
    const int l = a.tile_expert[mt];
    const int p0 = a.offsets[l] + (mt - a.mtiles[l]) * (16 * TOKT);
    const int p1 = min(a.offsets[l + 1], p0 + 16 * TOKT);
    const int ntiles = min(4, (H - n0) / 16);

    const uint8_t* hrow[TOKT];
    const uint8_t* hsrow[TOKT];
    bool valid[TOKT];
#pragma unroll
    for (int tt = 0; tt < TOKT; ++tt) {
      const int64_t p = p0 + 16 * tt + r;
      valid[tt] = p < p1;
      const int64_t pp = valid[tt] ? p : 0;
      hrow[tt] = static_cast<const uint8_t*>(a.act) + pp * hrow_bytes;
      hsrow[tt] = FP8 ? a.act_scale + pp * nkb : nullptr;
    }
    const uint8_t* wrow[4];
    const uint8_t* srow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = (int64_t)l * H + min(n0 + 16 * q + r, H - 1);
      wrow[q] = a.w + row * (int64_t)(K / 2);
      srow[q] = a.ws + row * (int64_t)nkb;
    }

    f32x4 acc[4][TOKT];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int tt = 0; tt < TOKT; ++tt) acc[q][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j < steps; ++j) {
      const int kb = 4 * j + g;
      const bool kin = kb < nkb;
      uint4 wv[4];
      uint32_t sv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = kin && q < ntiles;
        wv[q] = ok ? ld16(wrow[q] + kb * 16) : make_uint4(0, 0, 0, 0);
        sv[q] = ok ? srow[q][kb] : 127u;
      }
      if constexpr (!FP8) {
        uint4 xv[TOKT][4];
#pragma unroll
        for (int tt = 0; tt < TOKT; ++tt)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            xv[tt][c] = (kin && valid[tt]) ? ld16(hrow[tt] + kb * 64 + 16 * c) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sc = e8m0_to_f32(sv[q]);
          uint32_t wb[16];
          fp4x8_to_bf16x8(wv[q].x, sc, wb + 0);
          fp4x8_to_bf16x8(wv[q].y, sc, wb + 4);
          fp4x8_to_bf16x8(wv[q].z, sc, wb + 8);
          fp4x8_to_bf16x8(wv[q].w, sc, wb + 12);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int tt = 0; tt < TOKT; ++tt) {
              const uint32_t bb[4] = {xv[tt][qq].x, xv[tt][qq].y, xv[tt][qq].z, xv[tt][qq].w};
              acc[q][tt] = mfma_bf16_16x16x32(wb + 4 * qq, bb, acc[q][tt]);
            }
        }
      } else {
        // E4M3 operand: this lane's bytes 0..15 are K 128j + 16g .. +15 (block 4j + g/2),
        // bytes 16..31 are K 128j + 64 + 16g .. +15 (block 4j + 2 + g/2); see mfma_scale_fp4_fp8
        const int kb_lo = 4 * j + (g >> 1);
        const int kb_hi = 4 * j + 2 + (g >> 1);
        uint32_t xv[TOKT][8];
        uint32_t xs[TOKT];
#pragma unroll
        for (int tt = 0; tt < TOKT; ++tt) {
          const bool ok = kin && valid[tt];
          const uint4 v0 = (valid[tt] && kb_lo < nkb) ? ld16(hrow[tt] + 128 * j + 16 * g) : make_uint4(0, 0, 0, 0);
          const uint4 v1 = (valid[tt] && kb_hi < nkb) ? ld16(hrow[tt] + 128 * j + 64 + 16 * g) : make_uint4(0, 0, 0, 0);
          xv[tt][0] = v0.x; xv[tt][1] = v0.y; xv[tt][2] = v0.z; xv[tt][3] = v0.w;
          xv[tt][4] = v1.x; xv[tt][5] = v1.y; xv[tt][6] = v1.z; xv[tt][7] = v1.w;
          xs[tt] = ok ? hsrow[tt][kb] : 127u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t av[4] = {wv[q].x, wv[q].y, wv[q].z, wv[q].w};
#pragma unroll
          for (int tt = 0; tt < TOKT; ++tt) acc[q][tt] = mfma_scale_fp4_fp8(av, xv[tt], sv[q], xs[tt], acc[q][tt]);
        }
      }
    }

#pragma unroll
    for (int tt = 0; tt < TOKT; ++tt) {
      if (!valid[tt]) continue;
      const int64_t p = p0 + 16 * tt + r;
      float* yrow = static_cast<float*>(a.out) + p * H + n0 + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < ntiles) *reinterpret_cast<f32x4*>(yrow + 16 * q) = acc[q][tt];
    }
  }
}

hipError_t launch_fc1(int tactic, const GemmArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (tactic) {
    case FC1_W4A16_M16: hipLaunchKernelGGL((fc1_kernel<false, 1>), dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    case FC1_W4A16_M64: hipLaunchKernelGGL((fc1_kernel<false, 4>), dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    case FC1_W4A8_M16: hipLaunchKernelGGL((fc1_kernel<true, 1>), dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    case FC1_W4A8_M64: hipLaunchKernelGGL((fc1_kernel<true, 4>), dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fc2(int tactic, const GemmArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (tactic) {
    case FC2_W4A16_M16: hipLaunchKernelGGL((fc2_kernel<false, 1>), dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    case FC2_W4A16_M64: hipLaunchKernelGGL((fc2_kernel<false, 4>), dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    case FC2_W4A8_M16: hipLaunchKernelGGL((fc2_kernel<true, 1>), dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    case FC2_W4A8_M64: hipLaunchKernelGGL((fc2_kernel<true, 4>), dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace situ

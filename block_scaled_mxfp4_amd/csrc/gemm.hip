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
#include <map>
#include <mutex>
#include <tuple>

#include "common.hpp"
#include "dma.hpp"
#include "epilogue.hpp"
#include "internal.hpp"

namespace situ {

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <bool FP8, int TOKT, bool NV = false, bool GEN = false>
__global__ __launch_bounds__(kGemmThreads) void fc1_kernel(GemmArgs a) {
  static_assert(!(NV && FP8), "NVFP4 weights are served with bf16 activations");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int I = a.N, K = a.K;
  const int nkb = K / 32, steps = (nkb + 3) / 4;
  const int sbr = NV ? 2 * nkb : nkb;   // scale bytes per weight row
  // weights in rows of K / 2 bytes, or fragment-tiled (MXFP4 only)
  const bool tiled = !NV && a.tiled;
  const int wstep = tiled ? 1024 : 64, sstep = tiled ? 64 : 4;   // bytes between K steps
  const int units = I / kFc1ColsPerWave;
  const int n_wgn = (units + 3) / 4;
  const int total = ((cptr)a.mtiles)[a.E_l] * n_wgn;
  const int64_t xrow_bytes = FP8 ? (int64_t)K : (int64_t)K * 2;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int mt = w / n_wgn;
    const int unit = (w % n_wgn) * 4 + wave;
    if (unit >= units) continue;
    const int l = ((cptr)a.tile_expert)[mt];
    const int p0 = ((cptr)a.offsets)[l] + (mt - ((cptr)a.mtiles)[l]) * (16 * TOKT);
    const int p1 = min(((cptr)a.offsets)[l + 1], p0 + 16 * TOKT);
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
    // this lane's 16 weight bytes and scale byte of each tile at K step 0
    const uint8_t* wrow[4];
    const uint8_t* srow[4];
    {
      const int tiles[4] = {n0 / 16, n0 / 16 + 1, (I + n0) / 16, (I + n0) / 16 + 1};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (tiled) {
          const int64_t t = (int64_t)l * (2 * I / 16) + tiles[q];
          wrow[q] = a.w + t * steps * 1024 + lane * 16;
          srow[q] = a.ws + t * steps * 64 + lane;
        } else {
          const int64_t row = (int64_t)l * (2 * I) + 16 * tiles[q] + r;
          wrow[q] = a.w + row * (K / 2) + 16 * g;
          srow[q] = a.ws + row * sbr + (NV ? 2 : 1) * g;
        }
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
        wv[q] = kin ? ld16(wrow[q] + j * wstep) : make_uint4(0, 0, 0, 0);
        // NVFP4: the two E4M3 scales of this 32-K block in one 16-bit load
        sv[q] = NV ? (kin ? (uint32_t)*reinterpret_cast<const uint16_t*>(srow[q] + 8 * j) : 0x3838u)
                   : (kin ? (uint32_t)srow[q][j * sstep] : 127u);
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
          uint32_t wb[16];
          dequant_w4a16<NV>(wv[q], sv[q], wb);
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

    // epilogue: alpha (and a LoRA delta), the activation, rounding point R1,
    // store h in perm order (and by expanded index for the down LoRA)
    ActItem ai{};
    SituK sk{};
    if constexpr (GEN) ai = act_item(a, l);
    else sk = situ_item(a, l);
#pragma unroll
    for (int tt = 0; tt < TOKT; ++tt) {
      const int64_t p = p0 + 16 * tt + r;
      const int64_t j = (GEN && valid[tt] && (ai.lora || a.lora_out)) ? (int64_t)a.perm[p] : 0;
      float hv[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if constexpr (GEN) {
          float xg[4], xu[4];
          const float ag4[4] = {acc[half][tt][0], acc[half][tt][1], acc[half][tt][2], acc[half][tt][3]};
          const float au4[4] = {acc[2 + half][tt][0], acc[2 + half][tt][1], acc[2 + half][tt][2],
                                acc[2 + half][tt][3]};
          act_inputs(ai, a.lora_delta + j * (2 * I) + n0 + 16 * half + 4 * g, I, ag4, au4, xg, xu);
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[half][i] = act_h(xg[i], xu[i], ai.k);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[half][i] = situ_h(acc[half][tt][i], acc[2 + half][tt][i], sk);
        }
      }
      if constexpr (!FP8) {
        if (valid[tt]) {
          uint16_t* hrow = static_cast<uint16_t*>(a.out) + p * I + n0 + 4 * g;
          uint16_t* lrow = (GEN && a.lora_out) ? a.lora_out + j * I + n0 + 4 * g : nullptr;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t lo = f32_to_bf16_rne(hv[half][0]) | (f32_to_bf16_rne(hv[half][1]) << 16);
            const uint32_t hi = f32_to_bf16_rne(hv[half][2]) | (f32_to_bf16_rne(hv[half][3]) << 16);
            *reinterpret_cast<uint2*>(hrow + 16 * half) = make_uint2(lo, hi);
            if (lrow) *reinterpret_cast<uint2*>(lrow + 16 * half) = make_uint2(lo, hi);
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
          uint16_t* lrow = (GEN && a.lora_out) ? a.lora_out + j * I + n0 + 4 * g : nullptr;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            uint32_t packed = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) packed |= e4m3_encode(__builtin_ldexpf(hv[half][i], sh)) << (8 * i);
            *reinterpret_cast<uint32_t*>(hrow + 16 * half) = packed;
            if (lrow) *reinterpret_cast<uint2*>(lrow + 16 * half) = e4m3x4_to_bf16x4(packed, (int)code);
          }
          if (g == 0) a.out_scale[p * (I / 32) + n0 / 32] = (uint8_t)code;
        }
      }
    }
  }
}

template <bool FP8, int TOKT, bool NV = false>
__global__ __launch_bounds__(kGemmThreads) void fc2_kernel(GemmArgs a) {
  static_assert(!(NV && FP8), "NVFP4 weights are served with bf16 activations");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int H = a.N, K = a.K;
  const int nkb = K / 32, steps = (nkb + 3) / 4;
  const int sbr = NV ? 2 * nkb : nkb;   // scale bytes per weight row
  const bool tiled = !NV && a.tiled;
  const int wstep = tiled ? 1024 : 64, sstep = tiled ? 64 : 4;   // bytes between K steps
  const int wg_rows = 4 * kFc2RowsPerWave;
  const int n_wgn = (H + wg_rows - 1) / wg_rows;
  const int total = ((cptr)a.mtiles)[a.E_l] * n_wgn;
  const int64_t hrow_bytes = FP8 ? (int64_t)K : (int64_t)K * 2;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int mt = w / n_wgn;
    const int n0 = (w % n_wgn) * wg_rows + wave * kFc2RowsPerWave;
    if (n0 >= H) continue;
    const int l = ((cptr)a.tile_expert)[mt];
    const int p0 = ((cptr)a.offsets)[l] + (mt - ((cptr)a.mtiles)[l]) * (16 * TOKT);
    const int p1 = min(((cptr)a.offsets)[l + 1], p0 + 16 * TOKT);
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
    // this lane's 16 weight bytes and scale byte of each tile at K step 0
    // (tiles past H are clamped; their loads are skipped)
    const uint8_t* wrow[4];
    const uint8_t* srow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tile = min(n0 / 16 + q, H / 16 - 1);
      if (tiled) {
        const int64_t t = (int64_t)l * (H / 16) + tile;
        wrow[q] = a.w + t * steps * 1024 + lane * 16;
        srow[q] = a.ws + t * steps * 64 + lane;
      } else {
        const int64_t row = (int64_t)l * H + 16 * tile + r;
        wrow[q] = a.w + row * (int64_t)(K / 2) + 16 * g;
        srow[q] = a.ws + row * (int64_t)sbr + (NV ? 2 : 1) * g;
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
        const bool ok = kin && q < ntiles;
        wv[q] = ok ? ld16(wrow[q] + j * wstep) : make_uint4(0, 0, 0, 0);
        sv[q] = NV ? (ok ? (uint32_t)*reinterpret_cast<const uint16_t*>(srow[q] + 8 * j) : 0x3838u)
                   : (ok ? (uint32_t)srow[q][j * sstep] : 127u);
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
          uint32_t wb[16];
          dequant_w4a16<NV>(wv[q], sv[q], wb);
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

// ---------------------------------------------------------------------------
// Decode-shaped variant (16-row m-tiles).  A group holds one to ten rows, so
// the kernel is a weight stream and is tuned for the bytes it keeps in
// flight and the requests it makes:
//  - the waves of a workgroup split the K steps of one unit by interleaving
//    them (wave ks takes steps ks, ks + KSPLIT, ...): a step reads 64 bytes
//    of each weight row, and sibling waves then request the two halves of a
//    128-byte line together, so they meet before the L2.  With contiguous
//    ranges a wave read the halves a step apart and the L2 had evicted 16 %
//    of the lines before their second half (TP8 decode FC1: 13.8 M L2
//    requests and 8.1 M misses, interleaved 9.4 M and 7.2 M; FC1 -4 %);
//  - each wave keeps the weights of its next kDecodeDepth steps in flight
//    while it converts and multiplies the current one (a ring of register
//    buffers, rotated by unrolling);
//  - the unit's E8M0 scales (its rows are contiguous in the scale tensor)
//    are staged in LDS once per work item with 16-byte loads; one byte per
//    lane per tile per step straight from memory costs a request each and
//    measured ~30 % of the achievable stream rate;
//  - the activation pieces are requested ahead of their use (loading them
//    just in time stalled every step on its latency): w4a8 carries them in
//    the weights' ring, w4a16 one step ahead in a ring of their own, from
//    LDS when its m-tile is small enough to be staged there, else from L2,
//    so that its weights can run further ahead;
//  - partial sums meet in LDS in a fixed order (bitwise reproducible).
// FC1 units are 32 gate + 32 up rows; FC2 units are 64 output rows.
//
// Loads go through buffer resources: 32-bit offsets from a per-expert (or
// per-tensor) base, and an offset past the resource's size reads zeros, which
// masks K tails, missing tokens and rows past H without per-dword selects.

constexpr uint32_t kOob = 0x80000000u;   // an offset past every resource: reads 0

// K steps in flight per wave, and the occupancy the register budget
// targets (waves per SIMD): four for the w4a16 FC1 kernel with K split in
// two or not at all, whose ring fits 128 registers (TP8 decode FC1 -1 %, EP8
// -1.5 %), three elsewhere (FC2's deeper weight ring needs a few more, and a
// four-way split's partial sums would spill).
constexpr int kDecodeDepth = 1;
__host__ __device__ constexpr int decode_waves(bool fp8, bool fc1, int ksplit) {
  return (!fp8 && fc1 && ksplit <= 2) ? 4 : 3;
}
// w4a16 weight steps in flight (the activation pieces stay one step ahead):
// two for FC2 with its K split (EP8 decode FC2 -3 %), one elsewhere (the
// unsplit three-step FC2 of TP8 decode measured 2 % slower with two, FC1 no
// faster).
constexpr int kDecodeWDepthFc1 = 1;
constexpr int kDecodeWDepthFc2Split = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// voff carries the per-lane offset (kOob masks the lane); soff is a
// wave-uniform offset added to it (a tile's row delta), only ever used for
// rows that exist, so the range check never depends on it.
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  // soff is wave-uniform by contract; readfirstlane keeps it in an SGPR (a
  // value the compiler cannot prove uniform would make it loop over lanes)
  v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, __builtin_amdgcn_readfirstlane((int)soff), 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

struct DecodeGeo {
  __amdgpu_buffer_rsrc_t wr, xr, xsr;
  uint32_t w_row;          // byte offset of this lane's 16 bytes of tile 0 at K step 0 in the expert's weights
  uint32_t w_step;         // bytes between K steps: 64 (rows of K / 2 bytes) or 1024 (fragment-tiled)
  uint32_t w_delta[4];     // tile q relative to tile 0, in weight bytes (uniform)
  const uint8_t* s_lds;    // this unit's staged scales: 4 tiles x 16 sbr bytes
  uint32_t s_lane;         // this lane's scale byte of step 0 in a staged tile
  uint32_t s_step;         // bytes between K steps there: 4 (rows of sbr bytes) or 64 (tiled)
  uint32_t x_row;          // byte offset of this lane's activation row (kOob if none)
  uint32_t xs_row;
  const uint8_t* x_lds;    // w4a16: the m-tile's activation rows staged in LDS, or null
  uint32_t x_lds_off;      // this lane's row in them (bytes)
  int nkb, sbr, g, r, ntiles;   // sbr: staged scale bytes per weight row (scale_row_bytes)
};

// One K step's operands for a wave: four 16-row weight tiles (16 bytes of
// E2M1 per lane each) and the activation piece of this lane's token.
template <bool FP8>
struct Step {
  uint4 w[4];
  uint4 x[FP8 ? 2 : 4];
  uint32_t xs;
};

// w4a16 with the activation rows staged in LDS (d.x_lds set): this lane's
// piece of step j from there, zero past the group or past K.
__device__ __forceinline__ void load_x_lds(uint4 x[4], const DecodeGeo& d, int j) {
  const int kb = 4 * j + d.g;
  const bool ok = kb < d.nkb && d.x_row != kOob;
  const uint8_t* src = d.x_lds + (ok ? d.x_lds_off + (uint32_t)kb * 64u : 0u);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + 16 * c);
    x[c] = ok ? v : make_uint4(0, 0, 0, 0);
  }
}

// The four weight tiles' pieces of step j (zero past K).
__device__ __forceinline__ void load_w(uint4 w[4], const DecodeGeo& d, int j) {
  const int kb = 4 * j + d.g;
  const uint32_t wo = kb < d.nkb ? d.w_row + (uint32_t)j * d.w_step : kOob;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = q < d.ntiles ? bload16(d.wr, wo, d.w_delta[q]) : make_uint4(0, 0, 0, 0);   // q < ntiles: uniform
}

// w4a16: the activation pieces of step j from memory (zero past the group or
// past K).  A lane computes with K block g of its token's 256-byte step
// (64 bytes, four 16-byte pieces), but the four lanes of a token load
// request c together as the token's bytes 64 c .. 64 c + 63, so that each
// request touches one 64-byte piece of a cache line per token instead of
// four pieces spread over two lines (the address unit's cost is per line,
// and from memory these loads were as many lookups as the weights);
// x_transpose then gives each lane its own block.
__device__ __forceinline__ void load_x_mem(uint4 x[4], const DecodeGeo& d, int j) {
  const uint32_t base = d.x_row != kOob ? d.x_row + 256u * (uint32_t)j + 16u * (uint32_t)d.g : kOob;
#pragma unroll
  for (int c = 0; c < 4; ++c) x[c] = bload16(d.xr, (base != kOob && 4 * j + c < d.nkb) ? base + 64u * c : kOob);
}

// After load_x_mem, lane group g (lanes 16 g .. 16 g + 15) holds piece g of
// block c in x[c]; this turns it into piece c of block g (a 4 x 4 transpose
// between the register index and the lane group, per 32-bit word): swap the
// upper half of x[0] (x[1]) with the lower half of x[2] (x[3]), then the odd
// lane groups of x[0] (x[2]) with the even ones of x[1] (x[3]).
__device__ __forceinline__ void x_transpose(uint4 x[4]) {
  uint32_t w[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    w[c][0] = x[c].x; w[c][1] = x[c].y; w[c][2] = x[c].z; w[c][3] = x[c].w;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const auto s32 = __builtin_amdgcn_permlane32_swap(w[c][e], w[c + 2][e], false, false);
      w[c][e] = s32[0];
      w[c + 2][e] = s32[1];
    }
#pragma unroll
    for (int c = 0; c < 4; c += 2) {
      const auto s16 = __builtin_amdgcn_permlane16_swap(w[c][e], w[c + 1][e], false, false);
      w[c][e] = s16[0];
      w[c + 1][e] = s16[1];
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) x[c] = make_uint4(w[c][0], w[c][1], w[c][2], w[c][3]);
}

// Step j's weights and this lane's activation piece, both from memory.
template <bool FP8>
__device__ __forceinline__ void load_step(Step<FP8>& b, const DecodeGeo& d, int j) {
  const int kb = 4 * j + d.g;
  const bool kin = kb < d.nkb;
  load_w(b.w, d, j);
  if constexpr (!FP8) {
    load_x_mem(b.x, d, j);
    b.xs = 127u;
  } else {
    // E4M3 operand: bytes 0..15 are K 128j + 16g .. +15 (block 4j + g/2), bytes
    // 16..31 are K 128j + 64 + 16g .. +15 (block 4j + 2 + g/2); see mfma_scale_fp4_fp8
    const bool has = d.x_row != kOob;
    const uint32_t lo = (has && 4 * j + (d.g >> 1) < d.nkb) ? d.x_row + 128u * j + 16u * d.g : kOob;
    const uint32_t hi = (has && 4 * j + 2 + (d.g >> 1) < d.nkb) ? d.x_row + 128u * j + 64u + 16u * d.g : kOob;
    b.x[0] = bload16(d.xr, lo);
    b.x[1] = bload16(d.xr, hi);
    b.xs = (has && kin) ? bload8(d.xsr, d.xs_row + (uint32_t)kb) : 127u;
  }
}

// w4a8 step j with the activation rows in LDS (the fused kernel's FC2 reads
// its m-tile's h there: E4M3 [16][K], then the E8M0 scales [16][K / 32]):
// the weights from memory, this lane's pieces and scale from LDS.
__device__ __forceinline__ void load_step_x8_lds(Step<true>& b, const DecodeGeo& d, int j) {
  load_w(b.w, d, j);
  const int kb = 4 * j + d.g;
  const bool has = d.x_row != kOob;
  const bool lo_ok = has && 4 * j + (d.g >> 1) < d.nkb, hi_ok = has && 4 * j + 2 + (d.g >> 1) < d.nkb;
  const uint8_t* row = d.x_lds + d.x_lds_off + 128u * j + 16u * d.g;
  const uint4 lo = *reinterpret_cast<const uint4*>(lo_ok ? row : d.x_lds);
  const uint4 hi = *reinterpret_cast<const uint4*>(hi_ok ? row + 64 : d.x_lds);
  b.x[0] = lo_ok ? lo : make_uint4(0, 0, 0, 0);
  b.x[1] = hi_ok ? hi : make_uint4(0, 0, 0, 0);
  b.xs = (has && kb < d.nkb) ? (uint32_t)d.x_lds[16 * 32 * d.nkb + d.xs_row + kb] : 127u;
}

// w4a16 step j: the weight pieces dequantized to bf16 by their E8M0 scales
// (staged in LDS), times the activation piece.
template <bool NV = false>
__device__ __forceinline__ void compute_w4a16(const uint4 w[4], const uint4 x[4], const DecodeGeo& d, int j,
                                              f32x4 acc[4]) {
  const int kb = 4 * j + d.g;
  const bool kin = kb < d.nkb;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t wb[16];
    if constexpr (NV) {
      // NVFP4: two E4M3 scales per 32 K (one per 16), non powers of two
      const uint8_t* sp = d.s_lds + (16 * q + d.r) * d.sbr + 2 * kb;
      const float s0 = kin ? e4m3_to_f32(sp[0]) : 1.0f;
      const float s1 = kin ? e4m3_to_f32(sp[1]) : 1.0f;
      fp4x8_to_bf16x8_mul(w[q].x, s0, wb + 0);
      fp4x8_to_bf16x8_mul(w[q].y, s0, wb + 4);
      fp4x8_to_bf16x8_mul(w[q].z, s1, wb + 8);
      fp4x8_to_bf16x8_mul(w[q].w, s1, wb + 12);
    } else {
      const float sc = e8m0_to_f32(kin ? (uint32_t)d.s_lds[16 * q * d.sbr + d.s_lane + j * d.s_step] : 127u);
      fp4x8_to_bf16x8(w[q].x, sc, wb + 0);
      fp4x8_to_bf16x8(w[q].y, sc, wb + 4);
      fp4x8_to_bf16x8(w[q].z, sc, wb + 8);
      fp4x8_to_bf16x8(w[q].w, sc, wb + 12);
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint32_t xb[4] = {x[qq].x, x[qq].y, x[qq].z, x[qq].w};
      acc[q] = mfma_bf16_16x16x32(wb + 4 * qq, xb, acc[q]);
    }
  }
}

template <bool FP8>
__device__ __forceinline__ void compute_step(const Step<FP8>& b, const DecodeGeo& d, int j, f32x4 acc[4]) {
  if constexpr (!FP8) {
    compute_w4a16(b.w, b.x, d, j, acc);
  } else {
    const int kb = 4 * j + d.g;
    const bool kin = kb < d.nkb;
    const uint32_t xb[8] = {b.x[0].x, b.x[0].y, b.x[0].z, b.x[0].w, b.x[1].x, b.x[1].y, b.x[1].z, b.x[1].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t av[4] = {b.w[q].x, b.w[q].y, b.w[q].z, b.w[q].w};
      const uint32_t sv = kin ? (uint32_t)d.s_lds[16 * q * d.sbr + d.s_lane + j * d.s_step] : 127u;
      acc[q] = mfma_scale_fp4_fp8(av, xb, sv, b.xs, acc[q]);
    }
  }
}

// Dynamic LDS of a decode launch: staged scales of the workgroup's units,
// then one region that holds the staged activation rows during the K loop
// and the split-K partial sums after it.
__host__ __device__ constexpr uint32_t decode_lds_scales(int units_per_wg, int sbr) {
  return (uint32_t)(units_per_wg * 64 * sbr + 15) / 16u * 16u;
}
// split-K partial sums: one 4-tile set per wave that is not its unit's lead
__host__ __device__ constexpr uint32_t decode_lds_red(int ksplit) {
  return ksplit > 1 ? (uint32_t)((4 / ksplit) * (ksplit - 1)) * 4u * kWave * 16u : 0u;
}
// w4a16: an m-tile of at most decode_x_rows() tokens has its activation rows
// staged in LDS once per work item; its pieces then travel in the register
// ring from LDS instead of every wave loading its lanes' pieces (mostly past
// the group: decode m-tiles hold one or two tokens) from memory beside the
// weights each step (TP8 decode FC1 -2..5 %, FC2 -6 %).  The rows get what is
// left of the LDS share of one of the decode_waves() workgroups of a CU after
// the scales, 16 at most (FC1 at H = 3584: three rows, FC2 at I = 384: 16).
__host__ __device__ constexpr int decode_x_rows(int ksplit, int sbr, int K, bool fp8, bool fc1) {
  const uint32_t budget = 160u * 1024u / (uint32_t)decode_waves(fp8, fc1, ksplit) - 512u;
  const uint32_t used = decode_lds_scales(4 / ksplit, sbr);
  const uint32_t left = budget > used ? budget - used : 0u;
  const int rows = (int)(left / ((uint32_t)K * 2u));
  return fp8 ? 0 : (rows < 16 ? rows : 16);
}
__host__ __device__ constexpr uint32_t decode_lds_x(bool fp8, bool fc1, int ksplit, int K, int sbr) {
  return (uint32_t)decode_x_rows(ksplit, sbr, K, fp8, fc1) * (uint32_t)K * 2u;
}
__host__ __device__ constexpr uint32_t decode_lds_bytes(int ksplit, int sbr, uint32_t x_bytes) {
  return decode_lds_scales(4 / ksplit, sbr) + (x_bytes > decode_lds_red(ksplit) ? x_bytes : decode_lds_red(ksplit));
}

// Decode epilogue of one wave's 16-row group: FC1 applies alpha and SiTU and
// rounds h (bf16, or MXFP8 with one E8M0 scale per 32 columns); FC2 writes
// fp32 y.  acc[q] holds weight tile q x the group's 16 tokens; this lane owns
// token p (valid: inside the group) and rows 4g..4g+3 of each tile.
// Per-expert parameters come through scalar loads.
// FUSED (FC1 of the fused decode kernel): h goes to the m-tile's rows in LDS
// at hb (bf16 [16][I], or E4M3 [16][I] then the E8M0 scales [16][I / 32])
// instead of to memory; row p - p0.
template <bool FP8, bool FC1, bool GEN, bool FUSED = false>
__device__ __forceinline__ void decode_epilogue(const GemmArgs& a, const f32x4 acc[4], int l, int p, bool valid,
                                                int n0, int g, int ntiles, uint8_t* hb = nullptr, int p0 = 0) {
  if constexpr (FC1) {
    const int I = a.N;
    float hv[2][4];
    int64_t j = 0;
    if constexpr (GEN) {
      const ActItem ai = act_item(a, l);
      // the pair's expanded index: the row of its LoRA delta and down-LoRA input
      j = (valid && (ai.lora || a.lora_out)) ? (int64_t)a.perm[p] : 0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float xg[4], xu[4];
        const float ag4[4] = {acc[half][0], acc[half][1], acc[half][2], acc[half][3]};
        const float au4[4] = {acc[2 + half][0], acc[2 + half][1], acc[2 + half][2], acc[2 + half][3]};
        act_inputs(ai, a.lora_delta + j * (2 * I) + n0 + 16 * half + 4 * g, I, ag4, au4, xg, xu);
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[half][i] = act_h(xg[i], xu[i], ai.k);
      }
    } else {   // SiTU without LoRA bridges
      const SituK sk = situ_item(a, l);
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[half][i] = situ_h(acc[half][i], acc[2 + half][i], sk);
    }
    if constexpr (!FP8) {
      if (valid) {
        uint16_t* hrow = FUSED ? reinterpret_cast<uint16_t*>(hb) + (p - p0) * I + n0 + 4 * g
                               : static_cast<uint16_t*>(a.out) + (int64_t)p * I + n0 + 4 * g;
        uint16_t* lrow = (GEN && a.lora_out) ? a.lora_out + j * I + n0 + 4 * g : nullptr;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t lo = f32_to_bf16_rne(hv[half][0]) | (f32_to_bf16_rne(hv[half][1]) << 16);
          const uint32_t hi = f32_to_bf16_rne(hv[half][2]) | (f32_to_bf16_rne(hv[half][3]) << 16);
          *reinterpret_cast<uint2*>(hrow + 16 * half) = make_uint2(lo, hi);
          if (lrow) *reinterpret_cast<uint2*>(lrow + 16 * half) = make_uint2(lo, hi);
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
      if (valid) {
        const uint32_t code = e8m0_code_for_e4m3(amax);
        const int sh = 127 - (int)code;
        uint8_t* hrow = FUSED ? hb + (p - p0) * I + n0 + 4 * g : static_cast<uint8_t*>(a.out) + (int64_t)p * I + n0 + 4 * g;
        uint16_t* lrow = (GEN && a.lora_out) ? a.lora_out + j * I + n0 + 4 * g : nullptr;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t packed = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) packed |= e4m3_encode(__builtin_ldexpf(hv[half][i], sh)) << (8 * i);
          *reinterpret_cast<uint32_t*>(hrow + 16 * half) = packed;
          if (lrow) *reinterpret_cast<uint2*>(lrow + 16 * half) = e4m3x4_to_bf16x4(packed, (int)code);
        }
        if (g == 0) {
          if (FUSED) hb[16 * I + (p - p0) * (I / 32) + n0 / 32] = (uint8_t)code;
          else a.out_scale[(int64_t)p * (I / 32) + n0 / 32] = (uint8_t)code;
        }
      }
    }
  } else {
    if (valid) {
      float* yrow = static_cast<float*>(a.out) + (int64_t)p * a.N + n0 + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < ntiles) *reinterpret_cast<f32x4*>(yrow + 16 * q) = acc[q];
    }
  }
}

// One work item of a decode GEMM: the workgroup's UNITS_PER_WG units (weight
// row groups) starting at unit0 for m-tile mt.  FUSED: a pass of the fused
// decode kernel, whose m-tile rows of h live in LDS at hb: FC1 writes them
// there (and stages no activation rows), FC2 reads them there.
// TL: the weights are fragment-tiled (a compile-time choice: runtime strides
// cost the decode kernels a few dozen more scalar registers, spilled).
template <bool FP8, bool FC1, int KSPLIT, bool NV, bool GEN, bool FUSED, bool TL>
__device__ __forceinline__ void decode_pass(const GemmArgs& a, uint8_t* lds, int mt, int unit0, uint8_t* hb) {
  static_assert(!(NV && FP8), "NVFP4 weights are served with bf16 activations");
  static_assert(!(FUSED && NV), "the fused decode kernel takes MXFP4 weights");
  static_assert(!(NV && TL), "NVFP4 weights are row-major");
  constexpr int UNITS_PER_WG = 4 / KSPLIT;
  // wave-uniform values are made visibly uniform (readfirstlane, scalar
  // loads of the routing tables) so buffer resources stay in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const cptr tile_expert = (cptr)a.tile_expert, offsets = (cptr)a.offsets, mtiles = (cptr)a.mtiles;
  const int r = lane & 15, g = lane >> 4;
  const int ks = wave % KSPLIT;
  const int uw = wave / KSPLIT;
  const int K = a.K, nkb = K / 32, steps = (nkb + 3) / 4;
  constexpr bool tiled = TL;
  const int sbr = NV ? 2 * nkb : (tiled ? 4 * steps : nkb);   // staged scale bytes per weight row
  const int units = FC1 ? a.N / kFc1ColsPerWave : (a.N + kFc2RowsPerWave - 1) / kFc2RowsPerWave;
  const uint32_t arow_bytes = FP8 ? (uint32_t)K : (uint32_t)K * 2u;
  const int n_rows = FC1 ? 2 * a.N : a.N;          // weight rows per expert
  // this wave's K steps: every KSPLIT-th step from ks (interleaved)
  const int my_steps = steps > ks ? (steps - ks + KSPLIT - 1) / KSPLIT : 0;
  auto jstep = [&](int s) { return ks + KSPLIT * s; };
  // the activation rows during the K loop, then the split-K partial sums
  uint8_t* const x_stage = lds + decode_lds_scales(UNITS_PER_WG, sbr);
  f32x4* red = reinterpret_cast<f32x4*>(x_stage);
  constexpr bool XL = !FP8;                    // w4a16 may stage its activation rows
  constexpr int DW = FC1 ? kDecodeWDepthFc1 : (KSPLIT > 1 ? kDecodeWDepthFc2Split : 1);

  const int unit = unit0 + uw;
  const bool active = unit < units;  // uniform per wave; idle waves still meet the barriers
  const int l = tile_expert[mt];
  const int p0 = offsets[l] + (mt - mtiles[l]) * 16;
  const int p1 = min(offsets[l + 1], p0 + 16);
  const int p = p0 + r;
  const bool valid = p < p1;

  // stage the scales of the workgroup's units in LDS (16-byte loads); the
  // scales of 16 consecutive rows are 16 sbr contiguous bytes in either layout
  {
    const size_t sexp = (size_t)n_rows * sbr;
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.ws + (size_t)l * sexp, (uint32_t)sexp);
    const int chunks_per_unit = 4 * sbr;       // 64 rows x sbr bytes / 16
    for (int c = threadIdx.x; c < UNITS_PER_WG * chunks_per_unit; c += kGemmThreads) {
      const int u = c / chunks_per_unit, cc = c % chunks_per_unit;
      uint32_t src;
      if constexpr (FC1) {
        const int half = cc / (2 * sbr), within = cc % (2 * sbr);
        const int row = (half ? a.N : 0) + (unit0 + u) * kFc1ColsPerWave;
        src = (unit0 + u < units) ? (uint32_t)row * sbr + 16u * within : kOob;
      } else {
        src = (uint32_t)(unit0 + u) * kFc2RowsPerWave * sbr + 16u * cc;   // rows past H read 0
      }
      *reinterpret_cast<uint4*>(lds + (size_t)u * 64 * sbr + 16 * cc) = bload16(sr, src);
    }
  }
  // w4a16 with few tokens: stage the m-tile's activation rows (16-byte loads);
  // the fused FC2 finds its rows (h) in LDS already, the fused FC1 reads x from memory
  const bool x_in_lds = FUSED ? !FC1 : p1 - p0 <= decode_x_rows(KSPLIT, sbr, K, FP8, FC1);   // uniform
  if constexpr (XL && !FUSED) {
    if (x_in_lds) {
      const int row_chunks = K / 8;               // K bf16 values / 16 bytes
      // FC1 rows x[perm[p] / k]; FC2 rows h[p], addressed from the m-tile's first
      const __amdgpu_buffer_rsrc_t xr =
          FC1 ? make_rsrc(a.act, 0x7fffffff)
              : make_rsrc(static_cast<const uint8_t*>(a.act) + (size_t)p0 * arow_bytes, 16u * arow_bytes);
      for (int c = threadIdx.x; c < (p1 - p0) * row_chunks; c += kGemmThreads) {
        const int i = c / row_chunks, cc = c % row_chunks;
        const uint32_t row = FC1 ? (uint32_t)(a.perm[p0 + i] / a.top_k) : (uint32_t)i;
        *reinterpret_cast<uint4*>(x_stage + (size_t)i * K * 2 + 16 * cc) = bload16(xr, row * arow_bytes + 16u * cc);
      }
    }
  }

  f32x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

  DecodeGeo d;
  int n0 = 0, ntiles = 4;
  if (active) {
    const size_t wexp = expert_w_bytes(tiled, n_rows, K);
    d.wr = make_rsrc(a.w + (size_t)l * wexp, (uint32_t)wexp);
    d.nkb = nkb;
    d.sbr = sbr;
    d.g = g;
    d.r = r;
    uint32_t dr[4];
    if constexpr (FC1) {
      n0 = unit * kFc1ColsPerWave;
      dr[0] = 0; dr[1] = 16; dr[2] = a.N; dr[3] = a.N + 16;
    } else {
      n0 = unit * kFc2RowsPerWave;
      ntiles = min(4, (a.N - n0) / 16);
      dr[0] = 0; dr[1] = 16; dr[2] = 32; dr[3] = 48;
    }
    d.ntiles = ntiles;
    if constexpr (tiled) {
      const uint32_t tile_bytes = (uint32_t)steps * 1024u;   // a 16-row tile over all of K
#pragma unroll
      for (int q = 0; q < 4; ++q) d.w_delta[q] = dr[q] / 16u * tile_bytes;
      d.w_row = (uint32_t)(n0 / 16) * tile_bytes + (uint32_t)lane * 16u;
      d.w_step = 1024u;
      d.s_lane = (uint32_t)lane;
      d.s_step = 64u;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) d.w_delta[q] = dr[q] * (uint32_t)(K / 2);
      d.w_row = (uint32_t)(n0 + r) * (uint32_t)(K / 2) + 16u * (uint32_t)g;
      d.w_step = 64u;
      d.s_lane = (uint32_t)(r * sbr + g);
      d.s_step = 4u;
    }
    d.s_lds = lds + (size_t)uw * 64 * sbr;
    d.x_lds = x_in_lds ? (FUSED ? hb : x_stage) : nullptr;
    d.x_lds_off = valid ? (uint32_t)r * arow_bytes : 0u;
    if constexpr (FC1) {
      const uint32_t t = valid ? (uint32_t)(a.perm[p] / a.top_k) : 0u;
      d.xr = make_rsrc(a.act, 0x7fffffff);
      d.x_row = valid ? t * arow_bytes : kOob;
      d.xsr = make_rsrc(FP8 ? a.act_scale : a.act, 0x7fffffff);
      d.xs_row = t * (uint32_t)nkb;
    } else {
      d.xr = make_rsrc(static_cast<const uint8_t*>(a.act) + (size_t)p0 * arow_bytes, 16u * arow_bytes);
      d.x_row = valid ? (uint32_t)r * arow_bytes : kOob;
      d.xsr = make_rsrc(FP8 ? a.act_scale + (size_t)p0 * nkb : static_cast<const uint8_t*>(a.act),
                        16u * (uint32_t)nkb);
      d.xs_row = (uint32_t)r * (uint32_t)nkb;
      if constexpr (FUSED && FP8) d.x_lds = hb;
    }
  }
  if constexpr (XL) {
    // w4a16: weights DW steps ahead in a ring of DW + 1 register sets (the
    // first DW requested before the staging barrier), the activation piece
    // of the next step in a ring of two, read during the current step from
    // LDS (staged m-tile) or from memory; NU steps per pass keep both ring
    // indices compile-time constants
    constexpr int NW = DW + 1, NU = NW % 2 == 0 ? NW : 2 * NW;
    Step<FP8> wr[NW], xr[2];           // .w of the one ring, .x of the other
    if (active) {
#pragma unroll
      for (int u = 0; u < DW; ++u)
        if (u < my_steps) load_w(wr[u].w, d, jstep(u));
      if (!x_in_lds && my_steps > 0) load_x_mem(xr[0].x, d, jstep(0));
    }
    __syncthreads();   // staged scales and activation rows visible
    if (active) {
      if (x_in_lds && my_steps > 0) load_x_lds(xr[0].x, d, jstep(0));
#pragma unroll 1
      for (int i = 0; i < my_steps; i += NU) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int s = i + u;
          if (s < my_steps) {
            if (s + DW < my_steps) load_w(wr[(u + DW) % NW].w, d, jstep(s + DW));
            if (s + 1 < my_steps) {
              if (x_in_lds) load_x_lds(xr[(u + 1) % 2].x, d, jstep(s + 1));
              else load_x_mem(xr[(u + 1) % 2].x, d, jstep(s + 1));
            }
            __builtin_amdgcn_sched_barrier(0);
            if (!x_in_lds) x_transpose(xr[u % 2].x);   // uniform
            compute_w4a16<NV>(wr[u % NW].w, xr[u % 2].x, d, jstep(s), acc);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  } else {
    // w4a8: the weights and activation pieces of the next kDecodeDepth
    // steps are in flight while the current one is computed (the first
    // ones requested before the staging barrier); a ring of kDecodeDepth + 1
    // register buffers rotated by unrolling (compile-time indices);
    // sched_barrier(0) keeps each prefetch ahead of its compute
    constexpr int NB = kDecodeDepth + 1;
    Step<FP8> buf[NB];
    if (active) {
#pragma unroll
      for (int u = 0; u < kDecodeDepth; ++u)
        if (u < my_steps) {
          if constexpr (FUSED && FP8 && !FC1) load_step_x8_lds(buf[u], d, jstep(u));
          else load_step<FP8>(buf[u], d, jstep(u));
        }
    }
    __syncthreads();   // staged scales visible
    if (active) {
#pragma unroll 1
      for (int i = 0; i < my_steps; i += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          if (i + u < my_steps) {
            if (i + u + kDecodeDepth < my_steps) {
              if constexpr (FUSED && FP8 && !FC1) load_step_x8_lds(buf[(u + kDecodeDepth) % NB], d, jstep(i + u + kDecodeDepth));
              else load_step<FP8>(buf[(u + kDecodeDepth) % NB], d, jstep(i + u + kDecodeDepth));
            }
            __builtin_amdgcn_sched_barrier(0);
            compute_step<FP8>(buf[u], d, jstep(i + u), acc);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  }

  // split-K reduction in a fixed order
  bool lead = active;
  if constexpr (KSPLIT > 1) {
    if (XL && x_in_lds) __syncthreads();   // uniform: every wave is done with the staged rows
    if (active && ks != 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) red[((uw * (KSPLIT - 1) + ks - 1) * 4 + q) * kWave + lane] = acc[q];
    }
    __syncthreads();
    lead = active && ks == 0;
    if (lead) {
#pragma unroll
      for (int s2 = 1; s2 < KSPLIT; ++s2)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += red[((uw * (KSPLIT - 1) + s2 - 1) * 4 + q) * kWave + lane];
    }
  }

  if (lead) decode_epilogue<FP8, FC1, GEN, FUSED && FC1>(a, acc, l, p, valid, n0, g, ntiles, hb, p0);
  __syncthreads();   // staged scales and partial sums are reused by the next work item
}

template <bool FP8, bool FC1, int KSPLIT, bool NV = false, bool GEN = false, bool TL = false>
__global__ __launch_bounds__(kGemmThreads, decode_waves(FP8, FC1, KSPLIT)) void decode_gemm_kernel(GemmArgs a) {
  constexpr int UNITS_PER_WG = 4 / KSPLIT;
  extern __shared__ __align__(16) uint8_t lds[];
  const int units = FC1 ? a.N / kFc1ColsPerWave : (a.N + kFc2RowsPerWave - 1) / kFc2RowsPerWave;
  const int n_wgn = (units + UNITS_PER_WG - 1) / UNITS_PER_WG;
  const int total = ((cptr)a.mtiles)[a.E_l] * n_wgn;
  for (int w = blockIdx.x; w < total; w += gridDim.x)
    decode_pass<FP8, FC1, KSPLIT, NV, GEN, false, TL>(a, lds, w / n_wgn, (w % n_wgn) * UNITS_PER_WG, nullptr);
}

// K split for the decode kernels: long K loops are shared by the four waves.
static int decode_ksplit(int K) {
  const int steps = (K / 32 + 3) / 4;
  const int m = 8;   // steps per wave below which K is not split further
  return steps >= 4 * m ? 4 : (steps >= 2 * m ? 2 : 1);
}

// Resident workgroups per CU of a kernel (from its register and LDS use),
// queried once per kernel; a persistent grid is sized to what fits.
using GemmKernel = void (*)(GemmArgs);

int resident_per_cu(const void* kernel, int threads, uint32_t lds_bytes) {
  // queried once per (kernel, block size, dynamic LDS size), under a lock:
  // launches may come from several host threads at once
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, uint32_t>, int> cache;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_tuple(kernel, threads, lds_bytes);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds_bytes) != hipSuccess || n < 1) n = 1;
  cache.emplace(key, n);
  return n;
}

template <GemmKernel KERNEL>
static hipError_t launch_persistent(const GemmArgs& a, int64_t work, int cus, hipStream_t s, uint32_t lds_bytes = 0) {
  const int per_cu = resident_per_cu(reinterpret_cast<const void*>(KERNEL), kGemmThreads, lds_bytes);
  const int64_t cap = (int64_t)cus * per_cu;
  const int grid = (int)(work < cap ? work : cap);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(KERNEL, dim3(grid), dim3(kGemmThreads), lds_bytes, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused decode (the MegaMoE idea of PR 17865, one kernel for both GEMMs, on
// this library's decode kernels): a workgroup takes one 16-row m-tile through
// all of FC1 and then all of FC2, and the m-tile's rows of h never leave the
// CU: FC1's epilogue writes them (bf16, or E4M3 with their E8M0 scales) to
// LDS, and FC2 reads its activation pieces there.  One launch instead of two,
// no h round trip through memory, and a CU that finishes its FC1 share goes
// on to FC2 without waiting for the rest of the grid.  The passes are the
// unfused kernels' work items (same K split, reduction order and epilogue),
// so the output equals the unfused path's bit for bit.  Offered where h of
// one m-tile is small (I <= 768: at most 24 KB of bf16) and FC2's K is not
// split; MXFP4 weights.  Measured slower than the two unfused launches at 64
// tokens x 896 experts (H 3584, I 384: 0.326 against 0.282 ms for both
// GEMMs): its work item is a whole m-tile, about 700 of them for 1024
// workgroup slots, where the unfused kernels cut each expert into six FC1
// and fourteen FC2 items; so it is not the planner's first choice.
struct FusedArgs {
  GemmArgs fc1, fc2;
};

__host__ __device__ constexpr uint32_t fused_h_offset(int ks1, int sbr1, int sbr2) {
  const uint32_t s1 = decode_lds_scales(4 / ks1, sbr1) + decode_lds_red(ks1);
  const uint32_t s2 = decode_lds_scales(4, sbr2);
  return ((s1 > s2 ? s1 : s2) + 15u) / 16u * 16u;
}
__host__ __device__ constexpr uint32_t fused_h_bytes(bool fp8, int I) {
  return fp8 ? 16u * (uint32_t)I + 16u * (uint32_t)(I / 32) : 32u * (uint32_t)I;
}

template <bool FP8, int KS1, bool GEN, bool TL>
__global__ __launch_bounds__(kGemmThreads, 4) void decode_fused_kernel(FusedArgs f) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int I = f.fc1.N, H = f.fc2.N;
  uint8_t* hb = lds + fused_h_offset(KS1, scale_row_bytes(false, f.fc1.tiled, H), scale_row_bytes(false, f.fc2.tiled, I));
  const int units1 = I / kFc1ColsPerWave, units2 = (H + kFc2RowsPerWave - 1) / kFc2RowsPerWave;
  const int total = ((cptr)f.fc1.mtiles)[f.fc1.E_l];
  for (int mt = blockIdx.x; mt < total; mt += gridDim.x) {
    // every pass ends with a workgroup barrier: FC2 starts on complete rows
    // of h, and the next m-tile's FC1 overwrites them only after FC2
    for (int u0 = 0; u0 < units1; u0 += 4 / KS1) decode_pass<FP8, true, KS1, false, GEN, true, TL>(f.fc1, lds, mt, u0, hb);
    for (int u0 = 0; u0 < units2; u0 += 4) decode_pass<FP8, false, 1, false, false, true, TL>(f.fc2, lds, mt, u0, hb);
  }
}

bool fused_decode_ok(int H, int I) {
  return I % kFc1ColsPerWave == 0 && I <= 768 && (I / 32 + 3) / 4 < 16 && H % 32 == 0;
}

template <bool FP8, int KS1, bool GEN, bool TL>
static hipError_t launch_fused_kt(const FusedArgs& f, int max_mtiles, int cus, hipStream_t s) {
  const uint32_t lds = fused_h_offset(KS1, scale_row_bytes(false, TL, f.fc1.K),
                                      scale_row_bytes(false, TL, f.fc2.K)) + fused_h_bytes(FP8, f.fc1.N);
  const int per_cu = resident_per_cu(reinterpret_cast<const void*>(decode_fused_kernel<FP8, KS1, GEN, TL>), kGemmThreads, lds);
  const int64_t cap = (int64_t)cus * per_cu;
  const int grid = (int)(max_mtiles < cap ? max_mtiles : cap);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_fused_kernel<FP8, KS1, GEN, TL>), dim3(grid), dim3(kGemmThreads), lds, s, f);
  return hipGetLastError();
}
template <bool FP8, int KS1, bool GEN>
static hipError_t launch_fused_k(const FusedArgs& f, int max_mtiles, int cus, hipStream_t s) {
  return f.fc1.tiled ? launch_fused_kt<FP8, KS1, GEN, true>(f, max_mtiles, cus, s)
                     : launch_fused_kt<FP8, KS1, GEN, false>(f, max_mtiles, cus, s);
}

template <bool FP8, bool GEN>
static hipError_t launch_fused_g(const FusedArgs& f, int max_mtiles, int cus, hipStream_t s) {
  switch (decode_ksplit(f.fc1.K)) {
    case 4: return launch_fused_k<FP8, 4, GEN>(f, max_mtiles, cus, s);
    case 2: return launch_fused_k<FP8, 2, GEN>(f, max_mtiles, cus, s);
    default: return launch_fused_k<FP8, 1, GEN>(f, max_mtiles, cus, s);
  }
}

hipError_t launch_fused_decode(const GemmArgs& fc1, const GemmArgs& fc2, bool fp8, int max_mtiles, int cus,
                               hipStream_t s) {
  if (fc1.nvfp4 || !fused_decode_ok(fc2.N, fc1.N) || decode_ksplit(fc2.K) != 1) return hipErrorInvalidValue;
  const FusedArgs f{fc1, fc2};
  const bool gen = general_epilogue(fc1);
  if (fp8) return gen ? launch_fused_g<true, true>(f, max_mtiles, cus, s) : launch_fused_g<true, false>(f, max_mtiles, cus, s);
  return gen ? launch_fused_g<false, true>(f, max_mtiles, cus, s) : launch_fused_g<false, false>(f, max_mtiles, cus, s);
}

template <bool FP8, bool FC1, bool NV, bool GEN, bool TL>
hipError_t launch_decode_kt(const GemmArgs& a, int64_t work, int cus, hipStream_t s) {
  const int sbr = scale_row_bytes(NV, TL, a.K);   // staged scale bytes per weight row
  switch (decode_ksplit(a.K)) {
    case 4: return launch_persistent<decode_gemm_kernel<FP8, FC1, 4, NV, GEN, TL>>(a, work, cus, s, decode_lds_bytes(4, sbr, decode_lds_x(FP8, FC1, 4, a.K, sbr)));
    case 2: return launch_persistent<decode_gemm_kernel<FP8, FC1, 2, NV, GEN, TL>>(a, work, cus, s, decode_lds_bytes(2, sbr, decode_lds_x(FP8, FC1, 2, a.K, sbr)));
    default: return launch_persistent<decode_gemm_kernel<FP8, FC1, 1, NV, GEN, TL>>(a, work, cus, s, decode_lds_bytes(1, sbr, decode_lds_x(FP8, FC1, 1, a.K, sbr)));
  }
}
template <bool FP8, bool FC1, bool NV, bool GEN>
hipError_t launch_decode_k(const GemmArgs& a, int64_t work, int cus, hipStream_t s) {
  if constexpr (!NV) {
    if (a.tiled) return launch_decode_kt<FP8, FC1, NV, GEN, true>(a, work, cus, s);
  }
  return launch_decode_kt<FP8, FC1, NV, GEN, false>(a, work, cus, s);
}
template <bool FP8, bool FC1>
hipError_t launch_decode(const GemmArgs& a, int64_t work, int cus, hipStream_t s) {
  const bool gen = FC1 && general_epilogue(a);
  if constexpr (!FP8) {
    if (a.nvfp4) return gen ? launch_decode_k<false, FC1, true, FC1>(a, work, cus, s)
                            : launch_decode_k<false, FC1, true, false>(a, work, cus, s);
  }
  return gen ? launch_decode_k<FP8, FC1, false, FC1>(a, work, cus, s)
             : launch_decode_k<FP8, FC1, false, false>(a, work, cus, s);
}

// Work items of one launch, upper bound: m-tiles x column units per workgroup.
static int64_t work_items(bool fc1, bool decode, const GemmArgs& a, int max_mtiles) {
  int64_t units, per_wg;
  if (fc1) units = a.N / kFc1ColsPerWave;
  else units = (a.N + kFc2RowsPerWave - 1) / kFc2RowsPerWave;
  per_wg = decode ? 4 / decode_ksplit(a.K) : 4;
  return (int64_t)max_mtiles * ((units + per_wg - 1) / per_wg);
}

hipError_t launch_fc1(int tactic, const GemmArgs& a, int max_mtiles, int cus, hipStream_t s) {
  const bool decode = tactic == FC1_W4A16_M16 || tactic == FC1_W4A8_M16;
  const int64_t work = work_items(true, decode, a, max_mtiles);
  switch (tactic) {
    case FC1_W4A16_M16: return launch_decode<false, true>(a, work, cus, s);
    case FC1_W4A16_M64:
      if (general_epilogue(a))
        return a.nvfp4 ? launch_persistent<fc1_kernel<false, 4, true, true>>(a, work, cus, s)
                       : launch_persistent<fc1_kernel<false, 4, false, true>>(a, work, cus, s);
      return a.nvfp4 ? launch_persistent<fc1_kernel<false, 4, true>>(a, work, cus, s)
                     : launch_persistent<fc1_kernel<false, 4>>(a, work, cus, s);
    case FC1_W4A8_M16: return launch_decode<true, true>(a, work, cus, s);
    case FC1_W4A8_M64:
      if (a.K % 128 == 0 && a.N % 128 == 0) return launch_prefill<true>(a, max_mtiles, cus, s);
      return general_epilogue(a) ? launch_persistent<fc1_kernel<true, 4, false, true>>(a, work, cus, s)
                                 : launch_persistent<fc1_kernel<true, 4>>(a, work, cus, s);
    case FC1_W4A8_M128:   // offered only where K and N are multiples of 128
      if (a.K % 128 == 0 && a.N % 128 == 0) return launch_prefill_wide<true>(a, max_mtiles, cus, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fc2(int tactic, const GemmArgs& a, int max_mtiles, int cus, hipStream_t s) {
  const bool decode = tactic == FC2_W4A16_M16 || tactic == FC2_W4A8_M16;
  const int64_t work = work_items(false, decode, a, max_mtiles);
  switch (tactic) {
    case FC2_W4A16_M16: return launch_decode<false, false>(a, work, cus, s);
    case FC2_W4A16_M64:
      return a.nvfp4 ? launch_persistent<fc2_kernel<false, 4, true>>(a, work, cus, s)
                     : launch_persistent<fc2_kernel<false, 4>>(a, work, cus, s);
    case FC2_W4A8_M16: return launch_decode<true, false>(a, work, cus, s);
    case FC2_W4A8_M64:   // the LDS kernel addresses h with 32-bit offsets
      if (a.K % 128 == 0 && (int64_t)max_mtiles * 64 * a.K < ((int64_t)1 << 31))
        return launch_prefill<false>(a, max_mtiles, cus, s);
      return launch_persistent<fc2_kernel<true, 4>>(a, work, cus, s);
    case FC2_W4A8_M128:
      if (a.K % 128 == 0 && (int64_t)max_mtiles * 128 * a.K < ((int64_t)1 << 31))
        return launch_prefill_wide<false>(a, max_mtiles, cus, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace situ

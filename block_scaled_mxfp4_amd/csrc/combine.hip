// Top-k weighted combine into the shard's partial output.
//
// out[t, :] = sum over slots s = 0..k-1 whose pair is local, in slot order,
// of weight[t, s] * y[inv[t*k + s], :], accumulated in fp32 (the golden
// skeleton's `out += weight * (h @ w2.T)` in the review of
// test_kimi_k3_situ_moe.py, pull request 17865).  A token with no local slot
// gets an exact zero row ("TokenSpeed SiTU", "Supported contract": the
// output is a partial sum the caller all-reduces, so nothing is
// renormalized).  A workgroup covers 512 columns of one token (fp32 y: four
// per lane of two waves; fp16 y: eight per lane of one wave); slot rows are
// fetched eight at a time and summed in slot order.  fp16 y carries a
// power-of-two scale 2^(E-127) per 64 columns, decoded exactly to fp32 here.
#include "common.hpp"
#include "dma.hpp"
#include "internal.hpp"

namespace situ {

// The routing weight of slot s (bf16 bits wb) as fp32, times the FC2 output
// scale alpha_down of the slot's expert where one is given (one fp32
// product; the expert comes from the slot's global id).
template <bool AD>
__device__ __forceinline__ float slot_weight(const CombineArgs& a, int64_t t, int s, int pos, uint32_t wb, cptr pk) {
  float w = bf16_to_f32(wb);
  if (AD && pos >= 0) {
    const int id = a.packed ? (int)((uint32_t)pk[s] & 0xffffu) : a.ids[t * a.k + s];
    w = w * a.alpha_down[id - a.off];
  }
  return w;
}

constexpr int kCombineThreads = 128;
constexpr int kCombineCols = kCombineThreads * 4;   // columns per workgroup
constexpr int kSlotBatch = 8;                       // slot loads kept in flight together

// AD: a per-expert FC2 output scale (alpha_down) is given.
template <bool Y16, bool AD>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  const int nblk = (a.H + kCombineCols - 1) / kCombineCols;
  const int64_t items = a.T * nblk;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t t = it / nblk;
    const int c = (int)(it % nblk) * kCombineCols + threadIdx.x * 4;
    if (c >= a.H) continue;
    const cptr inv = (cptr)(a.inv + t * a.k);          // the token's slots: scalar loads
    const cptr pk = (cptr)(a.packed ? a.packed + t * a.k : a.inv);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.k; s0 += kSlotBatch) {
      int pos[kSlotBatch];
      float wgt[kSlotBatch];
      f32x4 yv[kSlotBatch];
#pragma unroll
      for (int u = 0; u < kSlotBatch; ++u) {
        const int s = s0 + u;
        pos[u] = s < a.k ? inv[s] : -1;
        const uint32_t wb = s < a.k ? (a.packed ? ((uint32_t)pk[s] >> 16) : a.weights[t * a.k + s]) : 0u;
        wgt[u] = slot_weight<AD>(a, t, s, pos[u], wb, pk);
      }
      if constexpr (Y16) {
        const int64_t nb64 = (a.H + 63) / 64;
        uint2 hv[kSlotBatch];
        uint32_t ev[kSlotBatch];
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u)
          if (pos[u] >= 0) {
            hv[u] = *reinterpret_cast<const uint2*>(a.y16 + (int64_t)pos[u] * a.H + c);
            ev[u] = a.y_exp[(int64_t)pos[u] * nb64 + c / 64];
          }
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u)
          if (pos[u] >= 0) {
            const float sc = __builtin_bit_cast(float, ev[u] << 23);   // 2^(E - 127), E in [1, 254]
            yv[u][0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[u].x & 0xffffu)) * sc;
            yv[u][1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[u].x >> 16)) * sc;
            yv[u][2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[u].y & 0xffffu)) * sc;
            yv[u][3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[u].y >> 16)) * sc;
          }
      } else {
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u)
          if (pos[u] >= 0) yv[u] = *reinterpret_cast<const f32x4*>(a.y + (int64_t)pos[u] * a.H + c);
      }
#pragma unroll
      for (int u = 0; u < kSlotBatch; ++u)    // accumulate in slot order
        if (pos[u] >= 0) {
          acc[0] = __builtin_fmaf(wgt[u], yv[u][0], acc[0]);
          acc[1] = __builtin_fmaf(wgt[u], yv[u][1], acc[1]);
          acc[2] = __builtin_fmaf(wgt[u], yv[u][2], acc[2]);
          acc[3] = __builtin_fmaf(wgt[u], yv[u][3], acc[3]);
        }
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

// fp16 y: one wave per 512 columns of a token, eight columns (16 bytes of y)
// per lane; the token's slot positions and weights come through scalar loads.
constexpr int kY16Cols = 512;

template <bool AD>
__global__ __launch_bounds__(kWave) void combine_y16_kernel(CombineArgs a) {
  const int nblk = (a.H + kY16Cols - 1) / kY16Cols;
  const int64_t items = a.T * nblk;
  const int64_t nb64 = (a.H + 63) / 64;
  const int lane = threadIdx.x;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t t = it / nblk;
    const int c = (int)(it % nblk) * kY16Cols + lane * 8;
    const cptr inv = (cptr)(a.inv + t * a.k);
    const cptr pk = (cptr)(a.packed ? a.packed + t * a.k : a.inv);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.k; s0 += kSlotBatch) {
      int pos[kSlotBatch];
      float wgt[kSlotBatch];
#pragma unroll
      for (int u = 0; u < kSlotBatch; ++u) {
        const int s = s0 + u;
        pos[u] = s < a.k ? inv[s] : -1;
        const uint32_t wb = s < a.k ? (a.packed ? ((uint32_t)pk[s] >> 16) : a.weights[t * a.k + s]) : 0u;
        wgt[u] = slot_weight<AD>(a, t, s, pos[u], wb, pk);
      }
      uint4 hv[kSlotBatch];
      uint32_t ev[kSlotBatch];
#pragma unroll
      for (int u = 0; u < kSlotBatch; ++u)
        if (pos[u] >= 0 && c < a.H) {
          hv[u] = *reinterpret_cast<const uint4*>(a.y16 + (int64_t)pos[u] * a.H + c);
          ev[u] = a.y_exp[(int64_t)pos[u] * nb64 + c / 64];
        }
#pragma unroll
      for (int u = 0; u < kSlotBatch; ++u)    // accumulate in slot order
        if (pos[u] >= 0 && c < a.H) {
          const float sc = __builtin_bit_cast(float, ev[u] << 23);   // 2^(E - 127), E in [1, 254]
          const uint32_t w4[4] = {hv[u].x, hv[u].y, hv[u].z, hv[u].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint16_t b = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
            acc[e] = __builtin_fmaf(wgt[u], (float)__builtin_bit_cast(_Float16, b) * sc, acc[e]);
          }
        }
    }
    if (c < a.H) {
      if (a.out_bf16) {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16_rne(acc[2 * e]) | (f32_to_bf16_rne(acc[2 * e + 1]) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + t * a.H + c) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        float* orow = static_cast<float*>(a.out) + t * a.H + c;
        *reinterpret_cast<f32x4*>(orow) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(orow + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
      }
    }
  }
}

// Zero rows of pairs outside the shard: one wave per row, 16 bytes per lane.
__global__ __launch_bounds__(256) void zero_nonlocal_rows_kernel(const int32_t* inv, uint16_t* rows, int64_t TK,
                                                                  int32_t I) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= TK || inv[row] >= 0) return;
  uint16_t* r = rows + row * I;
  for (int c = (threadIdx.x % kWave) * 8; c < I; c += kWave * 8)
    *reinterpret_cast<uint4*>(r + c) = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero_nonlocal_rows(const int32_t* inv, uint16_t* rows, int64_t TK, int32_t I, hipStream_t s) {
  if (TK == 0) return hipSuccess;
  const int64_t grid = (TK + 3) / 4;
  hipLaunchKernelGGL(zero_nonlocal_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, inv, rows, TK, I);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t nblk = (a.H + kCombineCols - 1) / kCombineCols;
  const int64_t items = a.T * nblk;
  const int64_t grid = items < (1 << 20) ? items : (1 << 20);
  const bool ad = a.alpha_down != nullptr;
  if (a.y16 && a.H % 8 == 0) {
    const int64_t nb16 = (a.H + kY16Cols - 1) / kY16Cols;
    const int64_t it16 = a.T * nb16;
    const int64_t g16 = it16 < (1 << 20) ? it16 : (1 << 20);
    if (ad) hipLaunchKernelGGL(combine_y16_kernel<true>, dim3((unsigned)g16), dim3(kWave), 0, s, a);
    else hipLaunchKernelGGL(combine_y16_kernel<false>, dim3((unsigned)g16), dim3(kWave), 0, s, a);
  } else if (a.y16) {
    if (ad) hipLaunchKernelGGL((combine_kernel<true, true>), dim3((unsigned)grid), dim3(kCombineThreads), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<true, false>), dim3((unsigned)grid), dim3(kCombineThreads), 0, s, a);
  } else {
    if (ad) hipLaunchKernelGGL((combine_kernel<false, true>), dim3((unsigned)grid), dim3(kCombineThreads), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<false, false>), dim3((unsigned)grid), dim3(kCombineThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace situ

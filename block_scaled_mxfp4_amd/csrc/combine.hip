// Top-k weighted combine into the shard's partial output.
//
// out[t, :] = sum over slots s = 0..k-1 whose pair is local, in slot order,
// of weight[t, s] * y[inv[t*k + s], :], accumulated in fp32 (the golden
// skeleton's `out += weight * (h @ w2.T)` in the review of
// test_kimi_k3_situ_moe.py, pull request 17865).  A token with no local slot
// gets an exact zero row ("TokenSpeed SiTU", "Supported contract": the
// output is a partial sum the caller all-reduces, so nothing is
// renormalized).  A workgroup covers 512 columns of one token, four per lane;
// slot rows are fetched eight at a time and summed in slot order.  y is fp32,
// or fp16 with a power-of-two scale 2^(E-127) per 64 columns (decoded
// exactly to fp32 here).
#include "common.hpp"
#include "internal.hpp"

namespace situ {

constexpr int kCombineThreads = 128;
constexpr int kCombineCols = kCombineThreads * 4;   // columns per workgroup
constexpr int kSlotBatch = 8;                       // slot loads kept in flight together

template <bool Y16>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  const int nblk = (a.H + kCombineCols - 1) / kCombineCols;
  const int64_t items = a.T * nblk;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t t = it / nblk;
    const int c = (int)(it % nblk) * kCombineCols + threadIdx.x * 4;
    if (c >= a.H) continue;
    const int32_t* inv = a.inv + t * a.k;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.k; s0 += kSlotBatch) {
      int pos[kSlotBatch];
      float wgt[kSlotBatch];
      f32x4 yv[kSlotBatch];
#pragma unroll
      for (int u = 0; u < kSlotBatch; ++u) {
        const int s = s0 + u;
        pos[u] = s < a.k ? inv[s] : -1;
        const uint32_t wb = s < a.k ? (a.packed ? ((uint32_t)a.packed[t * a.k + s] >> 16) : a.weights[t * a.k + s]) : 0u;
        wgt[u] = bf16_to_f32(wb);
      }
      if constexpr (Y16) {
        const int64_t rows = a.T * a.k;
        uint2 hv[kSlotBatch];
        uint32_t ev[kSlotBatch];
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u)
          if (pos[u] >= 0) {
            hv[u] = *reinterpret_cast<const uint2*>(a.y16 + (int64_t)pos[u] * a.H + c);
            ev[u] = a.y_exp[(int64_t)(c / 64) * rows + pos[u]];
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

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t nblk = (a.H + kCombineCols - 1) / kCombineCols;
  const int64_t items = a.T * nblk;
  const int64_t grid = items < (1 << 20) ? items : (1 << 20);
  if (a.y16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)grid), dim3(kCombineThreads), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)grid), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace situ

// Shard filter, per-expert histogram, exclusive scans and the deterministic
// permutation of (token, slot) pairs into per-expert groups.
//
// "TokenSpeed SiTU", "Supported contract": top-k ids are GLOBAL; experts
// outside the rank's contiguous shard are filtered out and the rest produce
// a partial output.  Pairs are grouped by local expert l = id - offset, and
// inside a group they keep ascending expanded index j = t*k + s, so the
// grouping is a stable sort on (l, j) and the same on every run.
//
// Small batches: one workgroup of 16 waves does it all in LDS:
//   A. wave w counts the pairs of its contiguous chunk of j into cnt[w][l];
//   B. per expert, an exclusive scan over waves turns cnt into per-wave
//      bases; a workgroup scan over experts gives offsets[] and the m-tile
//      prefix mtiles[]; each expert writes its m-tiles' entries of
//      tile_expert[];
//   C. each wave walks its chunk again 64 pairs at a time; a lane's rank
//      among the lanes holding the same expert comes from ballots over the
//      key bits (a wavefront "match"), so position = base + rank needs no
//      atomics and is independent of scheduling.
// Large batches split the pairs into contiguous blocks: per-block histograms,
// one scan workgroup (prefix over blocks, then over experts), and a scatter
// in which every block repeats A and C on its own pairs from its own bases.
// With bf16 activations in w4a8, further workgroups of the first launch
// (the router's, or the histograms') quantize them to MXFP8 meanwhile: the
// quantization moves into the permute step's launch.
// Every position depends only on the input, never on timing.
#include "common.hpp"
#include "internal.hpp"
#include "quant.hpp"

namespace situ {

constexpr int kRouteWaves = 16;
static_assert(kRouteThreads == kRouteWaves * kWave, "the routing workgroup is 16 waves");

__device__ __forceinline__ int local_expert_of(const RouteArgs& a, int64_t j) {
  int id = a.packed ? (a.packed[j] & 0xFFFF) : a.ids[j];
  int l = id - a.off;
  return (l >= 0 && l < a.E_l) ? l : -1;
}

// Pairs [j0, j1) are split into kRouteWaves contiguous sub-chunks, one per
// wave, in order.  Each wave counts its sub-chunk into cnt[wave][l]; the
// local experts of a lane's first kRouteKept pairs stay in lv[] for the
// scatter (a sub-chunk of blocks of up to 4096 pairs needs no reload).
constexpr int kRouteKept = 4;
__device__ void count_waves(const RouteArgs& a, int64_t j0, int64_t j1, int (*cnt)[kMaxLocalExperts],
                            int lv[kRouteKept]) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  for (int i = tid; i < kRouteWaves * kMaxLocalExperts; i += kRouteThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int64_t chunk = (j1 - j0 + kRouteWaves - 1) / kRouteWaves;
  const int64_t w0 = j0 + (int64_t)wave * chunk;
  const int64_t w1 = w0 + chunk < j1 ? w0 + chunk : j1;
#pragma unroll
  for (int it = 0; it < kRouteKept; ++it) {
    const int64_t j = w0 + (int64_t)it * kWave + lane;
    lv[it] = j < w1 ? local_expert_of(a, j) : -1;
    if (lv[it] >= 0) atomicAdd(&cnt[wave][lv[it]], 1);
  }
  for (int64_t base = w0 + (int64_t)kRouteKept * kWave; base < w1; base += kWave) {
    const int64_t j = base + lane;
    if (j < w1) {
      const int l = local_expert_of(a, j);
      if (l >= 0) atomicAdd(&cnt[wave][l], 1);
    }
  }
  __syncthreads();
}

// cnt[w][l] holds the first position of wave w's pairs of expert l; walk the
// sub-chunks again 64 pairs at a time and place each pair at base + its rank
// among the lanes holding the same expert (ballots over the key bits).
__device__ void scatter_waves(const RouteArgs& a, int64_t j0, int64_t j1, int (*cnt)[kMaxLocalExperts],
                              const int lv[kRouteKept]) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t chunk = (j1 - j0 + kRouteWaves - 1) / kRouteWaves;
  const int64_t w0 = j0 + (int64_t)wave * chunk;
  const int64_t w1 = w0 + chunk < j1 ? w0 + chunk : j1;
  int nbits = 0;
  while ((1 << nbits) < a.E_l) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int it = 0;
  for (int64_t base = w0; base < w1; base += kWave, ++it) {
    const int64_t j = base + lane;
    const bool in = j < w1;
    int l = -1;
    if (it < kRouteKept) {             // uniform; the register copy, selected without indexing
#pragma unroll
      for (int q = 0; q < kRouteKept; ++q) l = it == q ? lv[q] : l;
    } else {
      l = in ? local_expert_of(a, j) : -1;
    }
    const bool loc = l >= 0;
    uint64_t eq = __ballot(loc);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = loc && ((l >> b) & 1);
      const uint64_t bb = __ballot(bit);
      eq &= bit ? bb : ~bb;
    }
    if (loc) {
      const int rank = __popcll(eq & lt_mask);
      const int total = __popcll(eq);
      const int pos = cnt[wave][l] + rank;
      a.perm[pos] = (int)j;
      a.inv[j] = pos;
      if (rank == total - 1) cnt[wave][l] = pos + 1;
    } else if (in) {
      a.inv[j] = -1;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Workgroup exclusive scans over the experts (E_l <= 1024, one per thread) of
// the totals and of their m-tile counts; writes counts, offsets, mtiles and
// the tile -> expert list.  Returns the exclusive offset of expert tid.
__device__ int scan_experts(const RouteArgs& a, int total_of_tid, int (*wave_sums)[kRouteWaves]) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int va = tid < a.E_l ? total_of_tid : 0;
  const int vb = tid < a.E_l ? (va + a.block_m - 1) / a.block_m : 0;
  int ia = va, ib = vb;
  for (int d = 1; d < kWave; d <<= 1) {
    const int ta = __shfl_up(ia, d, kWave);
    const int tb = __shfl_up(ib, d, kWave);
    if (lane >= d) { ia += ta; ib += tb; }
  }
  if (lane == kWave - 1) { wave_sums[0][wave] = ia; wave_sums[1][wave] = ib; }
  __syncthreads();
  int pa = 0, pb = 0;
  for (int w = 0; w < wave; ++w) { pa += wave_sums[0][w]; pb += wave_sums[1][w]; }
  const int excl_a = pa + ia - va;
  const int excl_b = pb + ib - vb;
  if (tid < a.E_l) {
    a.counts[tid] = va;
    a.offsets[tid] = excl_a;
    a.mtiles[tid] = excl_b;
    for (int m = 0; m < vb; ++m) {
      a.tile_expert[excl_b + m] = tid;
      a.tile_rows[2 * (excl_b + m)] = excl_a + m * a.block_m;
      a.tile_rows[2 * (excl_b + m) + 1] = min(excl_a + va, excl_a + (m + 1) * a.block_m);
    }
  }
  if (tid == a.E_l - 1) {
    a.offsets[a.E_l] = excl_a + va;
    a.mtiles[a.E_l] = excl_b + vb;
  }
  return excl_a;
}

// Workgroups past the router's (blockIdx.x >= first) quantize the bf16
// activations to MXFP8, 8-element pieces in a grid-stride loop: the
// quantization overlaps the routing and needs no launch of its own.
__device__ __forceinline__ bool quant_block(const RouteArgs& a, int first) {
  if ((int)blockIdx.x < first) return false;
  // grid-stride over the pieces: a block's lanes stay in whole 32-element
  // blocks (the stride is a multiple of 4 and cols / 8 is a multiple of 4),
  // so the four lanes of a block always leave the loop together
  const int64_t n8 = quant_pieces(a.quant);
  const int64_t stride = (int64_t)(gridDim.x - first) * kRouteThreads;
  for (int64_t c = (int64_t)(blockIdx.x - first) * kRouteThreads + threadIdx.x; c < n8; c += stride)
    quant_mxfp8_piece(a.quant, c);
  return true;
}

// Small batches: one workgroup does everything in LDS.
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  __shared__ int cnt[kRouteWaves][kMaxLocalExperts];
  __shared__ int offs[kMaxLocalExperts];
  __shared__ int wave_sums[2][kRouteWaves];
  if (quant_block(a, 1)) return;   // uniform per workgroup
  const int tid = threadIdx.x;
  int lv[kRouteKept];
  count_waves(a, 0, a.TK, cnt, lv);
  // per expert: exclusive scan over waves, total
  int total = 0;
  for (int l = tid; l < a.E_l; l += kRouteThreads) {
    int run = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = cnt[w][l];
      cnt[w][l] = run;
      run += c;
    }
    total = run;
  }
  __syncthreads();
  const int excl = scan_experts(a, total, wave_sums);
  if (tid < a.E_l) offs[tid] = excl;
  __syncthreads();
  for (int i = tid; i < kRouteWaves * a.E_l; i += kRouteThreads) cnt[i / a.E_l][i % a.E_l] += offs[i % a.E_l];
  __syncthreads();
  scatter_waves(a, 0, a.TK, cnt, lv);
}

// Large batches, three launches.  Block b owns the pairs [b*C, (b+1)*C).
// 1. per-block histograms -> hist[b][l]
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(RouteArgs a) {
  __shared__ int h[kMaxLocalExperts];
  if (quant_block(a, a.nblocks)) return;   // uniform per workgroup
  const int tid = threadIdx.x;
  for (int l = tid; l < kMaxLocalExperts; l += kRouteThreads) h[l] = 0;
  __syncthreads();
  const int64_t j0 = (int64_t)blockIdx.x * a.chunk;
  const int64_t j1 = j0 + a.chunk < a.TK ? j0 + a.chunk : a.TK;
  for (int64_t j = j0 + tid; j < j1; j += kRouteThreads) {
    const int l = local_expert_of(a, j);
    if (l >= 0) atomicAdd(&h[l], 1);
  }
  __syncthreads();
  for (int l = tid; l < a.E_l; l += kRouteThreads) a.hist[(int64_t)blockIdx.x * a.E_l + l] = h[l];
}

// 2. one workgroup: per expert, exclusive prefix over blocks (hist[b][l]
//    becomes the first position of block b's pairs of expert l within the
//    expert's group), then the expert scans.  The blocks' counts are read 16
//    at a time so their loads overlap (one dependent round trip per block
//    cost ~0.35 us each).
constexpr int kScanBatch = 16;
__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(RouteArgs a) {
  __shared__ int wave_sums[2][kRouteWaves];
  const int tid = threadIdx.x;
  int total = 0;
  if (tid < a.E_l) {
    int run = 0;
    for (int b0 = 0; b0 < a.nblocks; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        c[u] = b0 + u < a.nblocks ? a.hist[(int64_t)(b0 + u) * a.E_l + tid] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (b0 + u < a.nblocks) a.hist[(int64_t)(b0 + u) * a.E_l + tid] = run;
        run += c[u];
      }
    }
    total = run;
  }
  scan_experts(a, total, wave_sums);
}

// 3. per block: per-wave counts again, bases from offsets[l] + hist[b][l],
//    scatter.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(RouteArgs a) {
  __shared__ int cnt[kRouteWaves][kMaxLocalExperts];
  const int tid = threadIdx.x;
  const int64_t j0 = (int64_t)blockIdx.x * a.chunk;
  const int64_t j1 = j0 + a.chunk < a.TK ? j0 + a.chunk : a.TK;
  int lv[kRouteKept];
  count_waves(a, j0, j1, cnt, lv);
  for (int l = tid; l < a.E_l; l += kRouteThreads) {
    int run = a.offsets[l] + a.hist[(int64_t)blockIdx.x * a.E_l + l];
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = cnt[w][l];
      cnt[w][l] = run;
      run += c;
    }
  }
  __syncthreads();
  scatter_waves(a, j0, j1, cnt, lv);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const unsigned qb = a.quant_blocks > 0 ? (unsigned)a.quant_blocks : 0u;
  if (a.nblocks <= 1) {
    hipLaunchKernelGGL(route_kernel, dim3(1 + qb), dim3(kRouteThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)a.nblocks + qb), dim3(kRouteThreads), 0, s, a);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteThreads), 0, s, a);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(a.nblocks), dim3(kRouteThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace situ

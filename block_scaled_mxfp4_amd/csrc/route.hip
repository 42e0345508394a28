// Shard filter, per-expert histogram, exclusive scans and the deterministic
// permutation of (token, slot) pairs into per-expert groups.
//
// "TokenSpeed SiTU", "Supported contract": top-k ids are GLOBAL; experts
// outside the rank's contiguous shard are filtered out and the rest produce
// a partial output.  Pairs are grouped by local expert l = id - offset, and
// inside a group they keep ascending expanded index j = t*k + s, so the
// grouping is a stable sort on (l, j) and the same on every run.
//
// One workgroup of 16 waves does it all in LDS, with wavefront ballots:
//   A. wave w counts the pairs of its contiguous chunk of j into cnt[w][l];
//   B. per expert, an exclusive scan over waves turns cnt into per-wave
//      bases; a workgroup scan over experts gives offsets[] and the m-tile
//      prefix mtiles[]; each expert writes its m-tiles' entries of
//      tile_expert[];
//   C. each wave walks its chunk again 64 pairs at a time; a lane's rank
//      among the lanes holding the same expert comes from ballots over the
//      key bits (a wavefront "match"), so position = base + rank needs no
//      atomics and is independent of scheduling.
#include "common.hpp"
#include "internal.hpp"

namespace situ {

constexpr int kRouteWaves = 16;
constexpr int kRouteThreads = kRouteWaves * kWave;

__device__ __forceinline__ int local_expert_of(const RouteArgs& a, int64_t j) {
  int id = a.packed ? (a.packed[j] & 0xFFFF) : a.ids[j];
  int l = id - a.off;
  return (l >= 0 && l < a.E_l) ? l : -1;
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  __shared__ int cnt[kRouteWaves][kMaxLocalExperts];
  __shared__ int scan_a[kMaxLocalExperts];
  __shared__ int scan_b[kMaxLocalExperts];
  __shared__ int wave_sums[2][kRouteWaves];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int64_t TK = a.TK;
  const int64_t chunk = (TK + kRouteWaves - 1) / kRouteWaves;
  const int64_t j0 = (int64_t)wave * chunk;
  const int64_t j1 = j0 + chunk < TK ? j0 + chunk : TK;

  for (int i = tid; i < kRouteWaves * kMaxLocalExperts; i += kRouteThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();

  // A. per-wave histogram
  for (int64_t base = j0; base < j1; base += kWave) {
    int64_t j = base + lane;
    if (j < j1) {
      int l = local_expert_of(a, j);
      if (l >= 0) atomicAdd(&cnt[wave][l], 1);
    }
  }
  __syncthreads();

  // B1. per expert: exclusive scan over waves; totals into scan_a / scan_b
  for (int l = tid; l < a.E_l; l += kRouteThreads) {
    int run = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      int c = cnt[w][l];
      cnt[w][l] = run;
      run += c;
    }
    scan_a[l] = run;
    scan_b[l] = (run + a.block_m - 1) / a.block_m;
  }
  __syncthreads();

  // B2. workgroup exclusive scan over experts (E_l <= 1024 = one value per thread)
  int va = tid < a.E_l ? scan_a[tid] : 0;
  int vb = tid < a.E_l ? scan_b[tid] : 0;
  int ia = va, ib = vb;  // inclusive scan within the wave
  for (int d = 1; d < kWave; d <<= 1) {
    int ta = __shfl_up(ia, d, kWave);
    int tb = __shfl_up(ib, d, kWave);
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
    for (int m = 0; m < vb; ++m) a.tile_expert[excl_b + m] = tid;
  }
  if (tid == a.E_l - 1) {
    a.offsets[a.E_l] = excl_a + va;
    a.mtiles[a.E_l] = excl_b + vb;
  }
  __syncthreads();
  if (tid < a.E_l) scan_a[tid] = excl_a;   // group start of expert tid
  __syncthreads();
  for (int i = tid; i < kRouteWaves * a.E_l; i += kRouteThreads) {
    int w = i / a.E_l, l = i % a.E_l;
    cnt[w][l] += scan_a[l];
  }
  __syncthreads();

  // C. ranks by ballot match; positions; perm and inv
  int nbits = 0;
  while ((1 << nbits) < a.E_l) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int64_t base = j0; base < j1; base += kWave) {
    int64_t j = base + lane;
    bool in = j < j1;
    int l = in ? local_expert_of(a, j) : -1;
    bool loc = l >= 0;
    uint64_t eq = __ballot(loc);
    for (int b = 0; b < nbits; ++b) {
      bool bit = loc && ((l >> b) & 1);
      uint64_t bb = __ballot(bit);
      eq &= bit ? bb : ~bb;
    }
    if (loc) {
      int rank = __popcll(eq & lt_mask);
      int total = __popcll(eq);
      int pos = cnt[wave][l] + rank;
      a.perm[pos] = (int)j;
      a.inv[j] = pos;
      if (rank == total - 1) cnt[wave][l] = pos + 1;
    } else if (in) {
      a.inv[j] = -1;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace situ

// Prefill-shaped grouped GEMMs in w4a8: block-scaled MFMA with LDS tiles.
//
// Same arithmetic as the decode kernels (gemm.hip): FC1 = SiTU of the
// alpha-scaled gate/up halves of x.W1^T, rounded through MXFP8 per 32 along
// I ("TokenSpeed SiTU", "Activation precision": the FC1 fp8 output is
// dequantized before FC2); FC2 = h.W2^T in fp32.  Groups are hundreds to thousands of
// rows here, so the work is a contraction that should run at the matrix
// cores' rate, not a weight stream:
//  - a work item is 256 weight rows (FC1: 128 gate + the matching 128 up
//    rows) x 64 token rows of one expert; each of the 4 waves computes 128
//    weight rows x 32 tokens = 8 x 2 tiles of v_mfma_scale_f32_16x16x128
//    (E2M1 weights x E4M3 activations, both E8M0 scales per 32 K);
//  - per 128-wide K step the workgroup stages 16 KB of weights, 8 KB of
//    activations and their scales in LDS, laid out as the MFMA fragments
//    themselves (lane l's 16 bytes at 16*l), so the fragment reads are
//    conflict-free ds_read_b128; two LDS stages, and the global loads of
//    step j+2 travel in registers while step j is multiplied;
//  - work items are ordered expert-major with the 64-row m-tiles fastest,
//    so consecutive items reuse one weight tile, and each XCD walks its own
//    contiguous range of items (blockIdx % 8 picks the XCD), keeping a
//    weight tile in one XCD's L2 while its m-tiles run.
// K must be a multiple of 128 (H = 3584 is 28 steps; I = 384 or 3072); the
// planner routes other shapes to the 16-row kernels.
#include "common.hpp"
#include "internal.hpp"

namespace situ {

namespace {

constexpr int kPfRows = 256;      // weight rows per work item
constexpr int kPfTok = 64;        // token rows per work item (the m-tile)
constexpr int kStageA = 16 * 1024;
constexpr int kStageB = 4 * 2048;
constexpr int kStageSA = kPfRows * 4;
constexpr int kStageSB = kPfTok * 4;
constexpr int kStage = kStageA + kStageB + kStageSA + kStageSB;   // 25856 bytes

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
constexpr uint32_t kOobPf = 0x80000000u;   // past every resource: reads 0

// What one thread loads for one K step (then writes to LDS).
struct PfRegs {
  uint4 a[4];     // 4 weight tiles' fragments of this lane
  uint4 b[2];     // lo / hi halves of one activation tile's fragment
  uint32_t sa;    // scale dword (4 K blocks) of weight row `tid`
  uint32_t sb;    // scale dword of token `tid` (tid < 64)
};

struct PfGeo {
  __amdgpu_buffer_rsrc_t wr, sr, xr, xsr;
  uint32_t a_row[4];   // byte offset of this lane's row in each of its 4 weight tiles
  uint32_t sa_row;     // scale row offset of weight row `tid`
  uint32_t b_row;      // byte offset of this lane's activation row (kOobPf if none)
  uint32_t sb_row;     // scale row offset of token `tid` (kOobPf if none)
  int g;
};

__device__ __forceinline__ void pf_load(PfRegs& rg, const PfGeo& d, int j) {
#pragma unroll
  for (int i = 0; i < 4; ++i) rg.a[i] = ld16(d.wr, d.a_row[i] + (uint32_t)(4 * j + d.g) * 16u);
  const uint32_t lo = d.b_row == kOobPf ? kOobPf : d.b_row + 128u * j + 16u * d.g;
  rg.b[0] = ld16(d.xr, lo);
  rg.b[1] = ld16(d.xr, lo == kOobPf ? kOobPf : lo + 64u);
  rg.sa = ld4(d.sr, d.sa_row + 4u * j);
  rg.sb = ld4(d.xsr, d.sb_row == kOobPf ? kOobPf : d.sb_row + 4u * j);
}

__device__ __forceinline__ void pf_store(uint8_t* st, const PfRegs& rg, int wave, int lane, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(st + (4 * wave + i) * 1024 + lane * 16) = rg.a[i];
  *reinterpret_cast<uint4*>(st + kStageA + wave * 2048 + lane * 16) = rg.b[0];
  *reinterpret_cast<uint4*>(st + kStageA + wave * 2048 + 1024 + lane * 16) = rg.b[1];
  *reinterpret_cast<uint32_t*>(st + kStageA + kStageB + tid * 4) = rg.sa;
  if (tid < kPfTok) *reinterpret_cast<uint32_t*>(st + kStageA + kStageB + kStageSA + tid * 4) = rg.sb;
}

// One K step of one wave: 8 weight tiles x 2 token tiles of MFMAs.
__device__ __forceinline__ void pf_compute(const uint8_t* st, bool fc1, int wn, int wm, int lane, f32x4 acc[8][2]) {
  const int r = lane & 15, g = lane >> 4;
  uint32_t bf[2][8], sb[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tile = 2 * wm + tt;
    const uint4 lo = *reinterpret_cast<const uint4*>(st + kStageA + tile * 2048 + lane * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(st + kStageA + tile * 2048 + 1024 + lane * 16);
    bf[tt][0] = lo.x; bf[tt][1] = lo.y; bf[tt][2] = lo.z; bf[tt][3] = lo.w;
    bf[tt][4] = hi.x; bf[tt][5] = hi.y; bf[tt][6] = hi.z; bf[tt][7] = hi.w;
    sb[tt] = st[kStageA + kStageB + kStageSA + (16 * tile + r) * 4 + g];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // FC1: gate tiles 4wn..4wn+3 then the matching up tiles 8+4wn..; FC2: tiles 8wn..8wn+7
    const int tile = fc1 ? (i < 4 ? 4 * wn + i : 8 + 4 * wn + (i - 4)) : 8 * wn + i;
    const uint4 av = *reinterpret_cast<const uint4*>(st + tile * 1024 + lane * 16);
    const uint32_t a4[4] = {av.x, av.y, av.z, av.w};
    const uint32_t sa = st[kStageA + kStageB + (16 * tile + r) * 4 + g];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) acc[i][tt] = mfma_scale_fp4_fp8(a4, bf[tt], sa, sb[tt], acc[i][tt]);
  }
}

}  // namespace

template <bool FC1>
__global__ __launch_bounds__(kGemmThreads, 2) void prefill_gemm_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];   // 2 stages
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  const int K = a.K, nkb = K / 32, steps = K / 128;
  const int n_tiles = FC1 ? a.N / 128 : (a.N + kPfRows - 1) / kPfRows;
  const int total = a.mtiles[a.E_l] * n_tiles;
  const int n_rows = FC1 ? 2 * a.N : a.N;
  // XCD-aware walk: workgroup b runs on XCD b % 8; each XCD takes a contiguous
  // range of items so consecutive items (same weight tile) share its L2.
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd_wgs = (gridDim.x + 7 - xcd) / 8;
  const int chunk = (total + 7) / 8;
  const int i_begin = xcd * chunk, i_end = min(total, i_begin + chunk);

  for (int it = i_begin + slot; it < i_end; it += per_xcd_wgs) {
    // item -> (expert, n-tile, m-tile of the expert), m fastest
    const int l = a.tile_expert[it / n_tiles];
    const int m_l = a.mtiles[l + 1] - a.mtiles[l];
    const int rr = it - a.mtiles[l] * n_tiles;
    const int nt = rr / m_l, m = rr % m_l;
    const int p0 = a.offsets[l] + m * kPfTok;
    const int p1 = min(a.offsets[l + 1], p0 + kPfTok);

    PfGeo d;
    d.g = g;
    const size_t wexp = (size_t)n_rows * (size_t)(K / 2);
    d.wr = rsrc(a.w + (size_t)l * wexp, (uint32_t)wexp);
    d.sr = rsrc(a.ws + (size_t)l * n_rows * nkb, (uint32_t)(n_rows * nkb));
    const int n0 = FC1 ? nt * 128 : nt * kPfRows;
    // weight rows of the 4 tiles this thread loads (tiles 4*wave .. 4*wave+3)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * wave + i;
      const int row = FC1 ? (t < 8 ? n0 + 16 * t : a.N + n0 + 16 * (t - 8)) + r : n0 + 16 * t + r;
      d.a_row[i] = (uint32_t)row * (uint32_t)(K / 2);       // rows past H (FC2) read zeros
    }
    {
      const int row = FC1 ? (tid < 128 ? n0 + tid : a.N + n0 + tid - 128) : n0 + tid;
      d.sa_row = (uint32_t)row * (uint32_t)nkb;
    }
    // activation rows: this thread loads token tile `wave`, token r of it
    {
      const int p = p0 + 16 * wave + r;
      const bool ok = p < p1;
      int64_t trow = 0;
      if (ok) trow = FC1 ? (int64_t)(a.perm[p] / a.top_k) : (int64_t)p;
      d.xr = rsrc(a.act, 0x7fffffff);
      d.b_row = ok ? (uint32_t)(trow * K) : kOobPf;
      const int ps = p0 + tid;
      const bool oks = tid < kPfTok && ps < p1;
      int64_t srow = 0;
      if (oks) srow = FC1 ? (int64_t)(a.perm[ps] / a.top_k) : (int64_t)ps;
      d.xsr = rsrc(a.act_scale, 0x7fffffff);
      d.sb_row = oks ? (uint32_t)(srow * nkb) : kOobPf;
    }

    f32x4 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    PfRegs rg;
    pf_load(rg, d, 0);
    pf_store(lds, rg, wave, lane, tid);
    if (steps > 1) pf_load(rg, d, 1);
    __syncthreads();
    for (int j = 0; j < steps; ++j) {
      uint8_t* cur = lds + (j & 1) * kStage;
      uint8_t* nxt = lds + ((j + 1) & 1) * kStage;
      pf_compute(cur, FC1, wn, wm, lane, acc);
      if (j + 1 < steps) {
        pf_store(nxt, rg, wave, lane, tid);
        if (j + 2 < steps) pf_load(rg, d, j + 2);
      }
      __syncthreads();
    }

    // epilogue
    if constexpr (FC1) {
      const int I = a.N;
      const float ag = a.alpha_g ? a.alpha_g[l] : 1.0f;
      const float au = a.alpha_u ? a.alpha_u[l] : 1.0f;
      const float bb = a.beta[l], lb = a.lbeta[l];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int p = p0 + 32 * wm + 16 * tt + r;
        const bool valid = p < p1;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {      // two 32-column MXFP8 blocks per wave
          float hv[2][4];
          float amax = 0.0f;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 2 * blk + h2;
              hv[h2][e] = situ_act(ag * acc[i][tt][e], au * acc[4 + i][tt][e], bb, lb);
              amax = fmaxf(amax, fabsf(hv[h2][e]));
            }
          amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
          amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
          const int col0 = n0 + 64 * wn + 32 * blk;     // first gate column of this block
          if (valid) {
            const uint32_t code = e8m0_code_for_e4m3(amax);
            const int sh = 127 - (int)code;
            uint8_t* hrow = static_cast<uint8_t*>(a.out) + (int64_t)p * I + col0 + 4 * g;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              uint32_t packed = 0;
#pragma unroll
              for (int e = 0; e < 4; ++e) packed |= e4m3_encode(__builtin_ldexpf(hv[h2][e], sh)) << (8 * e);
              *reinterpret_cast<uint32_t*>(hrow + 16 * h2) = packed;
            }
            if (g == 0) a.out_scale[(int64_t)p * (I / 32) + col0 / 32] = (uint8_t)code;
          }
        }
      }
    } else {
      const int H = a.N;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int p = p0 + 32 * wm + 16 * tt + r;
        if (p >= p1) continue;
        float* yrow = static_cast<float*>(a.out) + (int64_t)p * H;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row0 = n0 + 16 * (8 * wn + i);
          if (row0 >= H) continue;                 // uniform: H is a multiple of 16
          *reinterpret_cast<f32x4*>(yrow + row0 + 4 * g) = acc[i][tt];
        }
      }
    }
  }
}

uint32_t prefill_lds_bytes() { return 2 * kStage; }

template <bool FC1>
hipError_t launch_prefill(const GemmArgs& a, int max_mtiles, int cus, hipStream_t s) {
  static int per_cu = 0;
  if (!per_cu) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_gemm_kernel<FC1>, kGemmThreads, 2 * kStage) !=
            hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  const int n_tiles = FC1 ? a.N / 128 : (a.N + kPfRows - 1) / kPfRows;
  const int64_t work = (int64_t)max_mtiles * n_tiles;
  int64_t grid = (int64_t)cus * per_cu;
  if (grid > work) grid = (work + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_gemm_kernel<FC1>, dim3((unsigned)grid), dim3(kGemmThreads), 2 * kStage, s, a);
  return hipGetLastError();
}

template hipError_t launch_prefill<true>(const GemmArgs&, int, int, hipStream_t);
template hipError_t launch_prefill<false>(const GemmArgs&, int, int, hipStream_t);

}  // namespace situ

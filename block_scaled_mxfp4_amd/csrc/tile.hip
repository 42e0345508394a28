// MXFP4 expert weights rearranged into the fragment-tiled layout the GEMM
// kernels read fastest (SITU_WEIGHTS_MXFP4_TILED).
//
// The values are the caller's MXFP4 weights unchanged; only their order in
// memory differs.  Each (16-row tile, 128-wide K step) becomes one 1024-byte
// block of E2M1 in MFMA lane order (lane l's 16 bytes: row l % 16 of the
// tile, K block 4 j + l / 16, as the matrix cores take them) and one 64-byte
// block of E8M0 scales in the same lane order; tiles of an expert run
// row-tile-major, K steps fastest.  A kernel then requests a weight fragment
// as 1 KB of contiguous memory, where from rows of K / 2 bytes it touches 16
// rows x 64 bytes (the address unit's slowest pattern, measured on gfx950 at
// half the rate of whole contiguous lines), and a tile's K stream is one
// contiguous range.  Blocks past K (a K tail) hold zero codes and scale 127.
//
// The layout is this library's own arrangement of the weights: the pages
// leave weight arrangement to each MoE backend ("bring up Kimi K3 NVFP4 with
// CUTLASS and cuteDSL MegaMoE SiTU", the expert loader's note that every
// backend-specific decision stays owned by the backend).
#include "common.hpp"
#include "internal.hpp"

namespace situ {

// One thread per 16 bytes of the tiled E2M1 output (and one scale byte).
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint8_t* __restrict__ w,
                                                           const uint8_t* __restrict__ ws, uint8_t* __restrict__ wt,
                                                           uint8_t* __restrict__ st, int64_t n16, int R, int K) {
  const int nkb = K / 32, S = tiled_steps(K), tiles = R / 16;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n16; c += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c % 64);
    const int64_t blk = c / 64;                     // (expert, tile, step) block
    const int j = (int)(blk % S);
    const int64_t et = blk / S;                     // expert * tiles + tile
    const int64_t e = et / tiles;
    const int rt = (int)(et % tiles);
    const int row = 16 * rt + lane % 16, kb = 4 * j + lane / 16;
    uint4 v = make_uint4(0, 0, 0, 0);
    uint8_t sc = 127;
    if (kb < nkb) {
      const int64_t r = e * R + row;
      v = *reinterpret_cast<const uint4*>(w + r * (K / 2) + (int64_t)kb * 16);
      sc = ws[r * nkb + kb];
    }
    reinterpret_cast<uint4*>(wt)[c] = v;
    st[c] = sc;
  }
}

hipError_t launch_tile_weights(const uint8_t* w, const uint8_t* ws, uint8_t* wt, uint8_t* st, int E, int R, int K,
                               hipStream_t s) {
  const int64_t n16 = (int64_t)E * (R / 16) * tiled_steps(K) * 64;
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(tile_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, ws, wt, st, n16, R, K);
  return hipGetLastError();
}

}  // namespace situ

// Internal interfaces between the host planner (situ_moe_api.cpp) and the
// kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/situ_moe.h"

namespace situ {

constexpr int kMaxLocalExperts = 1024;

struct QuantArgs {
  const uint16_t* x;       // bf16 [rows, cols]
  uint8_t* codes;          // [rows, cols]
  uint8_t* scales;         // [rows, cols/32]
  int64_t rows;
  int32_t cols;
};

struct RouteArgs {
  const int32_t* ids;      // [T*k] or null when packed
  const int32_t* packed;   // [T*k] or null
  int64_t TK;
  int32_t off, E_l, block_m;
  int32_t* counts;         // [E_l]
  int32_t* offsets;        // [E_l+1]
  int32_t* mtiles;         // [E_l+1]
  int32_t* tile_expert;    // [max_mtiles]
  int32_t* tile_rows;      // [max_mtiles, 2] (p0, p1) of each m-tile
  int32_t* perm;           // [TK]
  int32_t* inv;            // [TK]
  int32_t* hist;           // [nblocks, E_l] (multi-block routing only)
  int64_t chunk;           // pairs per block
  int32_t nblocks;         // 1 = single-workgroup routing
  // w4a8 with bf16 input: the activations' MXFP8 quantization runs in the
  // same launch as the router (single-workgroup routing) or as its count
  // step, in quant_blocks further workgroups of kRouteThreads pieces (0: none)
  QuantArgs quant;
  int32_t quant_blocks;
};

constexpr int kRouteThreads = 1024;   // the routing kernels' workgroup (16 waves)
// 8-element pieces of a quantization (one thread each)
__host__ __device__ inline int64_t quant_pieces(const QuantArgs& a) { return a.rows * (int64_t)(a.cols / 8); }



// Grouped GEMM arguments shared by FC1 and FC2.  Rows of the A side (the
// token-expert pairs) are found through the tile list built by the router.
struct GemmArgs {
  // activations of the K loop: FC1 reads the token rows x[t] (t = perm[p] / k),
  // FC2 reads the FC1 output rows h[p] directly.
  const void* act;            // bf16 [rows, K] or E4M3 codes [rows, K]
  const uint8_t* act_scale;   // E8M0 [rows, K/32] (fp8 activations only)
  const int32_t* perm;        // FC1 only: row p -> expanded index
  int32_t top_k;              // FC1 only
  const int32_t* offsets;     // [E_l+1]
  const int32_t* mtiles;      // [E_l+1] (mtiles[E_l] = number of m-tiles)
  const int32_t* tile_expert; // [max_mtiles]
  const int32_t* tile_rows;   // [max_mtiles, 2] first / one-past-last pair of each m-tile
  const uint8_t* w;           // MXFP4 [E_l, N_total, K/2]
  const uint8_t* ws;          // E8M0 [E_l, N_total, K/32]
  int32_t K;                  // contraction length (H for FC1, I for FC2)
  int32_t N;                  // FC1: I (gate columns; up rows at I + n); FC2: H
  int32_t E_l;
  // FC1 epilogue: the gated activation (kActSitu / kActSwiglu / kActSwigluBias)
  // and its two per-expert parameters (SiTU: beta, linear beta; SwigluBias:
  // alpha, beta; SwiGLU: none, may be null)
  int32_t act_kind;
  const float* beta;
  const float* lbeta;
  const float* alpha_g;       // may be null
  const float* alpha_u;       // may be null
  const uint16_t* lora_delta; // FC1: bf16 [T*k, 2I] added to the alpha-scaled halves, by expanded index, or null
  uint16_t* lora_out;         // FC1: bf16 [T*k, I] receives h by expanded index, or null
  // weights: 0 = MXFP4 (E8M0 per 32 along K), 1 = NVFP4 (E4M3 per 16; w4a16 kernels only)
  int32_t nvfp4;
  // MXFP4 weights in the fragment-tiled layout (tiled_w_offset / tiled_s_offset)
  int32_t tiled;
  // outputs
  void* out;                  // FC1: h bf16 [P, I] or E4M3 [P, I]; FC2: y float [P, H] or fp16 [P, H]
  uint8_t* out_scale;         // FC1 w4a8: E8M0 [P, I/32]; FC2: null (fp32 y) or y's exponents [ceil(H/64), out_rows]
  int32_t out_rows;           // FC2 with fp16 y: rows of y (the exponent array's leading dimension)
};

struct CombineArgs {
  const float* y;             // [P, H] fp32, or null when y16 is given
  const uint16_t* y16;        // [P, H] fp16 scaled per 64 columns by 2^(y_exp - 127), or null
  const uint8_t* y_exp;       // [T*k, ceil(H/64)]: row-major
  const int32_t* inv;         // [T*k]
  const uint16_t* weights;    // bf16 [T, k] or null
  const int32_t* packed;      // [T, k] or null
  void* out;                  // [T, H]
  int64_t T;
  int32_t H, k, out_bf16;
  const float* alpha_down;    // [E_l] per-expert FC2 output scale, or null
  const int32_t* ids;         // [T, k] global ids (unpacked routing; packed carries them in the low 16 bits)
  int32_t off;                // local expert offset
};

// Zero the rows [T*k, I] of pairs outside the shard (inv < 0) in the bf16
// down-LoRA input (the FC1 epilogues write the local rows).
hipError_t launch_zero_nonlocal_rows(const int32_t* inv, uint16_t* rows, int64_t TK, int32_t I, hipStream_t s);

// FC1 epilogues come in two compiled forms: SiTU without LoRA bridges (the
// default path, with the fewest registers), and the general one (every
// activation kind, the LoRA delta and the down-LoRA rows).
inline bool general_epilogue(const GemmArgs& a) {
  return a.act_kind != 0 || a.lora_delta != nullptr || a.lora_out != nullptr;
}

// Record a formatted message for situ_moe_last_error() and return `status`
// (the planner's error reporting, shared with the other entry points).
situ_status fail_status(situ_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Workgroups of `kernel` resident per CU at this block size and dynamic LDS
// size (hipOccupancyMaxActiveBlocksPerMultiprocessor, cached; thread-safe).
int resident_per_cu(const void* kernel, int threads, uint32_t lds_bytes);

hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_quant_mxfp8(const QuantArgs& a, hipStream_t s);
// tactic ids select the activation format and the token tile count
// The GEMM launchers size a persistent grid from the m-tile bound and the CU count.
hipError_t launch_fc1(int tactic, const GemmArgs& a, int max_mtiles, int cus, hipStream_t s);
hipError_t launch_fc2(int tactic, const GemmArgs& a, int max_mtiles, int cus, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
// LDS-tiled block-scaled MFMA kernels for prefill-sized groups in w4a8
// (K a multiple of 128; FC1 also needs I a multiple of 128).
template <bool FC1>
hipError_t launch_prefill(const GemmArgs& a, int max_mtiles, int cus, hipStream_t s);
template <bool FC1>
hipError_t launch_prefill_wide(const GemmArgs& a, int max_mtiles, int cus, hipStream_t s);

// Tactic family: (activation format, token tiles of 16 per m-tile)
enum Tactic : int32_t {
  FC1_W4A16_M16 = 0,
  FC1_W4A16_M64 = 1,
  FC1_W4A8_M16 = 2,
  FC1_W4A8_M64 = 3,
  FC1_W4A8_M128 = 4,
  FC1_FUSED_W4A16_M16 = 5,   // the fused decode kernel: both GEMMs in one launch
  FC1_FUSED_W4A8_M16 = 6,
  FC2_W4A16_M16 = 16,
  FC2_W4A16_M64 = 17,
  FC2_W4A8_M16 = 18,
  FC2_W4A8_M64 = 19,
  FC2_W4A8_M128 = 20,
  FC2_FUSED_W4A16_M16 = 21,  // the FC2 half of the fused pairs
  FC2_FUSED_W4A8_M16 = 22,
};

// The fused decode kernel (FC1 then FC2 per 16-row m-tile, h kept in LDS):
// offered for these sizes (hidden H, intermediate I).
bool fused_decode_ok(int H, int I);
hipError_t launch_fused_decode(const GemmArgs& fc1, const GemmArgs& fc2, bool fp8, int max_mtiles, int cus,
                               hipStream_t s);

// The fragment-tiled MXFP4 layout (SITU_WEIGHTS_MXFP4_TILED): an expert's
// R x K weight matrix as (R / 16) x S blocks, S = ceil(K / 128), block
// (rt, j) = rows 16 rt .. + 15, K 128 j .. + 127.  The E2M1 block is 1024
// bytes in MFMA lane order (lane l's 16 bytes: row 16 rt + l % 16, K block
// 4 j + l / 16), its E8M0 block 64 bytes (byte l, the same row and block).
__host__ __device__ constexpr int tiled_steps(int K) { return (K / 32 + 3) / 4; }
__host__ __device__ constexpr uint64_t tiled_w_offset(int rt, int j, int S) { return ((uint64_t)rt * S + j) * 1024u; }
__host__ __device__ constexpr uint64_t tiled_s_offset(int rt, int j, int S) { return ((uint64_t)rt * S + j) * 64u; }
// bytes of one expert's matrix in either layout
__host__ __device__ constexpr uint64_t expert_w_bytes(bool tiled, int R, int K) {
  return tiled ? (uint64_t)R * tiled_steps(K) * 64u : (uint64_t)R * (uint64_t)(K / 2);
}
// scale bytes per weight row as the kernels stage them: MXFP4 K / 32, NVFP4
// K / 16, tiled 4 S (a K tail's blocks are padded to whole steps)
__host__ __device__ constexpr int scale_row_bytes(bool nv, bool tiled, int K) {
  return nv ? K / 16 : (tiled ? 4 * tiled_steps(K) : K / 32);
}

hipError_t launch_tile_weights(const uint8_t* w, const uint8_t* ws, uint8_t* wt, uint8_t* st, int E, int R, int K,
                               hipStream_t s);

// `blocks` workgroups of 4 waves, each running `iters` rounds of 8 block-scaled
// FP4 x FP8 MFMAs on registers (the matrix-core peak measurement).
hipError_t launch_mfma_peak(int iters, int blocks, hipStream_t s);

// Workgroup shapes of the grouped GEMMs (4 waves of 64 lanes).
constexpr int kGemmThreads = 256;
constexpr int kFc1ColsPerWave = 32;    // gate columns per wave (with the matching up columns)
constexpr int kFc2RowsPerWave = 64;    // output columns of y per wave

}  // namespace situ

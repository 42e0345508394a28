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
//    conflict-free ds_read_b128;
//  - the stages are filled by LDS DMA (buffer_load ... lds): global data goes
//    straight to LDS without passing through registers, so a ring of
//    kPfStages stages keeps kPfStages - 1 K steps in flight while one is
//    multiplied.  Each stage is its own LDS array, which lets the compiler
//    wait for exactly the DMA that filled the stage being read; the
//    workgroup barrier that publishes a stage waits on this wave's DMA count
//    explicitly (all loads return in order);
//  - work items are ordered expert-major with the 64-row m-tiles fastest,
//    so consecutive items reuse one weight tile, and each XCD walks its own
//    contiguous range of items (blockIdx % 8 picks the XCD), keeping a
//    weight tile in one XCD's L2 while its m-tiles run.
// K must be a multiple of 128 (H = 3584 is 28 steps; I = 384 or 3072); the
// planner routes other shapes to the 16-row kernels.
#include "common.hpp"
#include "dma.hpp"
#include "epilogue.hpp"
#include "internal.hpp"

namespace situ {

namespace {

constexpr int kPfRows = 256;      // weight rows per work item
constexpr int kPfTok = 64;        // token rows per work item (the m-tile)
constexpr int kStageA = 16 * 1024;
// activation tile: 2 DMA blocks of 8 tokens x 128 B (full cache lines) with
// 128 B between them.  On gfx950 that gap makes each 16-token fragment read a
// two-way bank conflict (back to back they are conflict-free); the wide
// kernel with the blocks back to back measured no faster (FC2 slower), so the
// layout stays.
constexpr int kTileB = 2 * (1024 + 128);
constexpr int kStageB = 4 * kTileB;
constexpr int kStageSA = kPfRows * 4;
constexpr int kStageSB = kPfTok * 4;
constexpr int kStage = kStageA + kStageB + kStageSA + kStageSB;   // 25856 bytes
constexpr int kPfStages = 3;    // 3 x 25856 B: two workgroups per CU

constexpr uint32_t kOobPf = kOobOff;

struct PfGeo {
  v4i wr, sr, xr, xsr;
  uint32_t a_row[4];   // this lane's 16 bytes of each of its 4 weight tiles at K step 0
  uint32_t sa_row;     // this lane's scale dword at K step 0 (weight row 64*wave + lane, or tiled: 4 bytes of tile 4*wave + l/16)
  uint32_t a_step, sa_step;   // bytes between K steps: 64 and 4 (rows), 1024 and 64 (fragment-tiled)
  uint32_t b_row[2];   // activation row of token l/8 (+8 for the second block) of the wave's tile (kOobPf: none)
  uint32_t sb_row;     // scale row offset of token l%16 (kOobPf if none)
  int g, lane;
};

// This wave's share of one K step, as kPfDmas DMA instructions: its 4 weight
// tiles, the lo / hi halves of its token tile, the scale dwords of weight
// rows 64*wave .. +63 and of tokens 16*wave .. +15 (lanes 0..15).  A lane
// past the data reads zeros; a DMA writes lane l's bytes at dst + size * l.
constexpr int kPfDmas = 8;
__device__ __forceinline__ void pf_issue(uint32_t st, const PfGeo& d, int j, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16(d.wr, st + (4 * wave + i) * 1024, d.a_row[i] + (uint32_t)j * d.a_step);
  // activations: lane l moves 16-byte chunk (l%8) ^ (l/8) of token 8h + l/8 (h = block),
  // so each instruction reads 8 whole 128-byte K slices and a token's chunk c
  // lands in slot c ^ (token % 8) of its row
  const uint32_t chunk = (uint32_t)(((d.lane & 7) ^ (d.lane >> 3)) * 16);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    dma16(d.xr, st + kStageA + wave * kTileB + h * (1024 + 128),
          d.b_row[h] == kOobPf ? kOobPf : d.b_row[h] + 128u * j + chunk);
  dma4(d.sr, st + kStageA + kStageB + wave * 256, d.sa_row + (uint32_t)j * d.sa_step);
  if (lane < 16)
    dma4(d.xsr, st + kStageA + kStageB + kStageSA + wave * 64, d.sb_row == kOobPf ? kOobPf : d.sb_row + 4u * j);
}

// `after` = K steps whose DMAs this wave issued after the one to wait for
// (output stores issued after that DMA are waited for as well: the count
// covers every vector-memory operation of the wave).
__device__ __forceinline__ void step_barrier(int after) {
  if (after >= 2) dma_barrier<2 * kPfDmas>();
  else if (after == 1) dma_barrier<kPfDmas>();
  else dma_barrier<0>();
}

// One K step of one wave: 8 weight tiles x 2 token tiles of MFMAs.  All of
// the step's fragment reads are issued before the first MFMA, so each MFMA
// pair waits only for its own weight fragment while the later reads are in
// flight (one register set per fragment: 58 VGPRs).  The weight scales sit
// per tile in 64 bytes, this lane's at s_rd (4 r + g from rows of scale
// dwords, 16 g + r from tiled scales).
__device__ __forceinline__ void pf_compute(const uint8_t* st, bool fc1, int wn, int wm, int lane, uint32_t s_rd,
                                           f32x4 acc[8][2]) {
  const int r = lane & 15, g = lane >> 4;
  uint4 blo[2], bhi[2];
  uint32_t sb[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tile = 2 * wm + tt;
    // token r: K 16g.. (chunk g) and K 64 + 16g.. (chunk 4 + g), in their swizzled slots
    const uint8_t* row = st + kStageA + tile * kTileB + (r >> 3) * (1024 + 128) + (r & 7) * 128;
    blo[tt] = *reinterpret_cast<const uint4*>(row + 16 * (g ^ (r & 7)));
    bhi[tt] = *reinterpret_cast<const uint4*>(row + 16 * ((4 + g) ^ (r & 7)));
    sb[tt] = st[kStageA + kStageB + kStageSA + (16 * tile + r) * 4 + g];
  }
  uint4 av[8];
  uint32_t sa[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // FC1: gate tiles 4wn..4wn+3 then the matching up tiles 8+4wn..; FC2: tiles 8wn..8wn+7
    const int tile = fc1 ? (i < 4 ? 4 * wn + i : 8 + 4 * wn + (i - 4)) : 8 * wn + i;
    av[i] = *reinterpret_cast<const uint4*>(st + tile * 1024 + lane * 16);
    sa[i] = st[kStageA + kStageB + tile * 64 + s_rd];
  }
  uint32_t bf[2][8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    bf[tt][0] = blo[tt].x; bf[tt][1] = blo[tt].y; bf[tt][2] = blo[tt].z; bf[tt][3] = blo[tt].w;
    bf[tt][4] = bhi[tt].x; bf[tt][5] = bhi[tt].y; bf[tt][6] = bhi[tt].z; bf[tt][7] = bhi[tt].w;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a4[4] = {av[i].x, av[i].y, av[i].z, av[i].w};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) acc[i][tt] = mfma_scale_fp4_fp8(a4, bf[tt], sa[i], sb[tt], acc[i][tt]);
  }
  // keep that order: the scheduler would otherwise sink each read to its
  // MFMA pair to save registers, exposing every read's latency
  __builtin_amdgcn_sched_group_barrier(0x100, 22, 0);   // 22 LDS reads
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);   // then the 16 MFMAs
}

// Work item -> expert, n-tile and pair range; items are ordered expert-major
// with the m-tiles of one n-tile fastest.
struct PfItem {
  int l, nt, p0, p1;
};
__device__ __forceinline__ PfItem pf_item(const GemmArgs& a, int it, int n_tiles) {
  const cptr te = (cptr)a.tile_expert, mt = (cptr)a.mtiles, of = (cptr)a.offsets;
  PfItem x;
  x.l = te[it / n_tiles];
  const int m0 = mt[x.l], m_l = mt[x.l + 1] - m0;
  const int rr = it - m0 * n_tiles;
  x.nt = rr / m_l;
  x.p0 = of[x.l] + (rr % m_l) * kPfTok;
  x.p1 = min(of[x.l + 1], x.p0 + kPfTok);
  return x;
}
// Activation rows of the tokens this lane touches in its wave's token tile
// (tile `wave_u`): token l%16 (its scale dword) and tokens l/8, 8 + l/8
// (its 16-byte chunks).  FC1 reads x[perm[p] / k], FC2 reads h[p]; -1 past
// the group.  The tile's 16 perm entries come in one scalar load (the perm
// region is padded by a tile's worth of entries past its end).
struct PfRows {
  int32_t t_s, t_a, t_b;
};
template <bool FC1>
__device__ __forceinline__ PfRows pf_act_rows(const GemmArgs& a, const PfItem& x, int wave_u, int lane) {
  const int base = x.p0 + 16 * wave_u;
  const int i_s = lane & 15, i_a = lane >> 3, i_b = 8 + (lane >> 3);
  PfRows t{-1, -1, -1};
  if (base >= x.p1) return t;                       // uniform: the whole tile is past the group
  if constexpr (!FC1) {
    t.t_s = base + i_s;
    t.t_a = base + i_a;
    t.t_b = base + i_b;
  } else {
    typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
    const i32x16 win = *(const __attribute__((address_space(4))) i32x16*)((cptr)a.perm + base);
    int32_t vs = win[0], va = win[0], vb = win[8];
#pragma unroll
    for (int i = 1; i < 16; ++i) vs = i_s == i ? win[i] : vs;
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      va = i_a == i ? win[i] : va;
      vb = i_b == 8 + i ? win[8 + i] : vb;
    }
    t.t_s = vs / a.top_k;
    t.t_a = va / a.top_k;
    t.t_b = vb / a.top_k;
  }
  if (base + i_s >= x.p1) t.t_s = -1;
  if (base + i_a >= x.p1) t.t_a = -1;
  if (base + i_b >= x.p1) t.t_b = -1;
  return t;
}

// Load geometry of one item for this thread.
template <bool FC1>
__device__ __forceinline__ PfGeo pf_geo(const GemmArgs& a, const PfItem& x, const PfRows& tr, int tid, int wave,
                                        int lane) {
  const int r = lane & 15, g = lane >> 4;
  const int K = a.K, nkb = K / 32;
  const int n_rows = FC1 ? 2 * a.N : a.N;
  PfGeo d;
  d.g = g;
  d.lane = lane;
  const bool tiled = a.tiled != 0;
  const int S = tiled_steps(K);
  const size_t wexp = expert_w_bytes(tiled, n_rows, K);
  const size_t sexp = (size_t)n_rows * scale_row_bytes(false, tiled, K);
  d.wr = rsrc4(a.w + (size_t)x.l * wexp, (uint32_t)wexp);
  d.sr = rsrc4(a.ws + (size_t)x.l * sexp, (uint32_t)sexp);
  const int n0 = FC1 ? x.nt * 128 : x.nt * kPfRows;
  // first row of the item's weight tile t (tiles past H, in FC2, read zeros)
  auto tile_row = [&](int t) { return FC1 ? (t < 8 ? n0 + 16 * t : a.N + n0 + 16 * (t - 8)) : n0 + 16 * t; };
  // the 4 tiles this thread loads (tiles 4*wave .. 4*wave+3)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row0 = tile_row(4 * wave + i);
    d.a_row[i] = tiled ? (uint32_t)(row0 / 16) * (uint32_t)S * 1024u + (uint32_t)lane * 16u
                       : (uint32_t)(row0 + r) * (uint32_t)(K / 2) + 16u * (uint32_t)g;
  }
  if (tiled) {
    d.sa_row = (uint32_t)(tile_row(4 * wave + (lane >> 4)) / 16) * (uint32_t)S * 64u + (uint32_t)(lane & 15) * 4u;
  } else {
    const int srow = FC1 ? (tid < 128 ? n0 + tid : a.N + n0 + tid - 128) : n0 + tid;
    d.sa_row = (uint32_t)srow * (uint32_t)nkb;
  }
  d.a_step = tiled ? 1024u : 64u;
  d.sa_step = tiled ? 64u : 4u;
  d.xr = rsrc4(a.act, 0x7fffffff);
  d.xsr = rsrc4(a.act_scale, 0x7fffffff);
  d.b_row[0] = tr.t_a >= 0 ? (uint32_t)tr.t_a * (uint32_t)K : kOobPf;
  d.b_row[1] = tr.t_b >= 0 ? (uint32_t)tr.t_b * (uint32_t)K : kOobPf;
  d.sb_row = tr.t_s >= 0 ? (uint32_t)tr.t_s * (uint32_t)nkb : kOobPf;
  return d;
}

// Output stores as inline assembly too (lanes with nothing to store use an
// offset past the buffer, which drops the write).  The stage waits count
// every vector-memory operation of the wave, so the waits of the next item's
// first steps, issued after these stores, wait for them as well.  The
// compiler's hazard checks do not look inside inline assembly, so
// these carry their own: the data must not come straight from an MFMA (whose
// result may still be in flight), so st16 takes it through a VALU add (+0
// turns -0 into +0) that the compiler orders after the MFMA, with two wait
// states before the store reads it; and a store reads its data registers
// after issue, so wait states follow it before any later write of them.
__device__ __forceinline__ void st16(const v4i& r, uint32_t voff, f32x4 v) {
  const f32x4 w = v + 0.0f;
  asm volatile("s_nop 1\n\tbuffer_store_dwordx4 %0, %1, %2, 0 offen\n\ts_nop 3" ::"v"(w), "v"(voff), "s"(r)
               : "memory");
}
__device__ __forceinline__ void st4(const v4i& r, uint32_t voff, uint32_t v) {
  asm volatile("buffer_store_dword %0, %1, %2, 0 offen\n\ts_nop 3" ::"v"(v), "v"(voff), "s"(r) : "memory");
}
__device__ __forceinline__ void st1(const v4i& r, uint32_t voff, uint32_t v) {
  asm volatile("buffer_store_byte %0, %1, %2, 0 offen\n\ts_nop 3" ::"v"(v), "v"(voff), "s"(r) : "memory");
}
static_assert(4 * 4352 <= kStage, "FC2 transpose scratch fits one stage");

// FC1: alpha, SiTU and the MXFP8 rounding of h (32 columns per block);
// FC2: the fp32 rows of y.  acc[i][tt] holds weight tile i x token tile tt.
// NCOL: gate columns of an FC1 work item; NG: gate tiles per wave (its up
// tiles follow them in acc), two per 32-column MXFP8 block;
// the token tiles used are acc[.][tt0 .. tt0 + 1] of a [2 NG][TT] accumulator set.
// GEN: the general FC1 epilogue (every activation kind, LoRA bridges); else
// SiTU only, with the fewest registers.
template <bool FC1, int TOK = kPfTok, int NCOL = 128, int TT = 2, bool GEN = false, int NG = 4>
__device__ __forceinline__ void pf_epilogue(const GemmArgs& a, const PfItem& x, f32x4 (&acc)[2 * NG][TT], int wn, int wm,
                                            int wave, int lane, uint8_t* scratch, int ntt = 2, int tt0 = 0) {
  const int r = lane & 15, g = lane >> 4;
  const int n0 = FC1 ? x.nt * NCOL : x.nt * kPfRows;
  if constexpr (FC1) {
    const int I = a.N;
    ActItem ai{};
    SituK sk{};
    if constexpr (GEN) ai = act_item(a, x.l);
    else sk = situ_item(a, x.l);
    const float blb = GEN ? act_blb(ai.k) : sk.blb;
    const bool bridges = GEN && (ai.lora || a.lora_out);   // uniform
    const v4i hr = rsrc4(static_cast<uint8_t*>(a.out) + (size_t)x.p0 * I, (uint32_t)(TOK * I));
    const v4i sr = rsrc4(a.out_scale + (size_t)x.p0 * (I / 32), (uint32_t)(TOK * (I / 32)));
    // the pairs' expanded indices (the rows of their LoRA deltas and down-LoRA
    // inputs), then every delta piece of the call, requested together: read
    // one by one beside the h stores, each would wait out its own latency
    // (without branches per piece: rows outside the group read pair 0's
    // entries, which are never used)
    int64_t jt[2] = {0, 0};
    DeltaPiece dl[2][NG / 2][2];
    if constexpr (GEN) {
      if (bridges) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bool ok = tt < ntt && x.p0 + 32 * wm + 16 * tt + r < x.p1;
          const int pv = a.perm[ok ? x.p0 + 32 * wm + 16 * tt + r : 0];
          jt[tt] = ok ? pv : 0;
        }
      }
      if (ai.lora) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int blk = 0; blk < NG / 2; ++blk)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
              dl[tt][blk][h2] = load_delta(a.lora_delta + jt[tt] * (2 * I) + n0 + 16 * NG * wn + 32 * blk +
                                               16 * h2 + 4 * g, I);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt >= ntt) break;                          // uniform: a tile of padding rows only
      const int pr = 32 * wm + 16 * tt + r;          // row within the m-tile
      const bool valid = x.p0 + pr < x.p1;
      const int64_t j = jt[tt];
#pragma unroll
      for (int blk = 0; blk < NG / 2; ++blk) {     // NG / 2 32-column MXFP8 blocks per wave
        // h = q * blb with q = act_q (SiTU: blb = b*lb, else 1): the block
        // maximum of |h| is blb times that of |q| (rounding is monotone), and
        // h * 2^sh is q * (blb * 2^sh) in one product, exact whenever the
        // block's scale leaves the elements that get a nonzero E4M3 code in
        // fp32's normal range (sh <= 108); other blocks (all zero, or below
        // 2^-100) take h and then 2^sh
        const int col0 = n0 + 16 * NG * wn + 32 * blk;   // first gate column of this block
        float qv[2][4];
        float amax = 0.0f;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int i = 2 * blk + h2;
          const f32x4& gv = acc[i][tt0 + tt];
          const f32x4& uv = acc[NG + i][tt0 + tt];
          if constexpr (GEN) {
            float xg[4], xu[4];
            const float ag4[4] = {gv[0], gv[1], gv[2], gv[3]};
            const float au4[4] = {uv[0], uv[1], uv[2], uv[3]};
            act_inputs_of(ai, dl[tt][blk][h2], ag4, au4, xg, xu);
#pragma unroll
            for (int e = 0; e < 4; ++e) qv[h2][e] = act_q(xg[e], xu[e], ai.k);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) qv[h2][e] = situ_q(gv[e], uv[e], sk);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(qv[h2][e]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        const uint32_t code = e8m0_code_for_e4m3(amax * blb);
        const int sh = 127 - (int)code;
        // rows past the group are not stored: their blocks do not matter
        const bool direct = __builtin_amdgcn_ballot_w64(valid && sh > 108) == 0;   // uniform
        // E4M3 codes by the hardware conversion (round to nearest even) of
        // the scaled values clamped to +-448, which gives the MX rule's
        // saturating codes; a negative value that rounds to zero keeps its
        // sign (code 0x80, the value zero)
        float sv[2][4];
        if (direct) {
          const float scl = __builtin_ldexpf(blb, sh);
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[h2][e] = qv[h2][e] * scl;
        } else {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[h2][e] = __builtin_ldexpf(qv[h2][e] * blb, sh);
        }
        uint32_t packed[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[h2][e] = fminf(fmaxf(sv[h2][e], -448.0f), 448.0f);
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sv[h2][0], sv[h2][1], 0, false);
          packed[h2] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sv[h2][2], sv[h2][3], lo, true);
        }
        const uint32_t ho = valid ? (uint32_t)(pr * I + col0 + 4 * g) : kOobPf;
        st4(hr, ho, packed[0]);
        st4(hr, valid ? ho + 16u : kOobPf, packed[1]);
        st1(sr, (valid && g == 0) ? (uint32_t)(pr * (I / 32) + col0 / 32) : kOobPf, code);
        if (GEN && a.lora_out && valid) {   // the down LoRA's input: h as bf16 by expanded index
          uint16_t* lrow = a.lora_out + j * I + col0 + 4 * g;
          *reinterpret_cast<uint2*>(lrow) = e4m3x4_to_bf16x4(packed[0], (int)code);
          *reinterpret_cast<uint2*>(lrow + 16) = e4m3x4_to_bf16x4(packed[1], (int)code);
        }
      }
    }
    if constexpr (GEN) {
      // every delta piece counts as read here, on every path (those of a token
      // tile of padding rows are not read above; without a delta nothing was
      // requested and nothing is waited for): the compiler then waits for them
      // here, behind nothing, instead of waiting for every request in flight
      // (the next item's stages) where it next writes their registers
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int blk = 0; blk < NG / 2; ++blk)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const DeltaPiece& dp = dl[tt][blk][h2];
            asm volatile("" ::"v"(dp.g.x), "v"(dp.g.y), "v"(dp.u.x), "v"(dp.u.y));
          }
    }
  } else {
    // y rows leave through LDS: a 16-token x 64-column block of the wave's
    // tiles is written in the MFMA layout and read back row by row, so that
    // each store instruction writes 4 tokens x 256 contiguous bytes (full
    // cache lines) instead of 16 tokens x 64 bytes.  scratch = 4352 bytes of
    // this wave's, in the stage the next item's first requests leave free.
    const int H = a.N;
    const v4i yr = rsrc4(static_cast<float*>(a.out) + (size_t)x.p0 * H, (uint32_t)(TOK * H * 4));
    constexpr int kRowPitch = 64 * 4 + 16;          // padded: the tile writes hit 16 distinct bank groups
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<f32x4*>(scratch + r * kRowPitch + (16 * i + 4 * g) * 4) = acc[4 * half + i][tt0 + tt];
        const int tok = lane >> 4, chunk = lane & 15;
        const int col = n0 + 16 * 8 * wn + 64 * half + 4 * chunk;
        // all four reads first: the stores below are ordered memory operations
        // the compiler does not move reads across
        f32x4 vk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) vk[k] = *reinterpret_cast<const f32x4*>(scratch + (4 * k + tok) * kRowPitch + 16 * chunk);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = 4 * k + tok;                  // token within the 16-token tile
          const f32x4 v = vk[k];
          const int pr = 32 * wm + 16 * tt + t;
          const bool ok = x.p0 + pr < x.p1 && col < H;
          st16(yr, ok ? (uint32_t)(pr * H + col) * 4u : kOobPf, v);
        }
      }
  }
}

}  // namespace

template <bool FC1, bool GEN = false>
__global__ __launch_bounds__(kGemmThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t st0[kStage];
  __shared__ __align__(16) uint8_t st1[kStage];
  __shared__ __align__(16) uint8_t st2[kStage];
  uint8_t* const stg[kPfStages] = {st0, st1, st2};
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  const int K = a.K, steps = K / 128;
  const int n_tiles = FC1 ? a.N / 128 : (a.N + kPfRows - 1) / kPfRows;
  const int total = a.mtiles[a.E_l] * n_tiles;
  // XCD-aware walk: workgroup b runs on XCD b % 8; each XCD takes a contiguous
  // range of items so consecutive items (same weight tile) share its L2.
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd_wgs = (gridDim.x + 7 - xcd) / 8;
  const int chunk = (total + 7) / 8;
  const int i_begin = xcd * chunk, i_end = min(total, i_begin + chunk);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t s_rd = a.tiled ? (uint32_t)(16 * g + r) : (uint32_t)(4 * r + g);

  // The ring restarts at stage 0 for every item; the next item's first
  // kPfStages - 1 stages are requested before this item's output stores, so
  // their latency overlaps the epilogue; the waits of its first steps then
  // also wait for the previous item's output stores.
  int it = i_begin + slot;
  PfItem cur{0, 0, 0, 0};
  PfGeo d{};
  if (it < i_end) {
    cur = pf_item(a, it, n_tiles);
    d = pf_geo<FC1>(a, cur, pf_act_rows<FC1>(a, cur, wave_u, lane), tid, wave, lane);
    lds_barrier();
#pragma unroll
    for (int u = 0; u < kPfStages - 1; ++u)
      if (u < steps) pf_issue(lds_addr_of(stg[u]), d, u, wave, lane);
  }
  for (; it < i_end; it += per_xcd_wgs) {
    // the next item's geometry (scalar loads) while the first stages load
    const int it_next = it + per_xcd_wgs;
    PfItem nxt{0, 0, 0, 0};
    PfRows trow2{-1, -1, -1};
    if (it_next < i_end) {
      nxt = pf_item(a, it_next, n_tiles);
      trow2 = pf_act_rows<FC1>(a, nxt, wave_u, lane);
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < steps; j0 += kPfStages) {
#pragma unroll
      for (int u = 0; u < kPfStages; ++u) {
        const int j = j0 + u;
        if (j < steps) {
          step_barrier(min(kPfStages - 2, steps - 1 - j));
          if (j + kPfStages - 1 < steps)
            pf_issue(lds_addr_of(stg[(u + kPfStages - 1) % kPfStages]), d, j + kPfStages - 1, wave, lane);
          pf_compute(stg[u], FC1, wn, wm, lane, s_rd, acc);
        }
      }
    }

    // every wave is done with the stages: request the next item's first ones
    lds_barrier();
    if (it_next < i_end) {
      d = pf_geo<FC1>(a, nxt, trow2, tid, wave, lane);
#pragma unroll
      for (int u = 0; u < kPfStages - 1; ++u)
        if (u < steps) pf_issue(lds_addr_of(stg[u]), d, u, wave, lane);
    }
    // the last stage is free for FC2's transpose
    pf_epilogue<FC1, kPfTok, 128, 2, GEN>(a, cur, acc, wn, wm, wave, lane, stg[kPfStages - 1] + wave * 4352);
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// Wide prefill kernel: 256 weight rows x 128 tokens per item, 8 waves (each
// 128 rows x 32 tokens, the same 8 x 2 MFMA tiles), stages of two K steps.
// With two K steps a weight row contributes 128 contiguous bytes per stage,
// so the weight DMAs also move whole cache lines (8 rows x 128 B per
// instruction, swizzled like the activations); the larger token tile halves
// the weight bytes staged per MFMA.  Two stages of 75 KB: one workgroup per
// CU.  Routed with 128-row m-tiles.
namespace {

constexpr int kWRows = 256, kWTok = 128, kWThreads = 512;
constexpr int kWTileSw = 2 * (1024 + 128);                 // one 16-row (or 16-token) swizzled tile
constexpr int kWStA = 0;                                    // 16 weight tiles
constexpr int kWStB = kWStA + 16 * kWTileSw;                // [2 steps][8 token tiles]
constexpr int kWStSA = kWStB + 16 * kWTileSw;               // [2 steps][256 rows] scale dwords
constexpr int kWStSB = kWStSA + 2 * kWRows * 4;             // [8 token tiles][2 steps][16 tokens]
constexpr int kWStage = kWStSB + kWTok * 2 * 4;             // 76800 bytes
constexpr int kWDmas = 10;                                  // DMAs per wave per stage


struct PwGeo {
  v4i wr, sr, xr, xsr;
  uint32_t a_row[2][2];  // [tile][block]: row offset of this lane's row (kOobPf: none); tiled:
                         // [tile][step of the stage]: offset of this lane's 16 bytes in stage 0
  uint32_t sa_row;       // scale row of weight row 64*(wave&3) + lane; tiled: this lane's scale
                         // dword of tile 4*(wave&3) + l/16 at K step 0
  uint32_t sa_step;      // scale bytes between K steps: 4 (rows) or 64 (tiled)
  int tiled;
  uint32_t b_row[2];     // activation rows of tokens 16*wave + l/8 (+8)
  uint32_t sb_row;       // scale row of token 16*wave + l%16
  int wave, lane, K;
};

template <bool FC1>
__device__ __forceinline__ int pw_wrow(const GemmArgs& a, int n0, int t) {   // first row of weight tile t
  return FC1 ? (t < 8 ? n0 + 16 * t : a.N + n0 + 16 * (t - 8)) : n0 + 16 * t;
}

template <bool FC1>
__device__ __forceinline__ PwGeo pw_geo(const GemmArgs& a, const PfItem& x, const PfRows& tr, int wave, int lane) {
  const int K = a.K, nkb = K / 32;
  const int n_rows = FC1 ? 2 * a.N : a.N;
  const bool tiled = a.tiled != 0;
  const int S = tiled_steps(K);
  PwGeo d;
  d.wave = wave;
  d.lane = lane;
  d.K = K;
  d.tiled = tiled;
  const size_t wexp = expert_w_bytes(tiled, n_rows, K);
  const size_t sexp = (size_t)n_rows * scale_row_bytes(false, tiled, K);
  d.wr = rsrc4(a.w + (size_t)x.l * wexp, (uint32_t)wexp);
  d.sr = rsrc4(a.ws + (size_t)x.l * sexp, (uint32_t)sexp);
  const int n0 = FC1 ? x.nt * 128 : x.nt * kWRows;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row0 = pw_wrow<FC1>(a, n0, 2 * wave + i);
      if (tiled)
        d.a_row[i][h] = (FC1 || row0 < a.N) ? ((uint32_t)(row0 / 16) * (uint32_t)S + (uint32_t)h) * 1024u + (uint32_t)lane * 16u
                                            : kOobPf;
      else {
        const int row = row0 + 8 * h + (lane >> 3);
        d.a_row[i][h] = (FC1 || row < a.N) ? (uint32_t)row * (uint32_t)(K / 2) : kOobPf;
      }
    }
  if (tiled) {
    const int row0 = pw_wrow<FC1>(a, n0, 4 * (wave & 3) + (lane >> 4));
    d.sa_row = (FC1 || row0 < a.N) ? (uint32_t)(row0 / 16) * (uint32_t)S * 64u + (uint32_t)(lane & 15) * 4u : kOobPf;
  } else {
    const int q = wave & 3, row_in = 64 * q + lane;            // weight row 0..255 of the item
    const int row = FC1 ? (row_in < 128 ? n0 + row_in : a.N + n0 + row_in - 128) : n0 + row_in;
    d.sa_row = (FC1 || row < a.N) ? (uint32_t)row * (uint32_t)nkb : kOobPf;
  }
  d.sa_step = tiled ? 64u : 4u;
  d.xr = rsrc4(a.act, 0x7fffffff);
  d.xsr = rsrc4(a.act_scale, 0x7fffffff);
  d.b_row[0] = tr.t_a >= 0 ? (uint32_t)tr.t_a * (uint32_t)K : kOobPf;
  d.b_row[1] = tr.t_b >= 0 ? (uint32_t)tr.t_b * (uint32_t)K : kOobPf;
  d.sb_row = tr.t_s >= 0 ? (uint32_t)tr.t_s * (uint32_t)nkb : kOobPf;
  return d;
}

// This wave's kWDmas DMAs of stage J (K steps 2J and 2J + 1; a step past K reads zeros).
// Weights in rows: tile block h = rows 8h .. 8h + 7, 128 bytes (both K steps) each,
// swizzled; fragment-tiled: block h = K step 2J + h, 1 KB in lane order.
__device__ __forceinline__ void pw_issue(uint32_t st, const PwGeo& d, int J) {
  const int w = d.wave, l = d.lane;
  const uint32_t chunk = (uint32_t)(((l & 7) ^ (l >> 3)) * 16);
  const uint32_t half_row = (uint32_t)d.K / 2u;              // bytes of a weight row
  const uint32_t ka = 128u * J + chunk;                      // weight bytes: 2 K steps per row
  const int steps = d.K / 128;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool past = d.tiled ? 2 * J + h >= steps : ka >= half_row;
      const uint32_t off = d.tiled ? d.a_row[i][h] + 2048u * (uint32_t)J : d.a_row[i][h] + ka;
      dma16(d.wr, st + kWStA + (2 * w + i) * kWTileSw + h * (1024 + 128),
            (d.a_row[i][h] == kOobPf || past) ? kOobPf : off);
    }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      dma16(d.xr, st + kWStB + (8 * s + w) * kWTileSw + h * (1024 + 128),
            (d.b_row[h] == kOobPf || 2 * J + s >= steps) ? kOobPf : d.b_row[h] + 128u * (2 * J + s) + chunk);
  {
    const int s = w >> 2;
    dma4(d.sr, st + kWStSA + s * 1024 + (w & 3) * 256,
         (d.sa_row == kOobPf || 2 * J + s >= steps) ? kOobPf : d.sa_row + d.sa_step * (uint32_t)(2 * J + s));
  }
  if (l < 32) {
    const int s = l >> 4;
    dma4(d.xsr, st + kWStSB + w * 128,
         (d.sb_row == kOobPf || 2 * J + s >= steps) ? kOobPf : d.sb_row + 4u * (2 * J + s));
  }
}

// The MFMAs of one K step (8 weight tiles x NTT token tiles) and their
// interleave with the step's LDS reads: the token fragments and the first
// weight tiles' reads, then each pair of MFMAs followed by more reads, so
// only the first reads' latency precedes the MFMAs (all reads first measured
// 7 % slower on FC1).  NTT = 2: 22 reads, 16 MFMAs; NTT = 1: 19 and 8.
template <int NTT>
__device__ __forceinline__ void pw_mfmas(const uint4 blo[2], const uint4 bhi[2], const uint32_t sb[2],
                                         const uint4 av[8], const uint32_t sa[8], f32x4 acc[8][2]) {
  uint32_t bf[2][8];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    bf[tt][0] = blo[tt].x; bf[tt][1] = blo[tt].y; bf[tt][2] = blo[tt].z; bf[tt][3] = blo[tt].w;
    bf[tt][4] = bhi[tt].x; bf[tt][5] = bhi[tt].y; bf[tt][6] = bhi[tt].z; bf[tt][7] = bhi[tt].w;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a4[4] = {av[i].x, av[i].y, av[i].z, av[i].w};
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[i][tt] = mfma_scale_fp4_fp8(a4, bf[tt], sa[i], sb[tt], acc[i][tt]);
  }
  if constexpr (NTT == 2) {
    __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  } else {   // one MFMA per weight tile: the reads run four tiles ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 11, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
}

// Token tiles of a wave's 32 rows that hold any row of the group (0, 1 or 2):
// the others are padding of the group's last m-tile, whose MFMAs, and FC1
// epilogue, are skipped (their rows are never stored).
__device__ __forceinline__ int pw_active_tiles(const PfItem& x, int wm) {
  const int left = x.p1 - (x.p0 + 32 * wm);
  return left <= 0 ? 0 : (left <= 16 ? 1 : 2);
}

// Where this lane's weight fragment of K step s (0, 1) of a stage sits in a
// staged tile, and its scale byte in a staged tile's 64 bytes: swizzled rows,
// or lane order (fragment-tiled weights).
struct PwRd {
  uint32_t a[2], s;
};
__device__ __forceinline__ PwRd pw_rd(bool tiled, int lane) {
  const int r = lane & 15, g = lane >> 4, rr = r & 7;
  PwRd d;
#pragma unroll
  for (int s = 0; s < 2; ++s)
    d.a[s] = tiled ? (uint32_t)(s * (1024 + 128) + 16 * lane)
                   : (uint32_t)((r >> 3) * (1024 + 128) + rr * 128 + 16 * ((4 * s + g) ^ rr));
  d.s = tiled ? (uint32_t)(16 * g + r) : (uint32_t)(4 * r + g);
  return d;
}

// K step s of a stage for one wave: 8 weight tiles x NTT token tiles of MFMAs.
template <int NTT>
__device__ __forceinline__ void pw_compute(const uint8_t* st, int s, bool fc1, int wn, int wm, int lane,
                                           const PwRd& rd, f32x4 acc[8][2]) {
  const int r = lane & 15, g = lane >> 4, rr = r & 7;
  const int rowoff = (r >> 3) * (1024 + 128) + rr * 128;
  uint4 blo[2], bhi[2];
  uint32_t sb[2];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int tile = 2 * wm + tt;
    const uint8_t* row = st + kWStB + (8 * s + tile) * kWTileSw + rowoff;
    blo[tt] = *reinterpret_cast<const uint4*>(row + 16 * (g ^ rr));
    bhi[tt] = *reinterpret_cast<const uint4*>(row + 16 * ((4 + g) ^ rr));
    sb[tt] = st[kWStSB + tile * 128 + s * 64 + r * 4 + g];
  }
  uint4 av[8];
  uint32_t sa[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tile = fc1 ? (i < 4 ? 4 * wn + i : 8 + 4 * wn + (i - 4)) : 8 * wn + i;
    av[i] = *reinterpret_cast<const uint4*>(st + kWStA + tile * kWTileSw + rd.a[s]);
    sa[i] = st[kWStSA + s * 1024 + tile * 64 + rd.s];
  }
  pw_mfmas<NTT>(blo, bhi, sb, av, sa, acc);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// A store whose data comes from LDS reads (not from an MFMA), so no VALU
// pass is needed before it; wait states after it cover its late read of
// the data registers.
__device__ __forceinline__ void st16u(const v4i& r, uint32_t voff, u32x4 v) {
  asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen\n\ts_nop 3" ::"v"(v), "v"(voff), "s"(r) : "memory");
}

// FC2 epilogue of the wide kernel's 128 x 32 wave tile: fp16 y with one
// exponent per 64 columns of a row.  For each 16-token x 64-column block the
// row maximum (over the 4 lanes that share a token), the exponent and the
// fp16 codes are made in the MFMA layout; the codes then go through the
// wave's LDS scratch (16 rows of 144 bytes) so that a row store covers 8
// tokens x 128 contiguous bytes, and the block's 16 exponent bytes leave in
// one store: 12 stores per wave and item.  The rows and exponents are made
// at the item's end (pw_y16_prepare) but their stores leave four at a time
// during the next item's first K steps (pw_y16_store), so that they drain
// while the matrix cores run instead of stalling all eight waves at once.
constexpr int kWYPitch = 128 + 16;
constexpr int kWYScratch = 16 * kWYPitch;
struct YPend {
  u32x4 rows[8];     // [2 * block + k]
  uint32_t e[4];     // exponent of token r's row segment, per block
};
// TT, TT0: token tiles TT0, TT0 + 1 of an [8][TT] accumulator set.
template <int TT = 2, int TT0 = 0>
__device__ __forceinline__ void pw_y16_prepare(f32x4 (&acc)[8][TT], int lane, uint8_t* scratch, YPend& yp) {
  const int r = lane & 15, g = lane >> 4;
  const int t8 = lane >> 3, c8 = lane & 7;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(acc[4 * half + i][TT0 + tt][e]));
      m = fmaxf(m, __shfl_xor(m, 16, kWave));       // columns past H hold zeros
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      const int ex = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xffu) - 127;   // floor(log2 m)
      const int E = min(max(ex + 113, 1), 254);
      const float inv = __builtin_bit_cast(float, (uint32_t)(254 - E) << 23);        // 2^(127 - E)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 v = acc[4 * half + i][TT0 + tt];
        const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)(v[0] * inv));
        const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)(v[1] * inv));
        const uint32_t h2 = __builtin_bit_cast(uint16_t, (_Float16)(v[2] * inv));
        const uint32_t h3 = __builtin_bit_cast(uint16_t, (_Float16)(v[3] * inv));
        // token r, columns 16i + 4g .. +3 of the block
        *reinterpret_cast<uint2*>(scratch + r * kWYPitch + 32 * i + 8 * g) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
      }
      const int blk = 2 * tt + half;
#pragma unroll
      for (int k = 0; k < 2; ++k) yp.rows[2 * blk + k] = *reinterpret_cast<const u32x4*>(scratch + (8 * k + t8) * kWYPitch + 16 * c8);
      yp.e[blk] = (uint32_t)E;
    }
}
// Stores 4 PART .. 4 PART + 3 of the 12: per block, two row stores (8 tokens
// each) and the exponent store.  NROWS: weight rows (y columns) of a work
// item; tok0: the first of the 32 tokens (within the m-tile) held in yp.
template <int PART, int NROWS = kWRows>
__device__ __forceinline__ void pw_y16_store(const GemmArgs& a, const PfItem& x, const YPend& yp, int wn, int tok0,
                                             int lane) {
  const int r = lane & 15, g = lane >> 4;
  const int t8 = lane >> 3, c8 = lane & 7;
  const int H = a.N, n0 = x.nt * NROWS;
  const int nb64 = (H + 63) / 64;
  const v4i yr = rsrc4(static_cast<uint16_t*>(a.out) + (size_t)x.p0 * H, (uint32_t)(kWTok * H * 2));
  const v4i er = rsrc4(a.out_scale, (uint32_t)nb64 * (uint32_t)a.out_rows);
#pragma unroll
  for (int j = 4 * PART; j < 4 * PART + 4; ++j) {
    const int blk = j / 3, kind = j % 3, tt = blk >> 1, half = blk & 1;
    const int col0 = n0 + 128 * wn + 64 * half;
    if (kind < 2) {
      const int pr = tok0 + 16 * tt + 8 * kind + t8;
      const int col = col0 + 8 * c8;
      const bool ok = x.p0 + pr < x.p1 && col < H;
      st16u(yr, ok ? (uint32_t)(pr * H + col) * 2u : kOobPf, yp.rows[2 * blk + kind]);
    } else {
      const int pe = tok0 + 16 * tt + r;
      const bool oke = g == 0 && x.p0 + pe < x.p1 && col0 < H;
      st1(er, oke ? (uint32_t)(x.p0 + pe) * (uint32_t)nb64 + (uint32_t)(col0 / 64) : kOobPf, yp.e[blk]);
    }
  }
}

// Item -> expert, n-tile and pair range (128-row routing tiles, exact ranges
// from the router's table); items ordered expert-major, m-tiles fastest.
__device__ __forceinline__ PfItem pw_item(const GemmArgs& a, int it, int n_tiles) {
  const cptr te = (cptr)a.tile_expert, mt = (cptr)a.mtiles, tr = (cptr)a.tile_rows;
  PfItem x;
  x.l = te[it / n_tiles];
  const int m0 = mt[x.l], m_l = mt[x.l + 1] - m0;
  const int rr = it - m0 * n_tiles;
  x.nt = rr / m_l;
  const int m = m0 + rr % m_l;
  x.p0 = tr[2 * m];
  x.p1 = tr[2 * m + 1];
  return x;
}

}  // namespace

template <bool FC1, bool GEN = false>
__global__ __launch_bounds__(kWThreads, 1) void prefill_wide_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t st0[kWStage];
  __shared__ __align__(16) uint8_t st1[kWStage];
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wn = wave & 1, wm = wave >> 1;
  const int K = a.K, steps = K / 128, n_st = (steps + 1) / 2;
  const int n_tiles = FC1 ? a.N / 128 : (a.N + kWRows - 1) / kWRows;
  const int total = ((cptr)a.mtiles)[a.E_l] * n_tiles;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd_wgs = (gridDim.x + 7 - xcd) / 8;
  const int chunk = (total + 7) / 8;
  const int i_begin = xcd * chunk, i_end = min(total, i_begin + chunk);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const PwRd rd = pw_rd(a.tiled != 0, lane);

  // Two stages per item: stage 0 is requested before the previous item's
  // output stores (so its latency overlaps them), stage J + 1 while stage J
  // is multiplied.
  int it = i_begin + slot;
  PfItem cur{0, 0, 0, 0};
  PwGeo d{};
  if (it < i_end) {
    cur = pw_item(a, it, n_tiles);
    d = pw_geo<FC1>(a, cur, pf_act_rows<FC1>(a, cur, wave_u, lane), wave, lane);
    lds_barrier();
    pw_issue(lds_addr_of(st0), d, 0);
  }
  // FC2: the previous item's y stores leave during this item's first K steps
  // (before the stage requests when an item has three or more stages)
  bool pend = false;
  PfItem px{0, 0, 0, 0};
  YPend yp;
  for (; it < i_end; it += per_xcd_wgs) {
    const int it_next = it + per_xcd_wgs;
    PfItem nxt{0, 0, 0, 0};
    PfRows trow2{-1, -1, -1};
    if (it_next < i_end) {
      nxt = pw_item(a, it_next, n_tiles);
      trow2 = pf_act_rows<FC1>(a, nxt, wave_u, lane);
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ntt = pw_active_tiles(cur, wm);   // uniform per wave
    for (int J0 = 0; J0 < n_st; J0 += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int J = J0 + u;
        if (J < n_st) {
          dma_barrier<0>();                                  // stage J has landed everywhere
          if constexpr (!FC1) {
            if (pend) {
              if (J == 0) pw_y16_store<0>(a, px, yp, wn, 32 * wm, lane);
              else if (J == 1) {
                if (n_st >= 3) pw_y16_store<1>(a, px, yp, wn, 32 * wm, lane);
                else pw_y16_store<2>(a, px, yp, wn, 32 * wm, lane);
              }
              else if (J == 2) pw_y16_store<2>(a, px, yp, wn, 32 * wm, lane);
            }
          }
          if (J + 1 < n_st) pw_issue(lds_addr_of(u ? st0 : st1), d, J + 1);
          const uint8_t* stc = u ? st1 : st0;
          if (ntt == 2) pw_compute<2>(stc, 0, FC1, wn, wm, lane, rd, acc);
          else if (ntt == 1) pw_compute<1>(stc, 0, FC1, wn, wm, lane, rd, acc);
          if constexpr (!FC1) {
            if (pend && J == 0 && n_st < 3) pw_y16_store<1>(a, px, yp, wn, 32 * wm, lane);
          }
          if (2 * J + 1 < steps) {
            if (ntt == 2) pw_compute<2>(stc, 1, FC1, wn, wm, lane, rd, acc);
            else if (ntt == 1) pw_compute<1>(stc, 1, FC1, wn, wm, lane, rd, acc);
          }
        }
      }
    }
    if constexpr (!FC1) {
      if (pend && n_st < 2) pw_y16_store<2>(a, px, yp, wn, 32 * wm, lane);
    }

    // every wave is done with the stages: request the next item's first one
    lds_barrier();
    if (it_next < i_end) {
      d = pw_geo<FC1>(a, nxt, trow2, wave, lane);
      pw_issue(lds_addr_of(st0), d, 0);
    }
    // the second stage is free for FC2's output transpose
    if constexpr (FC1) {
      pf_epilogue<true, kWTok, 128, 2, GEN>(a, cur, acc, wn, wm, wave, lane, nullptr, ntt);
    } else {
      pw_y16_prepare(acc, lane, st1 + wave * kWYScratch, yp);
      px = cur;
      pend = true;
      if (it_next >= i_end) {        // the last item: nothing to hide the stores behind
        pw_y16_store<0>(a, px, yp, wn, 32 * wm, lane);
        pw_y16_store<1>(a, px, yp, wn, 32 * wm, lane);
        pw_y16_store<2>(a, px, yp, wn, 32 * wm, lane);
      }
    }
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// FC1 with 512 weight rows per work item, for fragment-tiled weights and an
// intermediate size that is a multiple of 256 (the EP shards, I = 3072).  A
// work item is 256 gate columns with their 256 up rows x 128 tokens of one
// expert: per 128-wide K step 32 KB of E2M1 weights and 16 KB of E4M3
// activations, 25 % fewer staged bytes per MFMA than the 256-row kernel.
// From tiled weights each weight request is 1 KB of contiguous memory and
// each scale request 4 tiles x 64 contiguous bytes; from rows the same
// stages cost the address unit a cache-line lookup per row (16 per weight
// request, 64 per scale request), and the 512-row item then ran no faster
// than the 256-row one.  8 waves, each 64 gate + 64 up rows x 64 tokens =
// 8 x 4 tiles of v_mfma_scale_f32_16x16x128_f8f6f4.  Stages hold one K step
// (52.5 KB), three in a ring.  FC1 runs the pipelined K loop below (the
// barrier in mid-step, the next step's fragments read behind the current
// step's MFMAs, the stage requests spread between them); the ring restarts
// with every work item: its first three stages are requested once every
// wave is past the previous item's last step (before that item's epilogue),
// every wave issues 8 requests per stage (out of range past the item's last
// stage), each stage is certified before it is read, and the kernel waits
// for all of its requests before it exits.  FC2 keeps the simpler loop (its
// y transpose needs the third buffer after the last step): two stages ahead,
// the barrier at each step's start.  Weights land as they are stored (lane
// l's 16 bytes at 16 l of a tile), activations in the 256-row kernel's
// swizzled tiles.  Same MFMA operands per 16 x 16 tile and K order as the
// 256-row kernel, so the same h bit for bit.
namespace {

constexpr int kBRows = 512, kBTok = 128, kBThreads = 512;
constexpr int kBStA = 0;                              // 32 weight tiles of 1 KB, lane order
constexpr int kBStB = kBStA + 32 * 1024;              // 8 token tiles (swizzled, kWTileSw each)
constexpr int kBStSA = kBStB + 8 * kWTileSw;          // 32 weight tiles x 64 E8M0 bytes, lane order
constexpr int kBStSB = kBStSA + kBRows * 4;           // 128 tokens x 4 bytes
constexpr int kBStage = kBStSB + kBTok * 4;           // 53760 bytes
constexpr int kBStages = 3;
constexpr int kBDmas = 8;                             // DMAs per wave per stage
static_assert(kBStages * kBStage <= 160 * 1024, "stage ring fits the LDS");

struct PbGeo {
  v4i wr, sr, xr, xsr;
  uint32_t a_row[4];   // this lane's 16 bytes of each of the wave's 4 weight tiles at K step 0
  uint32_t sa_row;     // this lane's scale dword at K step 0 (tile 4 wave + l/16)
  uint32_t b_row[2];   // activation rows of tokens l/8 and 8 + l/8 of the wave's token tile (kOobPf: none)
  uint32_t sb_row;     // scale row offset of token l%16 of the tile (kOobPf: none)
  int wave, lane, K;
};

// Item row t (0..511) -> weight row.  FC1: t < 256 gate column n0 + t, else
// up row I + n0 + t - 256; FC2: row n0 + t (rows past H read zeros).
template <bool FC1>
__device__ __forceinline__ int pb_wrow(const GemmArgs& a, int n0, int t) {
  return FC1 ? (t < 256 ? n0 + t : a.N + n0 + (t - 256)) : n0 + t;
}

template <bool FC1>
__device__ __forceinline__ PbGeo pb_geo(const GemmArgs& a, const PfItem& x, const PfRows& tr, int wave, int lane) {
  const int K = a.K, nkb = K / 32, S = tiled_steps(K);
  const int n_rows = FC1 ? 2 * a.N : a.N;
  PbGeo d;
  d.wave = wave;
  d.lane = lane;
  d.K = K;
  const size_t wexp = expert_w_bytes(true, n_rows, K);
  const size_t sexp = (size_t)n_rows * scale_row_bytes(false, true, K);
  d.wr = rsrc4(a.w + (size_t)x.l * wexp, (uint32_t)wexp);
  d.sr = rsrc4(a.ws + (size_t)x.l * sexp, (uint32_t)sexp);
  const int n0 = x.nt * (FC1 ? 256 : kBRows);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row0 = pb_wrow<FC1>(a, n0, 16 * (4 * wave + i));
    d.a_row[i] = row0 < n_rows ? (uint32_t)(row0 / 16) * (uint32_t)S * 1024u + (uint32_t)lane * 16u : kOobPf;
  }
  const int srow0 = pb_wrow<FC1>(a, n0, 16 * (4 * wave + (lane >> 4)));
  d.sa_row = srow0 < n_rows ? (uint32_t)(srow0 / 16) * (uint32_t)S * 64u + (uint32_t)(lane & 15) * 4u : kOobPf;
  d.xr = rsrc4(a.act, 0x7fffffff);
  d.xsr = rsrc4(a.act_scale, 0x7fffffff);
  d.b_row[0] = tr.t_a >= 0 ? (uint32_t)tr.t_a * (uint32_t)K : kOobPf;
  d.b_row[1] = tr.t_b >= 0 ? (uint32_t)tr.t_b * (uint32_t)K : kOobPf;
  d.sb_row = tr.t_s >= 0 ? (uint32_t)tr.t_s * (uint32_t)nkb : kOobPf;
  return d;
}

// This wave's kBDmas DMAs of K step j into stage `st`: weight tiles 4w..4w+3
// (1 KB each), the two 8-token halves of token tile w, the scales of weight
// tiles 4w..4w+3 (64 bytes each) and of the tile's 16 tokens (lanes 0..15).
__device__ __forceinline__ void pb_issue(uint32_t st, const PbGeo& d, int j) {
  const int w = d.wave, l = d.lane;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dma16(d.wr, st + kBStA + (4 * w + i) * 1024, d.a_row[i] == kOobPf ? kOobPf : d.a_row[i] + 1024u * (uint32_t)j);
  const uint32_t chunk = (uint32_t)(((l & 7) ^ (l >> 3)) * 16);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    dma16(d.xr, st + kBStB + w * kWTileSw + h * (1024 + 128),
          d.b_row[h] == kOobPf ? kOobPf : d.b_row[h] + 128u * j + chunk);
  dma4(d.sr, st + kBStSA + w * 256, d.sa_row == kOobPf ? kOobPf : d.sa_row + 64u * (uint32_t)j);
  if (l < 16) dma4(d.xsr, st + kBStSB + w * 64, d.sb_row == kOobPf ? kOobPf : d.sb_row + 4u * j);
}

// The DMAs of the pipelined FC1 loop.  A wave's four weight tiles are one
// contiguous run of rows, so their requests share one vector offset (16 per
// lane) and differ by a scalar offset, as do its scale requests; only the
// token rows (routed, per lane) need vector offsets of their own.
struct PbDma {
  v4i wr, sr, xr, xsr;
  uint32_t w_soff;     // the wave's first weight tile at K step 0 (uniform)
  uint32_t tile_b;     // bytes of one 16-row tile's E2M1 over all K steps (uniform)
  uint32_t sa_soff;    // its scale block at K step 0 (uniform)
  uint32_t w_lane;     // 16 lane
  uint32_t sa_lane;    // (lane / 16) row tiles + 4 (lane % 16) bytes into a scale block
  uint32_t b_row[2];   // token rows l/8 and 8 + l/8 of the wave's token tile, plus the lane's swizzled chunk (kOobPf: none)
  uint32_t sb_row;     // scale row of token l%16 of the tile (kOobPf: none)
  int wave, lane;
};

__device__ __forceinline__ PbDma pb_dma_geo(const GemmArgs& a, const PfItem& x, const PfRows& tr, int wave, int lane) {
  const int K = a.K, nkb = K / 32, S = tiled_steps(K);
  const int n_rows = 2 * a.N;
  PbDma d;
  d.wave = wave;
  d.lane = lane;
  const size_t wexp = expert_w_bytes(true, n_rows, K);
  const size_t sexp = (size_t)n_rows * scale_row_bytes(false, true, K);
  d.wr = rsrc4(a.w + (size_t)x.l * wexp, (uint32_t)wexp);
  d.sr = rsrc4(a.ws + (size_t)x.l * sexp, (uint32_t)sexp);
  // item rows 64 w .. 64 w + 63: gate columns (w < 4) or up rows, all within the matrix
  const int rt0 = pb_wrow<true>(a, x.nt * 256, 64 * wave) / 16;
  d.tile_b = (uint32_t)S * 1024u;
  d.w_soff = (uint32_t)rt0 * d.tile_b;
  d.sa_soff = (uint32_t)rt0 * (uint32_t)S * 64u;
  d.w_lane = (uint32_t)lane * 16u;
  d.sa_lane = (uint32_t)(lane >> 4) * (uint32_t)S * 64u + (uint32_t)(lane & 15) * 4u;
  d.xr = rsrc4(a.act, 0x7fffffff);
  d.xsr = rsrc4(a.act_scale, 0x7fffffff);
  const uint32_t chunk = (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
  d.b_row[0] = tr.t_a >= 0 ? (uint32_t)tr.t_a * (uint32_t)K + chunk : kOobPf;
  d.b_row[1] = tr.t_b >= 0 ? (uint32_t)tr.t_b * (uint32_t)K + chunk : kOobPf;
  d.sb_row = tr.t_s >= 0 ? (uint32_t)tr.t_s * (uint32_t)nkb : kOobPf;
  return d;
}

// This wave's DMAs of K step j into the stage at LDS address st, one at a
// time: q = 0..3 weight tiles 4w..4w+3 (1 KB each), 4 and 5 the two 8-token
// halves of token tile w, 6 the weight tiles' scales (64 bytes each); the
// token tile's scales (lanes 0..15) by pb_dma_xs.  Same destinations and
// bytes as pb_issue.  With live false the requests are out of range: they
// write zeros to the same destinations and count like the others (a stage
// past the item's last keeps every wave's request count, so its waits, the
// same at every step).
template <int Q>
__device__ __forceinline__ void pb_dma(uint32_t st, const PbDma& d, int j, bool live) {
  const int w = d.wave;
  if constexpr (Q < 4) {
    dma16s(d.wr, st + kBStA + (4 * w + Q) * 1024, live ? d.w_lane : kOobPf,
           d.w_soff + (uint32_t)Q * d.tile_b + 1024u * (uint32_t)j);
  } else if constexpr (Q < 6) {
    dma16s(d.xr, st + kBStB + w * kWTileSw + (Q - 4) * (1024 + 128), live ? d.b_row[Q - 4] : kOobPf,
           128u * (uint32_t)j);
  } else {
    dma4s(d.sr, st + kBStSA + w * 256, live ? d.sa_lane : kOobPf, d.sa_soff + 64u * (uint32_t)j);
  }
}
__device__ __forceinline__ void pb_dma_xs(uint32_t st, const PbDma& d, int j, bool live) {
  if (d.lane < 16) dma4s(d.xsr, st + kBStSB + d.wave * 64, live ? d.sb_row : kOobPf, 4u * (uint32_t)j);
}
__device__ __forceinline__ void pb_dma_all(uint32_t st, const PbDma& d, int j, bool live) {
  pb_dma<0>(st, d, j, live);
  pb_dma<1>(st, d, j, live);
  pb_dma<2>(st, d, j, live);
  pb_dma<3>(st, d, j, live);
  pb_dma<4>(st, d, j, live);
  pb_dma<5>(st, d, j, live);
  pb_dma<6>(st, d, j, live);
  pb_dma_xs(st, d, j, live);
}

// One K step of one wave from stage `st`: weight tiles (FC1: gate 4wn..4wn+3,
// up 16+4wn..; FC2: 8wn..8wn+7), token tiles 4wm..4wm+NTT-1; the reads are
// interleaved with the MFMAs so only the first ones' latency precedes them.
template <bool FC1, int NTT>
__device__ __forceinline__ void pb_compute(const uint8_t* st, int wn, int wm, int lane, f32x4 acc[8][4]) {
  const int r = lane & 15, g = lane >> 4, rr = r & 7;
  const int rowoff = (r >> 3) * (1024 + 128) + rr * 128;
  uint32_t bf[NTT][8];
  uint32_t sb[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int tile = 4 * wm + tt;
    const uint8_t* row = st + kBStB + tile * kWTileSw + rowoff;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + 16 * (g ^ rr));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + 16 * ((4 + g) ^ rr));
    bf[tt][0] = lo.x; bf[tt][1] = lo.y; bf[tt][2] = lo.z; bf[tt][3] = lo.w;
    bf[tt][4] = hi.x; bf[tt][5] = hi.y; bf[tt][6] = hi.z; bf[tt][7] = hi.w;
    sb[tt] = st[kBStSB + (16 * tile + r) * 4 + g];
  }
  // weight tiles stream through a window of three register sets: tile i + 2
  // is read while tile i's MFMAs run
  auto a_tile = [&](int i) { return FC1 ? (i < 4 ? 4 * wn + i : 16 + 4 * wn + (i - 4)) : 8 * wn + i; };
  uint4 av[3];
  uint32_t sa[3];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    av[i] = *reinterpret_cast<const uint4*>(st + kBStA + a_tile(i) * 1024 + 16 * lane);
    sa[i] = st[kBStSA + a_tile(i) * 64 + 16 * g + r];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i + 2 < 8) {
      av[(i + 2) % 3] = *reinterpret_cast<const uint4*>(st + kBStA + a_tile(i + 2) * 1024 + 16 * lane);
      sa[(i + 2) % 3] = st[kBStSA + a_tile(i + 2) * 64 + 16 * g + r];
    }
    const uint32_t a4[4] = {av[i % 3].x, av[i % 3].y, av[i % 3].z, av[i % 3].w};
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[i][tt] = mfma_scale_fp4_fp8(a4, bf[tt], sa[i % 3], sb[tt], acc[i][tt]);
  }
  // token fragments and the first two weight tiles' reads, then the MFMAs of
  // each weight tile behind the reads of the tile two ahead
  __builtin_amdgcn_sched_group_barrier(0x100, 3 * NTT + 4, 0);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NTT, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * NTT, 0);
}

// The pipelined K loop of the 512-row FC1 kernel.  A wave keeps all 8 of its
// weight tiles and its 4 token tiles of a K step in registers and runs the
// step in two halves: the MFMAs of token tiles 0 and 1 with every weight
// tile (while token tiles 2 and 3 are read), then, after the workgroup
// barrier, those of token tiles 2 and 3, each weight tile's registers being
// refilled with the next step's tile right after their last MFMA, and token
// tiles 0 and 1 with the next step's at the half's start.  The barrier sits
// where every read of stage j is done (its buffer is then free for stage
// j + 3) and, once this wave's DMAs of stage j + 1 have landed, certifies
// that stage for the reads that follow it.  The matrix cores so have 16
// MFMAs a wave ready across every barrier (where a barrier at the step's
// start left them idle until the first fragments had arrived), and two
// stages stay in flight.  Measured on the EP8 shard: 0.77 ms without the
// stage requests against 0.89 for the step-start barrier, 1.073 ms with
// them against 1.092.
struct PbTok {
  uint32_t bf[8];
  uint32_t sb;
};
struct PbW {
  uint32_t a[4];
  uint32_t sa;
};

// A lane's fragment offsets within a stage (fixed for the kernel): weight
// tile 0 of its wave column and that tile's scale byte, the low and high
// 16 bytes of its row of token tile 4 wm and that row's scale byte.  Tile
// i of the column is then a constant offset away, and a read is one base
// register plus an immediate.
struct PbLane {
  uint32_t w, sa, tlo, thi, sb;
};

template <bool FC1>
__device__ __forceinline__ PbLane pb_lane(int wn, int wm, int lane) {
  const int r = lane & 15, g = lane >> 4, rr = r & 7;
  const int t0 = FC1 ? 4 * wn : 8 * wn;
  const int row = kBStB + 4 * wm * kWTileSw + (r >> 3) * (1024 + 128) + rr * 128;
  return PbLane{(uint32_t)(kBStA + t0 * 1024 + 16 * lane), (uint32_t)(kBStSA + t0 * 64 + 16 * g + r),
                (uint32_t)(row + 16 * (g ^ rr)), (uint32_t)(row + 16 * ((4 + g) ^ rr)),
                (uint32_t)(kBStSB + (64 * wm + r) * 4 + g)};
}

// Weight tile i (0..7) of a wave column, relative to its tile 0: FC1 gate
// tiles 4wn.. then up tiles 16 + 4wn..; FC2 tiles 8wn..
template <bool FC1>
__device__ __forceinline__ constexpr int pb_a_rel(int i) {
  return FC1 ? (i < 4 ? i : 12 + i) : i;
}

// token tile tt (0..3) of the wave from the stage at `st`
__device__ __forceinline__ void pb_read_tok(const uint8_t* st, const PbLane& o, int tt, PbTok& t) {
  const uint4 lo = *reinterpret_cast<const uint4*>(st + o.tlo + tt * kWTileSw);
  const uint4 hi = *reinterpret_cast<const uint4*>(st + o.thi + tt * kWTileSw);
  t.bf[0] = lo.x; t.bf[1] = lo.y; t.bf[2] = lo.z; t.bf[3] = lo.w;
  t.bf[4] = hi.x; t.bf[5] = hi.y; t.bf[6] = hi.z; t.bf[7] = hi.w;
  t.sb = st[o.sb + tt * 64];
}

template <bool FC1>
__device__ __forceinline__ void pb_read_w(const uint8_t* st, const PbLane& o, int i, PbW& w) {
  const uint4 v = *reinterpret_cast<const uint4*>(st + o.w + pb_a_rel<FC1>(i) * 1024);
  w.a[0] = v.x; w.a[1] = v.y; w.a[2] = v.z; w.a[3] = v.w;
  w.sa = st[o.sa + pb_a_rel<FC1>(i) * 64];
}

__device__ __forceinline__ f32x4 pb_mfma(const PbW& w, const PbTok& t, f32x4 acc) {
  return mfma_scale_fp4_fp8(w.a, t.bf, w.sa, t.sb, acc);
}

// The barrier in step j (a step follows): stage j + 1 has landed (the only
// requests this wave issued after it are the 8 for stage j + 2, real or
// past the item's end, besides, at step 0, the previous item's epilogue
// stores, which only lengthen the wait) and every wave is done reading stage
// j, whose buffer then takes stage j + 3.
__device__ __forceinline__ void pb_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  dma_barrier<kBDmas>();
}

// The first half of a step: token tiles 2 and 3 read, the MFMAs of tiles 0
// and 1 with every weight tile.
__device__ __forceinline__ void pb_half0(const uint8_t* stc, const PbLane& o, PbTok (&tok)[4], const PbW (&w)[8],
                                         f32x4 (&acc)[8][4]) {
  pb_read_tok(stc, o, 2, tok[2]);
  pb_read_tok(stc, o, 3, tok[3]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i][0] = pb_mfma(w[i], tok[0], acc[i][0]);
    acc[i][1] = pb_mfma(w[i], tok[1], acc[i][1]);
  }
  // the six reads first, then the sixteen MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
}

// The second half of a step that another follows: the MFMAs of token tiles
// 2 and 3, each weight tile's registers refilled from the next stage (stn)
// after its last MFMA, and between them this wave's DMAs 0..6 of stage
// j + 3 (live when it exists) into st_free, one per weight tile, so that the
// address unit takes them while the matrix cores run (issued back to back
// they filled its queue, and a wave waiting to issue one could issue no
// MFMA).
template <bool FC1>
__device__ __forceinline__ void pb_half1(const uint8_t* stn, const PbLane& o, const PbTok (&tok)[4], PbW (&w)[8],
                                         f32x4 (&acc)[8][4], uint32_t st_free, const PbDma& d, int j3, bool live) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i][2] = pb_mfma(w[i], tok[2], acc[i][2]);
    acc[i][3] = pb_mfma(w[i], tok[3], acc[i][3]);
    pb_read_w<FC1>(stn, o, i, w[i]);
    if (i == 0) pb_dma<0>(st_free, d, j3, live);
    if (i == 1) pb_dma<1>(st_free, d, j3, live);
    if (i == 2) pb_dma<2>(st_free, d, j3, live);
    if (i == 3) pb_dma<3>(st_free, d, j3, live);
    if (i == 4) pb_dma<4>(st_free, d, j3, live);
    if (i == 5) pb_dma<5>(st_free, d, j3, live);
    if (i == 6) pb_dma<6>(st_free, d, j3, live);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// The item's stages 0..2 (live where they exist), requested into stage
// buffers 0..2 of the ring at `ring` once every wave is done with the
// previous item's stages.
__device__ __forceinline__ void pb_issue_first(uint32_t ring, const PbDma& d, int steps) {
  pb_dma_all(ring, d, 0, true);
  pb_dma_all(ring + kBStage, d, 1, steps > 1);
  pb_dma_all(ring + 2 * kBStage, d, 2, steps > 2);
}

// The K loop of one item over the ring of three stages at `ring` (stage j
// in buffer j mod 3).  First stage 0 is certified (the requests of stages 1
// and 2 are newer than its own, besides the previous item's epilogue
// stores, which only lengthen the wait) and its weight tiles and token tiles
// 0 and 1 are read.  Every wave takes the same barriers and issues the same
// requests, active or not.
template <bool FC1>
__device__ __forceinline__ void pb_k_loop(uint8_t* ring, const PbDma& d, const PbLane& o, int steps, bool active,
                                          f32x4 (&acc)[8][4]) {
  dma_barrier<2 * kBDmas>();
  const uint32_t ring_addr = lds_addr_of(ring);
  if (!active) {   // a wave with no token rows in the group: its barriers and DMAs only
    for (int j = 0, bc = 0; j + 1 < steps; ++j, bc = bc == 2 ? 0 : bc + 1) {
      pb_barrier();
      pb_dma_all(ring_addr + bc * kBStage, d, j + 3, j + 3 < steps);
    }
    return;
  }
  PbTok tok[4];
  PbW w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pb_read_w<FC1>(ring, o, i, w[i]);
  pb_read_tok(ring, o, 0, tok[0]);
  pb_read_tok(ring, o, 1, tok[1]);
  int bc = 0;   // stage j's buffer
  for (int j = 0; j + 1 < steps; ++j) {
    const int bn = bc == 2 ? 0 : bc + 1;
    const uint8_t* stn = ring + bn * kBStage;
    const uint32_t st_free = ring_addr + bc * kBStage;
    const bool live = j + 3 < steps;
    pb_half0(ring + bc * kBStage, o, tok, w, acc);
    pb_barrier();
    pb_read_tok(stn, o, 0, tok[0]);
    pb_read_tok(stn, o, 1, tok[1]);
    pb_dma_xs(st_free, d, j + 3, live);
    pb_half1<FC1>(stn, o, tok, w, acc, st_free, d, j + 3, live);
    bc = bn;
  }
  // the last step
  pb_half0(ring + bc * kBStage, o, tok, w, acc);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i][2] = pb_mfma(w[i], tok[2], acc[i][2]);
    acc[i][3] = pb_mfma(w[i], tok[3], acc[i][3]);
  }
}

// Token tiles of a wave's 64 rows that hold any row of the group (0 to 4).
__device__ __forceinline__ int pb_active_tiles(const PfItem& x, int wm) {
  const int left = x.p1 - (x.p0 + 64 * wm);
  return left <= 0 ? 0 : (left >= 64 ? 4 : (left + 15) / 16);
}

}  // namespace

template <bool GEN>
__global__ __launch_bounds__(kBThreads, 1) void prefill_fc1_512_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t ring[kBStages * kBStage];
  const int tid = threadIdx.x;
  // the wave index made visibly uniform, so that per-wave choices (its
  // active token tiles) are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int wn = wave & 3, wm = wave >> 2;
  const int K = a.K, steps = K / 128;
  const int n_tiles = a.N / 256;
  const int total = ((cptr)a.mtiles)[a.E_l] * n_tiles;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd_wgs = (gridDim.x + 7 - xcd) / 8;
  const int chunk = (total + 7) / 8;
  const int i_begin = xcd * chunk, i_end = min(total, i_begin + chunk);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  int it = i_begin + slot;
  PfItem cur{0, 0, 0, 0};
  PbDma d{};
  if (it < i_end) {
    cur = pw_item(a, it, n_tiles);
    d = pb_dma_geo(a, cur, pf_act_rows<true>(a, cur, wave_u, lane), wave, lane);
    lds_barrier();
    pb_issue_first(lds_addr_of(ring), d, steps);
  }
  const PbLane o = pb_lane<true>(wn, wm, lane);
  for (; it < i_end; it += per_xcd_wgs) {
    const int it_next = it + per_xcd_wgs;
    PfItem nxt{0, 0, 0, 0};
    PfRows trow2{-1, -1, -1};
    if (it_next < i_end) {
      nxt = pw_item(a, it_next, n_tiles);
      trow2 = pf_act_rows<true>(a, nxt, wave_u, lane);
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[i][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ntt = pb_active_tiles(cur, wm);     // uniform per wave
    pb_k_loop<true>(ring, d, o, steps, ntt > 0, acc);

    // every wave is done with the stages: request the next item's first three
    lds_barrier();
    if (it_next < i_end) {
      d = pb_dma_geo(a, nxt, trow2, wave, lane);
      pb_issue_first(lds_addr_of(ring), d, steps);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int nh = min(2, max(0, ntt - 2 * half));   // uniform
      if (nh > 0) pf_epilogue<true, kBTok, 256, 4, GEN>(a, cur, acc, wn, 2 * wm + half, wave, lane, nullptr, nh, 2 * half);
    }
    cur = nxt;
  }
  // the last item's out-of-range requests land before the workgroup leaves
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// FC1 with 384 weight rows per work item, for fragment-tiled weights and an
// intermediate size that is a multiple of 192 but not of 256 (the TP8
// shard, I = 384: two items per m-tile where the 256-row kernel takes three):
// 192 gate columns with their 192 up rows x 128 tokens of one expert, per
// 128-wide K step 24 KB of weights and 16 KB of activations, 17 % fewer
// staged bytes per MFMA than the 256-row item.  8 waves, each 96 gate + 96
// up rows x 32 tokens = 12 x 2 MFMA tiles (three 32-column MXFP8 blocks of h
// per wave); stages of one K step (44 KB), three in a ring, the same
// protocol as the 512-row kernel.  Same MFMA operands per 16 x 16 tile and
// K order as the 256-row kernel, so the same h bit for bit.
namespace {

constexpr int kCTok = 128, kCThreads = 512;
constexpr int kCStA = 0;                              // 24 weight tiles of 1 KB, lane order
constexpr int kCStB = kCStA + 24 * 1024;              // 8 token tiles (swizzled, kWTileSw each)
constexpr int kCStSA = kCStB + 8 * kWTileSw;          // 24 weight tiles x 64 E8M0 bytes, lane order
constexpr int kCStSB = kCStSA + 24 * 64;              // 128 tokens x 4 bytes
constexpr int kCStage = kCStSB + kCTok * 4;           // 45056 bytes
constexpr int kCStages = 3;
constexpr int kCDmas = 7;                             // DMAs per wave per stage
static_assert(kCStages * kCStage <= 160 * 1024, "stage ring fits the LDS");

struct PcGeo {
  v4i wr, sr, xr, xsr;
  uint32_t a_row[3];   // this lane's 16 bytes of each of the wave's 3 weight tiles at K step 0
  uint32_t sa_row;     // lanes 0..47: this lane's scale dword at K step 0 (tile 3 wave + l/16)
  uint32_t b_row[2];   // activation rows of tokens l/8 and 8 + l/8 of the wave's token tile (kOobPf: none)
  uint32_t sb_row;     // scale row offset of token l%16 of the tile (kOobPf: none)
  int wave, lane;
};

// Item tile t (0..23) -> first weight row: t < 12 gate columns n0 + 16 t, else up rows I + n0 + 16 (t - 12).
__device__ __forceinline__ int pc_wrow(const GemmArgs& a, int n0, int t) {
  return t < 12 ? n0 + 16 * t : a.N + n0 + 16 * (t - 12);
}

__device__ __forceinline__ PcGeo pc_geo(const GemmArgs& a, const PfItem& x, const PfRows& tr, int wave, int lane) {
  const int K = a.K, nkb = K / 32, S = tiled_steps(K);
  const int n_rows = 2 * a.N;
  PcGeo d;
  d.wave = wave;
  d.lane = lane;
  const size_t wexp = expert_w_bytes(true, n_rows, K);
  const size_t sexp = (size_t)n_rows * scale_row_bytes(false, true, K);
  d.wr = rsrc4(a.w + (size_t)x.l * wexp, (uint32_t)wexp);
  d.sr = rsrc4(a.ws + (size_t)x.l * sexp, (uint32_t)sexp);
  const int n0 = x.nt * 192;
#pragma unroll
  for (int i = 0; i < 3; ++i)
    d.a_row[i] = (uint32_t)(pc_wrow(a, n0, 3 * wave + i) / 16) * (uint32_t)S * 1024u + (uint32_t)lane * 16u;
  d.sa_row = lane < 48 ? (uint32_t)(pc_wrow(a, n0, 3 * wave + (lane >> 4)) / 16) * (uint32_t)S * 64u +
                             (uint32_t)(lane & 15) * 4u
                       : kOobPf;
  d.xr = rsrc4(a.act, 0x7fffffff);
  d.xsr = rsrc4(a.act_scale, 0x7fffffff);
  d.b_row[0] = tr.t_a >= 0 ? (uint32_t)tr.t_a * (uint32_t)K : kOobPf;
  d.b_row[1] = tr.t_b >= 0 ? (uint32_t)tr.t_b * (uint32_t)K : kOobPf;
  d.sb_row = tr.t_s >= 0 ? (uint32_t)tr.t_s * (uint32_t)nkb : kOobPf;
  return d;
}

// This wave's kCDmas DMAs of K step j into stage `st`: weight tiles 3w..3w+2
// (1 KB each), the two 8-token halves of token tile w, the scales of weight
// tiles 3w..3w+2 (64 bytes each, lanes 0..47) and of the tile's 16 tokens
// (lanes 0..15).  The lane-masked requests write only their lanes' bytes.
__device__ __forceinline__ void pc_issue(uint32_t st, const PcGeo& d, int j) {
  const int w = d.wave, l = d.lane;
#pragma unroll
  for (int i = 0; i < 3; ++i) dma16(d.wr, st + kCStA + (3 * w + i) * 1024, d.a_row[i] + 1024u * (uint32_t)j);
  const uint32_t chunk = (uint32_t)(((l & 7) ^ (l >> 3)) * 16);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    dma16(d.xr, st + kCStB + w * kWTileSw + h * (1024 + 128),
          d.b_row[h] == kOobPf ? kOobPf : d.b_row[h] + 128u * j + chunk);
  if (l < 48) dma4(d.sr, st + kCStSA + 3 * w * 64, d.sa_row + 64u * (uint32_t)j);
  if (l < 16) dma4(d.xsr, st + kCStSB + w * 64, d.sb_row == kOobPf ? kOobPf : d.sb_row + 4u * j);
}

// One K step of one wave from stage `st`: weight tiles gate 6wn..6wn+5, up
// 12+6wn.., token tiles 2wm..2wm+NTT-1; the weight tiles stream through a
// window of three register sets, read two ahead of their MFMAs.
template <int NTT>
__device__ __forceinline__ void pc_compute(const uint8_t* st, int wn, int wm, int lane, f32x4 acc[12][2]) {
  const int r = lane & 15, g = lane >> 4, rr = r & 7;
  const int rowoff = (r >> 3) * (1024 + 128) + rr * 128;
  uint32_t bf[NTT][8];
  uint32_t sb[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int tile = 2 * wm + tt;
    const uint8_t* row = st + kCStB + tile * kWTileSw + rowoff;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + 16 * (g ^ rr));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + 16 * ((4 + g) ^ rr));
    bf[tt][0] = lo.x; bf[tt][1] = lo.y; bf[tt][2] = lo.z; bf[tt][3] = lo.w;
    bf[tt][4] = hi.x; bf[tt][5] = hi.y; bf[tt][6] = hi.z; bf[tt][7] = hi.w;
    sb[tt] = st[kCStSB + (16 * tile + r) * 4 + g];
  }
  auto a_tile = [&](int i) { return i < 6 ? 6 * wn + i : 12 + 6 * wn + (i - 6); };
  uint4 av[3];
  uint32_t sa[3];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    av[i] = *reinterpret_cast<const uint4*>(st + kCStA + a_tile(i) * 1024 + 16 * lane);
    sa[i] = st[kCStSA + a_tile(i) * 64 + 16 * g + r];
  }
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    if (i + 2 < 12) {
      av[(i + 2) % 3] = *reinterpret_cast<const uint4*>(st + kCStA + a_tile(i + 2) * 1024 + 16 * lane);
      sa[(i + 2) % 3] = st[kCStSA + a_tile(i + 2) * 64 + 16 * g + r];
    }
    const uint32_t a4[4] = {av[i % 3].x, av[i % 3].y, av[i % 3].z, av[i % 3].w};
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[i][tt] = mfma_scale_fp4_fp8(a4, bf[tt], sa[i % 3], sb[tt], acc[i][tt]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 3 * NTT + 4, 0);
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NTT, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * NTT, 0);
}

}  // namespace

template <bool GEN>
__global__ __launch_bounds__(kCThreads, 1) void prefill_fc1_384_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t sg0[kCStage];
  __shared__ __align__(16) uint8_t sg1[kCStage];
  __shared__ __align__(16) uint8_t sg2[kCStage];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int wn = wave & 1, wm = wave >> 1;
  const int K = a.K, steps = K / 128;
  const int n_tiles = a.N / 192;
  const int total = ((cptr)a.mtiles)[a.E_l] * n_tiles;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd_wgs = (gridDim.x + 7 - xcd) / 8;
  const int chunk = (total + 7) / 8;
  const int i_begin = xcd * chunk, i_end = min(total, i_begin + chunk);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  int it = i_begin + slot;
  PfItem cur{0, 0, 0, 0};
  PcGeo d{};
  if (it < i_end) {
    cur = pw_item(a, it, n_tiles);
    d = pc_geo(a, cur, pf_act_rows<true>(a, cur, wave_u, lane), wave, lane);
    lds_barrier();
    pc_issue(lds_addr_of(sg0), d, 0);
    if (steps > 1) pc_issue(lds_addr_of(sg1), d, 1);
  }
  for (; it < i_end; it += per_xcd_wgs) {
    const int it_next = it + per_xcd_wgs;
    PfItem nxt{0, 0, 0, 0};
    PfRows trow2{-1, -1, -1};
    if (it_next < i_end) {
      nxt = pw_item(a, it_next, n_tiles);
      trow2 = pf_act_rows<true>(a, nxt, wave_u, lane);
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[12][2];
#pragma unroll
    for (int i = 0; i < 12; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ntt = pw_active_tiles(cur, wm);     // uniform per wave
    for (int j0 = 0; j0 < steps; j0 += kCStages) {
#pragma unroll
      for (int u = 0; u < kCStages; ++u) {
        const int j = j0 + u;
        if (j < steps) {
          // step j has landed (the only DMAs this wave issued after it are
          // step j + 1's) and every wave is done reading step j - 1
          if (j + 1 < steps) dma_barrier<kCDmas>();
          else dma_barrier<0>();
          if (j + 2 < steps) pc_issue(lds_addr_of(u == 0 ? sg2 : (u == 1 ? sg0 : sg1)), d, j + 2);
          const uint8_t* stc = u == 0 ? sg0 : (u == 1 ? sg1 : sg2);
          // a wave with one token tile of the group also multiplies the other
          // (zero rows): a second instance of the step, for one tile, would
          // double the registers the kernel needs
          if (ntt > 0) pc_compute<2>(stc, wn, wm, lane, acc);
        }
      }
    }

    // every wave is done with the stages: request the next item's first two
    lds_barrier();
    if (it_next < i_end) {
      d = pc_geo(a, nxt, trow2, wave, lane);
      pc_issue(lds_addr_of(sg0), d, 0);
      if (steps > 1) pc_issue(lds_addr_of(sg1), d, 1);
    }
    pf_epilogue<true, kCTok, 192, 2, GEN, 6>(a, cur, acc, wn, wm, wave, lane, nullptr, ntt);
    cur = nxt;
  }
}

// FC2 with 512 weight rows (y columns) per work item, for fragment-tiled
// weights (the EP shards at K = I = 3072; at K = 384, the TP8 shard, it
// also beats the short-K kernel: 0.745 against 0.80 ms): the FC1 kernel's stages
// and wave tiles (128 rows x 64 tokens per wave), y written fp16 with one
// exponent per 64 columns as in the 256-row kernel.  The y tile of a wave is
// made and stored in two 32-token halves at the item's end, through the
// third stage buffer (free from the last step's reads, which the barrier
// after the K loop closes, to the next item's first barrier).  Same MFMA
// operands per 16 x 16 tile, K order and y arithmetic as the 256-row kernel,
// so the same y bit for bit.
__global__ __launch_bounds__(kBThreads, 1) void prefill_fc2_512_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t sg0[kBStage];
  __shared__ __align__(16) uint8_t sg1[kBStage];
  __shared__ __align__(16) uint8_t sg2[kBStage];
  static_assert(8 * kWYScratch <= kBStage, "the y transpose fits a stage");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int wn = wave & 3, wm = wave >> 2;
  const int K = a.K, steps = K / 128;
  const int n_tiles = (a.N + kBRows - 1) / kBRows;
  const int total = ((cptr)a.mtiles)[a.E_l] * n_tiles;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd_wgs = (gridDim.x + 7 - xcd) / 8;
  const int chunk = (total + 7) / 8;
  const int i_begin = xcd * chunk, i_end = min(total, i_begin + chunk);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  int it = i_begin + slot;
  PfItem cur{0, 0, 0, 0};
  PbGeo d{};
  if (it < i_end) {
    cur = pw_item(a, it, n_tiles);
    d = pb_geo<false>(a, cur, pf_act_rows<false>(a, cur, wave_u, lane), wave, lane);
    lds_barrier();
    pb_issue(lds_addr_of(sg0), d, 0);
    if (steps > 1) pb_issue(lds_addr_of(sg1), d, 1);
  }
  for (; it < i_end; it += per_xcd_wgs) {
    const int it_next = it + per_xcd_wgs;
    PfItem nxt{0, 0, 0, 0};
    PfRows trow2{-1, -1, -1};
    if (it_next < i_end) {
      nxt = pw_item(a, it_next, n_tiles);
      trow2 = pf_act_rows<false>(a, nxt, wave_u, lane);
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[i][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int ntt = pb_active_tiles(cur, wm);     // uniform per wave
    for (int j0 = 0; j0 < steps; j0 += kBStages) {
#pragma unroll
      for (int u = 0; u < kBStages; ++u) {
        const int j = j0 + u;
        if (j < steps) {
          if (j + 1 < steps) dma_barrier<kBDmas>();
          else dma_barrier<0>();
          if (j + 2 < steps) pb_issue(lds_addr_of(u == 0 ? sg2 : (u == 1 ? sg0 : sg1)), d, j + 2);
          const uint8_t* stc = u == 0 ? sg0 : (u == 1 ? sg1 : sg2);
          if (ntt > 0) pb_compute<false, 4>(stc, wn, wm, lane, acc);
        }
      }
    }

    // every wave is done with the stages: request the next item's first two
    // (into sg0 and sg1; sg2 holds the y transposes until the next barrier)
    lds_barrier();
    if (it_next < i_end) {
      d = pb_geo<false>(a, nxt, trow2, wave, lane);
      pb_issue(lds_addr_of(sg0), d, 0);
      if (steps > 1) pb_issue(lds_addr_of(sg1), d, 1);
    }
    uint8_t* scratch = sg2 + wave * kWYScratch;
    YPend yp;
    if (ntt > 0) {
      pw_y16_prepare<4, 0>(acc, lane, scratch, yp);
      pw_y16_store<0, kBRows>(a, cur, yp, wn, 64 * wm, lane);
      pw_y16_store<1, kBRows>(a, cur, yp, wn, 64 * wm, lane);
      pw_y16_store<2, kBRows>(a, cur, yp, wn, 64 * wm, lane);
    }
    if (ntt > 2) {
      pw_y16_prepare<4, 2>(acc, lane, scratch, yp);
      pw_y16_store<0, kBRows>(a, cur, yp, wn, 64 * wm + 32, lane);
      pw_y16_store<1, kBRows>(a, cur, yp, wn, 64 * wm + 32, lane);
      pw_y16_store<2, kBRows>(a, cur, yp, wn, 64 * wm + 32, lane);
    }
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// FC2 at short K (at most three 128-wide K steps, as at I = 384): a work item
// is one 128-row m-tile x two 256-row n-tiles.  The m-tile's activations for
// the whole of K are requested once per item and stay in LDS, and the second
// n-tile's weights (256 rows x K) are requested while the first one is
// multiplied, into the other of two buffers; one wait per item then covers
// all of K instead of one per two-step stage.  TP8 prefill FC2 -8 % against
// the two-stage kernel (one n-tile per item -5 %, three -7 %: with more the
// work items are too few for an even spread over the CUs).  Waves, MFMA
// tiles and the fp16 y epilogue are those of the wide kernel.
namespace {

constexpr int kSMaxSteps = 3;
constexpr int kSNtPerItem = 2;                                // n-tiles per work item
constexpr int kSH = 0;                                        // activations: [step][8 token tiles]
constexpr int kSHS = kSH + kSMaxSteps * 8 * kWTileSw;         // [8 token tiles][step][16 tokens] scale dwords
constexpr int kSW = kSHS + 8 * kSMaxSteps * 16 * 4;           // two weight buffers
constexpr int kSWScales = kSMaxSteps * 16 * 1024;             // in a buffer: [step][16 tiles] of 16 rows x 64 B, then
constexpr int kSWBuf = kSWScales + kSMaxSteps * kWRows * 4;   // [step][256 rows] scale dwords
constexpr int kSLds = kSW + 2 * kSWBuf;                       // 161280 bytes
static_assert(kSLds <= 160 * 1024, "short-K FC2 LDS");
static_assert(8 * kWYScratch <= kSWBuf, "the y transpose fits a weight buffer");

struct PsGeo {
  v4i wr, sr, xr, xsr;
  uint32_t b_row[2];   // activation rows of tokens 16*wave + l/8 (+8)
  uint32_t sb_row;     // scale row of token 16*wave + l%16
  int K, steps, nkb, tiled;
};

__device__ __forceinline__ PsGeo ps_geo(const GemmArgs& a, const PfItem& x, const PfRows& tr) {
  PsGeo d;
  d.K = a.K;
  d.steps = a.K / 128;
  d.nkb = a.K / 32;
  d.tiled = a.tiled;
  const size_t wexp = expert_w_bytes(a.tiled != 0, a.N, a.K);
  const size_t sexp = (size_t)a.N * scale_row_bytes(false, a.tiled != 0, a.K);
  d.wr = rsrc4(a.w + (size_t)x.l * wexp, (uint32_t)wexp);
  d.sr = rsrc4(a.ws + (size_t)x.l * sexp, (uint32_t)sexp);
  d.xr = rsrc4(a.act, 0x7fffffff);
  d.xsr = rsrc4(a.act_scale, 0x7fffffff);
  d.b_row[0] = tr.t_a >= 0 ? (uint32_t)tr.t_a * (uint32_t)a.K : kOobPf;
  d.b_row[1] = tr.t_b >= 0 ? (uint32_t)tr.t_b * (uint32_t)a.K : kOobPf;
  d.sb_row = tr.t_s >= 0 ? (uint32_t)tr.t_s * (uint32_t)d.nkb : kOobPf;
  return d;
}

// This wave's token tile of the m-tile for every K step (the wide kernel's
// swizzled layout), and its scale dwords.
__device__ __forceinline__ void ps_issue_act(uint8_t* lds, const PsGeo& d, int w, int l) {
  const uint32_t chunk = (uint32_t)(((l & 7) ^ (l >> 3)) * 16);
#pragma unroll
  for (int s = 0; s < kSMaxSteps; ++s)
    if (s < d.steps) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        dma16(d.xr, lds_addr_of(lds + kSH + (8 * s + w) * kWTileSw + h * (1024 + 128)),
              d.b_row[h] == kOobPf ? kOobPf : d.b_row[h] + 128u * s + chunk);
    }
  if (l < 16 * d.steps)   // lane l: step l / 16, token l % 16
    dma4(d.xsr, lds_addr_of(lds + kSHS + w * (kSMaxSteps * 64)),
         d.sb_row == kOobPf ? kOobPf : d.sb_row + 4u * (uint32_t)(l >> 4));
}

// This wave's two 16-row weight tiles of n-tile rows n0.. for every K step,
// stored in lane order (from rows: 16 rows x 64 B per request; fragment-tiled:
// 1 KB contiguous), and a share of the n-tile's scales: per step 256 rows x
// one dword (from rows) or 16 tiles x 64 bytes in lane order (tiled).
__device__ __forceinline__ void ps_issue_w(uint8_t* wb, const PsGeo& d, int N, int n0, int w, int l) {
  const int r = l & 15, g = l >> 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row0 = n0 + 16 * (2 * w + i);
    const uint32_t ar = row0 >= N ? kOobPf
                        : d.tiled ? (uint32_t)(row0 / 16) * (uint32_t)d.steps * 1024u + (uint32_t)l * 16u
                                  : (uint32_t)(row0 + r) * (uint32_t)(d.K / 2) + 16u * (uint32_t)g;
    const uint32_t astep = d.tiled ? 1024u : 64u;
#pragma unroll
    for (int s = 0; s < kSMaxSteps; ++s)
      if (s < d.steps)
        dma16(d.wr, lds_addr_of(wb + (16 * s + 2 * w + i) * 1024), ar == kOobPf ? kOobPf : ar + (uint32_t)s * astep);
  }
#pragma unroll
  for (int q = w; q < 4 * kSMaxSteps; q += 8) {   // per step four blocks of 64 rows (4 tiles)
    const int s = q >> 2, blk = q & 3;
    if (s < d.steps) {
      uint32_t so;
      if (d.tiled) {
        const int row0 = n0 + 64 * blk + 16 * (l >> 4);
        so = row0 < N ? ((uint32_t)(row0 / 16) * (uint32_t)d.steps + (uint32_t)s) * 64u + (uint32_t)(l & 15) * 4u : kOobPf;
      } else {
        const int row = n0 + 64 * blk + l;
        so = row < N ? (uint32_t)row * (uint32_t)d.nkb + 4u * (uint32_t)s : kOobPf;
      }
      dma4(d.sr, lds_addr_of(wb + kSWScales + s * 1024 + blk * 256), so);
    }
  }
}

// K step s for one wave: 8 weight tiles x NTT token tiles of MFMAs, the reads
// and MFMAs interleaved as in the wide kernel.
template <int NTT>
__device__ __forceinline__ void ps_compute(const uint8_t* lds, const uint8_t* wb, int s, int wn, int wm, int lane,
                                           uint32_t s_rd, f32x4 acc[8][2]) {
  const int r = lane & 15, g = lane >> 4, rr = r & 7;
  const int rowoff = (r >> 3) * (1024 + 128) + rr * 128;
  uint4 blo[2], bhi[2];
  uint32_t sb[2];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int tile = 2 * wm + tt;
    const uint8_t* row = lds + kSH + (8 * s + tile) * kWTileSw + rowoff;
    blo[tt] = *reinterpret_cast<const uint4*>(row + 16 * (g ^ rr));
    bhi[tt] = *reinterpret_cast<const uint4*>(row + 16 * ((4 + g) ^ rr));
    sb[tt] = lds[kSHS + tile * (kSMaxSteps * 64) + s * 64 + r * 4 + g];
  }
  uint4 av[8];
  uint32_t sa[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tile = 8 * wn + i;
    av[i] = *reinterpret_cast<const uint4*>(wb + (16 * s + tile) * 1024 + lane * 16);
    sa[i] = wb[kSWScales + s * 1024 + tile * 64 + s_rd];
  }
  pw_mfmas<NTT>(blo, bhi, sb, av, sa, acc);
}

}  // namespace

__global__ __launch_bounds__(kWThreads, 1) void prefill_fc2_short_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t lds[kSLds];
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wn = wave & 1, wm = wave >> 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int steps = a.K / 128;
  const uint32_t s_rd = a.tiled ? (uint32_t)(16 * (lane >> 4) + (lane & 15)) : (uint32_t)(4 * (lane & 15) + (lane >> 4));
  const int n_tiles = (a.N + kWRows - 1) / kWRows;
  const int groups = (n_tiles + kSNtPerItem - 1) / kSNtPerItem;   // work items per m-tile
  const cptr te = (cptr)a.tile_expert, tr = (cptr)a.tile_rows;
  const int total = ((cptr)a.mtiles)[a.E_l] * groups;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd_wgs = (gridDim.x + 7 - xcd) / 8;
  const int chunk = (total + 7) / 8;
  const int i_begin = xcd * chunk, i_end = min(total, i_begin + chunk);

  // the y rows of the previous n-tile leave during the next one's K steps
  bool pend = false;
  PfItem px{0, 0, 0, 0};
  YPend yp;
  for (int it = i_begin + slot; it < i_end; it += per_xcd_wgs) {
    const int m = it / groups, grp = it % groups;
    PfItem x;
    x.l = te[m];
    x.nt = 0;
    x.p0 = tr[2 * m];
    x.p1 = tr[2 * m + 1];
    const int nt0 = grp * kSNtPerItem, nt1 = min(n_tiles, nt0 + kSNtPerItem);
    const int ntt = pw_active_tiles(x, wm);   // uniform per wave
    const PsGeo d = ps_geo(a, x, pf_act_rows<false>(a, x, wave_u, lane));
    lds_barrier();                      // every wave is done with the previous item's LDS
    ps_issue_act(lds, d, wave, lane);
    ps_issue_w(lds + kSW, d, a.N, nt0 * kWRows, wave, lane);
    for (int nt = nt0; nt < nt1; ++nt) {
      const int b = (nt - nt0) & 1;
      uint8_t* wb = lds + kSW + b * kSWBuf;
      dma_barrier<0>();                 // activations and this n-tile's weights have landed everywhere
      if (nt + 1 < nt1) ps_issue_w(lds + kSW + (b ^ 1) * kSWBuf, d, a.N, (nt + 1) * kWRows, wave, lane);
      f32x4 acc[8][2];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kSMaxSteps; ++s) {
        if (s < steps) {
          if (pend) {                   // parts 0, 1, 2 at steps 0, 1, 2 (the last step takes the rest)
            if (s == 0) pw_y16_store<0>(a, px, yp, wn, 32 * wm, lane);
            if (s == min(1, steps - 1)) pw_y16_store<1>(a, px, yp, wn, 32 * wm, lane);
            if (s == min(2, steps - 1)) pw_y16_store<2>(a, px, yp, wn, 32 * wm, lane);
          }
          if (ntt == 2) ps_compute<2>(lds, wb, s, wn, wm, lane, s_rd, acc);
          else if (ntt == 1) ps_compute<1>(lds, wb, s, wn, wm, lane, s_rd, acc);
        }
      }
      lds_barrier();                    // every wave is done reading wb: it holds the y transpose now
      pw_y16_prepare(acc, lane, wb + wave * kWYScratch, yp);
      px = x;
      px.nt = nt;
      pend = true;
    }
  }
  if (pend) {
    pw_y16_store<0>(a, px, yp, wn, 32 * wm, lane);
    pw_y16_store<1>(a, px, yp, wn, 32 * wm, lane);
    pw_y16_store<2>(a, px, yp, wn, 32 * wm, lane);
  }
}

template <bool FC1>
hipError_t launch_prefill_wide(const GemmArgs& a, int max_mtiles, int cus, hipStream_t s) {
  if constexpr (!FC1) {
    if (a.tiled && a.K % 128 == 0) {   // 512 y columns per item (fragment-tiled weights)
      const int64_t work = (int64_t)max_mtiles * ((a.N + kBRows - 1) / kBRows);
      int64_t grid = cus;                                    // one workgroup per CU
      if (grid > work) grid = (work + 7) / 8 * 8;
      if (grid <= 0) return hipSuccess;
      hipLaunchKernelGGL(prefill_fc2_512_kernel, dim3((unsigned)grid), dim3(kBThreads), 0, s, a);
      return hipGetLastError();
    }
    if (a.K % 128 == 0 && a.K <= 128 * kSMaxSteps) {     // the m-tile's activations fit beside two n-tiles
      const int64_t work = (int64_t)max_mtiles * ((a.N + kWRows - 1) / kWRows + kSNtPerItem - 1) / kSNtPerItem;
      int64_t grid = cus;                                    // one workgroup per CU
      if (grid > work) grid = (work + 7) / 8 * 8;
      if (grid <= 0) return hipSuccess;
      hipLaunchKernelGGL(prefill_fc2_short_kernel, dim3((unsigned)grid), dim3(kWThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (FC1) {
    if (a.tiled && a.N % 256 != 0 && a.N % 192 == 0) {   // 384 weight rows per item (tiled weights only)
      const int64_t work = (int64_t)max_mtiles * (a.N / 192);
      int64_t grid = cus;                                    // one workgroup per CU
      if (grid > work) grid = (work + 7) / 8 * 8;
      if (grid <= 0) return hipSuccess;
      if (general_epilogue(a))
        hipLaunchKernelGGL(prefill_fc1_384_kernel<true>, dim3((unsigned)grid), dim3(kCThreads), 0, s, a);
      else
        hipLaunchKernelGGL(prefill_fc1_384_kernel<false>, dim3((unsigned)grid), dim3(kCThreads), 0, s, a);
      return hipGetLastError();
    }
    if (a.tiled && a.N % 256 == 0) {   // 512 weight rows per item (tiled weights only)
      const int64_t work = (int64_t)max_mtiles * (a.N / 256);
      int64_t grid = cus;                                    // one workgroup per CU
      if (grid > work) grid = (work + 7) / 8 * 8;
      if (grid <= 0) return hipSuccess;
      if (general_epilogue(a))
        hipLaunchKernelGGL(prefill_fc1_512_kernel<true>, dim3((unsigned)grid), dim3(kBThreads), 0, s, a);
      else
        hipLaunchKernelGGL(prefill_fc1_512_kernel<false>, dim3((unsigned)grid), dim3(kBThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  const int n_tiles = FC1 ? a.N / 128 : (a.N + kWRows - 1) / kWRows;
  const int64_t work = (int64_t)max_mtiles * n_tiles;
  int64_t grid = cus;                                        // one workgroup per CU
  if (grid > work) grid = (work + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  if (FC1 && general_epilogue(a))
    hipLaunchKernelGGL((prefill_wide_kernel<FC1, FC1>), dim3((unsigned)grid), dim3(kWThreads), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_wide_kernel<FC1, false>), dim3((unsigned)grid), dim3(kWThreads), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_prefill_wide<true>(const GemmArgs&, int, int, hipStream_t);
template hipError_t launch_prefill_wide<false>(const GemmArgs&, int, int, hipStream_t);

template <bool FC1>
hipError_t launch_prefill(const GemmArgs& a, int max_mtiles, int cus, hipStream_t s) {
  const bool gen = FC1 && general_epilogue(a);
  const void* kern = gen ? reinterpret_cast<const void*>(prefill_gemm_kernel<FC1, FC1>)
                         : reinterpret_cast<const void*>(prefill_gemm_kernel<FC1, false>);
  const int per_cu = resident_per_cu(kern, kGemmThreads, 0);
  const int n_tiles = FC1 ? a.N / 128 : (a.N + kPfRows - 1) / kPfRows;
  const int64_t work = (int64_t)max_mtiles * n_tiles;
  int64_t grid = (int64_t)cus * per_cu;
  if (grid > work) grid = (work + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  if (gen)
    hipLaunchKernelGGL((prefill_gemm_kernel<FC1, FC1>), dim3((unsigned)grid), dim3(kGemmThreads), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_gemm_kernel<FC1, false>), dim3((unsigned)grid), dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_prefill<true>(const GemmArgs&, int, int, hipStream_t);
template hipError_t launch_prefill<false>(const GemmArgs&, int, int, hipStream_t);

}  // namespace situ

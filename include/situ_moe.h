/*
 * situ_moe.h -- C ABI of the MXFP4 + SiTU routed-MoE expert layer on MI355X (gfx950).
 *
 * One call computes ONE tensor- or expert-parallel shard's partial output of
 * a routed Mixture-of-Experts layer whose expert weights are MXFP4 (E2M1
 * values, one E8M0 scale per 32 elements along K) and whose gated activation
 * is SiTU.  The contract follows the pages' description of the layer:
 *
 *  - "TokenSpeed SiTU" (PyPI page of tokenspeed-situ), "Supported contract":
 *    BF16 activations (w4a16) or MXFP8 activations with a per-token block
 *    scale tensor (w4a8); MXFP4 weights; precomputed packed or unpacked
 *    top-k with GLOBAL expert ids; experts outside the rank's contiguous
 *    shard [local_expert_offset, local_expert_offset + local_num_experts)
 *    are dropped and the result is a PARTIAL output that the caller sums
 *    over the MoE TP/EP group (this library owns no communication).
 *  - same page, "Activation precision (w4a16 vs w4a8)": in w4a8 the FC1
 *    output is rounded through MXFP8 and dequantized before a w4a16 FC2.
 *  - same page, "Runtime API": the caller passes the physical intermediate
 *    size, the global expert count, the local expert offset and count; the
 *    default tactic (-1, -1) is the first valid configuration for the
 *    runtime shape, with no autotuning.
 *  - "bring up Kimi K3 NVFP4 with CUTLASS and cuteDSL MegaMoE SiTU"
 *    (TensorRT-LLM pull request 17865), review of test_kimi_k3_situ_moe.py:
 *    act(g, u) = [beta*tanh(g/beta)*sigmoid(g)] * [lbeta*tanh(u/lbeta)] and
 *    out[t] += weight[t,s] * (act(g,u) @ w2^T); review of moe_kernels.h /
 *    moeOp.cpp: SiTU's beta arrays are required, never defaulted.
 *  - "FlashInfer 0.6.18 SM100a+SM103a MoE-LoRA AOT -- Kimi-K3 SiTU" release
 *    notes, "Changes since 875b7d7": per-expert beta and linear beta; the up
 *    half rescaled by alpha_up / alpha_gate before the tanh; the decomposed
 *    MoE-LoRA op takes a gate_up LoRA delta (added to the FC1 output before
 *    the activation) and hands back the activation input of the down LoRA,
 *    and runs the plain pipeline when both are empty.
 *  - pull request 17865, review of test_kimi_k3_situ_moe.py: the same
 *    routed skeleton with the SwiGLU and CUTLASS SwigluBias activations
 *    (gate * sigmoid(gate * alpha) * (linear + beta)); the NVFP4 Kimi-K3
 *    checkpoint (E2M1 weights with E4M3 scales per 16 elements and a
 *    per-tensor scale, here the per-expert alphas).
 *
 * Conventions for every entry point:
 *  - Plain C.  Pointers marked (device) are HIP device pointers, (host) are
 *    host pointers.  All arrays are dense and row-major.  The device arrays
 *    of situ_moe_tensors must be 16-byte aligned, except the per-expert
 *    float arrays (4-byte aligned); situ_moe_run returns SITU_E_BAD_SHAPE
 *    otherwise.
 *  - The caller owns every buffer: inputs, the output and the workspace.
 *    The library allocates no device memory and holds no device state.
 *  - Every function returns situ_status; no exception crosses the ABI.  On
 *    a non-OK status, situ_moe_last_error() returns a message for the
 *    calling thread.
 *  - Work is enqueued on the given hipStream_t (NULL = the null stream) and
 *    never synchronized; no device data is read back to the host.
 */
#ifndef SITU_MOE_H
#define SITU_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SITU_MOE_ABI_VERSION 3

typedef enum situ_status {
  SITU_OK = 0,
  SITU_E_NULL_ARG = 1,       /* a required pointer is NULL */
  SITU_E_BAD_SHAPE = 2,      /* sizes inconsistent or out of range */
  SITU_E_UNSUPPORTED = 3,    /* valid request this library does not implement (incl. a tactic outside the family) */
  SITU_E_MISSING_SCALE = 4,  /* w4a8 with prequantized input but no hidden_states_scale */
  SITU_E_DEVICE = 5,         /* no device, or the current device is not gfx950 */
  SITU_E_WORKSPACE = 6,      /* workspace NULL or smaller than the plan needs */
  SITU_E_LAUNCH = 7          /* a kernel launch failed */
} situ_status;

enum { SITU_ACT_W4A16 = 0, SITU_ACT_W4A8 = 1 };
enum { SITU_OUT_F32 = 0, SITU_OUT_BF16 = 1 };
/* Gated activation h = act(g, u) of g = alpha_gate * acc_gate, u = alpha_up * acc_up:
 *  SiTU        [beta * tanh(g / beta) * sigmoid(g)] * [lbeta * tanh(u / lbeta)]
 *  SwiGLU      g * sigmoid(g) * u
 *  SwigluBias  g * sigmoid(g * swiglu_alpha) * (u + swiglu_beta)          */
enum { SITU_ACTIVATION_SITU = 0, SITU_ACTIVATION_SWIGLU = 1, SITU_ACTIVATION_SWIGLU_BIAS = 2 };
/* Expert weight format: MXFP4 = E2M1 + E8M0 scale per 32 along K;
 * NVFP4 = E2M1 + E4M3 scale per 16 along K (w4a16 only);
 * MXFP4_TILED = the same MXFP4 values in the fragment-tiled layout made by
 * situ_moe_tile_weights (ABI 3; see there).  The layer computes the same
 * result bit for bit from MXFP4 and MXFP4_TILED weights. */
enum { SITU_WEIGHTS_MXFP4 = 0, SITU_WEIGHTS_NVFP4 = 1, SITU_WEIGHTS_MXFP4_TILED = 2 };

/* The runtime shape of one shard (host POD). */
typedef struct situ_moe_problem {
  int32_t num_tokens;           /* T >= 0 */
  int32_t hidden_size;          /* H, multiple of 32 */
  int32_t intermediate_size;    /* physical I of this shard, multiple of 32 */
  int32_t num_experts;          /* global expert count E_g, 1..65535 */
  int32_t local_expert_offset;  /* off >= 0 */
  int32_t local_num_experts;    /* E_l, 1..1024, off + E_l <= E_g */
  int32_t top_k;                /* k, 1..E_g */
  int32_t act_mode;             /* SITU_ACT_W4A16 or SITU_ACT_W4A8 (fixed for the process on the pages; per plan here) */
  int32_t act_prequantized;     /* w4a8 only: 1 = hidden_states are E4M3 codes + E8M0 scales; 0 = bf16, quantized here */
  int32_t topk_packed;          /* 0 = topk_ids int32 + topk_weights bf16; 1 = topk_packed int32 (bf16 weight << 16 | id) */
  int32_t out_dtype;            /* SITU_OUT_F32 or SITU_OUT_BF16 (round-to-nearest-even of the fp32 result) */
  int32_t tactic_fc1;           /* -1 = first valid; else a value from situ_moe_valid_tactics */
  int32_t tactic_fc2;           /* -1 = first valid */
  int32_t activation;           /* SITU_ACTIVATION_* */
  int32_t weight_format;        /* SITU_WEIGHTS_* */
} situ_moe_problem;

/* A resolved plan (host POD, reusable, no device state).  The workspace
 * region offsets are part of the ABI so that tests can inspect the routing
 * results and intermediates a run leaves in the workspace. */
typedef struct situ_moe_plan_t {
  situ_moe_problem prob;
  int32_t fc1_tactic;           /* resolved tactic ids */
  int32_t fc2_tactic;
  int32_t block_m;              /* rows (token-expert pairs) per m-tile */
  int32_t max_mtiles;           /* upper bound of m-tiles: T*k / block_m + E_l */
  int32_t route_blocks;         /* 1 = one-workgroup routing; else blocks of route_chunk pairs */
  int32_t route_chunk;
  uint64_t workspace_bytes;     /* bytes the caller must provide */
  /* byte offsets into the workspace (each 256-byte aligned) */
  uint64_t off_counts;          /* int32 [E_l]      pairs per local expert */
  uint64_t off_offsets;         /* int32 [E_l + 1]  exclusive prefix sum of counts */
  uint64_t off_mtiles;          /* int32 [E_l + 1]  exclusive prefix sum of ceil(counts / block_m) */
  uint64_t off_tile_expert;     /* int32 [max_mtiles] local expert of each m-tile, in order */
  uint64_t off_perm;            /* int32 [T*k]      perm[offsets[l] + r] = expanded index t*k+s */
  uint64_t off_inv;             /* int32 [T*k]      position of pair t*k+s in perm, -1 if not local */
  uint64_t off_xq;              /* uint8 [T, H]     E4M3 codes of bf16 input (w4a8, not prequantized) */
  uint64_t off_xs;              /* uint8 [T, H/32]  their E8M0 scales */
  uint64_t off_h;               /* FC1 output rows in perm order: bf16 [T*k, I] (w4a16) or E4M3 [T*k, I] (w4a8) */
  uint64_t off_hs;              /* uint8 [T*k, I/32] E8M0 scales of h (w4a8) */
  uint64_t off_y;               /* FC2 output rows in perm order: float [T*k, H] (y_format 0), or
                                   fp16 [T*k, H] scaled by 2^(y_exp - 127) per 64 columns (y_format 1) */
  uint64_t off_route_hist;      /* int32 [route_blocks, E_l] per-block histograms, then each block's first position
                                   within its expert's group (route_blocks > 1) */
  uint64_t off_tile_rows;       /* int32 [max_mtiles, 2] first and one-past-last perm position of each m-tile */
  uint64_t off_y_exp;           /* uint8 [T*k, ceil(H/64)] block exponents of y (y_format 1), row-major,
                                   inside the y region */
  int32_t y_format;             /* 0: fp32 y; 1: fp16 y with an exponent per 64 columns (the 128-row w4a8 tactic) */
  uint32_t reserved[3];
} situ_moe_plan_t;

/* Device tensors of one call.  Shapes use T, H, I, k, E_l of the problem. */
typedef struct situ_moe_tensors {
  const void* hidden_states;          /* (device) bf16 [T, H]; or E4M3 codes uint8 [T, H] if act_prequantized */
  const uint8_t* hidden_states_scale; /* (device) E8M0 uint8 [T, H/32], per token per 32 along H; w4a8 prequantized only */
  const int32_t* topk_ids;            /* (device) int32 [T, k], GLOBAL ids; any id outside the shard is skipped */
  const uint16_t* topk_weights;       /* (device) bf16 [T, k] routing weights, applied in the combine */
  const int32_t* topk_packed;         /* (device) int32 [T, k] = (bf16 weight bits << 16) | (id & 0xFFFF); topk_packed only */
  const uint8_t* w1;                  /* (device) E2M1 [E_l, 2I, H/2]: rows [0,I) gate, [I,2I) up; low nibble = even k
                                         (MXFP4_TILED: situ_moe_tile_weights of it, rows = 2I, k = H) */
  const uint8_t* w1_scale;            /* (device) MXFP4: E8M0 [E_l, 2I, H/32]; NVFP4: E4M3 [E_l, 2I, H/16] */
  const uint8_t* w2;                  /* (device) E2M1 [E_l, H, I/2] (MXFP4_TILED: tiled with rows = H, k = I) */
  const uint8_t* w2_scale;            /* (device) MXFP4: E8M0 [E_l, H, I/32]; NVFP4: E4M3 [E_l, H, I/16] */
  const float* situ_beta;             /* (device) float [E_l]; required with SiTU, else ignored */
  const float* situ_linear_beta;      /* (device) float [E_l]; required with SiTU, else ignored */
  const float* alpha_gate;            /* (device) float [E_l] or NULL (= 1.0) */
  const float* alpha_up;              /* (device) float [E_l] or NULL (= 1.0) */
  void* out;                          /* (device) [T, H] float or bf16 per out_dtype; every element is written */
  /* ABI 2 */
  const float* swiglu_alpha;          /* (device) float [E_l]; required with SwigluBias, else ignored */
  const float* swiglu_beta;           /* (device) float [E_l]; required with SwigluBias, else ignored */
  const float* alpha_down;            /* (device) float [E_l] or NULL (= 1.0): per-expert scale of the FC2
                                         output (the NVFP4 per-tensor scale of w2), applied to the routing
                                         weight in the combine as one fp32 product */
  const uint16_t* gate_up_lora_delta; /* (device) bf16 [T*k, 2I] or NULL: a LoRA adapter's FC1 output for
                                         pair j = t*k + s (gate columns, then up), added in fp32 to the
                                         alpha-scaled halves before the activation (alpha_gate and alpha_up
                                         must then be nonzero); an all-zero delta gives the output of a
                                         call without it bit for bit; rows of pairs outside the shard are
                                         not read */
  uint16_t* activation_lora_input;    /* (device) bf16 [T*k, I] or NULL: receives h of pair j (the input of
                                         the down LoRA, after the rounding point; exact in bf16 in both
                                         modes), zero rows for pairs outside the shard */
} situ_moe_tensors;

/* Validate a problem and resolve its tactics, block size and workspace
 * layout.  Host only; needs no device.  Returns SITU_E_BAD_SHAPE or
 * SITU_E_UNSUPPORTED on a problem it cannot serve, never a silent fallback. */
situ_status situ_moe_plan(const situ_moe_problem* problem, situ_moe_plan_t* plan);

/* List the (fc1, fc2) tactic pairs valid for a problem, first-valid first
 * ("Runtime API": the tactic list of get_valid_k3_situ_configs).  Writes at
 * most `capacity` pairs to fc1[] / fc2[] (host) and the total to *count. */
situ_status situ_moe_valid_tactics(const situ_moe_problem* problem, int32_t* fc1, int32_t* fc2,
                                   int32_t capacity, int32_t* count);

/* Run the whole layer: shard filter and routing, [MXFP8 quantize of bf16
 * input in w4a8], FC1 + alpha + SiTU, FC2, weighted combine into `out`.
 * Asynchronous on `hip_stream`; capture-safe (no host synchronization, no
 * allocation).  Calls sharing one workspace must not overlap in time. */
situ_status situ_moe_run(const situ_moe_plan_t* plan, const situ_moe_tensors* tensors,
                         void* workspace, uint64_t workspace_bytes, void* hip_stream);

/* situ_moe_run that also records caller-created hipEvent_t handles on the
 * stream at the stage boundaries, for timing each kernel on the stream it
 * runs on: [0] before routing, [1] after routing, [2] after the MXFP8
 * quantization (recorded right after [1] when there is none), [3] after
 * FC1, [4] after FC2, [5] after the combine.  n_events must be 6.  The
 * kernels and results are exactly those of situ_moe_run. */
situ_status situ_moe_run_profiled(const situ_moe_plan_t* plan, const situ_moe_tensors* tensors,
                                  void* workspace, uint64_t workspace_bytes, void* hip_stream,
                                  void* const* hip_events, int32_t n_events);

/* situ_moe_run without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the routing tables and intermediates go
 * to the library's own scratch array of SITU_MOE_STATIC_SCRATCH_BYTES, one
 * per device, held from the first call on that device until the process
 * ends.  Allocates nothing.  A plan whose workspace_bytes exceed the array
 * returns SITU_E_WORKSPACE (decode-sized shards fit; prefill shards need
 * situ_moe_run).  Calls that overlap in time on one device race on the
 * array; the array keeps the last call's contents and nothing in it is
 * assumed to start at zero.  Otherwise exactly situ_moe_run (same kernels,
 * same results bit for bit). */
#define SITU_MOE_STATIC_SCRATCH_BYTES (128u * 1024u * 1024u)
situ_status situ_moe_run_static(const situ_moe_plan_t* plan, const situ_moe_tensors* tensors, void* hip_stream);

/* The routing stage alone: fills counts, offsets, mtiles, perm and inv in
 * the workspace (offsets in the plan).  Reads only the top-k tensors. */
situ_status situ_moe_route(const situ_moe_plan_t* plan, const situ_moe_tensors* tensors,
                           void* workspace, uint64_t workspace_bytes, void* hip_stream);

/* MXFP4 expert weights in the fragment-tiled layout (SITU_WEIGHTS_MXFP4_TILED).
 * Callers that cannot allocate it themselves call this once per weight
 * tensor when the weights are loaded (the layout is this library's own: the
 * pages leave the arrangement of expert weights to each MoE backend, "bring
 * up Kimi K3 NVFP4 with CUTLASS and cuteDSL MegaMoE SiTU", the note on the
 * expert loader).  The values are unchanged; only their order differs, and
 * every GEMM kernel then reads a weight fragment as one contiguous 1 KB.
 *
 * Input: w E2M1 [experts, rows, k/2] and w_scale E8M0 [experts, rows, k/32]
 * (device, row-major as in situ_moe_tensors).  With S = ceil(k / 128), each
 * expert's matrix becomes rows/16 x S blocks, row tile rt major and K step j
 * fastest:
 *   w_tiled     (device) [experts, rows/16, S, 1024] bytes: byte 16*l + b of
 *               block (rt, j) is byte b of row 16*rt + l%16, K block
 *               4*j + l/16 (the 16 bytes row-major holds at
 *               row*(k/2) + 16*(4*j + l/16)); zero for K blocks >= k/32
 *   scale_tiled (device) [experts, rows/16, S, 64] bytes: byte l of block
 *               (rt, j) is the E8M0 scale of that row and K block; 127 for K
 *               blocks >= k/32
 * rows a positive multiple of 16, k a positive multiple of 32, one expert's
 * tiled matrix below 2 GiB (rows * S * 64 bytes); w, w_tiled 16-byte
 * aligned.  The outputs must not overlap the inputs.  Asynchronous on
 * hip_stream.  SITU_E_BAD_SHAPE / SITU_E_NULL_ARG on bad arguments. */
situ_status situ_moe_tile_weights(const uint8_t* w, const uint8_t* w_scale, int32_t experts, int32_t rows, int32_t k,
                                  uint8_t* w_tiled, uint8_t* scale_tiled, void* hip_stream);

/* MXFP8 quantization of a bf16 matrix [rows, cols] (cols multiple of 32),
 * per row per 32 consecutive columns, by the OCP MX v1.0 rule: scale code =
 * floor(log2(block amax)) - 8 + 127 clamped to [0, 254] (0 for an all-zero
 * block), element = E4M3 round-to-nearest-even of x / 2^(code-127),
 * saturating to +-448.  codes uint8 [rows, cols], scales uint8 [rows, cols/32]
 * (all device).  Input NaN/Inf give unspecified codes. */
situ_status situ_moe_quantize_mxfp8(const uint16_t* x_bf16, int64_t rows, int32_t cols,
                                    uint8_t* codes, uint8_t* scales, void* hip_stream);

/* Measurement aid for the roofline of the w4a8 GEMMs (not part of the
 * layer): the sustained rate of v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 x
 * E4M3 operands (the instruction the w4a8 FC1 kernels issue; 65536 flops
 * each) on the current device, every SIMD running 4 waves of 8 independent
 * accumulators for `iters` rounds on register operands.  Writes TFLOP/s to
 * *tflops.  Synchronous (one warm-up launch, then one timed launch on a
 * stream of its own); allocates no device memory.  iters in [1, 1 << 20]
 * (SITU_E_BAD_SHAPE otherwise); SITU_E_NULL_ARG if tflops is NULL;
 * SITU_E_DEVICE without a gfx950 device; SITU_E_LAUNCH on a runtime error. */
situ_status situ_moe_measure_mfma_peak(int32_t iters, double* tflops);

const char* situ_moe_status_string(situ_status status);
const char* situ_moe_last_error(void);
/* Human-readable build description: ABI version, gfx target, tactic family. */
const char* situ_moe_build_info(void);
/* Name of a tactic id, or NULL if the id is not in the family. */
const char* situ_moe_tactic_name(int32_t tactic);
int32_t situ_moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SITU_MOE_H */

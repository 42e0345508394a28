// Host side of the C ABI declared in include/situ_moe.h: problem validation,
// tactic selection, workspace layout and the ordered launch of the layer's
// kernels on the caller's stream.
//
// The validation rules follow the pages: SiTU's beta arrays are required,
// never defaulted to zero (review of moe_kernels.h / moeOp.cpp in
// TensorRT-LLM pull request 17865); a tactic outside the family is an error,
// not a silent fallback (same pull request, the create_moe fallback
// finding); the FC1 weight has 2*I rows for a gated activation (its
// "fc1_expert_weights inter size must be 2 times fc2" check); the device
// architecture is checked rather than assumed (xorl-wheels release notes,
// "Install and architecture").
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/situ_moe.h"
#include "internal.hpp"

#ifndef SITU_GIT_REV
#define SITU_GIT_REV "unknown"
#endif

namespace {

thread_local std::string g_last_error;

situ_status fail(situ_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
situ_status fail(situ_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

}  // namespace

namespace situ {
situ_status fail_status(situ_status status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}
}  // namespace situ

namespace {

constexpr uint64_t kAlign = 256;
constexpr int64_t kRouteSingleMax = 32768;   // pairs routed by a single workgroup
constexpr double kWideRowsPerExpert = 192.0; // mean group size above which 128-row m-tiles come first
uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct TacticInfo {
  int32_t id;
  const char* name;
  int32_t act_mode;
  int32_t block_m;
  bool fc1;
};

const TacticInfo kTactics[] = {
    {situ::FC1_W4A16_M16, "fc1_w4a16_bf16mfma_m16", SITU_ACT_W4A16, 16, true},
    {situ::FC1_W4A16_M64, "fc1_w4a16_bf16mfma_m64", SITU_ACT_W4A16, 64, true},
    {situ::FC1_W4A8_M16, "fc1_w4a8_scalemfma_m16", SITU_ACT_W4A8, 16, true},
    {situ::FC1_W4A8_M64, "fc1_w4a8_scalemfma_m64", SITU_ACT_W4A8, 64, true},
    {situ::FC1_W4A8_M128, "fc1_w4a8_scalemfma_m128", SITU_ACT_W4A8, 128, true},
    {situ::FC1_FUSED_W4A16_M16, "fused_decode_w4a16_bf16mfma_m16", SITU_ACT_W4A16, 16, true},
    {situ::FC1_FUSED_W4A8_M16, "fused_decode_w4a8_scalemfma_m16", SITU_ACT_W4A8, 16, true},
    {situ::FC2_W4A16_M16, "fc2_w4a16_bf16mfma_m16", SITU_ACT_W4A16, 16, false},
    {situ::FC2_W4A16_M64, "fc2_w4a16_bf16mfma_m64", SITU_ACT_W4A16, 64, false},
    {situ::FC2_W4A8_M16, "fc2_w4a8_scalemfma_m16", SITU_ACT_W4A8, 16, false},
    {situ::FC2_W4A8_M64, "fc2_w4a8_scalemfma_m64", SITU_ACT_W4A8, 64, false},
    {situ::FC2_W4A8_M128, "fc2_w4a8_scalemfma_m128", SITU_ACT_W4A8, 128, false},
    {situ::FC2_FUSED_W4A16_M16, "fused_decode_w4a16_fc2_half", SITU_ACT_W4A16, 16, false},
    {situ::FC2_FUSED_W4A8_M16, "fused_decode_w4a8_fc2_half", SITU_ACT_W4A8, 16, false},
};

const TacticInfo* find_tactic(int32_t id) {
  for (const auto& t : kTactics)
    if (t.id == id) return &t;
  return nullptr;
}

situ_status validate(const situ_moe_problem* p) {
  if (!p) return fail(SITU_E_NULL_ARG, "problem is NULL");
  if (p->num_tokens < 0) return fail(SITU_E_BAD_SHAPE, "num_tokens %d < 0", p->num_tokens);
  if (p->hidden_size <= 0 || p->hidden_size % 32)
    return fail(SITU_E_BAD_SHAPE, "hidden_size %d must be a positive multiple of 32", p->hidden_size);
  if (p->intermediate_size <= 0 || p->intermediate_size % 32)
    return fail(SITU_E_BAD_SHAPE, "intermediate_size %d must be a positive multiple of 32 (pad the physical size)",
                p->intermediate_size);
  if (p->num_experts <= 0 || p->num_experts >= 65536)
    return fail(SITU_E_BAD_SHAPE, "num_experts %d must be in [1, 65535]", p->num_experts);
  if (p->local_expert_offset < 0) return fail(SITU_E_BAD_SHAPE, "local_expert_offset %d < 0", p->local_expert_offset);
  if (p->local_num_experts <= 0) return fail(SITU_E_BAD_SHAPE, "local_num_experts %d <= 0", p->local_num_experts);
  if ((int64_t)p->local_expert_offset + p->local_num_experts > p->num_experts)
    return fail(SITU_E_BAD_SHAPE, "local shard [%d, %d) exceeds num_experts %d", p->local_expert_offset,
                p->local_expert_offset + p->local_num_experts, p->num_experts);
  if (p->local_num_experts > situ::kMaxLocalExperts)
    return fail(SITU_E_UNSUPPORTED, "local_num_experts %d > %d", p->local_num_experts, situ::kMaxLocalExperts);
  if (p->top_k <= 0 || p->top_k > p->num_experts)
    return fail(SITU_E_BAD_SHAPE, "top_k %d must be in [1, num_experts]", p->top_k);
  if (p->act_mode != SITU_ACT_W4A16 && p->act_mode != SITU_ACT_W4A8)
    return fail(SITU_E_UNSUPPORTED, "act_mode %d", p->act_mode);
  if (p->act_prequantized != 0 && p->act_prequantized != 1)
    return fail(SITU_E_BAD_SHAPE, "act_prequantized must be 0 or 1");
  if (p->act_prequantized && p->act_mode != SITU_ACT_W4A8)
    return fail(SITU_E_UNSUPPORTED, "prequantized (MXFP8) activations need act_mode w4a8");
  if (p->topk_packed != 0 && p->topk_packed != 1) return fail(SITU_E_BAD_SHAPE, "topk_packed must be 0 or 1");
  if (p->out_dtype != SITU_OUT_F32 && p->out_dtype != SITU_OUT_BF16)
    return fail(SITU_E_UNSUPPORTED, "out_dtype %d", p->out_dtype);
  if (p->activation != SITU_ACTIVATION_SITU && p->activation != SITU_ACTIVATION_SWIGLU &&
      p->activation != SITU_ACTIVATION_SWIGLU_BIAS)
    return fail(SITU_E_UNSUPPORTED, "activation %d", p->activation);
  if (p->weight_format != SITU_WEIGHTS_MXFP4 && p->weight_format != SITU_WEIGHTS_NVFP4 &&
      p->weight_format != SITU_WEIGHTS_MXFP4_TILED)
    return fail(SITU_E_UNSUPPORTED, "weight_format %d", p->weight_format);
  if (p->weight_format == SITU_WEIGHTS_NVFP4 && p->act_mode != SITU_ACT_W4A16)
    return fail(SITU_E_UNSUPPORTED, "NVFP4 weights are served with bf16 activations (w4a16) only");
  const int64_t tk = (int64_t)p->num_tokens * p->top_k;
  if (tk >= (int64_t)1 << 31) return fail(SITU_E_UNSUPPORTED, "num_tokens * top_k = %lld exceeds int32", (long long)tk);
  // one expert's weights are addressed with 32-bit offsets from one buffer resource
  const bool tiled = p->weight_format == SITU_WEIGHTS_MXFP4_TILED;
  const uint64_t w1e = situ::expert_w_bytes(tiled, 2 * p->intermediate_size, p->hidden_size);
  const uint64_t w2e = situ::expert_w_bytes(tiled, p->hidden_size, p->intermediate_size);
  if (w1e >= (uint64_t)1 << 31 || w2e >= (uint64_t)1 << 31)
    return fail(SITU_E_UNSUPPORTED, "one expert's weights (%llu, %llu bytes) exceed 2 GiB", (unsigned long long)w1e,
                (unsigned long long)w2e);
  // activation rows are addressed with 32-bit offsets from one buffer resource
  if ((int64_t)p->num_tokens * p->hidden_size * 2 >= (int64_t)1 << 31)
    return fail(SITU_E_UNSUPPORTED, "hidden states of %lld bytes exceed 2 GiB",
                (long long)p->num_tokens * p->hidden_size * 2);
  return SITU_OK;
}

// Valid (fc1, fc2) pairs, first-valid first: small groups (decode) take
// 16-row m-tiles, large groups (prefill) 64-row m-tiles, and in w4a8 very
// large groups 128-row m-tiles (the wide kernel: K and the intermediate size
// multiples of 128, h addressable with 32-bit offsets).
int valid_pairs(const situ_moe_problem* p, int32_t* fc1, int32_t* fc2, int cap) {
  const bool w4a8 = p->act_mode == SITU_ACT_W4A8;
  const int32_t m16[2] = {w4a8 ? situ::FC1_W4A8_M16 : situ::FC1_W4A16_M16,
                          w4a8 ? situ::FC2_W4A8_M16 : situ::FC2_W4A16_M16};
  const int32_t m64[2] = {w4a8 ? situ::FC1_W4A8_M64 : situ::FC1_W4A16_M64,
                          w4a8 ? situ::FC2_W4A8_M64 : situ::FC2_W4A16_M64};
  const int32_t m128[2] = {situ::FC1_W4A8_M128, situ::FC2_W4A8_M128};
  // the fused decode pair (both GEMMs in one launch, h kept on chip)
  const int32_t fused[2] = {w4a8 ? situ::FC1_FUSED_W4A8_M16 : situ::FC1_FUSED_W4A16_M16,
                            w4a8 ? situ::FC2_FUSED_W4A8_M16 : situ::FC2_FUSED_W4A16_M16};
  const bool fuse = p->weight_format != SITU_WEIGHTS_NVFP4 && situ::fused_decode_ok(p->hidden_size, p->intermediate_size);
  const int64_t TK = (int64_t)p->num_tokens * p->top_k;
  const int64_t mt128 = (TK + 127) / 128 + p->local_num_experts;
  const bool wide = w4a8 && p->hidden_size % 128 == 0 && p->intermediate_size % 128 == 0 &&
                    mt128 * 128 * p->intermediate_size < ((int64_t)1 << 31);
  // the expected group size: the plan is made without the routing, so the
  // batch's T*k pairs are taken as spread evenly over all E_g experts (in an
  // EP shard only about E_l / E_g of them are local)
  const double rows_per_expert = (double)TK / p->num_experts;
  const int32_t* order[4] = {m16, m64, m128, fused};
  int n_order = wide ? 3 : 2;
  if (wide && rows_per_expert > kWideRowsPerExpert) {
    order[0] = m128; order[1] = m64; order[2] = m16;
  } else if (rows_per_expert > 48.0) {
    order[0] = m64; order[1] = m16;
  }
  if (fuse) order[n_order++] = fused;
  int n = 0;
  for (int i = 0; i < n_order; ++i) {
    if (n < cap) { fc1[n] = order[i][0]; fc2[n] = order[i][1]; }
    ++n;
  }
  return n;
}

struct DeviceInfo {
  bool checked = false;
  bool ok = false;
  int cus = 0;
  std::string arch;
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

situ_status device_check(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(SITU_E_DEVICE, "no current HIP device");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(SITU_E_DEVICE, "hipGetDeviceProperties failed");
    d.arch = prop.gcnArchName;
    d.cus = prop.multiProcessorCount;
    d.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.checked = true;
  }
  if (!d.ok) return fail(SITU_E_DEVICE, "device %d is %s; this library is built for gfx950 only", dev, d.arch.c_str());
  *cus = d.cus;
  return SITU_OK;
}

situ_status launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SITU_OK;
  return fail(SITU_E_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
}

situ_status check_run_args(const situ_moe_plan_t* plan, const situ_moe_tensors* t, void* ws, uint64_t ws_bytes,
                           bool route_only) {
  if (!plan) return fail(SITU_E_NULL_ARG, "plan is NULL");
  if (!t) return fail(SITU_E_NULL_ARG, "tensors is NULL");
  const situ_moe_problem& p = plan->prob;
  situ_status st = validate(&p);
  if (st != SITU_OK) return st;
  if (p.num_tokens == 0) return SITU_OK;  // nothing is read or written; empty arrays may be NULL
  if (p.topk_packed ? !t->topk_packed : (!t->topk_ids || !t->topk_weights))
    return fail(SITU_E_NULL_ARG, p.topk_packed ? "topk_packed is NULL" : "topk_ids or topk_weights is NULL");
  if (!route_only) {
    if (!t->hidden_states) return fail(SITU_E_NULL_ARG, "hidden_states is NULL");
    if (p.act_prequantized && !t->hidden_states_scale)
      return fail(SITU_E_MISSING_SCALE, "w4a8 prequantized input needs hidden_states_scale");
    if (!t->w1 || !t->w1_scale || !t->w2 || !t->w2_scale) return fail(SITU_E_NULL_ARG, "a weight or scale is NULL");
    if (p.activation == SITU_ACTIVATION_SITU && (!t->situ_beta || !t->situ_linear_beta))
      return fail(SITU_E_NULL_ARG, "SiTU needs situ_beta and situ_linear_beta (no default is substituted)");
    if (p.activation == SITU_ACTIVATION_SWIGLU_BIAS && (!t->swiglu_alpha || !t->swiglu_beta))
      return fail(SITU_E_NULL_ARG, "SwigluBias needs swiglu_alpha and swiglu_beta (no default is substituted)");
    if (!t->out) return fail(SITU_E_NULL_ARG, "out is NULL");
  }
  // the kernels move rows in 16-byte pieces from these bases (and 4-byte
  // words from the per-expert parameter arrays)
  const struct { const void* ptr; const char* name; uintptr_t align; } ptrs[] = {
      {t->hidden_states, "hidden_states", 16}, {t->hidden_states_scale, "hidden_states_scale", 16},
      {t->topk_ids, "topk_ids", 16}, {t->topk_weights, "topk_weights", 16}, {t->topk_packed, "topk_packed", 16},
      {t->w1, "w1", 16}, {t->w1_scale, "w1_scale", 16}, {t->w2, "w2", 16}, {t->w2_scale, "w2_scale", 16},
      {t->out, "out", 16}, {t->situ_beta, "situ_beta", 4}, {t->situ_linear_beta, "situ_linear_beta", 4},
      {t->alpha_gate, "alpha_gate", 4}, {t->alpha_up, "alpha_up", 4}, {t->swiglu_alpha, "swiglu_alpha", 4},
      {t->swiglu_beta, "swiglu_beta", 4}, {t->alpha_down, "alpha_down", 4},
      {t->gate_up_lora_delta, "gate_up_lora_delta", 16}, {t->activation_lora_input, "activation_lora_input", 16}};
  for (const auto& q : ptrs)
    if (reinterpret_cast<uintptr_t>(q.ptr) % q.align)
      return fail(SITU_E_BAD_SHAPE, "%s must be %u-byte aligned", q.name, (unsigned)q.align);
  if (!ws && plan->workspace_bytes) return fail(SITU_E_WORKSPACE, "workspace is NULL");
  if (ws_bytes < plan->workspace_bytes)
    return fail(SITU_E_WORKSPACE, "workspace %llu bytes < %llu needed", (unsigned long long)ws_bytes,
                (unsigned long long)plan->workspace_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(SITU_E_WORKSPACE, "workspace must be 256-byte aligned");
  return SITU_OK;
}

template <typename T>
T* at(void* ws, uint64_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

situ::RouteArgs route_args(const situ_moe_plan_t* plan, const situ_moe_tensors* t, void* ws) {
  const situ_moe_problem& p = plan->prob;
  situ::RouteArgs r;
  r.ids = p.topk_packed ? nullptr : t->topk_ids;
  r.packed = p.topk_packed ? t->topk_packed : nullptr;
  r.TK = (int64_t)p.num_tokens * p.top_k;
  r.off = p.local_expert_offset;
  r.E_l = p.local_num_experts;
  r.block_m = plan->block_m;
  r.counts = at<int32_t>(ws, plan->off_counts);
  r.offsets = at<int32_t>(ws, plan->off_offsets);
  r.mtiles = at<int32_t>(ws, plan->off_mtiles);
  r.tile_expert = at<int32_t>(ws, plan->off_tile_expert);
  r.tile_rows = at<int32_t>(ws, plan->off_tile_rows);
  r.perm = at<int32_t>(ws, plan->off_perm);
  r.inv = at<int32_t>(ws, plan->off_inv);
  r.hist = at<int32_t>(ws, plan->off_route_hist);
  r.chunk = plan->route_chunk;
  r.nblocks = plan->route_blocks;
  r.quant = situ::QuantArgs{};
  r.quant_blocks = 0;
  return r;
}

}  // namespace

extern "C" {

situ_status situ_moe_plan(const situ_moe_problem* problem, situ_moe_plan_t* plan) {
  if (!plan) return fail(SITU_E_NULL_ARG, "plan is NULL");
  situ_status st = validate(problem);
  if (st != SITU_OK) return st;
  const situ_moe_problem& p = *problem;
  int32_t f1[4], f2[4];
  const int n = valid_pairs(&p, f1, f2, 4);
  int32_t t1 = p.tactic_fc1, t2 = p.tactic_fc2;
  if (t1 == -1 && t2 == -1) {
    t1 = f1[0];
    t2 = f2[0];
  } else if (t1 == -1 || t2 == -1) {
    for (int i = 0; i < n; ++i)
      if ((t1 == -1 && f2[i] == t2) || (t2 == -1 && f1[i] == t1)) { t1 = f1[i]; t2 = f2[i]; break; }
  }
  bool ok = false;
  for (int i = 0; i < n; ++i) ok = ok || (f1[i] == t1 && f2[i] == t2);
  if (!ok) return fail(SITU_E_UNSUPPORTED, "tactic pair (%d, %d) is not valid for this problem", p.tactic_fc1, p.tactic_fc2);

  std::memset(plan, 0, sizeof(*plan));
  plan->prob = p;
  plan->fc1_tactic = t1;
  plan->fc2_tactic = t2;
  plan->block_m = find_tactic(t1)->block_m;
  const int64_t T = p.num_tokens, H = p.hidden_size, I = p.intermediate_size, TK = T * p.top_k;
  const int64_t E_l = p.local_num_experts;
  const int64_t max_mtiles = (TK + plan->block_m - 1) / plan->block_m + E_l;
  if (max_mtiles >= (int64_t)1 << 30) return fail(SITU_E_UNSUPPORTED, "too many m-tiles");
  plan->max_mtiles = (int32_t)max_mtiles;
  uint64_t off = 0;
  auto region = [&](uint64_t bytes) {
    uint64_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  plan->off_counts = region(4 * E_l);
  plan->off_offsets = region(4 * (E_l + 1));
  plan->off_mtiles = region(4 * (E_l + 1));
  plan->off_tile_expert = region(4 * max_mtiles);
  plan->off_tile_rows = region(8 * max_mtiles);
  plan->off_perm = region(4 * (TK + 64));   // a 64-row tile may read its perm entries past the end
  plan->off_inv = region(4 * TK);
  const bool w4a8 = p.act_mode == SITU_ACT_W4A8;
  const bool quant_here = w4a8 && !p.act_prequantized;
  plan->off_xq = region(quant_here ? T * H : 0);
  plan->off_xs = region(quant_here ? T * H / 32 : 0);
  plan->off_h = region(TK * I * (w4a8 ? 1 : 2));
  plan->off_hs = region(w4a8 ? TK * I / 32 : 0);
  // y: fp32, or (the 128-row w4a8 tactic) fp16 with a power-of-two scale per
  // 64 columns, which halves its write and read traffic
  plan->y_format = plan->fc2_tactic == situ::FC2_W4A8_M128 ? 1 : 0;
  if (plan->y_format == 1) {
    plan->off_y = region(align_up(TK * H * 2) + TK * ((H + 63) / 64));
    plan->off_y_exp = plan->off_y + align_up(TK * H * 2);
  } else {
    plan->off_y = region(TK * H * 4);
    plan->off_y_exp = plan->off_y;
  }
  // routing: one workgroup for small batches, else blocks of >= 4096 pairs (<= 1024 blocks)
  if (TK <= kRouteSingleMax) {
    plan->route_blocks = 1;
    plan->route_chunk = (int32_t)TK;
  } else {
    int64_t chunk = 4096;
    if ((TK + chunk - 1) / chunk > 1024) chunk = (TK + 1023) / 1024;
    plan->route_chunk = (int32_t)chunk;
    plan->route_blocks = (int32_t)((TK + chunk - 1) / chunk);
  }
  plan->off_route_hist = region(plan->route_blocks > 1 ? 4 * (uint64_t)plan->route_blocks * E_l : 0);
  plan->workspace_bytes = off;
  return SITU_OK;
}

situ_status situ_moe_valid_tactics(const situ_moe_problem* problem, int32_t* fc1, int32_t* fc2, int32_t capacity,
                                   int32_t* count) {
  situ_status st = validate(problem);
  if (st != SITU_OK) return st;
  if (!count || (capacity > 0 && (!fc1 || !fc2))) return fail(SITU_E_NULL_ARG, "output arrays are NULL");
  int32_t a[8], b[8];
  const int n = valid_pairs(problem, a, b, 8);
  for (int i = 0; i < n && i < capacity; ++i) { fc1[i] = a[i]; fc2[i] = b[i]; }
  *count = n;
  return SITU_OK;
}

situ_status situ_moe_route(const situ_moe_plan_t* plan, const situ_moe_tensors* tensors, void* workspace,
                           uint64_t workspace_bytes, void* hip_stream) {
  situ_status st = check_run_args(plan, tensors, workspace, workspace_bytes, true);
  if (st != SITU_OK) return st;
  int cus = 0;
  if ((st = device_check(&cus)) != SITU_OK) return st;
  if (plan->prob.num_tokens == 0) return SITU_OK;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  return launch_status(situ::launch_route(route_args(plan, tensors, workspace), s), "route");
}

}  // extern "C"

namespace {

situ_status run_impl(const situ_moe_plan_t* plan, const situ_moe_tensors* t, void* ws, uint64_t ws_bytes,
                     void* hip_stream, void* const* events) {
  situ_status st = check_run_args(plan, t, ws, ws_bytes, false);
  if (st != SITU_OK) return st;
  int cus = 0;
  if ((st = device_check(&cus)) != SITU_OK) return st;
  const situ_moe_problem& p = plan->prob;
  if (p.num_tokens == 0) return SITU_OK;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int64_t T = p.num_tokens, H = p.hidden_size, I = p.intermediate_size;
  const bool w4a8 = p.act_mode == SITU_ACT_W4A8;

  auto mark = [&](int i) -> situ_status {
    if (!events) return SITU_OK;
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
    return e == hipSuccess ? SITU_OK : fail(SITU_E_LAUNCH, "hipEventRecord: %s", hipGetErrorString(e));
  };
  if ((st = mark(0)) != SITU_OK) return st;
  situ::RouteArgs ra = route_args(plan, t, ws);
  const void* act = t->hidden_states;
  const uint8_t* act_scale = t->hidden_states_scale;
  if (w4a8 && !p.act_prequantized) {   // quantized in the routing launch, beside the router
    ra.quant = situ::QuantArgs{static_cast<const uint16_t*>(t->hidden_states), at<uint8_t>(ws, plan->off_xq),
                               at<uint8_t>(ws, plan->off_xs), T, (int32_t)H};
    const int64_t need = (situ::quant_pieces(ra.quant) + situ::kRouteThreads - 1) / situ::kRouteThreads;
    ra.quant_blocks = (int32_t)(need < 4 * (int64_t)cus ? need : 4 * (int64_t)cus);   // at most 4 per CU
    act = ra.quant.codes;
    act_scale = ra.quant.scales;
  }
  if ((st = launch_status(situ::launch_route(ra, s), "route")) != SITU_OK) return st;
  if ((st = mark(1)) != SITU_OK) return st;
  // (the quantization's stage is part of the routing launch's)
  if ((st = mark(2)) != SITU_OK) return st;

  situ::GemmArgs g{};
  g.offsets = ra.offsets;
  g.mtiles = ra.mtiles;
  g.tile_expert = ra.tile_expert;
  g.tile_rows = ra.tile_rows;
  g.E_l = p.local_num_experts;
  g.act_kind = p.activation;   // the SITU_ACTIVATION_* values are the kernels' kAct* kinds
  g.beta = p.activation == SITU_ACTIVATION_SITU ? t->situ_beta
                                                : p.activation == SITU_ACTIVATION_SWIGLU_BIAS ? t->swiglu_alpha : nullptr;
  g.lbeta = p.activation == SITU_ACTIVATION_SITU ? t->situ_linear_beta
                                                 : p.activation == SITU_ACTIVATION_SWIGLU_BIAS ? t->swiglu_beta : nullptr;
  g.alpha_g = t->alpha_gate;
  g.alpha_u = t->alpha_up;
  g.nvfp4 = p.weight_format == SITU_WEIGHTS_NVFP4 ? 1 : 0;
  g.tiled = p.weight_format == SITU_WEIGHTS_MXFP4_TILED ? 1 : 0;

  // FC1 + SiTU
  g.act = act;
  g.act_scale = w4a8 ? act_scale : nullptr;
  g.perm = ra.perm;
  g.top_k = p.top_k;
  g.w = t->w1;
  g.ws = t->w1_scale;
  g.K = (int32_t)H;
  g.N = (int32_t)I;
  g.out = at<void>(ws, plan->off_h);
  g.out_scale = w4a8 ? at<uint8_t>(ws, plan->off_hs) : nullptr;
  g.lora_delta = t->gate_up_lora_delta;
  g.lora_out = t->activation_lora_input;
  if (t->activation_lora_input &&
      (st = launch_status(situ::launch_zero_nonlocal_rows(ra.inv, t->activation_lora_input, (int64_t)T * p.top_k,
                                                          (int32_t)I, s), "lora rows")) != SITU_OK)
    return st;
  const bool fused = plan->fc1_tactic == situ::FC1_FUSED_W4A16_M16 || plan->fc1_tactic == situ::FC1_FUSED_W4A8_M16;
  if (!fused) {
    if ((st = launch_status(situ::launch_fc1(plan->fc1_tactic, g, plan->max_mtiles, cus, s), "fc1")) != SITU_OK) return st;
    if ((st = mark(3)) != SITU_OK) return st;
  }
  const situ::GemmArgs g1 = g;

  // FC2
  g.act = at<void>(ws, plan->off_h);
  g.act_scale = w4a8 ? at<uint8_t>(ws, plan->off_hs) : nullptr;
  g.perm = nullptr;
  g.lora_delta = nullptr;
  g.lora_out = nullptr;
  g.w = t->w2;
  g.ws = t->w2_scale;
  g.K = (int32_t)I;
  g.N = (int32_t)H;
  g.out = at<void>(ws, plan->off_y);
  g.out_scale = plan->y_format == 1 ? at<uint8_t>(ws, plan->off_y_exp) : nullptr;
  g.out_rows = (int32_t)((int64_t)T * p.top_k);
  if (fused) {   // one launch for both GEMMs: its time is the FC1 stage's
    if ((st = launch_status(situ::launch_fused_decode(g1, g, w4a8, plan->max_mtiles, cus, s), "fused fc1+fc2")) != SITU_OK)
      return st;
    if ((st = mark(3)) != SITU_OK) return st;
  } else if ((st = launch_status(situ::launch_fc2(plan->fc2_tactic, g, plan->max_mtiles, cus, s), "fc2")) != SITU_OK) {
    return st;
  }
  if ((st = mark(4)) != SITU_OK) return st;

  // combine
  const bool y16 = plan->y_format == 1;
  situ::CombineArgs c{y16 ? nullptr : at<float>(ws, plan->off_y), y16 ? at<uint16_t>(ws, plan->off_y) : nullptr,
                      y16 ? at<uint8_t>(ws, plan->off_y_exp) : nullptr, ra.inv,
                      p.topk_packed ? nullptr : t->topk_weights,
                      p.topk_packed ? t->topk_packed : nullptr, t->out, T, (int32_t)H, p.top_k,
                      p.out_dtype == SITU_OUT_BF16 ? 1 : 0, t->alpha_down,
                      p.topk_packed ? nullptr : t->topk_ids, p.local_expert_offset};
  if ((st = launch_status(situ::launch_combine(c, s), "combine")) != SITU_OK) return st;
  return mark(5);
}

}  // namespace

extern "C" {

situ_status situ_moe_run(const situ_moe_plan_t* plan, const situ_moe_tensors* t, void* ws, uint64_t ws_bytes,
                         void* hip_stream) {
  return run_impl(plan, t, ws, ws_bytes, hip_stream, nullptr);
}

situ_status situ_moe_run_profiled(const situ_moe_plan_t* plan, const situ_moe_tensors* t, void* ws,
                                  uint64_t ws_bytes, void* hip_stream, void* const* hip_events, int32_t n_events) {
  if (!hip_events || n_events != 6) return fail(SITU_E_NULL_ARG, "run_profiled needs 6 hipEvent_t handles");
  for (int i = 0; i < 6; ++i)
    if (!hip_events[i]) return fail(SITU_E_NULL_ARG, "hip_events[%d] is NULL", i);
  return run_impl(plan, t, ws, ws_bytes, hip_stream, hip_events);
}

situ_status situ_moe_tile_weights(const uint8_t* w, const uint8_t* w_scale, int32_t experts, int32_t rows, int32_t k,
                                  uint8_t* w_tiled, uint8_t* scale_tiled, void* hip_stream) {
  if (experts <= 0 || rows <= 0 || rows % 16 || k <= 0 || k % 32)
    return fail(SITU_E_BAD_SHAPE, "experts %d, rows %d (multiple of 16), k %d (multiple of 32)", experts, rows, k);
  if (situ::expert_w_bytes(true, rows, k) >= (uint64_t)1 << 31)
    return fail(SITU_E_BAD_SHAPE, "one expert's tiled weights exceed 2 GiB");
  if (!w || !w_scale || !w_tiled || !scale_tiled) return fail(SITU_E_NULL_ARG, "a pointer is NULL");
  if (reinterpret_cast<uintptr_t>(w) % 16 || reinterpret_cast<uintptr_t>(w_tiled) % 16)
    return fail(SITU_E_BAD_SHAPE, "w and w_tiled must be 16-byte aligned");
  int cus = 0;
  situ_status st = device_check(&cus);
  if (st != SITU_OK) return st;
  return launch_status(situ::launch_tile_weights(w, w_scale, w_tiled, scale_tiled, experts, rows, k,
                                                 static_cast<hipStream_t>(hip_stream)), "tile weights");
}

situ_status situ_moe_quantize_mxfp8(const uint16_t* x_bf16, int64_t rows, int32_t cols, uint8_t* codes,
                                    uint8_t* scales, void* hip_stream) {
  if (rows < 0 || cols <= 0 || cols % 32) return fail(SITU_E_BAD_SHAPE, "rows %lld, cols %d (multiple of 32)",
                                                      (long long)rows, cols);
  if (rows == 0) return SITU_OK;
  if (!x_bf16 || !codes || !scales) return fail(SITU_E_NULL_ARG, "a pointer is NULL");
  int cus = 0;
  situ_status st = device_check(&cus);
  if (st != SITU_OK) return st;
  situ::QuantArgs q{x_bf16, codes, scales, rows, cols};
  return launch_status(situ::launch_quant_mxfp8(q, static_cast<hipStream_t>(hip_stream)), "quantize");
}

situ_status situ_moe_measure_mfma_peak(int32_t iters, double* tflops) {
  if (!tflops) return fail(SITU_E_NULL_ARG, "tflops is NULL");
  if (iters < 1 || iters > (1 << 20)) return fail(SITU_E_BAD_SHAPE, "iters %d not in [1, 2^20]", iters);
  int cus = 0;
  situ_status st = device_check(&cus);
  if (st != SITU_OK) return st;
  const int blocks = 4 * cus;   // 16 waves per CU: 4 per SIMD
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipStreamCreate(&s);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = situ::launch_mfma_peak(iters, blocks, s);   // warm-up (clocks, code load)
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) e = situ::launch_mfma_peak(iters, blocks, s);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e1) (void)hipEventDestroy(e1);
  if (e0) (void)hipEventDestroy(e0);
  if (s) (void)hipStreamDestroy(s);
  if (e != hipSuccess) return launch_status(e, "MFMA peak measurement");
  const double flops = (double)blocks * 4.0 * (double)iters * 8.0 * 65536.0;
  *tflops = ms > 0.f ? flops / (ms * 1e-3) / 1e12 : 0.0;
  return SITU_OK;
}

const char* situ_moe_status_string(situ_status s) {
  switch (s) {
    case SITU_OK: return "SITU_OK";
    case SITU_E_NULL_ARG: return "SITU_E_NULL_ARG";
    case SITU_E_BAD_SHAPE: return "SITU_E_BAD_SHAPE";
    case SITU_E_UNSUPPORTED: return "SITU_E_UNSUPPORTED";
    case SITU_E_MISSING_SCALE: return "SITU_E_MISSING_SCALE";
    case SITU_E_DEVICE: return "SITU_E_DEVICE";
    case SITU_E_WORKSPACE: return "SITU_E_WORKSPACE";
    case SITU_E_LAUNCH: return "SITU_E_LAUNCH";
  }
  return "SITU_E_UNKNOWN";
}

const char* situ_moe_last_error(void) { return g_last_error.c_str(); }

const char* situ_moe_build_info(void) {
  static const std::string info = [] {
    std::string s = "situ_moe abi " + std::to_string(SITU_MOE_ABI_VERSION) + "; target gfx950; rev " SITU_GIT_REV
                    "; tactics:";
    for (const auto& t : kTactics) s += std::string(" ") + std::to_string(t.id) + "=" + t.name;
    return s;
  }();
  return info.c_str();
}

const char* situ_moe_tactic_name(int32_t tactic) {
  const TacticInfo* t = find_tactic(tactic);
  return t ? t->name : nullptr;
}

int32_t situ_moe_abi_version(void) { return SITU_MOE_ABI_VERSION; }

}  // extern "C"

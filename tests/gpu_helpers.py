"""Shared helpers of the GPU tests: move seeded inputs to the device, run the
layer through the C ABI, compare with the oracle."""

import functools

import numpy as np
import torch

import block_scaled_mxfp4_amd as B
import synthetic as S
from oracle import formats as F
from oracle import moe as M

# The parity bar: cosine >= 0.9995 and max-abs <= 1e-2 * RMS(oracle) on the
# fp32 outputs over every element, zero rows included.
COS_MIN = 0.9995
MAXABS_FRAC = 1e-2


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to("cuda")


@functools.lru_cache(maxsize=2)
def config_inputs(cfg):
    return S.generate(cfg)


def run_layer(inp, spec, *, mode=None, out_dtype="f32", tactic=(-1, -1), prequantized=False,
              keep=False, workspace=None):
    """Run the layer on the GPU; returns (out numpy, plan, workspace, device tensors)."""
    mode = mode or spec.get("mode", "w4a16")
    T, H, I, k = spec["T"], spec["H"], spec["I"], spec["k"]
    packed = inp.get("topk_packed") is not None
    prob = B.make_problem(num_tokens=T, hidden_size=H, intermediate_size=I, num_experts=spec["E_g"],
                          local_expert_offset=spec["off"], local_num_experts=spec["E_l"], top_k=k,
                          act_mode=mode, act_prequantized=prequantized, topk_packed=packed,
                          out_dtype=out_dtype, tactic=tactic)
    plan = B.situ_moe_plan(prob)
    d = {}
    if prequantized:
        codes, scales = F.mx_quantize(F.bf16_to_f64(inp["hidden_states"]), "e4m3")
        d["hidden_states"] = dev(codes)
        d["hidden_states_scale"] = dev(scales)
    else:
        d["hidden_states"] = dev(inp["hidden_states"])
    if packed:
        d["topk_packed"] = dev(inp["topk_packed"])
    else:
        d["topk_ids"] = dev(inp["topk_ids"].astype(np.int32))
        d["topk_weights"] = dev(inp["topk_weights"])
    for key in ("w1", "w1_scale", "w2", "w2_scale", "situ_beta", "situ_linear_beta", "alpha_gate", "alpha_up"):
        if inp.get(key) is not None:
            d[key] = dev(inp[key])
    d["out"] = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32, device="cuda")
    ts = B.make_tensors(prob, **d)
    ws = workspace if workspace is not None else B.new_workspace(plan)
    B.situ_moe_run(plan, ts, ws)
    torch.cuda.synchronize()
    out = d["out"].float().cpu().numpy() if out_dtype == "f32" else \
        d["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    return out, plan, ws, d


def oracle_out(inp, spec, mode=None, tokens=None, prequantized=False, keep=False):
    mode = mode or spec.get("mode", "w4a16")
    o_inp = dict(inp)
    if prequantized:
        codes, scales = F.mx_quantize(F.bf16_to_f64(inp["hidden_states"]), "e4m3")
        o_inp["hidden_states"], o_inp["hidden_states_scale"] = codes, scales
    return M.moe_forward(o_inp, local_expert_offset=spec["off"], local_num_experts=spec["E_l"],
                         act_mode=mode, act_prequantized=prequantized, tokens=tokens, keep_intermediates=keep)


def parity(got, want, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = np.sqrt(np.mean(want ** 2))
    maxabs = np.max(np.abs(got - want)) if got.size else 0.0
    denom = np.linalg.norm(got) * np.linalg.norm(want)
    cos = float(np.dot(got.ravel(), want.ravel()) / denom) if denom > 0 else (1.0 if maxabs == 0 else 0.0)
    msg = f"{what}: cosine {cos:.7f}, max-abs {maxabs:.3e} = {maxabs / max(rms, 1e-300):.2e} x RMS {rms:.3e}"
    print(msg, flush=True)
    assert cos >= COS_MIN, msg
    assert maxabs <= MAXABS_FRAC * rms, msg
    return cos, maxabs / max(rms, 1e-300)


def ws_region(plan, ws, name, dtype, shape):
    return B.workspace_view(plan, ws, name, dtype, shape).cpu().numpy()

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


# Relative distance to a rounding midpoint below which either rounding of an
# element of h is a correct result, for the SiTU evaluation alone: the GPU
# evaluates SiTU in fp32 within a few ulp (~1e-7), so 2^-16 leaves a wide
# margin.
AMBIGUITY = 2.0 ** -16


def acc_error_ulps(K):
    """Bound, in fp32 ulps of sum_k |x_k w_k|, of how far an FC1 output the
    GPU accumulates (exact block products summed in fp32, in an order other
    than the oracle's float64 sum) may lie from the oracle's: a fixed part
    for the sums inside the matrix-core instructions plus one ulp per 64
    products.  Measured on the device at K = 640: flips that needed up to
    10 ulp on elements whose flip matters (one tiny element of a block
    needed 23)."""
    return 8 + K / 64


def h_uncertainty(inp, spec, ref, mode):
    """Per element of ref["h_pre"], a bound of |GPU h - oracle h| before the
    rounding point: the FC1 accumulation bound (acc_error_ulps times
    sum_k |x_k w_k| on the gate and up sums, propagated through alpha and
    SiTU by evaluating SiTU at the perturbed inputs) plus the SiTU
    evaluation error (AMBIGUITY relative)."""
    I, H = spec["I"], spec["H"]
    eps = acc_error_ulps(H) * 2.0 ** -24
    xf = M.activations(inp, mode, False)[0]
    pairs, offsets, perm = ref["pairs"], ref["offsets"], ref["perm"]
    k = spec["k"]
    acc = ref["acc"]
    hpre = ref["h_pre"]
    out = np.zeros_like(hpre)
    E_l = spec["E_l"]
    ones = np.ones(E_l, np.float32)
    a_g = ones if inp.get("alpha_gate") is None else np.asarray(inp["alpha_gate"], np.float64)
    a_u = ones if inp.get("alpha_up") is None else np.asarray(inp["alpha_up"], np.float64)
    beta = np.asarray(inp["situ_beta"], np.float64)
    lbeta = np.asarray(inp["situ_linear_beta"], np.float64)
    for l in range(E_l):
        q = np.nonzero((pairs >= offsets[l]) & (pairs < offsets[l + 1]))[0]
        if q.size == 0:
            continue
        W = np.abs(F.dequant_mxfp4(inp["w1"][l], inp["w1_scale"][l]))
        S = np.abs(xf[perm[pairs[q]] // k]) @ W.T               # [n, 2I] sums of |x w|
        g = a_g[l] * acc[q, :I]
        u = a_u[l] * acc[q, I:]
        dg = a_g[l] * eps * S[:, :I]
        du = a_u[l] * eps * S[:, I:]
        h0 = M.situ(g, u, beta[l], lbeta[l])
        d = np.zeros_like(h0)
        for sg, su in ((1, 0), (-1, 0), (0, 1), (0, -1)):
            d = np.maximum(d, np.abs(M.situ(g + sg * dg, u + su * du, beta[l], lbeta[l]) - h0))
        out[q] = 1.5 * d + AMBIGUITY * np.abs(hpre[q])
    return out


def _bf16_ambiguity(v, tol=None):
    """Size of the other bf16 rounding choice of v where v lies within tol
    (default AMBIGUITY * |v|) of a bf16 rounding midpoint, else 0."""
    v = np.asarray(v, np.float64)
    q = F.bf16_to_f64(F.f32_to_bf16_rne(v.astype(np.float32)))
    a = np.abs(v)
    tol = AMBIGUITY * a if tol is None else tol
    ulp = np.ldexp(1.0, F.floor_log2(np.where(a > 0, a, 1.0)) - 7)
    amb = (a > 0) & (ulp / 2 - np.abs(v - q) <= tol)
    return np.where(amb, ulp, 0.0)


def _mxfp8_ambiguity(v, tol=None):
    """The same for MXFP8 rows (32-element blocks along the last axis): an
    element within tol of an E4M3 rounding midpoint under its block scale, or
    a whole block whose max lies within its tol of a power of two (two
    candidate E8M0 scales), may round either way."""
    v = np.asarray(v, np.float64)
    n, I = v.shape
    tol = AMBIGUITY * np.abs(v) if tol is None else np.asarray(tol, np.float64)
    codes, sc = F.mx_quantize(v, "e4m3")
    q = F.mx_dequantize(codes, sc, "e4m3")
    scale = np.repeat(F.decode_e8m0(sc), 32, axis=-1)
    s = v / scale
    a = np.abs(s)
    spacing = np.where(a < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, F.floor_log2(np.where(a > 0, a, 1.0)) - 3))
    amb = (a > 0) & (a < 448.0) & (spacing / 2 - np.abs(s - q / scale) <= tol / scale)
    d = np.where(amb, spacing * scale, 0.0)
    # block scale ambiguity: the block max within its element's tol of a power of two
    av = np.abs(v).reshape(n, I // 32, 32)
    arg = av.argmax(-1)
    blocks = np.take_along_axis(av, arg[..., None], -1)[..., 0]
    btol = np.take_along_axis(tol.reshape(n, I // 32, 32), arg[..., None], -1)[..., 0]
    p2 = np.ldexp(1.0, F.floor_log2(np.where(blocks > 0, blocks, 1.0)))
    near = (blocks > 0) & ((blocks - p2 <= btol) | (2 * p2 - blocks <= btol))
    if near.any():
        for sgn in (-1, 1):
            alt_sc = np.clip(sc.astype(np.int64) + sgn, 0, 254).astype(np.uint8)
            alt_scale = np.repeat(F.decode_e8m0(alt_sc), 32, axis=-1)
            alt_q = F.mx_dequantize(F.encode_e4m3(v / alt_scale), alt_sc, "e4m3")
            dd = np.abs(alt_q - q) * np.repeat(near, 32, axis=-1)
            d = np.maximum(d, dd)
    return d


def _pair_effects(inp, spec, ref, mode):
    """{pair index: bound of the change of that pair's FC2 output y} for the
    pairs whose h holds an element on a rounding boundary (see AMBIGUITY)."""
    hpre = ref["h_pre"]
    tol = h_uncertainty(inp, spec, ref, mode)
    d = _bf16_ambiguity(hpre, tol) if mode == "w4a16" else _mxfp8_ambiguity(hpre, tol)
    rows = np.nonzero(d.any(axis=1))[0]
    pairs = ref["pairs"]
    offsets = ref["offsets"]
    effect = {}
    for q in rows:
        p = int(pairs[q])
        l = int(np.searchsorted(offsets, p, side="right") - 1)
        W2 = np.abs(F.dequant_mxfp4(inp["w2"][l], inp["w2_scale"][l]))
        effect[p] = W2 @ d[q]
    return effect


def rounding_allowance(inp, spec, ref, mode):
    """Per-output-element bound of how far a correct result may differ from
    the oracle's because of the rounding point after FC1 alone (see
    AMBIGUITY).  ref must come from oracle_out(..., keep=True).  Zero for
    almost every element."""
    effect = _pair_effects(inp, spec, ref, mode)
    tokens = ref["tokens"]
    A = np.zeros((tokens.shape[0], spec["H"]))
    if not effect:
        return A
    ids, wts = M.topk_of(inp)
    k = spec["k"]
    inv = ref["inv"].reshape(-1, k)
    for i, t in enumerate(tokens):
        for s_ in range(k):
            p = int(inv[t, s_])
            if p in effect:
                A[i] += abs(wts[t, s_]) * effect[p]
    return A


def y_rounding_allowance(inp, spec, ref, mode, n_pairs):
    """The same bound for the per-pair FC2 outputs y (rows by pair index)."""
    A = np.zeros((n_pairs, spec["H"]))
    for p, e in _pair_effects(inp, spec, ref, mode).items():
        A[p] = e
    return A


def parity(got, want, what="", allowance=None):
    """The parity bar: cosine >= 0.9995 and max-abs <= 1e-2 x RMS(oracle), on
    the fp32 outputs; where allowance is given, the part of an element's
    difference that a legitimately different rounding decision explains
    (rounding_allowance) is not counted against max-abs."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = np.sqrt(np.mean(want ** 2))
    diff = np.abs(got - want)
    raw = np.max(diff) if got.size else 0.0
    if allowance is not None:
        diff = np.maximum(diff - allowance, 0.0)
    maxabs = np.max(diff) if got.size else 0.0
    denom = np.linalg.norm(got) * np.linalg.norm(want)
    cos = float(np.dot(got.ravel(), want.ravel()) / denom) if denom > 0 else (1.0 if maxabs == 0 else 0.0)
    n_amb = int(np.count_nonzero(allowance)) if allowance is not None else 0
    msg = (f"{what}: cosine {cos:.7f}, max-abs {maxabs:.3e} = {maxabs / max(rms, 1e-300):.2e} x RMS {rms:.3e}"
           f" (raw {raw / max(rms, 1e-300):.2e}; {n_amb} elements with a rounding allowance)")
    print(msg, flush=True)
    assert cos >= COS_MIN, msg
    assert maxabs <= MAXABS_FRAC * rms, msg
    return cos, maxabs / max(rms, 1e-300)


def ws_region(plan, ws, name, dtype, shape):
    return B.workspace_view(plan, ws, name, dtype, shape).cpu().numpy()


def read_y(plan, ws, P, H):
    """The FC2 output rows y [P, H] as float64, decoded from the plan's y
    format: fp32, or fp16 with exponent byte E (scale 2^(E-127)) per 64
    columns."""
    if plan.y_format == 0:
        return ws_region(plan, ws, "y", torch.float32, (P, H)).astype(np.float64)
    nb = (H + 63) // 64
    y16 = ws_region(plan, ws, "y", torch.float16, (P, H)).astype(np.float64)
    rows = plan.prob.num_tokens * plan.prob.top_k
    e = ws_region(plan, ws, "y_exp", torch.uint8, (rows, nb))[:P].astype(np.int64)
    assert np.all((e >= 1) & (e <= 254))
    return y16 * np.ldexp(1.0, np.repeat(e, 64, axis=1)[:, :H] - 127)

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
              keep=False, workspace=None, lora_out=False, tiled=False):
    """Run the layer on the GPU; returns (out numpy, plan, workspace, device tensors).
    The activation and weight format come from spec ("activation",
    "weight_format"); lora_out=True also asks for the down-LoRA input rows
    (device tensor d["activation_lora_input"]); tiled=True hands the layer
    the MXFP4 weights in the fragment-tiled layout, made from the row-major
    ones by situ_moe_tile_weights."""
    mode = mode or spec.get("mode", "w4a16")
    T, H, I, k = spec["T"], spec["H"], spec["I"], spec["k"]
    packed = inp.get("topk_packed") is not None
    wf = spec.get("weight_format", "mxfp4")
    if tiled:
        assert wf == "mxfp4"
        wf = "mxfp4_tiled"
    prob = B.make_problem(num_tokens=T, hidden_size=H, intermediate_size=I, num_experts=spec["E_g"],
                          local_expert_offset=spec["off"], local_num_experts=spec["E_l"], top_k=k,
                          act_mode=mode, act_prequantized=prequantized, topk_packed=packed,
                          out_dtype=out_dtype, tactic=tactic, activation=spec.get("activation", "situ"),
                          weight_format=wf)
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
    for key in ("w1", "w1_scale", "w2", "w2_scale", "situ_beta", "situ_linear_beta", "alpha_gate", "alpha_up",
                "swiglu_alpha", "swiglu_beta", "alpha_down"):
        if inp.get(key) is not None:
            d[key] = dev(inp[key])
    if tiled:
        d["w1"], d["w1_scale"] = B.situ_moe_tile_weights(d["w1"], d["w1_scale"])
        d["w2"], d["w2_scale"] = B.situ_moe_tile_weights(d["w2"], d["w2_scale"])
    if isinstance(inp.get("gate_up_lora_delta"), torch.Tensor):   # already on the device
        d["gate_up_lora_delta"] = inp["gate_up_lora_delta"]
    elif inp.get("gate_up_lora_delta") is not None:
        d["gate_up_lora_delta"] = dev(np.asarray(inp["gate_up_lora_delta"]).reshape(T * k, 2 * I))
    if lora_out:   # filled with a pattern the layer must overwrite everywhere
        d["activation_lora_input"] = torch.full((T * k, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    d["out"] = torch.empty((T, H), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32, device="cuda")
    ts = B.make_tensors(prob, **d)
    ws = workspace if workspace is not None else B.new_workspace(plan)
    B.situ_moe_run(plan, ts, ws)
    torch.cuda.synchronize()
    out = d["out"].float().cpu().numpy() if out_dtype == "f32" else \
        d["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    return out, plan, ws, d


def oracle_out(inp, spec, mode=None, tokens=None, prequantized=False, keep=False, h_given=None,
               want_act_lora=False):
    mode = mode or spec.get("mode", "w4a16")
    o_inp = dict(inp)
    if prequantized:
        codes, scales = F.mx_quantize(F.bf16_to_f64(inp["hidden_states"]), "e4m3")
        o_inp["hidden_states"], o_inp["hidden_states_scale"] = codes, scales
    return M.moe_forward(o_inp, local_expert_offset=spec["off"], local_num_experts=spec["E_l"],
                         act_mode=mode, act_prequantized=prequantized, tokens=tokens, keep_intermediates=keep,
                         activation=spec.get("activation", "situ"),
                         weight_format=spec.get("weight_format", "mxfp4"), h_given=h_given,
                         want_act_lora=want_act_lora)


# Relative distance to a rounding midpoint below which either rounding of an
# element of h is a correct result, for the activation's evaluation alone:
# the GPU evaluates it in fp32 within a few ulp (~1e-7), so 2^-16 leaves a
# wide margin.
AMBIGUITY = 2.0 ** -16


def acc_error_ulps(K):
    """Bound, in fp32 ulps of sum_k |x_k w_k|, of how far an FC1 output the
    GPU accumulates (exact products summed in fp32, in an order other than
    the oracle's float64 sum) may lie from the oracle's: a fixed part for the
    sums inside the matrix-core instructions plus one ulp per 64 products.
    The bf16 matrix-core instruction stays within 1.5 ulps per 32 products
    (measured on the device over 4096 random 16x16x32 tiles)."""
    return 8 + K / 64


# The block-scaled FP8 x FP4 matrix-core instruction (16x16x128) does not
# sum its products to fp32 accuracy: measured on the device, each
# instruction's result is off by up to 2^-12.1 of the largest |product| of
# its 128-long K chunk (1024-2048 random tiles per input kind: Gaussian
# activations, wide weight and activation scales, spiky activations; chains
# of 3 to 28 instructions as in the GEMM kernels), i.e. up to ~700 fp32 ulps
# of sum |x w| where the products span many binades.  The w4a8 bound adds
# MXFP8_MFMA_REL (twice the largest seen) times the sum over K chunks of the
# chunk's largest |product|.
MXFP8_MFMA_REL = 2.0 ** -11


def _chunk_max_sum(xa, wa):
    """sum over 128-wide K chunks of max_k |x_k w_k|, row by row ([n, K] each)."""
    n, K = xa.shape
    Kp = -(-K // 128) * 128
    prod = np.zeros((n, Kp))
    prod[:, :K] = np.abs(xa) * np.abs(wa)
    return prod.reshape(n, Kp // 128, 128).max(axis=2).sum(axis=1)


def _ulp32(v):
    a = np.abs(np.asarray(v, np.float64))
    return np.ldexp(1.0, np.maximum(F.floor_log2(np.where(a > 0, a, 1.0)), -126) - 23)


def h_tolerance(inp, spec, ref, mode, q, cols):
    """Bound of |GPU h - oracle h| before the rounding point for the selected
    elements (q: rows of ref's computed pairs, cols: columns < I): the FC1
    accumulation bound (acc_error_ulps times sum_k |x_k w_k| on the gate and
    up sums; in w4a8 plus MXFP8_MFMA_REL times the sum of the K chunks'
    largest |x_k w_k|; plus two fp32 ulps of g and u for their own
    rounding), carried through the activation by evaluating it at the
    perturbed inputs (x1.5), plus AMBIGUITY relative for the activation's
    evaluation."""
    q = np.asarray(q, np.int64)
    cols = np.asarray(cols, np.int64)
    out = np.zeros(q.shape[0])
    if q.size == 0:
        return out
    I, H, k, E_l = spec["I"], spec["H"], spec["k"], spec["E_l"]
    act = spec.get("activation", "situ")
    dequant = F.dequant_mxfp4 if spec.get("weight_format", "mxfp4") == "mxfp4" else F.dequant_nvfp4
    eps = acc_error_ulps(H) * 2.0 ** -24
    xf = M.activations(inp, mode, False)[0]
    pairs, offsets, perm = ref["pairs"], ref["offsets"], ref["perm"]
    acc, hpre = ref["acc"], ref["h_pre"]
    ones = np.ones(E_l, np.float32)
    a_g = ones if inp.get("alpha_gate") is None else np.asarray(inp["alpha_gate"], np.float64)
    a_u = ones if inp.get("alpha_up") is None else np.asarray(inp["alpha_up"], np.float64)
    p0, p1 = M.activation_params(inp, act, E_l)
    delta = inp.get("gate_up_lora_delta")
    if delta is not None:
        delta = F.bf16_to_f64(np.asarray(delta).reshape(-1, 2 * I))
    expert = np.searchsorted(offsets, pairs[q], side="right") - 1
    for l in np.unique(expert):
        sel = np.nonzero(expert == l)[0]
        qs, cs = q[sel], cols[sel]
        uq, qi = np.unique(qs, return_inverse=True)
        uc, ci = np.unique(cs, return_inverse=True)
        rows = np.concatenate([uc, I + uc])
        W = np.abs(dequant(inp["w1"][l][rows], inp["w1_scale"][l][rows]))
        Sx = np.abs(xf[perm[pairs[uq]] // k]) @ W.T                       # [n_q, 2 n_c]
        Sg, Su = Sx[qi, ci], Sx[qi, uc.size + ci]
        ag_err, au_err = eps * Sg, eps * Su
        if mode == "w4a8":
            xrows = xf[perm[pairs[qs]] // k]
            for b0 in range(0, qs.size, 1024):
                bs = slice(b0, b0 + 1024)
                ag_err[bs] += MXFP8_MFMA_REL * _chunk_max_sum(xrows[bs], W[ci[bs]])
                au_err[bs] += MXFP8_MFMA_REL * _chunk_max_sum(xrows[bs], W[uc.size + ci[bs]])
        g = a_g[l] * acc[qs, cs]
        u = a_u[l] * acc[qs, I + cs]
        if delta is not None:
            j = perm[pairs[qs]]
            g = g + delta[j, cs]
            u = u + delta[j, I + cs]
        # the GPU adds a LoRA delta as acc + d / alpha: a few more roundings of
        # the terms' own size
        extra_g = 2 * (_ulp32(a_g[l] * acc[qs, cs]) + _ulp32(g - a_g[l] * acc[qs, cs]))
        extra_u = 2 * (_ulp32(a_u[l] * acc[qs, I + cs]) + _ulp32(u - a_u[l] * acc[qs, I + cs]))
        dg = a_g[l] * ag_err + 2 * _ulp32(g) + extra_g
        du = a_u[l] * au_err + 2 * _ulp32(u) + extra_u
        h0 = M.gated_activation(act, g, u, p0[l], p1[l])
        d = np.zeros_like(h0)
        for sg, su in ((1, 0), (-1, 0), (0, 1), (0, -1)):
            d = np.maximum(d, np.abs(M.gated_activation(act, g + sg * dg, u + su * du, p0[l], p1[l]) - h0))
        out[sel] = 1.5 * d + AMBIGUITY * np.abs(hpre[qs, cs])
    return out


def _bf16_of(v):
    return F.bf16_to_f64(F.f32_to_bf16_rne(np.asarray(v, np.float64).astype(np.float32)))


def _e8m0_for_e4m3(amax):
    """OCP MX scale code of an MXFP8 block from its |max| (0 for a zero block)."""
    amax = np.asarray(amax, np.float64)
    e = np.where(amax > 0, F.floor_log2(np.where(amax > 0, amax, 1.0)) - F.E4M3_EMAX, -127)
    return (np.clip(e, -127, 127) + 127).astype(np.int64)


def gpu_h(plan, ws, P, I, mode):
    """The FC1 output rows the GPU left in the workspace, [P, I]: values
    (float64), and in w4a8 also the E4M3 codes and E8M0 scale codes."""
    if mode == "w4a16":
        bits = ws_region(plan, ws, "h", torch.int16, (P, I)).view(np.uint16)
        return dict(vals=F.bf16_to_f64(bits))
    codes = ws_region(plan, ws, "h", torch.uint8, (P, I))
    sc = ws_region(plan, ws, "hs", torch.uint8, (P, I // 32))
    return dict(vals=F.mx_dequantize(codes, sc, "e4m3"), codes=codes, scales=sc)


def check_h(hg, inp, spec, ref, mode, what=""):
    """Every element of the GPU's h must be the oracle's rounding of its
    pre-rounding value, or -- only where that value lies within its
    tolerance (h_tolerance) of a rounding boundary -- the rounding of another
    value inside the tolerance: in w4a16 a bf16 value between the roundings
    of h_pre - tol and h_pre + tol; in w4a8 an E8M0 block scale between the
    scales of the block maxima reachable inside the tolerances, and under the
    GPU's own scale an E4M3 value between the encodings of h_pre - tol and
    h_pre + tol.  Checks the rows of ref's computed pairs; returns the number
    of elements that differ from the oracle's own rounding."""
    pairs = ref["pairs"]
    I = spec["I"]
    got = hg["vals"][pairs]
    want, hpre = ref["h"], ref["h_pre"]
    if mode == "w4a16":
        q, c = np.nonzero(got != want)
        tol = h_tolerance(inp, spec, ref, mode, q, c)
        lo = _bf16_of(hpre[q, c] - tol)
        hi = _bf16_of(hpre[q, c] + tol)
        bad = ~((got[q, c] >= lo) & (got[q, c] <= hi))
        n_diff = q.size
    else:
        gs = hg["scales"][pairs].astype(np.int64)
        ws_ = F.mx_block_scale_codes(hpre, F.E4M3_EMAX).astype(np.int64)
        # blocks whose scale or any element differs from the oracle's
        diff_el = got != want
        blk = (gs != ws_) | diff_el.reshape(diff_el.shape[0], I // 32, 32).any(axis=-1)
        bq, bb = np.nonzero(blk)
        q = np.repeat(bq, 32)
        c = (bb[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
        tol = h_tolerance(inp, spec, ref, mode, q, c).reshape(-1, 32)
        v = hpre[bq[:, None], bb[:, None] * 32 + np.arange(32)[None, :]]
        amax_lo = np.max(np.maximum(np.abs(v) - tol, 0.0), axis=1)
        amax_hi = np.max(np.abs(v) + tol, axis=1)
        s_ok = (gs[bq, bb] >= _e8m0_for_e4m3(amax_lo)) & (gs[bq, bb] <= _e8m0_for_e4m3(amax_hi))
        scale = np.ldexp(1.0, gs[bq, bb] - 127)[:, None]
        lo = F.decode_e4m3(F.encode_e4m3((v - tol) / scale)) * scale
        hi = F.decode_e4m3(F.encode_e4m3((v + tol) / scale)) * scale
        gv = got[bq[:, None], bb[:, None] * 32 + np.arange(32)[None, :]]
        el_ok = (gv >= lo) & (gv <= hi)
        bad = ~(el_ok & s_ok[:, None])
        n_diff = int(np.count_nonzero(diff_el)) + int(np.count_nonzero(gs != ws_))
    n_bad = int(np.count_nonzero(bad))
    print(f"{what}: h {got.size} elements, {n_diff} differ from the oracle's rounding, {n_bad} outside its "
          f"tolerance", flush=True)
    if n_bad:   # name the first offenders: pair, column, values, tolerance, accumulators
        if mode == "w4a16":
            qq, cc = q[bad], c[bad]
            for i in range(min(5, qq.size)):
                print(f"  pair {int(pairs[qq[i]])} col {int(cc[i])}: gpu {got[qq[i], cc[i]]!r} oracle "
                      f"{want[qq[i], cc[i]]!r} pre {hpre[qq[i], cc[i]]!r} acc_g {ref['acc'][qq[i], cc[i]]!r} "
                      f"acc_u {ref['acc'][qq[i], I + cc[i]]!r}", flush=True)
        else:
            bi, ei = np.nonzero(bad)
            for i in range(min(5, bi.size)):
                qq, cc = bq[bi[i]], bb[bi[i]] * 32 + ei[i]
                print(f"  pair {int(pairs[qq])} col {int(cc)}: gpu {gv[bi[i], ei[i]]!r} oracle {want[qq, cc]!r} "
                      f"pre {hpre[qq, cc]!r} tol {tol[bi[i], ei[i]]!r} interval [{lo[bi[i], ei[i]]!r}, "
                      f"{hi[bi[i], ei[i]]!r}] scale gpu {int(gs[qq, bb[bi[i]]])} oracle {int(ws_[qq, bb[bi[i]]])} "
                      f"scale ok {bool(s_ok[bi[i]])} acc_g {ref['acc'][qq, cc]!r} acc_u {ref['acc'][qq, I + cc]!r}",
                      flush=True)
    assert n_bad == 0, f"{what}: {n_bad} elements of h are not a valid rounding"
    return n_diff


def layer_check(got, inp, spec, mode, plan, ws, tokens=None, raw_required=False, what=""):
    """The layer's parity checks: (1) the GPU's h is valid element by element
    (check_h); (2) the oracle's FC2 and combine run on the GPU's own h give
    the GPU output within the bar, with nothing discounted; (3) the GPU output
    against the plain oracle output: raw_required True asserts the whole
    bar, "cosine" asserts the cosine and reports max-abs, False reports both
    (a legitimately different rounding decision of one element of h moves
    the output elements of its token by up to several percent of the RMS:
    on small shapes, and in w4a8 at full size, where the matrix cores' FP8
    accumulation makes such decisions differ for ~1 in 2000 elements).  got
    holds the rows of `tokens` (all tokens if None)."""
    ref = oracle_out(inp, spec, mode=mode, tokens=tokens, keep=True)
    P, I = int(ref["offsets"][-1]), spec["I"]
    hg = gpu_h(plan, ws, P, I, mode)
    check_h(hg, inp, spec, ref, mode, what)
    cond = oracle_out(inp, spec, mode=mode, tokens=tokens, h_given=hg["vals"])
    parity(got, cond["out"], f"{what} vs oracle FC2 + combine of the GPU's h")
    if raw_required is True:
        parity(got, ref["out"], f"{what} vs oracle (raw)")
    else:
        cos, _ = report(got, ref["out"], f"{what} vs oracle (raw, max-abs reported)")
        if raw_required == "cosine":
            assert cos >= COS_MIN, f"{what}: raw cosine {cos}"
    return ref


def _measure(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    rms = np.sqrt(np.mean(want ** 2)) if want.size else 0.0
    maxabs = np.max(np.abs(got - want)) if got.size else 0.0
    denom = np.linalg.norm(got) * np.linalg.norm(want)
    cos = float(np.dot(got.ravel(), want.ravel()) / denom) if denom > 0 else (1.0 if maxabs == 0 else 0.0)
    return cos, maxabs, rms


def report(got, want, what=""):
    cos, maxabs, rms = _measure(got, want)
    print(f"{what}: cosine {cos:.7f}, max-abs {maxabs:.3e} = {maxabs / max(rms, 1e-300):.2e} x RMS {rms:.3e}",
          flush=True)
    return cos, maxabs / max(rms, 1e-300)


def parity(got, want, what=""):
    """The parity bar: cosine >= 0.9995 and max-abs <= 1e-2 x RMS(want), on
    the fp32 outputs over every element."""
    assert np.all(np.isfinite(np.asarray(got, np.float64))), f"{what}: non-finite output"
    cos, maxabs, rms = _measure(got, want)
    msg = f"{what}: cosine {cos:.7f}, max-abs {maxabs:.3e} = {maxabs / max(rms, 1e-300):.2e} x RMS {rms:.3e}"
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

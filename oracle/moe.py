"""The routed MXFP4 + SiTU MoE expert layer, computed plainly on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, step by step, and where each step comes from:

1. Top-k unpack.  "TokenSpeed SiTU", "Supported contract": routing arrives as
   precomputed packed or unpacked top-k with GLOBAL expert ids.  The packed
   word is this library's own format (the pages do not define one): bits
   0..15 hold the expert id, bits 16..31 the bf16 bits of the routing weight.
2. Shard filter and grouping.  Same section: experts outside the rank's
   contiguous shard [off, off + E_l) are dropped and the result is a partial
   output that the caller all-reduces.  Within an expert, pairs keep the
   order of their expanded index j = t*k + s (a stable sort on (l, j)).
3. Activations.  "Activation precision (w4a16 vs w4a8)": bf16 in w4a16;
   MXFP8 (E4M3 with one E8M0 scale per 32 along H, per token) in w4a8.
4. FC1 (gate rows [0, I), up rows [I, 2I)) as a dense product with the
   exactly dequantized MXFP4 weights, then the alpha scaling and SiTU.  The
   SiTU formula and the per-token, per-slot skeleton are the golden reference
   in the review of test_kimi_k3_situ_moe.py (pull request 17865):
       act(g, u) = [beta * tanh(g / beta) * sigmoid(g)] * [lbeta * tanh(u / lbeta)]
       out[t] += weight[t, s] * (act(g, u) @ w2.T)
   Per-expert beta and linear beta, and "the up half is rescaled by
   g1_alphas_up / g1_alphas before the tanh": xorl-wheels release notes,
   "Changes since 875b7d7".  With the GEMM output scaled by alpha_gate and
   the up half then rescaled by alpha_up / alpha_gate, g = alpha_gate * acc_g
   and u = alpha_up * acc_u.
5. Rounding point R1 after FC1: w4a16 rounds h to bf16; w4a8 quantizes h to
   MXFP8 (per 32 along I) and dequantizes it ("the FC1 fp8 output is
   dequantized to bf16 before FC2").
6. FC2 down product, y in fp32.
7. Combine: out[t] = sum over local slots, in slot order, of w[t, s] * y.
   Tokens with no local slot give an exact zero row.

Precision modes.  "f64" (the parity reference): every product and sum in
float64, rounded to float32 at each point where the layer holds float32
(acc, g, u, h, y, out).  With rounding=False the rounding points R1 are
skipped too, giving the exact real-number result used by the shard-sum
invariants.  "f32": float32 BLAS, the timed CPU baseline.

Pins (tests/test_oracle_moe.py): brute-force dense unrouted MoE on tiny
shapes; the golden per-token skeleton; top-1 single expert reducing to the
dense MLP; integer exactness of the products; zero contribution of
out-of-shard experts; sum of all EP shards and of all TP shards equal to the
unsharded layer; zero-padding of I; packed and unpacked routing bitwise
equal; SiTU limits and the tanh/sigmoid identity.  End-to-end values: the
pages print no worked example, so whole-layer values beyond these pins are
"parity unpinned".
"""

import numpy as np

from . import formats as F


# --------------------------------------------------------------------------
# Routing

def unpack_topk(packed):
    """Packed int32 [T, k] -> (ids int64, bf16 weight bits uint16)."""
    w = np.asarray(packed).astype(np.int64) & 0xFFFFFFFF
    ids = w & 0xFFFF
    wbits = ((w >> 16) & 0xFFFF).astype(np.uint16)
    return ids, wbits


def route(ids, local_expert_offset, local_num_experts):
    """Shard filter + per-expert grouping.

    Returns counts [E_l], offsets [E_l + 1] (exclusive prefix sum), perm [P]
    (perm[offsets[l] + r] = expanded index j of the r-th pair of expert l,
    ascending j) and inv [T*k] (position of pair j in perm, -1 if not local).
    An id outside [off, off + E_l), negative ids included, is not local.
    """
    ids = np.asarray(ids).astype(np.int64)
    T, k = ids.shape
    j = np.arange(T * k, dtype=np.int64)
    l = ids.reshape(-1) - int(local_expert_offset)
    local = (l >= 0) & (l < local_num_experts)
    jl = j[local]
    ll = l[local]
    counts = np.bincount(ll, minlength=local_num_experts).astype(np.int32)
    offsets = np.zeros(local_num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.lexsort((jl, ll))          # primary key l, then j
    perm = jl[order].astype(np.int32)
    inv = np.full(T * k, -1, dtype=np.int32)
    inv[perm] = np.arange(perm.shape[0], dtype=np.int32)
    return counts, offsets, perm, inv


# --------------------------------------------------------------------------
# Activation

def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def situ(g, u, beta, linear_beta):
    """SiTU gated activation in float64, exactly as the golden reference writes it.

    act(g, u) = [beta * tanh(g / beta) * sigmoid(g)] * [linear_beta * tanh(u / linear_beta)]
    The sigmoid takes the (alpha-scaled) gate g itself.
    """
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    linear_beta = np.asarray(linear_beta, dtype=np.float64)
    return (beta * np.tanh(g / beta) * sigmoid(g)) * (linear_beta * np.tanh(u / linear_beta))


def swiglu(g, u):
    """SwiGLU: g * sigmoid(g) * u (the trusted fused SwiGLU the pages compare
    SiTU against; also the limit of SiTU as both betas grow)."""
    g = np.asarray(g, dtype=np.float64)
    return g * sigmoid(g) * np.asarray(u, dtype=np.float64)


def swiglu_bias(g, u, alpha, beta):
    """CUTLASS SwigluBias as the review of test_kimi_k3_situ_moe.py writes it
    (pull request 17865, _swiglu_bias_act): gate * sigmoid(gate * alpha) *
    (linear + beta), with per-expert alpha and beta."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return g * sigmoid(g * np.float64(alpha)) * (u + np.float64(beta))


ACTIVATIONS = ("situ", "swiglu", "swiglu_bias")


def gated_activation(kind, g, u, p0, p1):
    """h = act(g, u) for one expert: SiTU (p0 = beta, p1 = linear beta),
    SwiGLU (no parameters) or SwigluBias (p0 = alpha, p1 = beta)."""
    if kind == "situ":
        return situ(g, u, p0, p1)
    if kind == "swiglu":
        return swiglu(g, u)
    if kind == "swiglu_bias":
        return swiglu_bias(g, u, p0, p1)
    raise ValueError(kind)


def activation_params(inp, kind, E_l):
    """Per-expert (p0, p1) float32 arrays of the activation (zeros for SwiGLU,
    which has none)."""
    if kind == "situ":
        return np.asarray(inp["situ_beta"], np.float32), np.asarray(inp["situ_linear_beta"], np.float32)
    if kind == "swiglu":
        z = np.zeros(E_l, np.float32)
        return z, z
    if kind == "swiglu_bias":
        return np.asarray(inp["swiglu_alpha"], np.float32), np.asarray(inp["swiglu_beta"], np.float32)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# The layer

def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def activations(inp, act_mode, act_prequantized):
    """Float values of the FC1 input rows, [T, H] float64.

    w4a16: the bf16 hidden states.  w4a8: E4M3 codes times their E8M0 block
    scales; bf16 input is first quantized with the MX rule (mx_quantize).
    Returns (xf, codes, scales) -- codes/scales are None in w4a16.
    """
    if act_mode == "w4a16":
        return F.bf16_to_f64(inp["hidden_states"]), None, None
    if act_mode != "w4a8":
        raise ValueError(act_mode)
    if act_prequantized:
        codes = np.asarray(inp["hidden_states"], dtype=np.uint8)
        scales = np.asarray(inp["hidden_states_scale"], dtype=np.uint8)
    else:
        codes, scales = F.mx_quantize(F.bf16_to_f64(inp["hidden_states"]), "e4m3")
    return F.mx_dequantize(codes, scales, "e4m3"), codes, scales


def topk_of(inp):
    """(ids int64 [T,k], weights float64 [T,k]) from either routing format."""
    if inp.get("topk_packed") is not None:
        ids, wbits = unpack_topk(inp["topk_packed"])
    else:
        ids = np.asarray(inp["topk_ids"]).astype(np.int64)
        wbits = np.asarray(inp["topk_weights"], dtype=np.uint16)
    return ids, F.bf16_to_f64(wbits)


def moe_forward(inp, *, local_expert_offset, local_num_experts, act_mode="w4a16",
                act_prequantized=False, precision="f64", rounding=True, tokens=None,
                keep_intermediates=False, activation="situ", weight_format="mxfp4", h_given=None,
                want_act_lora=False):
    """Partial output of one shard of the routed MXFP4 + SiTU MoE layer.

    inp holds numpy arrays:
      hidden_states  uint16 bf16 bits [T, H] (or uint8 E4M3 codes when
                     act_prequantized, with hidden_states_scale uint8 [T, H/32])
      topk_ids int [T, k] + topk_weights uint16 bf16 bits [T, k], or
      topk_packed int32 [T, k]
      w1 uint8 [E_l, 2I, H/2], w1_scale uint8 [E_l, 2I, H/32]
      w2 uint8 [E_l, H, I/2],  w2_scale uint8 [E_l, H, I/32]
        (weight_format "nvfp4": E4M3 scales [E_l, 2I, H/16] and [E_l, H, I/16])
      situ_beta, situ_linear_beta float32 [E_l] (activation "situ"), or
      swiglu_alpha, swiglu_beta float32 [E_l] (activation "swiglu_bias")
      alpha_gate, alpha_up float32 [E_l] or None (meaning 1.0)
      alpha_down float32 [E_l] or None: per-expert scale of the FC2 output,
        applied with the routing weight in the combine
      gate_up_lora_delta uint16 bf16 bits [T*k, 2I] or None: a low-rank
        adapter's contribution to the FC1 output of pair j = t*k + s, added
        to the alpha-scaled gate and up halves before the activation
    tokens: optional array of token indices; only those rows are computed and
    returned (the layer is independent per token, routing is still global).
    h_given: optional [P, I] FC1 outputs (after the rounding point) in
    permuted order, used instead of computing FC1: the FC2 and combine of
    given rows.
    Returns dict(out=float32 [len(tokens) or T, H], out_bf16=uint16 bits,
    counts, offsets, perm, inv, and with keep_intermediates the per-pair h
    (float64 after R1) and y (float64) in permuted order for the computed
    pairs; with want_act_lora the FC1 output rows by expanded index
    [T*k, I] (float64, zero rows for pairs outside the shard or not computed).
    """
    if precision not in ("f64", "f32"):
        raise ValueError(precision)
    if weight_format not in ("mxfp4", "nvfp4"):
        raise ValueError(weight_format)
    dequant = F.dequant_mxfp4 if weight_format == "mxfp4" else F.dequant_nvfp4
    E_l = int(local_num_experts)
    ids, wts = topk_of(inp)
    T, k = ids.shape
    counts, offsets, perm, inv = route(ids, local_expert_offset, E_l)

    xf, _, _ = activations(inp, act_mode, act_prequantized)
    H = xf.shape[1]
    w1, w1s, w2, w2s = inp["w1"], inp["w1_scale"], inp["w2"], inp["w2_scale"]
    I = w2.shape[2] * 2
    assert w1.shape[1] == 2 * I and w1.shape[2] * 2 == H

    ones = np.ones(E_l, dtype=np.float32)
    a_g = ones if inp.get("alpha_gate") is None else np.asarray(inp["alpha_gate"], np.float32)
    a_u = ones if inp.get("alpha_up") is None else np.asarray(inp["alpha_up"], np.float32)
    a_d = None if inp.get("alpha_down") is None else np.asarray(inp["alpha_down"], np.float32)
    p0, p1 = activation_params(inp, activation, E_l)
    delta = inp.get("gate_up_lora_delta")
    if delta is not None:
        delta = F.bf16_to_f64(np.asarray(delta).reshape(T * k, 2 * I))

    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)

    dt = np.float64 if precision == "f64" else np.float32
    if precision == "f64" and rounding:
        def rnd(a):
            return _f32(a).astype(np.float64)
    else:
        def rnd(a):
            return a

    # Pairs whose FC2 rows the requested tokens need, in permuted order.
    P = perm.shape[0]
    slot_pos = inv.reshape(T, k)[tokens]                         # [n_tok, k]
    need = np.unique(slot_pos[slot_pos >= 0])
    compact = np.full(P, -1, dtype=np.int64)
    compact[need] = np.arange(need.shape[0])
    Y = np.zeros((need.shape[0], H), dtype=dt)
    Hq = np.zeros((need.shape[0], I), dtype=np.float64) if keep_intermediates else None
    Acc = np.zeros((need.shape[0], 2 * I), dtype=np.float64) if keep_intermediates else None
    Hpre = np.zeros((need.shape[0], I), dtype=np.float64) if keep_intermediates else None
    ActLora = np.zeros((T * k, I), dtype=np.float64) if want_act_lora else None

    for l in range(E_l):
        p_lo, p_hi = int(offsets[l]), int(offsets[l + 1])
        pos = need[(need >= p_lo) & (need < p_hi)]
        if pos.shape[0] == 0:
            continue
        if h_given is None:
            rows_t = perm[pos] // k
            xa = xf[rows_t].astype(dt)
            W1d = dequant(w1[l], w1s[l]).astype(dt, copy=False)    # [2I, H]
            acc = rnd(xa @ W1d.T)                                  # [n, 2I]
            if precision == "f64":
                g = rnd(np.float64(a_g[l]) * acc[:, :I])
                u = rnd(np.float64(a_u[l]) * acc[:, I:])
                if delta is not None:
                    g = rnd(g + delta[perm[pos], :I])
                    u = rnd(u + delta[perm[pos], I:])
                h = rnd(gated_activation(activation, g, u, p0[l], p1[l]))
            else:
                g = np.float32(a_g[l]) * acc[:, :I]
                u = np.float32(a_u[l]) * acc[:, I:]
                if delta is not None:
                    g = g + delta[perm[pos], :I].astype(np.float32)
                    u = u + delta[perm[pos], I:].astype(np.float32)
                h = gated_activation(activation, g, u, p0[l], p1[l]).astype(np.float32)
            if rounding:
                if act_mode == "w4a16":
                    hq = F.bf16_to_f64(F.f32_to_bf16_rne(_f32(h)))
                else:
                    hc, hs = F.mx_quantize(np.asarray(h, np.float64), "e4m3")
                    hq = F.mx_dequantize(hc, hs, "e4m3")
            else:
                hq = np.asarray(h, np.float64)
        else:
            hq = np.asarray(h_given, np.float64)[pos]
        W2d = dequant(w2[l], w2s[l]).astype(dt, copy=False)        # [H, I]
        Y[compact[pos]] = rnd(hq.astype(dt) @ W2d.T)               # [n, H]
        if keep_intermediates:
            Hq[compact[pos]] = hq
            if h_given is None:
                Acc[compact[pos]] = acc
                Hpre[compact[pos]] = np.asarray(h, np.float64)
        if want_act_lora:
            ActLora[perm[pos]] = hq

    # Combine in slot order; a token with no local slot keeps its zero row.
    # The FC2 output scale alpha_down, where given, multiplies the routing
    # weight (one fp32 product per slot).
    out = np.zeros((tokens.shape[0], H), dtype=np.float64)
    for s in range(k):
        p = slot_pos[:, s]
        has = p >= 0
        if has.any():
            wsl = wts[tokens[has], s]
            if a_d is not None:
                wsl = wsl * a_d[ids[tokens[has], s] - int(local_expert_offset)].astype(np.float64)
                if rounding or precision == "f32":
                    wsl = _f32(wsl).astype(np.float64)
            out[has] += wsl[:, None] * Y[compact[p[has]]].astype(np.float64)
    out32 = _f32(out) if (rounding or precision == "f32") else out
    res = dict(out=out32, counts=counts, offsets=offsets, perm=perm, inv=inv, P=P,
               tokens=tokens)
    if rounding or precision == "f32":
        res["out_bf16"] = F.f32_to_bf16_rne(out32)
    if keep_intermediates:
        res["pairs"] = need          # permuted positions of the rows below
        res["h"] = Hq
        res["y"] = Y.astype(np.float64)
        if h_given is None:
            res["acc"] = Acc
            res["h_pre"] = Hpre        # activation output before the rounding point R1
    if want_act_lora:
        res["act_lora"] = ActLora
    return res


def active_experts(counts):
    """Number of local experts that receive at least one pair."""
    return int(np.count_nonzero(np.asarray(counts)))

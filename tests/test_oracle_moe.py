"""Pins of the oracle's routed MoE layer against independent formulations.

None of these re-types the oracle: each compares it with a different
algorithm (a dense unrouted MoE, the golden per-token skeleton, an integer
matmul, a brute-force recount) or with an invariant the layer must satisfy
(shard sums, zero contribution, zero padding, format equivalence).
"""

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import formats as F
from oracle import moe as M


def _spec(**kw):
    base = dict(T=6, H=128, I=64, E_g=8, E_l=8, off=0, k=3, seed=11)
    base.update(kw)
    return base


def _fwd(inp, spec, **kw):
    return M.moe_forward(inp, local_expert_offset=spec["off"], local_num_experts=spec["E_l"], **kw)


def _dense_weights(inp):
    W1 = np.stack([F.dequant_mxfp4(inp["w1"][e], inp["w1_scale"][e]) for e in range(inp["w1"].shape[0])])
    W2 = np.stack([F.dequant_mxfp4(inp["w2"][e], inp["w2_scale"][e]) for e in range(inp["w2"].shape[0])])
    return W1, W2


# ---------------------------------------------------------------- routing

def test_route_matches_bruteforce_recount():
    rng = np.random.default_rng(5)
    T, k, E_g, off, E_l = 37, 5, 40, 12, 9
    ids = rng.integers(-3, E_g + 3, size=(T, k))
    counts, offsets, perm, inv = M.route(ids, off, E_l)
    # brute force: walk experts, then pairs in expanded order
    want_perm, want_counts = [], []
    for l in range(E_l):
        c = 0
        for t in range(T):
            for s in range(k):
                if ids[t, s] == off + l:
                    want_perm.append(t * k + s)
                    c += 1
        want_counts.append(c)
    assert counts.tolist() == want_counts
    assert offsets.tolist() == [sum(want_counts[:i]) for i in range(E_l + 1)]
    assert perm.tolist() == want_perm
    for j in range(T * k):
        if j in want_perm:
            assert inv[j] == want_perm.index(j)
        else:
            assert inv[j] == -1


def test_packed_and_unpacked_routing_bitwise_equal():
    spec = _spec(packed=True, T=9, E_g=12, E_l=6, off=3)
    inp = S.generate(spec)
    a = _fwd(inp, spec)
    unpacked = dict(inp)
    unpacked["topk_packed"] = None
    b = _fwd(unpacked, spec)
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
    ids, wbits = M.unpack_topk(inp["topk_packed"])
    assert np.array_equal(ids, inp["topk_ids"]) and np.array_equal(wbits, inp["topk_weights"])


# ---------------------------------------------------------------- SiTU

def test_situ_large_beta_is_swiglu():
    rng = np.random.default_rng(6)
    g = rng.standard_normal(1000) * 3
    u = rng.standard_normal(1000) * 3
    got = M.situ(g, u, 1e6, 1e6)
    swiglu = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    assert np.max(np.abs(got - swiglu) / (np.abs(swiglu) + 1e-12)) < 1e-9


def test_situ_zeros_and_bounds():
    rng = np.random.default_rng(7)
    g = rng.standard_normal(1000) * 50
    u = rng.standard_normal(1000) * 50
    assert np.all(M.situ(np.zeros(5), rng.standard_normal(5), 2.0, 3.0) == 0)
    assert np.all(M.situ(rng.standard_normal(5), np.zeros(5), 2.0, 3.0) == 0)
    v = M.situ(g, u, 4.0, 25.0)
    assert np.all(np.abs(v) <= 4.0 * 25.0)
    # the gate factor is bounded below by -beta * sigmoid(g) -> 0 for g -> -inf
    assert abs(M.situ(-800.0, 1.0, 4.0, 25.0)) < 1e-300


def test_tanh_sigmoid_identity_at_k3_constants():
    # beta * tanh(x / beta) == 2 * beta * sigmoid(2 x / beta) - beta; K3 uses
    # beta = 4 and linear beta = 25 (MegaMoE commit message, "SiTU in the kernel").
    x = np.linspace(-60, 60, 100001)
    for beta in (4.0, 25.0):
        lhs = beta * np.tanh(x / beta)
        rhs = 2 * beta * M.sigmoid(2 * x / beta) - beta
        assert np.max(np.abs(lhs - rhs)) < 1e-13 * beta


def test_situ_with_k3_constants_matches_mpmath_free_closed_form():
    # g = 0.5, u = 2 at beta 4, linear beta 25, from the closed form with math.tanh/exp
    import math
    g, u = 0.5, 2.0
    want = (4 * math.tanh(g / 4) / (1 + math.exp(-g))) * (25 * math.tanh(u / 25))
    assert abs(M.situ(g, u, 4.0, 25.0) - want) < 1e-15


# ---------------------------------------------------------------- the layer

@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_routed_equals_dense_unrouted_moe(mode):
    spec = _spec(mode=mode, T=7, E_g=10, E_l=10, k=3)
    inp = S.generate(spec)
    got = _fwd(inp, spec, act_mode=mode, rounding=False)["out"]
    # dense: run EVERY expert on EVERY token, multiply by a dense gate matrix
    ids, w = M.topk_of(inp)
    T, k = ids.shape
    G = np.zeros((T, spec["E_g"]))
    for t in range(T):
        for s in range(k):
            G[t, ids[t, s]] += w[t, s]
    xf, _, _ = M.activations(inp, mode, False)
    W1, W2 = _dense_weights(inp)
    I = spec["I"]
    out = np.zeros((T, spec["H"]))
    for e in range(spec["E_g"]):
        acc = xf @ W1[e].T
        h = M.situ(inp["alpha_gate"][e] * acc[:, :I], inp["alpha_up"][e] * acc[:, I:],
                   inp["situ_beta"][e], inp["situ_linear_beta"][e])
        out += G[:, e:e + 1] * (h @ W2[e].T)
    np.testing.assert_allclose(got, out, rtol=1e-12, atol=1e-14)


def test_golden_per_token_skeleton():
    # the skeleton of the golden reference: loop tokens and slots,
    # g = x.w1, u = x.w3, out += weight * (act(g, u) @ w2.T)
    spec = _spec(T=5, k=2, E_g=6, E_l=6)
    inp = S.generate(spec)
    got = _fwd(inp, spec, rounding=False)["out"]
    W1, W2 = _dense_weights(inp)
    I = spec["I"]
    ids, w = M.topk_of(inp)
    x = F.bf16_to_f64(inp["hidden_states"])
    out = np.zeros_like(got)
    for t in range(ids.shape[0]):
        for s in range(ids.shape[1]):
            e = ids[t, s]
            g = inp["alpha_gate"][e] * (x[t] @ W1[e, :I].T)
            u = inp["alpha_up"][e] * (x[t] @ W1[e, I:].T)
            act = (inp["situ_beta"][e] * np.tanh(g / inp["situ_beta"][e]) / (1 + np.exp(-g))) * \
                  (inp["situ_linear_beta"][e] * np.tanh(u / inp["situ_linear_beta"][e]))
            out[t] += w[t, s] * (act @ W2[e].T)
    np.testing.assert_allclose(got, out, rtol=1e-12, atol=1e-14)


def test_top1_single_expert_is_dense_mlp():
    spec = _spec(T=4, k=1, E_g=1, E_l=1)
    inp = S.generate(spec)
    inp["topk_weights"][:] = 0x3F80  # bf16 1.0
    got = _fwd(inp, spec, rounding=False)["out"]
    W1, W2 = _dense_weights(inp)
    I = spec["I"]
    x = F.bf16_to_f64(inp["hidden_states"])
    h = M.situ(inp["alpha_gate"][0] * x @ W1[0, :I].T, inp["alpha_up"][0] * x @ W1[0, I:].T,
               inp["situ_beta"][0], inp["situ_linear_beta"][0])
    np.testing.assert_allclose(got, h @ W2[0].T, rtol=1e-12, atol=1e-14)


def test_fc1_products_integer_exact():
    # weights with scale 2^0 and small-integer activations: the FC1 accumulator
    # is an integer matmul, exactly.
    spec = _spec(T=8, k=2, E_g=4, E_l=4, H=256)
    inp = S.generate(spec)
    inp["w1_scale"][:] = 127
    rng = np.random.default_rng(8)
    xi = rng.integers(-8, 9, size=(spec["T"], spec["H"]))
    inp["hidden_states"] = F.f32_to_bf16_rne(xi.astype(np.float32))
    r = _fwd(inp, spec, keep_intermediates=True)
    codes = F.unpack_fp4(inp["w1"], spec["H"])
    wint2 = (F.decode_e2m1(codes) * 2).astype(np.int64)            # 2*w is an integer
    for q, p in enumerate(r["pairs"]):
        t, l = r["perm"][p] // spec["k"], np.searchsorted(r["offsets"], p, side="right") - 1
        exact2 = wint2[l] @ xi[t]
        assert np.array_equal(r["acc"][q] * 2, exact2.astype(np.float64))


def test_out_of_shard_ids_contribute_nothing():
    spec = _spec(T=10, k=4, E_g=20, E_l=5, off=7)
    inp = S.generate(spec)
    a = _fwd(inp, spec)
    ids = inp["topk_ids"].copy()
    nonlocal_ = (ids < 7) | (ids >= 12)
    rng = np.random.default_rng(9)
    repl = rng.choice(np.r_[np.arange(-5, 7), np.arange(12, 30)], size=ids.shape)
    inp2 = dict(inp)
    inp2["topk_ids"] = np.where(nonlocal_, repl, ids).astype(np.int32)
    b = _fwd(inp2, spec)
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
    none = ~((ids >= 7) & (ids < 12)).any(axis=1)
    assert none.any()
    assert np.all(a["out"][none] == 0) and not np.any(np.signbit(a["out"][none]))


def test_ep_shards_sum_to_unsharded():
    full = _spec(T=9, k=3, E_g=16, E_l=16, off=0, seed=21)
    inp = S.generate(full)
    ref = _fwd(inp, full, rounding=False)["out"]
    total = np.zeros_like(ref)
    for r in range(4):
        sl = slice(4 * r, 4 * r + 4)
        shard = dict(inp)
        for key in ("w1", "w1_scale", "w2", "w2_scale", "situ_beta", "situ_linear_beta",
                    "alpha_gate", "alpha_up"):
            shard[key] = inp[key][sl]
        total += M.moe_forward(shard, local_expert_offset=4 * r, local_num_experts=4,
                               rounding=False)["out"]
    np.testing.assert_allclose(total, ref, rtol=1e-12, atol=1e-14)


def test_tp_shards_sum_to_unsharded():
    full = _spec(T=9, k=3, E_g=4, E_l=4, I=128, seed=22)
    inp = S.generate(full)
    ref = _fwd(inp, full, rounding=False)["out"]
    I = full["I"]
    total = np.zeros_like(ref)
    for q in range(4):
        gate = np.arange(32 * q, 32 * q + 32)
        rows = np.r_[gate, I + gate]
        shard = dict(inp)
        shard["w1"] = inp["w1"][:, rows]
        shard["w1_scale"] = inp["w1_scale"][:, rows]
        shard["w2"] = inp["w2"][:, :, 16 * q:16 * q + 16]
        shard["w2_scale"] = inp["w2_scale"][:, :, q:q + 1]
        total += _fwd(shard, full, rounding=False)["out"]
    np.testing.assert_allclose(total, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_zero_padding_of_intermediate_is_exact(mode):
    spec = _spec(T=6, k=2, E_g=5, E_l=5, I=64, mode=mode, seed=23)
    inp = S.generate(spec)
    a = _fwd(inp, spec, act_mode=mode)
    I, Ip = 64, 96
    pad = dict(inp)
    E, H = spec["E_l"], spec["H"]
    w1 = np.zeros((E, 2 * Ip, H // 2), np.uint8)
    w1s = np.full((E, 2 * Ip, H // 32), 127, np.uint8)
    w1[:, :I], w1s[:, :I] = inp["w1"][:, :I], inp["w1_scale"][:, :I]
    w1[:, Ip:Ip + I], w1s[:, Ip:Ip + I] = inp["w1"][:, I:], inp["w1_scale"][:, I:]
    w2 = np.zeros((E, H, Ip // 2), np.uint8)
    w2s = np.full((E, H, Ip // 32), 127, np.uint8)
    w2[:, :, :I // 2], w2s[:, :, :I // 32] = inp["w2"], inp["w2_scale"]
    pad.update(w1=w1, w1_scale=w1s, w2=w2, w2_scale=w2s)
    b = _fwd(pad, spec, act_mode=mode)
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))


def test_w4a8_activation_scale_applied_once():
    # prequantized MXFP8 input == the same values fed as bf16 (exact: E4M3 * 2^k
    # fits bf16 here), in exact arithmetic; a scale applied twice would differ by 2^k.
    spec = _spec(T=6, k=2, E_g=4, E_l=4, mode="w4a8", seed=24)
    inp = S.generate(spec)
    codes, scales = F.mx_quantize(F.bf16_to_f64(inp["hidden_states"]), "e4m3")
    pre = dict(inp, hidden_states=codes, hidden_states_scale=scales)
    a = _fwd(pre, spec, act_mode="w4a8", act_prequantized=True, rounding=False)["out"]
    deq = F.mx_dequantize(codes, scales, "e4m3")
    as_bf16 = dict(inp, hidden_states=F.f32_to_bf16_rne(deq.astype(np.float32)))
    assert np.array_equal(F.bf16_to_f64(as_bf16["hidden_states"]), deq)
    b = _fwd(as_bf16, spec, act_mode="w4a16", rounding=False)["out"]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    # and the library quantizes bf16 input exactly as the prequantized path
    c = _fwd(inp, spec, act_mode="w4a8", rounding=False)["out"]
    assert np.array_equal(a, c)


def test_token_subset_equals_full_rows():
    spec = _spec(T=12, k=3, E_g=8, E_l=5, off=2, seed=25)
    inp = S.generate(spec)
    full = _fwd(inp, spec)["out"]
    sub = _fwd(inp, spec, tokens=np.array([10, 0, 7]))["out"]
    assert np.array_equal(sub, full[[10, 0, 7]])


def test_f32_mode_close_to_f64_mode():
    spec = _spec(T=8, k=3, E_g=8, E_l=8, H=256, I=64, seed=26)
    inp = S.generate(spec)
    a = _fwd(inp, spec)["out"]
    b = _fwd(inp, spec, precision="f32")["out"]
    rms = np.sqrt(np.mean(a.astype(np.float64) ** 2))
    assert np.max(np.abs(a - b)) < 1e-2 * rms


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_fc1_output_rounding_point(mode):
    # "the FC1 fp8 output is dequantized to bf16 before FC2": in w4a8 every
    # 32-block of h along I lies on one E4M3 * 2^e grid whose top binade holds
    # the block max; in w4a16 h is bf16.  Both are within half an element ulp
    # of the unrounded activation.
    spec = _spec(T=8, k=3, E_g=6, E_l=6, H=256, I=96, mode=mode, seed=27)
    inp = S.generate(spec)
    r = _fwd(inp, spec, act_mode=mode, keep_intermediates=True)
    e = _fwd(inp, spec, act_mode=mode, keep_intermediates=True, rounding=False)
    h, hx = r["h"], e["h"]
    assert h.shape == hx.shape and h.shape[1] == spec["I"]
    if mode == "w4a16":
        assert np.array_equal(F.bf16_to_f64(F.f32_to_bf16_rne(h.astype(np.float32))), h)
        assert np.all(np.abs(h - hx) <= np.abs(hx) * 2.0 ** -8 + 1e-30)
    else:
        blocks = h.reshape(h.shape[0], -1, 32)
        xb = hx.reshape(h.shape[0], -1, 32)
        for q in range(blocks.shape[0]):
            for b in range(blocks.shape[1]):
                amax = np.max(np.abs(xb[q, b]))
                if amax == 0:
                    assert np.all(blocks[q, b] == 0)
                    continue
                sc = 2.0 ** (F.floor_log2(amax) - 8)
                grid = F.decode_e4m3(np.arange(0x7F))
                m = np.abs(blocks[q, b]) / sc
                assert np.all(np.isin(m, grid))
                err = np.abs(blocks[q, b] - xb[q, b]) / sc
                clip = np.maximum(np.abs(xb[q, b]) / sc - 448.0, 0.0)   # OCP rule saturates at 448
                assert np.all(err <= np.maximum(np.maximum(m, 2.0 ** -6) * 2.0 ** -4, clip) + 1e-6)

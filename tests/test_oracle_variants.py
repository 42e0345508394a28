"""Pins of the oracle's layer variants: the SwiGLU and SwigluBias activations,
NVFP4 weights with the FC2 output scale alpha_down, and the LoRA bridges
(gate_up delta in, down-LoRA input out).

Each compares the oracle with an independent formulation: the golden
per-token skeleton with the activation written out as the review of
test_kimi_k3_situ_moe.py writes it (pull request 17865), a limit of SiTU,
the NVFP4 decode built from torch's float8 dtype and the literal E2M1 table,
closed forms where the FC1 weights are zero, and exact identities (a zero
delta changes nothing, a power-of-two alpha_down scales the output exactly).
"""

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import formats as F
from oracle import moe as M


def _spec(**kw):
    base = dict(T=6, H=128, I=64, E_g=8, E_l=8, off=0, k=3, seed=21)
    base.update(kw)
    return S.spec_of(base)


def _fwd(inp, spec, **kw):
    kw.setdefault("activation", spec["activation"])
    kw.setdefault("weight_format", spec["weight_format"])
    return M.moe_forward(inp, local_expert_offset=spec["off"], local_num_experts=spec["E_l"], **kw)


E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP MX v1.0, FP4 E2M1 magnitudes


def _nvfp4_dense(packed, scales):
    """Independent NVFP4 decode: nibbles by shifting, E2M1 from the literal
    table, the E4M3 block scale through torch.float8_e4m3fn."""
    p = np.asarray(packed).astype(np.int64)
    codes = np.stack([p & 15, p >> 4], axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * 2,))
    mag = np.array(E2M1_TABLE)[codes & 7]
    vals = np.where(codes & 8, -mag, mag)
    sc = torch.from_numpy(np.asarray(scales).astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return vals * np.repeat(sc, 16, axis=-1)


def _golden(inp, spec, act, dense_w):
    """out[t] += weight * (act(e, g, u) @ w2.T) over tokens and slots, with
    g = alpha_g * x.w1, u = alpha_u * x.w3, in float64."""
    I = spec["I"]
    ids, w = M.topk_of(inp)
    x = F.bf16_to_f64(inp["hidden_states"])
    W1 = [dense_w(inp["w1"][e], inp["w1_scale"][e]) for e in range(spec["E_l"])]
    W2 = [dense_w(inp["w2"][e], inp["w2_scale"][e]) for e in range(spec["E_l"])]
    a_d = inp.get("alpha_down")
    out = np.zeros((ids.shape[0], spec["H"]))
    for t in range(ids.shape[0]):
        for s in range(ids.shape[1]):
            e = int(ids[t, s]) - spec["off"]
            if not 0 <= e < spec["E_l"]:
                continue
            g = inp["alpha_gate"][e] * (x[t] @ W1[e][:I].T)
            u = inp["alpha_up"][e] * (x[t] @ W1[e][I:].T)
            wt = w[t, s] * (1.0 if a_d is None else a_d[e])
            out[t] += wt * (act(e, g, u) @ W2[e].T)
    return out


def test_swiglu_bias_golden_skeleton():
    spec = _spec(activation="swiglu_bias")
    inp = S.generate(spec)
    got = _fwd(inp, spec, rounding=False)["out"]

    def act(e, g, u):    # gate * sigmoid(gate * alpha) * (linear + beta)
        return g / (1 + np.exp(-g * inp["swiglu_alpha"][e])) * (u + inp["swiglu_beta"][e])
    want = _golden(inp, spec, act, F.dequant_mxfp4)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_swiglu_is_situ_with_large_betas():
    spec = _spec(activation="swiglu")
    inp = S.generate(spec)
    got = _fwd(inp, spec, rounding=False)["out"]
    big = dict(inp, situ_beta=np.full(spec["E_l"], 1e7, np.float32),
               situ_linear_beta=np.full(spec["E_l"], 1e7, np.float32))
    lim = _fwd(big, spec, activation="situ", rounding=False)["out"]
    assert np.max(np.abs(got - lim)) <= 1e-9 * np.sqrt(np.mean(got ** 2))


def test_swiglu_bias_with_unit_alpha_zero_beta_is_swiglu():
    spec = _spec(activation="swiglu_bias")
    inp = S.generate(spec)
    inp = dict(inp, swiglu_alpha=np.ones(spec["E_l"], np.float32), swiglu_beta=np.zeros(spec["E_l"], np.float32))
    for mode in ("w4a16", "w4a8"):
        a = _fwd(inp, spec, act_mode=mode)["out"]
        b = _fwd(inp, spec, act_mode=mode, activation="swiglu")["out"]
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_nvfp4_decode_every_code_and_scale():
    codes = np.arange(256, dtype=np.uint8)[None, :].repeat(126, 0)          # every byte = two E2M1 codes
    scales = np.repeat(np.arange(126, dtype=np.uint8)[:, None], 32, 1)       # every finite positive E4M3
    got = F.dequant_nvfp4(codes, scales)
    np.testing.assert_array_equal(got, _nvfp4_dense(codes, scales))
    # a hand-worked block: bytes 0x21 (elements 0.5, 1.0) and 0xF7 (6.0, -6.0)
    # under scale 0x3C = 1.5 (exponent 7 - 7 = 0, mantissa 4/8)
    blk = np.zeros((1, 8), np.uint8)
    blk[0, 0], blk[0, 1] = 0x21, 0xF7
    v = F.dequant_nvfp4(blk, np.array([[0x3C]], np.uint8))
    assert v[0, :4].tolist() == [0.75, 1.5, 9.0, -9.0] and not v[0, 4:].any()


@pytest.mark.parametrize("activation", ["situ", "swiglu_bias"])
def test_nvfp4_layer_golden_skeleton(activation):
    spec = _spec(weight_format="nvfp4", activation=activation, T=7, E_g=10, E_l=6, off=2, k=3)
    inp = S.generate(spec)
    assert inp["w1_scale"].shape[-1] == spec["H"] // 16 and inp.get("alpha_down") is not None
    got = _fwd(inp, spec, rounding=False)["out"]
    if activation == "situ":
        def act(e, g, u):
            b, lb = inp["situ_beta"][e], inp["situ_linear_beta"][e]
            return b * np.tanh(g / b) / (1 + np.exp(-g)) * lb * np.tanh(u / lb)
    else:
        def act(e, g, u):
            return g / (1 + np.exp(-g * inp["swiglu_alpha"][e])) * (u + inp["swiglu_beta"][e])
    want = _golden(inp, spec, act, _nvfp4_dense)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14 * np.abs(want).max())


def test_alpha_down_power_of_two_scales_output_exactly():
    spec = _spec()
    inp = S.generate(spec)
    base = _fwd(inp, spec)["out"].astype(np.float64)
    scaled = _fwd(dict(inp, alpha_down=np.full(spec["E_l"], 0.25, np.float32)), spec)["out"].astype(np.float64)
    assert np.array_equal(scaled, base * 0.25)


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_zero_lora_delta_is_the_plain_layer(mode):
    spec = _spec(lora=True)
    inp = S.generate(spec)
    zero = dict(inp, gate_up_lora_delta=np.zeros_like(inp["gate_up_lora_delta"]))
    plain = dict(inp, gate_up_lora_delta=None)
    a = _fwd(zero, spec, act_mode=mode)["out"]
    b = _fwd(plain, spec, act_mode=mode)["out"]
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = _fwd(inp, spec, act_mode=mode)["out"]
    assert not np.array_equal(a, c)          # a nonzero delta does change the output


def test_lora_delta_with_zero_fc1_weights_is_the_activation_of_the_delta():
    """With every FC1 weight zero the accumulators vanish and the activation
    sees the delta alone: h = act(d_gate, d_up), then FC2 and the combine."""
    spec = _spec(lora=True, activation="swiglu_bias", T=5, k=2)
    inp = S.generate(spec)
    inp = dict(inp, w1=np.zeros_like(inp["w1"]))
    got = _fwd(inp, spec, rounding=False)["out"]
    I, k = spec["I"], spec["k"]
    d = F.bf16_to_f64(inp["gate_up_lora_delta"]).reshape(spec["T"], k, 2 * I)
    ids, w = M.topk_of(inp)
    out = np.zeros_like(got)
    for t in range(spec["T"]):
        for s in range(k):
            e = int(ids[t, s])
            g, u = d[t, s, :I], d[t, s, I:]
            h = g / (1 + np.exp(-g * inp["swiglu_alpha"][e])) * (u + inp["swiglu_beta"][e])
            out[t] += w[t, s] * (h @ F.dequant_mxfp4(inp["w2"][e], inp["w2_scale"][e]).T)
    np.testing.assert_allclose(got, out, rtol=1e-12, atol=1e-14)


def test_down_lora_input_rows():
    """The down-LoRA input holds h of pair j = t*k + s in row j (after the
    rounding point), zero rows for pairs outside the shard."""
    spec = _spec(lora=True, E_g=12, E_l=5, off=4, T=9)
    inp = S.generate(spec)
    r = _fwd(inp, spec, keep_intermediates=True, want_act_lora=True)
    rows = r["act_lora"]
    j = r["perm"][r["pairs"]]
    np.testing.assert_array_equal(rows[j], r["h"])
    mask = np.ones(rows.shape[0], bool)
    mask[j] = False
    assert not rows[mask].any()
    assert mask.any()     # the shard leaves some pairs out

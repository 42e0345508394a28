"""CPU checks of the GPU tests' parity machinery (tests/gpu_helpers.py).

The GPU tests accept an element of h that differs from the oracle's rounding
only where the oracle's pre-rounding value lies within its tolerance of a
rounding boundary, and then compare the GPU output with the oracle's FC2 and
combine of the GPU's own h, and with the plain oracle, at the bar with
nothing discounted.  Here the oracle's own float32 path stands in for a
correct GPU (it must pass), and planted mistakes stand in for a wrong one
(each must fail).
"""

import numpy as np
import pytest

import synthetic as S
from oracle import formats as F
from oracle import moe as M

from gpu_helpers import check_h, oracle_out, parity

SHAPE = dict(T=64, H=640, I=256, E_g=8, E_l=8, off=0, k=4, seed=61, skew=True)


def _as_gpu_h(h_rows, mode):
    """A GPU-style h record from rows of h values (already at the rounding point)."""
    if mode == "w4a16":
        return dict(vals=np.asarray(h_rows, np.float64))
    codes, sc = F.mx_quantize(np.asarray(h_rows, np.float64), "e4m3")
    return dict(vals=F.mx_dequantize(codes, sc, "e4m3"), codes=codes, scales=sc)


def _full_rows(ref, P, I):
    h = np.zeros((P, I))
    h[ref["pairs"]] = ref["h"]
    return h


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_float32_path_passes(mode):
    """The oracle's float32 BLAS path, a correct computation in another
    order, passes every check."""
    spec = S.spec_of(SHAPE)
    inp = S.generate(spec)
    ref = oracle_out(inp, spec, mode=mode, keep=True)
    P, I = int(ref["offsets"][-1]), spec["I"]
    f32 = M.moe_forward(inp, local_expert_offset=0, local_num_experts=spec["E_l"], act_mode=mode,
                        precision="f32", keep_intermediates=True)
    hg = _as_gpu_h(_full_rows(f32, P, I), mode)
    n_diff = check_h(hg, inp, spec, ref, mode, f"float32 path {mode}")
    cond = oracle_out(inp, spec, mode=mode, h_given=hg["vals"])
    parity(f32["out"], cond["out"], "float32 path vs oracle FC2 of its h")


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_planted_h_mistake_fails(mode):
    """One element of h moved to the next representable value where the
    oracle's value is far from a rounding boundary is rejected."""
    spec = S.spec_of(SHAPE)
    inp = S.generate(spec)
    ref = oracle_out(inp, spec, mode=mode, keep=True)
    P, I = int(ref["offsets"][-1]), spec["I"]
    h = _full_rows(ref, P, I)
    hp = np.zeros((P, I))
    hp[ref["pairs"]] = ref["h_pre"]
    # the element whose pre-rounding value sits closest to a representable value
    err = np.abs(hp - h) / np.maximum(np.abs(h), 1e-30)
    err[h == 0] = np.inf
    p, c = np.unravel_index(np.argmin(err), err.shape)
    bad = h.copy()
    bad[p, c] = h[p, c] * (1 + 2.0 ** -7 if mode == "w4a16" else 1 + 2.0 ** -3)
    with pytest.raises(AssertionError):
        check_h(_as_gpu_h(bad, mode), inp, spec, ref, mode, f"planted h {mode}")


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_planted_alpha_mistake_fails(mode):
    """A GPU that used alpha_up 2 % too large produces an h that fails."""
    spec = S.spec_of(SHAPE)
    inp = S.generate(spec)
    ref = oracle_out(inp, spec, mode=mode, keep=True)
    P, I = int(ref["offsets"][-1]), spec["I"]
    wrong = dict(inp, alpha_up=np.asarray(inp["alpha_up"], np.float32) * np.float32(1.02))
    wref = oracle_out(wrong, spec, mode=mode, keep=True)
    with pytest.raises(AssertionError):
        check_h(_as_gpu_h(_full_rows(wref, P, I), mode), inp, spec, ref, mode, f"alpha_up +2 % {mode}")


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [1, 3])
def test_output_offset_of_two_percent_rms_fails(cfg):
    """On the TP8 decode and prefill workloads, an output off by a uniform
    2 % of its RMS fails the comparison with the oracle's FC2 and combine of
    a valid h (and the raw comparison) -- nothing is discounted."""
    inp = S.generate(cfg)
    spec = inp["spec"]
    tokens = np.arange(3)
    ref = oracle_out(inp, spec, tokens=tokens, keep=True)
    P, I = int(ref["offsets"][-1]), spec["I"]
    hrows = _full_rows(ref, P, I)
    cond = oracle_out(inp, spec, tokens=tokens, h_given=hrows)
    rms = np.sqrt(np.mean(ref["out"].astype(np.float64) ** 2))
    got = ref["out"].astype(np.float64) + 0.02 * rms
    parity(ref["out"], cond["out"], "unchanged output")
    with pytest.raises(AssertionError):
        parity(got, cond["out"], "offset output vs oracle FC2 of h")
    with pytest.raises(AssertionError):
        parity(got, ref["out"], "offset output vs oracle")


@pytest.mark.slow
def test_w4a8_output_is_ill_conditioned_in_the_fc1_accumulator():
    """The raw max-abs bar cannot hold in w4a8 for a computation whose FC1
    sums differ from the exact ones by the FP8 matrix cores' accumulation
    error (measured: up to 2^-12 of a 128-long K chunk's largest product):
    perturbing the oracle's own FC1 accumulators by 2^-14 of their K chunks'
    largest |product| (a quarter of that) moves under 1 % of the MXFP8
    rounding decisions of h, and the output of 16 TP8 prefill tokens by
    more than 1e-2 x RMS of the oracle's."""
    inp = S.generate(3)
    spec = inp["spec"]
    tokens = np.arange(16)
    ref = oracle_out(inp, spec, tokens=tokens, keep=True)
    I, H, k = spec["I"], spec["H"], spec["k"]
    rng = np.random.default_rng(3)
    xf = M.activations(inp, "w4a8", False)[0]
    pairs, offsets, perm = ref["pairs"], ref["offsets"], ref["perm"]
    P = int(offsets[-1])
    h_new = np.zeros((P, I))
    n_flip = 0
    for l in np.unique(np.searchsorted(offsets, pairs, side="right") - 1):
        q = np.nonzero((pairs >= offsets[l]) & (pairs < offsets[l + 1]))[0]
        W = F.dequant_mxfp4(inp["w1"][l], inp["w1_scale"][l])
        X = xf[perm[pairs[q]] // k]
        cm = np.stack([np.max(np.abs(X[:, None, c:c + 128]) * np.abs(W[None, :, c:c + 128]), axis=2)
                       for c in range(0, H, 128)]).sum(0)                     # [n, 2I]
        acc = ref["acc"][q] + rng.uniform(-1, 1, size=cm.shape) * 2.0 ** -14 * cm
        g = inp["alpha_gate"][l].astype(np.float64) * acc[:, :I]
        u = inp["alpha_up"][l].astype(np.float64) * acc[:, I:]
        h = M.situ(g, u, inp["situ_beta"][l], inp["situ_linear_beta"][l]).astype(np.float32).astype(np.float64)
        hq = F.mx_dequantize(*F.mx_quantize(h, "e4m3"), "e4m3")
        n_flip += int(np.count_nonzero(hq != ref["h"][q]))
        h_new[pairs[q]] = hq
    cond = oracle_out(inp, spec, tokens=tokens, h_given=h_new)
    rms = np.sqrt(np.mean(ref["out"].astype(np.float64) ** 2))
    dev = np.max(np.abs(cond["out"].astype(np.float64) - ref["out"]))
    frac = n_flip / (len(pairs) * I)
    print(f"perturbed accumulators: {n_flip} of {len(pairs) * I} h elements ({frac:.2e}) round the other way; "
          f"output max-abs {dev / rms:.2e} x RMS", flush=True)
    assert 0 < frac < 0.01
    assert dev > 1e-2 * rms

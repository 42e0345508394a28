"""CPU checks of the parity comparison used by the GPU tests.

The oracle's float32 mode (float32 BLAS, float32 SiTU) takes some rounding
decisions at the FC1 rounding point differently from the float64 reference,
exactly as a GPU would; the comparison must accept it.  A planted arithmetic
mistake must still be rejected, allowance or not.
"""

import numpy as np
import pytest

import synthetic as S
from oracle import moe as M

from gpu_helpers import _bf16_ambiguity, _mxfp8_ambiguity, h_uncertainty, oracle_out, parity, rounding_allowance

SHAPE = dict(T=600, H=512, I=256, E_g=8, E_l=6, off=1, k=4, seed=35, skew=True)


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_float32_path_passes_with_allowance(mode):
    spec = S.spec_of(dict(SHAPE, mode=mode))
    inp = S.generate(spec)
    ref = oracle_out(inp, spec, mode=mode, keep=True)
    f32 = M.moe_forward(inp, local_expert_offset=spec["off"], local_num_experts=spec["E_l"],
                        act_mode=mode, precision="f32")["out"]
    A = rounding_allowance(inp, spec, ref, mode)
    parity(f32, ref["out"], f"oracle f32 vs f64 ({mode})", A)
    # only elements of h on a rounding boundary are excused: a small fraction
    d = _bf16_ambiguity(ref["h_pre"]) if mode == "w4a16" else _mxfp8_ambiguity(ref["h_pre"])
    assert 0 < np.count_nonzero(d) < 1e-2 * d.size
    # with the FC1 accumulation bound: still a minority (bf16's grid is 16x finer than E4M3's)
    tol = h_uncertainty(inp, spec, ref, mode)
    d = _bf16_ambiguity(ref["h_pre"], tol) if mode == "w4a16" else _mxfp8_ambiguity(ref["h_pre"], tol)
    assert np.count_nonzero(d) < (0.15 if mode == "w4a16" else 0.02) * d.size
    # and the allowance is small next to the output scale
    assert np.max(A) < 0.2 * np.sqrt(np.mean(ref["out"] ** 2))


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_planted_mistake_still_fails(mode):
    spec = S.spec_of(dict(SHAPE, mode=mode))
    inp = S.generate(spec)
    ref = oracle_out(inp, spec, mode=mode, keep=True)
    bad = dict(inp, alpha_up=inp["alpha_up"] * np.float32(1.02))      # 2 % off on one factor
    wrong = M.moe_forward(bad, local_expert_offset=spec["off"], local_num_experts=spec["E_l"],
                          act_mode=mode)["out"]
    A = rounding_allowance(inp, spec, ref, mode)
    with pytest.raises(AssertionError):
        parity(wrong, ref["out"], f"planted mistake ({mode})", A)

"""GPU parity over a seeded sweep of layer shapes.

Twenty-four shapes drawn once from a fixed seed (hidden and intermediate
sizes from 64 to 768, multiples of 32 that are and are not multiples of
128, 1 to 16 local experts at any offset inside up to 40 global ones, top-1
to top-8, 1 to 400 tokens, uniform or skewed routing), each run in both
activation modes with the planner's tactics: the output is held to the
oracle (the GPU's h valid element by element, the oracle's FC2 and combine
on that h within the bar), and the fragment-tiled weights give the
row-major weights' output bit for bit.  Where K and I are multiples of 128,
the 128-row w4a8 tactic is also run from tiled weights (the 512-, 384- or
256-row kernels, by I) and from rows (the 256-row kernel): equal bit for bit
and held to the oracle.  w4a8 takes bf16 input, so its quantization runs in
the routing launch.
"""

import numpy as np
import pytest
import torch

import synthetic as S

from gpu_helpers import layer_check, run_layer

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sweep(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.choice([96, 128, 224, 256, 384, 512, 640, 768]))
        I = int(rng.choice([64, 96, 128, 160, 192, 256, 384, 512]))
        E_g = int(rng.integers(4, 41))
        E_l = int(rng.integers(1, min(E_g, 16) + 1))
        off = int(rng.integers(0, E_g - E_l + 1))
        k = int(rng.integers(1, min(8, E_g) + 1))
        T = int(rng.integers(1, 401))
        out.append(dict(T=T, H=H, I=I, E_g=E_g, E_l=E_l, off=off, k=k, seed=3000 + i,
                        skew=bool(rng.integers(0, 2))))
    return out


SWEEP = _sweep()


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("i", range(len(SWEEP)))
def test_shape_sweep(i):
    spec = S.spec_of(SWEEP[i])
    inp = S.generate(spec)
    for mode in ("w4a16", "w4a8"):
        got, plan, ws, _ = run_layer(inp, spec, mode=mode)
        layer_check(got, inp, spec, mode, plan, ws, what=f"sweep {i} {mode} {SWEEP[i]}")
        tiled, plan_t, _, _ = run_layer(inp, spec, mode=mode, tiled=True)
        assert (plan_t.fc1_tactic, plan_t.fc2_tactic) == (plan.fc1_tactic, plan.fc2_tactic)
        assert np.array_equal(_bits(got), _bits(tiled)), f"sweep {i} {mode}: tiled != row-major"
    if spec["H"] % 128 == 0 and spec["I"] % 128 == 0:
        rows, *_ = run_layer(inp, spec, mode="w4a8", tactic=(4, 20))
        tiled, plan_t, ws_t, _ = run_layer(inp, spec, mode="w4a8", tactic=(4, 20), tiled=True)
        assert np.array_equal(_bits(rows), _bits(tiled)), f"sweep {i} 128-row: tiled != row-major"
        layer_check(tiled, inp, spec, "w4a8", plan_t, ws_t, what=f"sweep {i} 128-row tiled {SWEEP[i]}")

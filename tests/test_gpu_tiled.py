"""GPU tests of the fragment-tiled MXFP4 weight layout (SITU_WEIGHTS_MXFP4_TILED)
through the C ABI.

situ_moe_tile_weights only moves bytes, so its output is checked byte for
byte against the layout as include/situ_moe.h defines it, restated here in
numpy.  The kernels compute the same products and sums in the same order
from either layout, so the layer's output from tiled weights must equal its
output from the row-major weights bit for bit, in every tactic (the 16-row
decode kernels, the fused decode kernel, the 64-row kernels of both
activation modes, the 128-row kernels with 256- and 512-row work items and
the short-K FC2 kernel), with
K tails, the general epilogue with LoRA bridges, and at full size; the
row-major runs are the ones the layer parity tests hold to the oracle, and
one tiled run is held to the oracle here as well.
"""

import numpy as np
import pytest
import torch

import block_scaled_mxfp4_amd as B
import synthetic as S

from gpu_helpers import dev, layer_check, run_layer

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def tiled_reference(w, ws):
    """The documented layout: block (rt, j) of expert e holds, at byte
    16 l + b, byte b of row 16 rt + l % 16, K block 4 j + l // 16 (zero past
    K); its scale block holds that row and block's scale at byte l (127 past K)."""
    E, R, half_k = w.shape
    nkb = 2 * half_k // 32
    S_ = (nkb + 3) // 4
    wt = np.zeros((E, R // 16, S_, 1024), np.uint8)
    st = np.full((E, R // 16, S_, 64), 127, np.uint8)
    for rt in range(R // 16):
        for j in range(S_):
            for l in range(64):
                row, kb = 16 * rt + l % 16, 4 * j + l // 16
                if kb < nkb:
                    wt[:, rt, j, 16 * l:16 * l + 16] = w[:, row, 16 * kb:16 * kb + 16]
                    st[:, rt, j, l] = ws[:, row, kb]
    return wt, st


@pytest.mark.parametrize("E,R,K", [(3, 48, 96), (2, 32, 384), (2, 16, 416), (1, 64, 3584)])
def test_tile_weights_layout(E, R, K):
    rng = np.random.default_rng(E * 1000 + R + K)
    w = rng.integers(0, 256, (E, R, K // 2), dtype=np.uint8)
    ws = rng.integers(100, 140, (E, R, K // 32), dtype=np.uint8)
    # outputs prefilled with a pattern the call must overwrite everywhere
    shp_w, shp_s = B.tiled_shapes(E, R, K)
    wt = torch.full(shp_w, 0xA5, dtype=torch.uint8, device="cuda")
    st = torch.full(shp_s, 0x5A, dtype=torch.uint8, device="cuda")
    B.situ_moe_tile_weights(dev(w), dev(ws), wt, st)
    torch.cuda.synchronize()
    ref_w, ref_s = tiled_reference(w, ws)
    assert np.array_equal(wt.cpu().numpy(), ref_w)
    assert np.array_equal(st.cpu().numpy(), ref_s)


def test_tile_weights_rejects_bad_shapes():
    w = torch.zeros((1, 24, 64), dtype=torch.uint8, device="cuda")
    s = torch.zeros((1, 24, 4), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.SituMoeError):   # rows not a multiple of 16
        B.situ_moe_tile_weights(w, s)


SHAPES = {
    # 16-row decode kernels, several m-tiles per expert
    "decode": dict(T=200, H=640, I=512, E_g=8, E_l=8, off=0, k=4, seed=91, skew=True),
    # FC1 K split in two (H = 3584), I = 384
    "tp": dict(T=24, H=3584, I=384, E_g=96, E_l=96, off=0, k=8, seed=92, skew=True),
    # K tails: H = 96 and I = 96 are partial 128-wide steps
    "ragged": dict(T=37, H=96, I=96, E_g=13, E_l=5, off=4, k=3, seed=93),
    # prefill-sized groups; H = 384 is an odd number of K steps (the wide
    # kernel's last two-step stage is half empty), FC2 at K = I = 512 takes
    # the wide kernel
    "prefill": dict(T=900, H=384, I=512, E_g=6, E_l=4, off=1, k=3, seed=94, skew=True),
    # FC2 at K = I = 384 takes the short-K kernel, FC1 the 256-row kernel
    # (I not a multiple of 256)
    "short": dict(T=700, H=640, I=384, E_g=6, E_l=4, off=1, k=3, seed=95, skew=True),
    # I = 128: one 256-row FC1 n-tile per m-tile; FC2 at K = 128
    "narrow": dict(T=300, H=256, I=128, E_g=4, E_l=4, off=0, k=2, seed=96, skew=True),
    # the 512-row FC1 kernel's pipelined K loop at 1, 2 and 5 K steps (its
    # ring of three stages: no step after the first, no stage beyond the
    # first three, and a rotation that does not end on the ring's start)
    "k1": dict(T=600, H=128, I=256, E_g=4, E_l=4, off=0, k=2, seed=97, skew=True),
    "k2": dict(T=640, H=256, I=256, E_g=5, E_l=3, off=1, k=2, seed=98, skew=True),
    "k5": dict(T=700, H=640, I=512, E_g=5, E_l=4, off=0, k=3, seed=99, skew=True),
}
TACTICS = {"w4a16": [(0, 16), (1, 17), (5, 21)], "w4a8": [(2, 18), (3, 19), (4, 20), (6, 22)]}


def _cases():
    out = []
    for name, c in SHAPES.items():
        for mode, tacs in TACTICS.items():
            for tac in tacs:
                if tac == (4, 20) and (c["H"] % 128 or c["I"] % 128):
                    continue
                if tac[0] in (5, 6) and c["I"] > 768:
                    continue
                out.append((name, mode, tac))
    return out


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("name,mode,tactic", _cases())
def test_tiled_equals_row_major_bitwise(name, mode, tactic):
    spec = S.spec_of(SHAPES[name])
    inp = S.generate(spec)
    rows, plan_r, _, _ = run_layer(inp, spec, mode=mode, tactic=tactic)
    tiled, plan_t, _, _ = run_layer(inp, spec, mode=mode, tactic=tactic, tiled=True)
    assert (plan_t.fc1_tactic, plan_t.fc2_tactic) == (plan_r.fc1_tactic, plan_r.fc2_tactic) == tactic
    print(f"{name} {mode} {tactic}: {np.sum(_bits(rows) != _bits(tiled))} differing elements", flush=True)
    assert np.array_equal(_bits(rows), _bits(tiled))


@pytest.mark.parametrize("shape,mode,tactic", [("prefill", "w4a16", (0, 16)), ("prefill", "w4a16", (1, 17)),
                                               ("prefill", "w4a8", (3, 19)), ("prefill", "w4a8", (4, 20)),
                                               ("short", "w4a8", (4, 20))])
def test_tiled_general_epilogue_and_lora_bridges(shape, mode, tactic):
    spec = S.spec_of(dict(SHAPES[shape], activation="swiglu_bias", lora=True))
    inp = S.generate(spec)
    rows, _, _, dr = run_layer(inp, spec, mode=mode, tactic=tactic, lora_out=True)
    tiled, _, _, dt = run_layer(inp, spec, mode=mode, tactic=tactic, lora_out=True, tiled=True)
    assert np.array_equal(_bits(rows), _bits(tiled))
    a = dr["activation_lora_input"].view(torch.int16).cpu().numpy()
    b = dt["activation_lora_input"].view(torch.int16).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_tiled_layer_at_the_parity_bar(mode):
    """A tiled run held to the oracle directly (h valid, output within the bar)."""
    spec = S.spec_of(SHAPES["ragged"])
    inp = S.generate(spec)
    out, plan, ws, _ = run_layer(inp, spec, mode=mode, tiled=True)
    layer_check(out, inp, spec, mode, plan, ws, what=f"tiled ragged {mode}")


@pytest.mark.parametrize("cfg,prequantized", [(1, False), (2, False), (3, True), (4, True)])
def test_tiled_full_size_bitwise(cfg, prequantized):
    """The four shard workloads at full size, in the planner's tactics: tiled
    weights give the row-major output bit for bit."""
    spec = S.spec_of(cfg)
    inp = S.generate(spec)
    rows, plan_r, _, _ = run_layer(inp, spec, prequantized=prequantized)
    torch.cuda.empty_cache()
    tiled, plan_t, _, _ = run_layer(inp, spec, prequantized=prequantized, tiled=True)
    assert (plan_t.fc1_tactic, plan_t.fc2_tactic) == (plan_r.fc1_tactic, plan_r.fc2_tactic)
    assert np.isfinite(tiled).all()
    print(f"config {cfg}: {np.sum(_bits(rows) != _bits(tiled))} differing elements", flush=True)
    assert np.array_equal(_bits(rows), _bits(tiled))

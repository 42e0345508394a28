"""Checks of the seeded input generator (not of the layer).

The MXFP4 weights are drawn directly as codes from fixed tables; here the
tables are re-measured against the oracle's MX quantizer applied to real
N(0, 0.02) draws, and the routing constraints of each workload are checked.
"""

import numpy as np
import pytest

import synthetic as S
from oracle import formats as F
from oracle import moe as M


def test_weight_code_tables_match_quantized_gaussian():
    rng = np.random.default_rng(99)
    w = rng.standard_normal((200000, 32)) * 0.02
    codes, sc = F.mx_quantize(w, "e2m1")
    sc = sc[:, 0]
    got_p, got_s = S.draw_mxfp4([7, 1, 0], 2000, 3200)
    gs = got_s.ravel()
    for s in (119, 120, 121):
        assert abs(np.mean(sc == s) - np.mean(gs == s)) < 0.004, s
    # element code frequencies under the dominant scale 120
    want = np.bincount(codes[sc == 120].ravel(), minlength=16) / codes[sc == 120].size
    el = F.unpack_fp4(got_p, 3200)
    mask = np.repeat(got_s == 120, 32, axis=1)
    have = np.bincount(el[mask].ravel(), minlength=16) / mask.sum()
    assert np.max(np.abs(want - have)) < 0.006
    # the drawn weights have the recipe's spread
    vals = F.dequant_mxfp4(got_p, got_s)
    assert abs(vals.std() - 0.02) < 0.0015


def test_generation_is_deterministic():
    a = S.generate(dict(T=5, H=64, I=32, E_g=6, E_l=3, off=2, k=2, seed=3, packed=True))
    b = S.generate(dict(T=5, H=64, I=32, E_g=6, E_l=3, off=2, k=2, seed=3, packed=True))
    for key in a:
        if key != "spec":
            assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_workload_routing_statistics(cfg):
    d = S.generate(cfg, weights=False)
    s = d["spec"]
    ids = d["topk_ids"]
    assert ids.shape == (s["T"], s["k"])
    # no duplicate expert within one token's top-k
    srt = np.sort(ids, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])
    counts, offsets, perm, inv = M.route(ids, s["off"], s["E_l"])
    if cfg == 4:
        nolocal = (inv.reshape(s["T"], s["k"]) < 0).all(axis=1).sum()
        assert nolocal == int(0.3 * s["T"])
        assert (counts == 0).sum() == 8
        ids2, wbits = M.unpack_topk(d["topk_packed"])
        assert np.array_equal(ids2, ids) and np.array_equal(wbits, d["topk_weights"])
    # softmax weights over the k slots sum to ~1 (bf16 truncation loses < 1%)
    w = F.bf16_to_f64(d["topk_weights"]).sum(axis=1)
    assert np.all((w > 0.97) & (w <= 1.0 + 1e-6))

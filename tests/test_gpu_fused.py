"""GPU tests of the fused decode kernel (FC1 and FC2 of each 16-row m-tile in
one launch, h kept in LDS) through the C ABI.

The fused kernel runs the unfused decode kernels' work items (same K split,
reduction order and epilogue arithmetic), so its output must equal the
unfused 16-row path bit for bit, on the same inputs; the unfused path is the
one the layer parity tests hold to the oracle.  Covered: both activation
modes, the three FC1 K splits (H = 640, 3584, 4096), ragged groups and K
tails, the general epilogue (SwigluBias) with the LoRA bridges, the full-size
TP8 decode shard, and the sizes where the fused pair is not offered.
"""

import numpy as np
import pytest
import torch

import block_scaled_mxfp4_amd as B
import synthetic as S

from gpu_helpers import layer_check, run_layer

pytestmark = pytest.mark.gpu

FUSED = {"w4a16": (5, 21), "w4a8": (6, 22)}
UNFUSED = {"w4a16": (0, 16), "w4a8": (2, 18)}

SHAPES = {
    # several m-tiles per expert, FC1 K not split (5 steps)
    "decode": dict(T=200, H=640, I=512, E_g=8, E_l=8, off=0, k=4, seed=81, skew=True),
    # TP8-like: H = 3584 (FC1 K split in two), I = 384, many small groups
    "tp": dict(T=24, H=3584, I=384, E_g=96, E_l=96, off=0, k=8, seed=82, skew=True),
    # FC1 K split in four (32 steps), a shard of the experts
    "deep": dict(T=40, H=4096, I=256, E_g=32, E_l=12, off=10, k=6, seed=83),
    # K tails: H = 96 and I = 96 are partial 128-wide steps
    "ragged": dict(T=37, H=96, I=96, E_g=13, E_l=5, off=4, k=3, seed=84),
}


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
@pytest.mark.parametrize("name", list(SHAPES))
def test_fused_equals_unfused_bitwise(name, mode):
    spec = S.spec_of(SHAPES[name])
    inp = S.generate(spec)
    fused, plan_f, _, _ = run_layer(inp, spec, mode=mode, tactic=FUSED[mode])
    assert (plan_f.fc1_tactic, plan_f.fc2_tactic) == FUSED[mode]
    plain, plan_u, ws_u, _ = run_layer(inp, spec, mode=mode, tactic=UNFUSED[mode])
    print(f"{name} {mode}: fused vs unfused, {np.sum(_bits(fused) != _bits(plain))} differing elements", flush=True)
    assert np.array_equal(_bits(fused), _bits(plain))
    # the unfused run itself at the parity bar (h valid, output against the oracle)
    layer_check(plain, inp, spec, mode, plan_u, ws_u, what=f"unfused {name} {mode}")


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_fused_general_epilogue_and_lora_bridges(mode):
    """SwigluBias with a gate_up LoRA delta and the down-LoRA input rows: the
    general epilogue inside the fused kernel."""
    spec = S.spec_of(dict(SHAPES["decode"], activation="swiglu_bias", lora=True))
    inp = S.generate(spec)
    fused, _, _, df = run_layer(inp, spec, mode=mode, tactic=FUSED[mode], lora_out=True)
    plain, _, _, du = run_layer(inp, spec, mode=mode, tactic=UNFUSED[mode], lora_out=True)
    assert np.array_equal(_bits(fused), _bits(plain))
    a = df["activation_lora_input"].view(torch.int16).cpu().numpy()
    b = du["activation_lora_input"].view(torch.int16).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_fused_full_size_tp8_decode(mode):
    """The TP8 decode shard at full size (64 tokens, 896 local experts,
    H = 3584, I = 384): the fused pair is offered and equals the unfused
    path bit for bit."""
    spec = S.spec_of(1)
    inp = S.generate(spec)
    prob = B.make_problem(num_tokens=spec["T"], hidden_size=spec["H"], intermediate_size=spec["I"],
                          num_experts=spec["E_g"], local_expert_offset=spec["off"], local_num_experts=spec["E_l"],
                          top_k=spec["k"], act_mode=mode)
    assert FUSED[mode] in B.situ_moe_valid_tactics(prob)
    fused, *_ = run_layer(inp, spec, mode=mode, tactic=FUSED[mode])
    plain, *_ = run_layer(inp, spec, mode=mode, tactic=UNFUSED[mode])
    assert np.isfinite(fused).all()
    assert np.array_equal(_bits(fused), _bits(plain))


def test_fused_not_offered_where_h_does_not_fit():
    """I = 3072 (the EP8 shards): 16 rows of h exceed the fused kernel's LDS
    share; the pair is not offered, and asking for it is an error."""
    spec = S.spec_of(2)
    prob = B.make_problem(num_tokens=spec["T"], hidden_size=spec["H"], intermediate_size=spec["I"],
                          num_experts=spec["E_g"], local_expert_offset=spec["off"], local_num_experts=spec["E_l"],
                          top_k=spec["k"], act_mode="w4a16", tactic=FUSED["w4a16"])
    assert FUSED["w4a16"] not in B.situ_moe_valid_tactics(prob)
    with pytest.raises(B.SituMoeError):
        B.situ_moe_plan(prob)

"""situ_moe_run_static (no workspace, no allocation) against situ_moe_run on
the same inputs: identical outputs bit for bit, on two calls in a row, the
second with a smaller batch, through the C ABI."""

import ctypes

import numpy as np
import pytest
import torch

import block_scaled_mxfp4_amd as B
import synthetic as S

from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _tensors(inp, spec, mode):
    T, H, I, k = spec["T"], spec["H"], spec["I"], spec["k"]
    prob = B.make_problem(num_tokens=T, hidden_size=H, intermediate_size=I, num_experts=spec["E_g"],
                          local_expert_offset=spec["off"], local_num_experts=spec["E_l"], top_k=k, act_mode=mode)
    d = {key: dev(inp[key]) for key in ("hidden_states", "topk_ids", "topk_weights", "w1", "w1_scale", "w2",
                                        "w2_scale", "situ_beta", "situ_linear_beta", "alpha_gate", "alpha_up")}
    d["out"] = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    return prob, d


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_static_scratch_matches_workspace_run(mode):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = S.spec_of(dict(S.CONFIGS[1], T=64, mode=mode, seed=101))     # the TP8 decode shard
    small = S.spec_of(dict(S.CONFIGS[1], T=9, mode=mode, seed=102))
    for spec in (big, small):                                           # two calls, the second smaller
        inp = S.generate(spec)
        prob, d = _tensors(inp, spec, mode)
        plan = B.situ_moe_plan(prob)
        assert plan.workspace_bytes <= B.STATIC_SCRATCH_BYTES
        ts = B.make_tensors(prob, **d)
        B.situ_moe_run_static(plan, ts)
        torch.cuda.synchronize()
        got = d["out"].clone()
        d["out"].fill_(float("nan"))
        ws = B.new_workspace(plan)
        B.situ_moe_run(plan, ts, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all()
        assert torch.equal(got.view(torch.int32), d["out"].view(torch.int32)), spec["T"]
        print(f"T={spec['T']} {mode}: static scratch output equals the workspace run bit for bit", flush=True)


def test_static_scratch_rejects_large_plans():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    prob = B.make_problem(num_tokens=16384, hidden_size=3584, intermediate_size=384, num_experts=896,
                          local_expert_offset=0, local_num_experts=896, top_k=16, act_mode="w4a8")
    plan = B.situ_moe_plan(prob)
    assert plan.workspace_bytes > B.STATIC_SCRATCH_BYTES
    with pytest.raises(B.SituMoeError) as e:
        B.situ_moe_run_static(plan, B.SituMoeTensors())
    assert e.value.status_name == "SITU_E_WORKSPACE"

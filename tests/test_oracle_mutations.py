"""Plant plausible mistakes in a copy of the oracle and check a pin catches each.

Each mutation rewrites one line of oracle source in a fresh module (the real
oracle is untouched), points the pin tests at the mutant, and requires at
least one pin to fail.  This shows the pins are sharp enough to notice a
dropped term, a wrong sign or index, or a swapped operand.
"""

import importlib.util
import inspect
import sys
import types

import numpy as np
import pytest

import oracle.formats as real_F
import oracle.moe as real_M

import test_oracle_formats as TF
import test_oracle_moe as TM


def _mutant(module, old, new):
    src = inspect.getsource(module)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType(module.__name__ + "_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src, module.__name__ + "_mutant", "exec"), mod.__dict__)
    return mod


def _run_pins(tests, golden_dir):
    failures = 0
    for fn in tests:
        params = inspect.signature(fn).parameters
        kwargs = {}
        if "golden_dir" in params:
            kwargs["golden_dir"] = golden_dir
        variants = [{}]
        if "mode" in params:
            variants = [{"mode": "w4a16"}, {"mode": "w4a8"}]
        for v in variants:
            try:
                fn(**kwargs, **v)
            except (AssertionError, ValueError, IndexError):
                failures += 1
    return failures


MOE_PINS = [TM.test_routed_equals_dense_unrouted_moe, TM.test_golden_per_token_skeleton,
            TM.test_top1_single_expert_is_dense_mlp, TM.test_route_matches_bruteforce_recount,
            TM.test_out_of_shard_ids_contribute_nothing, TM.test_fc1_output_rounding_point,
            TM.test_w4a8_activation_scale_applied_once, TM.test_fc1_products_integer_exact,
            TM.test_situ_large_beta_is_swiglu, TM.test_situ_zeros_and_bounds,
            TM.test_situ_with_k3_constants_matches_mpmath_free_closed_form,
            TM.test_tp_shards_sum_to_unsharded]

MOE_MUTATIONS = [
    ("sigmoid of the squashed gate", "(beta * np.tanh(g / beta) * sigmoid(g))",
     "(beta * np.tanh(g / beta) * sigmoid(beta * np.tanh(g / beta)))"),
    ("beta and linear beta swapped", "return (beta * np.tanh(g / beta) * sigmoid(g)) * (linear_beta * np.tanh(u / linear_beta))",
     "return (linear_beta * np.tanh(g / linear_beta) * sigmoid(g)) * (beta * np.tanh(u / beta))"),
    ("gate and up halves swapped", "g = rnd(np.float64(a_g[l]) * acc[:, :I])", "g = rnd(np.float64(a_g[l]) * acc[:, I:])"),
    ("alpha_up dropped", "u = rnd(np.float64(a_u[l]) * acc[:, I:])", "u = rnd(acc[:, I:])"),
    ("alpha_gate used for up", "u = rnd(np.float64(a_u[l]) * acc[:, I:])", "u = rnd(np.float64(a_g[l]) * acc[:, I:])"),
    ("perm ordered by j only", "order = np.lexsort((jl, ll))", "order = np.argsort(jl, kind='stable')"),
    ("off-by-one shard filter", "local = (l >= 0) & (l < local_num_experts)", "local = (l >= 0) & (l <= local_num_experts)"),
    ("token index from wrong divisor", "rows_t = perm[pos] // k", "rows_t = perm[pos] % T"),
    ("combine weight of wrong slot", "wsl = wts[tokens[has], s]", "wsl = wts[tokens[has], 0]"),
    ("no bf16 rounding of h", "hq = F.bf16_to_f64(F.f32_to_bf16_rne(_f32(h)))", "hq = np.asarray(h, np.float64)"),
    ("activation scale applied twice",
     "return F.mx_dequantize(codes, scales, \"e4m3\"), codes, scales",
     "return F.mx_dequantize(codes, scales, \"e4m3\") * F.mx_dequantize(np.full_like(codes, 0x38), scales, \"e4m3\"), codes, scales"),
    ("W2 transposed operand", "W2d = dequant(w2[l], w2s[l]).astype(dt, copy=False)        # [H, I]",
     "W2d = dequant(w2[l], w2s[l]).astype(dt, copy=False)[::-1]"),
]


@pytest.mark.parametrize("name,old,new", MOE_MUTATIONS, ids=[m[0] for m in MOE_MUTATIONS])
def test_moe_pins_catch_mutation(name, old, new, golden_dir, monkeypatch):
    mut = _mutant(real_M, old, new)
    monkeypatch.setattr(TM, "M", mut)
    assert _run_pins(MOE_PINS, golden_dir) > 0, f"no pin caught: {name}"


FORMAT_PINS = [TF.test_e2m1_decode_matches_ocp_table, TF.test_e2m1_decode_matches_bitfields,
               TF.test_e4m3_decode_matches_torch_all_codes, TF.test_e8m0_decode_matches_torch_all_codes,
               TF.test_fp4_nibble_order_roundtrip, TF.test_bf16_rne_matches_torch,
               TF.test_e4m3_encode_bruteforce_all_bf16, TF.test_e2m1_encode_bruteforce,
               TF.test_mx_scale_rule_at_powers_of_two, TF.test_mxfp8_hand_worked_block,
               TF.test_mx_quantize_error_bound_and_top_binade, TF.test_floor_log2_exact_near_powers_of_two]

FORMAT_MUTATIONS = [
    ("nibble order reversed", "out[..., 0::2] = lo\n    out[..., 1::2] = hi", "out[..., 0::2] = hi\n    out[..., 1::2] = lo"),
    ("E8M0 bias off by one", "val = np.ldexp(1.0, codes - 127)", "val = np.ldexp(1.0, codes - 126)"),
    ("E4M3 subnormal exponent", "np.ldexp(m.astype(np.float64), -9)", "np.ldexp(m.astype(np.float64), -10)"),
    ("E2M1 table entry", "np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]", "np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0]"),
    ("ties away from zero", "((d_hi == d_lo) & ((c_hi & 1) == 0))", "(d_hi == d_lo)"),
    ("float log2 for the scale", "_, ex = np.frexp(np.asarray(a, dtype=np.float64))\n    return ex.astype(np.int64) - 1",
     "return np.floor(np.log2(np.asarray(a, dtype=np.float64)) + 1e-15).astype(np.int64)"),
    ("wrong element emax", "emax, enc = E4M3_EMAX, encode_e4m3", "emax, enc = E4M3_EMAX - 1, encode_e4m3"),
    ("bf16 ties up", "round_up = (rem > half) | ((rem == half) & (lsb == 1))", "round_up = rem >= half"),
]


@pytest.mark.parametrize("name,old,new", FORMAT_MUTATIONS, ids=[m[0] for m in FORMAT_MUTATIONS])
def test_format_pins_catch_mutation(name, old, new, golden_dir, monkeypatch):
    mut = _mutant(real_F, old, new)
    monkeypatch.setattr(TF, "F", mut)
    assert _run_pins(FORMAT_PINS, golden_dir) > 0, f"no pin caught: {name}"

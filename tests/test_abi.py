"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load here, export every entry point include/situ_moe.h
declares, agree with the Python binding on struct layouts, and return the
documented status for every error the host can detect.
"""

import ctypes
import os
import re
import subprocess

import pytest

import block_scaled_mxfp4_amd as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "situ_moe.h")


def _header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(situ_moe_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = B.load()
    names = _header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert B.situ_moe_abi_version() == B.ABI_VERSION == 3
    info = B.situ_moe_build_info()
    assert "gfx950" in info and "abi 3" in info


def test_struct_layout_matches_header(tmp_path):
    fields = {
        "situ_moe_problem": [f[0] for f in B.SituMoeProblem._fields_],
        "situ_moe_plan_t": [f[0] for f in B.SituMoePlan._fields_],
        "situ_moe_tensors": [f[0] for f in B.SituMoeTensors._fields_],
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void) {"]
    for st, fs in fields.items():
        lines.append(f'printf("{st} size %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'printf("{st} {f} %zu\\n", offsetof({st}, {f}));')
    lines.append("return 0; }")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(c), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    py = {"situ_moe_problem": B.SituMoeProblem, "situ_moe_plan_t": B.SituMoePlan,
          "situ_moe_tensors": B.SituMoeTensors}
    n = 0
    for line in out:
        if not line:
            continue
        st, f, v = line.split()
        cls = py[st]
        if f == "size":
            assert ctypes.sizeof(cls) == int(v), st
        else:
            assert getattr(cls, f).offset == int(v), (st, f)
        n += 1
    assert n == sum(len(v) + 1 for v in fields.values())


def _prob(**kw):
    base = dict(num_tokens=64, hidden_size=3584, intermediate_size=384, num_experts=896,
                local_expert_offset=0, local_num_experts=896, top_k=16)
    base.update(kw)
    return B.make_problem(**base)


def _status(fn):
    try:
        fn()
    except B.SituMoeError as e:
        return e.status_name
    return "SITU_OK"


@pytest.mark.parametrize("kw,want", [
    (dict(), "SITU_OK"),
    (dict(hidden_size=3600), "SITU_E_BAD_SHAPE"),
    (dict(intermediate_size=400), "SITU_E_BAD_SHAPE"),
    (dict(num_tokens=-1), "SITU_E_BAD_SHAPE"),
    (dict(num_experts=65536), "SITU_E_BAD_SHAPE"),
    (dict(local_expert_offset=800, local_num_experts=112), "SITU_E_BAD_SHAPE"),
    (dict(local_expert_offset=-1), "SITU_E_BAD_SHAPE"),
    (dict(local_num_experts=0), "SITU_E_BAD_SHAPE"),
    (dict(num_experts=4096, local_num_experts=2048), "SITU_E_UNSUPPORTED"),
    (dict(top_k=0), "SITU_E_BAD_SHAPE"),
    (dict(top_k=897), "SITU_E_BAD_SHAPE"),
    (dict(act_mode=7), "SITU_E_UNSUPPORTED"),
    (dict(act_prequantized=True), "SITU_E_UNSUPPORTED"),
    (dict(act_mode="w4a8", act_prequantized=True), "SITU_OK"),
    (dict(out_dtype=5), "SITU_E_UNSUPPORTED"),
    (dict(tactic=(99, -1)), "SITU_E_UNSUPPORTED"),
    (dict(tactic=(0, 17)), "SITU_E_UNSUPPORTED"),    # m-tile sizes differ
    (dict(tactic=(2, 18)), "SITU_E_UNSUPPORTED"),    # w4a8 tactics on a w4a16 problem
    (dict(tactic=(0, -1)), "SITU_OK"),
    (dict(num_tokens=0), "SITU_OK"),
    (dict(num_tokens=300000), "SITU_E_UNSUPPORTED"),   # 2.15 GB of hidden states
    (dict(activation="swiglu"), "SITU_OK"),
    (dict(activation="swiglu_bias", act_mode="w4a8"), "SITU_OK"),
    (dict(activation=3), "SITU_E_UNSUPPORTED"),
    (dict(weight_format="nvfp4"), "SITU_OK"),
    (dict(weight_format="nvfp4", act_mode="w4a8"), "SITU_E_UNSUPPORTED"),   # NVFP4 with bf16 activations only
    (dict(weight_format="mxfp4_tiled"), "SITU_OK"),
    (dict(weight_format="mxfp4_tiled", act_mode="w4a8"), "SITU_OK"),
    (dict(weight_format=3), "SITU_E_UNSUPPORTED"),
])
def test_plan_validation(kw, want):
    assert _status(lambda: B.situ_moe_plan(_prob(**kw))) == want


def test_plan_layout_and_tactics():
    for kw in (dict(), dict(num_tokens=16384, act_mode="w4a8"),
               dict(num_tokens=32768, local_num_experts=112, local_expert_offset=336,
                    intermediate_size=3072, act_mode="w4a8", topk_packed=True)):
        p = _prob(**kw)
        plan = B.situ_moe_plan(p)
        pairs = B.situ_moe_valid_tactics(p)
        assert (plan.fc1_tactic, plan.fc2_tactic) == pairs[0]
        assert B.situ_moe_tactic_name(plan.fc1_tactic).startswith("fc1_")
        assert B.situ_moe_tactic_name(plan.fc2_tactic).startswith("fc2_")
        T, k, E, H, I = p.num_tokens, p.top_k, p.local_num_experts, p.hidden_size, p.intermediate_size
        w4a8 = p.act_mode == B.ACT_W4A8
        sizes = {"off_counts": 4 * E, "off_offsets": 4 * (E + 1), "off_mtiles": 4 * (E + 1),
                 "off_tile_expert": 4 * plan.max_mtiles, "off_perm": 4 * (T * k + 64), "off_inv": 4 * T * k,
                 "off_xq": T * H if w4a8 else 0, "off_xs": T * H // 32 if w4a8 else 0,
                 "off_h": T * k * I * (1 if w4a8 else 2), "off_hs": T * k * I // 32 if w4a8 else 0,
                 "off_y": (-(-2 * T * k * H // 256) * 256 + T * k * -(-H // 64)) if plan.y_format else 4 * T * k * H,
                 "off_route_hist": 4 * plan.route_blocks * E if plan.route_blocks > 1 else 0,
                 "off_tile_rows": 8 * plan.max_mtiles}
        spans = sorted((getattr(plan, n), getattr(plan, n) + s) for n, s in sizes.items())
        for (a0, a1), (b0, _) in zip(spans, spans[1:]):
            assert a1 <= b0
        assert all(getattr(plan, n) % 256 == 0 for n in sizes)
        assert spans[-1][1] <= plan.workspace_bytes
        assert plan.max_mtiles >= (T * k + plan.block_m - 1) // plan.block_m
        # compact y (fp16 + one exponent byte per 64 columns) only with the 128-row tactic
        assert plan.y_format == (1 if plan.fc2_tactic == 20 else 0)
        if plan.y_format:
            assert plan.off_y_exp == plan.off_y + -(-2 * T * k * H // 256) * 256
    # decode batches are routed by one workgroup, prefill batches by blocks
    assert B.situ_moe_plan(_prob()).route_blocks == 1
    big = B.situ_moe_plan(_prob(num_tokens=32768, local_num_experts=112, local_expert_offset=336))
    assert big.route_blocks == 128 and big.route_chunk == 4096
    # decode shapes take 16-row m-tiles, prefill shapes 64-row ones, and
    # w4a8 groups of more than 192 rows on average 128-row ones
    assert B.situ_moe_plan(_prob()).block_m == 16
    assert B.situ_moe_plan(_prob(num_tokens=4096, act_mode="w4a8")).block_m == 64
    assert B.situ_moe_plan(_prob(num_tokens=16384, act_mode="w4a16")).block_m == 64
    assert B.situ_moe_plan(_prob(num_tokens=16384, act_mode="w4a8")).block_m == 128
    assert B.situ_moe_valid_tactics(_prob(num_tokens=16384, act_mode="w4a8"))[:2] == [(4, 20), (3, 19)]
    # an EP shard's groups are sized by the whole batch over all E_g experts:
    # 256 decode tokens over 56 of 896 experts average ~4.6 local rows each
    ep16 = dict(num_tokens=256, intermediate_size=3072, local_num_experts=56, local_expert_offset=280)
    assert B.situ_moe_plan(_prob(**ep16)).block_m == 16
    assert B.situ_moe_plan(_prob(**dict(ep16, num_tokens=32768, act_mode="w4a8"))).block_m == 128
    # the 128-row kernel needs sizes that are multiples of 128
    assert (4, 20) not in B.situ_moe_valid_tactics(_prob(num_tokens=16384, act_mode="w4a8", intermediate_size=416))


def test_run_argument_errors_before_any_device_work():
    lib = B.load()
    p = _prob(num_tokens=4, hidden_size=256, intermediate_size=64, num_experts=8, local_num_experts=8, top_k=2)
    plan = B.situ_moe_plan(p)
    fake = 1 << 20   # never dereferenced: every case fails on the host first
    full = dict(hidden_states=fake, topk_ids=fake, topk_weights=fake, w1=fake, w1_scale=fake, w2=fake,
                w2_scale=fake, situ_beta=fake, situ_linear_beta=fake, out=fake)

    def run(plan_, ws_bytes=plan.workspace_bytes, ws=256 * 1024, **over):
        t = B.SituMoeTensors(**dict(full, **over))
        return lib.situ_moe_run(ctypes.byref(plan_), ctypes.byref(t), ctypes.c_void_p(ws), ws_bytes, None)

    assert run(plan, situ_beta=None) == 1                       # beta required, never defaulted
    assert run(plan, situ_linear_beta=None) == 1
    assert run(plan, w2_scale=None) == 1
    assert run(plan, topk_weights=None) == 1
    assert run(plan, out=None) == 1
    assert run(plan, ws_bytes=plan.workspace_bytes - 1) == 6
    assert run(plan, ws=0) == 6
    assert run(plan, ws=256 * 1024 + 8) == 6                    # unaligned
    p8 = _prob(num_tokens=4, hidden_size=256, intermediate_size=64, num_experts=8, local_num_experts=8,
               top_k=2, act_mode="w4a8", act_prequantized=True)
    plan8 = B.situ_moe_plan(p8)
    assert run(plan8, ws_bytes=plan8.workspace_bytes) == 4      # MXFP8 input without its scales
    assert lib.situ_moe_run(None, None, None, 0, None) == 1
    assert "NULL" in B.situ_moe_last_error() or "null" in B.situ_moe_last_error().lower()
    # 16-byte alignment of the row arrays, 4-byte of the per-expert floats
    assert run(plan, w1=fake + 8) == 2 and "w1" in B.situ_moe_last_error()
    assert run(plan, hidden_states=fake + 2) == 2
    assert run(plan, out=fake + 4) == 2
    assert run(plan, alpha_gate=fake + 4) != 2              # 4-byte aligned floats pass the alignment check
    assert run(plan, situ_beta=fake + 2) == 2
    assert run(plan, gate_up_lora_delta=fake + 8) == 2
    # SwigluBias needs its two parameter arrays; SwiGLU needs none, SiTU's betas are then ignored
    pb = _prob(num_tokens=4, hidden_size=256, intermediate_size=64, num_experts=8, local_num_experts=8, top_k=2,
               activation="swiglu_bias")
    planb = B.situ_moe_plan(pb)
    assert run(planb, ws_bytes=planb.workspace_bytes) == 1
    assert run(planb, ws_bytes=planb.workspace_bytes, swiglu_alpha=fake) == 1


def test_no_device_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = B.load()
    p = _prob(num_tokens=4, hidden_size=256, intermediate_size=64, num_experts=8, local_num_experts=8, top_k=2)
    plan = B.situ_moe_plan(p)
    fake = 1 << 20
    t = B.SituMoeTensors(hidden_states=fake, topk_ids=fake, topk_weights=fake, w1=fake, w1_scale=fake,
                         w2=fake, w2_scale=fake, situ_beta=fake, situ_linear_beta=fake, out=fake)
    st = lib.situ_moe_run(ctypes.byref(plan), ctypes.byref(t), ctypes.c_void_p(256 * 1024),
                          plan.workspace_bytes, None)
    assert st == 5, B.situ_moe_last_error()
    assert B.situ_moe_status_string(5) == "SITU_E_DEVICE"


def test_tile_weights_argument_errors_before_any_device_work():
    lib = B.load()
    fake = 1 << 20   # never dereferenced: every case fails on the host first

    def tile(E=2, R=32, K=256, w=fake, s=fake, wt=fake + (1 << 24), st=fake + (1 << 25)):
        return lib.situ_moe_tile_weights(ctypes.c_void_p(w), ctypes.c_void_p(s), E, R, K, ctypes.c_void_p(wt),
                                         ctypes.c_void_p(st), None)

    assert tile(R=24) == 2                      # rows a multiple of 16
    assert tile(K=48) == 2                      # k a multiple of 32
    assert tile(E=0) == 2
    assert tile(R=1 << 20, K=1 << 14) == 2      # one expert's tiled matrix beyond 2 GiB
    assert tile(w=0) == 1
    assert tile(st=0) == 1
    assert tile(w=fake + 8) == 2                # 16-byte alignment
    assert tile(wt=fake + (1 << 24) + 4) == 2
    assert B.tiled_shapes(3, 48, 96) == ((3, 3, 1, 1024), (3, 3, 1, 64))
    assert B.tiled_shapes(1, 6144, 3584) == ((1, 384, 28, 1024), (1, 384, 28, 64))


def test_measure_mfma_peak_argument_errors_before_any_device_work():
    lib = B.load()
    out = ctypes.c_double(-1.0)
    assert lib.situ_moe_measure_mfma_peak(0, ctypes.byref(out)) == 2          # iters >= 1
    assert lib.situ_moe_measure_mfma_peak((1 << 20) + 1, ctypes.byref(out)) == 2
    assert lib.situ_moe_measure_mfma_peak(100, None) == 1
    assert out.value == -1.0

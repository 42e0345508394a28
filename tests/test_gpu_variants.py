"""GPU parity of the layer's variants through the C ABI: the SwiGLU and
SwigluBias activations, NVFP4 weights with the FC2 output scale alpha_down,
the LoRA bridges, the EP16 shard and uneven EP partitions, a TP-shard sum,
SiTU at the Kimi-K3 constants, weight and activation scales far from 1, and
the hidden size that is not a multiple of 1024 run in a child process under a
time limit.  Every layer comparison is gpu_helpers.layer_check: h valid
element by element, the output within the bar against the oracle's FC2 and
combine of the GPU's h (and against the plain oracle where noted).
"""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import block_scaled_mxfp4_amd as B
import synthetic as S
from oracle import formats as F
from oracle import moe as M

from gpu_helpers import check_h, config_inputs, gpu_h, layer_check, oracle_out, parity, run_layer

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SHAPES = {
    # 16-row decode kernels: several m-tiles per expert, K = 640 and 512
    "decode": dict(T=200, H=640, I=512, E_g=8, E_l=8, off=0, k=4, seed=71, skew=True),
    # LDS-tiled prefill kernels (sizes multiples of 128), ragged m-tiles
    "prefill": dict(T=700, H=640, I=384, E_g=6, E_l=4, off=1, k=3, seed=72, skew=True),
    # K tails: H = 96 (a partial K step), I = 96
    "ragged": dict(T=37, H=96, I=96, E_g=13, E_l=5, off=4, k=3, seed=73),
}
# (mode, tactic) pairs: the three m-tile sizes of w4a8 and two of w4a16
TACTICS = [("w4a16", (0, 16)), ("w4a16", (1, 17)), ("w4a8", (2, 18)), ("w4a8", (3, 19)), ("w4a8", (4, 20))]


def _cases(names):
    out = []
    for n in names:
        for mode, tac in TACTICS:
            c = SHAPES[n]
            if tac == (4, 20) and (c["H"] % 128 or c["I"] % 128):
                continue
            out.append((n, mode, tac))
    return out


@pytest.mark.parametrize("activation", ["swiglu", "swiglu_bias"])
@pytest.mark.parametrize("name,mode,tactic", _cases(["decode", "prefill", "ragged"]))
def test_activation_variants(activation, name, mode, tactic):
    spec = S.spec_of(dict(SHAPES[name], activation=activation))
    inp = S.generate(spec)
    got, plan, ws, _ = run_layer(inp, spec, mode=mode, tactic=tactic)
    layer_check(got, inp, spec, mode, plan, ws, what=f"{activation} {name} {mode} {tactic}")


@pytest.mark.parametrize("name,mode,tactic", _cases(["decode", "prefill", "ragged"]))
def test_lora_bridges(name, mode, tactic):
    """A gate_up LoRA delta added before the activation, and the down-LoRA
    input rows (h by expanded index, zero rows outside the shard)."""
    spec = S.spec_of(dict(SHAPES[name], lora=True))
    inp = S.generate(spec)
    got, plan, ws, d = run_layer(inp, spec, mode=mode, tactic=tactic, lora_out=True)
    ref = layer_check(got, inp, spec, mode, plan, ws, what=f"lora {name} {mode} {tactic}")
    T, k, I = spec["T"], spec["k"], spec["I"]
    rows = d["activation_lora_input"].view(torch.int16).cpu().numpy().view(np.uint16)
    P = int(ref["offsets"][-1])
    h = gpu_h(plan, ws, P, I, mode)["vals"]
    perm, inv = ref["perm"], ref["inv"]
    np.testing.assert_array_equal(F.bf16_to_f64(rows[perm]), h)          # local rows: the GPU's own h
    assert np.all(rows[inv < 0] == 0)                                    # pairs outside the shard: +0
    # the same call without bridges equals a zero delta bit for bit
    zero = dict(inp, gate_up_lora_delta=np.zeros_like(inp["gate_up_lora_delta"]))
    a, *_ = run_layer(zero, spec, mode=mode, tactic=tactic)
    b, *_ = run_layer(dict(inp, gate_up_lora_delta=None), spec, mode=mode, tactic=tactic)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("name,shard,mode,tactic,tiled", [("decode", dict(E_l=6, off=1), "w4a16", (0, 16), False),
                                                          ("prefill", {}, "w4a8", (4, 20), True)])
def test_graph_replay_with_lora_bridges(name, shard, mode, tactic, tiled):
    """The step with the LoRA bridges and SwigluBias captured into a HIP
    graph (the zeroing of the down-LoRA rows outside the shard is a kernel,
    not a memset node): every replay, with eager work between replays, gives
    the eager output and down-LoRA rows bit for bit, the rows outside the
    shard rewritten as +0."""
    spec = S.spec_of(dict(SHAPES[name], **shard, activation="swiglu_bias", lora=True))
    inp = S.generate(spec)
    eager, plan, ws, d = run_layer(inp, spec, mode=mode, tactic=tactic, lora_out=True, tiled=tiled)
    eager_rows = d["activation_lora_input"].clone()
    prob = B.make_problem(num_tokens=spec["T"], hidden_size=spec["H"], intermediate_size=spec["I"],
                          num_experts=spec["E_g"], local_expert_offset=spec["off"],
                          local_num_experts=spec["E_l"], top_k=spec["k"], act_mode=mode,
                          topk_packed=inp.get("topk_packed") is not None, out_dtype="f32", tactic=tactic,
                          activation="swiglu_bias", weight_format="mxfp4_tiled" if tiled else "mxfp4")
    ts = B.make_tensors(prob, **d)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        B.situ_moe_run(plan, ts, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.situ_moe_run(plan, ts, ws)
    inv = M.route(inp["topk_ids"], spec["off"], spec["E_l"])[3]
    assert np.any(inv < 0) and np.any(inv >= 0)
    for rep in range(3):
        d["out"].fill_(float("nan"))
        d["activation_lora_input"].fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda") * 3.0     # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = d["out"].float().cpu().numpy()
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"replay {rep}"
        assert torch.equal(d["activation_lora_input"].view(torch.int16), eager_rows.view(torch.int16)), f"rows {rep}"
        del junk


@pytest.mark.parametrize("cfg,overrides", [(1, {"weight_format": "nvfp4"}), (2, {"weight_format": "nvfp4"}),
                                           (2, {"activation": "swiglu_bias"})])
def test_decode_variants_full_size(cfg, overrides):
    """NVFP4 weights on the TP8 and EP8 decode shards and SwigluBias on the
    EP8 decode shard at full size, in the planner's tactics (the 16-row
    decode kernels with K split): every token's h valid element by element
    and the output within the whole bar, against the oracle's FC2 and combine
    of the GPU's h and against the plain oracle."""
    spec = S.spec_of(dict(S.spec_of(cfg), **overrides))
    inp = S.generate(spec)
    got, plan, ws, _ = run_layer(inp, spec)
    layer_check(got, inp, spec, spec["mode"], plan, ws, raw_required=True,
                what=f"{spec['name']} {overrides} all {spec['T']} tokens")


def test_lora_bridges_full_size_ep8_prefill():
    """The LoRA bridges on the EP8 prefill shard at full size (32768 tokens,
    T*k = 524288 pairs: the bf16 delta is 6.4 GB and the down-LoRA input 3.2
    GB, so the rows of the last pairs lie beyond 2^31 and 2^32 bytes), in the
    launch the benchmark times.  The delta is zero except for eight tokens,
    four of them the last ones with a local slot; the oracle runs on those
    eight tokens alone (the layer is independent per token), and the GPU's h
    rows of their pairs, taken from the full batch's permuted order, must be
    valid element by element and give the output within the bar through the
    oracle's FC2 and combine.  Their down-LoRA rows equal h, the rows of
    their pairs outside the shard and the last rows of the buffer are +0."""
    inp = config_inputs(4)
    spec = inp["spec"]
    T, k, I, mode = spec["T"], spec["k"], spec["I"], spec["mode"]
    counts, offsets, perm, inv = M.route(inp["topk_ids"], spec["off"], spec["E_l"])
    has_local = np.nonzero((inv.reshape(T, k) >= 0).any(axis=1))[0]
    rng = np.random.default_rng(404)
    tok = np.unique(np.concatenate([has_local[-4:], rng.choice(has_local[:-4], 4, replace=False)]))
    n = tok.size
    rows = S.bf16_truncate(rng.standard_normal((n * k, 2 * I)).astype(np.float32) * 0.5)
    j_rows = (tok[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    assert int(j_rows.max()) * 2 * I * 2 > 2 ** 32
    delta = torch.zeros((T * k, 2 * I), dtype=torch.bfloat16, device="cuda")
    delta[torch.from_numpy(j_rows).cuda()] = torch.from_numpy(rows.view(np.int16)).cuda().view(torch.bfloat16)
    got, plan, ws, d = run_layer(dict(inp, gate_up_lora_delta=delta), spec, mode=mode, lora_out=True)
    del delta
    P = int(offsets[-1])
    hg = gpu_h(plan, ws, P, I, mode)

    # the eight tokens as a batch of their own
    sub = dict(inp, gate_up_lora_delta=rows)
    for key in ("hidden_states", "topk_ids", "topk_weights", "topk_packed"):
        if inp.get(key) is not None:
            sub[key] = np.ascontiguousarray(inp[key][tok])
    spec_sub = dict(spec, T=n)
    ref = oracle_out(sub, spec_sub, mode=mode, keep=True)
    # the sub-batch's pair p' is the full batch's pair inv[tok*k + s]
    full_of = np.full(int(ref["offsets"][-1]), -1, np.int64)
    sub_inv = ref["inv"].reshape(n, k)
    loc = sub_inv >= 0
    full_of[sub_inv[loc]] = inv.reshape(T, k)[tok][loc]
    assert np.all(full_of >= 0)
    hg_sub = {key: v[full_of] for key, v in hg.items()}
    check_h(hg_sub, sub, spec_sub, ref, mode, "EP8 prefill LoRA, 8 tokens")
    cond = oracle_out(sub, spec_sub, mode=mode, h_given=hg_sub["vals"])
    parity(got[tok], cond["out"], "EP8 prefill LoRA, 8 tokens vs oracle FC2 + combine of the GPU's h")

    # down-LoRA rows: h of the local pairs, +0 elsewhere (the sampled tokens'
    # pairs and the buffer's last 4096 rows)
    lo = d["activation_lora_input"]
    check_j = np.unique(np.concatenate([j_rows, np.arange(T * k - 4096, T * k)]))
    got_rows = lo[torch.from_numpy(check_j).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    p_of = inv[check_j]
    np.testing.assert_array_equal(F.bf16_to_f64(got_rows[p_of >= 0]), hg["vals"][p_of[p_of >= 0]])
    assert np.all(got_rows[p_of < 0] == 0)
    print(f"EP8 prefill LoRA: {n} tokens, {int(loc.sum())} local pairs, {int((p_of >= 0).sum())} local and "
          f"{int((p_of < 0).sum())} other down-LoRA rows checked", flush=True)


@pytest.mark.parametrize("activation", ["situ", "swiglu_bias"])
@pytest.mark.parametrize("name,tactic", [("decode", (0, 16)), ("decode", (1, 17)), ("prefill", (0, 16)),
                                         ("prefill", (1, 17)), ("ragged", (0, 16)), ("ragged", (1, 17))])
def test_nvfp4_weights(activation, name, tactic):
    spec = S.spec_of(dict(SHAPES[name], weight_format="nvfp4", activation=activation))
    inp = S.generate(spec)
    assert inp["alpha_down"] is not None
    got, plan, ws, _ = run_layer(inp, spec, mode="w4a16", tactic=tactic)
    layer_check(got, inp, spec, "w4a16", plan, ws, what=f"nvfp4 {activation} {name} {tactic}")


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_alpha_down_mxfp4(mode):
    spec = S.spec_of(SHAPES["prefill"])
    inp = S.generate(spec)
    rng = np.random.default_rng(5)
    inp = dict(inp, alpha_down=rng.uniform(0.5, 2.0, spec["E_l"]).astype(np.float32))
    got, plan, ws, _ = run_layer(inp, spec, mode=mode)
    layer_check(got, inp, spec, mode, plan, ws, what=f"alpha_down {mode}")


def test_k3_constants():
    """SiTU at Kimi-K3's beta = 4 and linear beta = 25 (the MegaMoE commit
    message, "SiTU in the kernel"), both modes, default tactics."""
    spec = S.spec_of(SHAPES["prefill"])
    inp = S.generate(spec)
    inp = dict(inp, situ_beta=np.full(spec["E_l"], 4.0, np.float32),
               situ_linear_beta=np.full(spec["E_l"], 25.0, np.float32))
    for mode in ("w4a16", "w4a8"):
        got, plan, ws, _ = run_layer(inp, spec, mode=mode)
        layer_check(got, inp, spec, mode, plan, ws, what=f"K3 constants {mode}")


# EP16: 56 local experts of 896 at the full hidden and intermediate sizes
# (the pull request's DEP16 deployment), decode and prefill batch shapes.
EP16 = dict(H=3584, I=3072, E_g=896, E_l=56, off=5 * 56, k=16, skew=True)


@pytest.mark.parametrize("T,mode", [(128, "w4a16"), (2048, "w4a8")])
def test_ep16_shard(T, mode):
    spec = S.spec_of(dict(EP16, T=T, mode=mode, seed=80 + T))
    inp = S.generate(spec)
    got, plan, ws, _ = run_layer(inp, spec, mode=mode)
    counts = M.route(inp["topk_ids"], spec["off"], spec["E_l"])[0]
    print(f"EP16 T={T}: {int(counts.sum())} local pairs, {int((counts > 0).sum())} active experts, "
          f"tactic {B.situ_moe_tactic_name(plan.fc1_tactic)}", flush=True)
    layer_check(got, inp, spec, mode, plan, ws, raw_required=True if mode == "w4a16" else "cosine",
                what=f"EP16 T={T} {mode}")


def _ep_partition(E, ranks):
    """Contiguous expert ranges of an uneven EP split: the first E % ranks
    ranks hold one expert more (the expert partition of the pull request's
    _compute_ep_partition commit)."""
    base, extra = divmod(E, ranks)
    sizes = [base + (1 if r < extra else 0) for r in range(ranks)]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    return list(zip(offs.tolist(), sizes))


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_uneven_ep_partition_sums_to_unsharded(mode):
    full = S.spec_of(dict(T=60, H=256, I=128, E_g=13, E_l=13, off=0, k=4, seed=81, skew=True))
    inp = S.generate(full)
    ref, *_ = run_layer(inp, full, mode=mode)
    total = np.zeros_like(ref, dtype=np.float64)
    part = _ep_partition(13, 3)
    assert part == [(0, 5), (5, 4), (9, 4)]
    for off, n in part:
        shard = dict(inp)
        for key in ("w1", "w1_scale", "w2", "w2_scale", "situ_beta", "situ_linear_beta", "alpha_gate", "alpha_up"):
            shard[key] = inp[key][off:off + n]
        spec = dict(full, off=off, E_l=n)
        out, plan, ws, _ = run_layer(shard, spec, mode=mode)
        layer_check(out, shard, spec, mode, plan, ws, what=f"EP shard [{off}, {off + n}) {mode}")
        total += out
    parity(total, ref, f"sum of 3 uneven EP shards vs unsharded {mode}")


_EP6 = dict(H=3584, I=3072, E_g=896, E_l=149, off=150 + 150 + 149 + 149, k=16, skew=True)


@pytest.mark.parametrize("cfg", [
    dict(S.spec_of(4), activation="swiglu_bias"),
    dict(EP16, name="ep16_prefill", T=32768, mode="w4a8", packed=True, seed=162),
    dict(_EP6, name="uneven_ep6_prefill", T=32768, mode="w4a8", packed=True, seed=164)])
def test_prefill_variants_full_size(cfg):
    """SwigluBias on the EP8 prefill shard, the EP16 shard (56 of 896 experts)
    and an uneven EP shard (149 experts, rank 4 of 896 over 6) at 32768
    tokens, in the planner's tactics (the 128-row kernels): 12 tokens, the
    last 6 with a local slot among them, their h valid element by element and
    the output within the bar against the oracle's FC2 and combine of the
    GPU's h, and the cosine against the plain oracle."""
    spec = S.spec_of(cfg)
    inp = S.generate(spec)
    got, plan, ws, _ = run_layer(inp, spec)
    T, k = spec["T"], spec["k"]
    inv = M.route(inp["topk_ids"], spec["off"], spec["E_l"])[3]
    has_local = np.nonzero((inv.reshape(T, k) >= 0).any(axis=1))[0]
    rng = np.random.default_rng(spec["seed"])
    tok = np.unique(np.concatenate([has_local[-6:], rng.choice(T, 6, replace=False)]))
    assert B.situ_moe_tactic_name(plan.fc1_tactic).endswith("m128")
    layer_check(got[tok], inp, spec, spec["mode"], plan, ws, tokens=tok, raw_required="cosine",
                what=f"{spec['name']} {spec['activation']} {tok.size} of {T} tokens")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_tp_shards_sum_to_unsharded(mode):
    """TP: every shard holds all experts with a slice of the intermediate
    size (gate and up rows sliced together, FC2's K columns matching)."""
    full = S.spec_of(dict(T=48, H=256, I=256, E_g=6, E_l=6, off=0, k=2, seed=82))
    inp = S.generate(full)
    ref, *_ = run_layer(inp, full, mode=mode)
    I, tp = full["I"], 4
    sl = I // tp
    total = np.zeros_like(ref, dtype=np.float64)
    for r in range(tp):
        rows = np.r_[r * sl:(r + 1) * sl, I + r * sl:I + (r + 1) * sl]
        shard = dict(inp, w1=inp["w1"][:, rows], w1_scale=inp["w1_scale"][:, rows],
                     w2=inp["w2"][:, :, r * sl // 2:(r + 1) * sl // 2],
                     w2_scale=inp["w2_scale"][:, :, r * sl // 32:(r + 1) * sl // 32])
        spec = dict(full, I=sl)
        out, plan, ws, _ = run_layer(shard, spec, mode=mode)
        layer_check(out, shard, spec, mode, plan, ws, what=f"TP shard {r} {mode}")
        total += out
    parity(total, ref, f"sum of {tp} TP shards vs unsharded {mode}")


def _extreme_inputs(seed):
    """Weight scale codes spread over [100, 140] with blocks at 1, 2, 253 and
    254, token rows scaled by 2^+20 or 2^-20, SiTU at beta 4 / linear beta 25.
    Kept finite: a block at code 253 (254) holds E2M1 magnitudes up to 3
    (1.5), the largest that stay below the fp32 maximum; expert 0, whose FC1
    has the 253/254 blocks, is routed only tokens at 2^-20; W2 blocks at
    253/254 sit where h is exactly zero (expert 3's gate rows of its first 32
    columns are zero, and SiTU(0, u) = 0)."""
    spec = S.spec_of(dict(T=64, H=256, I=128, E_g=6, E_l=6, off=0, k=2, seed=seed))
    inp = S.generate(spec)
    rng = np.random.default_rng(seed)
    T, H, I, E = spec["T"], spec["H"], spec["I"], spec["E_l"]
    w1s = rng.integers(100, 141, size=inp["w1_scale"].shape).astype(np.uint8)
    w2s = rng.integers(100, 141, size=inp["w2_scale"].shape).astype(np.uint8)
    w1, w2 = inp["w1"].copy(), inp["w2"].copy()
    # tiny scales anywhere
    for arr in (w1s, w2s):
        m = rng.random(arr.shape) < 0.05
        arr[m] = rng.choice([1, 2], size=int(m.sum()))
    # expert 0: FC1 blocks at 253 / 254 with magnitudes capped
    def cap(packed, maxcode):
        lo, hi = packed & 15, packed >> 4
        lo = np.where((lo & 7) > maxcode, (lo & 8) | maxcode, lo)
        hi = np.where((hi & 7) > maxcode, (hi & 8) | maxcode, hi)
        return (lo | (hi << 4)).astype(np.uint8)
    big = rng.random(w1s[0].shape) < 0.1
    code = rng.choice([253, 254], size=w1s[0].shape)
    w1s[0] = np.where(big, code, w1s[0])
    for r_, b_ in zip(*np.nonzero(big)):
        w1[0, r_, 16 * b_:16 * b_ + 16] = cap(w1[0, r_, 16 * b_:16 * b_ + 16], 5 if code[r_, b_] == 253 else 3)
    # expert 3: zero gate rows for columns [0, 32) -> h[:, :32] == 0; W2 K block 0 at 253/254
    w1[3, 0:32] = 0
    w2s[3, :, 0] = rng.choice([253, 254], size=H)
    for n_ in range(H):
        w2[3, n_, 0:16] = cap(w2[3, n_, 0:16], 5 if w2s[3, n_, 0] == 253 else 3)
    x = F.bf16_to_f64(inp["hidden_states"])
    up = rng.random(T) < 0.5
    x = x * np.where(up, 2.0 ** 20, 2.0 ** -20)[:, None]
    ids = inp["topk_ids"].copy()
    # tokens at 2^+20 never route to expert 0
    for t in np.nonzero(up)[0]:
        for s_ in range(2):
            if ids[t, s_] == 0:
                ids[t, s_] = 1 if ids[t, 1 - s_] != 1 else 2
    inp = dict(inp, w1=w1, w1_scale=w1s, w2=w2, w2_scale=w2s, topk_ids=ids.astype(np.int32),
               hidden_states=F.f32_to_bf16_rne(x.astype(np.float32)),
               situ_beta=np.full(E, 4.0, np.float32), situ_linear_beta=np.full(E, 25.0, np.float32))
    return spec, inp


@pytest.mark.parametrize("mode,tactic", [("w4a16", (0, 16)), ("w4a16", (1, 17)), ("w4a8", (2, 18)),
                                         ("w4a8", (3, 19)), ("w4a8", (4, 20))])
def test_extreme_scales(mode, tactic):
    spec, inp = _extreme_inputs(90)
    got, plan, ws, _ = run_layer(inp, spec, mode=mode, tactic=tactic)
    assert np.all(np.isfinite(got))
    layer_check(got, inp, spec, mode, plan, ws, what=f"extreme scales {mode} {tactic}")


CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import synthetic as S
from gpu_helpers import run_layer, layer_check
spec = S.spec_of(dict(T=24, H={H}, I=128, E_g=16, E_l=16, off=0, k=4, seed=91, mode={mode!r}))
inp = S.generate(spec)
got, plan, ws, _ = run_layer(inp, spec, mode={mode!r})
layer_check(got, inp, spec, {mode!r}, plan, ws, what="child H={H} {mode}")
print("CHILD_OK", flush=True)
"""


@pytest.mark.parametrize("H", [3584, 3616])
@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_hidden_not_multiple_of_1024_in_child_process(H, mode):
    """The pages' gate_up GEMM hung the GPU whenever hidden % 1024 != 0; the
    layer runs such sizes (3584 = 3.5 x 1024, and 3616, not a multiple of
    128 either) in a child process that must finish within its time limit."""
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), H=H, mode=mode)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "CHILD_OK" in r.stdout


def test_measured_mfma_peak_is_plausible():
    """The measurement aid returns a rate between a fifth of the published FP8
    peak (5.0 PFLOP/s, the rate E2M1 x E4M3 issues at) and that peak plus 10 %."""
    tf = B.situ_moe_measure_mfma_peak(500)
    print(f"block-scaled FP4 x FP8 MFMA: {tf:.0f} TFLOP/s", flush=True)
    assert 1000.0 < tf < 5500.0

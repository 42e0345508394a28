"""Benchmark of the MXFP4 + SiTU routed-MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C] [--decode-config D]
                    [--no-cpu-baseline] [--no-decode]

A step is one call of the whole layer (routing, FC1 + SiTU, FC2, combine)
over one batch of synthetic tokens already resident in HBM.  The headline
workload is the largest single-GPU shard, the EP8 prefill batch (config 4:
32768 tokens, hidden 3584, 112 of 896 experts at offset 336, intermediate
3072, top-16, packed routing, MXFP8 activations, 30 % of the tokens with no
local expert and 8 local experts with none), measured against the FP8 matrix
core peak; the TP8 decode batch (config 1: 64 tokens, 896 local experts,
intermediate 384, w4a16), measured against HBM bandwidth, is reported beside
it under "decode".  --config / --decode-config select other shard shapes.
The w4a8 prefill shards take their activations MXFP8-quantized per token,
as the workload defines them (quantized once by the library before timing);
the step with bf16 input and the library's own quantization is reported
beside it.

value comes from K plain (eager) calls between two synchronizations.  A
second pass times every call on its own (HIP events on the stream) for the
median, p10 and p90; a third records six events per call at the stage
boundaries (situ_moe_run_profiled) for each kernel's average duration on the
stream it runs on.  A fourth pass reads a 512 MiB buffer before every call
(outside the timed events) so that nothing of the previous call is left in
the 256 MiB MALL (median, p10, p90).  The step is also captured into a HIP graph and
replayed; its time and whether its output equals the eager one bit for bit
are reported.  Each roofline also carries the achieved rate against a
measured ceiling: the device's plain copy bandwidth (HBM-bound kernels) or
the sustained rate of the block-scaled FP4 x FP8 MFMA (the w4a8 GEMMs),
both measured at the start of the run.

Prints one JSON line: tokens/s, ms per step, the roofline of the dominant
kernel (algorithmic bytes or flops per launch over its average duration),
per-stage times, and the CPU oracle timed on a bounded sample of the same
workload.

    python bench.py --no-headline --variants all | NAME,NAME,...

times the layer's variants at full size (the fused decode kernel, NVFP4
weights, the LoRA bridges, SwiGLU and SwigluBias, the EP16 shard and an
uneven EP shard; VARIANTS below), each with its dominant kernel's roofline
and the oracle on a small sample of its batch; without --no-headline they
are added to the line under "variants".

    python bench.py --summarize-stats DIR --workload W --command "..."
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR --workload W --stage S --command "..."
    python bench.py --summarize-pmc DIR --workload W --command "..."

turn rocprofv3 CSV output (kernel stats, FETCH_SIZE / WRITE_SIZE passes, or
any counter pass) into the text summaries kept under profiles/.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
# Sources whose change invalidates stored HBM-traffic counters of the GEMM kernels.
GEMM_SOURCES = ("block_scaled_mxfp4_amd/csrc/gemm.hip", "block_scaled_mxfp4_amd/csrc/prefill.hip",
                "block_scaled_mxfp4_amd/csrc/dma.hpp",
                "block_scaled_mxfp4_amd/csrc/common.hpp", "block_scaled_mxfp4_amd/csrc/internal.hpp",
                "block_scaled_mxfp4_amd/csrc/epilogue.hpp", "block_scaled_mxfp4_amd/build.py")
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 10100.0}
STAGES = ("route", "quantize", "fc1", "fc2", "combine")


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_work(spec, counts, tokens_used, y_format=0, lora=False):
    """Bytes and flops the layer must move / compute, per stage: every active
    expert's packed E2M1 weights with their scales (E8M0 per 32, or E4M3 per
    16 for NVFP4), each used token's input row as the kernel reads it, h and
    y once each, and 2 flops per multiply-add of the two contractions.
    y_format 1: y is fp16 with one exponent byte per 64 columns.  lora: FC1
    also reads each local pair's bf16 gate_up delta row and writes the bf16
    down-LoRA input, every one of its T*k rows (zeros outside the shard)."""
    T, H, I, k = spec["T"], spec["H"], spec["I"], spec["k"]
    counts = np.asarray(counts, np.int64)
    A = int(np.count_nonzero(counts))
    P = int(counts.sum())
    w4a8 = spec["mode"] == "w4a8"
    blk = 16 if spec.get("weight_format") == "nvfp4" else 32   # K elements per weight scale byte
    fc1_w = 2 * I * (H // 2 + H // blk)             # packed E2M1 + scales per expert
    fc2_w = H * (I // 2 + I // blk)
    x_row = H + H // 32 if w4a8 else 2 * H          # the FC1 input row as the kernel reads it
    h_row = I + I // 32 if w4a8 else 2 * I
    lora_bytes = P * 2 * I * 2 + T * k * I * 2 if lora else 0
    work = {
        "A": A, "P": P,
        "fc1_bytes": A * fc1_w + tokens_used * x_row + P * h_row + lora_bytes,
        "fc2_bytes": A * fc2_w + P * h_row + (P * (2 * H + (H + 63) // 64) if y_format else P * H * 4),
        "fc1_flops": 2.0 * P * H * 2 * I,
        "fc2_flops": 2.0 * P * I * H,
        # the layer's own inputs and output: weights of the active experts, the
        # activations as the workload gives them (w4a8: MXFP8 per token), routing, fp32 out
        "layer_bytes": A * (fc1_w + fc2_w) + T * x_row + T * k * 6 + T * H * 4,
        "quantize_bytes": T * 2 * H + T * (H + H // 32) if w4a8 else 0,
    }
    # the fused decode kernel: both GEMMs in one launch, h never leaves LDS
    work["fused_bytes"] = work["fc1_bytes"] + work["fc2_bytes"] - 2 * P * h_row
    work["fused_flops"] = work["fc1_flops"] + work["fc2_flops"]
    return work


def gemm_sources_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, stage):
    """HBM bytes per launch of one stage's kernel from the committed counter
    summary (profiles/<workload>_<stage>_traffic.txt: rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes, each scaled by the same counter's reading for a copy of
    known size).  None when there is no summary or the GEMM sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_{stage}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("{"):
                rec = json.loads(line)
    if not rec or rec.get("sources_digest") != gemm_sources_digest():
        return None
    return int(rec["hbm_bytes_per_launch"])


def copy_probe(mib, reps):
    """A plain device copy of known size (mib MiB read + mib MiB written per
    launch), run so that a counter pass over this process can calibrate
    FETCH_SIZE / WRITE_SIZE against known bytes."""
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    _log(f"copy probe: {reps} x {mib} MiB device-to-device")


def reference_rates(dev):
    """Measured ceilings beside the published ones: the device's plain copy
    bandwidth (1 GiB device-to-device, read + written bytes, best of five)
    and the sustained rate of the block-scaled FP4 x FP8 MFMA (the library's
    measurement aid, best of three)."""
    import torch
    import block_scaled_mxfp4_amd as B
    n = 2**30 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = 0.0
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = max(best, 2 * 2**30 / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    peak = max(B.situ_moe_measure_mfma_peak(2000) for _ in range(3))
    return {"copy_gbs": round(best, 1), "mfma_scale_fp4_fp8_tflops": round(peak, 1)}


def with_measured(roof, refs):
    """A roofline dict with its achieved rate also set against the measured
    ceiling of its kind (copy bandwidth for HBM-bound kernels, the sustained
    block-scaled MFMA rate for the w4a8 matrix-core-bound ones)."""
    if refs is None or roof.get("achieved") is None:
        return roof
    if roof["bound"] == "hbm":
        ref, what = refs["copy_gbs"], "device-to-device copy, GB/s"
    elif roof["bound"] == "mfma" and roof["peak"] == MFMA_PEAK_TFLOPS["mxfp8"]:
        ref, what = refs["mfma_scale_fp4_fp8_tflops"], "v_mfma_scale_f32_16x16x128_f8f6f4 E2M1 x E4M3, TFLOP/s"
    else:
        return roof
    return dict(roof, measured_peak=ref, measured_peak_kind=what, frac_of_measured_peak=round(roof["achieved"] / ref, 4))


def _first_tokens(inp, n):
    """The same batch cut to its first n tokens (the layer is independent per
    token: each kept token's output row is unchanged)."""
    sub = dict(inp)
    for key in ("hidden_states", "topk_ids", "topk_weights", "topk_packed"):
        if sub.get(key) is not None:
            sub[key] = np.ascontiguousarray(sub[key][:n])
    return sub


def cpu_baseline(inp, spec, budget_s=30.0, lora=False):
    """The oracle (float32 mode, as it stands) on a bounded sample: the first n
    tokens of the same batch, n chosen for about budget_s seconds of CPU work
    (w4a8: including the oracle's own MXFP8 quantization of those tokens).
    lora: the sample's pairs get gate_up delta rows ~ N(0, 0.05) of their own
    (the device draws the full batch's rows)."""
    from oracle import moe as M
    try:
        from threadpoolctl import threadpool_info
        blas = [d.get("num_threads") for d in threadpool_info() if d.get("user_api") == "blas"]
        threads = int(blas[0]) if blas else os.cpu_count()
    except Exception:
        threads = os.cpu_count()
    cores = len(os.sched_getaffinity(0))
    T = spec["T"]

    def run(n):
        sub = _first_tokens(inp, n)
        if lora:
            rng = np.random.default_rng(spec["seed"])
            d = (rng.standard_normal((n * spec["k"], 2 * spec["I"])) * 0.05).astype(np.float32)
            sub["gate_up_lora_delta"] = (d.view(np.uint32) >> 16).astype(np.uint16)
        t0 = time.perf_counter()
        M.moe_forward(sub, local_expert_offset=spec["off"], local_num_experts=spec["E_l"],
                      act_mode=spec["mode"], precision="f32", activation=spec["activation"],
                      weight_format=spec["weight_format"])
        return time.perf_counter() - t0

    n = min(T, 4)
    dt = run(n)
    if dt < budget_s / 3 and n < T:
        n = int(min(T, max(n + 1, n * budget_s / max(dt, 1e-3) * 0.6)))
        dt = run(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": f"first {n} of {T} tokens of the same batch, float32 numpy/OpenBLAS oracle, "
                      f"{dt:.1f} s wall, {threads} BLAS threads on {cores} host cores"}


def _percentiles(ms):
    a = np.asarray(ms, np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.quantile(a, 0.1)), 5),
            "p90": round(float(np.quantile(a, 0.9)), 5)}


def measure(cfg, steps, warmup, dev, want_cpu, mall_flush, tactic=(-1, -1), weights="tiled", rows_beside=True,
            refs=None, overrides=None, lora=False, lean=False, cpu_budget=30.0):
    """Time one workload; returns the result fields of its line.  weights:
    "tiled" hands the layer its MXFP4 weights in the fragment-tiled layout
    (made once by situ_moe_tile_weights before timing; the same values, so
    the same output bit for bit) and times the row-major weights beside it;
    "rows" times the row-major weights only (rows_beside=False: tiled
    only, so that a profiler sees one layout's launches).  overrides: spec
    fields replaced (activation, weight_format; NVFP4 weights stay
    row-major); lora: the layer also takes a bf16 gate_up delta per pair
    (drawn on the device, seeded) and writes the down-LoRA input; lean:
    only the eager, per-call and per-stage passes (no graph replay and no
    bf16-input step)."""
    import torch
    import block_scaled_mxfp4_amd as B
    import synthetic as S

    spec = S.spec_of(cfg)
    if overrides:
        spec = S.spec_of(dict(spec, **overrides))
    _log(f"generating inputs for config {cfg} ({spec['name']})")
    t0 = time.perf_counter()
    inp = S.generate(spec)
    _log(f"generated in {time.perf_counter() - t0:.1f} s")

    def d(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.to(dev)

    packed = inp.get("topk_packed") is not None
    T, H, I, k = spec["T"], spec["H"], spec["I"], spec["k"]
    w4a8 = spec["mode"] == "w4a8"

    nv = spec["weight_format"] == "nvfp4"
    tiled = weights == "tiled" and not nv
    wf = "nvfp4" if nv else ("mxfp4_tiled" if tiled else "mxfp4")

    def problem(prequantized, weight_format=wf):
        return B.make_problem(num_tokens=T, hidden_size=H, intermediate_size=I, num_experts=spec["E_g"],
                              local_expert_offset=spec["off"], local_num_experts=spec["E_l"], top_k=k,
                              act_mode=spec["mode"], act_prequantized=prequantized, topk_packed=packed,
                              out_dtype="f32", tactic=tactic, activation=spec["activation"],
                              weight_format=weight_format)

    x_bf16 = d(inp["hidden_states"])
    prob = problem(w4a8)
    plan = B.situ_moe_plan(prob)
    if w4a8:   # the workload's activations arrive MXFP8-quantized per token
        x_codes = torch.empty((T, H), dtype=torch.uint8, device=dev)
        x_scales = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        B.situ_moe_quantize_mxfp8(x_bf16, x_codes, x_scales)
        torch.cuda.synchronize()
    tens = dict(hidden_states=x_codes if w4a8 else x_bf16, w1=d(inp["w1"]), w1_scale=d(inp["w1_scale"]),
                w2=d(inp["w2"]), w2_scale=d(inp["w2_scale"]), situ_beta=d(inp["situ_beta"]),
                situ_linear_beta=d(inp["situ_linear_beta"]), alpha_gate=d(inp["alpha_gate"]),
                alpha_up=d(inp["alpha_up"]), out=torch.empty((T, H), dtype=torch.float32, device=dev))
    if w4a8:
        tens["hidden_states_scale"] = x_scales
    for key in ("swiglu_alpha", "swiglu_beta", "alpha_down"):
        if inp.get(key) is not None:
            tens[key] = d(inp[key])
    if lora:   # a LoRA adapter's FC1 contribution per pair, N(0, 0.05) as bf16
        gen = torch.Generator(device=dev)
        gen.manual_seed(7000 + spec["seed"])
        delta = torch.empty((T * k, 2 * I), dtype=torch.bfloat16, device=dev)
        for r0 in range(0, T * k, 65536):
            r1 = min(T * k, r0 + 65536)
            delta[r0:r1] = (torch.randn((r1 - r0, 2 * I), generator=gen, device=dev) * 0.05).to(torch.bfloat16)
        tens["gate_up_lora_delta"] = delta
        tens["activation_lora_input"] = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
    if packed:
        tens["topk_packed"] = d(inp["topk_packed"])
    else:
        tens["topk_ids"] = d(inp["topk_ids"])
        tens["topk_weights"] = d(inp["topk_weights"])
    row_major = {key: tens[key] for key in ("w1", "w1_scale", "w2", "w2_scale")}
    if tiled:   # the weights' one-time rearrangement, outside every timed region
        tens["w1"], tens["w1_scale"] = B.situ_moe_tile_weights(tens["w1"], tens["w1_scale"])
        tens["w2"], tens["w2_scale"] = B.situ_moe_tile_weights(tens["w2"], tens["w2_scale"])
        torch.cuda.synchronize()
    ts = B.make_tensors(prob, **tens)
    ws = B.new_workspace(plan, dev)
    stream = torch.cuda.current_stream(dev)
    _log(f"plan: fc1={B.situ_moe_tactic_name(plan.fc1_tactic)} fc2={B.situ_moe_tactic_name(plan.fc2_tactic)} "
         f"block_m={plan.block_m} workspace={plan.workspace_bytes / 2**20:.1f} MiB")

    for _ in range(warmup):
        B.situ_moe_run(plan, ts, ws)
    torch.cuda.synchronize()

    # Timed region: K plain calls between two synchronizations -> value.
    K = steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(K):
        B.situ_moe_run(plan, ts, ws)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    eager_ms = start.elapsed_time(end) / K
    eager_out = tens["out"].clone()
    _log(f"config {cfg}: {eager_ms:.4f} ms per step")

    # Every call timed on its own: median / p10 / p90.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a_, b_ in evs:
        a_.record(stream)
        B.situ_moe_run(plan, ts, ws)
        b_.record(stream)
    torch.cuda.synchronize()
    per_call = [a_.elapsed_time(b_) for a_, b_ in evs]

    flushed = None
    if mall_flush:   # a 512 MiB read before every call, outside its events
        # (a read leaves clean lines behind; a write would leave 256 MiB of
        # dirty ones whose write-back then competes with the timed call)
        junk = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        fevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for a_, b_ in fevs:
            torch.sum(junk, dim=0, out=sink)
            a_.record(stream)
            B.situ_moe_run(plan, ts, ws)
            b_.record(stream)
        torch.cuda.synchronize()
        flushed = _percentiles([a_.elapsed_time(b_) for a_, b_ in fevs])
        flushed["note"] = "each call preceded by a 512 MiB device read (the MALL holds 256 MiB)"
        del junk, sink

    # The same step captured once into a HIP graph, replayed K times.
    graph_ms = graph_same = graph_error = None
    try:
        if lean:
            raise RuntimeError("not measured for this workload")
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            B.situ_moe_run(plan, ts, ws)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            B.situ_moe_run(plan, ts, ws)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs.record(stream)
        for _ in range(K):
            graph.replay()
        ge.record(stream)
        torch.cuda.synchronize()
        graph_same = bool(torch.equal(tens["out"].view(torch.int32), eager_out.view(torch.int32)))
        graph_ms = gs.elapsed_time(ge) / K
        del graph
    except Exception as e:   # capture unavailable: reported, the eager number stands regardless
        graph_error = f"{type(e).__name__}: {e}"

    rows_ms = None
    if tiled and rows_beside:   # the same step from the row-major weights
        plan_r = B.situ_moe_plan(problem(w4a8, "mxfp4"))
        assert plan_r.workspace_bytes <= plan.workspace_bytes
        out_r = torch.empty_like(tens["out"])
        ts_r = B.make_tensors(plan_r.prob, **dict(tens, out=out_r, **row_major))
        for _ in range(3):
            B.situ_moe_run(plan_r, ts_r, ws)
        torch.cuda.synchronize()
        rs, re_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        rs.record(stream)
        for _ in range(K):
            B.situ_moe_run(plan_r, ts_r, ws)
        re_.record(stream)
        torch.cuda.synchronize()
        rows_ms = rs.elapsed_time(re_) / K
        rows_same = bool(torch.equal(out_r.view(torch.int32), eager_out.view(torch.int32)))
        del out_r

    bf16_input_ms = None
    if w4a8 and not lean:   # bf16 activations, quantized by the library inside the step
        prob16 = problem(False)
        plan16 = B.situ_moe_plan(prob16)
        t16 = dict(tens, hidden_states=x_bf16)
        t16.pop("hidden_states_scale")
        ts16 = B.make_tensors(prob16, **t16)
        ws16 = B.new_workspace(plan16, dev)
        for _ in range(3):
            B.situ_moe_run(plan16, ts16, ws16)
        torch.cuda.synchronize()
        bs, be = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        bs.record(stream)
        for _ in range(K):
            B.situ_moe_run(plan16, ts16, ws16)
        be.record(stream)
        torch.cuda.synchronize()
        bf16_input_ms = bs.elapsed_time(be) / K
        del ws16

    # Kernel durations: K more calls, each recording six HIP events on the
    # library's stream at the stage boundaries (the events themselves add a
    # few microseconds per call, so they stay out of the value above).
    sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for i in range(K):
        B.situ_moe_run_profiled(plan, ts, ws, sevs[i])
    torch.cuda.synchronize()
    stage_ms = {}
    for j, name in enumerate(STAGES):
        stage_ms[name] = float(np.mean([sevs[i][j].elapsed_time(sevs[i][j + 1]) for i in range(K)]))

    counts = B.workspace_view(plan, ws, "counts", torch.int32, (spec["E_l"],)).cpu().numpy()
    inv = B.workspace_view(plan, ws, "inv", torch.int32, (T * k,)).cpu().numpy().reshape(T, k)
    tokens_used = int(np.count_nonzero((inv >= 0).any(axis=1)))
    work = algorithmic_work(spec, counts, tokens_used, plan.y_format, lora)

    workload = f"{spec['name']}_{spec['mode']}"
    variant = [v for v in (spec["activation"] != "situ" and spec["activation"], nv and "nvfp4", lora and "lora") if v]
    if variant:
        workload += "_" + "_".join(variant)
    peak_tf = MFMA_PEAK_TFLOPS["mxfp8"] if w4a8 else MFMA_PEAK_TFLOPS["bf16"]

    def roofline(stage):
        """The stage's kernel against the roofline that bounds it: the larger
        of its algorithmic bytes / HBM peak and its flops / MFMA peak."""
        t = stage_ms[stage] * 1e-3
        t_hbm = work[f"{stage}_bytes"] / (HBM_PEAK_GBS * 1e9)
        t_mfma = work[f"{stage}_flops"] / (peak_tf * 1e12)
        if t_hbm >= t_mfma:
            achieved = work[f"{stage}_bytes"] / t / 1e9
            return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "kernel": stage,
                    "algorithmic_bytes_per_launch": work[f"{stage}_bytes"], "avg_launch_ms": round(stage_ms[stage], 5)}
        achieved = work[f"{stage}_flops"] / t / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(achieved / peak_tf, 4), "kernel": stage,
                "algorithmic_flops_per_launch": work[f"{stage}_flops"], "avg_launch_ms": round(stage_ms[stage], 5)}

    fused = B.situ_moe_tactic_name(plan.fc1_tactic).startswith("fused")
    if fused:
        # one launch runs both GEMMs: its time sits between the FC1 marks and
        # the FC2 marks are back to back
        stage_ms["fused"] = stage_ms["fc1"] + stage_ms["fc2"]
        roof = roofline("fused")
        roof["traffic"] = None
        other = {"kernel": "none (FC1 and FC2 in one launch)", "bound": None, "achieved": None, "peak": None,
                 "unit": None, "frac": None, "traffic": None}
    else:
        # the dominant kernel: the GEMM that takes longer
        dom = "fc1" if stage_ms["fc1"] >= stage_ms["fc2"] else "fc2"
        roof = roofline(dom)
        roof["traffic"] = stored_traffic(workload, dom)
        other = roofline("fc2" if dom == "fc1" else "fc1")
        other["traffic"] = stored_traffic(workload, other["kernel"])
    layer_gbs = work["layer_bytes"] / (eager_ms * 1e-3) / 1e9
    layer_tf = (work["fc1_flops"] + work["fc2_flops"]) / (eager_ms * 1e-3) / 1e12

    res = {
        "value": round(T / (eager_ms * 1e-3), 1),
        "ms_per_step": round(eager_ms, 5),
        "step_ms": _percentiles(per_call),
        "dtype": "mxfp8" if w4a8 else "bf16",
        "config": {"workload": workload, "tokens": T, "hidden": H, "intermediate": I,
                   "experts_global": spec["E_g"], "experts_local": spec["E_l"],
                   "local_expert_offset": spec["off"], "top_k": k,
                   "topk_format": "packed" if packed else "ids+weights",
                   "active_local_experts": work["A"], "local_pairs": work["P"],
                   "fc1_tactic": B.situ_moe_tactic_name(plan.fc1_tactic),
                   "fc2_tactic": B.situ_moe_tactic_name(plan.fc2_tactic),
                   "activation": spec["activation"], "lora_bridges": bool(lora),
                   "weights": "NVFP4 (E4M3 scale per 16), row-major" if nv else
                              "MXFP4, fragment-tiled once by situ_moe_tile_weights before timing" if tiled
                              else "MXFP4, row-major"},
        "roofline": with_measured(roof, refs),
        "roofline_other_gemm": with_measured({kk: other[kk] for kk in ("kernel", "bound", "achieved", "peak", "unit",
                                                                       "frac", "traffic")}, refs),
        "stage_ms": {kk: round(v, 5) for kk, v in stage_ms.items()},
        "layer_hbm_gbs": round(layer_gbs, 1),
        "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
        "layer_tflops": round(layer_tf, 1),
        "layer_mfma_frac": round(layer_tf / peak_tf, 4),
        "wall_s_timed_region": round(wall, 4),
        "graph_replay": {"ms_per_step": round(graph_ms, 5) if graph_ms is not None else None,
                         "bitwise_equal_to_eager": graph_same, "error": graph_error},
        "activations": "MXFP8 per token (prequantized)" if w4a8 else "bf16",
    }
    if flushed is not None:
        res["step_ms_mall_flushed"] = flushed
    if rows_ms is not None:
        res["row_major_weights"] = {"ms_per_step": round(rows_ms, 5), "tokens_per_s": round(T / (rows_ms * 1e-3), 1),
                                    "bitwise_equal_to_tiled": rows_same,
                                    "note": "the same step from the row-major MXFP4 weights"}
    if bf16_input_ms is not None:
        res["bf16_input"] = {"ms_per_step": round(bf16_input_ms, 5),
                             "tokens_per_s": round(T / (bf16_input_ms * 1e-3), 1),
                             "note": "the same step with bf16 activations quantized by the library (eager)"}
    if want_cpu:
        _log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(inp, spec, cpu_budget, lora)
    del ws
    torch.cuda.empty_cache()
    return res


# The layer's variants at full size, each timed like the workloads above
# (lean: eager, per-call and per-stage passes), its dominant kernel against
# its roofline and the oracle on a small sample of the same batch beside it:
# the fused decode kernel, NVFP4 weights, the LoRA bridges, the SwiGLU and
# SwigluBias activations, the EP16 shard (56 of 896 experts) and an uneven
# EP shard (896 experts over 6 ranks: 150, 150, 149, 149, 149, 149; rank 4).
# name -> (config id or spec, spec overrides, measure() options)
_EP16 = dict(H=3584, I=3072, E_g=896, E_l=56, off=5 * 56, k=16, skew=True)
_EP6 = dict(H=3584, I=3072, E_g=896, E_l=149, off=150 + 150 + 149 + 149, k=16, skew=True)
VARIANTS = {
    "tp8_decode_fused": (1, {}, dict(tactic=(5, 21))),
    "tp8_decode_nvfp4": (1, {"weight_format": "nvfp4"}, {}),
    "ep8_decode_nvfp4": (2, {"weight_format": "nvfp4"}, {}),
    "tp8_decode_lora": (1, {}, dict(lora=True)),
    "tp8_prefill_lora": (3, {}, dict(lora=True)),
    "ep8_prefill_lora": (4, {}, dict(lora=True)),
    "tp8_decode_swiglu_bias": (1, {"activation": "swiglu_bias"}, {}),
    "ep8_prefill_swiglu": (4, {"activation": "swiglu"}, {}),
    "ep8_prefill_swiglu_bias": (4, {"activation": "swiglu_bias"}, {}),
    "ep16_decode": (dict(_EP16, name="ep16_decode", T=256, mode="w4a16", seed=161), {}, {}),
    "ep16_prefill": (dict(_EP16, name="ep16_prefill", T=32768, mode="w4a8", packed=True, seed=162), {}, {}),
    "uneven_ep6_decode": (dict(_EP6, name="uneven_ep6_decode", T=256, mode="w4a16", seed=163), {}, {}),
    "uneven_ep6_prefill": (dict(_EP6, name="uneven_ep6_prefill", T=32768, mode="w4a8", packed=True, seed=164),
                           {}, {}),
}


def measure_variants(names, steps, warmup, dev, refs, want_cpu):
    out = {}
    for name in names:
        cfg, overrides, opts = VARIANTS[name]
        _log(f"variant {name}")
        r = measure(cfg, steps, warmup, dev, want_cpu, mall_flush=False, rows_beside=False, refs=refs,
                    overrides=overrides, lean=True, cpu_budget=6.0, **opts)
        for key in ("graph_replay", "wall_s_timed_region", "activations"):
            r.pop(key, None)
        out[name] = {"tokens_per_s": r.pop("value"), **r}
    return out


# ---------------------------------------------------------------- rocprofv3 summaries

def _csvs(directory, suffix):
    import glob
    return sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))


def summarize_stats(directory, workload, command):
    """profiles/<workload>_kernel_stats.txt from rocprofv3 --kernel-trace --stats output."""
    import csv
    files = _csvs(directory, "kernel_stats.csv")
    assert files, f"no *kernel_stats.csv under {directory}"
    rows = list(csv.DictReader(open(files[0])))
    lines = [f"# kernel durations, {workload}", f"# command: {command}",
             "# source: rocprofv3 --kernel-trace --stats, kernel_stats.csv (durations in microseconds)",
             f"{'kernel':66s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{r['Name'][:66]:66s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    path = os.path.join(ROOT, "profiles", f"{workload}_kernel_stats.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


def _counter_rows(directory):
    import csv
    files = _csvs(directory, "counter_collection.csv")
    assert files, f"no *counter_collection.csv under {directory}"
    return list(csv.DictReader(open(files[0])))


def _per_kernel(rows, counter):
    """{kernel name: [value per dispatch, in dispatch order]} for one counter."""
    out = {}
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        if r["Counter_Name"] == counter:
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


STAGE_KERNELS = {"fc1": ("decode_gemm_kernel<false, true", "decode_gemm_kernel<true, true", "fc1_kernel",
                         "prefill_wide_kernel<true", "prefill_gemm_kernel<true", "prefill_fc1_512_kernel",
                         "prefill_fc1_384_kernel"),
                 "fc2": ("decode_gemm_kernel<false, false", "decode_gemm_kernel<true, false", "fc2_kernel",
                         "prefill_wide_kernel<false", "prefill_gemm_kernel<false", "prefill_fc2_short_kernel",
                         "prefill_fc2_512_kernel")}


def _stage_kernel(names, stage):
    for n in names:
        if any(p in n for p in STAGE_KERNELS[stage]):
            return n
    raise SystemExit(f"no {stage} kernel among {sorted(names)}")


def summarize_traffic(fetch_dir, write_dir, workload, stage, command):
    """profiles/<workload>_<stage>_traffic.txt: HBM bytes per launch of the
    stage's kernel from a FETCH_SIZE pass and a WRITE_SIZE pass, each scaled
    by the same counter's reading for the last three dispatches of the run (a
    512 MiB device copy, bench.py --copy-probe-mib 512)."""
    f = _per_kernel(_counter_rows(fetch_dir), "FETCH_SIZE")
    w = _per_kernel(_counter_rows(write_dir), "WRITE_SIZE")
    kern = _stage_kernel(f.keys(), stage)
    copy = [n for n in f if "copyBuffer" in n]
    assert copy, "the runs need the copy probe"
    cf = float(np.mean(f[copy[0]][-3:]))
    cw = float(np.mean(w[copy[0]][-3:]))
    ff, wf = 524288.0 / cf, 524288.0 / cw
    fk = float(np.median(f[kern][1:] or f[kern]))     # the first dispatch is the cold warm-up
    wk = float(np.median(w[kern][1:] or w[kern]))
    hbm = int(round((fk * ff + wk * wf) * 1024))
    lines = [f"# HBM traffic of the {stage.upper()} kernel, {workload}", f"# kernel: {kern}",
             "# commands (one counter per run):"] + [f"#   {c}" for c in command.split(" ;; ")] + [
        "# calibration: the runs end with three 512 MiB device-to-device copies (the last three dispatches);",
        f"#   FETCH_SIZE reads {cf:.1f} KiB and WRITE_SIZE {cw:.1f} KiB for 524288 KiB moved,",
        f"#   so fetch is scaled by {ff:.4f} and write by {wf:.4f}.",
        f"# per launch (median over dispatches after the first): fetch {fk:.1f} KiB x {ff:.4f} + write {wk:.1f} KiB"
        f" x {wf:.4f} = {hbm / 1e6:.1f} MB",
        "# sources_digest: sha256 prefix of the GEMM sources the counters were taken on",
        json.dumps({"workload": workload, "stage": stage, "kernel": kern, "fetch_kib_per_dispatch": round(fk, 1),
                    "write_kib_per_dispatch": round(wk, 1), "dispatches": [len(f[kern]), len(w[kern])],
                    "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1), "fetch_factor": round(ff, 4),
                    "write_factor": round(wf, 4), "hbm_bytes_per_launch": hbm,
                    "sources_digest": gemm_sources_digest()})]
    path = os.path.join(ROOT, "profiles", f"{workload}_{stage}_traffic.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


# MI355X: 8 XCDs of 32 CUs, 4 SIMDs a CU; GRBM_GUI_ACTIVE reads once per XCD.
_XCDS, _CUS, _SIMDS = 8, 256, 1024


def _derived(v):
    """Ratios a reader needs from one kernel's counters (those present)."""
    out = []
    gui = v.get("GRBM_GUI_ACTIVE")
    cyc = gui / _XCDS if gui else None              # the kernel's duration in GPU clocks
    if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
        out.append(("MFMA busy, % of SIMD cycles", 100.0 * v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * _SIMDS)))
    if "SQ_LDS_BANK_CONFLICT" in v and v.get("SQ_LDS_IDX_ACTIVE"):
        out.append(("LDS bank-conflict cycles, % of LDS active", 100.0 * v["SQ_LDS_BANK_CONFLICT"] / v["SQ_LDS_IDX_ACTIVE"]))
    if cyc and "TA_TA_BUSY" in v:
        out.append(("TA busy, % of CU cycles", 100.0 * v["TA_TA_BUSY"] / (cyc * _CUS)))
    if cyc and "TA_ADDR_STALLED_BY_TC_CYCLES" in v:
        out.append(("TA address path stalled by the L1, % of CU cycles", 100.0 * v["TA_ADDR_STALLED_BY_TC_CYCLES"] / (cyc * _CUS)))
    if cyc and "TCP_PENDING_STALL_CYCLES" in v:
        out.append(("L1 stalled on data pending from L2, % of CU cycles", 100.0 * v["TCP_PENDING_STALL_CYCLES"] / (cyc * _CUS)))
    if cyc and "SQ_VMEM_TA_CMD_FIFO_FULL" in v:
        out.append(("vector-memory command FIFO full, % of CU cycles", 100.0 * v["SQ_VMEM_TA_CMD_FIFO_FULL"] / (cyc * _CUS)))
    if v.get("TCC_REQ") and "TCC_HIT" in v:
        out.append(("L2 hit rate, %", 100.0 * v["TCC_HIT"] / v["TCC_REQ"]))
    if v.get("TCP_TCC_READ_REQ") and "TCP_TCC_READ_REQ_LATENCY" in v:
        out.append(("L1->L2 read latency, cycles (mean)", v["TCP_TCC_READ_REQ_LATENCY"] / v["TCP_TCC_READ_REQ"]))
        if cyc:
            out.append(("L1->L2 reads in flight per CU (mean)", v["TCP_TCC_READ_REQ_LATENCY"] / (cyc * _CUS)))
    if "SQ_INSTS_MFMA" in v:
        out.append(("16x16x128 MFMAs, TFLOP issued (x 65536 flop)", v["SQ_INSTS_MFMA"] * 65536 / 1e12))
    return out


def summarize_pmc(directories, workload, command, tag):
    """profiles/<workload>_<tag>_counters.txt: the counters of one or more
    rocprofv3 --pmc passes (comma-separated directories), per GEMM kernel
    (median per dispatch over the dispatches after the first), with the
    ratios they give."""
    per = {}
    for directory in directories.split(","):
        rows = _counter_rows(directory)
        for c in sorted({r["Counter_Name"] for r in rows}):
            for kern, vals in _per_kernel(rows, c).items():
                per.setdefault(kern, {})[c] = float(np.median(vals[1:] or vals))
    lines = [f"# hardware counters of the GEMM kernels, {workload}",
             "# commands (one pass each):"] + [f"#   {c}" for c in command.split(" ;; ")] + [
             "# values: median per dispatch over the dispatches after the first (the cold warm-up);",
             "# sums over the chip's instances; GRBM_GUI_ACTIVE once per XCD (8), so duration = it / 8 clocks",
             f"# sources_digest: {gemm_sources_digest()}"]
    for stage in ("fc1", "fc2"):
        try:
            kern = _stage_kernel(per.keys(), stage)
        except SystemExit:
            continue
        v = per[kern]
        lines.append(f"{stage}: {kern}")
        for c in sorted(v):
            lines.append(f"  {c:44s} {v[c]:20.1f}")
        for name, x in _derived(v):
            lines.append(f"  = {name:52s} {x:10.2f}")
    path = os.path.join(ROOT, "profiles", f"{workload}_{tag}_counters.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="headline workload (default: the EP8 prefill shard)")
    ap.add_argument("--decode-config", type=int, default=1, help="workload reported beside it (-1: none)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tactic", default="-1,-1", help="FC1,FC2 tactic ids of the headline workload (-1,-1: the planner's)")
    ap.add_argument("--decode-tactic", default="-1,-1", help="FC1,FC2 tactic ids of the workload beside it")
    ap.add_argument("--weights", choices=("tiled", "rows"), default="tiled",
                    help="MXFP4 weight layout handed to the layer (tiled: the row-major step is timed beside it)")
    ap.add_argument("--no-row-major", action="store_true",
                    help="with tiled weights, skip the row-major step (profiling runs: one layout's launches)")
    ap.add_argument("--variants", default="",
                    help="comma-separated variant workloads measured after the others, or 'all': "
                         + ", ".join(VARIANTS))
    ap.add_argument("--no-headline", action="store_true",
                    help="measure the variants only (profiling runs); the line then carries no value")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy this many MiB device-to-device 3 times (counter calibration)")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--workload")
    ap.add_argument("--stage")
    ap.add_argument("--tag", default="pmc")
    ap.add_argument("--command", default="")
    args = ap.parse_args(argv)
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.workload, args.command)
        return 0
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.workload, args.stage, args.command)
        return 0
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.workload, args.command, args.tag)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this layer computes one TP/EP shard's partial output "
              f"on one MI355X (the cross-GPU all-reduce is the caller's); --gpus {args.gpus} is not run.",
              file=sys.stderr)
        return 2

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tac = tuple(int(v) for v in args.tactic.split(","))
    dtac = tuple(int(v) for v in args.decode_tactic.split(","))
    refs = reference_rates(dev)
    _log(f"measured ceilings: {refs}")
    names = list(VARIANTS) if args.variants == "all" else [v for v in args.variants.split(",") if v]
    for v in names:
        if v not in VARIANTS:
            raise SystemExit(f"unknown variant {v!r}; known: {', '.join(VARIANTS)}")
    if args.no_headline:
        res = {"variants": measure_variants(names, args.steps, args.warmup, dev, refs, not args.no_cpu_baseline),
               "measured_ceilings": refs, "steps": args.steps, "warmup": args.warmup}
        if args.copy_probe_mib > 0:
            copy_probe(args.copy_probe_mib, 3)
        print(json.dumps(res), flush=True)
        return 0
    head = measure(args.config, args.steps, args.warmup, dev, not args.no_cpu_baseline, mall_flush=True, tactic=tac,
                   weights=args.weights, rows_beside=not args.no_row_major, refs=refs)
    res = {
        "metric": "MoE-layer tokens/s at 1 GPU + % of HBM roofline (decode) / MFMA peak (prefill)",
        "value": head.pop("value"),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head.pop("dtype"),
        "data": "synthetic",
        "config": head.pop("config"),
        "roofline": head.pop("roofline"),
    }
    cpu = head.pop("cpu_baseline", None)
    res.update(head)
    res["measured_ceilings"] = refs
    if cpu is not None:
        res["cpu_baseline"] = cpu
    if not args.no_decode and args.decode_config >= 0 and args.decode_config != args.config:
        dec = measure(args.decode_config, max(args.steps, 20), args.warmup, dev, False, mall_flush=True, tactic=dtac,
                      weights=args.weights, rows_beside=not args.no_row_major, refs=refs)
        res["decode"] = {"metric_value_tokens_per_s": dec.pop("value"), **dec}
    if names:
        res["variants"] = measure_variants(names, args.steps, args.warmup, dev, refs, not args.no_cpu_baseline)
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, 3)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

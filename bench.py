"""Benchmark of the MXFP4 + SiTU routed-MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C] [--no-cpu-baseline]

A step is one call of the whole layer (routing, FC1 + SiTU, FC2, combine)
over one batch of synthetic tokens already resident in HBM.  The default
workload is the TP8-shard decode batch the metric is quoted on (config 1:
64 tokens, hidden 3584, 896 local experts, intermediate 384, top-16,
w4a16); --config selects another shard shape.  The w4a8 prefill shards take
their activations MXFP8-quantized per token, as the workload defines them
(quantized once by the library before timing); the step with bf16 input and
the library's own quantization is reported beside it.

value comes from plain (eager) calls.  The step is also captured once into a
HIP graph and replayed (the layer runs no host synchronization and records
no memset node); the replay time and whether its output equals the eager
one bit for bit are reported beside it.

Prints one JSON line: tokens/s, ms per step, the roofline of the dominant
kernel (algorithmic bytes or flops per launch over its average duration
from HIP events on the stream it runs on), per-stage times, and the CPU
oracle timed on a bounded sample of the same workload.
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
                "block_scaled_mxfp4_amd/build.py")
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 10100.0}
STAGES = ("route", "quantize", "fc1", "fc2", "combine")


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_work(spec, counts, tokens_used, y_format=0):
    """Bytes and flops the layer must move / compute, per stage: every active
    expert's packed E2M1 weights with their E8M0 scales, each used token's
    input row as the kernel reads it, h and y once each, and 2 flops per
    multiply-add of the two contractions.  y_format 1: y is fp16 with one
    exponent byte per 64 columns."""
    T, H, I, k = spec["T"], spec["H"], spec["I"], spec["k"]
    counts = np.asarray(counts, np.int64)
    A = int(np.count_nonzero(counts))
    P = int(counts.sum())
    w4a8 = spec["mode"] == "w4a8"
    fc1_w = 2 * I * (H // 2 + H // 32)              # packed E2M1 + E8M0 per expert
    fc2_w = H * (I // 2 + I // 32)
    x_row = H + H // 32 if w4a8 else 2 * H          # the FC1 input row as the kernel reads it
    h_row = I + I // 32 if w4a8 else 2 * I
    work = {
        "A": A, "P": P,
        "fc1_bytes": A * fc1_w + tokens_used * x_row + P * h_row,
        "fc2_bytes": A * fc2_w + P * h_row + (P * (2 * H + (H + 63) // 64) if y_format else P * H * 4),
        "fc1_flops": 2.0 * P * H * 2 * I,
        "fc2_flops": 2.0 * P * I * H,
        # the layer's own inputs and output: weights of the active experts, the
        # activations as the workload gives them (w4a8: MXFP8 per token), routing, fp32 out
        "layer_bytes": A * (fc1_w + fc2_w) + T * x_row + T * k * 6 + T * H * 4,
        "quantize_bytes": T * 2 * H + T * (H + H // 32) if w4a8 else 0,
    }
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


def cpu_baseline(inp, spec, budget_s=15.0):
    """The oracle (float32 mode, as it stands) on a bounded sample of tokens."""
    from oracle import moe as M
    try:
        from threadpoolctl import threadpool_info
        blas = [d.get("num_threads") for d in threadpool_info() if d.get("user_api") == "blas"]
        threads = int(blas[0]) if blas else os.cpu_count()
    except Exception:
        threads = os.cpu_count()
    cores = len(os.sched_getaffinity(0))
    T = spec["T"]
    n = min(T, 4)
    tokens = np.arange(n)
    t0 = time.perf_counter()
    M.moe_forward(inp, local_expert_offset=spec["off"], local_num_experts=spec["E_l"],
                  act_mode=spec["mode"], precision="f32", tokens=tokens)
    dt = time.perf_counter() - t0
    if dt < budget_s / 3 and n < T:
        n = int(min(T, max(n + 1, n * budget_s / max(dt, 1e-3) * 0.6)))
        tokens = np.arange(n)
        t0 = time.perf_counter()
        M.moe_forward(inp, local_expert_offset=spec["off"], local_num_experts=spec["E_l"],
                      act_mode=spec["mode"], precision="f32", tokens=tokens)
        dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": f"first {n} of {T} tokens of the same batch, float32 numpy/OpenBLAS oracle, "
                      f"{dt:.1f} s wall, {threads} BLAS threads on {cores} host cores"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy this many MiB device-to-device 3 times (counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this layer computes one TP/EP shard's partial output "
              f"on one MI355X (the cross-GPU all-reduce is the caller's); --gpus {args.gpus} is not run.",
              file=sys.stderr)
        return 2

    import torch
    import block_scaled_mxfp4_amd as B
    import synthetic as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = S.spec_of(args.config)
    _log(f"generating inputs for config {args.config} ({spec['name']})")
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

    def problem(prequantized):
        return B.make_problem(num_tokens=T, hidden_size=H, intermediate_size=I, num_experts=spec["E_g"],
                              local_expert_offset=spec["off"], local_num_experts=spec["E_l"], top_k=k,
                              act_mode=spec["mode"], act_prequantized=prequantized, topk_packed=packed,
                              out_dtype="f32")

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
    if packed:
        tens["topk_packed"] = d(inp["topk_packed"])
    else:
        tens["topk_ids"] = d(inp["topk_ids"])
        tens["topk_weights"] = d(inp["topk_weights"])
    ts = B.make_tensors(prob, **tens)
    ws = B.new_workspace(plan, dev)
    stream = torch.cuda.current_stream(dev)
    _log(f"plan: fc1={B.situ_moe_tactic_name(plan.fc1_tactic)} fc2={B.situ_moe_tactic_name(plan.fc2_tactic)} "
         f"block_m={plan.block_m} workspace={plan.workspace_bytes / 2**20:.1f} MiB")

    for _ in range(args.warmup):
        B.situ_moe_run(plan, ts, ws)
    torch.cuda.synchronize()

    # Timed region: K plain calls between two synchronizations -> value.
    K = args.steps
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

    # The same step captured once into a HIP graph, replayed K times.
    graph_ms = None
    graph_same = None
    graph_error = None
    try:
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
    ms_per_step = eager_ms

    bf16_input_ms = None
    if w4a8:   # bf16 activations, quantized by the library inside the step
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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for i in range(K):
        B.situ_moe_run_profiled(plan, ts, ws, evs[i])
    torch.cuda.synchronize()
    stage_ms = {}
    for j, name in enumerate(STAGES):
        stage_ms[name] = float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)]))

    counts = B.workspace_view(plan, ws, "counts", torch.int32, (spec["E_l"],)).cpu().numpy()
    inv = B.workspace_view(plan, ws, "inv", torch.int32, (T * k,)).cpu().numpy().reshape(T, k)
    tokens_used = int(np.count_nonzero((inv >= 0).any(axis=1)))
    work = algorithmic_work(spec, counts, tokens_used, plan.y_format)

    dom = "fc1" if stage_ms["fc1"] >= stage_ms["fc2"] else "fc2"
    workload = f"{spec['name']}_{spec['mode']}"
    traffic = stored_traffic(workload, dom)
    def roofline(stage):
        """The stage's kernel against the roofline that bounds it: the larger
        of its algorithmic bytes / HBM peak and its flops / MFMA peak."""
        t = stage_ms[stage] * 1e-3
        peak_tf = MFMA_PEAK_TFLOPS["mxfp8"] if w4a8 else MFMA_PEAK_TFLOPS["bf16"]
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

    roof = roofline(dom)
    roof["traffic"] = traffic
    other = roofline("fc2" if dom == "fc1" else "fc1")
    layer_gbs = work["layer_bytes"] / (ms_per_step * 1e-3) / 1e9

    res = {
        "metric": "MoE-layer tokens/s at 1 GPU + % of HBM roofline (decode) / MFMA peak (prefill)",
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8" if w4a8 else "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "tokens": T, "hidden": H, "intermediate": I,
                   "experts_global": spec["E_g"], "experts_local": spec["E_l"],
                   "local_expert_offset": spec["off"], "top_k": k, "topk_format": "packed" if packed else "ids+weights",
                   "active_local_experts": work["A"], "local_pairs": work["P"],
                   "fc1_tactic": B.situ_moe_tactic_name(plan.fc1_tactic),
                   "fc2_tactic": B.situ_moe_tactic_name(plan.fc2_tactic)},
        "roofline": roof,
        "roofline_other_gemm": {kk: other[kk] for kk in ("kernel", "bound", "achieved", "unit", "frac")},
        "stage_ms": {kk: round(v, 5) for kk, v in stage_ms.items()},
        "layer_hbm_gbs": round(layer_gbs, 1),
        "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
        "wall_s_timed_region": round(wall, 4),
        "graph_replay": {"ms_per_step": round(graph_ms, 5) if graph_ms is not None else None,
                         "bitwise_equal_to_eager": graph_same, "error": graph_error},
        "activations": "MXFP8 per token (prequantized)" if w4a8 else "bf16",
    }
    if bf16_input_ms is not None:
        res["bf16_input"] = {"ms_per_step": round(bf16_input_ms, 5),
                             "tokens_per_s": round(T / (bf16_input_ms * 1e-3), 1),
                             "note": "the same step with bf16 activations quantized by the library (eager)"}
    if not args.no_cpu_baseline:
        _log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(inp, spec)
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, 3)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Python binding of libsitu_moe.so, the MXFP4 + SiTU routed-MoE layer for MI355X.

Argument marshalling only: every step of the layer runs in the library's
HIP kernels (see include/situ_moe.h).  PyTorch provides device memory and
the current stream; nothing here computes on tensor values.

The shared library is loaded on first use, not at import (as the pages'
sidecar does: "Runtime API", importing loads nothing).  If it has not been
built, every entry point raises; there is no CPU fallback.

Names mirror the C entry points: situ_moe_plan, situ_moe_valid_tactics,
situ_moe_run, situ_moe_run_profiled, situ_moe_run_static, situ_moe_route, situ_moe_quantize_mxfp8,
situ_moe_tile_weights, situ_moe_status_string,
situ_moe_last_error, situ_moe_build_info, situ_moe_tactic_name,
situ_moe_abi_version, and the measurement aid situ_moe_measure_mfma_peak.
situ_moe(...) is the keyword-only one-call form.
"""

import ctypes
import os

__all__ = [
    "SituMoeError", "SituMoeProblem", "SituMoePlan", "SituMoeTensors", "library_path", "load",
    "situ_moe_plan", "situ_moe_valid_tactics", "situ_moe_run", "situ_moe_run_profiled", "situ_moe_run_static",
    "situ_moe_route",
    "situ_moe_quantize_mxfp8", "situ_moe_tile_weights", "situ_moe_measure_mfma_peak", "situ_moe_status_string",
    "situ_moe_last_error",
    "situ_moe_build_info", "situ_moe_tactic_name", "situ_moe_abi_version", "situ_moe",
    "make_problem", "make_tensors", "new_workspace", "workspace_view", "ACT_W4A16", "ACT_W4A8", "OUT_F32", "OUT_BF16",
]

ACT_W4A16, ACT_W4A8 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
ACTIVATIONS = {"situ": 0, "swiglu": 1, "swiglu_bias": 2}
WEIGHT_FORMATS = {"mxfp4": 0, "nvfp4": 1, "mxfp4_tiled": 2}
ABI_VERSION = 3
STATUS_NAMES = {0: "SITU_OK", 1: "SITU_E_NULL_ARG", 2: "SITU_E_BAD_SHAPE", 3: "SITU_E_UNSUPPORTED",
                4: "SITU_E_MISSING_SCALE", 5: "SITU_E_DEVICE", 6: "SITU_E_WORKSPACE", 7: "SITU_E_LAUNCH"}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.path.join(_HERE, "lib", "libsitu_moe.so")


class SituMoeError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class SituMoeProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "hidden_size", "intermediate_size", "num_experts", "local_expert_offset",
        "local_num_experts", "top_k", "act_mode", "act_prequantized", "topk_packed", "out_dtype",
        "tactic_fc1", "tactic_fc2", "activation", "weight_format")]


class SituMoePlan(ctypes.Structure):
    _fields_ = [("prob", SituMoeProblem),
                ("fc1_tactic", ctypes.c_int32), ("fc2_tactic", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("max_mtiles", ctypes.c_int32),
                ("route_blocks", ctypes.c_int32), ("route_chunk", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)] + \
               [(n, ctypes.c_uint64) for n in (
                   "off_counts", "off_offsets", "off_mtiles", "off_tile_expert", "off_perm", "off_inv",
                   "off_xq", "off_xs", "off_h", "off_hs", "off_y", "off_route_hist", "off_tile_rows",
                   "off_y_exp")] + \
               [("y_format", ctypes.c_int32), ("reserved", ctypes.c_uint32 * 3)]


class SituMoeTensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "hidden_states", "hidden_states_scale", "topk_ids", "topk_weights", "topk_packed",
        "w1", "w1_scale", "w2", "w2_scale", "situ_beta", "situ_linear_beta", "alpha_gate",
        "alpha_up", "out", "swiglu_alpha", "swiglu_beta", "alpha_down", "gate_up_lora_delta",
        "activation_lora_input")]


_LIB = None


def load():
    """Load libsitu_moe.so (once).  Imports torch first so that the library
    binds to the HIP runtime torch already mapped (both are libamdhip64.so.7)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  (maps the HIP runtime before the library needs it)
    path = library_path()
    if not os.path.exists(path):
        raise SituMoeError(5, f"{path} is not built; run `python -m block_scaled_mxfp4_amd.build`")
    lib = ctypes.CDLL(path)
    lib.situ_moe_abi_version.restype = ctypes.c_int32
    if lib.situ_moe_abi_version() != ABI_VERSION:
        raise SituMoeError(5, f"{path} has ABI {lib.situ_moe_abi_version()}, this binding needs {ABI_VERSION}; rebuild it")
    P = ctypes.POINTER
    c_int, c_i64, c_u64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
    sig = {
        "situ_moe_plan": (c_int, [P(SituMoeProblem), P(SituMoePlan)]),
        "situ_moe_valid_tactics": (c_int, [P(SituMoeProblem), P(c_int), P(c_int), c_int, P(c_int)]),
        "situ_moe_run": (c_int, [P(SituMoePlan), P(SituMoeTensors), vp, c_u64, vp]),
        "situ_moe_route": (c_int, [P(SituMoePlan), P(SituMoeTensors), vp, c_u64, vp]),
        "situ_moe_run_profiled": (c_int, [P(SituMoePlan), P(SituMoeTensors), vp, c_u64, vp, P(vp), c_int]),
        "situ_moe_run_static": (c_int, [P(SituMoePlan), P(SituMoeTensors), vp]),
        "situ_moe_quantize_mxfp8": (c_int, [vp, c_i64, c_int, vp, vp, vp]),
        "situ_moe_tile_weights": (c_int, [vp, vp, c_int, c_int, c_int, vp, vp, vp]),
        "situ_moe_measure_mfma_peak": (c_int, [c_int, P(ctypes.c_double)]),
        "situ_moe_status_string": (ctypes.c_char_p, [c_int]),
        "situ_moe_last_error": (ctypes.c_char_p, []),
        "situ_moe_build_info": (ctypes.c_char_p, []),
        "situ_moe_tactic_name": (ctypes.c_char_p, [c_int]),
        "situ_moe_abi_version": (c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status):
    if status != 0:
        raise SituMoeError(status, load().situ_moe_last_error().decode())


def _stream(stream):
    """A hipStream_t from a torch.cuda.Stream, a raw handle (int), or None
    (torch's current stream)."""
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    handle = getattr(stream, "cuda_stream", stream)
    return ctypes.c_void_p(int(handle))


# ------------------------------------------------------------------ C names

def situ_moe_status_string(status):
    return load().situ_moe_status_string(int(status)).decode()


def situ_moe_last_error():
    return load().situ_moe_last_error().decode()


def situ_moe_build_info():
    return load().situ_moe_build_info().decode()


def situ_moe_tactic_name(tactic):
    r = load().situ_moe_tactic_name(int(tactic))
    return None if r is None else r.decode()


def situ_moe_abi_version():
    return int(load().situ_moe_abi_version())


def situ_moe_plan(problem):
    plan = SituMoePlan()
    _check(load().situ_moe_plan(ctypes.byref(problem), ctypes.byref(plan)))
    return plan


def situ_moe_valid_tactics(problem):
    n = ctypes.c_int32(0)
    _check(load().situ_moe_valid_tactics(ctypes.byref(problem), None, None, 0, ctypes.byref(n)))
    a = (ctypes.c_int32 * max(n.value, 1))()
    b = (ctypes.c_int32 * max(n.value, 1))()
    _check(load().situ_moe_valid_tactics(ctypes.byref(problem), a, b, n.value, ctypes.byref(n)))
    return [(a[i], b[i]) for i in range(n.value)]


def situ_moe_run(plan, tensors, workspace, stream=None):
    ws, nbytes = _ws(workspace)
    _check(load().situ_moe_run(ctypes.byref(plan), ctypes.byref(tensors), ws, nbytes, _stream(stream)))


STATIC_SCRATCH_BYTES = 128 * 1024 * 1024   # SITU_MOE_STATIC_SCRATCH_BYTES


def situ_moe_run_static(plan, tensors, stream=None):
    """situ_moe_run on the library's own per-device scratch array: no
    workspace, no allocation (plans needing more than STATIC_SCRATCH_BYTES
    raise SITU_E_WORKSPACE; overlapping calls on one device race)."""
    _check(load().situ_moe_run_static(ctypes.byref(plan), ctypes.byref(tensors), _stream(stream)))


def situ_moe_run_profiled(plan, tensors, workspace, events, stream=None):
    """situ_moe_run recording six caller-created torch.cuda.Event objects (enable_timing=True)
    at the stage boundaries: start, routed, quantized, FC1, FC2, combined."""
    if len(events) != 6:
        raise SituMoeError(1, "six events are needed")
    handles = (ctypes.c_void_p * 6)()
    for i, e in enumerate(events):
        if not e.cuda_event:          # torch creates the event at its first record
            e.record()
        handles[i] = e.cuda_event
    ws, nbytes = _ws(workspace)
    _check(load().situ_moe_run_profiled(ctypes.byref(plan), ctypes.byref(tensors), ws, nbytes, _stream(stream),
                                        handles, 6))


def situ_moe_route(plan, tensors, workspace, stream=None):
    ws, nbytes = _ws(workspace)
    _check(load().situ_moe_route(ctypes.byref(plan), ctypes.byref(tensors), ws, nbytes, _stream(stream)))


def situ_moe_quantize_mxfp8(x, codes, scales, stream=None):
    """x: bf16 [rows, cols] (cuda); codes: uint8 [rows, cols]; scales: uint8 [rows, cols/32]."""
    import torch
    _need(x, torch.bfloat16, x.shape, "x")
    rows, cols = x.shape
    _need(codes, torch.uint8, (rows, cols), "codes")
    _need(scales, torch.uint8, (rows, cols // 32), "scales")
    _check(load().situ_moe_quantize_mxfp8(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))


def tiled_shapes(experts, rows, k):
    """Shapes of the fragment-tiled weights and scales of an [experts, rows, k] MXFP4 matrix."""
    steps = (k // 32 + 3) // 4
    return (experts, rows // 16, steps, 1024), (experts, rows // 16, steps, 64)


def situ_moe_measure_mfma_peak(iters=2000):
    """TFLOP/s the current device sustains on the block-scaled FP4 x FP8 MFMA
    of the w4a8 GEMMs (a measurement aid; synchronous)."""
    out = ctypes.c_double(0.0)
    _check(load().situ_moe_measure_mfma_peak(int(iters), ctypes.byref(out)))
    return out.value


def situ_moe_tile_weights(w, w_scale, w_tiled=None, scale_tiled=None, stream=None):
    """MXFP4 weights w uint8 [E, rows, k/2] with scales uint8 [E, rows, k/32]
    (cuda) in the fragment-tiled layout of situ_moe_tile_weights; returns
    (w_tiled, scale_tiled), allocated here when not given."""
    import torch
    if w.dim() != 3:
        raise SituMoeError(2, "w must be [experts, rows, k/2]")
    E, R, half_k = w.shape
    k = 2 * half_k
    _need(w, torch.uint8, (E, R, half_k), "w")
    _need(w_scale, torch.uint8, (E, R, k // 32), "w_scale")
    ws_shape, ss_shape = tiled_shapes(E, R, k)
    if w_tiled is None:
        w_tiled = torch.empty(ws_shape, dtype=torch.uint8, device=w.device)
    if scale_tiled is None:
        scale_tiled = torch.empty(ss_shape, dtype=torch.uint8, device=w.device)
    _need(w_tiled, torch.uint8, ws_shape, "w_tiled")
    _need(scale_tiled, torch.uint8, ss_shape, "scale_tiled")
    _check(load().situ_moe_tile_weights(_ptr(w), _ptr(w_scale), E, R, k, _ptr(w_tiled), _ptr(scale_tiled),
                                        _stream(stream)))
    return w_tiled, scale_tiled


# ------------------------------------------------------------------ helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ws(workspace):
    if workspace is None:
        return None, 0
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def _need(t, dtype, shape, name):
    if t is None:
        raise SituMoeError(1, f"{name} is None")
    if not t.is_cuda:
        raise SituMoeError(5, f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise SituMoeError(2, f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise SituMoeError(2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise SituMoeError(2, f"{name} must be contiguous")


def make_problem(*, num_tokens, hidden_size, intermediate_size, num_experts, local_expert_offset,
                 local_num_experts, top_k, act_mode="w4a16", act_prequantized=False, topk_packed=False,
                 out_dtype="f32", tactic=(-1, -1), activation="situ", weight_format="mxfp4"):
    act = {"w4a16": ACT_W4A16, "w4a8": ACT_W4A8}[act_mode] if isinstance(act_mode, str) else int(act_mode)
    od = {"f32": OUT_F32, "float32": OUT_F32, "bf16": OUT_BF16, "bfloat16": OUT_BF16}[out_dtype] \
        if isinstance(out_dtype, str) else int(out_dtype)
    ak = ACTIVATIONS[activation] if isinstance(activation, str) else int(activation)
    wf = WEIGHT_FORMATS[weight_format] if isinstance(weight_format, str) else int(weight_format)
    return SituMoeProblem(num_tokens, hidden_size, intermediate_size, num_experts, local_expert_offset,
                          local_num_experts, top_k, act, int(bool(act_prequantized)), int(bool(topk_packed)),
                          od, int(tactic[0]), int(tactic[1]), ak, wf)


def make_tensors(problem, *, hidden_states, hidden_states_scale=None, topk_ids=None, topk_weights=None,
                 topk_packed=None, w1, w1_scale, w2, w2_scale, situ_beta=None, situ_linear_beta=None,
                 alpha_gate=None, alpha_up=None, out, swiglu_alpha=None, swiglu_beta=None, alpha_down=None,
                 gate_up_lora_delta=None, activation_lora_input=None):
    """Check dtypes/shapes/devices of torch tensors against the problem and
    return the C struct of their device pointers."""
    import torch
    p = problem
    T, H, I, k, E = p.num_tokens, p.hidden_size, p.intermediate_size, p.top_k, p.local_num_experts
    if p.act_prequantized:
        _need(hidden_states, torch.uint8, (T, H), "hidden_states")
        if hidden_states_scale is None:
            raise SituMoeError(4, "w4a8 prequantized input needs hidden_states_scale")
        _need(hidden_states_scale, torch.uint8, (T, H // 32), "hidden_states_scale")
    else:
        _need(hidden_states, torch.bfloat16, (T, H), "hidden_states")
    if p.topk_packed:
        _need(topk_packed, torch.int32, (T, k), "topk_packed")
    else:
        _need(topk_ids, torch.int32, (T, k), "topk_ids")
        _need(topk_weights, torch.bfloat16, (T, k), "topk_weights")
    if p.weight_format == WEIGHT_FORMATS["mxfp4_tiled"]:
        w1_shape, s1_shape = tiled_shapes(E, 2 * I, H)
        w2_shape, s2_shape = tiled_shapes(E, H, I)
    else:
        sblk = 16 if p.weight_format == WEIGHT_FORMATS["nvfp4"] else 32   # K elements per weight scale
        w1_shape, s1_shape = (E, 2 * I, H // 2), (E, 2 * I, H // sblk)
        w2_shape, s2_shape = (E, H, I // 2), (E, H, I // sblk)
    _need(w1, torch.uint8, w1_shape, "w1")
    _need(w1_scale, torch.uint8, s1_shape, "w1_scale")
    _need(w2, torch.uint8, w2_shape, "w2")
    _need(w2_scale, torch.uint8, s2_shape, "w2_scale")
    required = {0: ("situ_beta", "situ_linear_beta"), 1: (), 2: ("swiglu_alpha", "swiglu_beta")}[p.activation]
    params = {"situ_beta": situ_beta, "situ_linear_beta": situ_linear_beta, "swiglu_alpha": swiglu_alpha,
              "swiglu_beta": swiglu_beta, "alpha_gate": alpha_gate, "alpha_up": alpha_up, "alpha_down": alpha_down}
    for name, t in params.items():
        if name in required or t is not None:
            _need(t, torch.float32, (E,), name)
    if gate_up_lora_delta is not None:
        _need(gate_up_lora_delta, torch.bfloat16, (T * k, 2 * I), "gate_up_lora_delta")
    if activation_lora_input is not None:
        _need(activation_lora_input, torch.bfloat16, (T * k, I), "activation_lora_input")
    _need(out, torch.bfloat16 if p.out_dtype == OUT_BF16 else torch.float32, (T, H), "out")
    ts = SituMoeTensors()
    for name, t in (("hidden_states", hidden_states), ("hidden_states_scale", hidden_states_scale),
                    ("topk_ids", topk_ids), ("topk_weights", topk_weights), ("topk_packed", topk_packed),
                    ("w1", w1), ("w1_scale", w1_scale), ("w2", w2), ("w2_scale", w2_scale),
                    ("out", out), ("gate_up_lora_delta", gate_up_lora_delta),
                    ("activation_lora_input", activation_lora_input)) + tuple(params.items()):
        setattr(ts, name, None if t is None else t.data_ptr())
    return ts


def new_workspace(plan, device=None):
    """A device byte tensor of the plan's workspace size (256-byte aligned by the allocator)."""
    import torch
    return torch.empty(max(int(plan.workspace_bytes), 1), dtype=torch.uint8, device=device or "cuda")


_REGIONS = {"counts": "off_counts", "offsets": "off_offsets", "mtiles": "off_mtiles",
            "tile_expert": "off_tile_expert", "perm": "off_perm", "inv": "off_inv", "xq": "off_xq",
            "xs": "off_xs", "h": "off_h", "hs": "off_hs", "y": "off_y", "route_hist": "off_route_hist",
            "tile_rows": "off_tile_rows", "y_exp": "off_y_exp"}


def workspace_view(plan, workspace, region, dtype, shape):
    """A typed view of one workspace region (the routing results and
    intermediates a run leaves there)."""
    import math
    off = int(getattr(plan, _REGIONS[region]))
    n = math.prod(shape) * dtype.itemsize
    return workspace[off:off + n].view(dtype).view(*shape)


def situ_moe(*, hidden_states, hidden_states_scale=None, topk_ids=None, topk_weights=None,
             topk_packed=None, w1, w1_scale, w2, w2_scale, situ_beta=None, situ_linear_beta=None,
             alpha_gate=None, alpha_up=None, num_experts, local_expert_offset, local_num_experts,
             intermediate_size, act_mode="w4a16", out_dtype=None, tactic=(-1, -1), out=None,
             workspace=None, stream=None, activation="situ", weight_format="mxfp4", swiglu_alpha=None,
             swiglu_beta=None, alpha_down=None, gate_up_lora_delta=None, activation_lora_input=None):
    """One call of the layer on torch device tensors (keyword-only, like the
    pages' mxfp4_situ_routed_moe): returns the [T, H] partial output.

    stream: a torch.cuda.Stream, a raw hipStream_t handle, or None for the
    current stream.  `out` and the workspace, when this function allocates
    them, come from torch's caching allocator on that stream, so they are not
    handed to another allocation while the layer's kernels still use them."""
    import torch
    T, H = hidden_states.shape
    k = (topk_packed if topk_packed is not None else topk_ids).shape[1]
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    od = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    prob = make_problem(num_tokens=T, hidden_size=H, intermediate_size=intermediate_size,
                        num_experts=num_experts, local_expert_offset=local_expert_offset,
                        local_num_experts=local_num_experts, top_k=k, act_mode=act_mode,
                        act_prequantized=hidden_states.dtype == torch.uint8,
                        topk_packed=topk_packed is not None, out_dtype=od, tactic=tactic,
                        activation=activation, weight_format=weight_format)
    plan = situ_moe_plan(prob)
    dev = hidden_states.device
    if stream is None:
        stream_obj = torch.cuda.current_stream(dev)
    elif isinstance(stream, torch.cuda.Stream):
        stream_obj = stream
    else:
        stream_obj = torch.cuda.ExternalStream(int(stream), device=dev)
    with torch.cuda.stream(stream_obj):
        if out is None:
            out = torch.empty((T, H), dtype=out_dtype, device=dev)
        if workspace is None:
            workspace = new_workspace(plan, dev)
    ts = make_tensors(prob, hidden_states=hidden_states, hidden_states_scale=hidden_states_scale,
                      topk_ids=topk_ids, topk_weights=topk_weights, topk_packed=topk_packed, w1=w1,
                      w1_scale=w1_scale, w2=w2, w2_scale=w2_scale, situ_beta=situ_beta,
                      situ_linear_beta=situ_linear_beta, alpha_gate=alpha_gate, alpha_up=alpha_up, out=out,
                      swiglu_alpha=swiglu_alpha, swiglu_beta=swiglu_beta, alpha_down=alpha_down,
                      gate_up_lora_delta=gate_up_lora_delta, activation_lora_input=activation_lora_input)
    situ_moe_run(plan, ts, workspace, stream_obj)
    return out

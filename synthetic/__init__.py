"""Seeded synthetic inputs for the MXFP4 + SiTU routed-MoE layer.

This module is shared by the tests, the benchmark and the smoke check.  It
holds none of the layer's arithmetic: it draws random numbers, selects top-k
experts, and lays the draws out in the layer's input formats.  Neither the
CPU oracle nor the HIP library is imported here, and neither imports this.

The workloads (shapes, routing skew, activation mode) are those of the five
synthetic configurations the layer is measured on: a tiny all-local case, a
tensor-parallel (TP8) decode shard, an expert-parallel (EP8) decode shard,
and the two matching prefill shards ("TokenSpeed SiTU", "Supported contract":
hidden 3584, 896 experts, top-16, TP8 with intermediate 384 or EP8 with 112
local experts at offset ep_rank * 112 and intermediate 3072).

Recipe (fixed draw order from one PCG64 stream seeded with the config seed):
  1. router logits [T, E_g] ~ N(0, 1), float32;
  2. if skewed: logits += r**-1.1 with r = 1 + a random permutation of the
     experts (a Zipf(1.1) popularity bias);
  3. if constrained: the dead local experts and the tokens that must get no
     local slot;
  4. hidden states [T, H] ~ N(0, 1), float32, kept as bf16 by truncating to
     the upper 16 bits (an input draw, not a rounding the layer performs);
  5. SiTU beta and linear beta ~ U[0.5, 2], then alpha_gate and alpha_up ~
     U[0.8, 1.2], float32, one per local expert.
Each expert's W1 and W2 are drawn in MXFP4 form (see below) from streams of
their own, seeded with (seed, 1, expert) and (seed, 2, expert).
Top-k: the k largest logits (stable order, lower expert id first on ties);
weights = float32 softmax over the k selected logits, kept as bf16 by
truncation.  Constrained routing (the EP8 prefill shard): the dead experts
and, for the chosen tokens, every local expert get logit -inf; a token that
is not chosen but still has no local expert in its top-k gets its last slot
replaced by its best live local expert.

MXFP4 weights.  The weights stand for N(0, 0.02) draws quantized to MXFP4
with one E8M0 scale per 32 along K.  They are drawn in the encoded domain:
each 32-block first draws its scale code from {119, 120, 121}, then each
element draws its 4-bit code from a fixed 256-way table for that scale.  The
tables hold the code frequencies of N(0, 0.02) blocks quantized with the OCP
MX rule, measured once on a million blocks and rounded to 1/256 (and the
scale frequencies to 1/65536); a CPU test re-measures them against the
oracle's quantizer.  Two codes per byte, the low nibble the even element.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Per-scale frequency of each E2M1 magnitude code 1..7 (out of 256 draws);
# the sign is drawn symmetric, code 0 takes the rest of the 256.
_MAG_COUNTS = {
    119: (11, 11, 11, 16, 19, 24, 30),
    120: (20, 18, 17, 21, 20, 16, 6),
    121: (36, 28, 19, 15, 6, 4, 0),
}
_SCALE_CODES = (119, 120, 121)
# P(scale code 119) and P(121) out of 65536; 120 takes the rest.
_SCALE_119_OF_65536 = 1176
_SCALE_121_OF_65536 = 3628


def _code_table(mag_counts):
    """256-entry table: uniform byte -> 4-bit code with the given frequencies."""
    tab = []
    for m, c in enumerate(mag_counts, start=1):
        tab += [m] * c           # positive magnitude code m
        tab += [m | 8] * c       # the same magnitude, sign bit set
    tab += [0] * (256 - len(tab))
    assert len(tab) == 256
    return np.array(tab, dtype=np.uint8)


def _byte_tables():
    """[3 * 65536] table: (scale index, 16 random bits) -> one packed byte."""
    out = np.empty((3, 65536), dtype=np.uint8)
    r = np.arange(65536)
    for i, s in enumerate(_SCALE_CODES):
        t = _code_table(_MAG_COUNTS[s])
        out[i] = t[r & 0xFF] | (t[r >> 8] << 4)
    return out.reshape(-1)


_BYTE_TABLE = _byte_tables()


def draw_mxfp4(seed_words, rows, K):
    """One MXFP4 matrix [rows, K]: (packed bytes [rows, K/2], scale codes [rows, K/32]).

    Drawn from its own PCG64 stream seeded with `seed_words`, so the matrices
    of different experts can be drawn in parallel and in any order.
    """
    assert K % 32 == 0
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed_words)))
    r = np.frombuffer(rng.bytes(rows * (K // 32) * 2), dtype=np.uint16).reshape(rows, K // 32)
    sidx = ((r >= _SCALE_119_OF_65536).astype(np.uint8)
            + (r >= 65536 - _SCALE_121_OF_65536).astype(np.uint8))
    bits = np.frombuffer(rng.bytes(rows * (K // 2) * 2), dtype=np.uint16).reshape(rows, K // 2)
    idx = np.repeat(sidx, 16, axis=1).astype(np.int32) << 16
    idx |= bits
    return _BYTE_TABLE[idx], (np.uint8(_SCALE_CODES[0]) + sidx).astype(np.uint8)


# NVFP4 weights (E2M1 with an E4M3 scale per 16 along K) are drawn in the
# encoded domain as well: elements from the middle table above, block scales
# uniformly from the E4M3 codes of [0.5, 2) (0x30..0x3F), and the per-tensor
# scale that makes them stand for N(0, 0.02) weights (2^-7) goes into the
# per-expert alphas.
NVFP4_TENSOR_SCALE = 2.0 ** -7


def draw_nvfp4(seed_words, rows, K):
    """One NVFP4 matrix [rows, K]: (packed bytes [rows, K/2], E4M3 scale codes [rows, K/16])."""
    assert K % 32 == 0
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed_words)))
    sc = (0x30 + rng.integers(0, 16, size=(rows, K // 16))).astype(np.uint8)
    bits = np.frombuffer(rng.bytes(rows * (K // 2) * 2), dtype=np.uint16).reshape(rows, K // 2)
    idx = (np.int32(1) << 16) | bits.astype(np.int32)      # the scale-120 element table
    return _BYTE_TABLE[idx], sc


def bf16_truncate(x):
    """float32 -> bf16 bit pattern by keeping the upper 16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (x.view(np.uint32) >> 16).astype(np.uint16)


CONFIGS = {
    0: dict(name="tiny", T=4, H=256, I=64, E_g=8, E_l=8, off=0, k=2,
            mode="w4a16", skew=False, packed=False, seed=0),
    1: dict(name="tp8_decode", T=64, H=3584, I=384, E_g=896, E_l=896, off=0, k=16,
            mode="w4a16", skew=True, packed=False, seed=1),
    2: dict(name="ep8_decode", T=256, H=3584, I=3072, E_g=896, E_l=112, off=336, k=16,
            mode="w4a16", skew=True, packed=False, seed=2),
    3: dict(name="tp8_prefill", T=16384, H=3584, I=384, E_g=896, E_l=896, off=0, k=16,
            mode="w4a8", skew=True, packed=False, seed=3),
    4: dict(name="ep8_prefill", T=32768, H=3584, I=3072, E_g=896, E_l=112, off=336, k=16,
            mode="w4a8", skew=True, packed=True, seed=4, n_dead=8, no_local_frac=0.3),
}


def spec_of(cfg):
    """A config id or a spec dict -> a full spec dict with defaults filled in."""
    s = dict(CONFIGS[cfg]) if isinstance(cfg, int) else dict(cfg)
    s.setdefault("name", "custom")
    s.setdefault("off", 0)
    s.setdefault("E_l", s["E_g"])
    s.setdefault("mode", "w4a16")
    s.setdefault("skew", False)
    s.setdefault("packed", False)
    s.setdefault("seed", 0)
    s.setdefault("n_dead", 0)
    s.setdefault("no_local_frac", 0.0)
    s.setdefault("activation", "situ")
    s.setdefault("weight_format", "mxfp4")
    s.setdefault("lora", False)
    return s


def _topk(logits, k):
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def _softmax_rows(v):
    v = v.astype(np.float32)
    m = np.max(v, axis=1, keepdims=True)
    e = np.exp(v - m)
    return (e / np.sum(e, axis=1, keepdims=True)).astype(np.float32)


def generate(cfg, weights=True):
    """Draw every input of one configuration.  Returns a dict of numpy arrays.

    Keys: hidden_states (uint16 bf16 bits [T, H]); topk_ids (int32 [T, k]) and
    topk_weights (uint16 bf16 bits [T, k]); topk_packed (int32 [T, k]) when the
    spec asks for the packed format; w1, w1_scale, w2, w2_scale (uint8);
    situ_beta, situ_linear_beta, alpha_gate, alpha_up (float32 [E_l]); spec.
    With weights=False the expert weights are skipped (routing-only use); the
    draws after them then differ, so such inputs are never mixed with full ones.
    Spec options drawn after everything above (so they leave those draws
    unchanged): activation "swiglu_bias" adds swiglu_alpha ~ U[0.5, 2] and
    swiglu_beta ~ U[0.5, 1.5]; weight_format "nvfp4" draws NVFP4 weights, folds
    the per-tensor scale into alpha_gate / alpha_up and adds alpha_down (the
    same scale times U[0.8, 1.2]); lora adds gate_up_lora_delta, bf16
    [T*k, 2I] ~ N(0, 0.05), a LoRA adapter's FC1 contribution per pair.
    """
    s = spec_of(cfg)
    T, H, I, E_g, E_l, off, k = (s[x] for x in ("T", "H", "I", "E_g", "E_l", "off", "k"))
    assert H % 32 == 0 and I % 32 == 0 and 0 <= off and off + E_l <= E_g and 1 <= k <= E_g
    rng = np.random.Generator(np.random.PCG64(s["seed"]))

    logits = rng.standard_normal((T, E_g), dtype=np.float32)
    if s["skew"]:
        r = 1.0 + rng.permutation(E_g).astype(np.float64)
        logits += (r ** -1.1).astype(np.float32)[None, :]
    dead = np.zeros(0, dtype=np.int64)
    none = np.zeros(0, dtype=np.int64)
    if s["n_dead"] or s["no_local_frac"]:
        dead = off + np.sort(rng.choice(E_l, s["n_dead"], replace=False))
        n_none = int(np.floor(s["no_local_frac"] * T))
        none = np.sort(rng.choice(T, n_none, replace=False))
        logits[:, dead] = -np.inf
        logits[np.ix_(none, np.arange(off, off + E_l))] = -np.inf

    x = rng.standard_normal((T, H), dtype=np.float32)

    ids = _topk(logits, k)
    if len(none) or len(dead):
        local = (ids >= off) & (ids < off + E_l)
        is_none = np.zeros(T, dtype=bool)
        is_none[none] = True
        fix = ~local.any(axis=1) & ~is_none
        if fix.any():
            best = off + np.argmax(logits[np.ix_(np.nonzero(fix)[0], np.arange(off, off + E_l))], axis=1)
            ids[fix, k - 1] = best
        local = (ids >= off) & (ids < off + E_l)
        assert int((~local.any(axis=1)).sum()) == len(none), "constrained routing: no-local count"
        used = np.zeros(E_l, dtype=bool)
        used[ids[local] - off] = True
        assert set(np.nonzero(~used)[0] + off) == set(dead.tolist()), "constrained routing: dead experts"
    sel = np.take_along_axis(logits, ids, axis=1)
    wts = _softmax_rows(sel)

    out = dict(spec=s, hidden_states=bf16_truncate(x),
               topk_ids=ids.astype(np.int32), topk_weights=bf16_truncate(wts))
    if s["packed"]:
        assert E_g < 65536
        words = (out["topk_weights"].astype(np.uint32) << 16) | ids.astype(np.uint32)
        out["topk_packed"] = words.view(np.int32)
    if weights:
        w1 = np.empty((E_l, 2 * I, H // 2), dtype=np.uint8)
        w1s = np.empty((E_l, 2 * I, H // 32), dtype=np.uint8)
        w2 = np.empty((E_l, H, I // 2), dtype=np.uint8)
        w2s = np.empty((E_l, H, I // 32), dtype=np.uint8)

        nv = s["weight_format"] == "nvfp4"
        if nv:
            w1s = np.empty((E_l, 2 * I, H // 16), dtype=np.uint8)
            w2s = np.empty((E_l, H, I // 16), dtype=np.uint8)
        draw = draw_nvfp4 if nv else draw_mxfp4

        def fill(job):
            which, l = job
            if which == 1:
                w1[l], w1s[l] = draw([s["seed"], 1, l], 2 * I, H)
            else:
                w2[l], w2s[l] = draw([s["seed"], 2, l], H, I)

        jobs = [(1, l) for l in range(E_l)] + [(2, l) for l in range(E_l)]
        with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
            list(ex.map(fill, jobs))
        out.update(w1=w1, w1_scale=w1s, w2=w2, w2_scale=w2s)
    out["situ_beta"] = rng.uniform(0.5, 2.0, E_l).astype(np.float32)
    out["situ_linear_beta"] = rng.uniform(0.5, 2.0, E_l).astype(np.float32)
    out["alpha_gate"] = rng.uniform(0.8, 1.2, E_l).astype(np.float32)
    out["alpha_up"] = rng.uniform(0.8, 1.2, E_l).astype(np.float32)
    if s["activation"] == "swiglu_bias":
        out["swiglu_alpha"] = rng.uniform(0.5, 2.0, E_l).astype(np.float32)
        out["swiglu_beta"] = rng.uniform(0.5, 1.5, E_l).astype(np.float32)
    if s["weight_format"] == "nvfp4":
        g = np.float32(NVFP4_TENSOR_SCALE)
        out["alpha_gate"] = (out["alpha_gate"] * g).astype(np.float32)
        out["alpha_up"] = (out["alpha_up"] * g).astype(np.float32)
        out["alpha_down"] = (rng.uniform(0.8, 1.2, E_l).astype(np.float32) * g).astype(np.float32)
    if s["lora"]:
        out["gate_up_lora_delta"] = bf16_truncate(rng.standard_normal((T * k, 2 * I), dtype=np.float32) * 0.05)
    return out

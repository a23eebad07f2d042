"""Seeded synthetic workloads for padded sigmoid attention.

This module draws sequence lengths and input tensors, rounds them to the storage
dtype, and counts the FLOPs used for reporting. It holds none of the attention
arithmetic and imports neither the oracle nor the GPU binding; both consume what it
produces, so the two sides always receive the same input bits.

Workloads (shapes follow the kernel benchmark of "Better Models, Faster Training:
Sigmoid Attention for single-cell Foundation Models", §4.1 "Kernel Performance", the
160M layer shape of its Table 2, and the GPT-2-shaped gated decoder of "Sigmoid
Attention as a Better Substrate for Learned KV Cache Eviction"):

=====================  =====  ==  ==  ===  =====  ===========================================
name                   dtype  B   H   d    Lmax   lengths / values
=====================  =====  ==  ==  ===  =====  ===========================================
tiny_fp32              f32    2   2   64   128    n = {128, 77}; N(0,1)
bidir_2k               bf16   8   16  64   2048   n ~ U{1024..2048}; N(0,1)
long_8k_s1             bf16   4   12  64   8192   n ~ U{4096..8192}; Q,K ~ N(0,1)
long_8k_s4             bf16   4   12  64   8192   n ~ U{4096..8192}; Q,K ~ N(0,16)
pad_sweep_{0,25,50}    bf16   16  16  128  4096   mean padding fixed at 0/25/50 %
causal_gated_512       bf16   16  12  64   512    causal, all valid; RMS-normalised Q,K;
                                                  gate g = logistic(z), z ~ N(2, var 2)
causal_forced_drop_512 bf16   16  12  64   512    as above, plus g = 0.01 on a seeded 20%
                                                  of keys j >= 4 (exercises hard dropping)
sweep_16k_d64_p25      bf16   1   32  64   16384  kernel-sweep extremes (B*L = 16384 tokens):
sweep_16k_d128         bf16   1   16  128  16384  25 % / 0 % padding; the sweep itself
sweep_512_d128_p25     bf16   32  16  128  512    (bench.py --sweep) covers every L and d
decode_gpt2_512        bf16   16  12  64   512    KV cache of a 512-token prefill, gates as in
                                                  causal_forced_drop_512; one decode query
decode_long            bf16   32  16  128  16384  KV cache of prefills n ~ U{8192..16384},
                                                  gates as above; one decode query
decode_long_64         bf16   32  12  64   16384  same lengths and gates, d = 64
=====================  =====  ==  ==  ===  =====  ===========================================

Decode workloads (``generate_decode``) draw, in order: lengths, the prefill K and V,
the prefill gates, then one new token per sequence (its query, key, value and gate).

Draw order with ``numpy.random.default_rng(seed)``: lengths, Q, K, V, dO, gate. Draws
are float32 standard normals, scaled, then rounded to bf16 (round to nearest even) for
bf16 workloads. Padded slots hold ordinary draws, or NaN when ``poison=True``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "generate", "generate_decode", "round_to_bf16",
           "seqlens_of", "valid_pairs", "flops_forward", "flops_backward"]


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "bf16" or "f32"
    B: int
    H: int
    d: int
    L: int
    lengths: tuple        # ("fixed", [n...]) | ("uniform", lo, hi) | ("mean_pad", p)
    seed: int
    qk_std: float = 1.0
    causal: bool = False
    rmsnorm_qk: bool = False
    gate: tuple | None = None   # ("logistic_normal", mean, var[, forced_frac, forced_value])
    tau: float = 0.0
    sink: int = 4
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", "f32", 2, 2, 64, 128, ("fixed", [128, 77]), seed=0),
        Workload("bidir_2k", "bf16", 8, 16, 64, 2048, ("uniform", 1024, 2048), seed=1),
        Workload("long_8k_s1", "bf16", 4, 12, 64, 8192, ("uniform", 4096, 8192), seed=2),
        Workload("long_8k_s4", "bf16", 4, 12, 64, 8192, ("uniform", 4096, 8192), seed=3,
                 qk_std=4.0),
        Workload("pad_sweep_0", "bf16", 16, 16, 128, 4096, ("mean_pad", 0.0), seed=4),
        Workload("pad_sweep_25", "bf16", 16, 16, 128, 4096, ("mean_pad", 0.25), seed=5),
        Workload("pad_sweep_50", "bf16", 16, 16, 128, 4096, ("mean_pad", 0.5), seed=6),
        Workload("causal_gated_512", "bf16", 16, 12, 64, 512, ("fixed", [512] * 16), seed=7,
                 causal=True, rmsnorm_qk=True, gate=("logistic_normal", 2.0, 2.0),
                 tau=0.05, sink=4),
        Workload("causal_forced_drop_512", "bf16", 16, 12, 64, 512, ("fixed", [512] * 16),
                 seed=8, causal=True, rmsnorm_qk=True,
                 gate=("logistic_normal", 2.0, 2.0, 0.2, 0.01), tau=0.05, sink=4),
        # extremes of the kernel sweep (B * L = 16384 tokens, hidden 2048)
        Workload("sweep_16k_d64_p25", "bf16", 1, 32, 64, 16384, ("mean_pad", 0.25), seed=12),
        Workload("sweep_16k_d128", "bf16", 1, 16, 128, 16384, ("mean_pad", 0.0), seed=13),
        Workload("sweep_512_d128_p25", "bf16", 32, 16, 128, 512, ("mean_pad", 0.25), seed=14),
        Workload("decode_gpt2_512", "bf16", 16, 12, 64, 512, ("fixed", [512] * 16), seed=9,
                 causal=True, rmsnorm_qk=True, gate=("logistic_normal", 2.0, 2.0, 0.2, 0.01),
                 tau=0.05, sink=4, extra={"cap": 1024}),
        Workload("decode_long", "bf16", 32, 16, 128, 16384, ("uniform", 8192, 16384), seed=10,
                 gate=("logistic_normal", 2.0, 2.0, 0.2, 0.01), tau=0.05, sink=4,
                 extra={"cap": 16384}),
        Workload("decode_long_64", "bf16", 32, 12, 64, 16384, ("uniform", 8192, 16384),
                 seed=11, gate=("logistic_normal", 2.0, 2.0, 0.2, 0.01), tau=0.05, sink=4,
                 extra={"cap": 16384}),
    ]
}


def get(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. smaller B or L)."""
    return replace(WORKLOADS[name], **overrides)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 array holding the nearest bf16 values (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).copy()
    out[np.isnan(x)] = np.nan
    return out


def _lengths(w: Workload, rng) -> np.ndarray:
    kind = w.lengths[0]
    if kind == "fixed":
        n = np.asarray(w.lengths[1], dtype=np.int64)
        if len(n) != w.B:
            n = np.resize(n, w.B)
    elif kind == "uniform":
        lo, hi = min(w.lengths[1], w.L), min(w.lengths[2], w.L)
        n = rng.integers(lo, hi + 1, size=w.B)
    elif kind == "mean_pad":
        p = w.lengths[1]
        if p == 0.0:
            n = np.full(w.B, w.L, dtype=np.int64)
        else:
            # mean exactly m = (1-p) L: draw half, mirror the other half around m
            m = int(round((1.0 - p) * w.L))
            lo = max(1, 2 * m - w.L)
            half = w.B // 2
            a = rng.integers(lo, w.L, size=half)
            n = np.concatenate([a, 2 * m - a])
            if len(n) < w.B:
                n = np.concatenate([n, [m]])
    else:
        raise ValueError(kind)
    return np.clip(n, 0, w.L).astype(np.int32)


def seqlens_of(w: Workload | str) -> np.ndarray:
    """The valid lengths of a workload: the first draw of ``generate`` (same seed, so the
    same lengths)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return _lengths(w, np.random.default_rng(w.seed))


def generate(w: Workload | str, poison: bool = False, with_do: bool = True) -> dict:
    """Draw one batch. Returns numpy arrays (float32 values, bf16-exact for bf16)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    seqlens = _lengths(w, rng)
    shape = (w.B, w.H, w.L, w.d)

    def draw(std=1.0):
        return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)

    q, k = draw(w.qk_std), draw(w.qk_std)
    v = draw()
    do = draw() if with_do else None
    if w.rmsnorm_qk:
        # per-head RMS normalisation of each q and k vector over d, no learned weight
        for t in (q, k):
            t /= np.sqrt(np.mean(t * t, axis=-1, keepdims=True) + np.float32(1e-6))
    gate = None
    if w.gate is not None:
        kind, mean, var = w.gate[0], w.gate[1], w.gate[2]
        assert kind == "logistic_normal"
        z = rng.standard_normal((w.B, w.L)) * math.sqrt(var) + mean
        gate = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
        if len(w.gate) > 3:
            frac, val = w.gate[3], w.gate[4]
            pick = rng.random((w.B, w.L)) < frac
            pick[:, : w.sink] = False
            gate[pick] = np.float32(val)
    tensors = [q, k, v] + ([do] if with_do else [])
    if w.dtype == "bf16":
        tensors = [round_to_bf16(t) for t in tensors]
    if poison:
        for t in tensors:
            for b in range(w.B):
                t[b, :, seqlens[b]:, :] = np.nan
    out = dict(q=tensors[0], k=tensors[1], v=tensors[2], do=tensors[3] if with_do else None,
               seqlens=seqlens, gate=gate, causal=w.causal, tau=w.tau, sink=w.sink,
               workload=w)
    return out


def _gates(w: Workload, rng, shape):
    kind, mean, var = w.gate[0], w.gate[1], w.gate[2]
    assert kind == "logistic_normal"
    z = rng.standard_normal(shape) * math.sqrt(var) + mean
    gate = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    if len(w.gate) > 3:
        frac, val = w.gate[3], w.gate[4]
        pick = rng.random(shape) < frac
        if len(shape) == 2:
            pick[:, : w.sink] = False
        gate[pick] = np.float32(val)
    return gate


def generate_decode(w: Workload | str) -> dict:
    """A KV-cache workload: a prefill (K, V [B, H, L, d], gates [B, L], lengths) and one
    new token per sequence (q, k, v [B, H, d], gate [B]). Values as in ``generate``."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    seqlens = _lengths(w, rng)
    shape = (w.B, w.H, w.L, w.d)
    k = rng.standard_normal(shape, dtype=np.float32) * np.float32(w.qk_std)
    v = rng.standard_normal(shape, dtype=np.float32)
    gate = None if w.gate is None else _gates(w, rng, (w.B, w.L))
    q_new = rng.standard_normal((w.B, w.H, w.d), dtype=np.float32) * np.float32(w.qk_std)
    k_new = rng.standard_normal((w.B, w.H, w.d), dtype=np.float32) * np.float32(w.qk_std)
    v_new = rng.standard_normal((w.B, w.H, w.d), dtype=np.float32)
    g_new = None if w.gate is None else _gates(w, rng, (w.B,))
    if w.rmsnorm_qk:
        for t in (k, q_new, k_new):
            t /= np.sqrt(np.mean(t * t, axis=-1, keepdims=True) + np.float32(1e-6))
    k, v, q_new, k_new, v_new = (round_to_bf16(t) for t in (k, v, q_new, k_new, v_new))
    return dict(k=k, v=v, gate=gate, seqlens=seqlens, q=q_new, k_new=k_new, v_new=v_new,
                g_new=g_new, tau=w.tau, sink=w.sink, cap=int(w.extra.get("cap", w.L)),
                workload=w)


def valid_pairs(seqlens, causal: bool) -> int:
    """Number of (query, key) pairs counted per head: n^2, or n(n+1)/2 when causal."""
    n = np.asarray(seqlens, dtype=np.int64)
    return int(np.sum(n * (n + 1) // 2) if causal else np.sum(n * n))


def flops_forward(seqlens, H: int, d: int, causal: bool) -> float:
    """4 d per valid pair per head: two matmuls of 2 d FLOPs each (valid tokens only)."""
    return 4.0 * d * H * valid_pairs(seqlens, causal)


def flops_backward(seqlens, H: int, d: int, causal: bool) -> float:
    """2.5 times the forward count, as in the pages' FLOP appendix."""
    return 2.5 * flops_forward(seqlens, H, d, causal)

"""Sigmoid attention oracle: a plain, slow, obviously correct fp64 CPU reference.

TEST INFRASTRUCTURE. Only the test suite, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import or call this module. The product path
(the HIP library under ``sigmoid_attention_amd/`` and its Python binding) never imports,
calls or links anything here, and this module imports nothing from it.

What is computed, and where it comes from
-----------------------------------------
Sources are three web pages:

* [SA-bio] "Better Models, Faster Training: Sigmoid Attention for single-cell Foundation
  Models" (arXiv 2604.27124): §3 "Sigmoid Attention" display equation
  (O = sigma(Q K^T / sqrt(d) + b) V, element-wise), §4 "Block-sparse computation"
  (fully padded query and key blocks contribute nothing), appendix A.1.2 (the Jacobian
  of the element-wise sigmoid is diagonal with entries sigma(1 - sigma)).
* [SA-bio-nl] the gist.science summary of the same paper (in Dutch), §2A "Sigmoid
  Attention Mechanisme": sigma(x) = 1/(1 + e^-x) and the bias b = -log(n).
* [KV-evict] "Sigmoid Attention as a Better Substrate for Learned KV Cache Eviction"
  (arXiv 2608.23296), gate paragraphs: a token-wise gate g_j enters through both the
  logits (+ log(g_j + eps), eps = 1e-8) and the values (g_j * v_j); hard deletion drops
  keys with g_j < tau; the random-removal probe excludes the first four positions and
  treats a removed key as masked out of the logits with its value zeroed.

Readings taken where the pages are silent (each is also listed in the design notes):

* n in b = -log(n) is the sequence's valid (unpadded) length, natural log, the same for
  every query of that sequence (also under the causal mask). n = 1 gives b = 0; n = 0
  produces all-zero outputs and b is never evaluated.
* Padded query rows of O, dQ, dK, dV are exactly zero; padded keys contribute exactly
  zero whatever the padded slots hold.
* Causal means key j is allowed for query i iff j <= i.
* Gate: x_ij += log(g_j + eps) and V'_j = g_j * v_j; the gate is per key, shared by all
  heads. A key is dropped iff j >= sink and g_j < tau; a dropped key is treated exactly
  like padding.
* The backward follows from the forward by the chain rule with the diagonal Jacobian:
  dV'_j = sum_i P_ij dO_i (so dV_j = g_j sum_i P_ij dO_i), dP_ij = dO_i . V'_j,
  dS_ij = dP_ij P_ij (1 - P_ij), dQ_i = s sum_j dS_ij k_j, dK_j = s sum_i dS_ij q_i.
* The gate gradient (not written out in the pages; the gate is trained, so it is
  needed) follows by the same chain rule through both places g_j enters:
  dg_j = sum_i dS_ij / (g_j + eps) + v_j . sum_i P_ij dO_i, per head; the gate is shared
  by the heads, so the gradient of the shared gate is the sum over heads. The hard drop
  is a step function of g: a dropped key gets derivative 0, like a padded key.
* Packed batches with separate query and key lengths (not in the pages; needed to run a
  query shard of a sequence on one GPU): sequence b owns query rows cu_q[b]..cu_q[b+1]-1
  and key rows cu_k[b]..cu_k[b+1]-1; beta_b = -log(nk_b) unless given; the causal rule
  is aligned at the bottom right, key j allowed for query i iff j <= i + nk_b - nq_b,
  which for nq = nk is the rule above and for a shard of queries s..s+m-1 given keys
  0..s+m-1 is the rule of the full sequence.
* Decode with eviction ([KV-evict] gate paragraphs): after prefill the entries with
  g_j < tau (j >= sink) are physically removed; each entry written during decode is kept
  or removed by the same rule when it is written; kept entries keep their log-gate on
  the logits and their gate factor on the values. The cache holds the kept entries in
  position order. A decode step writes the new token's entry first and then lets the
  new query attend to the whole cache, so a dropped new entry is not seen even by its
  own query (as a dropped key is masked for every query in the forward). The bias of a
  decode step is an input (the model's beta, e.g. -log n of the sequence length it was
  trained with); with it, decoding query i against the cache of tokens 0..i gives row i
  of the causal forward with hard dropping.
* Row mass ([KV-evict] row-sum diagnostic): sum_j P_ij over the allowed keys of query
  i, i.e. the sum of the attention weights of the row, with the gate's log term in the
  logits but without the value factor g_j. Padded rows give 0.

All arithmetic is float64 on whatever values are passed in (the GPU's bf16 inputs are
passed here widened, so both sides see the same bits). Library primitives used as steps:
numpy matmul and exp. No blocking or fusion beyond splitting query rows into chunks to
bound memory, which does not change any value beyond summation order in fp64.
"""

from __future__ import annotations

import math

import numpy as np

GATE_EPS = 1e-8  # [KV-evict] gate paragraph: eps avoids log 0
DEFAULT_SINK = 4  # [KV-evict] removal probe: the first four positions are never removed

__all__ = [
    "GATE_EPS",
    "DEFAULT_SINK",
    "logistic",
    "logistic_tanh",
    "sequence_bias",
    "kept_keys",
    "forward",
    "backward",
    "forward_rows",
    "dq_rows",
    "dkdv_rows",
    "gate_grad",
    "gate_grad_rows",
    "row_mass",
    "forward_varlen",
    "backward_varlen",
    "cache_compact",
    "cache_append",
    "decode",
    "forward_naive",
    "backward_naive",
]


# ----------------------------------------------------------------------------------
# scalar definitions
# ----------------------------------------------------------------------------------

def logistic(x):
    """sigma(x) = 1 / (1 + e^-x)  ([SA-bio-nl] §2A), evaluated without overflow.

    For x >= 0 the defining form is used directly; for x < 0 the algebraically equal
    e^x / (1 + e^x) is used so that e^-x never overflows.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def logistic_tanh(x):
    """The tanh form 0.5 * (tanh(x/2) + 1) that [SA-bio] §4 "Fused operations" uses.

    It is an exact identity for sigma; kept as an independent second formula.
    """
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (np.tanh(0.5 * x) + 1.0)


def sequence_bias(n: int) -> float:
    """b = -log(n) for a sequence of n valid tokens ([SA-bio-nl] §2A); natural log."""
    if n < 1:
        raise ValueError("the bias is only defined for n >= 1")
    return -math.log(n)


def kept_keys(n: int, L: int, gate=None, tau: float = 0.0, sink: int = DEFAULT_SINK):
    """Boolean [L]: key j takes part iff it is valid (j < n) and, when gated, not dropped.

    Dropping ([KV-evict] hard-deletion rule): j >= sink and g_j < tau.
    """
    keep = np.zeros(L, dtype=bool)
    keep[:n] = True
    if gate is not None and tau > 0.0:
        g = np.asarray(gate, dtype=np.float64)[:L]
        j = np.arange(L)
        keep &= ~((j >= sink) & (g < tau))
    return keep


# ----------------------------------------------------------------------------------
# per-head building blocks
# ----------------------------------------------------------------------------------

def _params(d, scale):
    return (1.0 / math.sqrt(d)) if (scale is None or scale == 0.0) else float(scale)


def _head_setup(b, n, L, gate, tau, sink, bias, eps):
    """Per-sequence quantities: beta, the key-keep mask and the per-key log-gate term."""
    beta = sequence_bias(n) if bias is None else float(bias[b])
    g = None if gate is None else np.asarray(gate[b], dtype=np.float64)
    keep = kept_keys(n, L, g, tau, sink)
    logg = np.zeros(L) if g is None else np.log(g + eps)
    return beta, g, keep, logg


def _allowed(rows, cols, keep, causal):
    """allowed[i, j]: key cols[j] is kept and (bidirectional or cols[j] <= rows[i])."""
    a = np.broadcast_to(keep[cols][None, :], (len(rows), len(cols))).copy()
    if causal:
        a &= cols[None, :] <= rows[:, None]
    return a


def _P(qr, kh, rows, cols, s, beta, logg, keep, causal):
    """P[i, j] = sigma(s q_i.k_j + beta + log(g_j + eps)) where allowed, else exactly 0."""
    x = s * (qr @ kh.T) + beta + logg[cols][None, :]
    allowed = _allowed(rows, cols, keep, causal)
    P = np.zeros_like(x)
    P[allowed] = logistic(x[allowed])
    return P


def _vprime(vh, g, cols):
    return vh if g is None else vh * g[cols][:, None]


# ----------------------------------------------------------------------------------
# full forward / backward
# ----------------------------------------------------------------------------------

def _as64(a):
    return np.asarray(a, dtype=np.float64)


def forward(q, k, v, seqlens, causal=False, gate=None, tau=0.0, sink=DEFAULT_SINK,
            eps=GATE_EPS, scale=None, bias=None, chunk=512):
    """O[b,h] = sigma(s Q K^T + b_b [+ log(g+eps)]) V' over valid, kept keys.

    q, k, v: [B, H, L, d]; seqlens: [B]; gate: [B, L] or None.
    Returns float64 [B, H, L, d]; rows i >= n_b are exactly 0.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, L, d = q.shape
    s = _params(d, scale)
    O = np.zeros((B, H, L, d))
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:
            continue
        beta, g, keep, logg = _head_setup(b, n, L, gate, tau, sink, bias, eps)
        cols = np.arange(n)
        for h in range(H):
            kh, vp = k[b, h, :n], _vprime(v[b, h, :n], g, cols)
            for r0 in range(0, n, chunk):
                rows = np.arange(r0, min(n, r0 + chunk))
                P = _P(q[b, h, rows], kh, rows, cols, s, beta, logg, keep, causal)
                O[b, h, rows] = P @ vp
    return O


def backward(q, k, v, do, seqlens, causal=False, gate=None, tau=0.0, sink=DEFAULT_SINK,
             eps=GATE_EPS, scale=None, bias=None, chunk=512, absolute=False):
    """Gradients (dQ, dK, dV) of sum(dO * O) with respect to q, k and the caller's v.

    dV_j = g_j sum_i P_ij dO_i; dS_ij = (dO_i . V'_j) P_ij (1 - P_ij);
    dQ_i = s sum_j dS_ij k_j; dK_j = s sum_i dS_ij q_i. dO rows of padded queries are
    ignored; rows of padded or dropped keys and padded queries are exactly 0.

    absolute=True returns the magnitude sums of the same products instead:
    s sum_j |dS_ij| |k_j|, s sum_i |dS_ij| |q_i| and g_j sum_i P_ij |dO_i| (element-wise
    absolute values), which bound how rounding of dS or P propagates to each output.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, L, d = q.shape
    s = _params(d, scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:
            continue
        beta, g, keep, logg = _head_setup(b, n, L, gate, tau, sink, bias, eps)
        cols = np.arange(n)
        for h in range(H):
            kh, vp = k[b, h, :n], _vprime(v[b, h, :n], g, cols)
            dvp = np.zeros((n, d))
            dkh = np.zeros((n, d))
            for r0 in range(0, n, chunk):
                rows = np.arange(r0, min(n, r0 + chunk))
                qr, dor = q[b, h, rows], do[b, h, rows]
                P = _P(qr, kh, rows, cols, s, beta, logg, keep, causal)
                dP = dor @ vp.T
                dS = dP * P * (1.0 - P)
                if absolute:
                    dS, qr, dor = np.abs(dS), np.abs(qr), np.abs(dor)
                dq[b, h, rows] = s * (dS @ (np.abs(kh) if absolute else kh))
                dkh += s * (dS.T @ qr)
                dvp += P.T @ dor
            dk[b, h, :n] = dkh
            dv[b, h, :n] = dvp if g is None else dvp * g[:n, None]
    return dq, dk, dv


# ----------------------------------------------------------------------------------
# sampled rows (for checking large problems one output row at a time)
# ----------------------------------------------------------------------------------

def forward_rows(q, k, v, seqlens, b, h, rows, causal=False, gate=None, tau=0.0,
                 sink=DEFAULT_SINK, eps=GATE_EPS, scale=None, bias=None):
    """O[b, h, rows] computed from the full keys of (b, h); padded rows give 0."""
    rows = np.asarray(rows, dtype=np.int64)
    d = q.shape[-1]
    out = np.zeros((len(rows), d))
    n = int(seqlens[b])
    if n == 0:
        return out
    s = _params(d, scale)
    beta, g, keep, logg = _head_setup(b, n, q.shape[2], gate, tau, sink, bias, eps)
    cols = np.arange(n)
    live = rows < n
    r = rows[live]
    kh, vp = _as64(k[b, h, :n]), _vprime(_as64(v[b, h, :n]), g, cols)
    P = _P(_as64(q[b, h, r]), kh, r, cols, s, beta, logg, keep, causal)
    out[live] = P @ vp
    return out


def dq_rows(q, k, v, do, seqlens, b, h, rows, causal=False, gate=None, tau=0.0,
            sink=DEFAULT_SINK, eps=GATE_EPS, scale=None, bias=None, absolute=False):
    """dQ[b, h, rows]; padded rows give 0. absolute=True: s sum_j |dS_ij| |k_j|."""
    rows = np.asarray(rows, dtype=np.int64)
    d = q.shape[-1]
    out = np.zeros((len(rows), d))
    n = int(seqlens[b])
    if n == 0:
        return out
    s = _params(d, scale)
    beta, g, keep, logg = _head_setup(b, n, q.shape[2], gate, tau, sink, bias, eps)
    cols = np.arange(n)
    live = rows < n
    r = rows[live]
    kh, vp = _as64(k[b, h, :n]), _vprime(_as64(v[b, h, :n]), g, cols)
    P = _P(_as64(q[b, h, r]), kh, r, cols, s, beta, logg, keep, causal)
    dS = (_as64(do[b, h, r]) @ vp.T) * P * (1.0 - P)
    if absolute:
        dS, kh = np.abs(dS), np.abs(kh)
    out[live] = s * (dS @ kh)
    return out


def dkdv_rows(q, k, v, do, seqlens, b, h, key_rows, causal=False, gate=None, tau=0.0,
              sink=DEFAULT_SINK, eps=GATE_EPS, scale=None, bias=None, absolute=False):
    """(dK[b, h, key_rows], dV[b, h, key_rows]) from all valid queries of (b, h).
    absolute=True: (s sum_i |dS_ij| |q_i|, g_j sum_i P_ij |dO_i|)."""
    key_rows = np.asarray(key_rows, dtype=np.int64)
    d = q.shape[-1]
    dk_out = np.zeros((len(key_rows), d))
    dv_out = np.zeros((len(key_rows), d))
    n = int(seqlens[b])
    if n == 0:
        return dk_out, dv_out
    s = _params(d, scale)
    beta, g, keep, logg = _head_setup(b, n, q.shape[2], gate, tau, sink, bias, eps)
    live = key_rows < n
    cols = key_rows[live]
    rows = np.arange(n)
    qh, doh = _as64(q[b, h, :n]), _as64(do[b, h, :n])
    kc, vc = _as64(k[b, h, cols]), _as64(v[b, h, cols])
    vpc = vc if g is None else vc * g[cols][:, None]
    P = _P(qh, kc, rows, cols, s, beta, logg, keep, causal)   # [n, len(cols)]
    dS = (doh @ vpc.T) * P * (1.0 - P)
    if absolute:
        dS, qh, doh = np.abs(dS), np.abs(qh), np.abs(doh)
    dk_out[live] = s * (dS.T @ qh)
    dvp = P.T @ doh
    dv_out[live] = dvp if g is None else dvp * g[cols][:, None]
    return dk_out, dv_out


# ----------------------------------------------------------------------------------
# gate gradient and row mass
# ----------------------------------------------------------------------------------

def gate_grad(q, k, v, do, seqlens, gate, causal=False, tau=0.0, sink=DEFAULT_SINK,
              eps=GATE_EPS, scale=None, bias=None, chunk=512, absolute=False):
    """Derivative of sum(dO * O) with respect to the per-key gate g[b, j].

    g_j enters twice ([KV-evict] gate paragraphs): x_ij += log(g_j + eps) and
    V'_j = g_j v_j. By the chain rule, per head h,
        dg_hj = sum_i dS_ij / (g_j + eps)  +  v_j . sum_i P_ij dO_i
    with dS_ij = (dO_i . V'_j) P_ij (1 - P_ij) as in the backward. The gate is shared by
    the heads, so dg_j = sum_h dg_hj.

    Returns (dg_head [B, H, L], dg [B, L]); padded and dropped keys give exactly 0.

    absolute=True returns the magnitude sums sum_i |dS_ij| / (g_j + eps) +
    sum_i P_ij |dO_i . v_j| instead, which bound how rounding of dS or P propagates.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    if gate is None:
        raise ValueError("gate_grad needs a gate")
    B, H, L, d = q.shape
    s = _params(d, scale)
    dg_head = np.zeros((B, H, L))
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:
            continue
        beta, g, keep, logg = _head_setup(b, n, L, gate, tau, sink, bias, eps)
        cols = np.arange(n)
        for h in range(H):
            kh, vh = k[b, h, :n], v[b, h, :n]
            vp = _vprime(vh, g, cols)
            sum_ds = np.zeros(n)          # sum_i dS_ij
            pdo = np.zeros((n, d))        # sum_i P_ij dO_i
            for r0 in range(0, n, chunk):
                rows = np.arange(r0, min(n, r0 + chunk))
                P = _P(q[b, h, rows], kh, rows, cols, s, beta, logg, keep, causal)
                dS = (do[b, h, rows] @ vp.T) * P * (1.0 - P)
                if absolute:
                    sum_ds += np.abs(dS).sum(axis=0)
                    pdo[:, 0] += np.sum(P * np.abs(do[b, h, rows] @ vh.T), axis=0)
                else:
                    sum_ds += dS.sum(axis=0)
                    pdo += P.T @ do[b, h, rows]
            if absolute:
                grad = sum_ds / (g[:n] + eps) + pdo[:, 0]
            else:
                grad = sum_ds / (g[:n] + eps) + np.einsum("jc,jc->j", vh, pdo)
            dg_head[b, h, :n] = np.where(keep[:n], grad, 0.0)
    return dg_head, dg_head.sum(axis=1)


def gate_grad_rows(q, k, v, do, seqlens, gate, b, h, key_rows, causal=False, tau=0.0,
                   sink=DEFAULT_SINK, eps=GATE_EPS, scale=None, bias=None):
    """dg_head[b, h, key_rows] (see gate_grad) from all valid queries of (b, h)."""
    key_rows = np.asarray(key_rows, dtype=np.int64)
    out = np.zeros(len(key_rows))
    n = int(seqlens[b])
    if n == 0:
        return out
    d = q.shape[-1]
    s = _params(d, scale)
    beta, g, keep, logg = _head_setup(b, n, q.shape[2], gate, tau, sink, bias, eps)
    live = key_rows < n
    cols = key_rows[live]
    rows = np.arange(n)
    qh, doh = _as64(q[b, h, :n]), _as64(do[b, h, :n])
    kc, vc = _as64(k[b, h, cols]), _as64(v[b, h, cols])
    P = _P(qh, kc, rows, cols, s, beta, logg, keep, causal)
    dS = (doh @ (vc * g[cols][:, None]).T) * P * (1.0 - P)
    grad = dS.sum(axis=0) / (g[cols] + eps) + np.einsum("jc,jc->j", vc, P.T @ doh)
    out[live] = np.where(keep[cols], grad, 0.0)
    return out


def row_mass(q, k, seqlens, causal=False, gate=None, tau=0.0, sink=DEFAULT_SINK,
             eps=GATE_EPS, scale=None, bias=None, chunk=512):
    """R[b, h, i] = sum_j P_ij over the allowed keys of query i ([KV-evict] row-sum
    diagnostic: under the sigmoid the row mass is free to vary with the query).
    Returns float64 [B, H, L]; rows i >= n_b are exactly 0."""
    q, k = _as64(q), _as64(k)
    B, H, L, d = q.shape
    s = _params(d, scale)
    R = np.zeros((B, H, L))
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:
            continue
        beta, g, keep, logg = _head_setup(b, n, L, gate, tau, sink, bias, eps)
        cols = np.arange(n)
        for h in range(H):
            for r0 in range(0, n, chunk):
                rows = np.arange(r0, min(n, r0 + chunk))
                P = _P(q[b, h, rows], k[b, h, :n], rows, cols, s, beta, logg, keep, causal)
                R[b, h, rows] = P.sum(axis=1)
    return R


# ----------------------------------------------------------------------------------
# packed batches with separate query and key lengths
# ----------------------------------------------------------------------------------

def _varlen_P(qb, kb, s, beta, logg, keep, causal, diag):
    """P[i, j] for one head of one packed sequence: keys kept, and (causal) j <= i + diag."""
    x = s * (qb @ kb.T) + beta + logg[None, :]
    allowed = np.broadcast_to(keep[None, :], x.shape).copy()
    if causal:
        i = np.arange(qb.shape[0])[:, None]
        j = np.arange(kb.shape[0])[None, :]
        allowed &= j <= i + diag
    P = np.zeros_like(x)
    P[allowed] = logistic(x[allowed])
    return P


def _varlen_seq(cu_q, cu_k, b, gate, tau, sink, eps, bias):
    q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
    nq, nk = q1 - q0, k1 - k0
    beta = (sequence_bias(nk) if nk > 0 else 0.0) if bias is None else float(bias[b])
    g = None if gate is None else np.asarray(gate, dtype=np.float64)[k0:k1]
    keep = kept_keys(nk, nk, g, tau, sink)
    logg = np.zeros(nk) if g is None else np.log(g + eps)
    return q0, q1, k0, k1, nk - nq, beta, g, keep, logg


def forward_varlen(q, k, v, cu_q, cu_k, causal=False, gate=None, tau=0.0, sink=DEFAULT_SINK,
                   eps=GATE_EPS, scale=None, bias=None):
    """O for packed sequences: q [Tq, H, d], k and v [Tk, H, d]; gate [Tk] or None.
    Rows outside the sequences are 0."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    H, d = q.shape[1], q.shape[2]
    s = _params(d, scale)
    O = np.zeros_like(q)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1, diag, beta, g, keep, logg = _varlen_seq(cu_q, cu_k, b, gate, tau, sink,
                                                                eps, bias)
        if q1 == q0:
            continue
        for h in range(H):
            vp = v[k0:k1, h] if g is None else v[k0:k1, h] * g[:, None]
            P = _varlen_P(q[q0:q1, h], k[k0:k1, h], s, beta, logg, keep, causal, diag)
            O[q0:q1, h] = P @ vp
    return O


def backward_varlen(q, k, v, do, cu_q, cu_k, causal=False, gate=None, tau=0.0,
                    sink=DEFAULT_SINK, eps=GATE_EPS, scale=None, bias=None):
    """(dQ, dK, dV) of sum(dO * O) for packed sequences (same layout as forward_varlen)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    H, d = q.shape[1], q.shape[2]
    s = _params(d, scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1, diag, beta, g, keep, logg = _varlen_seq(cu_q, cu_k, b, gate, tau, sink,
                                                                eps, bias)
        if q1 == q0 or k1 == k0:
            continue
        for h in range(H):
            kh = k[k0:k1, h]
            vp = v[k0:k1, h] if g is None else v[k0:k1, h] * g[:, None]
            P = _varlen_P(q[q0:q1, h], kh, s, beta, logg, keep, causal, diag)
            dS = (do[q0:q1, h] @ vp.T) * P * (1.0 - P)
            dq[q0:q1, h] = s * (dS @ kh)
            dk[k0:k1, h] = s * (dS.T @ q[q0:q1, h])
            dvp = P.T @ do[q0:q1, h]
            dv[k0:k1, h] = dvp if g is None else dvp * g[:, None]
    return dq, dk, dv


# ----------------------------------------------------------------------------------
# decode against a KV cache with threshold eviction
# ----------------------------------------------------------------------------------

def cache_compact(k, v, seqlens, cap, gate=None, tau=0.0, sink=DEFAULT_SINK):
    """Cache built from a prefill ([KV-evict]: entries with g_j < tau are removed after
    prefill, except the first `sink` positions): the kept keys of each sequence, in
    position order, in slots 0..count_b-1 of a cache of `cap` slots.

    k, v: [B, H, L, d]; gate: [B, L] or None (then every valid key is kept).
    Returns (Kc [B, H, cap, d], Vc, Gc [B, cap] or None, count [B], seen [B]) with unused
    slots 0 and seen_b = n_b (the number of positions written so far).
    """
    k, v = np.asarray(k), np.asarray(v)
    B, H, L, d = k.shape
    Kc, Vc = np.zeros((B, H, cap, d), k.dtype), np.zeros((B, H, cap, d), v.dtype)
    Gc = None if gate is None else np.zeros((B, cap), np.asarray(gate).dtype)
    count = np.zeros(B, np.int64)
    seen = np.asarray(seqlens, np.int64).copy()
    for b in range(B):
        n = int(seqlens[b])
        kept = np.nonzero(kept_keys(n, L, None if gate is None else gate[b], tau, sink))[0]
        if len(kept) > cap:
            raise ValueError("cache capacity exceeded")
        m = len(kept)
        Kc[b, :, :m] = k[b][:, kept]
        Vc[b, :, :m] = v[b][:, kept]
        if Gc is not None:
            Gc[b, :m] = gate[b][kept]
        count[b] = m
    return Kc, Vc, Gc, count, seen


def cache_append(Kc, Vc, Gc, count, seen, k_new, v_new, g_new=None, tau=0.0,
                 sink=DEFAULT_SINK):
    """One decode-time write ([KV-evict]: the threshold rule is applied to each newly
    written entry): the new token of sequence b sits at position seen_b; it is kept iff
    there is no gate, or seen_b < sink, or g_new_b >= tau. Kept entries go to slot
    count_b. Returns new (Kc, Vc, Gc, count, seen); the inputs are not modified.

    k_new, v_new: [B, H, d]; g_new: [B] or None.
    """
    Kc, Vc = Kc.copy(), Vc.copy()
    Gc = None if Gc is None else Gc.copy()
    count, seen = np.asarray(count).copy(), np.asarray(seen).copy()
    cap = Kc.shape[2]
    for b in range(Kc.shape[0]):
        keep = g_new is None or tau <= 0.0 or seen[b] < sink or g_new[b] >= tau
        if keep:
            if count[b] >= cap:
                raise ValueError("cache capacity exceeded")
            Kc[b, :, count[b]] = k_new[b]
            Vc[b, :, count[b]] = v_new[b]
            if Gc is not None:
                Gc[b, count[b]] = g_new[b]
            count[b] += 1
        seen[b] += 1
    return Kc, Vc, Gc, count, seen


def decode(q, Kc, Vc, Gc, count, bias, eps=GATE_EPS, scale=None):
    """One query per (b, h) against the live cache entries j < count_b:
        o = sum_j sigma(s q . k_j + beta_b [+ log(g_j + eps)]) [g_j] v_j
    (section 3 equation of [SA-bio] with the gate injection of [KV-evict]).
    q: [B, H, d]; bias: [B] (beta_b). Returns float64 [B, H, d]; count_b = 0 gives 0."""
    q = _as64(q)
    B, H, d = q.shape
    s = _params(d, scale)
    out = np.zeros((B, H, d))
    for b in range(B):
        m = int(count[b])
        if m == 0:
            continue
        x = s * np.einsum("hc,hjc->hj", q[b], _as64(Kc[b, :, :m])) + float(bias[b])
        vals = _as64(Vc[b, :, :m])
        if Gc is not None:
            g = _as64(Gc[b, :m])
            x = x + np.log(g + eps)[None, :]
            vals = vals * g[None, :, None]
        out[b] = np.einsum("hj,hjc->hc", logistic(x), vals)
    return out


# ----------------------------------------------------------------------------------
# naive scalar loops (tiny inputs only): a second, structurally different reading
# ----------------------------------------------------------------------------------

def _sig_scalar(x: float) -> float:
    if x >= 0.0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def forward_naive(q, k, v, seqlens, causal=False, gate=None, tau=0.0,
                  sink=DEFAULT_SINK, eps=GATE_EPS):
    """Triple loop over (query, key, feature) with scalar math; tiny inputs only."""
    B, H, L, d = np.shape(q)
    s = 1.0 / math.sqrt(d)
    O = np.zeros((B, H, L, d))
    for b in range(B):
        n = int(seqlens[b])
        for h in range(H):
            for i in range(n):
                for j in range(n):
                    if causal and j > i:
                        continue
                    gj = 1.0 if gate is None else float(gate[b][j])
                    if gate is not None and tau > 0.0 and j >= sink and gj < tau:
                        continue
                    dot = 0.0
                    for c in range(d):
                        dot += float(q[b][h][i][c]) * float(k[b][h][j][c])
                    x = s * dot - math.log(n)
                    if gate is not None:
                        x += math.log(gj + eps)
                    p = _sig_scalar(x)
                    for c in range(d):
                        O[b, h, i, c] += p * gj * float(v[b][h][j][c])
    return O


def backward_naive(q, k, v, do, seqlens, causal=False, gate=None, tau=0.0,
                   sink=DEFAULT_SINK, eps=GATE_EPS):
    """Scalar loops for dQ, dK, dV; tiny inputs only."""
    B, H, L, d = np.shape(q)
    s = 1.0 / math.sqrt(d)
    dq, dk, dv = np.zeros((B, H, L, d)), np.zeros((B, H, L, d)), np.zeros((B, H, L, d))
    for b in range(B):
        n = int(seqlens[b])
        for h in range(H):
            for i in range(n):
                for j in range(n):
                    if causal and j > i:
                        continue
                    gj = 1.0 if gate is None else float(gate[b][j])
                    if gate is not None and tau > 0.0 and j >= sink and gj < tau:
                        continue
                    dot = sum(float(q[b][h][i][c]) * float(k[b][h][j][c]) for c in range(d))
                    x = s * dot - math.log(n)
                    if gate is not None:
                        x += math.log(gj + eps)
                    p = _sig_scalar(x)
                    dpij = sum(float(do[b][h][i][c]) * gj * float(v[b][h][j][c])
                               for c in range(d))
                    dsij = dpij * p * (1.0 - p)
                    for c in range(d):
                        dq[b, h, i, c] += s * dsij * float(k[b][h][j][c])
                        dk[b, h, j, c] += s * dsij * float(q[b][h][i][c])
                        dv[b, h, j, c] += gj * p * float(do[b][h][i][c])
    return dq, dk, dv

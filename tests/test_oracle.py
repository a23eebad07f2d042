"""Pins for the fp64 oracle: facts that the pages and the mathematics fix.

Each test names the passage it follows. Together they are chosen so that a plausible
slip in the oracle (a wrong sign or argument of the bias, a wrong scale, a transposed
score matrix, a dropped sigma(1-sigma) factor, a wrong causal index, a missing gate
factor) fails at least one of them. None of them reads the GPU path.
"""

import ast
import json
import math
import operator
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------------
# hand-derived worked examples (tests/golden/worked_examples.json)
# ----------------------------------------------------------------------------------

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.USub: operator.neg, ast.UAdd: operator.pos}
_FUNCS = {"log": math.log, "log2": math.log2, "exp": math.exp}


def _eval(expr: str) -> float:
    """Evaluate a closed-form expression: numbers, + - * /, parentheses, log/log2/exp."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.left), ev(node.right))
        if isinstance(node, ast.UnaryOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.operand))
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
                and node.func.id in _FUNCS and len(node.args) == 1):
            return _FUNCS[node.func.id](ev(node.args[0]))
        raise ValueError(f"unsupported expression: {expr}")
    return ev(ast.parse(expr, mode="eval"))


def _tensor(rows, L, d):
    a = np.array([[_eval(x) for x in (r if isinstance(r, list) else [r])] for r in rows])
    return a.reshape(1, 1, L, d)


def _examples():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _examples(), ids=lambda e: e["name"])
def test_worked_examples(ex):
    """Forward and backward on hand-derived examples (definitions: §3 equation of the
    sigmoid-attention paper, b = -log n from its summary §2A, gate injection from the
    KV-eviction paper, backward from the diagonal Jacobian of appendix A.1.2)."""
    L, d, n = ex["L"], ex["d"], ex["n"]
    q, k, v, do = (_tensor(ex[t], L, d) for t in ("q", "k", "v", "do"))
    gate = None if ex["gate"] is None else np.array([[_eval(g) for g in ex["gate"]]])
    kw = dict(causal=ex["causal"], gate=gate)
    seqlens = [n]
    tol = ex.get("tol", 1e-13)
    want = {t: _tensor(ex[t], L, d) for t in ("O", "dQ", "dK", "dV")}
    for fwd, bwd in ((O.forward, O.backward), (O.forward_naive, O.backward_naive)):
        got_o = fwd(q, k, v, seqlens, **kw)
        dq, dk, dv = bwd(q, k, v, do, seqlens, **kw)
        for name, got in (("O", got_o), ("dQ", dq), ("dK", dk), ("dV", dv)):
            np.testing.assert_allclose(got, want[name], rtol=tol, atol=tol, err_msg=name)


# ----------------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 7, 100, 4096, 8192])
def test_sigma_of_bias_is_one_over_n_plus_one(n):
    """sigma(-ln n) = 1/(1+n) exactly (sigma and b from the summary page §2A)."""
    b = O.sequence_bias(n)
    assert O.logistic(np.array([b]))[0] == pytest.approx(1.0 / (n + 1), rel=1e-15)
    assert O.logistic_tanh(np.array([b]))[0] == pytest.approx(1.0 / (n + 1), rel=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_closed_form_qk_zero(causal):
    """Q = K = 0: every allowed logit is b = -ln n, so O_i = sum_{allowed j} V_j / (n+1)."""
    rng = np.random.default_rng(11)
    B, H, L, d = 3, 2, 40, 8
    seqlens = [40, 17, 1]
    z = np.zeros((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    out = O.forward(z, z, v, seqlens, causal=causal)
    for b, n in enumerate(seqlens):
        for i in range(L):
            if i >= n:
                want = np.zeros((H, d))
            else:
                hi = i + 1 if causal else n
                want = v[b, :, :hi].sum(axis=1) / (n + 1)
            np.testing.assert_allclose(out[b, :, i], want, rtol=1e-13, atol=1e-15)


def test_forward_closed_form_gated():
    """Q = K = 0 with a gate: P_ij = (g_j+eps)/(n+g_j+eps) and V'_j = g_j V_j."""
    rng = np.random.default_rng(12)
    B, H, L, d, n = 1, 2, 9, 4, 9
    g = rng.uniform(0.0, 1.0, (B, L))
    z = np.zeros((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    out = O.forward(z, z, v, [n], gate=g)
    eps = O.GATE_EPS
    p = (g[0] + eps) / (n + g[0] + eps)
    want = np.einsum("j,hjc->hc", p * g[0], v[0])
    for i in range(n):
        np.testing.assert_allclose(out[0, :, i], want, rtol=1e-12)


def test_backward_closed_form_k_zero():
    """K = 0: P = 1/(n+1), sigma' = n/(n+1)^2, so dQ = 0, dV_j = sum_i dO_i/(n+1) and
    dK_j = s n/(n+1)^2 sum_i (dO_i . v_j) q_i (appendix A.1.2 Jacobian)."""
    rng = np.random.default_rng(13)
    B, H, L, d = 2, 1, 12, 4
    seqlens = [12, 5]
    q = rng.standard_normal((B, H, L, d))
    k = np.zeros((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    do = rng.standard_normal((B, H, L, d))
    dq, dk, dv = O.backward(q, k, v, do, seqlens)
    s = 1.0 / math.sqrt(d)
    np.testing.assert_array_equal(dq, 0.0)
    for b, n in enumerate(seqlens):
        dv_want = do[b, 0, :n].sum(axis=0) / (n + 1)
        for j in range(n):
            np.testing.assert_allclose(dv[b, 0, j], dv_want, rtol=1e-12)
            coef = (do[b, 0, :n] @ v[b, 0, j]) * s * n / (n + 1) ** 2
            np.testing.assert_allclose(dk[b, 0, j], coef @ q[b, 0, :n], rtol=1e-12, atol=1e-14)
        assert np.all(dk[b, 0, n:] == 0) and np.all(dv[b, 0, n:] == 0)


# ----------------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------------

def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def test_padding_contributes_exactly_zero():
    """Padded keys contribute nothing and padded rows are zero, whatever padded slots
    hold (block-sparse padding, §4 of the sigmoid-attention paper; removed positions
    masked and zeroed, KV-eviction removal probe)."""
    B, H, L, d = 2, 2, 16, 8
    seqlens = [11, 16]
    q, k, v, do = (_rand((B, H, L, d), s) for s in range(4))
    clean = O.forward(q, k, v, seqlens), O.backward(q, k, v, do, seqlens)
    qp, kp, vp, dop = (t.copy() for t in (q, k, v, do))
    for t in (qp, kp, vp, dop):
        t[0, :, 11:] = np.nan
    pois = O.forward(qp, kp, vp, seqlens), O.backward(qp, kp, vp, dop, seqlens)
    np.testing.assert_array_equal(clean[0], pois[0])
    for a, b in zip(clean[1], pois[1]):
        np.testing.assert_array_equal(a, b)
    assert np.all(pois[0][0, :, 11:] == 0)
    for g in pois[1]:
        assert np.all(g[0, :, 11:] == 0)


def test_sigma_prime_bounded_by_quarter():
    """max sigma(1-sigma) = 1/4 at x = 0 (§3 of the sigmoid-attention paper). Probed
    through the public backward on one pair with d = 1: dK = sigma'(k) when q = v = dO = 1
    and n = 1 (b = 0)."""
    ks = np.concatenate([np.linspace(-40, 40, 801), [0.0]])
    vals = []
    for kk in ks:
        one = np.ones((1, 1, 1, 1))
        _, dk, _ = O.backward(one, np.full((1, 1, 1, 1), kk), one, one, [1])
        vals.append(dk[0, 0, 0, 0])
    vals = np.array(vals)
    assert np.all(vals <= 0.25 + 1e-16) and np.all(vals >= 0)
    assert vals[-1] == 0.25


def test_diagonal_jacobian_rank_one_update():
    """Changing a single key k_j changes only column j of P (appendix A.1.2: the
    Jacobian of sigma is diagonal), so O changes by a rank-one a v_j^T."""
    B, H, L, d, n, j = 1, 1, 10, 6, 10, 4
    q, k, v = (_rand((B, H, L, d), s) for s in (20, 21, 22))
    base = O.forward(q, k, v, [n])
    k2 = k.copy()
    k2[0, 0, j] += _rand(d, 23)
    diff = O.forward(q, k2, v, [n])[0, 0] - base[0, 0]
    vj = v[0, 0, j]
    a = diff @ vj / (vj @ vj)
    np.testing.assert_allclose(diff, np.outer(a, vj), atol=1e-13)
    assert np.linalg.matrix_rank(diff, tol=1e-10) == 1


@pytest.mark.parametrize("variant", ["bidir", "causal", "gated"])
def test_finite_differences(variant):
    """Central differences of L = <dO, O> match the analytic gradients (fp64, tiny)."""
    B, H, L, d = 2, 1, 8, 4
    seqlens = [8, 5]
    q, k, v, do = (_rand((B, H, L, d), 30 + s) for s in range(4))
    kw = {}
    if variant == "causal":
        kw["causal"] = True
    if variant == "gated":
        kw["gate"] = np.random.default_rng(40).uniform(0.05, 1.0, (B, L))
    dq, dk, dv = O.backward(q, k, v, do, seqlens, **kw)

    def loss(qq, kk, vv):
        return float(np.sum(do * O.forward(qq, kk, vv, seqlens, **kw)))

    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{a + a: b for a, b in args_p.items()}) -
                        loss(**{a + a: b for a, b in args_m.items()})) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("gated", [False, True])
def test_adjoint_identities(gated):
    """<dO,O> = <dV,V> and <dQ,Q> = <dK,K> (both sides equal sum dS * scaled scores)."""
    B, H, L, d = 2, 3, 20, 8
    seqlens = [20, 13]
    q, k, v, do = (_rand((B, H, L, d), 50 + s) for s in range(4))
    gate = np.random.default_rng(60).uniform(0.1, 1.0, (B, L)) if gated else None
    out = O.forward(q, k, v, seqlens, gate=gate)
    dq, dk, dv = O.backward(q, k, v, do, seqlens, gate=gate)
    assert np.sum(do * out) == pytest.approx(np.sum(dv * v), rel=1e-12)
    assert np.sum(dq * q) == pytest.approx(np.sum(dk * k), rel=1e-12)


def test_permutation_equivariance():
    """Bidirectional: the bias is position-free and sigma acts element-wise, so
    permuting the valid tokens permutes O, dQ, dK, dV the same way."""
    B, H, L, d = 1, 2, 12, 8
    n = 10
    q, k, v, do = (_rand((B, H, L, d), 70 + s) for s in range(4))
    perm = np.concatenate([np.random.default_rng(80).permutation(n), np.arange(n, L)])
    o1 = O.forward(q, k, v, [n])
    g1 = O.backward(q, k, v, do, [n])
    pq, pk, pv, pdo = (t[:, :, perm] for t in (q, k, v, do))
    o2 = O.forward(pq, pk, pv, [n])
    g2 = O.backward(pq, pk, pv, pdo, [n])
    np.testing.assert_allclose(o2, o1[:, :, perm], rtol=1e-12, atol=1e-14)
    for a, b in zip(g2, g1):
        np.testing.assert_allclose(a, b[:, :, perm], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("variant", ["bidir", "causal", "gated_drop"])
def test_naive_loops_match_vectorised(variant):
    """The scalar triple loop and the vectorised oracle agree to 1e-12."""
    B, H, L, d = 2, 2, 9, 5
    seqlens = [9, 6]
    q, k, v, do = (_rand((B, H, L, d), 90 + s) for s in range(4))
    kw = {}
    if variant == "causal":
        kw["causal"] = True
    if variant == "gated_drop":
        g = np.random.default_rng(99).uniform(0.0, 1.0, (B, L))
        g[:, 5] = 0.01
        g[:, 1] = 0.01   # inside the sink: kept
        kw.update(gate=g, tau=0.05, sink=4, causal=True)
    a = O.forward(q, k, v, seqlens, **kw)
    b = O.forward_naive(q, k, v, seqlens, **kw)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    for x, y in zip(O.backward(q, k, v, do, seqlens, **kw),
                    O.backward_naive(q, k, v, do, seqlens, **kw)):
        np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-13)


def test_zero_gate_equals_hard_drop():
    """g_j -> 0 drives key j's contribution to zero through both channels, matching
    hard deletion (KV-eviction paper, gate paragraph)."""
    B, H, L, d, n, j = 1, 2, 10, 6, 10, 7
    q, k, v, do = (_rand((B, H, L, d), 100 + s) for s in range(4))
    g = np.random.default_rng(105).uniform(0.2, 1.0, (B, L))
    g_zero = g.copy()
    g_zero[0, j] = 0.0                   # kept (tau = 0) but zero
    g_drop = g.copy()
    g_drop[0, j] = 0.01                  # dropped: j >= sink and g < tau
    a = O.forward(q, k, v, [n], gate=g_zero)
    b = O.forward(q, k, v, [n], gate=g_drop, tau=0.05, sink=4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)
    ga = O.backward(q, k, v, do, [n], gate=g_zero)
    gb = O.backward(q, k, v, do, [n], gate=g_drop, tau=0.05, sink=4)
    for x, y in zip(ga, gb):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-14)
    assert np.all(gb[1][0, :, j] == 0) and np.all(gb[2][0, :, j] == 0)


def test_unit_gate_equals_ungated():
    """g = 1 shifts each logit by log(1 + 1e-8) only: matches the ungated result to ~1e-8."""
    B, H, L, d = 1, 2, 10, 6
    q, k, v, do = (_rand((B, H, L, d), 110 + s) for s in range(4))
    ones = np.ones((B, L))
    a = O.forward(q, k, v, [10], gate=ones)
    b = O.forward(q, k, v, [10])
    # each P changes by at most a relative 1e-8, so |dO_i| <= 1e-8 sum_j |V_j|
    bound = 1.01e-8 * np.abs(v).sum(axis=2, keepdims=True)
    assert np.all(np.abs(a - b) <= bound)
    assert np.any(a != b)


def test_sink_positions_never_dropped():
    """Keys j < sink are kept whatever their gate (the first four positions excluded)."""
    keep = O.kept_keys(10, 12, gate=np.full(12, 0.001), tau=0.05, sink=4)
    assert keep.tolist() == [True] * 4 + [False] * 8


def test_large_logits_finite():
    """Q, K ~ N(0, 16) at d = 64 give logits of size ~80: no NaN/Inf, P in [0, 1]."""
    B, H, L, d = 1, 1, 64, 64
    q, k = _rand((B, H, L, d), 120, 4.0), _rand((B, H, L, d), 121, 4.0)
    v, do = _rand((B, H, L, d), 122), _rand((B, H, L, d), 123)
    out = O.forward(q, k, v, [L])
    assert np.all(np.isfinite(out))
    assert np.all(np.abs(out) <= np.abs(v[0, 0]).sum(axis=0) + 1e-9)
    for g in O.backward(q, k, v, do, [L]):
        assert np.all(np.isfinite(g))


def test_causality():
    """Under the causal rule, changing K or V at positions > i leaves O_i unchanged."""
    B, H, L, d, i = 1, 1, 16, 8, 6
    q, k, v = (_rand((B, H, L, d), 130 + s) for s in range(3))
    a = O.forward(q, k, v, [L], causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, i + 1:] += 5.0
    v2[0, 0, i + 1:] -= 3.0
    b = O.forward(q, k2, v2, [L], causal=True)
    np.testing.assert_array_equal(a[0, 0, : i + 1], b[0, 0, : i + 1])
    assert not np.allclose(a[0, 0, i + 1:], b[0, 0, i + 1:])


def test_tanh_form_identity():
    """The tanh form of the sigmoid-attention paper's §4 equals 1/(1+e^-x)."""
    x = np.linspace(-60, 60, 10001)
    np.testing.assert_allclose(O.logistic(x), O.logistic_tanh(x), rtol=0, atol=1e-15)


def test_empty_sequence_and_single_token():
    """n = 0 gives all-zero outputs; n = 1 uses b = 0."""
    B, H, L, d = 2, 1, 4, 2
    q, k, v, do = (_rand((B, H, L, d), 140 + s) for s in range(4))
    out = O.forward(q, k, v, [0, 1])
    assert np.all(out[0] == 0)
    x = q[1, 0, 0] @ k[1, 0, 0] / math.sqrt(d)
    np.testing.assert_allclose(out[1, 0, 0], v[1, 0, 0] / (1 + math.exp(-x)), rtol=1e-14)
    assert O.sequence_bias(1) == 0.0
    for g in O.backward(q, k, v, do, [0, 1]):
        assert np.all(g[0] == 0)


def test_sampled_rows_match_full():
    """The row-sampled entry points agree with the full oracle."""
    B, H, L, d = 2, 2, 24, 8
    seqlens = [24, 15]
    q, k, v, do = (_rand((B, H, L, d), 150 + s) for s in range(4))
    g = np.random.default_rng(160).uniform(0.0, 1.0, (B, L))
    kw = dict(causal=True, gate=g, tau=0.3, sink=4)
    full_o = O.forward(q, k, v, seqlens, **kw)
    fdq, fdk, fdv = O.backward(q, k, v, do, seqlens, **kw)
    rows = np.array([0, 3, 14, 15, 23])
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(O.forward_rows(q, k, v, seqlens, b, h, rows, **kw),
                                       full_o[b, h, rows], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(O.dq_rows(q, k, v, do, seqlens, b, h, rows, **kw),
                                       fdq[b, h, rows], rtol=1e-12, atol=1e-14)
            dk, dv = O.dkdv_rows(q, k, v, do, seqlens, b, h, rows, **kw)
            np.testing.assert_allclose(dk, fdk[b, h, rows], rtol=1e-11, atol=1e-14)
            np.testing.assert_allclose(dv, fdv[b, h, rows], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------------
# workloads and FLOP counts
# ----------------------------------------------------------------------------------

def test_flop_counts():
    """4 d per valid pair forward (two matmuls of 2 d), 2.5x that backward."""
    assert W.flops_forward([2], 1, 1, False) == 16.0
    assert W.flops_forward([2], 1, 1, True) == 12.0
    assert W.flops_forward([3, 0], 2, 64, False) == 4 * 64 * 2 * 9
    assert W.flops_backward([2], 1, 1, False) == 40.0


def test_bf16_rounding_matches_torch():
    """The generator's bf16 rounding agrees with torch's own float32 -> bfloat16 cast."""
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(170).standard_normal(200000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0]
    ours = W.round_to_bf16(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, theirs)


@pytest.mark.parametrize("name,mean", [("pad_sweep_25", 3072.0), ("pad_sweep_50", 2048.0)])
def test_padding_sweep_lengths(name, mean):
    w = W.get(name, H=1, d=8)
    n = W.generate(w, with_do=False)["seqlens"]
    assert n.mean() == mean and n.min() >= 1 and n.max() <= 4096


def test_generator_is_seeded():
    a = W.generate(W.get("bidir_2k", B=2, H=1, L=64))
    b = W.generate(W.get("bidir_2k", B=2, H=1, L=64))
    for t in ("q", "k", "v", "do", "seqlens"):
        np.testing.assert_array_equal(a[t], b[t])


def test_absolute_sums():
    """The magnitude sums equal the outputs for non-negative inputs (then every term is
    non-negative) and bound them otherwise."""
    B, H, L, d = 2, 2, 12, 4
    seqlens = [12, 7]
    rng = np.random.default_rng(180)
    q, k, v, do = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    g = rng.uniform(0.1, 1.0, (B, L))
    pos = [np.abs(t) for t in (q, k, v, do)]
    for kw in (dict(), dict(gate=g, causal=True)):
        plain = O.backward(*pos, seqlens, **kw)
        mag = O.backward(*pos, seqlens, absolute=True, **kw)
        for a, b in zip(plain, mag):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
        signed = O.backward(q, k, v, do, seqlens, **kw)
        mags = O.backward(q, k, v, do, seqlens, absolute=True, **kw)
        for a, m in zip(signed, mags):
            assert np.all(np.abs(a) <= m + 1e-12)
        rows = np.arange(L)
        for b in range(B):
            for h in range(H):
                np.testing.assert_allclose(O.dq_rows(q, k, v, do, seqlens, b, h, rows, absolute=True, **kw),
                                           mags[0][b, h], rtol=1e-12, atol=1e-15)
                dk, dv = O.dkdv_rows(q, k, v, do, seqlens, b, h, rows, absolute=True, **kw)
                np.testing.assert_allclose(dk, mags[1][b, h], rtol=1e-11, atol=1e-15)
                np.testing.assert_allclose(dv, mags[2][b, h], rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------------
# gate gradient and row mass
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["bidir", "causal", "drop"])
def test_gate_grad_finite_differences(variant):
    """Central differences of L = <dO, O> with respect to the shared gate g[b, j] match
    dg = sum_h dg_h (gate injection of the KV-eviction paper: log g on the logits, g on
    the values). Several heads, so the head sum is exercised; in the drop variant some
    gates sit far below tau, where the loss does not depend on them (derivative 0)."""
    B, H, L, d = 2, 3, 8, 4
    seqlens = [8, 6]
    q, k, v, do = (_rand((B, H, L, d), 50 + s) for s in range(4))
    g = np.random.default_rng(60).uniform(0.2, 1.0, (B, L))
    kw = dict(gate=g)
    if variant == "causal":
        kw["causal"] = True
    if variant == "drop":
        g[0, 5] = g[1, 2] = 0.01
        kw.update(tau=0.05, sink=1, causal=True)
    dg_head, dg = O.gate_grad(q, k, v, do, seqlens, **kw)
    np.testing.assert_allclose(dg, dg_head.sum(axis=1), rtol=1e-14, atol=0)

    def loss(gg):
        kk = dict(kw, gate=gg)
        return float(np.sum(do * O.forward(q, k, v, seqlens, **kk)))

    h = 1e-6
    num = np.zeros_like(g)
    for idx in np.ndindex(g.shape):
        gp, gm = g.copy(), g.copy()
        gp[idx] += h
        gm[idx] -= h
        num[idx] = (loss(gp) - loss(gm)) / (2 * h)
    np.testing.assert_allclose(dg, num, rtol=1e-6, atol=1e-8)
    if variant == "drop":
        assert dg[0, 5] == 0.0 and dg[1, 2] == 0.0
        assert np.all(dg_head[:, :, 5][0] == 0.0)
    for b, n in enumerate(seqlens):
        assert np.all(dg_head[b, :, n:] == 0.0)


def test_gate_grad_scaling_identity():
    """With eps = 0, scaling every gate by lam equals adding ln(lam) to the bias and
    scaling O by lam, so L(lam g) = lam L_{beta + ln lam}(g). Differentiating at lam = 1:
    sum_j g_j dg_j = L + dL/dbeta, where dL/dbeta is taken by central differences of the
    forward in the bias (an independent route to the same number)."""
    B, H, L, d = 2, 2, 10, 4
    seqlens = [10, 7]
    q, k, v, do = (_rand((B, H, L, d), 70 + s) for s in range(4))
    g = np.random.default_rng(80).uniform(0.1, 1.0, (B, L))
    kw = dict(gate=g, eps=0.0)
    for causal in (False, True):
        _, dg = O.gate_grad(q, k, v, do, seqlens, causal=causal, **kw)
        for b, n in enumerate(seqlens):
            beta = np.array([O.sequence_bias(m) for m in seqlens])

            def loss(bb):
                o = O.forward(q, k, v, seqlens, causal=causal, bias=bb, **kw)
                return float(np.sum(do[b] * o[b]))

            h = 1e-6
            bp, bm = beta.copy(), beta.copy()
            bp[b] += h
            bm[b] -= h
            dbeta = (loss(bp) - loss(bm)) / (2 * h)
            lhs = float(np.sum(g[b, :n] * dg[b, :n]))
            assert lhs == pytest.approx(loss(beta) + dbeta, rel=1e-7, abs=1e-9)


@pytest.mark.parametrize("causal", [False, True])
def test_gate_grad_closed_form_qk_zero(causal):
    """Q = K = 0: every P_ij = p_j = (g_j+eps)/(n+g_j+eps), so for each head
    dg_j = (sum over allowed i of dO_i) . v_j * (p_j + g_j p_j (1-p_j)/(g_j+eps))."""
    rng = np.random.default_rng(14)
    B, H, L, d, n = 1, 2, 9, 4, 8
    g = rng.uniform(0.05, 1.0, (B, L))
    z = np.zeros((B, H, L, d))
    v, do = rng.standard_normal((B, H, L, d)), rng.standard_normal((B, H, L, d))
    eps = O.GATE_EPS
    dg_head, _ = O.gate_grad(z, z, v, do, [n], gate=g, causal=causal)
    p = (g[0] + eps) / (n + g[0] + eps)
    for h in range(H):
        for j in range(L):
            if j >= n:
                assert dg_head[0, h, j] == 0.0
                continue
            lo = j if causal else 0
            sdo = do[0, h, lo:n].sum(axis=0)
            want = float(sdo @ v[0, h, j]) * (p[j] + g[0, j] * p[j] * (1 - p[j]) / (g[0, j] + eps))
            assert dg_head[0, h, j] == pytest.approx(want, rel=1e-12, abs=1e-14)


def test_gate_grad_rows_match_full():
    B, H, L, d = 2, 2, 33, 8
    seqlens = [33, 20]
    q, k, v, do = (_rand((B, H, L, d), 90 + s) for s in range(4))
    g = np.random.default_rng(95).uniform(0.0, 1.0, (B, L))
    for kw in (dict(), dict(causal=True, tau=0.3, sink=4)):
        dg_head, _ = O.gate_grad(q, k, v, do, seqlens, gate=g, chunk=7, **kw)
        rows = np.array([0, 3, 19, 20, 32])
        for b in range(B):
            for h in range(H):
                got = O.gate_grad_rows(q, k, v, do, seqlens, g, b, h, rows, **kw)
                np.testing.assert_allclose(got, dg_head[b, h, rows], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_row_mass_closed_form_qk_zero(causal):
    """Q = K = 0: each allowed weight is sigma(-ln n) = 1/(n+1), so the row mass is
    n/(n+1) (bidirectional) or (i+1)/(n+1) (causal); with a gate it is
    sum over allowed kept j of (g_j+eps)/(n+g_j+eps)."""
    B, H, L, d = 2, 2, 12, 4
    seqlens = [12, 5]
    z = np.zeros((B, H, L, d))
    R = O.row_mass(z, z, seqlens, causal=causal)
    g = np.random.default_rng(15).uniform(0.0, 1.0, (B, L))
    Rg = O.row_mass(z, z, seqlens, causal=causal, gate=g, tau=0.3, sink=2)
    eps = O.GATE_EPS
    for b, n in enumerate(seqlens):
        keep = O.kept_keys(n, L, g[b], 0.3, 2)
        for i in range(L):
            if i >= n:
                assert np.all(R[b, :, i] == 0.0) and np.all(Rg[b, :, i] == 0.0)
                continue
            hi = i + 1 if causal else n
            np.testing.assert_allclose(R[b, :, i], hi / (n + 1), rtol=1e-14)
            js = [j for j in range(hi) if keep[j]]
            want = sum((g[b, j] + eps) / (n + g[b, j] + eps) for j in js)
            np.testing.assert_allclose(Rg[b, :, i], want, rtol=1e-13)


def test_row_mass_is_forward_with_unit_values():
    """Ungated, the row mass is the output for V = 1 in every feature."""
    B, H, L, d = 2, 2, 20, 8
    seqlens = [20, 9]
    q, k = _rand((B, H, L, d), 100), _rand((B, H, L, d), 101)
    for causal in (False, True):
        R = O.row_mass(q, k, seqlens, causal=causal, chunk=6)
        o = O.forward(q, k, np.ones((B, H, L, d)), seqlens, causal=causal)
        for c in range(d):
            np.testing.assert_allclose(R, o[..., c], rtol=1e-13, atol=0)


def test_gate_grad_absolute_sums():
    """The magnitude sums of the gate gradient equal it when every term is non-negative
    and bound it otherwise."""
    B, H, L, d = 2, 2, 12, 4
    seqlens = [12, 7]
    rng = np.random.default_rng(181)
    q, k, v, do = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    g = rng.uniform(0.1, 1.0, (B, L))
    # dO . v_j >= 0 and sigma' > 0 make every term non-negative
    pos = [np.abs(t) for t in (q, k, v, do)]
    a, _ = O.gate_grad(*pos, seqlens, g, causal=True)
    m, _ = O.gate_grad(*pos, seqlens, g, causal=True, absolute=True)
    np.testing.assert_allclose(a, m, rtol=1e-12, atol=1e-15)
    a, _ = O.gate_grad(q, k, v, do, seqlens, g)
    m, _ = O.gate_grad(q, k, v, do, seqlens, g, absolute=True)
    assert np.all(np.abs(a) <= m + 1e-12)


# ----------------------------------------------------------------------------------
# decode against a KV cache with threshold eviction
# ----------------------------------------------------------------------------------

def _decode_case(seed, B=3, H=2, L=24, d=8):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    g = rng.uniform(0.0, 1.0, (B, L))
    g[:, 7] = 0.01                      # a dropped key at a fixed position
    g[:, 1] = 0.02                      # below tau but inside the sink: kept
    return q, k, v, g


@pytest.mark.parametrize("gated", [False, True])
def test_decode_matches_causal_forward_rows(gated):
    """Decoding query i against the cache of tokens 0..i (prefill compaction of the first
    p tokens, then one append per token) gives row i of the causal forward with hard
    dropping, at the sequence's bias: the eviction rule of the KV-eviction paper applied
    at prefill and to each newly written entry."""
    q, k, v, g = _decode_case(120)
    B, H, L, d = q.shape
    tau, sink = (0.3, 4) if gated else (0.0, 4)
    gate = g if gated else None
    seqlens = [L] * B
    bias = np.array([O.sequence_bias(L)] * B)
    ref = O.forward(q, k, v, seqlens, causal=True, gate=gate, tau=tau, sink=sink, bias=bias)
    p = 9
    state = O.cache_compact(k[:, :, :p], v[:, :, :p], [p] * B, L, gate=None if gate is None else gate[:, :p],
                            tau=tau, sink=sink)
    for i in range(L):
        if i >= p:
            state = O.cache_append(*state, k[:, :, i], v[:, :, i],
                                   None if gate is None else gate[:, i], tau=tau, sink=sink)
        if i < p - 1:
            # the cache of tokens 0..i, built by compaction of the prefix
            st = O.cache_compact(k[:, :, :i + 1], v[:, :, :i + 1], [i + 1] * B, L,
                                 gate=None if gate is None else gate[:, :i + 1], tau=tau, sink=sink)
        else:
            st = state
        Kc, Vc, Gc, count, seen = st
        assert np.all(seen == i + 1)
        got = O.decode(q[:, :, i], Kc, Vc, Gc, count, bias)
        np.testing.assert_allclose(got, ref[:, :, i], rtol=1e-12, atol=1e-14)


def test_cache_appends_equal_compaction():
    """Appending tokens one by one gives exactly the cache compaction of the whole
    prefill (same slots, same values, same counts)."""
    q, k, v, g = _decode_case(121)
    B, H, L, d = k.shape
    lens = [24, 10, 0]
    full = O.cache_compact(k, v, lens, 32, gate=g, tau=0.3, sink=4)
    st = O.cache_compact(k[:, :, :0], v[:, :, :0], [0] * B, 32, gate=g[:, :0], tau=0.3, sink=4)
    for i in range(L):
        nxt = O.cache_append(*st, k[:, :, i], v[:, :, i], g[:, i], tau=0.3, sink=4)
        # sequences shorter than i + 1 tokens do not advance
        keep_b = np.array([i < n for n in lens])
        st = tuple(np.where(keep_b.reshape((-1,) + (1,) * (a.ndim - 1)), a, b_)
                   if a is not None else None for a, b_ in zip(nxt, st))
    for a, b_ in zip(st, full):
        np.testing.assert_array_equal(a, b_)
    kept0 = [j for j in range(24) if j < 4 or g[0, j] >= 0.3]
    assert full[3][0] == len(kept0)
    np.testing.assert_array_equal(full[0][0, :, :len(kept0)], k[0][:, kept0])


def test_decode_closed_form_q_zero():
    """q = 0: every logit is beta + log(g_j + eps); with beta = -ln n the weight is
    (g_j + eps) / (n + g_j + eps), so o = sum_j g_j (g_j+eps)/(n+g_j+eps) v_j."""
    rng = np.random.default_rng(122)
    B, H, C, d = 2, 3, 10, 4
    Kc, Vc = rng.standard_normal((B, H, C, d)), rng.standard_normal((B, H, C, d))
    Gc = rng.uniform(0.05, 1.0, (B, C))
    count = np.array([10, 6])
    n = 40
    out = O.decode(np.zeros((B, H, d)), Kc, Vc, Gc, count, [-math.log(n)] * B)
    eps = O.GATE_EPS
    for b in range(B):
        m = count[b]
        w = Gc[b, :m] * (Gc[b, :m] + eps) / (n + Gc[b, :m] + eps)
        np.testing.assert_allclose(out[b], np.einsum("j,hjc->hc", w, Vc[b, :, :m]), rtol=1e-12)
    assert np.all(O.decode(np.zeros((B, H, d)), Kc, Vc, Gc, np.array([0, 0]), [0.0, 0.0]) == 0)


# ----------------------------------------------------------------------------------
# packed batches with separate query and key lengths
# ----------------------------------------------------------------------------------

def _pack(x, lens):
    """[B, H, L, d] padded -> [sum(lens), H, d] packed."""
    return np.concatenate([x[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)], axis=0)


@pytest.mark.parametrize("variant", ["bidir", "causal", "gated"])
def test_varlen_equal_lengths_is_the_padded_definition(variant):
    """With nq = nk the packed functions are the padded ones on the same rows."""
    B, H, L, d = 3, 2, 17, 4
    lens = [17, 5, 0]
    q, k, v, do = (_rand((B, H, L, d), 140 + s) for s in range(4))
    kw = {}
    g = np.random.default_rng(145).uniform(0.0, 1.0, (B, L))
    if variant == "causal":
        kw["causal"] = True
    if variant == "gated":
        kw.update(gate=g, tau=0.3, sink=2, causal=True)
    cu = np.concatenate([[0], np.cumsum(lens)])
    o = O.forward(q, k, v, lens, **kw)
    grads = O.backward(q, k, v, do, lens, **kw)
    kwv = dict(kw)
    if "gate" in kwv:
        kwv["gate"] = np.concatenate([g[b, :n] for b, n in enumerate(lens)])
    ov = O.forward_varlen(_pack(q, lens), _pack(k, lens), _pack(v, lens), cu, cu, **kwv)
    gv = O.backward_varlen(_pack(q, lens), _pack(k, lens), _pack(v, lens), _pack(do, lens),
                           cu, cu, **kwv)
    np.testing.assert_allclose(ov, _pack(o, lens), rtol=1e-13, atol=1e-15)
    for a, b_ in zip(gv, grads):
        np.testing.assert_allclose(a, _pack(b_, lens), rtol=1e-12, atol=1e-14)


def test_varlen_query_shards_reassemble_the_causal_sequence():
    """A causal sequence of N tokens split into query shards: the shard of rows s..s+m-1,
    given keys 0..s+m-1 and the sequence's bias, reproduces those rows of O and dQ, and
    the shards' dK and dV add up to the full ones (their sums over query rows split)."""
    N, H, d, m = 24, 2, 4, 8
    rng = np.random.default_rng(150)
    q, k, v, do = (rng.standard_normal((1, H, N, d)) for _ in range(4))
    bias = [O.sequence_bias(N)]
    o = O.forward(q, k, v, [N], causal=True, bias=bias)
    dq, dk, dv = O.backward(q, k, v, do, [N], causal=True, bias=bias)
    dk_sum, dv_sum = np.zeros((N, H, d)), np.zeros((N, H, d))
    for s0 in range(0, N, m):
        qs = q[0, :, s0:s0 + m].transpose(1, 0, 2)
        dos = do[0, :, s0:s0 + m].transpose(1, 0, 2)
        ks = k[0, :, :s0 + m].transpose(1, 0, 2)
        vs = v[0, :, :s0 + m].transpose(1, 0, 2)
        cu_q, cu_k = np.array([0, m]), np.array([0, s0 + m])
        os_ = O.forward_varlen(qs, ks, vs, cu_q, cu_k, causal=True, bias=bias)
        np.testing.assert_allclose(os_, o[0, :, s0:s0 + m].transpose(1, 0, 2), rtol=1e-12, atol=1e-15)
        gq, gk, gv = O.backward_varlen(qs, ks, vs, dos, cu_q, cu_k, causal=True, bias=bias)
        np.testing.assert_allclose(gq, dq[0, :, s0:s0 + m].transpose(1, 0, 2), rtol=1e-11, atol=1e-14)
        dk_sum[:s0 + m] += gk
        dv_sum[:s0 + m] += gv
    np.testing.assert_allclose(dk_sum, dk[0].transpose(1, 0, 2), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dv_sum, dv[0].transpose(1, 0, 2), rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_finite_differences(causal):
    """nq != nk (including a sequence with more queries than keys): central differences
    of <dO, O> match the packed backward."""
    H, d = 1, 3
    cu_q, cu_k = np.array([0, 3, 8]), np.array([0, 5, 7])
    rng = np.random.default_rng(160)
    q, do = rng.standard_normal((8, H, d)), rng.standard_normal((8, H, d))
    k, v = rng.standard_normal((7, H, d)), rng.standard_normal((7, H, d))
    g = rng.uniform(0.2, 1.0, 7)
    kw = dict(causal=causal, gate=g)
    grads = O.backward_varlen(q, k, v, do, cu_q, cu_k, **kw)

    def loss(qq, kk, vv):
        return float(np.sum(do * O.forward_varlen(qq, kk, vv, cu_q, cu_k, **kw)))

    h = 1e-6
    for idx_t, (x, gx) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[idx_t], args_m[idx_t] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(gx, num, rtol=1e-6, atol=1e-8)
    if causal:
        # sequence 1 has 5 queries and 2 keys: its first 3 queries see no key
        o = O.forward_varlen(q, k, v, cu_q, cu_k, **kw)
        assert np.all(o[3:6] == 0.0) and np.any(o[6:8] != 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_closed_form_qk_zero(causal):
    """Q = K = 0 with nq != nk: every allowed weight is sigma(-ln nk) = 1/(nk + 1), so
    O_i = sum over allowed keys of v_j / (nk + 1), the allowed keys being all nk of them,
    or (causal, bottom right) j <= i + nk - nq."""
    H, d = 2, 3
    cu_q, cu_k = np.array([0, 4, 4, 10]), np.array([0, 9, 12, 14])
    rng = np.random.default_rng(170)
    q, k = np.zeros((10, H, d)), np.zeros((14, H, d))
    v = rng.standard_normal((14, H, d))
    o = O.forward_varlen(q, k, v, cu_q, cu_k, causal=causal)
    for b in range(3):
        nq, nk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for i in range(nq):
            hi = min(nk, i + nk - nq + 1) if causal else nk
            want = v[cu_k[b]:cu_k[b] + max(hi, 0)].sum(axis=0) / (nk + 1)
            np.testing.assert_allclose(o[cu_q[b] + i], want, rtol=1e-13, atol=1e-15)

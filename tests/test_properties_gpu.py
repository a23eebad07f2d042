"""Properties of the HIP path that the pages fix, checked on the GPU:
padded slots are never read (poison leaves valid outputs bitwise unchanged), results
are deterministic, the Q = K = 0 and K = 0 closed forms, causality, permutation
equivariance of the queries, and zero gate = hard drop."""

import numpy as np
import pytest

import workloads as W
from gpu_util import need_gpu, note, run_gpu

pytestmark = pytest.mark.gpu


def _small(name="p", d=64, lengths=(600, 333, 1, 64, 65), **kw):
    return W.Workload(name, "bf16", len(lengths), 3, d, 600, ("fixed", list(lengths)),
                      seed=31 + d, **kw)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("variant", ["bidir", "causal_gated_drop"])
def test_poisoned_padding_is_never_read(d, variant):
    """NaN in every padded slot of Q, K, V and dO: valid outputs bitwise equal to the
    clean run, padded rows exactly 0 (block-sparse padding, section 4)."""
    torch = need_gpu()
    kw = {} if variant == "bidir" else dict(causal=True, gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01),
                                           tau=0.05, sink=4)
    w = _small(d=d, **kw)
    clean, pois = W.generate(w), W.generate(w, poison=True)
    assert np.isnan(pois["q"]).any()
    note(f"poison d={d} {variant}")
    a = run_gpu(clean, torch.bfloat16)
    b = run_gpu(pois, torch.bfloat16)
    mask = np.broadcast_to(np.arange(600)[None, None, :] < clean["seqlens"][:, None, None],
                           clean["q"].shape[:3])
    for key in a:
        assert np.array_equal(a[key][mask], b[key][mask]), key
        assert np.all(b[key][~mask] == 0.0), key


def test_bitwise_deterministic():
    """No atomics: repeated runs give identical bits."""
    torch = need_gpu()
    data = W.generate(W.get("bidir_2k", B=4, H=4))
    note("determinism bidir_2k B=4 H=4")
    a = run_gpu(data, torch.bfloat16)
    b = run_gpu(data, torch.bfloat16)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("causal", [False, True])
def test_closed_form_qk_zero(causal):
    """Q = K = 0: every logit is b = -ln n, sigma(b) = 1/(n+1), so O_i is the sum of the
    allowed V_j over (n+1); with K = 0 also dQ = 0 exactly and dV_j = sum_i dO_i/(n+1)."""
    torch = need_gpu()
    w = _small(causal=causal)
    data = W.generate(w)
    data["q"][:] = 0.0
    data["k"][:] = 0.0
    note(f"closed form causal={causal}")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    o16 = run_gpu(data, torch.bfloat16, passes=("o",), out_dtype=torch.float32, fast_math=2)["O"]
    for b, n in enumerate(data["seqlens"]):
        if n == 0:
            continue
        v = data["v"][b, :, :n].astype(np.float64)
        do = data["do"][b, :, :n].astype(np.float64)
        if causal:
            want_o = np.cumsum(v, axis=1) / (n + 1)
            want_dv = np.cumsum(do[:, ::-1], axis=1)[:, ::-1] / (n + 1)
        else:
            want_o = np.broadcast_to(v.sum(axis=1, keepdims=True), v.shape) / (n + 1)
            want_dv = np.broadcast_to(do.sum(axis=1, keepdims=True), do.shape) / (n + 1)
        # P = 1/(n+1) is carried as hi + lo bf16 (relative 2^-16), or for the forward with
        # fast_math = 2 rounded once to f16 (relative 2^-11), and summed in float
        # (relative n 2^-24): |error| <= (u_P + n 2^-24) sum_j |src_j| / (n+1)
        for got, want, src, u_p in ((gpu["O"][b, :, :n], want_o, v, 2.0 ** -16),
                                    (o16[b, :, :n], want_o, v, 2.0 ** -11),
                                    (gpu["dV"][b, :, :n], want_dv, do, 2.0 ** -16)):
            tol = (u_p + n * 2.0 ** -24) * np.abs(src).sum(axis=1, keepdims=True) / (n + 1)
            assert np.all(np.abs(got - want) <= 2 * tol + 1e-7)
        assert np.all(gpu["dQ"][b, :, :n] == 0.0)


def test_causal_future_keys_do_not_matter():
    """Changing K and V at positions >= m leaves O rows < m bitwise unchanged."""
    torch = need_gpu()
    w = _small(causal=True, lengths=(600, 600, 450))
    data = W.generate(w)
    m = 300
    alt = {k_: (v_.copy() if isinstance(v_, np.ndarray) else v_) for k_, v_ in data.items()}
    alt["k"][:, :, m:] = W.round_to_bf16(alt["k"][:, :, m:] * 2.0 + 1.0)
    alt["v"][:, :, m:] = W.round_to_bf16(-alt["v"][:, :, m:])
    note("causal future-key invariance")
    a = run_gpu(data, torch.bfloat16, passes=("o", "dq"))
    b = run_gpu(alt, torch.bfloat16, passes=("o", "dq"))
    assert np.array_equal(a["O"][:, :, :m], b["O"][:, :, :m])
    assert np.array_equal(a["dQ"][:, :, :m], b["dQ"][:, :, :m])
    assert not np.array_equal(a["O"][:, :, m:450], b["O"][:, :, m:450])


def test_query_permutation_is_bitwise():
    """Bidirectional: the bias has no position and sigma is element-wise, so permuting
    the valid queries (with their dO rows) permutes O and dQ rows exactly."""
    torch = need_gpu()
    w = _small(lengths=(600, 517))
    data = W.generate(w)
    rng = np.random.default_rng(3)
    data_copy = {k_: (v_.copy() if isinstance(v_, np.ndarray) else v_) for k_, v_ in data.items()}
    perms = []
    for b, n in enumerate(data["seqlens"]):
        p = np.concatenate([rng.permutation(n), np.arange(n, 600)])
        perms.append(p)
        data_copy["q"][b] = data["q"][b][:, p]
        data_copy["do"][b] = data["do"][b][:, p]
    note("query permutation")
    a = run_gpu(data, torch.bfloat16, passes=("o", "dq"))
    b = run_gpu(data_copy, torch.bfloat16, passes=("o", "dq"))
    for bi, p in enumerate(perms):
        assert np.array_equal(b["O"][bi], a["O"][bi][:, p])
        assert np.array_equal(b["dQ"][bi], a["dQ"][bi][:, p])


def test_zero_gate_equals_hard_drop():
    """g_j = 0 (kept) and g_j < tau (dropped) both remove key j exactly (both gate
    channels send its contribution to zero)."""
    torch = need_gpu()
    w = _small(lengths=(600, 333), gate=("logistic_normal", 2.0, 2.0))
    data = W.generate(w)
    g = data["gate"]
    pick = np.zeros_like(g, dtype=bool)
    pick[:, 10:600:7] = True
    zero = {k_: (v_.copy() if isinstance(v_, np.ndarray) else v_) for k_, v_ in data.items()}
    drop = {k_: (v_.copy() if isinstance(v_, np.ndarray) else v_) for k_, v_ in data.items()}
    zero["gate"][pick] = 0.0
    zero["tau"] = 0.0
    drop["gate"][pick] = 0.01
    drop["tau"] = 0.05
    drop["gate"][~pick] = np.maximum(drop["gate"][~pick], 0.05)
    zero["gate"][~pick] = drop["gate"][~pick]
    note("zero gate vs hard drop")
    a = run_gpu(zero, torch.bfloat16)
    b = run_gpu(drop, torch.bfloat16)
    for key in a:
        assert np.array_equal(a[key], b[key]), key

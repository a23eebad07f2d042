"""The autograd entry points (sigmoid_attention_amd.attention and attention_varlen) on
the GPU: the output and the gradients torch.autograd returns are bitwise those of the
direct calls with the same rounded dO (fwd; bwd, or bwd_dq and bwd_dkdv_dg when the gate
needs a gradient; fwd_varlen and bwd_varlen for packed batches), and they match the fp64
oracle at the stated bar."""

import math

import numpy as np
import pytest

import workloads as W
from gpu_util import (BF16_TOL, check_all, check_bounds, need_gpu, note, oracle_full,
                      oracle_magnitudes)

pytestmark = pytest.mark.gpu

CASES = {
    "bidir": dict(),
    "causal_gated": dict(causal=True, gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01), tau=0.05,
                         sink=4),
}


def _inputs(torch, case, d):
    w = W.Workload(f"autograd_{case}_{d}", "bf16", 3, 2, d, 200, ("fixed", [200, 77, 1]),
                   seed=700 + d, **CASES[case])
    data = W.generate(w)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(data[k]).to(torch.bfloat16).to(dev) for k in ("q", "k", "v", "do")}
    gate = None if data["gate"] is None else torch.from_numpy(data["gate"]).to(dev)
    return w, data, t, gate


@pytest.mark.parametrize("case,gate_grad", [("bidir", False), ("causal_gated", False),
                                             ("causal_gated", True)])
@pytest.mark.parametrize("d", [64, 128])
def test_autograd_matches_direct_calls(d, case, gate_grad):
    torch = need_gpu()
    import sigmoid_attention_amd as S
    w, data, t, gate = _inputs(torch, case, d)
    note(f"autograd d={d} {case} gate_grad={gate_grad}")
    kw = dict(causal=w.causal, tau=w.tau, sink=w.sink, out_dtype=torch.float32)
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    g = None if gate is None else gate.clone().requires_grad_(gate_grad)
    o = S.attention(q, k, v, data["seqlens"], gate=g, **kw)
    o.backward(t["do"].float())          # dO as float; the entry point rounds it to bf16
    torch.cuda.synchronize()

    o_ref = S.fwd(t["q"], t["k"], t["v"], data["seqlens"], gate=gate, **kw)
    dkw = dict(causal=w.causal, tau=w.tau, sink=w.sink, gate=gate)
    dq, dk, dv = S.bwd(t["q"], t["k"], t["v"], t["do"], data["seqlens"], **dkw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for name, got, ref in (("dQ", q.grad, dq), ("dK", k.grad, dk), ("dV", v.grad, dv)):
        assert got.dtype == torch.bfloat16
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), name
    if gate_grad:
        _, _, _, dg = S.bwd_dkdv_dg(t["q"], t["k"], t["v"], t["do"], data["seqlens"], **dkw)
        torch.cuda.synchronize()
        assert torch.equal(g.grad, dg)
    elif g is not None:
        assert g.grad is None


@pytest.mark.parametrize("fast_math", [1, 2])
def test_autograd_fast_modes_match_direct_calls(fast_math):
    """The precision modes pass through: single bf16 operands (1) and the f16 forward (2)
    give bitwise the direct calls' results under autograd too."""
    torch = need_gpu()
    import sigmoid_attention_amd as S
    w, data, t, gate = _inputs(torch, "causal_gated", 64)
    note(f"autograd fast_math={fast_math}")
    kw = dict(causal=True, tau=w.tau, sink=w.sink, gate=gate, fast_math=fast_math)
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = S.attention(q, k, v, data["seqlens"], out_dtype=torch.float32, **kw)
    o.backward(t["do"].float())
    o_ref = S.fwd(t["q"], t["k"], t["v"], data["seqlens"], out_dtype=torch.float32, **kw)
    refs = S.bwd(t["q"], t["k"], t["v"], t["do"], data["seqlens"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for name, got, ref in zip(("dQ", "dK", "dV"), (q.grad, k.grad, v.grad), refs):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), name


def test_autograd_against_oracle():
    """Float output of the forward at the bar; the bf16 gradients within the element-wise
    bounds that add their own bf16 rounding (the bounds the parity tests use for bf16
    outputs)."""
    torch = need_gpu()
    import sigmoid_attention_amd as S
    w, data, t, gate = _inputs(torch, "causal_gated", 64)
    note("autograd against the oracle")
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = S.attention(q, k, v, data["seqlens"], gate=gate, causal=True, tau=w.tau, sink=w.sink,
                    out_dtype=torch.float32)
    o.backward(t["do"].float())
    torch.cuda.synchronize()
    ref = oracle_full(data)
    print(check_all({"O": o.detach().cpu().numpy()}, ref, data["seqlens"], BF16_TOL,
                    "autograd O"))
    grads = {"dQ": q.grad.float().cpu().numpy(), "dK": k.grad.float().cpu().numpy(),
             "dV": v.grad.float().cpu().numpy()}
    print(check_bounds(grads, ref, oracle_magnitudes(data), data["seqlens"], True, False,
                       "autograd gradients"))


def _packed(torch, seed, lens_q, lens_k, H, d, gated, extra_rows=5):
    """Packed bf16 q, k, v, dO with rows past the last sequence, cu arrays on the device."""
    rng = np.random.default_rng(seed)
    tq, tk = int(np.sum(lens_q)) + extra_rows, int(np.sum(lens_k)) + extra_rows
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(rng.standard_normal((tq if n in ("q", "do") else tk, H, d),
                                                 dtype=np.float32)).to(torch.bfloat16).to(dev)
         for n in ("q", "k", "v", "do")}
    gate = None
    if gated:
        g = 1.0 / (1.0 + np.exp(-(rng.standard_normal(tk) * math.sqrt(2.0) + 1.0)))
        g[rng.random(tk) < 0.2] = 0.01
        gate = torch.from_numpy(g.astype(np.float32)).to(dev)
    cu = [torch.from_numpy(np.concatenate([[0], np.cumsum(x)]).astype(np.int32)).to(dev)
          for x in (lens_q, lens_k)]
    return t, gate, cu[0], cu[1], int(max(lens_q)), int(max(lens_k))


@pytest.mark.parametrize("causal,gated", [(False, False), (True, True)])
@pytest.mark.parametrize("d", [64, 128])
def test_attention_varlen_matches_direct_calls(d, causal, gated):
    """Unequal query and key lengths (one empty key set, one 1-row query) and five rows
    past the last sequence, which come out 0 in O and in every gradient."""
    torch = need_gpu()
    import sigmoid_attention_amd as S
    lens_q, lens_k = [128, 300, 40, 1, 200], [700, 300, 9, 33, 0]
    t, gate, cu_q, cu_k, mq, mk = _packed(torch, 900 + d, lens_q, lens_k, 2, d, gated)
    note(f"attention_varlen d={d} causal={causal} gated={gated}")
    kw = dict(causal=causal, gate=gate, tau=0.05 if gated else 0.0, sink=4)
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = S.attention_varlen(q, k, v, cu_q, cu_k, mq, mk, out_dtype=torch.float32, **kw)
    o.backward(t["do"].float())
    torch.cuda.synchronize()

    o_ref = torch.zeros(t["q"].shape, dtype=torch.float32, device=o.device)
    S.fwd_varlen(t["q"], t["k"], t["v"], cu_q, cu_k, mq, mk, out=o_ref, out_dtype=torch.float32,
                 **kw)
    refs = (torch.zeros_like(t["q"]), torch.zeros_like(t["k"]), torch.zeros_like(t["k"]))
    S.bwd_varlen(t["q"], t["k"], t["v"], t["do"], cu_q, cu_k, mq, mk, out=refs, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    nq, nk = sum(lens_q), sum(lens_k)
    assert torch.count_nonzero(o[nq:]) == 0
    for name, got, ref, n in (("dQ", q.grad, refs[0], nq), ("dK", k.grad, refs[1], nk),
                              ("dV", v.grad, refs[2], nk)):
        assert got.dtype == torch.bfloat16
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), name
        assert torch.count_nonzero(got[n:]) == 0, name

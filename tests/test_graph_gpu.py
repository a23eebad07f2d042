"""The library under HIP graph capture (torch.cuda.graph). Every entry point only enqueues
kernels on the caller's stream, with its arguments passed by value: no allocation, no
memset node, no host synchronisation. A captured step therefore replays to the eager
results bit for bit, also after new values are written into its input buffers between
replays, with eager work and synchronisations in between (each replay is checked, not
only the first). Covered: the padded forward and one-call backward (d = 64: one launch;
d = 128: two), the autograd entry point's forward and backward, the packed entry points
with new sequence bounds written into the device cu_seqlens arrays, and a token-by-token
decode loop (cache append, then decode with a workspace and without one) against a twin
cache driven eagerly."""

import math

import numpy as np
import pytest

import sigmoid_attention_amd as S
import workloads as W
from gpu_util import need_gpu, note

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _same_bits(torch, a, b):
    as_int = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.int32: torch.int32}
    return (a.dtype == b.dtype and a.shape == b.shape
            and torch.equal(a.view(as_int[a.dtype]), b.view(as_int[b.dtype])))


def _capture(torch, step):
    """Warm step() up on a side stream, then capture one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    return graph


def _bf16(torch, rng, shape):
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16).cuda()


def _gate(torch, rng, B, L):
    g = 1.0 / (1.0 + np.exp(-(rng.standard_normal((B, L)) * math.sqrt(2.0) + 2.0)))
    g[rng.random((B, L)) < 0.2] = 0.01
    return torch.from_numpy(g.astype(np.float32)).cuda()


@pytest.mark.parametrize("lengths", ["ragged", "one_length"])
@pytest.mark.parametrize("d", [64, 128])
def test_padded_step_replays(d, lengths):
    """Ragged lengths take the per-sequence work lists, one length the block-major ones."""
    torch = need_gpu()
    B, H, L = 3, 2, 200
    sl = [200, 77, 1] if lengths == "ragged" else [200, 200, 200]
    kw = dict(causal=True, tau=0.05, sink=4)
    rng = np.random.default_rng(40 + d)
    x = {n: _bf16(torch, rng, (B, H, L, d)) for n in ("q", "k", "v", "do")}
    gate = _gate(torch, rng, B, L)
    o = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(x["q"]) for _ in range(3))

    def step():
        S.fwd(x["q"], x["k"], x["v"], sl, gate=gate, out=o, out_dtype=torch.float32, **kw)
        S.bwd(x["q"], x["k"], x["v"], x["do"], sl, gate=gate, out=grads, **kw)

    note(f"graph capture: padded fwd + bwd d={d} {lengths}")
    graph = _capture(torch, step)
    for r in range(REPLAYS):
        if r:
            for t in x.values():
                t.copy_(_bf16(torch, rng, t.shape))
            gate.copy_(_gate(torch, rng, B, L))
        o_ref = S.fwd(x["q"], x["k"], x["v"], sl, gate=gate, out_dtype=torch.float32, **kw)
        g_ref = S.bwd(x["q"], x["k"], x["v"], x["do"], sl, gate=gate, **kw)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same_bits(torch, o, o_ref), f"O, replay {r}"
        for name, got, ref in zip(("dQ", "dK", "dV"), grads, g_ref):
            assert _same_bits(torch, got, ref), f"{name}, replay {r}"


def test_autograd_step_replays():
    """Forward and backward of attention() captured together, as a training step is; the
    gradients land in the tensors autograd allocated during capture."""
    torch = need_gpu()
    B, H, L, d = 2, 3, 160, 64
    sl = [160, 45]
    rng = np.random.default_rng(11)
    q, k, v = (_bf16(torch, rng, (B, H, L, d)).requires_grad_(True) for _ in range(3))
    do = _bf16(torch, rng, (B, H, L, d)).float()
    out = {}

    def step():
        q.grad = k.grad = v.grad = None
        o = S.attention(q, k, v, sl, causal=True, out_dtype=torch.float32)
        o.backward(do)
        out["o"] = o

    note("graph capture: autograd attention forward + backward")
    graph = _capture(torch, step)
    o, gq, gk, gv = out["o"], q.grad, k.grad, v.grad
    for r in range(REPLAYS):
        if r:
            with torch.no_grad():
                for t in (q, k, v):
                    t.copy_(_bf16(torch, rng, t.shape))
                do.copy_(_bf16(torch, rng, do.shape).float())
        qd, kd, vd = q.detach(), k.detach(), v.detach()
        o_ref = S.fwd(qd, kd, vd, sl, causal=True, out_dtype=torch.float32)
        g_ref = S.bwd(qd, kd, vd, do.to(torch.bfloat16), sl, causal=True)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same_bits(torch, o, o_ref), f"O, replay {r}"
        for name, got, ref in zip(("dQ", "dK", "dV"), (gq, gk, gv), g_ref):
            assert _same_bits(torch, got, ref), f"{name}, replay {r}"


def test_packed_step_replays_with_new_bounds():
    """The sequence bounds live in device arrays, so a captured packed step follows new
    bounds written there (same B, same totals, within the host bounds it was captured
    with)."""
    torch = need_gpu()
    H, d = 2, 64
    packings = [([128, 300, 40, 1, 200], [300, 128, 9, 33, 199]),
                ([300, 128, 1, 200, 40], [9, 300, 199, 128, 33]),
                ([1, 40, 128, 300, 200], [33, 199, 300, 9, 128])]
    tq, tk = sum(packings[0][0]) + 5, sum(packings[0][1]) + 5
    max_q = max(max(p[0]) for p in packings)
    max_k = max(max(p[1]) for p in packings)
    rng = np.random.default_rng(5)
    q, do = (_bf16(torch, rng, (tq, H, d)) for _ in range(2))
    k, v = (_bf16(torch, rng, (tk, H, d)) for _ in range(2))

    def cu(lens):
        return torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()

    cu_q, cu_k = cu(packings[0][0]), cu(packings[0][1])
    kw = dict(causal=True)
    o = torch.zeros((tq, H, d), dtype=torch.float32, device="cuda")
    grads = (torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(k))

    def step():
        S.fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k, out=o, out_dtype=torch.float32, **kw)
        S.bwd_varlen(q, k, v, do, cu_q, cu_k, max_q, max_k, out=grads, **kw)

    note("graph capture: packed fwd + bwd")
    graph = _capture(torch, step)
    for r, (lq, lk) in enumerate(packings):
        cu_q.copy_(cu(lq))
        cu_k.copy_(cu(lk))
        o_ref = torch.zeros_like(o)
        g_ref = tuple(torch.zeros_like(g) for g in grads)
        S.fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k, out=o_ref, out_dtype=torch.float32, **kw)
        S.bwd_varlen(q, k, v, do, cu_q, cu_k, max_q, max_k, out=g_ref, **kw)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # every row lies inside a sequence except the last five, which neither side writes
        assert _same_bits(torch, o[:-5], o_ref[:-5]), f"O, packing {r}"
        for name, got, ref in zip(("dQ", "dK", "dV"), grads, g_ref):
            assert _same_bits(torch, got[:-5], ref[:-5]), f"{name}, packing {r}"


@pytest.mark.parametrize("gated", [False, True])
def test_decode_loop_replays(gated):
    """One captured decode step (append the new entry, decode with a workspace, decode
    without one) replayed token by token against a twin cache driven eagerly: outputs,
    cache contents and counters bit for bit after every token."""
    torch = need_gpu()
    B, H, d, cap, T = 3, 2, 64, 96, 40
    tau, sink = 0.3, 4
    rng = np.random.default_rng(90 + int(gated))
    caches = [S.KVCache(B, H, d, cap, gated=gated, tau=tau, sink=sink) for _ in range(2)]
    pre = [40, 0, 7]
    kp, vp = (_bf16(torch, rng, (B, H, 64, d)) for _ in range(2))
    gp = _gate(torch, rng, B, 64) if gated else None
    for c in caches:
        c.build(kp, vp, pre, gate=gp)
    bias = [-math.log(64.0)] * B
    k_new, v_new, q = (_bf16(torch, rng, (B, H, d)) for _ in range(3))
    g_new = torch.empty(B, dtype=torch.float32, device="cuda") if gated else None
    ws = torch.empty(max(1, (caches[1].workspace_size() + 3) // 4), dtype=torch.float32,
                     device="cuda")
    outs = [torch.empty((B, H, d), dtype=torch.float32, device="cuda") for _ in range(2)]

    def step(c, o1, o2, workspace):
        c.append(k_new, v_new, g_new)
        c.decode(q, bias, out=o1, out_dtype=torch.float32, workspace=workspace)
        c.decode_noalloc(q, bias, out=o2, out_dtype=torch.float32)

    def fill():
        for t in (k_new, v_new, q):
            t.copy_(_bf16(torch, rng, t.shape))
        if gated:
            g_new.copy_(torch.from_numpy(rng.uniform(0.0, 1.0, B).astype(np.float32)))

    # capturing runs the step twice outside the graph: the eager twin does the same
    fill()
    note(f"graph capture: decode loop gated={gated}")
    graph = _capture(torch, lambda: step(caches[1], outs[0], outs[1], ws))
    ref_outs = [torch.empty_like(outs[0]) for _ in range(2)]
    for _ in range(2):
        step(caches[0], ref_outs[0], ref_outs[1], None)
    for i in range(T):
        fill()
        step(caches[0], ref_outs[0], ref_outs[1], None)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref_outs):
            assert _same_bits(torch, a, b), f"decode output, token {i}"
        for name in ("count", "seen"):
            assert torch.equal(getattr(caches[1], name), getattr(caches[0], name)), name
        for name in ("k", "v") + (("gate",) if gated else ()):
            assert torch.equal(getattr(caches[1], name), getattr(caches[0], name)), name

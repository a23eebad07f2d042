"""GPU parity of packed variable-length batches (device-side cu_seqlens, separate query
and key lengths, bottom-right causal alignment, no cap on B) against the fp64 oracle,
through the C ABI. The bar is the stated one, max |gpu - ref| / rms(ref) <= 2e-2 over the
rows of the sequences (float outputs); rows with no allowed key or no query are exactly
0, and rows outside the sequences are left untouched.
"""

import math

import numpy as np
import pytest

import oracle as O
import sigmoid_attention_amd as S
import workloads as W
from gpu_util import BF16_TOL, err_ratio, need_gpu, note

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _packed_case(seed, lens_q, lens_k, H, d, gated=False, extra_rows=5):
    rng = np.random.default_rng(seed)
    tq, tk = int(np.sum(lens_q)) + extra_rows, int(np.sum(lens_k)) + extra_rows
    q, do = (W.round_to_bf16(rng.standard_normal((tq, H, d), dtype=np.float32)) for _ in range(2))
    k, v = (W.round_to_bf16(rng.standard_normal((tk, H, d), dtype=np.float32)) for _ in range(2))
    gate = None
    if gated:
        gate = (1.0 / (1.0 + np.exp(-(rng.standard_normal(tk) * math.sqrt(2.0) + 1.0)))).astype(np.float32)
        gate[rng.random(tk) < 0.2] = np.float32(0.01)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    return dict(q=q, k=k, v=v, do=do, gate=gate, cu_q=cu_q, cu_k=cu_k,
                max_q=int(max(lens_q)), max_k=int(max(lens_k)))


def _run(torch, c, causal, tau=0.0, bias=None, passes=("o", "dq", "dkdv"), fast_math=0):
    dev = torch.device("cuda")
    t = {n: torch.from_numpy(c[n]).to(torch.bfloat16).to(dev) for n in ("q", "k", "v", "do")}
    cu_q = torch.from_numpy(c["cu_q"]).to(dev)
    cu_k = torch.from_numpy(c["cu_k"]).to(dev)
    gate = None if c["gate"] is None else torch.from_numpy(c["gate"]).to(dev)
    bias_t = None if bias is None else torch.tensor(bias, dtype=torch.float32, device=dev)
    kw = dict(causal=causal, gate=gate, tau=tau, sink=4, bias=bias_t, out_dtype=torch.float32,
              fast_math=fast_math)
    out = {}
    if "o" in passes:
        o = torch.full(t["q"].shape, SENTINEL, dtype=torch.float32, device=dev)
        out["O"] = S.fwd_varlen(t["q"], t["k"], t["v"], cu_q, cu_k, c["max_q"], c["max_k"], out=o, **kw)
    if "dq" in passes:
        dq = torch.full(t["q"].shape, SENTINEL, dtype=torch.float32, device=dev)
        out["dQ"] = S.bwd_dq_varlen(t["q"], t["k"], t["v"], t["do"], cu_q, cu_k, c["max_q"],
                                    c["max_k"], out=dq, **kw)
    if "dkdv" in passes:
        dk = torch.full(t["k"].shape, SENTINEL, dtype=torch.float32, device=dev)
        dv = torch.full(t["k"].shape, SENTINEL, dtype=torch.float32, device=dev)
        out["dK"], out["dV"] = S.bwd_dkdv_varlen(t["q"], t["k"], t["v"], t["do"], cu_q, cu_k,
                                                 c["max_q"], c["max_k"], out=(dk, dv), **kw)
    torch.cuda.synchronize()
    return {n: x.cpu().numpy() for n, x in out.items()}


def _check(gpu, c, causal, tau=0.0, bias=None, label=""):
    kw = dict(causal=causal, gate=c["gate"], tau=tau, sink=4, bias=bias)
    ref = {"O": O.forward_varlen(c["q"], c["k"], c["v"], c["cu_q"], c["cu_k"], **kw)}
    ref["dQ"], ref["dK"], ref["dV"] = O.backward_varlen(c["q"], c["k"], c["v"], c["do"],
                                                        c["cu_q"], c["cu_k"], **kw)
    rows_q, rows_k = int(c["cu_q"][-1]), int(c["cu_k"][-1])
    rep = {}
    for name in gpu:
        rows = rows_q if name in ("O", "dQ") else rows_k
        g, r = gpu[name], ref[name]
        assert np.all(g[rows:] == SENTINEL), f"{label} {name}: rows outside the sequences written"
        assert np.all(np.isfinite(g[:rows])), f"{label} {name}: non-finite values"
        zero = np.all(r[:rows] == 0.0, axis=(1, 2))
        assert np.all(g[:rows][zero] == 0.0), f"{label} {name}: rows that must be 0 are not"
        e = err_ratio(g[:rows], r[:rows], np.ones(g[:rows].shape, bool))
        rep[name] = e
        assert e <= BF16_TOL, f"{label} {name}: error ratio {e:.3e}"
    return rep


CASES = {
    # queries and keys of equal length, ragged, with an empty and a one-token sequence
    "equal": ([600, 0, 1, 129, 333, 64], [600, 0, 1, 129, 333, 64]),
    # more keys than queries (query shards), and more queries than keys
    "unequal": ([128, 300, 40, 1, 200], [700, 300, 9, 33, 0]),
}


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_against_oracle(d, case, causal, gated):
    torch = need_gpu()
    lq, lk = CASES[case]
    c = _packed_case(400 + d + len(case) + 2 * causal + gated, lq, lk, 3, d, gated=gated)
    tau = 0.05 if gated else 0.0
    note(f"varlen d={d} {case} causal={causal} gated={gated}")
    gpu = _run(torch, c, causal, tau=tau)
    print(_check(gpu, c, causal, tau=tau, label=f"{case} {d} {causal} {gated}"))


def test_varlen_more_than_256_sequences():
    """B = 300 short sequences (the padded entry points stop at 256)."""
    torch = need_gpu()
    rng = np.random.default_rng(410)
    lens = rng.integers(0, 70, 300).tolist()
    c = _packed_case(411, lens, lens, 2, 64)
    note("varlen B=300")
    gpu = _run(torch, c, True)
    print(_check(gpu, c, True, label="B=300"))


@pytest.mark.parametrize("causal", [False, True])
def test_context_parallel_shard(causal):
    """One GPU's share of 8-way context parallelism at 8192 tokens: the last 1024 query
    rows against all 8192 keys, with the sequence's bias -ln(8192). Sampled rows equal
    those rows of the full sequence's result (oracle, full-sequence definition)."""
    torch = need_gpu()
    N, m, H, d = 8192, 1024, 4, 64
    rng = np.random.default_rng(420)
    full = {n: W.round_to_bf16(rng.standard_normal((1, H, N, d), dtype=np.float32))
            for n in ("q", "k", "v", "do")}
    s0 = N - m
    c = {"q": np.ascontiguousarray(full["q"][0, :, s0:].transpose(1, 0, 2)),
         "do": np.ascontiguousarray(full["do"][0, :, s0:].transpose(1, 0, 2)),
         "k": np.ascontiguousarray(full["k"][0].transpose(1, 0, 2)),
         "v": np.ascontiguousarray(full["v"][0].transpose(1, 0, 2)),
         "gate": None, "cu_q": np.array([0, m], np.int32), "cu_k": np.array([0, N], np.int32),
         "max_q": m, "max_k": N}
    bias = [-math.log(N)]
    note(f"context-parallel shard causal={causal}")
    gpu = _run(torch, c, causal, bias=bias, passes=("o", "dq"))
    rows = np.array([0, 1, 31, 32, 511, 512, m - 2, m - 1])
    for h in range(H):
        o = O.forward_rows(full["q"], full["k"], full["v"], [N], 0, h, s0 + rows, causal=causal,
                           bias=bias)
        dq = O.dq_rows(full["q"], full["k"], full["v"], full["do"], [N], 0, h, s0 + rows,
                       causal=causal, bias=bias)
        for name, ref in (("O", o), ("dQ", dq)):
            e = err_ratio(gpu[name][rows, h], ref, np.ones(ref.shape, bool))
            assert e <= BF16_TOL, f"shard {name} head {h}: {e:.3e}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_length_grid(d, causal):
    """Every pair of query and key lengths from a grid around the 32-row chunk and the
    128-row tile (196 sequences, more queries than keys and the reverse)."""
    torch = need_gpu()
    grid = [1, 31, 32, 33, 63, 64, 65, 95, 96, 127, 128, 129, 160, 200]
    lq = [a for a in grid for _ in grid]
    lk = [b for _ in grid for b in grid]
    c = _packed_case(430 + d + causal, lq, lk, 1, d)
    note(f"varlen length grid d={d} causal={causal}")
    gpu = _run(torch, c, causal)
    print(_check(gpu, c, causal, label=f"grid {d} {causal}"))


def _one_call(torch, c, causal, tau=0.0, out_dtype=None, fast=False):
    dev = torch.device("cuda")
    t = {n: torch.from_numpy(c[n]).to(torch.bfloat16).to(dev) for n in ("q", "k", "v", "do")}
    cu_q = torch.from_numpy(c["cu_q"]).to(dev)
    cu_k = torch.from_numpy(c["cu_k"]).to(dev)
    gate = None if c["gate"] is None else torch.from_numpy(c["gate"]).to(dev)
    kw = dict(causal=causal, gate=gate, tau=tau, sink=4, out_dtype=out_dtype or torch.float32,
              fast_math=fast)
    args = (t["q"], t["k"], t["v"], t["do"], cu_q, cu_k, c["max_q"], c["max_k"])
    od = kw["out_dtype"]

    def filled(like):   # rows outside the sequences must stay as they are
        return torch.full(like.shape, SENTINEL, dtype=od, device=dev)

    one = S.bwd_varlen(*args, out=(filled(t["q"]), filled(t["k"]), filled(t["k"])), **kw)
    dq = S.bwd_dq_varlen(*args, out=filled(t["q"]), **kw)
    dk, dv = S.bwd_dkdv_varlen(*args, out=(filled(t["k"]), filled(t["k"])), **kw)
    torch.cuda.synchronize()
    return one, (dq, dk, dv)


@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("d", [64, 128])
def test_one_call_backward_bitwise(d, case, causal, gated, fast):
    """sigattn_bwd_varlen equals sigattn_bwd_dq_varlen + sigattn_bwd_dkdv_varlen bitwise
    (the same kernel bodies; one launch at d = 64), including unequal query and key
    lengths, so the two lists of items differ in length."""
    torch = need_gpu()
    lq, lk = CASES[case]
    c = _packed_case(450 + d + len(case) + 2 * causal + gated, lq, lk, 3, d, gated=gated)
    note(f"varlen one-call backward d={d} {case} causal={causal} gated={gated} fast={fast}")
    for od in (torch.float32, torch.bfloat16):
        one, sep = _one_call(torch, c, causal, tau=0.05 if gated else 0.0, out_dtype=od, fast=fast)
        for name, a, b in zip(("dQ", "dK", "dV"), one, sep):
            ia = a.view(torch.int16 if a.element_size() == 2 else torch.int32)
            ib = b.view(torch.int16 if b.element_size() == 2 else torch.int32)
            assert torch.equal(ia, ib), f"{case} d={d} {name}: one-call differs"


@pytest.mark.parametrize("causal", [False, True])
def test_one_call_backward_against_oracle(causal):
    """The packed one-call backward at the stated bar, on the length grid (196 sequences,
    more queries than keys and the reverse) and the unequal case."""
    torch = need_gpu()
    grid = [1, 31, 32, 33, 63, 64, 65, 95, 96, 127, 128, 129, 160, 200]
    lq = [a for a in grid for _ in grid]
    lk = [b for _ in grid for b in grid]
    c = _packed_case(470 + causal, lq, lk, 1, 64, gated=True)
    note(f"varlen one-call backward vs oracle causal={causal}")
    one, _ = _one_call(torch, c, causal, tau=0.05)
    rows_q, rows_k = int(c["cu_q"][-1]), int(c["cu_k"][-1])
    for g, rows in zip(one, (rows_q, rows_k, rows_k)):
        assert bool((g[rows:] == SENTINEL).all()), "rows outside the sequences written"
    kw = dict(causal=causal, gate=c["gate"], tau=0.05, sink=4)
    ref = O.backward_varlen(c["q"], c["k"], c["v"], c["do"], c["cu_q"], c["cu_k"], **kw)
    for name, g, r, rows in zip(("dQ", "dK", "dV"), one, ref, (rows_q, rows_k, rows_k)):
        g = g.cpu().numpy()[:rows]
        e = err_ratio(g, r[:rows], np.ones(g.shape, bool))
        assert e <= BF16_TOL, f"{name}: {e:.3e}"


def test_varlen_values_beyond_f16():
    """Packed batches with fast_math = 2 whose V exceeds the f16 range in one sequence:
    the forward's second pass on bf16 operands covers packed items too."""
    torch = need_gpu()
    c = _packed_case(480, [300, 129, 64], [300, 129, 64], 2, 64)
    c["v"][310:314] = W.round_to_bf16(c["v"][310:314] * np.float32(3e5))
    note("varlen V beyond f16")
    gpu = _run(torch, c, False, passes=("o",), fast_math=2)
    print(_check(gpu, c, False, label="varlen big V"))


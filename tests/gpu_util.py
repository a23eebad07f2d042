"""Helpers for the GPU parity tests: run the HIP path on seeded workloads and compare
with the fp64 oracle on the same input bits.

Two checks are used.

* The stated bar: max |gpu - ref| / rms(ref) <= 2e-2 over valid rows for bf16 inputs
  (1e-5 on the float32 debug path). It applies to float outputs with the default
  (split hi + lo) precision; bf16-stored outputs cannot meet it on heavy-tailed outputs
  (max/rms above ~10 makes half a bf16 ulp of the largest element exceed 2e-2 of rms).
* Element-wise bounds derived from the arithmetic, for bf16 outputs and for fast math,
  with u = 2^-8 the unit roundoff of bf16:
    bf16 output rounding        |d| <= u |ref|
    fast math (P or dS in bf16) |d| <= u A,  A = sum of |terms| of the product
                                (the oracle's absolute sums)
  plus 2^-12 A for the hi + lo residual and float accumulation (2^-11 A for the forward
  output with fast_math = 2, whose P V product takes P rounded once to f16, unit
  roundoff 2^-11), and 2e-3 rms(ref) for the float evaluation of sigma near saturation
  (|delta sigma'| <= 2^-23).
"""

import functools
import sys

import numpy as np
import pytest

import oracle as O
import sigmoid_attention_amd as S

BF16_TOL = 2e-2   # max |gpu - ref| / rms(ref) over valid rows, bf16 inputs
F32_TOL = 1e-5    # same measure on the float32 debug path
U_BF16 = 2.0 ** -8


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU is visible to torch")
    S.load()
    return torch


def note(msg):
    """Name the case before a GPU step, flushed, so a failure can be attributed."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(data, torch_dtype):
    import torch
    t = {}
    for name in ("q", "k", "v", "do"):
        t[name] = torch.from_numpy(np.ascontiguousarray(data[name])).to(torch_dtype).cuda()
    t["gate"] = None if data["gate"] is None else torch.from_numpy(data["gate"]).cuda()
    return t


def kwargs_of(data, gate_t):
    return dict(causal=bool(data["causal"]), gate=gate_t, tau=float(data["tau"]),
                sink=int(data["sink"]))


def run_gpu(data, torch_dtype, passes=("o", "dq", "dkdv"), out_dtype=None, fast_math=False):
    import torch
    t = to_device(data, torch_dtype)
    kw = kwargs_of(data, t["gate"])
    kw.update(out_dtype=out_dtype, fast_math=fast_math)
    out = {}
    sl = data["seqlens"]
    if "o" in passes:
        out["O"] = S.fwd(t["q"], t["k"], t["v"], sl, **kw)
    if "dq" in passes:
        out["dQ"] = S.bwd_dq(t["q"], t["k"], t["v"], t["do"], sl, **kw)
    if "dkdv" in passes:
        out["dK"], out["dV"] = S.bwd_dkdv(t["q"], t["k"], t["v"], t["do"], sl, **kw)
    torch.cuda.synchronize()
    return {k_: v_.float().cpu().numpy() for k_, v_ in out.items()}


def oracle_kwargs(data):
    g = None if data["gate"] is None else data["gate"].astype(np.float64)
    return dict(causal=bool(data["causal"]), gate=g, tau=float(data["tau"]),
                sink=int(data["sink"]))


@functools.lru_cache(maxsize=1)
def oracle_full_named(name):
    """oracle_full of a named workload's seeded inputs, kept for the next caller."""
    import workloads as W
    return oracle_full(W.generate(name))


def oracle_full(data):
    kw = oracle_kwargs(data)
    o = O.forward(data["q"], data["k"], data["v"], data["seqlens"], **kw)
    dq, dk, dv = O.backward(data["q"], data["k"], data["v"], data["do"], data["seqlens"], **kw)
    return {"O": o, "dQ": dq, "dK": dk, "dV": dv}


def oracle_magnitudes(data):
    """A for each output: the sums of |terms| of its defining product."""
    kw = oracle_kwargs(data)
    a_o = O.forward(data["q"], data["k"], np.abs(data["v"]), data["seqlens"], **kw)
    a_dq, a_dk, a_dv = O.backward(data["q"], data["k"], data["v"], data["do"], data["seqlens"],
                                  absolute=True, **kw)
    return {"O": a_o, "dQ": a_dq, "dK": a_dk, "dV": a_dv}


def valid_rows(seqlens, shape):
    B, H, L = shape[:3]
    m = np.arange(L)[None, None, :] < np.asarray(seqlens)[:, None, None]
    return np.broadcast_to(m, (B, H, L))


def err_ratio(gpu, ref, mask):
    """max |gpu - ref| / rms(ref), both over the rows selected by mask."""
    g, r = gpu[mask], ref[mask]
    rms = float(np.sqrt(np.mean(r * r)))
    if rms == 0.0:
        return float(np.max(np.abs(g - r))) if g.size else 0.0
    return float(np.max(np.abs(g - r))) / rms


def check_all(gpu, ref, seqlens, tol, label=""):
    """The stated bar on every output, plus exact zeros in padded rows."""
    mask = valid_rows(seqlens, ref["O"].shape)
    report = {}
    for name in ref:
        if name not in gpu:
            continue
        assert np.all(np.isfinite(gpu[name][mask])), f"{label} {name}: non-finite values"
        e = err_ratio(gpu[name], ref[name], mask)
        report[name] = e
        assert np.all(gpu[name][~mask] == 0.0), f"{label} {name}: padded rows not exactly 0"
        assert e <= tol, f"{label} {name}: error ratio {e:.3e} > {tol}"
    return report


def bound_excess(gpu, ref, mag, bf16_out, fast_math, rms, f16_p=False):
    """max over elements of |gpu - ref| / (derived bound); <= 1 passes. f16_p: the output
    of a product whose P operand is rounded to f16 (the forward with fast_math = 2)."""
    bound = (2.0 ** (-11 if f16_p and not fast_math else -12)) * mag + 2e-3 * rms
    if fast_math:
        bound = bound + U_BF16 * mag
    if bf16_out:
        bound = bound + U_BF16 * (np.abs(ref) + (U_BF16 * mag if fast_math else 0.0))
    return float(np.max(np.abs(gpu - ref) / bound)) if gpu.size else 0.0


def check_bounds(gpu, ref, mag, seqlens, bf16_out, fast_math, label="", f16=False):
    mask = valid_rows(seqlens, ref["O"].shape)
    report = {}
    for name in ref:
        if name not in gpu:
            continue
        g, r, m = gpu[name][mask], ref[name][mask], mag[name][mask]
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite values"
        assert np.all(gpu[name][~mask] == 0.0), f"{label} {name}: padded rows not exactly 0"
        rms = float(np.sqrt(np.mean(r * r)))
        x = bound_excess(g, r, m, bf16_out, fast_math, rms, f16_p=f16 and name == "O")
        report[name] = x
        assert x <= 1.0, f"{label} {name}: error exceeds the derived bound by {x:.2f}x"
    return report

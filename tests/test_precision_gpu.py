"""Evidence for the default operand precision (P and dS carried as hi + lo bf16 pairs),
through the C ABI against the fp64 oracle, with float outputs.

For every configuration of the benchmark set the single-rounded operand modes are
measured against the stated bar, max |gpu - ref| / rms(ref) <= 2e-2 over valid rows:

* fast_math = 1 (P and dS rounded once to bf16, unit roundoff 2^-8, in every pass);
* fast_math = 2 (P rounded once to f16, 2^-11, in the forward only; its backward is
  the default's).

What the tests hold, and the design relies on:

* single bf16 operands miss the bar on the 2K bidirectional batch and on the causal
  gated 512-token layer (the worst element's error comes from the rounding of a few of
  its row's largest weights, 2^-9 of each, times their values: more than 2e-2 of the
  batch's rms); so fast_math = 1 cannot be the default;
* f16 P meets the bar on every configuration of the set, but misses it on a batch in
  which some queries put most of their weight on one key with a large value (an output
  row far above the batch rms: its error follows the row's size, the bar divides by the
  batch's rms), where the default split stays two orders of magnitude inside the bar;
  so fast_math = 2 cannot be the default either.

Every measured ratio is printed (pytest -s) so that the design notes quote them.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import (BF16_TOL, err_ratio, need_gpu, note, oracle_full, oracle_full_named,
                      oracle_kwargs, run_gpu)

pytestmark = pytest.mark.gpu

FULL = ["tiny_bf16", "causal_gated_512", "causal_forced_drop_512", "bidir_2k"]
SAMPLED = ["long_8k_s1", "long_8k_s4", "pad_sweep_0", "pad_sweep_25", "pad_sweep_50"]


def _data(name):
    if name == "tiny_bf16":
        return W.generate(W.get("tiny_fp32", dtype="bf16"))
    return W.generate(name)


def _full_ratios(data, gpu, ref):
    mask = np.broadcast_to(np.arange(ref["O"].shape[2])[None, None, :]
                           < np.asarray(data["seqlens"])[:, None, None], ref["O"].shape[:3])
    return {k: err_ratio(gpu[k], ref[k], mask) for k in gpu}


def _sampled_ratios(data, gpu):
    """Every batch entry, its first and last head, sampled rows (first, last, tile
    edges, random), against the oracle's row functions."""
    kw = oracle_kwargs(data)
    sl = data["seqlens"]
    B, H, L, d = data["q"].shape
    rng = np.random.default_rng(11)
    refs = {k: [] for k in gpu}
    gots = {k: [] for k in gpu}
    for b in range(B):
        n = int(sl[b])
        if n == 0:
            continue
        rows = np.unique(np.concatenate([[0, n - 1], np.arange(127, n, 128),
                                         rng.integers(0, n, size=6)]))
        for h in sorted({0, H - 1}):
            if "O" in gpu:
                refs["O"].append(O.forward_rows(data["q"], data["k"], data["v"], sl, b, h, rows, **kw))
                gots["O"].append(gpu["O"][b, h, rows])
            if "dQ" in gpu:
                refs["dQ"].append(O.dq_rows(data["q"], data["k"], data["v"], data["do"], sl, b, h,
                                            rows, **kw))
                gots["dQ"].append(gpu["dQ"][b, h, rows])
            if "dK" in gpu:
                dk, dv = O.dkdv_rows(data["q"], data["k"], data["v"], data["do"], sl, b, h, rows, **kw)
                refs["dK"].append(dk)
                refs["dV"].append(dv)
                gots["dK"].append(gpu["dK"][b, h, rows])
                gots["dV"].append(gpu["dV"][b, h, rows])
    out = {}
    for k in gpu:
        r, g = np.concatenate(refs[k]), np.concatenate(gots[k])
        out[k] = err_ratio(g, r, np.ones(r.shape, bool))
    return out


def _measure(name):
    torch = need_gpu()
    data = _data(name)
    note(f"precision modes on {name}")
    single = run_gpu(data, torch.bfloat16, out_dtype=torch.float32, fast_math=1)
    f16 = run_gpu(data, torch.bfloat16, passes=("o",), out_dtype=torch.float32, fast_math=2)
    split = run_gpu(data, torch.bfloat16, out_dtype=torch.float32, fast_math=0)
    if name in FULL:
        ref = oracle_full(data) if name == "tiny_bf16" else oracle_full_named(name)
        res = {m: _full_ratios(data, g, ref) for m, g in (("bf16", single), ("f16", f16),
                                                          ("split", split))}
    else:
        res = {m: _sampled_ratios(data, g) for m, g in (("bf16", single), ("f16", f16),
                                                        ("split", split))}
    line = "; ".join(f"{m}: " + " ".join(f"{k} {v:.2e}" for k, v in r.items())
                     for m, r in res.items())
    print(f"[precision] {name}: {line}", flush=True)
    return res


@pytest.mark.parametrize("name", FULL + SAMPLED)
def test_operand_precision_on_the_benchmark_set(name):
    res = _measure(name)
    # the default split and the f16 forward meet the bar on every configuration
    for k, v in res["split"].items():
        assert v <= BF16_TOL, f"{name} split {k}: {v:.3e}"
    assert res["f16"]["O"] <= BF16_TOL, f"{name} f16 O: {res['f16']['O']:.3e}"
    # single bf16 operands miss it on these two, through the rounding of the largest
    # weights of some rows
    if name in ("bidir_2k", "causal_gated_512"):
        worst = max(res["bf16"].values())
        assert worst > BF16_TOL, f"{name}: single bf16 unexpectedly within the bar ({worst:.3e})"


def _f16_error(p):
    """|2^14 p - f16(2^14 p)| / 2^14: the forward's f16 rounding of a weight p."""
    x = np.float32(p) * np.float32(16384.0)
    return abs(float(np.float16(x)) - float(x)) / 16384.0


def test_f16_forward_misses_the_bar_on_dominant_key_rows():
    """A 4096-token sequence in which two queries put weight 0.55 and 0.81 on one key
    each, whose value is 8 in one feature: those two output entries are far above the
    batch rms (about 0.045), and an f16 rounding of the weight (up to 2^-12 absolute,
    picked near its worst case) moves them by about 2e-3, over 4 % of the rms. The
    default split's weight error is below 2^-17 relative."""
    torch = need_gpu()
    w = W.Workload("dominant_keys", "bf16", 1, 2, 64, 4096, ("fixed", [4096]), seed=77)
    data = W.generate(w)
    q, k, v = data["q"], data["k"], data["v"]
    n, s = 4096, 1.0 / 8.0
    for i, j in ((3, 1000), (7, 2500)):
        kj = k[0, 0, j].astype(np.float64)
        best = None
        for c in np.linspace(0.9, 1.4, 4000):
            qi = W.round_to_bf16((c * kj).astype(np.float32)).astype(np.float64)
            p = 1.0 / (1.0 + np.exp(-(s * qi.dot(kj) - np.log(n))))
            if 0.55 < p < 0.9 and (best is None or _f16_error(p) > best[0]):
                best = (_f16_error(p), c)
        q[0, 0, i] = W.round_to_bf16((best[1] * kj).astype(np.float32))
        v[0, 0, j, 0] = 8.0
    data["q"] = W.round_to_bf16(q)
    data["v"] = W.round_to_bf16(v)
    ref = O.forward(data["q"], data["k"], data["v"], data["seqlens"])
    mask = np.ones(ref.shape[:3], bool)
    note("dominant-key rows: single bf16, f16 and the default split")
    res = {}
    for mode in (1, 2, 0):
        g = run_gpu(data, torch.bfloat16, passes=("o",), out_dtype=torch.float32, fast_math=mode)
        res[mode] = err_ratio(g["O"], ref, mask)
    print(f"[precision] dominant-key rows: O bf16 {res[1]:.2e}, f16 {res[2]:.2e}, "
          f"split {res[0]:.2e}", flush=True)
    assert res[0] <= 1e-3, f"split: {res[0]:.3e}"
    assert res[2] > BF16_TOL, f"f16 unexpectedly within the bar: {res[2]:.3e}"
    assert res[1] > BF16_TOL

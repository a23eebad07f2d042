"""GPU checks of the one-call backward (sigattn_bwd), through the C ABI.

Its dQ, dK and dV must be bitwise those of sigattn_bwd_dq and sigattn_bwd_dkdv on the
same inputs (the same kernel bodies; at d = 64 only the launch is shared), for every
mode: bidirectional, causal, gated with dropped keys, fast math, bf16 and float outputs,
the float32 debug path, and the full-size benchmark shape. One small case is also held
to the stated bar against the fp64 oracle directly, padded rows exactly 0."""

import numpy as np
import pytest

import oracle as O
import sigmoid_attention_amd as S
import workloads as W
from gpu_util import BF16_TOL, check_all, err_ratio, need_gpu, note, oracle_full, to_device

pytestmark = pytest.mark.gpu

VARIANTS = {
    "bidir": dict(),
    "causal": dict(causal=True),
    "causal_gated_drop": dict(causal=True, gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01),
                              tau=0.05, sink=4),
    "gated_drop": dict(gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01), tau=0.05, sink=4),
}


def _both(torch, data, torch_dtype=None, **extra):
    torch_dtype = torch_dtype or torch.bfloat16
    t = to_device(data, torch_dtype)
    kw = dict(causal=bool(data["causal"]), gate=t["gate"], tau=float(data["tau"]),
              sink=int(data["sink"]), **extra)
    sl = data["seqlens"]
    fused = S.bwd(t["q"], t["k"], t["v"], t["do"], sl, **kw)
    dq = S.bwd_dq(t["q"], t["k"], t["v"], t["do"], sl, **kw)
    dk, dv = S.bwd_dkdv(t["q"], t["k"], t["v"], t["do"], sl, **kw)
    torch.cuda.synchronize()
    return fused, (dq, dk, dv)


def _assert_bitwise(torch, fused, sep, label):
    for name, a, b in zip(("dQ", "dK", "dV"), fused, sep):
        assert a.dtype == b.dtype and a.shape == b.shape
        assert torch.equal(a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                           b.view(torch.int16 if b.element_size() == 2 else torch.int32)), \
            f"{label} {name}: one-call backward differs from the separate passes"


@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("d", [64, 128])
def test_bitwise_equal_to_separate_passes(d, variant, fast):
    torch = need_gpu()
    w = W.Workload(f"fused_{variant}_{d}", "bf16", 5, 3, d, 700, ("fixed", [700, 0, 1, 333, 129]),
                   seed=600 + d + len(variant) + fast, **VARIANTS[variant])
    data = W.generate(w)
    note(f"one-call backward d={d} {variant} fast={fast}")
    for od in (torch.float32, torch.bfloat16):
        fused, sep = _both(torch, data, out_dtype=od, fast_math=fast)
        _assert_bitwise(torch, fused, sep, f"d={d} {variant} fast={fast} out={od}")


@pytest.mark.parametrize("variant", ["causal", "causal_gated_drop"])
@pytest.mark.parametrize("shape", [(16, 12, 512), (5, 3, 700), (2, 4, 4096), (1, 2, 8193),
                                   (3, 1, 1)])
def test_one_length_causal_bitwise(shape, variant):
    """Causal batches of one length: the one-call list merges both passes' tile blocks by
    cost (the separate passes take their own block orders); bitwise the same results.
    At 8193 rows the one-call list (130 tile blocks) keeps the per-sequence order while
    the separate passes (65 each) are block-major."""
    torch = need_gpu()
    B, H, L = shape
    w = W.Workload(f"fused_one_length_{variant}_{B}x{H}_{L}", "bf16", B, H, 64, L,
                   ("fixed", [L] * B), seed=640 + B + L, **VARIANTS[variant])
    data = W.generate(w)
    note(f"one-call backward, one length {B}x{H}x{L} {variant}")
    for od in (torch.float32, torch.bfloat16):
        fused, sep = _both(torch, data, out_dtype=od)
        _assert_bitwise(torch, fused, sep, f"one length {shape} {variant} out={od}")


@pytest.mark.parametrize("d", [64, 128])
def test_against_oracle(d):
    torch = need_gpu()
    w = W.Workload(f"fused_oracle_{d}", "bf16", 3, 2, d, 400, ("fixed", [400, 65, 1]), seed=620 + d,
                   causal=True, gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01), tau=0.05, sink=4)
    data = W.generate(w)
    note(f"one-call backward against the oracle d={d}")
    fused, _ = _both(torch, data, out_dtype=torch.float32)
    gpu = {n: x.cpu().numpy() for n, x in zip(("dQ", "dK", "dV"), fused)}
    ref = oracle_full(data)
    print(check_all(gpu, ref, data["seqlens"], BF16_TOL, f"one-call d={d}"))


def test_float32_debug_path():
    torch = need_gpu()
    w = W.WORKLOADS["tiny_fp32"]
    data = W.generate(w)
    note("one-call backward, float32 inputs")
    fused, sep = _both(torch, data, torch_dtype=torch.float32)
    _assert_bitwise(torch, fused, sep, "float32 path")


def test_benchmark_shape_bitwise_and_sampled():
    """long_8k_s1 (4 x 12 heads, n up to 7527, 4272 work items in one launch): bitwise
    equal to the separate passes, and sampled rows against the oracle."""
    torch = need_gpu()
    data = W.generate(W.WORKLOADS["long_8k_s1"])
    note("one-call backward long_8k_s1")
    fused, sep = _both(torch, data, out_dtype=torch.float32)
    _assert_bitwise(torch, fused, sep, "long_8k_s1")
    sl = data["seqlens"]
    dq, dk, dv = (x.cpu().numpy() for x in fused)
    for b, h in ((0, 0), (2, 11)):
        n = int(sl[b])
        rows = np.array([0, 1, 127, 128, n // 2, n - 1])
        rq = O.dq_rows(data["q"], data["k"], data["v"], data["do"], sl, b, h, rows)
        rk, rv = O.dkdv_rows(data["q"], data["k"], data["v"], data["do"], sl, b, h, rows)
        for name, got, ref in (("dQ", dq[b, h, rows], rq), ("dK", dk[b, h, rows], rk),
                               ("dV", dv[b, h, rows], rv)):
            e = err_ratio(got, ref, np.ones(ref.shape, bool))
            assert e <= BF16_TOL, f"long_8k_s1 b={b} h={h} {name}: {e:.3e}"
        assert np.all(dq[b, h, n:] == 0) and np.all(dk[b, h, n:] == 0) and np.all(dv[b, h, n:] == 0)

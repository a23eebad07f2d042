"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same
seeded input bits. The stated bar, max |gpu - ref| / rms(ref) <= 2e-2 over valid rows
(1e-5 on the float32 debug path), is checked with float outputs in the default split
precision, which is also what the benchmark times. bf16 outputs and fast math are
checked against element-wise bounds derived from bf16 rounding (see gpu_util). Padded
rows must be exactly 0 in every mode."""

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import (BF16_TOL, F32_TOL, bound_excess, check_all, check_bounds, err_ratio,
                      need_gpu, note, oracle_full, oracle_full_named, oracle_kwargs,
                      oracle_magnitudes, run_gpu)

pytestmark = pytest.mark.gpu


def test_tiny_fp32_debug_path():
    """Workload tiny_fp32 (B=2, H=2, d=64, Lmax=128, n = {128, 77}) on the float32 path."""
    torch = need_gpu()
    data = W.generate("tiny_fp32")
    note("tiny_fp32 f32 debug path: fwd, dq, dkdv")
    gpu = run_gpu(data, torch.float32)
    rep = check_all(gpu, oracle_full(data), data["seqlens"], F32_TOL, "tiny_fp32")
    print(rep)


def test_tiny_fp32_bf16_path():
    """The same tiny workload with bf16 inputs through the MFMA kernels."""
    torch = need_gpu()
    w = W.get("tiny_fp32", dtype="bf16")
    data = W.generate(w)
    ref, mag = oracle_full(data), oracle_magnitudes(data)
    note("tiny bf16 inputs, float outputs: fwd, dq, dkdv")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    print(check_all(gpu, ref, data["seqlens"], BF16_TOL, "tiny bf16"))
    for bf16_out in (False, True):
        for fast in (False, True):
            note(f"tiny bf16 inputs, bf16_out={bf16_out} fast_math={fast}")
            gpu = run_gpu(data, torch.bfloat16, out_dtype=None if bf16_out else torch.float32,
                          fast_math=fast)
            print(bf16_out, fast, check_bounds(gpu, ref, mag, data["seqlens"], bf16_out, fast))


SMALL_VARIANTS = {
    "bidir": dict(),
    "causal": dict(causal=True),
    "gated": dict(gate=("logistic_normal", 1.0, 2.0)),
    "causal_gated_drop": dict(causal=True, gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01),
                              tau=0.05, sink=4),
}


@pytest.mark.parametrize("variant", list(SMALL_VARIANTS))
@pytest.mark.parametrize("d", [64, 128])
def test_small_full_parity(d, variant):
    """Several tiles with ragged tails (n = 600, 333, 1, 64, 65) compared element by
    element with the full oracle."""
    torch = need_gpu()
    w = W.Workload(f"small_{variant}_{d}", "bf16", 5, 3, d, 600,
                   ("fixed", [600, 333, 1, 64, 65]), seed=21 + d, **SMALL_VARIANTS[variant])
    data = W.generate(w)
    ref, mag = oracle_full(data), oracle_magnitudes(data)
    note(f"small d={d} {variant}: float outputs")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    print(check_all(gpu, ref, data["seqlens"], BF16_TOL, f"small {variant} {d}"))
    print(check_bounds(gpu, ref, mag, data["seqlens"], False, False))
    note(f"small d={d} {variant}: bf16 outputs, fast math")
    gpu = run_gpu(data, torch.bfloat16, fast_math=True)
    print(check_bounds(gpu, ref, mag, data["seqlens"], True, True, f"small {variant} {d} fast"))


@pytest.mark.parametrize("variant", ["bidir", "causal_gated_drop"])
@pytest.mark.parametrize("d", [64, 128])
def test_lengths_at_chunk_multiples(d, variant):
    """Lengths that are exact multiples of the 32-row chunk, odd and even numbers of them
    (a tile of two chunks is then half valid), next to 1 and 64 + 1; full comparison."""
    torch = need_gpu()
    w = W.Workload(f"chunk_mult_{variant}_{d}", "bf16", 7, 2, d, 300,
                   ("fixed", [96, 32, 160, 288, 64, 1, 65]), seed=31 + d,
                   **SMALL_VARIANTS[variant])
    data = W.generate(w)
    note(f"chunk-multiple lengths d={d} {variant}")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    print(check_all(gpu, oracle_full(data), data["seqlens"], BF16_TOL, f"chunks {variant} {d}"))


@pytest.mark.parametrize("variant", ["bidir", "causal_gated_drop"])
def test_d128_long_query_tiles(variant):
    """d = 128 batches whose longest sequence reaches 1024 query rows run the dK/dV pass
    with 64-row query tiles; full comparison with a ragged partner sequence."""
    torch = need_gpu()
    w = W.Workload(f"d128_long_tiles_{variant}", "bf16", 2, 2, 128, 1100, ("fixed", [1100, 301]),
                   seed=77, **SMALL_VARIANTS[variant])
    data = W.generate(w)
    note(f"d=128 long query tiles {variant}")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    print(check_all(gpu, oracle_full(data), data["seqlens"], BF16_TOL, f"d128 long {variant}"))


ONE_LENGTH = [(64, 16, 8, 512), (128, 16, 8, 512), (64, 5, 3, 700), (128, 5, 3, 700)]


@pytest.mark.parametrize("d,B,H,L", ONE_LENGTH)
def test_one_length_causal_full(d, B, H, L):
    """Causal gated batches whose sequences share one length take block-major work lists
    (and, for 16 x 8 heads of 512 rows, the snake placement of a one-round forward);
    every pass, and the one-call backward, against the full oracle."""
    torch = need_gpu()
    w = W.Workload(f"one_length_{d}_{B}x{H}_{L}", "bf16", B, H, d, L, ("fixed", [L] * B),
                   seed=40 + d + L, causal=True, gate=("logistic_normal", 2.0, 2.0, 0.2, 0.01),
                   tau=0.05, sink=4)
    data = W.generate(w)
    ref = oracle_full(data)
    note(f"one-length causal d={d} B={B} H={H} L={L}: separate passes")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    print(check_all(gpu, ref, data["seqlens"], BF16_TOL, f"one-length {d} {B}x{H} {L}"))
    note(f"one-length causal d={d} B={B} H={H} L={L}: one-call backward")
    import sigmoid_attention_amd as S
    from gpu_util import kwargs_of, to_device
    t = to_device(data, torch.bfloat16)
    dq, dk, dv = S.bwd(t["q"], t["k"], t["v"], t["do"], data["seqlens"],
                       out_dtype=torch.float32, **kwargs_of(data, t["gate"]))
    torch.cuda.synchronize()
    fused = {"dQ": dq.cpu().numpy(), "dK": dk.cpu().numpy(), "dV": dv.cpu().numpy()}
    print(check_all(fused, ref, data["seqlens"], BF16_TOL, f"one-length one-call {d}"))


@pytest.mark.parametrize("name", ["causal_gated_512", "causal_forced_drop_512"])
def test_causal_gated_full(name):
    """Causal GPT-2-shaped gated layer (B=16, H=12, d=64, L=512) against the full oracle."""
    torch = need_gpu()
    data = W.generate(name)
    ref, mag = oracle_full(data), oracle_magnitudes(data)
    note(f"{name} full size, float outputs")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    print(check_all(gpu, ref, data["seqlens"], BF16_TOL, name))
    note(f"{name} full size, bf16 outputs, fast math")
    gf = run_gpu(data, torch.bfloat16, fast_math=True)
    print(check_bounds(gf, ref, mag, data["seqlens"], True, True, name + " fast"))
    if name == "causal_forced_drop_512":
        g = data["gate"]
        dropped = (g < data["tau"]) & (np.arange(g.shape[1])[None, :] >= data["sink"])
        assert dropped.sum() > 100
        for b, j in zip(*np.nonzero(dropped)):
            assert np.all(gpu["dK"][b, :, j] == 0) and np.all(gpu["dV"][b, :, j] == 0)


def _sample_rows(n, L, rng, tile=64):
    """Row indices that hit the first/last valid rows, tile boundaries, random interior
    rows, and padded rows."""
    rows = {0, 1, n - 1, max(0, n - 2), min(L - 1, n), L - 1}
    for t in range(tile, n, tile * 7):
        rows.update({t - 1, t})
    rows.update(rng.integers(0, max(n, 1), size=6).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < L))


@pytest.mark.parametrize("name", ["bidir_2k", "long_8k_s1", "long_8k_s4",
                                  "pad_sweep_0", "pad_sweep_25", "pad_sweep_50",
                                  "sweep_16k_d64_p25", "sweep_16k_d128", "sweep_512_d128_p25"])
def test_full_size_sampled(name):
    """Full-size workloads in the launch configuration the benchmark times, checked on
    sampled rows (first and last, tile edges, random) of the first and last head of every
    batch entry, which the oracle computes one by one."""
    torch = need_gpu()
    data = W.generate(name)
    note(f"{name} full size: fwd, dq, dkdv, float outputs")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    note(f"{name} full size: fwd, dq, dkdv, bf16 outputs, fast math")
    gfast = run_gpu(data, torch.bfloat16, fast_math=True)
    kw = oracle_kwargs(data)
    sl = data["seqlens"]
    B, H, L, d = data["q"].shape
    rng = np.random.default_rng(5)
    # every batch entry, its first and last head
    picks = {(b, h) for b in range(B) if sl[b] > 0 for h in (0, H - 1)}
    refs = {"O": [], "dQ": [], "dK": [], "dV": []}
    gots = {"O": [], "dQ": [], "dK": [], "dV": []}
    fasts = {"O": [], "dQ": [], "dK": [], "dV": []}
    mags = {"O": [], "dQ": [], "dK": [], "dV": []}
    for b, h in sorted(picks):
        n = int(sl[b])
        rows = _sample_rows(n, L, rng)
        live = rows < n
        o = O.forward_rows(data["q"], data["k"], data["v"], sl, b, h, rows, **kw)
        dq = O.dq_rows(data["q"], data["k"], data["v"], data["do"], sl, b, h, rows, **kw)
        dk, dv = O.dkdv_rows(data["q"], data["k"], data["v"], data["do"], sl, b, h, rows, **kw)
        ao = O.forward_rows(data["q"], data["k"], np.abs(data["v"]), sl, b, h, rows, **kw)
        adq = O.dq_rows(data["q"], data["k"], data["v"], data["do"], sl, b, h, rows,
                        absolute=True, **kw)
        adk, adv = O.dkdv_rows(data["q"], data["k"], data["v"], data["do"], sl, b, h, rows,
                               absolute=True, **kw)
        for key, ref, mag in (("O", o, ao), ("dQ", dq, adq), ("dK", dk, adk), ("dV", dv, adv)):
            got = gpu[key][b, h, rows]
            fst = gfast[key][b, h, rows]
            assert np.all(got[~live] == 0.0) and np.all(fst[~live] == 0.0), \
                f"{name} {key}: padded rows not zero"
            assert np.all(np.isfinite(got[live])) and np.all(np.isfinite(fst[live]))
            refs[key].append(ref[live])
            gots[key].append(got[live])
            fasts[key].append(fst[live])
            mags[key].append(mag[live])
    report = {}
    for key in refs:
        r, g = np.concatenate(refs[key]), np.concatenate(gots[key])
        f, m = np.concatenate(fasts[key]), np.concatenate(mags[key])
        report[key] = err_ratio(g, r, np.ones(r.shape, bool))
        rms = float(np.sqrt(np.mean(r * r)))
        fast_x = bound_excess(f, r, m, True, True, rms)
        print(f"{name} {key}: ratio {report[key]:.3e} (float out); fast bf16 bound use {fast_x:.2f}")
        assert report[key] <= BF16_TOL, f"{name} {key}: error ratio {report[key]:.3e}"
        assert fast_x <= 1.0, f"{name} {key}: fast path exceeds its derived bound ({fast_x:.2f}x)"
    # no output anywhere is NaN/Inf and every padded row is exactly 0
    mask = np.broadcast_to(np.arange(L)[None, None, :] < sl[:, None, None], (B, H, L))
    for out in (gpu, gfast):
        for key in ("O", "dQ", "dK", "dV"):
            assert np.all(np.isfinite(out[key][mask]))
            assert np.all(out[key][~mask] == 0.0)


def test_bidir_2k_full():
    """The 2K bidirectional batch (B=8, H=16, d=64, n ~ U{1024..2048}) compared element
    by element with the full fp64 oracle: every valid row of O, dQ, dK, dV of every head
    at the stated bar, padded rows exactly 0."""
    torch = need_gpu()
    data = W.generate("bidir_2k")
    note("bidir_2k full comparison, float outputs")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    print(check_all(gpu, oracle_full_named("bidir_2k"), data["seqlens"], BF16_TOL, "bidir_2k full"))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_values_beyond_f16(d, causal):
    """fast_math = 2 with V values beyond the f16 range (|v| >= 2^16) in some tiles: those
    items run again on bf16 hi + lo operands; everything still meets the stated bar,
    padded rows 0 (and the default mode, which never converts V, too)."""
    torch = need_gpu()
    w = W.Workload(f"big_v_{d}", "bf16", 3, 2, d, 600, ("fixed", [600, 333, 65]),
                   seed=700 + d + causal, causal=causal)
    data = W.generate(w)
    v = data["v"]
    v[0, 1, 100:104] *= 3e5                      # one tile of one head
    v[2, 0, 64] = W.round_to_bf16(np.full(d, -7.0e4, np.float32))
    v[1, 0, 5, 3] = np.float32(65280.0)           # the largest bf16 below 2^16 stays f16
    data["v"] = W.round_to_bf16(v)
    ref, mag = oracle_full(data), oracle_magnitudes(data)
    for mode in (2, 0):
        note(f"V beyond f16 d={d} causal={causal} fast_math={mode}")
        gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32, fast_math=mode)
        print(check_all(gpu, ref, data["seqlens"], BF16_TOL, f"big V {d}"))
        print(check_bounds(gpu, ref, mag, data["seqlens"], False, False, f"big V {d}", f16=mode == 2))


@pytest.mark.parametrize("variant", list(SMALL_VARIANTS))
@pytest.mark.parametrize("d", [64, 128])
def test_f16_forward_mode(d, variant):
    """fast_math = 2 (P V on f16 operands in the forward, hi + lo backward): the stated
    bar and the f16 bound on the forward output for ragged batches whose rows are of
    similar size; dQ, dK, dV bitwise those of the default mode."""
    torch = need_gpu()
    w = W.Workload(f"f16mode_{variant}_{d}", "bf16", 4, 3, d, 700, ("fixed", [700, 333, 129, 600]),
                   seed=740 + d, **SMALL_VARIANTS[variant])
    data = W.generate(w)
    ref, mag = oracle_full(data), oracle_magnitudes(data)
    note(f"f16 forward mode d={d} {variant}")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32, fast_math=2)
    print(check_all(gpu, ref, data["seqlens"], BF16_TOL, f"f16 mode {variant} {d}"))
    print(check_bounds(gpu, ref, mag, data["seqlens"], False, False, f"f16 mode {variant} {d}", f16=True))
    base = run_gpu(data, torch.bfloat16, passes=("dq", "dkdv"), out_dtype=torch.float32)
    for name in ("dQ", "dK", "dV"):
        assert np.array_equal(gpu[name], base[name]), f"{name} differs from the default mode"


def test_f16_forward_mode_long_sampled():
    """fast_math = 2 at the benchmark shape (long_8k_s1), sampled rows against the oracle."""
    torch = need_gpu()
    data = W.generate(W.WORKLOADS["long_8k_s1"])
    note("f16 forward mode long_8k_s1")
    gpu = run_gpu(data, torch.bfloat16, passes=("o",), out_dtype=torch.float32, fast_math=2)
    sl = data["seqlens"]
    for b, h in ((0, 0), (3, 5)):
        n = int(sl[b])
        rows = np.array([0, 1, 127, 128, n // 2, n - 1])
        ref = O.forward_rows(data["q"], data["k"], data["v"], sl, b, h, rows)
        e = err_ratio(gpu["O"][b, h, rows], ref, np.ones(ref.shape, bool))
        assert e <= BF16_TOL, f"long_8k_s1 f16 mode b={b} h={h}: {e:.3e}"


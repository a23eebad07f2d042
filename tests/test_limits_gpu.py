"""GPU parity at the boundary's limits, through the C ABI: the longest sequence the
padded entry points accept (Lmax = 65535), the largest batch (B = 256), and tensors that
are strided views of a [B, L, H, d] buffer rather than contiguous [B, H, L, d]. Checked
against the fp64 oracle at the stated bar (float outputs), padded rows exactly 0."""

import numpy as np
import pytest

import oracle as O
import sigmoid_attention_amd as S
import workloads as W
from gpu_util import BF16_TOL, check_all, err_ratio, need_gpu, note, oracle_full, run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
def test_longest_sequence(d):
    """Lmax = 65535 (the cap), one head: a full-length sequence and a ragged one, every
    pass, sampled rows against the oracle."""
    torch = need_gpu()
    L = 65535
    w = W.Workload(f"limit_L_{d}", "bf16", 2, 1, d, L, ("fixed", [L, 40001]), seed=500 + d)
    data = W.generate(w)
    note(f"Lmax=65535 d={d}: fwd, dq, dkdv")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    sl = data["seqlens"]
    for b in range(2):
        n = int(sl[b])
        rows = np.array([0, 1, 127, 128, n // 2, n - 2, n - 1, min(n, L - 1), L - 1])
        live = rows < n
        o = O.forward_rows(data["q"], data["k"], data["v"], sl, b, 0, rows)
        dq = O.dq_rows(data["q"], data["k"], data["v"], data["do"], sl, b, 0, rows)
        dk, dv = O.dkdv_rows(data["q"], data["k"], data["v"], data["do"], sl, b, 0, rows)
        for name, ref in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
            got = gpu[name][b, 0, rows]
            assert np.all(got[~live] == 0.0), f"{name}: padded rows not 0"
            e = err_ratio(got[live], ref[live], np.ones(ref[live].shape, bool))
            print(f"L=65535 d={d} b={b} {name}: {e:.3e}")
            assert e <= BF16_TOL


@pytest.mark.parametrize("causal", [False, True])
def test_largest_batch(causal):
    """B = 256 (the cap) short ragged sequences, including empty ones; full comparison."""
    torch = need_gpu()
    rng = np.random.default_rng(510)
    lens = rng.integers(0, 300, 256)
    lens[:4] = [0, 1, 299, 128]
    w = W.Workload("limit_B", "bf16", 256, 2, 64, 300, ("fixed", lens.tolist()), seed=511,
                   causal=causal)
    data = W.generate(w)
    note(f"B=256 causal={causal}")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    print(check_all(gpu, oracle_full(data), data["seqlens"], BF16_TOL, "B=256"))


@pytest.mark.parametrize("d", [64, 128])
def test_strided_blhd_views(d):
    """q, k, v, dO as [B, H, L, d] views of [B, L, H, d] buffers (stride_l = H d,
    stride_h = d): the same results as the oracle, padded rows 0."""
    torch = need_gpu()
    w = W.Workload(f"limit_view_{d}", "bf16", 3, 4, d, 700, ("fixed", [700, 333, 64]),
                   seed=520 + d, causal=True, gate=("logistic_normal", 1.0, 2.0, 0.2, 0.01),
                   tau=0.05, sink=4)
    data = W.generate(w)
    ref = oracle_full(data)
    dev = torch.device("cuda")
    t = {}
    for name in ("q", "k", "v", "do"):
        blhd = torch.from_numpy(np.ascontiguousarray(data[name].transpose(0, 2, 1, 3)))
        t[name] = blhd.to(torch.bfloat16).to(dev).transpose(1, 2)     # [B, H, L, d] view
    assert t["q"].stride(2) == 4 * d and t["q"].stride(1) == d
    gate = torch.from_numpy(data["gate"]).to(dev)
    kw = dict(causal=True, gate=gate, tau=0.05, sink=4, out_dtype=torch.float32)
    sl = data["seqlens"]
    note(f"BLHD views d={d}")
    o = torch.empty_strided(t["q"].shape, t["q"].stride(), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(o) for _ in range(3))
    S.fwd(t["q"], t["k"], t["v"], sl, out=o, **kw)
    S.bwd_dq(t["q"], t["k"], t["v"], t["do"], sl, out=dq, **kw)
    S.bwd_dkdv(t["q"], t["k"], t["v"], t["do"], sl, out=(dk, dv), **kw)
    torch.cuda.synchronize()
    gpu = {"O": o.cpu().numpy(), "dQ": dq.cpu().numpy(), "dK": dk.cpu().numpy(),
           "dV": dv.cpu().numpy()}
    print(check_all(gpu, ref, sl, BF16_TOL, f"BLHD d={d}"))


@pytest.mark.parametrize("variant", ["bidir", "causal", "causal_gated_drop"])
@pytest.mark.parametrize("d", [64, 128])
def test_every_length_up_to_256(d, variant):
    """One batch holding every length 1..256 (every residue modulo the 32-row chunk and
    the 128-row tile, odd and even chunk counts), all passes against the oracle."""
    torch = need_gpu()
    kw = {"bidir": dict(), "causal": dict(causal=True),
          "causal_gated_drop": dict(causal=True, gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01),
                                    tau=0.05, sink=4)}[variant]
    w = W.Workload(f"every_len_{variant}_{d}", "bf16", 256, 1, d, 256,
                   ("fixed", list(range(1, 257))), seed=530 + d, **kw)
    data = W.generate(w)
    note(f"every length 1..256 d={d} {variant}")
    gpu = run_gpu(data, torch.bfloat16, out_dtype=torch.float32)
    print(check_all(gpu, oracle_full(data), data["seqlens"], BF16_TOL, f"every length {d} {variant}"))

"""GPU parity of the side outputs against the fp64 oracle: the gate gradient
(sigattn_bwd_dkdv_dg) and the row mass (sigattn_fwd_rowsum).

Gate gradient:

dg_hj = sum_i dS_ij / (g_j + eps) + v_j . sum_i P_ij dO_i per head, and dg_j = sum_h dg_hj
for the gate shared by the heads (chain rule through the gate injection of "Sigmoid
Attention as a Better Substrate for Learned KV Cache Eviction"). The bar is the stated
one, max |gpu - ref| / rms(ref) <= 2e-2 over valid keys for bf16 inputs (1e-5 on the
float32 debug path); fast math is held to the bound that rounding P to bf16 implies.
Padded and dropped keys must be exactly 0, dK and dV must be bitwise those of
sigattn_bwd_dkdv, and dg must be the in-order float sum of dg_head over heads.

Row mass: R_i = sum_j P_ij over the allowed keys of query i (the row-sum diagnostic of
the KV-eviction paper), checked at the same bar; O must be bitwise that of sigattn_fwd
and padded rows exactly 0.
"""

import numpy as np
import pytest

import oracle as O
import sigmoid_attention_amd as S
import workloads as W
from gpu_util import BF16_TOL, F32_TOL, bound_excess, err_ratio, need_gpu, note, oracle_kwargs

pytestmark = pytest.mark.gpu


def _gpu_dg(data, torch, in_dtype, out_dtype=None, fast_math=False):
    t = {n: torch.from_numpy(np.ascontiguousarray(data[n])).to(in_dtype).cuda()
         for n in ("q", "k", "v", "do")}
    gate = torch.from_numpy(data["gate"]).cuda()
    kw = dict(causal=bool(data["causal"]), gate=gate, tau=float(data["tau"]),
              sink=int(data["sink"]), out_dtype=out_dtype, fast_math=fast_math)
    sl = data["seqlens"]
    dk, dv, dgh, dg = S.bwd_dkdv_dg(t["q"], t["k"], t["v"], t["do"], sl, **kw)
    dk0, dv0 = S.bwd_dkdv(t["q"], t["k"], t["v"], t["do"], sl, **kw)
    torch.cuda.synchronize()
    out = {n: x.float().cpu().numpy() for n, x in
           (("dK", dk), ("dV", dv), ("dK0", dk0), ("dV0", dv0), ("dg_head", dgh), ("dg", dg))}
    return out


def _key_mask(data):
    B, H, L, _ = data["q"].shape
    sl = np.asarray(data["seqlens"])
    valid = np.arange(L)[None, :] < sl[:, None]
    g = data["gate"]
    dropped = valid & (g < data["tau"]) & (np.arange(L)[None, :] >= data["sink"])
    return valid, dropped


def _check(gpu, data, fast_math=False, tol=BF16_TOL, label=""):
    kw = oracle_kwargs(data)
    args = (data["q"], data["k"], data["v"], data["do"], data["seqlens"])
    ref_h, ref = O.gate_grad(*args, **kw)
    mag_h, _ = O.gate_grad(*args, absolute=True, **kw)
    valid, dropped = _key_mask(data)
    H = data["q"].shape[1]
    vh = np.broadcast_to(valid[:, None, :], ref_h.shape)
    # exact structure
    assert np.array_equal(gpu["dK"], gpu["dK0"]), f"{label}: dK differs from bwd_dkdv"
    assert np.array_equal(gpu["dV"], gpu["dV0"]), f"{label}: dV differs from bwd_dkdv"
    assert np.all(gpu["dg_head"][~vh] == 0.0), f"{label}: padded dg_head not 0"
    assert np.all(gpu["dg"][~valid] == 0.0), f"{label}: padded dg not 0"
    assert np.all(gpu["dg"][dropped] == 0.0), f"{label}: dropped keys have dg != 0"
    assert np.all(np.isfinite(gpu["dg_head"])) and np.all(np.isfinite(gpu["dg"]))
    seq = np.zeros_like(gpu["dg"], dtype=np.float32)
    for h in range(H):
        seq = seq + gpu["dg_head"][:, h, :].astype(np.float32)
    assert np.array_equal(seq, gpu["dg"]), f"{label}: dg is not the in-order head sum"
    # accuracy
    rep = {}
    for name, g_, r_, m_, mask in (("dg_head", gpu["dg_head"], ref_h, mag_h, vh),
                                   ("dg", gpu["dg"], ref, None, valid)):
        e = err_ratio(g_, r_, mask)
        rep[name] = e
        if not fast_math:
            assert e <= tol, f"{label} {name}: error ratio {e:.3e} > {tol}"
        elif m_ is not None:
            rms = float(np.sqrt(np.mean(r_[mask] ** 2)))
            x = bound_excess(g_[mask], r_[mask], m_[mask], False, True, rms)
            rep[name + "_bound"] = x
            assert x <= 1.0, f"{label} {name}: fast math exceeds its bound ({x:.2f}x)"
    return rep


GATED_VARIANTS = {
    "gated": dict(gate=("logistic_normal", 1.0, 2.0)),
    "causal_gated_drop": dict(causal=True, gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01),
                              tau=0.05, sink=4),
    "gated_drop": dict(gate=("logistic_normal", 0.0, 2.0, 0.2, 0.01), tau=0.05, sink=4),
}


@pytest.mark.parametrize("variant", list(GATED_VARIANTS))
@pytest.mark.parametrize("d", [64, 128])
def test_gate_grad_small(d, variant):
    """Several key tiles with ragged tails and an empty and a one-token sequence."""
    torch = need_gpu()
    w = W.Workload(f"dg_{variant}_{d}", "bf16", 5, 3, d, 600,
                   ("fixed", [600, 0, 1, 129, 333]), seed=41 + d, **GATED_VARIANTS[variant])
    data = W.generate(w)
    note(f"gate grad small d={d} {variant}: float outputs")
    gpu = _gpu_dg(data, torch, torch.bfloat16, out_dtype=torch.float32)
    print(_check(gpu, data, label=f"{variant} {d}"))
    note(f"gate grad small d={d} {variant}: bf16 outputs, fast math")
    gpu = _gpu_dg(data, torch, torch.bfloat16, fast_math=True)
    print(_check(gpu, data, fast_math=True, label=f"{variant} {d} fast"))


def test_gate_grad_f32_debug_path():
    torch = need_gpu()
    w = W.get("tiny_fp32", gate=("logistic_normal", 1.0, 2.0, 0.25, 0.01), tau=0.05, sink=4,
              causal=True)
    data = W.generate(w)
    note("gate grad tiny f32 debug path")
    gpu = _gpu_dg(data, torch, torch.float32)
    print(_check(gpu, data, tol=F32_TOL, label="f32"))


@pytest.mark.parametrize("name", ["causal_gated_512", "causal_forced_drop_512"])
def test_gate_grad_gated_layer_full(name):
    """The gated GPT-2-shaped layer (B=16, H=12, d=64, L=512, causal) against the full
    oracle, in the launch configuration of the other passes."""
    torch = need_gpu()
    data = W.generate(name)
    note(f"gate grad {name} full size")
    gpu = _gpu_dg(data, torch, torch.bfloat16, out_dtype=torch.float32)
    print(_check(gpu, data, label=name))


def test_gate_grad_long_sampled():
    """8192-token sequences with a gate (the long workload's shapes, ragged lengths),
    checked on sampled key rows that the oracle computes one by one."""
    torch = need_gpu()
    w = W.get("long_8k_s1", gate=("logistic_normal", 2.0, 2.0, 0.1, 0.01), tau=0.05, sink=4)
    data = W.generate(w)
    note("gate grad long_8k gated, sampled keys")
    gpu = _gpu_dg(data, torch, torch.bfloat16, out_dtype=torch.float32)
    kw = oracle_kwargs(data)
    sl = data["seqlens"]
    B, H, L, _ = data["q"].shape
    rng = np.random.default_rng(9)
    refs, gots = [], []
    for b, h in ((int(np.argmin(sl)), 0), (int(np.argmax(sl)), H - 1)):
        n = int(sl[b])
        rows = np.unique(np.concatenate([[0, 1, 127, 128, n - 1, min(n, L - 1), L - 1],
                                         rng.integers(0, n, 10)]))
        ref = O.gate_grad_rows(data["q"], data["k"], data["v"], data["do"], sl, data["gate"],
                               b, h, rows, **{k_: v_ for k_, v_ in kw.items() if k_ != "gate"})
        got = gpu["dg_head"][b, h, rows]
        live = rows < n
        assert np.all(got[~live] == 0.0)
        refs.append(ref[live])
        gots.append(got[live])
    r, g = np.concatenate(refs), np.concatenate(gots)
    e = err_ratio(g, r, np.ones(r.shape, bool))
    print("long gated dg_head sampled ratio", e)
    assert e <= BF16_TOL
    assert np.array_equal(gpu["dK"], gpu["dK0"]) and np.array_equal(gpu["dV"], gpu["dV0"])


# ----------------------------------------------------------------------------------
# row mass
# ----------------------------------------------------------------------------------

def _gpu_rm(data, torch, in_dtype, out_dtype=None, fast_math=False):
    t = {n: torch.from_numpy(np.ascontiguousarray(data[n])).to(in_dtype).cuda()
         for n in ("q", "k", "v")}
    gate = None if data["gate"] is None else torch.from_numpy(data["gate"]).cuda()
    kw = dict(causal=bool(data["causal"]), gate=gate, tau=float(data["tau"]),
              sink=int(data["sink"]), out_dtype=out_dtype, fast_math=fast_math)
    o, rm = S.fwd_rowsum(t["q"], t["k"], t["v"], data["seqlens"], **kw)
    o0 = S.fwd(t["q"], t["k"], t["v"], data["seqlens"], **kw)
    torch.cuda.synchronize()
    return {n: x.float().cpu().numpy() for n, x in (("O", o), ("O0", o0), ("R", rm))}


def _check_rm(gpu, data, tol=BF16_TOL, label=""):
    ref = O.row_mass(data["q"], data["k"], data["seqlens"], **oracle_kwargs(data))
    B, H, L, _ = data["q"].shape
    valid = np.arange(L)[None, :] < np.asarray(data["seqlens"])[:, None]
    vh = np.broadcast_to(valid[:, None, :], ref.shape)
    assert np.array_equal(gpu["O"], gpu["O0"]), f"{label}: O differs from sigattn_fwd"
    assert np.all(gpu["R"][~vh] == 0.0), f"{label}: padded row mass not 0"
    assert np.all(np.isfinite(gpu["R"]))
    e = err_ratio(gpu["R"], ref, vh)
    assert e <= tol, f"{label}: row mass error ratio {e:.3e} > {tol}"
    return e


RM_VARIANTS = {
    "bidir": dict(),
    "causal": dict(causal=True),
    "causal_gated_drop": dict(causal=True, gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01),
                              tau=0.05, sink=4),
}


@pytest.mark.parametrize("variant", list(RM_VARIANTS))
@pytest.mark.parametrize("d", [64, 128])
def test_row_mass_small(d, variant):
    torch = need_gpu()
    w = W.Workload(f"rm_{variant}_{d}", "bf16", 5, 3, d, 600,
                   ("fixed", [600, 0, 1, 129, 333]), seed=61 + d, **RM_VARIANTS[variant])
    data = W.generate(w)
    note(f"row mass small d={d} {variant}: float outputs")
    print(_check_rm(_gpu_rm(data, torch, torch.bfloat16, out_dtype=torch.float32), data,
                    label=f"{variant} {d}"))
    note(f"row mass small d={d} {variant}: bf16 outputs, fast math")
    print(_check_rm(_gpu_rm(data, torch, torch.bfloat16, fast_math=True), data,
                    label=f"{variant} {d} fast"))


def test_row_mass_f32_debug_path():
    torch = need_gpu()
    w = W.get("tiny_fp32", gate=("logistic_normal", 1.0, 2.0, 0.25, 0.01), tau=0.05, sink=4)
    data = W.generate(w)
    note("row mass tiny f32 debug path")
    print(_check_rm(_gpu_rm(data, torch, torch.float32), data, tol=F32_TOL, label="f32"))


def test_row_mass_gated_layer_full():
    torch = need_gpu()
    data = W.generate("causal_forced_drop_512")
    note("row mass causal_forced_drop_512 full size")
    print(_check_rm(_gpu_rm(data, torch, torch.bfloat16, out_dtype=torch.float32), data,
                    label="causal_forced_drop_512"))


def test_row_mass_long_sampled():
    """8192-token ragged sequences, sampled query rows: the row mass equals the output
    for values that are 1 in every feature (ungated)."""
    torch = need_gpu()
    data = W.generate("long_8k_s1")
    note("row mass long_8k_s1, sampled rows")
    gpu = _gpu_rm(data, torch, torch.bfloat16, out_dtype=torch.float32)
    sl = data["seqlens"]
    B, H, L, d = data["q"].shape
    ones = np.broadcast_to(np.ones(1), (B, H, L, d))
    rng = np.random.default_rng(10)
    refs, gots = [], []
    for b, h in ((int(np.argmin(sl)), 0), (int(np.argmax(sl)), H - 1)):
        n = int(sl[b])
        rows = np.unique(np.concatenate([[0, 1, 127, 128, n - 1, min(n, L - 1), L - 1],
                                         rng.integers(0, n, 10)]))
        ref = O.forward_rows(data["q"], data["k"], ones, sl, b, h, rows)[:, 0]
        got = gpu["R"][b, h, rows]
        live = rows < n
        assert np.all(got[~live] == 0.0)
        refs.append(ref[live])
        gots.append(got[live])
    r, g = np.concatenate(refs), np.concatenate(gots)
    e = err_ratio(g, r, np.ones(r.shape, bool))
    print("long row mass sampled ratio", e)
    assert e <= BF16_TOL
    assert np.array_equal(gpu["O"], gpu["O0"])


@pytest.mark.parametrize("d", [64, 128])
def test_side_outputs_every_length(d):
    """Gate gradient and row mass on one batch holding every length 1..256, causal with
    dropped keys."""
    torch = need_gpu()
    w = W.Workload(f"side_every_{d}", "bf16", 256, 1, d, 256, ("fixed", list(range(1, 257))),
                   seed=560 + d, causal=True, gate=("logistic_normal", 2.0, 2.0, 0.3, 0.01),
                   tau=0.05, sink=4)
    data = W.generate(w)
    note(f"side outputs, every length 1..256, d={d}")
    print(_check(_gpu_dg(data, torch, torch.bfloat16, out_dtype=torch.float32), data,
                 label=f"dg every {d}"))
    print(_check_rm(_gpu_rm(data, torch, torch.bfloat16, out_dtype=torch.float32), data,
                    label=f"rm every {d}"))


@pytest.mark.parametrize("d", [64, 128])
def test_row_mass_with_values_beyond_f16(d):
    """fast_math = 2 with V beyond the f16 range in some tiles sends those items through
    the second pass on bf16 operands: the row mass is reset with the output, and both
    still equal the oracle's (O bitwise that of sigattn_fwd in the same mode)."""
    torch = need_gpu()
    w = W.Workload(f"rm_big_v_{d}", "bf16", 3, 2, d, 600, ("fixed", [600, 333, 65]),
                   seed=720 + d, causal=True)
    data = W.generate(w)
    v = data["v"]
    v[0, 1, 100:104] *= 3e5
    v[2, 0, 64] = np.float32(-7.0e4)
    data["v"] = W.round_to_bf16(v)
    note(f"row mass with V beyond f16 d={d}")
    gpu = _gpu_rm(data, torch, torch.bfloat16, out_dtype=torch.float32, fast_math=2)
    print(_check_rm(gpu, data, label=f"big V {d}"))
    ref_o = O.forward(data["q"], data["k"], data["v"], data["seqlens"], **oracle_kwargs(data))
    mask = np.broadcast_to(np.arange(600)[None, None, :] < np.asarray(data["seqlens"])[:, None, None],
                           ref_o.shape[:3])
    assert err_ratio(gpu["O"], ref_o, mask) <= BF16_TOL


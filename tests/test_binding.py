"""Host-side checks of the Python binding: every shape, stride, dtype and size the kernels
rely on is verified before a pointer reaches the C ABI. CPU tensors stand in for device
buffers; each case fails on the check under test, before any device is needed."""

import numpy as np
import pytest
import torch

import sigmoid_attention_amd as S


def _qkv(B=2, H=2, L=64, d=64, dtype=torch.bfloat16):
    return [torch.zeros((B, H, L, d), dtype=dtype) for _ in range(3)]


def test_gate_must_be_b_by_lmax():
    q, k, v = _qkv()
    one_row = torch.ones((1, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="gate must be a float32"):
        S.fwd(q, k, v, [64, 10], gate=one_row)


def test_expanded_gate_is_refused():
    q, k, v = _qkv()
    expanded = torch.ones((1, 64), dtype=torch.float32).expand(2, 64)
    assert expanded.stride(0) == 0
    with pytest.raises(ValueError, match="must not overlap"):
        S.fwd(q, k, v, [64, 10], gate=expanded)


def test_bias_needs_one_value_per_sequence():
    with pytest.raises(ValueError, match="bias has 1 entries"):
        S.make_problem(2, 1, 64, 64, [64, 10], bias=[0.0])
    p, keep = S.make_problem(2, 1, 64, 64, [64, 10], bias=[0.0, -1.0])
    assert S.validate(p) == 0


def _packed(rows_q=10, rows_k=12, H=2, d=64):
    q = torch.zeros((rows_q, H, d), dtype=torch.bfloat16)
    k = torch.zeros((rows_k, H, d), dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    do = torch.zeros_like(q)
    cu_q = torch.tensor([0, rows_q], dtype=torch.int32)
    cu_k = torch.tensor([0, rows_k], dtype=torch.int32)
    return q, k, v, do, cu_q, cu_k


def test_varlen_output_must_match_its_input():
    q, k, v, do, cu_q, cu_k = _packed()
    with pytest.raises(ValueError, match="out must match"):
        S.fwd_varlen(q, k, v, cu_q, cu_k, 10, 12, out=torch.zeros((5, 2, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must match"):   # float buffer, bf16 output
        S.fwd_varlen(q, k, v, cu_q, cu_k, 10, 12, out=torch.zeros((10, 2, 64), dtype=torch.float32))
    with pytest.raises(ValueError, match="dk must match"):    # dk shaped like q, not k
        S.bwd_dkdv_varlen(q, k, v, do, cu_q, cu_k, 10, 12,
                          out=(torch.zeros_like(q), torch.zeros_like(k)))
    with pytest.raises(ValueError, match="dq must match"):
        S.bwd_varlen(q, k, v, do, cu_q, cu_k, 10, 12,
                     out=(torch.zeros_like(k), torch.zeros_like(k), torch.zeros_like(k)))
    wide = torch.zeros((10, 2, 128), dtype=torch.bfloat16)[:, :, :64]   # other strides
    with pytest.raises(ValueError, match="dq must match"):
        S.bwd_dq_varlen(q, k, v, do, cu_q, cu_k, 10, 12, out=wide)


def test_varlen_shapes_and_output_dtype():
    q, k, v, do, cu_q, cu_k = _packed()
    with pytest.raises(ValueError, match="out_dtype"):
        S.fwd_varlen(q, k, v, cu_q, cu_k, 10, 12, out_dtype=torch.float16)
    with pytest.raises(ValueError, match="do and q"):
        S.bwd_dq_varlen(q, k, v, do[:5], cu_q, cu_k, 10, 12)
    with pytest.raises(ValueError, match="v and k"):
        S.fwd_varlen(q, k, v[:3], cu_q, cu_k, 10, 12)
    # well-formed arguments on the CPU stop at the device check, before the C ABI
    with pytest.raises(ValueError, match="on a GPU"):
        S.fwd_varlen(q, k, v, cu_q, cu_k, 10, 12)


def _cpu_cache(gated=True):
    return S.KVCache(2, 2, 64, 600, gated=gated, tau=0.05, device="cpu")


def test_decode_workspace_must_be_float32():
    c = _cpu_cache()
    q = torch.zeros((2, 2, 64), dtype=torch.bfloat16)
    small = torch.zeros(c.workspace_size() // 2, dtype=torch.bfloat16)   # same bytes / 2
    with pytest.raises(ValueError, match="workspace must be a contiguous float32"):
        c.decode(q, [0.0, 0.0], workspace=small)
    with pytest.raises(ValueError, match="out_dtype"):
        c.decode(q, [0.0, 0.0], out_dtype=torch.float16)
    with pytest.raises(ValueError, match="bias needs one value"):
        c.decode(q, [0.0])


def test_append_checks_gate_and_status():
    c = _cpu_cache()
    kn = torch.zeros((2, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="g_new is required"):
        c.append(kn, kn.clone())
    with pytest.raises(ValueError, match="g_new must be"):
        c.append(kn, kn.clone(), torch.ones(2, dtype=torch.float64))
    with pytest.raises(ValueError, match="g_new must be"):
        c.append(kn, kn.clone(), torch.ones(3, dtype=torch.float32))
    with pytest.raises(ValueError, match="status must be"):
        c.append(kn, kn.clone(), torch.ones(2, dtype=torch.float32),
                 status=torch.zeros(1, dtype=torch.int64))
    ungated = _cpu_cache(gated=False)
    with pytest.raises(ValueError, match="g_new is required"):
        ungated.append(kn, kn.clone(), torch.ones(2, dtype=torch.float32))


@pytest.mark.parametrize("strides,ok", [
    ((2 * 64 * 64, 64 * 64, 64), True),         # [B, H, L, d]
    ((64 * 2 * 64, 64, 2 * 64), True),          # [B, L, H, d]
    ((2 * 64 * 64, 0, 64), False),              # heads broadcast: output rows would race
    ((0, 64 * 64, 64), False),                  # batch broadcast
    ((2 * 64 * 64, 32 * 64, 64), False),        # heads overlap positions 32..63
    ((64 * 2 * 64, 64, 64), False),             # [B, L, H, d] with a row stride of one head
])
def test_problem_rejects_overlapping_rows(strides, ok):
    """Outputs share the inputs' strides, so rows of different (b, h, i) must not
    overlap (checked by sigattn_validate on the host)."""
    p, keep = S.make_problem(2, 2, 64, 64, [64, 30], strides=strides)
    assert S.validate(p) == (0 if ok else 1)


def test_attention_is_checked_like_fwd():
    """The autograd entry point goes through the same checks before any launch."""
    q, k, v = _qkv()
    for t in (q, k, v):
        t.requires_grad_(True)
    with pytest.raises(ValueError, match="same GPU"):
        S.attention(q, k, v, [64, 10])
    with pytest.raises(ValueError, match="gate must be a float32"):
        S.attention(q, k, v, [64, 10], gate=torch.ones((1, 64), dtype=torch.float32))


def test_attention_varlen_refuses_a_gate_gradient():
    """The packed entry points have no gate gradient, so a gate that asks for one is
    refused before anything is allocated; otherwise the same checks as fwd_varlen."""
    q, k, v, do, cu_q, cu_k = _packed()
    for t in (q, k, v):
        t.requires_grad_(True)
    gate = torch.ones(12, dtype=torch.float32, requires_grad=True)
    with pytest.raises(ValueError, match="no gate gradient"):
        S.attention_varlen(q, k, v, cu_q, cu_k, 10, 12, gate=gate)
    with pytest.raises(ValueError, match="same shape"):
        S.attention_varlen(q, k, v[:3], cu_q, cu_k, 10, 12)

"""Padded sigmoid attention on MI355X (gfx950): Python binding of libsigattn.so.

Argument marshalling only: every step runs in the HIP kernels of the library. PyTorch
supplies device buffers and the current stream, nothing else. The library must have
been built (``python -m sigmoid_attention_amd.build``); if it is missing every call
raises, there is no fallback.

    o = fwd(q, k, v, seqlens, causal=False, gate=None, tau=0.0, sink=4,
            out_dtype=None, fast_math=False)
    o, row_mass = fwd_rowsum(q, k, v, seqlens, ...)
    dq = bwd_dq(q, k, v, do, seqlens, ...)
    dk, dv = bwd_dkdv(q, k, v, do, seqlens, ...)
    dq, dk, dv = bwd(q, k, v, do, seqlens, ...)            # both backward kernels, one call
    dk, dv, dg_head, dg = bwd_dkdv_dg(q, k, v, do, seqlens, gate=g, ...)
    o = attention(q, k, v, seqlens, ...)                   # the same, under torch.autograd
    o = fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k)      # packed [rows, H, d] batches
    dq, dk, dv = bwd_varlen(q, k, v, do, cu_q, cu_k, max_q, max_k)
    o = attention_varlen(q, k, v, cu_q, cu_k, max_q, max_k)  # the same under torch.autograd
    cache = KVCache(B, H, d, cap, gated=True, tau=0.05)   # KV cache with eviction
    cache.build(k, v, seqlens, gate=g); cache.append(k1, v1, g1); o1 = cache.decode(q1, bias)
    o1 = cache.decode_noalloc(q1, bias, out=o1)              # no workspace, no allocation

Tensors are [B, H, Lmax, d] views (any strides with a contiguous last dimension, the
same strides for all of them), bf16 or float32 (the float32 debug path), on one GPU.
``seqlens`` holds the valid length of each batch entry (host ints). ``gate`` is an
optional [B, Lmax] float32 device tensor of per-key gates.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = ["fwd", "fwd_rowsum", "bwd_dq", "bwd_dkdv", "bwd", "bwd_dkdv_dg", "attention",
           "attention_varlen", "fwd_varlen", "bwd_dq_varlen", "bwd_dkdv_varlen", "bwd_varlen",
           "VarlenDesc", "KVCache", "CacheDesc", "validate", "plan", "calibrate_mfma",
           "library_path", "load", "Problem", "SigattnError", "STATUS", "VERSION",
           "NOALLOC_WORKSPACE_BYTES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsigattn.so")

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported problem",
          3: "misaligned pointer or stride", 4: "HIP runtime error"}
BF16, F32 = 0, 1
VERSION = 2
NOALLOC_WORKSPACE_BYTES = 16 << 20   # static decode workspace of sigattn_decode_noalloc


class SigattnError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS.get(code, 'unknown')} (status {code})")
        self.code = code


class Problem(ctypes.Structure):
    """Mirror of ``sigattn_problem`` in include/sigattn.h."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Lmax", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("fast_math", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
        ("stride_l", ctypes.c_int64),
        ("seqlens", ctypes.POINTER(ctypes.c_int32)),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("bias", ctypes.POINTER(ctypes.c_float)),
        ("gate", ctypes.c_void_p),
        ("gate_stride_b", ctypes.c_int64),
        ("gate_eps", ctypes.c_float),
        ("gate_tau", ctypes.c_float),
        ("gate_sink", ctypes.c_int32),
    ]


class VarlenDesc(ctypes.Structure):
    """Mirror of ``sigattn_varlen`` in include/sigattn.h."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("fast_math", ctypes.c_int32),
        ("stride_t", ctypes.c_int64), ("stride_h", ctypes.c_int64),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
        ("bias", ctypes.c_void_p), ("gate", ctypes.c_void_p),
        ("gate_eps", ctypes.c_float), ("gate_tau", ctypes.c_float),
        ("gate_sink", ctypes.c_int32),
    ]


class CacheDesc(ctypes.Structure):
    """Mirror of ``sigattn_cache`` in include/sigattn.h."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
        ("cap", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
        ("stride_l", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("gate", ctypes.c_void_p),
        ("count", ctypes.c_void_p), ("seen", ctypes.c_void_p),
        ("gate_eps", ctypes.c_float), ("gate_tau", ctypes.c_float),
        ("gate_sink", ctypes.c_int32),
    ]


_lib = None


def calibrate_mfma(nblocks: int = 2048, iters: int = 4096, device=None) -> dict:
    """The bf16 MFMA rate and shader clock this GPU sustains (sigattn_calibrate_mfma):
    one timed launch on the current stream after one warm-up launch. Returns the flops,
    the launch time in ms (HIP events), TFLOP/s and the mean clock in MHz from the
    per-workgroup shader-cycle and 100 MHz stamps."""
    torch = _torch()
    lib = load()
    dev = torch.device(device if device is not None else "cuda")
    sink = torch.empty(nblocks * 256, dtype=torch.float32, device=dev)
    clk = torch.empty(2 * nblocks, dtype=torch.int64, device=dev)
    st = torch.cuda.current_stream(dev)
    _check(lib.sigattn_calibrate_mfma(nblocks, iters, sink.data_ptr(), clk.data_ptr(),
                                      st.cuda_stream), "sigattn_calibrate_mfma")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    _check(lib.sigattn_calibrate_mfma(nblocks, iters, sink.data_ptr(), clk.data_ptr(),
                                      st.cuda_stream), "sigattn_calibrate_mfma")
    e1.record(st)
    e1.synchronize()
    ms = e0.elapsed_time(e1)
    c = clk.view(nblocks, 2).double().sum(0).cpu().numpy()
    flops = lib.sigattn_calibrate_mfma_flops(nblocks, iters)
    return {"flops": flops, "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "sclk_mhz": float(c[0] / c[1] * 100.0), "nblocks": nblocks, "iters": iters}


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libsigattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run python -m sigmoid_attention_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp = ctypes.c_void_p
    lib.sigattn_validate.argtypes = [P]
    lib.sigattn_fwd.argtypes = [P, vp, vp, vp, vp, vp]
    lib.sigattn_fwd_rowsum.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.sigattn_bwd_dq.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.sigattn_bwd_dkdv.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.sigattn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sigattn_bwd_dkdv_dg.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    VD = ctypes.POINTER(VarlenDesc)
    lib.sigattn_fwd_varlen.argtypes = [VD, vp, vp, vp, vp, vp]
    lib.sigattn_bwd_dq_varlen.argtypes = [VD, vp, vp, vp, vp, vp, vp]
    lib.sigattn_bwd_dkdv_varlen.argtypes = [VD, vp, vp, vp, vp, vp, vp, vp]
    lib.sigattn_bwd_varlen.argtypes = [VD, vp, vp, vp, vp, vp, vp, vp, vp]
    for f in (lib.sigattn_fwd_varlen, lib.sigattn_bwd_dq_varlen, lib.sigattn_bwd_dkdv_varlen,
              lib.sigattn_bwd_varlen):
        f.restype = ctypes.c_int
    C = ctypes.POINTER(CacheDesc)
    i64 = ctypes.c_int64
    lib.sigattn_cache_build.argtypes = [C, P, vp, vp, vp]
    lib.sigattn_cache_append.argtypes = [C, vp, vp, i64, i64, vp, vp, vp]
    lib.sigattn_decode_workspace_size.argtypes = [C]
    lib.sigattn_decode_workspace_size.restype = i64
    lib.sigattn_decode.argtypes = [C, vp, i64, i64, ctypes.POINTER(ctypes.c_float), ctypes.c_float,
                                   vp, ctypes.c_int32, vp, i64, vp]
    lib.sigattn_decode_noalloc.argtypes = [C, vp, i64, i64, ctypes.POINTER(ctypes.c_float),
                                           ctypes.c_float, vp, ctypes.c_int32, vp]
    for f in (lib.sigattn_cache_build, lib.sigattn_cache_append, lib.sigattn_decode,
              lib.sigattn_decode_noalloc):
        f.restype = ctypes.c_int
    lib.sigattn_plan.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                 ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)]
    lib.sigattn_plan.restype = ctypes.c_int64
    lib.sigattn_status_string.argtypes = [ctypes.c_int]
    lib.sigattn_status_string.restype = ctypes.c_char_p
    lib.sigattn_version.restype = ctypes.c_int
    lib.sigattn_calibrate_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
    lib.sigattn_calibrate_mfma.restype = ctypes.c_int
    lib.sigattn_calibrate_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.sigattn_calibrate_mfma_flops.restype = ctypes.c_double
    for f in (lib.sigattn_validate, lib.sigattn_fwd, lib.sigattn_fwd_rowsum, lib.sigattn_bwd_dq,
              lib.sigattn_bwd_dkdv, lib.sigattn_bwd, lib.sigattn_bwd_dkdv_dg):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _fast_math(fast_math):
    """False/0: hi + lo bf16 operands (default); True/1: single bf16; 2: f16 P V in the
    forward (see the header's precision notes)."""
    m = int(fast_math)
    if m not in (0, 1, 2):
        raise ValueError("fast_math must be 0 (or False), 1 (or True) or 2")
    return m


def make_problem(B, H, Lmax, d, seqlens, *, dtype=BF16, out_dtype=None, fast_math=False,
                 strides=None, causal=False, scale=0.0, bias=None, gate_ptr=None,
                 gate_stride_b=0, eps=1e-8, tau=0.0, sink=4):
    """Build a Problem. Returns (problem, keepalive) where keepalive owns host arrays."""
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32).reshape(-1))
    if sl.shape[0] != B:
        raise ValueError(f"seqlens has {sl.shape[0]} entries, expected B = {B}")
    if strides is None:
        strides = (H * Lmax * d, Lmax * d, d)
    p = Problem()
    p.struct_size = ctypes.sizeof(Problem)
    p.B, p.H, p.Lmax, p.d = B, H, Lmax, d
    p.dtype = dtype
    p.out_dtype = dtype if out_dtype is None else out_dtype
    p.fast_math = _fast_math(fast_math)
    p.stride_b, p.stride_h, p.stride_l = (int(s) for s in strides)
    p.seqlens = sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    p.causal = 1 if causal else 0
    p.scale = float(scale)
    keep = [sl]
    if bias is not None:
        bb = np.ascontiguousarray(np.asarray(bias, dtype=np.float32).reshape(-1))
        if bb.shape[0] != B:
            raise ValueError(f"bias has {bb.shape[0]} entries, expected B = {B}")
        keep.append(bb)
        p.bias = bb.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    p.gate = gate_ptr
    p.gate_stride_b = int(gate_stride_b)
    p.gate_eps = float(eps)
    p.gate_tau = float(tau)
    p.gate_sink = int(sink)
    return p, keep


def validate(problem: Problem) -> int:
    return load().sigattn_validate(ctypes.byref(problem))


def plan(problem: Problem, pass_: int):
    """Work list of a pass (0 forward, 1 dQ, 2 dK/dV, 3 the one-call backward at d = 64,
    whose dQ items carry tile -1 - t) as an int32 array [n, 3] of (b, h, tile) in launch
    order, and the tile height."""
    lib = load()
    tile = ctypes.c_int32(0)
    n = lib.sigattn_plan(ctypes.byref(problem), pass_, None, 0, ctypes.byref(tile))
    if n < 0:
        raise ValueError("invalid problem")
    out = np.zeros((max(n, 1), 3), dtype=np.int32)
    lib.sigattn_plan(ctypes.byref(problem), pass_,
                     out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n, ctypes.byref(tile))
    return out[:n], tile.value


# ----------------------------------------------------------------------------------
# torch-facing wrappers
# ----------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _describe(q, tensors, seqlens, causal, gate, tau, sink, eps, scale, bias,
              out_dtype=None, fast_math=False):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("expected [B, H, Lmax, d] tensors")
    B, H, L, d = q.shape
    for t in tensors:
        if t.shape != q.shape or t.stride() != q.stride() or t.dtype != q.dtype:
            raise ValueError("all tensors must share shape, strides and dtype")
    if q.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    if q.dtype == torch.bfloat16:
        dtype = BF16
    elif q.dtype == torch.float32:
        dtype = F32
    else:
        raise ValueError("dtype must be bfloat16 or float32")
    gate_ptr, gsb = None, 0
    if gate is not None:
        if gate.dtype != torch.float32 or gate.dim() != 2 or tuple(gate.shape) != (B, L):
            raise ValueError(f"gate must be a float32 [B, Lmax] = [{B}, {L}] tensor")
        if gate.stride(-1) != 1 or (B > 1 and gate.stride(0) < L):
            raise ValueError("gate rows must be contiguous and must not overlap")
        gate_ptr, gsb = gate.data_ptr(), gate.stride(0)
    for t in (q,) + tuple(tensors) + (() if gate is None else (gate,)):
        if t.device != q.device or t.device.type != "cuda":
            raise ValueError("all tensors must be on the same GPU")
    if hasattr(seqlens, "cpu"):
        seqlens = seqlens.cpu().numpy()
    if out_dtype is None or out_dtype == q.dtype:
        odt = dtype
    elif out_dtype == torch.float32:
        odt = F32
    elif out_dtype == torch.bfloat16:
        odt = BF16
    else:
        raise ValueError("out_dtype must be bfloat16 or float32")
    return make_problem(B, H, L, d, seqlens, dtype=dtype, out_dtype=odt,
                        fast_math=fast_math, strides=q.stride()[:3], causal=causal,
                        scale=scale, bias=bias, gate_ptr=gate_ptr, gate_stride_b=gsb,
                        eps=eps, tau=tau, sink=sink)


def _new_out(q, out_dtype):
    torch = _torch()
    dt = q.dtype if out_dtype is None else out_dtype
    return torch.empty_strided(q.shape, q.stride(), dtype=dt, device=q.device)


def _check_out(q, t, out_dtype):
    dt = q.dtype if out_dtype is None else out_dtype
    if t.shape != q.shape or t.stride() != q.stride() or t.dtype != dt or t.device != q.device:
        raise ValueError("output tensors must match q in shape and strides, with the output dtype")


def _stream(q):
    return _torch().cuda.current_stream(q.device).cuda_stream


def _check(code, what):
    if code != 0:
        raise SigattnError(code, what)


def fwd(q, k, v, seqlens, *, causal=False, gate=None, tau=0.0, sink=4, eps=1e-8,
        scale=0.0, bias=None, out=None, out_dtype=None, fast_math=False):
    """O = sigma(s Q K^T + b) V' over valid keys; rows past each length are 0."""
    lib = load()
    prob, keep = _describe(q, (k, v), seqlens, causal, gate, tau, sink, eps, scale, bias,
                           out_dtype, fast_math)
    if out is None:
        out = _new_out(q, out_dtype)
    _check_out(q, out, out_dtype)
    code = lib.sigattn_fwd(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           out.data_ptr(), _stream(q))
    del keep
    _check(code, "sigattn_fwd")
    return out


def bwd_dq(q, k, v, do, seqlens, *, causal=False, gate=None, tau=0.0, sink=4, eps=1e-8,
           scale=0.0, bias=None, out=None, out_dtype=None, fast_math=False):
    """dQ of sum(dO * O); rows past each length are 0."""
    lib = load()
    prob, keep = _describe(q, (k, v, do), seqlens, causal, gate, tau, sink, eps, scale, bias,
                           out_dtype, fast_math)
    if out is None:
        out = _new_out(q, out_dtype)
    _check_out(q, out, out_dtype)
    code = lib.sigattn_bwd_dq(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              do.data_ptr(), out.data_ptr(), _stream(q))
    del keep
    _check(code, "sigattn_bwd_dq")
    return out


def bwd_dkdv(q, k, v, do, seqlens, *, causal=False, gate=None, tau=0.0, sink=4, eps=1e-8,
             scale=0.0, bias=None, out=None, out_dtype=None, fast_math=False):
    """(dK, dV) of sum(dO * O); rows past each length and dropped keys are 0."""
    lib = load()
    prob, keep = _describe(q, (k, v, do), seqlens, causal, gate, tau, sink, eps, scale, bias,
                           out_dtype, fast_math)
    dk, dv = (_new_out(q, out_dtype), _new_out(q, out_dtype)) if out is None else out
    _check_out(q, dk, out_dtype)
    _check_out(q, dv, out_dtype)
    code = lib.sigattn_bwd_dkdv(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                do.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream(q))
    del keep
    _check(code, "sigattn_bwd_dkdv")
    return dk, dv


def bwd(q, k, v, do, seqlens, *, causal=False, gate=None, tau=0.0, sink=4, eps=1e-8,
        scale=0.0, bias=None, out=None, out_dtype=None, fast_math=False):
    """(dQ, dK, dV) in one call: the values of bwd_dq and bwd_dkdv, from one launch of both
    kernels at d = 64."""
    lib = load()
    prob, keep = _describe(q, (k, v, do), seqlens, causal, gate, tau, sink, eps, scale, bias,
                           out_dtype, fast_math)
    dq, dk, dv = tuple(_new_out(q, out_dtype) for _ in range(3)) if out is None else out
    for t in (dq, dk, dv):
        _check_out(q, t, out_dtype)
    code = lib.sigattn_bwd(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream(q))
    del keep
    _check(code, "sigattn_bwd")
    return dq, dk, dv


def _new_plane(q, shape):
    torch = _torch()
    return torch.empty(shape, dtype=torch.float32, device=q.device)


def _check_plane(q, t, shape):
    torch = _torch()
    if (tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or t.device != q.device
            or not t.is_contiguous()):
        raise ValueError(f"expected a contiguous float32 tensor of shape {tuple(shape)} on q's GPU")


def bwd_dkdv_dg(q, k, v, do, seqlens, *, gate, causal=False, tau=0.0, sink=4, eps=1e-8,
                scale=0.0, bias=None, out=None, dg_head=None, dg=None, out_dtype=None,
                fast_math=False, head_sum=True):
    """(dK, dV, dg_head, dg): dK and dV as bwd_dkdv, plus the gate gradient per head
    ([B, H, Lmax] float32) and summed over heads ([B, Lmax] float32, None when
    head_sum is False)."""
    if gate is None:
        raise ValueError("bwd_dkdv_dg needs a gate")
    lib = load()
    prob, keep = _describe(q, (k, v, do), seqlens, causal, gate, tau, sink, eps, scale, bias,
                           out_dtype, fast_math)
    dk, dv = (_new_out(q, out_dtype), _new_out(q, out_dtype)) if out is None else out
    _check_out(q, dk, out_dtype)
    _check_out(q, dv, out_dtype)
    B, H, L, _ = q.shape
    if dg_head is None:
        dg_head = _new_plane(q, (B, H, L))
    _check_plane(q, dg_head, (B, H, L))
    if head_sum:
        if dg is None:
            dg = _new_plane(q, (B, L))
        _check_plane(q, dg, (B, L))
    else:
        dg = None
    code = lib.sigattn_bwd_dkdv_dg(ctypes.byref(prob), q.data_ptr(), k.data_ptr(),
                                   v.data_ptr(), do.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                   dg_head.data_ptr(), None if dg is None else dg.data_ptr(),
                                   _stream(q))
    del keep
    _check(code, "sigattn_bwd_dkdv_dg")
    return dk, dv, dg_head, dg


def fwd_rowsum(q, k, v, seqlens, *, causal=False, gate=None, tau=0.0, sink=4, eps=1e-8,
               scale=0.0, bias=None, out=None, row_mass=None, out_dtype=None,
               fast_math=False):
    """(O, row_mass): O as fwd, plus sum_j P_ij per query ([B, H, Lmax] float32)."""
    lib = load()
    prob, keep = _describe(q, (k, v), seqlens, causal, gate, tau, sink, eps, scale, bias,
                           out_dtype, fast_math)
    if out is None:
        out = _new_out(q, out_dtype)
    _check_out(q, out, out_dtype)
    B, H, L, _ = q.shape
    if row_mass is None:
        row_mass = _new_plane(q, (B, H, L))
    _check_plane(q, row_mass, (B, H, L))
    code = lib.sigattn_fwd_rowsum(ctypes.byref(prob), q.data_ptr(), k.data_ptr(),
                                  v.data_ptr(), out.data_ptr(), row_mass.data_ptr(),
                                  _stream(q))
    del keep
    _check(code, "sigattn_fwd_rowsum")
    return out, row_mass


_ATTENTION_FN = None


def _attention_function():
    """The torch.autograd.Function behind attention(), defined on first use (torch is
    imported lazily by this module)."""
    global _ATTENTION_FN
    if _ATTENTION_FN is None:
        torch = _torch()

        class SigmoidAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, gate, seqlens, opts):
                o = fwd(q, k, v, seqlens, gate=gate, **opts)
                ctx.save_for_backward(q, k, v, gate)
                ctx.seqlens = seqlens
                ctx.opts = opts
                return o

            @staticmethod
            def backward(ctx, grad_o):
                q, k, v, gate = ctx.saved_tensors
                # dO enters the kernels in q's dtype and layout
                do = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
                do.copy_(grad_o)
                opts = dict(ctx.opts, out_dtype=None)   # gradients in the inputs' dtype
                if gate is not None and ctx.needs_input_grad[3]:
                    dq = bwd_dq(q, k, v, do, ctx.seqlens, gate=gate, **opts)
                    dk, dv, _, dg = bwd_dkdv_dg(q, k, v, do, ctx.seqlens, gate=gate, **opts)
                else:
                    dq, dk, dv = bwd(q, k, v, do, ctx.seqlens, gate=gate, **opts)
                    dg = None
                return dq, dk, dv, dg, None, None

        _ATTENTION_FN = SigmoidAttention
    return _ATTENTION_FN


def _zeros_like_layout(x, dtype):
    """Zeros with x's shape and strides (dtype None: x's dtype)."""
    torch = _torch()
    return torch.empty_strided(x.shape, x.stride(), dtype=x.dtype if dtype is None else dtype,
                               device=x.device).zero_()


_ATTENTION_VARLEN_FN = None


def _attention_varlen_function():
    global _ATTENTION_VARLEN_FN
    if _ATTENTION_VARLEN_FN is None:
        torch = _torch()

        class SigmoidAttentionVarlen(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, cu_q, cu_k, max_q, max_k, gate, bias, opts):
                # rows outside every sequence are not written by the kernels: start from 0
                o = _zeros_like_layout(q, opts["out_dtype"])
                fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k, gate=gate, bias=bias, out=o,
                           **opts)
                ctx.save_for_backward(q, k, v, cu_q, cu_k, gate, bias)
                ctx.bounds = (max_q, max_k)
                ctx.opts = opts
                return o

            @staticmethod
            def backward(ctx, grad_o):
                q, k, v, cu_q, cu_k, gate, bias = ctx.saved_tensors
                do = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
                do.copy_(grad_o)
                opts = dict(ctx.opts, out_dtype=None)
                out = (_zeros_like_layout(q, None), _zeros_like_layout(k, None),
                       _zeros_like_layout(k, None))
                dq, dk, dv = bwd_varlen(q, k, v, do, cu_q, cu_k, *ctx.bounds, gate=gate,
                                        bias=bias, out=out, **opts)
                return dq, dk, dv, None, None, None, None, None, None, None

        _ATTENTION_VARLEN_FN = SigmoidAttentionVarlen
    return _ATTENTION_VARLEN_FN


def attention_varlen(q, k, v, cu_q, cu_k, max_q, max_k, *, causal=False, gate=None, tau=0.0,
                     sink=4, eps=1e-8, scale=0.0, bias=None, out_dtype=None, fast_math=False):
    """O as fwd_varlen, differentiable with torch.autograd (the backward calls bwd_varlen).
    Rows outside every sequence are 0 in O and in the gradients (the outputs start from
    zeros, which the kernels leave there). The packed entry points have no gate gradient,
    so a gate that requires one is refused; cu_q, cu_k, the bounds, the gate and the bias
    are constants."""
    if gate is not None and getattr(gate, "requires_grad", False):
        raise ValueError("the packed entry points have no gate gradient: use attention() on "
                         "padded tensors, or pass a gate that does not require grad")
    opts = dict(causal=causal, tau=tau, sink=sink, eps=eps, scale=scale, out_dtype=out_dtype,
                fast_math=fast_math)
    return _attention_varlen_function().apply(q, k, v, cu_q, cu_k, max_q, max_k, gate, bias,
                                              opts)


def attention(q, k, v, seqlens, *, causal=False, gate=None, tau=0.0, sink=4, eps=1e-8,
              scale=0.0, bias=None, out_dtype=None, fast_math=False):
    """O as fwd, differentiable with torch.autograd: the backward calls bwd (one call for
    dQ, dK, dV), or bwd_dq and bwd_dkdv_dg when the gate also needs its gradient (the
    gate's gradient is the head sum of the per-head one; dropped and padded keys get 0).
    The incoming gradient is copied into q's dtype and layout, and the gradients come out
    in q's dtype. seqlens, tau, sink, eps, scale and bias are constants."""
    opts = dict(causal=causal, tau=tau, sink=sink, eps=eps, scale=scale, bias=bias,
                out_dtype=out_dtype, fast_math=fast_math)
    return _attention_function().apply(q, k, v, gate, seqlens, opts)


class KVCache:
    """A KV cache with threshold eviction on one GPU (see sigattn_cache in the header):
    keys and values [B, H, cap, d] bf16, gates [B, cap] float32 (when gated), and the
    device counters count [B] (live entries) and seen [B] (positions written)."""

    def __init__(self, B, H, d, cap, *, gated, eps=1e-8, tau=0.0, sink=4, device=None):
        torch = _torch()
        dev = torch.device("cuda") if device is None else torch.device(device)
        self.k = torch.zeros((B, H, cap, d), dtype=torch.bfloat16, device=dev)
        self.v = torch.zeros_like(self.k)
        self.gate = torch.zeros((B, cap), dtype=torch.float32, device=dev) if gated else None
        self.count = torch.zeros(B, dtype=torch.int32, device=dev)
        self.seen = torch.zeros(B, dtype=torch.int32, device=dev)
        c = CacheDesc()
        c.struct_size = ctypes.sizeof(CacheDesc)
        c.B, c.H, c.d, c.cap = B, H, d, cap
        c.stride_b, c.stride_h, c.stride_l = self.k.stride()[:3]
        c.k, c.v = self.k.data_ptr(), self.v.data_ptr()
        c.gate = None if self.gate is None else self.gate.data_ptr()
        c.count, c.seen = self.count.data_ptr(), self.seen.data_ptr()
        c.gate_eps, c.gate_tau, c.gate_sink = float(eps), float(tau), int(sink)
        self.desc = c
        self.shape = (B, H, d, cap)

    def _new_rows_ok(self, t, name):
        torch = _torch()
        B, H, d, _ = self.shape
        if (tuple(t.shape) != (B, H, d) or t.dtype != torch.bfloat16 or t.device != self.k.device
                or t.stride(-1) != 1):
            raise ValueError(f"{name} must be a bf16 [B, H, d] tensor on the cache's GPU "
                             "with a contiguous last dimension")

    def build(self, k, v, seqlens, gate=None):
        """Fill the cache from a prefill (k, v: [B, H, Lmax, d] bf16): kept rows only."""
        lib = load()
        prob, keep = _describe(k, (v,), seqlens, False, gate, 0.0, 0, 1e-8, 0.0, None)
        code = lib.sigattn_cache_build(ctypes.byref(self.desc), ctypes.byref(prob),
                                       k.data_ptr(), v.data_ptr(), _stream(k))
        del keep
        _check(code, "sigattn_cache_build")

    def append(self, k_new, v_new, g_new=None, status=None):
        """Write one new entry per sequence, kept or removed by the threshold rule."""
        self._new_rows_ok(k_new, "k_new")
        self._new_rows_ok(v_new, "v_new")
        if k_new.stride() != v_new.stride():
            raise ValueError("k_new and v_new must share strides")
        torch = _torch()
        B = self.shape[0]
        if (self.gate is None) != (g_new is None):
            raise ValueError("g_new is required exactly when the cache has gates")
        if g_new is not None and (g_new.dtype != torch.float32 or tuple(g_new.shape) != (B,)
                                  or not g_new.is_contiguous() or g_new.device != self.k.device):
            raise ValueError("g_new must be a contiguous float32 [B] tensor on the cache's GPU")
        if status is not None and (status.dtype != torch.int32 or status.numel() < 1
                                   or status.device != self.k.device):
            raise ValueError("status must be an int32 tensor on the cache's GPU")
        lib = load()
        code = lib.sigattn_cache_append(
            ctypes.byref(self.desc), k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0),
            k_new.stride(1), None if g_new is None else g_new.data_ptr(),
            None if status is None else status.data_ptr(), _stream(k_new))
        _check(code, "sigattn_cache_append")

    def workspace_size(self) -> int:
        return int(load().sigattn_decode_workspace_size(ctypes.byref(self.desc)))

    def _decode_args(self, q, bias, out, out_dtype):
        torch = _torch()
        self._new_rows_ok(q, "q")
        B = self.shape[0]
        bb = np.ascontiguousarray(np.asarray(bias, dtype=np.float32).reshape(-1))
        if bb.shape[0] != B:
            raise ValueError("bias needs one value per sequence")
        odt = torch.bfloat16 if out_dtype is None else out_dtype
        if odt not in (torch.bfloat16, torch.float32):
            raise ValueError("out_dtype must be bfloat16 or float32")
        if out is None:
            out = torch.empty_strided(q.shape, q.stride(), dtype=odt, device=q.device)
        if out.shape != q.shape or out.stride() != q.stride() or out.dtype != odt:
            raise ValueError("out must match q in shape and strides, with the output dtype")
        if out.device != q.device:
            raise ValueError("out must be on q's GPU")
        return bb, out, (F32 if odt == torch.float32 else BF16)

    def decode(self, q, bias, *, scale=0.0, out=None, out_dtype=None, workspace=None):
        """o[b, h] = sum over live entries of sigma(s q.k + beta_b [+ log(g+eps)]) [g] v.
        bias: host sequence of B floats (beta_b). workspace: optional float32 device
        tensor of at least workspace_size() bytes (allocated when omitted)."""
        torch = _torch()
        bb, out, code_dt = self._decode_args(q, bias, out, out_dtype)
        lib = load()
        if workspace is None:
            workspace = torch.empty(max(1, (self.workspace_size() + 3) // 4),
                                    dtype=torch.float32, device=q.device)
        if workspace.dtype != torch.float32 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous float32 tensor")
        if workspace.device != q.device:
            raise ValueError("workspace must be on q's GPU")
        code = lib.sigattn_decode(ctypes.byref(self.desc), q.data_ptr(), q.stride(0),
                                  q.stride(1), bb.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                  float(scale), out.data_ptr(), code_dt, workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), _stream(q))
        _check(code, "sigattn_decode")
        return out

    def decode_noalloc(self, q, bias, *, scale=0.0, out=None, out_dtype=None):
        """decode() through sigattn_decode_noalloc: no workspace, the library's static
        device array holds the partial sums (the cache's workspace_size() must not exceed
        16 MiB). With `out` given, nothing is allocated."""
        bb, out, code_dt = self._decode_args(q, bias, out, out_dtype)
        code = load().sigattn_decode_noalloc(
            ctypes.byref(self.desc), q.data_ptr(), q.stride(0), q.stride(1),
            bb.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), float(scale), out.data_ptr(),
            code_dt, _stream(q))
        _check(code, "sigattn_decode_noalloc")
        return out


def _varlen_desc(q, k, tensors, cu_q, cu_k, max_q, max_k, causal, gate, tau, sink, eps,
                 scale, bias, out_dtype, fast_math):
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or q.shape[1:] != k.shape[1:]:
        raise ValueError("expected packed [rows, H, d] tensors with the same H and d")
    for t in (q, k) + tuple(tensors):
        if t.stride() != q.stride() or t.dtype != torch.bfloat16 or t.device != q.device:
            raise ValueError("packed tensors must be bf16, on one GPU, with the same strides")
    if q.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    for c in (cu_q, cu_k):
        if c.dtype != torch.int32 or c.device != q.device or c.dim() != 1 or not c.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous int32 tensors on q's GPU")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need B + 1 entries each")
    if out_dtype is not None and out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bfloat16 or float32")
    for x in (gate, bias):
        if x is not None and (x.dtype != torch.float32 or x.device != q.device or not x.is_contiguous()):
            raise ValueError("gate and bias must be contiguous float32 tensors on q's GPU")
    p = VarlenDesc()
    p.struct_size = ctypes.sizeof(VarlenDesc)
    p.B, p.H, p.d = cu_q.numel() - 1, q.shape[1], q.shape[2]
    p.max_seqlen_q, p.max_seqlen_k = int(max_q), int(max_k)
    p.out_dtype = F32 if out_dtype == torch.float32 else BF16
    p.fast_math = _fast_math(fast_math)
    p.stride_t, p.stride_h = q.stride(0), q.stride(1)
    p.cu_seqlens_q, p.cu_seqlens_k = cu_q.data_ptr(), cu_k.data_ptr()
    p.causal = 1 if causal else 0
    p.scale = float(scale)
    p.bias = None if bias is None else bias.data_ptr()
    p.gate = None if gate is None else gate.data_ptr()
    p.gate_eps, p.gate_tau, p.gate_sink = float(eps), float(tau), int(sink)
    return p


def _new_like(x, out_dtype):
    torch = _torch()
    dt = torch.bfloat16 if out_dtype is None else out_dtype
    return torch.empty_strided(x.shape, x.stride(), dtype=dt, device=x.device)


def _check_like(x, t, out_dtype, name):
    """An output of a packed pass must match its input (q for o and dq, k for dk and dv)
    in shape, strides and device, with the output dtype."""
    torch = _torch()
    dt = torch.bfloat16 if out_dtype is None else out_dtype
    if (t.shape != x.shape or t.stride() != x.stride() or t.dtype != dt
            or t.device != x.device):
        raise ValueError(f"{name} must match its input in shape, strides and device, "
                         f"with dtype {dt}")


def _on_gpu(*tensors):
    for t in tensors:
        if t is not None and t.device.type != "cuda":
            raise ValueError("packed tensors must be on a GPU")


def _same_shape(a, b, what):
    if a.shape != b.shape:
        raise ValueError(f"{what} must have the same shape")


def fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k, *, causal=False, gate=None, tau=0.0,
               sink=4, eps=1e-8, scale=0.0, bias=None, out=None, out_dtype=None,
               fast_math=False):
    """O for packed sequences: q [rows_q, H, d], k, v [rows_k, H, d] (bf16); cu_q, cu_k
    device int32 [B + 1]; max_q, max_k host bounds on the sequence lengths; gate device
    float per key row; bias device float [B] (default -ln(nk))."""
    lib = load()
    _same_shape(v, k, "v and k")
    p = _varlen_desc(q, k, (v,), cu_q, cu_k, max_q, max_k, causal, gate, tau, sink, eps, scale,
                     bias, out_dtype, fast_math)
    out = _new_like(q, out_dtype) if out is None else out
    _check_like(q, out, out_dtype, "out")
    _on_gpu(q, k, v, out, cu_q, cu_k, gate, bias)
    _check(lib.sigattn_fwd_varlen(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  out.data_ptr(), _stream(q)), "sigattn_fwd_varlen")
    return out


def bwd_dq_varlen(q, k, v, do, cu_q, cu_k, max_q, max_k, *, causal=False, gate=None, tau=0.0,
                  sink=4, eps=1e-8, scale=0.0, bias=None, out=None, out_dtype=None,
                  fast_math=False):
    lib = load()
    _same_shape(v, k, "v and k")
    _same_shape(do, q, "do and q")
    p = _varlen_desc(q, k, (v, do), cu_q, cu_k, max_q, max_k, causal, gate, tau, sink, eps,
                     scale, bias, out_dtype, fast_math)
    out = _new_like(q, out_dtype) if out is None else out
    _check_like(q, out, out_dtype, "dq")
    _on_gpu(q, k, v, do, out, cu_q, cu_k, gate, bias)
    _check(lib.sigattn_bwd_dq_varlen(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     do.data_ptr(), out.data_ptr(), _stream(q)),
           "sigattn_bwd_dq_varlen")
    return out


def bwd_dkdv_varlen(q, k, v, do, cu_q, cu_k, max_q, max_k, *, causal=False, gate=None,
                    tau=0.0, sink=4, eps=1e-8, scale=0.0, bias=None, out=None, out_dtype=None,
                    fast_math=False):
    lib = load()
    _same_shape(v, k, "v and k")
    _same_shape(do, q, "do and q")
    p = _varlen_desc(q, k, (v, do), cu_q, cu_k, max_q, max_k, causal, gate, tau, sink, eps,
                     scale, bias, out_dtype, fast_math)
    dk, dv = (_new_like(k, out_dtype), _new_like(k, out_dtype)) if out is None else out
    _check_like(k, dk, out_dtype, "dk")
    _check_like(k, dv, out_dtype, "dv")
    _on_gpu(q, k, v, do, dk, dv, cu_q, cu_k, gate, bias)
    _check(lib.sigattn_bwd_dkdv_varlen(ctypes.byref(p), q.data_ptr(), k.data_ptr(),
                                       v.data_ptr(), do.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       _stream(q)), "sigattn_bwd_dkdv_varlen")
    return dk, dv


def bwd_varlen(q, k, v, do, cu_q, cu_k, max_q, max_k, *, causal=False, gate=None, tau=0.0,
               sink=4, eps=1e-8, scale=0.0, bias=None, out=None, out_dtype=None,
               fast_math=False):
    """(dQ, dK, dV) of packed sequences in one call: the values of bwd_dq_varlen and
    bwd_dkdv_varlen, from one launch of both kernels at d = 64."""
    lib = load()
    _same_shape(v, k, "v and k")
    _same_shape(do, q, "do and q")
    p = _varlen_desc(q, k, (v, do), cu_q, cu_k, max_q, max_k, causal, gate, tau, sink, eps,
                     scale, bias, out_dtype, fast_math)
    if out is None:
        dq, dk, dv = _new_like(q, out_dtype), _new_like(k, out_dtype), _new_like(k, out_dtype)
    else:
        dq, dk, dv = out
    _check_like(q, dq, out_dtype, "dq")
    _check_like(k, dk, out_dtype, "dk")
    _check_like(k, dv, out_dtype, "dv")
    _on_gpu(q, k, v, do, dq, dk, dv, cu_q, cu_k, gate, bias)
    _check(lib.sigattn_bwd_varlen(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                  _stream(q)), "sigattn_bwd_varlen")
    return dq, dk, dv

"""Valid calls of every C entry point with fake device pointers, for the sanitized
host-only build of the library (tests/host_san_stubs.cpp: launchers that touch no
device). Runs only inside tests/test_abi_sanitized.py's driver, which loads that build:
against the real library these calls would launch kernels on addresses that do not exist,
so the module refuses to run anywhere else. Not collected by a plain pytest run."""

import ctypes
import os

import numpy as np
import pytest

import sigmoid_attention_amd as S

STUB = os.environ.get("SIGATTN_SANITIZED_STUBS") == "1" and \
    S.library_path().endswith("libsigattn_san.so")
pytestmark = pytest.mark.skipif(not STUB, reason="only with the sanitized stub build")

vp = ctypes.c_void_p
F = [vp((1 << 28) * (i + 1)) for i in range(10)]   # distinct, aligned fake addresses


@pytest.fixture(scope="module")
def lib():
    return S.load()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("gated", [False, True])
def test_padded_entry_points(lib, d, causal, gated):
    rng = np.random.default_rng(d + causal)
    for B, L in ((256, 513), (3, 65535), (1, 1)):
        sl = rng.integers(0, L + 1, size=B)
        sl[0] = L
        p, keep = S.make_problem(B, 2, L, d, sl, causal=bool(causal),
                                 gate_ptr=F[9].value if gated else None, tau=0.05)
        assert S.validate(p) == 0
        for fm in (0, 1, 2):
            p.fast_math = fm
            assert lib.sigattn_fwd(ctypes.byref(p), F[0], F[1], F[2], F[3], None) == 0
            assert lib.sigattn_fwd_rowsum(ctypes.byref(p), F[0], F[1], F[2], F[3], F[8], None) == 0
            assert lib.sigattn_bwd_dq(ctypes.byref(p), F[0], F[1], F[2], F[4], F[5], None) == 0
            assert lib.sigattn_bwd_dkdv(ctypes.byref(p), F[0], F[1], F[2], F[4], F[5], F[6], None) == 0
            assert lib.sigattn_bwd(ctypes.byref(p), F[0], F[1], F[2], F[4], F[5], F[6], F[7], None) == 0
            if gated:
                assert lib.sigattn_bwd_dkdv_dg(ctypes.byref(p), F[0], F[1], F[2], F[4], F[5], F[6],
                                               F[7], F[8], None) == 0
        items, tile = S.plan(p, 0)
        assert len(items) == sum(2 * ((int(n) + tile - 1) // tile) for n in sl)


def test_float_debug_path(lib):
    p, keep = S.make_problem(5, 3, 300, 64, [300, 0, 1, 299, 77], dtype=1, out_dtype=1)
    assert lib.sigattn_fwd(ctypes.byref(p), F[0], F[1], F[2], F[3], None) == 0
    assert lib.sigattn_bwd(ctypes.byref(p), F[0], F[1], F[2], F[4], F[5], F[6], F[7], None) == 0


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_entry_points(lib, d):
    p = S.VarlenDesc()
    p.struct_size = ctypes.sizeof(S.VarlenDesc)
    p.B, p.H, p.d = 300, 4, d
    p.max_seqlen_q, p.max_seqlen_k = 1000, 4000
    p.stride_t, p.stride_h = 4 * d, d
    p.cu_seqlens_q, p.cu_seqlens_k = F[8].value, F[9].value
    p.gate_eps, p.gate_tau, p.gate_sink = 1e-8, 0.05, 4
    for causal in (0, 1):
        p.causal = causal
        assert lib.sigattn_fwd_varlen(ctypes.byref(p), F[0], F[1], F[2], F[3], None) == 0
        assert lib.sigattn_bwd_varlen(ctypes.byref(p), F[0], F[1], F[2], F[4], F[5], F[6], F[7],
                                      None) == 0
        assert lib.sigattn_bwd_dq_varlen(ctypes.byref(p), F[0], F[1], F[2], F[4], F[5], None) == 0
        assert lib.sigattn_bwd_dkdv_varlen(ctypes.byref(p), F[0], F[1], F[2], F[4], F[5], F[6],
                                           None) == 0


def test_cache_entry_points(lib):
    c = S.CacheDesc()
    c.struct_size = ctypes.sizeof(S.CacheDesc)
    c.B, c.H, c.d, c.cap = 256, 2, 128, 600
    c.stride_b, c.stride_h, c.stride_l = 2 * 600 * 128, 600 * 128, 128
    c.k, c.v, c.gate = F[0].value, F[1].value, F[2].value
    c.count, c.seen = F[3].value, F[3].value + 1024
    c.gate_eps, c.gate_tau, c.gate_sink = 1e-8, 0.05, 4
    p, keep = S.make_problem(256, 2, 600, 128, [600] * 128 + [0] * 128, gate_ptr=F[9].value)
    assert lib.sigattn_cache_build(ctypes.byref(c), ctypes.byref(p), F[4], F[5], None) == 0
    assert lib.sigattn_cache_append(ctypes.byref(c), F[4], F[5], 2 * 128, 128, F[6], F[7], None) == 0
    bias = (ctypes.c_float * 256)(*([-6.0] * 256))
    ws = lib.sigattn_decode_workspace_size(ctypes.byref(c))
    assert ws == 256 * 2 * 2 * 128 * 4
    assert lib.sigattn_decode(ctypes.byref(c), F[4], 2 * 128, 128, bias, 0.0, F[5], 1, F[6], ws,
                              None) == 0
    assert lib.sigattn_decode_noalloc(ctypes.byref(c), F[4], 2 * 128, 128, bias, 0.0, F[5], 0,
                                      None) == 0


def test_calibration_entry(lib):
    assert lib.sigattn_calibrate_mfma(2048, 4096, F[0], F[1], None) == 0
    assert lib.sigattn_calibrate_mfma_flops(2048, 4096) > 0

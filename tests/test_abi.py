"""Host-side tests of the C ABI: exported symbols, argument validation and the work
planner. None of these launch a kernel; they run without a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

import sigmoid_attention_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sigattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(S.library_path()):
        pytest.fail("libsigattn.so is not built (run python -m sigmoid_attention_amd.build)")
    return S.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sigattn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for f in ("sigattn_fwd", "sigattn_bwd_dq", "sigattn_bwd_dkdv", "sigattn_validate"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_problem_struct_matches_header_size(lib):
    # the library rejects a struct_size that differs from its own sizeof
    p, keep = S.make_problem(1, 1, 64, 64, [64])
    assert S.validate(p) == 0
    p.struct_size += 8
    assert S.validate(p) == 1


def test_version_and_status_strings(lib):
    assert lib.sigattn_version() == S.VERSION
    for code, text in S.STATUS.items():
        assert lib.sigattn_status_string(code).decode() == text


def _prob(**kw):
    base = dict(B=2, H=3, Lmax=256, d=64, seqlens=[256, 100])
    base.update(kw)
    B, H, L, d, sl = base.pop("B"), base.pop("H"), base.pop("Lmax"), base.pop("d"), base.pop("seqlens")
    return S.make_problem(B, H, L, d, sl, **base)


@pytest.mark.parametrize("mutate,code", [
    (lambda p: setattr(p, "d", 96), 2),
    (lambda p: setattr(p, "d", 32), 2),
    (lambda p: setattr(p, "B", 257), 2),
    (lambda p: setattr(p, "Lmax", 70000), 2),
    (lambda p: setattr(p, "H", 0), 1),
    (lambda p: setattr(p, "Lmax", 0), 1),
    (lambda p: setattr(p, "dtype", 7), 2),
    (lambda p: setattr(p, "out_dtype", 5), 2),
    (lambda p: (setattr(p, "dtype", 1), setattr(p, "out_dtype", 0)), 2),
    (lambda p: setattr(p, "fast_math", 3), 1),
    (lambda p: setattr(p, "fast_math", -1), 1),
    (lambda p: setattr(p, "fast_math", 2), 0),
    (lambda p: setattr(p, "causal", 2), 1),
    (lambda p: setattr(p, "stride_l", 32), 1),
    (lambda p: setattr(p, "stride_l", 68), 3),      # 136-byte rows: not 16-byte aligned
    (lambda p: setattr(p, "stride_h", 256 * 64 + 4), 3),
    (lambda p: setattr(p, "stride_l", (1 << 22) + 8), 2),  # beyond the 32-bit tile offsets
    (lambda p: setattr(p, "scale", float("nan")), 1),
    (lambda p: setattr(p, "scale", -1.0), 1),
    (lambda p: setattr(p, "seqlens", None), 1),
])
def test_validation_codes(lib, mutate, code):
    p, keep = _prob()
    mutate(p)
    assert S.validate(p) == code


def test_validation_rejects_bad_lengths(lib):
    p, keep = _prob(seqlens=[257, 10])
    assert S.validate(p) == 1
    p, keep = _prob(seqlens=[-1, 10])
    assert S.validate(p) == 1


def test_validation_gate_fields(lib):
    p, keep = _prob(gate_ptr=4096, tau=0.05)
    assert S.validate(p) == 0
    p.gate_tau = -1.0
    assert S.validate(p) == 1
    p.gate_tau = 0.05
    p.gate_eps = float("inf")
    assert S.validate(p) == 1
    p.gate_eps = 1e-8
    p.gate = 4098          # not 4-byte aligned
    assert S.validate(p) == 3
    p.gate = 4096
    p.gate_stride_b = 100  # shorter than Lmax
    assert S.validate(p) == 1


def test_work_item_cap(lib):
    """A pass of more than SIGATTN_MAX_ITEMS 128-row tiles is refused before launch (the
    one-call backward's grid holds two passes); the cap itself is accepted."""
    cap = (1 << 23) - 1
    # 256 sequences of 65535 rows = 512 tiles each: 131072 tiles per head
    p, keep = S.make_problem(256, 64, 65535, 64, [65535] * 256)
    assert S.validate(p) == 2            # 64 heads: 2^23 tiles, one too many
    p, keep = S.make_problem(256, 63, 65535, 64, [65535] * 256)
    assert S.validate(p) == 0            # 63 heads: below the cap
    assert 63 * 131072 <= cap < 64 * 131072


def test_entry_points_reject_before_launch(lib):
    """Argument errors are returned synchronously and nothing is launched; these calls
    pass fake device pointers, which would fault if anything were enqueued."""
    p, keep = _prob()
    ok = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    # null output
    assert lib.sigattn_fwd(ctypes.byref(p), ok, ok, ok, None, None) == 1
    # misaligned input
    assert lib.sigattn_fwd(ctypes.byref(p), odd, ok, ok, ctypes.c_void_p(1 << 21), None) == 3
    # output aliases an input
    assert lib.sigattn_fwd(ctypes.byref(p), ok, ok, ok, ok, None) == 1
    # dk and dv alias each other
    two = ctypes.c_void_p(1 << 22)
    assert lib.sigattn_bwd_dkdv(ctypes.byref(p), ok, ok, ok, ok, two, two, None) == 1
    # whole backward: an output aliases another output or an input, a null output
    three = ctypes.c_void_p(1 << 23)
    assert lib.sigattn_bwd(ctypes.byref(p), ok, ok, ok, ok, two, two, three, None) == 1
    assert lib.sigattn_bwd(ctypes.byref(p), ok, ok, ok, ok, two, three, two, None) == 1
    assert lib.sigattn_bwd(ctypes.byref(p), ok, ok, ok, ok, ok, two, three, None) == 1
    assert lib.sigattn_bwd(ctypes.byref(p), ok, ok, ok, ok, None, two, three, None) == 1
    assert lib.sigattn_bwd(ctypes.byref(p), ok, ok, ok, ok, two, three, odd, None) == 3
    # unsupported head size, valid pointers otherwise
    p.d = 80
    assert lib.sigattn_bwd(ctypes.byref(p), ok, ok, ok, ok, two, three, ctypes.c_void_p(1 << 24), None) == 2
    assert lib.sigattn_bwd_dq(ctypes.byref(p), ok, ok, ok, ok, two, None) == 2
    assert lib.sigattn_fwd(None, ok, ok, ok, two, None) == 1


def test_empty_batch_is_a_noop(lib):
    p, keep = S.make_problem(0, 2, 64, 64, [])
    assert S.validate(p) == 0
    # B = 0 enqueues nothing even with fake pointers
    a, b = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
    assert lib.sigattn_fwd(ctypes.byref(p), a, a, a, b, None) == 0
    assert S.plan(p, 0)[0].shape == (0, 3)


MIXED = [1000, 0, 1, 4096, 257, 4096, 3000]
ONE_LENGTH = [0, 1000, 1000, 1000, 0, 1000]     # one length (empty entries aside)


@pytest.mark.parametrize("pass_", [0, 1, 2])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("seqlens", [MIXED, ONE_LENGTH], ids=["mixed", "one_length"])
def test_plan_covers_exactly_the_valid_tiles(lib, pass_, causal, d, seqlens):
    """Every tile holding a valid row is listed exactly once; fully padded tiles never
    appear (block-sparse padding, section 4 of the sigmoid-attention paper)."""
    B, H, L = len(seqlens), 5, 4096
    p, keep = S.make_problem(B, H, L, d, seqlens, causal=causal)
    items, tile = S.plan(p, pass_)
    got = sorted(map(tuple, items.tolist()))
    want = sorted((b, h, t) for b, n in enumerate(seqlens) for h in range(H)
                  for t in range((n + tile - 1) // tile))
    assert got == want
    assert len(set(got)) == len(got)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seqlens", [MIXED, ONE_LENGTH], ids=["mixed", "one_length"])
def test_one_call_backward_list_covers_both_passes(lib, causal, seqlens):
    """The one-call backward's list (d = 64) holds every dK/dV tile and every dQ tile
    exactly once (dQ items reported with tile -1 - t); d = 128 has no such list."""
    B, H, L = len(seqlens), 3, 4096
    p, keep = S.make_problem(B, H, L, 64, seqlens, causal=causal)
    items, tile = S.plan(p, 3)
    want = sorted((b, h, t) for b, n in enumerate(seqlens) for h in range(H)
                  for t in range((n + tile - 1) // tile))
    got = items.tolist()
    assert sorted(tuple(x) for x in got if x[2] >= 0) == want
    assert sorted((b, h, -1 - t) for b, h, t in got if t < 0) == want
    p128, keep128 = S.make_problem(B, H, L, 128, seqlens, causal=causal)
    with pytest.raises(ValueError):
        S.plan(p128, 3)


def _causal_units(n, tile, t, key_side):
    """32 x 32 units of a causal tile, counted directly over its 32-row slices."""
    u = 0
    for r in range(t * tile // 32, min((t + 1) * tile // 32, -(-n // 32))):
        u += -(-n // 32) - r if key_side else r + 1
    return u


def _item_cost(n, tile, t, pass_):
    if pass_ == 3:
        return _causal_units(n, tile, t, True) * 1.42 if t >= 0 else _causal_units(n, tile, -1 - t, False)
    return _causal_units(n, tile, t, pass_ == 2)


@pytest.mark.parametrize("pass_", [0, 1, 2, 3])
def test_one_length_causal_batches_are_listed_tile_by_tile(lib, pass_):
    """Causal batches of one length, more items than one round of resident workgroups:
    each run of B * H consecutive items holds one tile of every (sequence, head), the
    runs in non-increasing work (the one-call list weighs a dK/dV unit 1.42 times a dQ
    unit), and item g runs on XCD g % 8, so that all tiles of one head share an XCD when
    B * H is a multiple of 8."""
    B, H, n = 8, 12, 2048
    p, keep = S.make_problem(B, H, 2048, 64, [n] * B, causal=True)
    items, tile = S.plan(p, pass_)
    m = B * H
    T = -(-n // tile)
    assert len(items) == m * T * (2 if pass_ == 3 else 1)
    costs = []
    for blk in range(len(items) // m):
        run = items[blk * m:(blk + 1) * m]
        assert sorted((b, h) for b, h, _ in run.tolist()) == [(b, h) for b in range(B) for h in range(H)]
        assert len(set(run[:, 2].tolist())) == 1
        costs.append(_item_cost(n, tile, int(run[0, 2]), pass_))
    assert costs == sorted(costs, reverse=True)
    xcd = {}
    for g, (b, h, _) in enumerate(items.tolist()):
        xcd.setdefault((b, h), set()).add(g % 8)
    assert all(len(x) == 1 for x in xcd.values())


@pytest.mark.parametrize("n,expect_blocks", [(1, True), (128, True), (8192, True),
                                              (8193, False)])
def test_one_call_list_block_limit(lib, n, expect_blocks):
    """The one-call list of a causal one-length batch is block-major up to 128 tile blocks
    (two passes of 64 tiles: n = 8192); one tile more keeps the per-sequence order. Both
    cover every tile of both passes exactly once."""
    B, H = 2, 3
    p, keep = S.make_problem(B, H, n, 64, [n] * B, causal=True)
    items, tile = S.plan(p, 3)
    T = -(-n // tile)
    want = sorted((b, h, t) for b in range(B) for h in range(H) for t in range(T))
    got = items.tolist()
    assert sorted(tuple(x) for x in got if x[2] >= 0) == want
    assert sorted((b, h, -1 - t) for b, h, t in got if t < 0) == want
    # block-major: the first B * H items are one tile of every (sequence, head)
    first = items[:B * H]
    is_block = (len(set(first[:, 2].tolist())) == 1
                and sorted((b, h) for b, h, _ in first.tolist()) == [(b, h) for b in range(B) for h in range(H)])
    assert is_block == expect_blocks or T == 1


def test_one_round_causal_forward_spreads_work_over_cus(lib):
    """A causal one-length forward that one round of resident workgroups holds (16 x 12
    heads x 4 tiles of 512 rows; three per CU): launch positions w, w + 256, w + 512 share
    a CU under round-robin dispatch, and every second span of 256 takes its items in
    reverse order of groups of 8, so the busiest CU carries at most 8 % more work than
    the average (24 % more in plain list order) while each head keeps its XCD."""
    B, H, n = 16, 12, 512
    p, keep = S.make_problem(B, H, 512, 64, [n] * B, causal=True)
    items, tile = S.plan(p, 0)
    assert len(items) == 768
    per_cu = np.zeros(256)
    for w, (b, h, t) in enumerate(items.tolist()):
        per_cu[w % 256] += _causal_units(n, tile, t, False)
    assert per_cu.max() <= 1.08 * per_cu.mean()
    xcd = {}
    for w, (b, h, _) in enumerate(items.tolist()):
        xcd.setdefault((b, h), set()).add(w % 8)
    assert all(len(x) == 1 for x in xcd.values())


def test_plan_orders_longest_first(lib):
    """Bidirectional work is listed longest sequence first (before the XCD grouping,
    which only permutes items within rounds of 8 chunks)."""
    os.environ.pop("SIGATTN_XCD_CHUNK", None)
    seqlens = [100, 4096, 2000]
    p, keep = S.make_problem(3, 2, 4096, 64, seqlens)
    items, tile = S.plan(p, 0)
    # items of batch 1 (longest) come first in any prefix of whole rounds
    first = items[: len(items) // 2, 0]
    assert (first == 1).mean() > 0.5


def test_plan_xcd_grouping_keeps_heads_together(lib):
    """Blocks w, w+8, w+16, ... (one XCD under round-robin dispatch) get consecutive
    items, so one head's tiles share an XCD."""
    p, keep = S.make_problem(4, 12, 8192, 64, [8192] * 4)
    items, tile = S.plan(p, 0)
    xcd0 = items[0::8][:16]
    assert len({(b, h) for b, h, t in xcd0.tolist()}) <= 2


def test_gate_gradient_entry_rejects_before_launch(lib):
    """sigattn_bwd_dkdv_dg needs a gate and a distinct, 4-byte aligned dg_head plane;
    every error is returned before anything is enqueued (fake pointers)."""
    vp = ctypes.c_void_p
    q, dk, dv, dgh, dg = (vp((1 << 20) * (i + 1)) for i in range(5))
    p, keep = _prob()
    f = lib.sigattn_bwd_dkdv_dg
    # no gate
    assert f(ctypes.byref(p), q, q, q, q, dk, dv, dgh, dg, None) == 1
    p, keep = _prob(gate_ptr=1 << 26)
    # missing dg_head
    assert f(ctypes.byref(p), q, q, q, q, dk, dv, None, dg, None) == 1
    # dg_head misaligned, or aliasing dk, or dg aliasing dg_head
    assert f(ctypes.byref(p), q, q, q, q, dk, dv, vp((1 << 23) + 2), dg, None) == 3
    assert f(ctypes.byref(p), q, q, q, q, dk, dv, dk, dg, None) == 1
    assert f(ctypes.byref(p), q, q, q, q, dk, dv, dgh, dgh, None) == 1
    # a bad problem is still reported first
    p.d = 96
    assert f(ctypes.byref(p), q, q, q, q, dk, dv, dgh, dg, None) == 2


def _cache(**kw):
    c = S.CacheDesc()
    c.struct_size = ctypes.sizeof(S.CacheDesc)
    c.B, c.H, c.d, c.cap = 2, 3, 64, 1000
    c.stride_b, c.stride_h, c.stride_l = 3 * 1000 * 64, 1000 * 64, 64
    c.k, c.v, c.gate = 1 << 20, 1 << 21, 1 << 22
    c.count, c.seen = 1 << 23, (1 << 23) + 64
    c.gate_eps, c.gate_tau, c.gate_sink = 1e-8, 0.05, 4
    for key, val in kw.items():
        setattr(c, key, val)
    return c


def test_decode_workspace_size(lib):
    c = _cache()
    # B * H * ceil(cap / 512) * d floats
    assert lib.sigattn_decode_workspace_size(ctypes.byref(c)) == 2 * 3 * 2 * 64 * 4
    c.cap = 1024
    assert lib.sigattn_decode_workspace_size(ctypes.byref(c)) == 2 * 3 * 2 * 64 * 4
    c.cap = 1025
    assert lib.sigattn_decode_workspace_size(ctypes.byref(c)) == 2 * 3 * 3 * 64 * 4
    c.struct_size += 4
    assert lib.sigattn_decode_workspace_size(ctypes.byref(c)) == -1


@pytest.mark.parametrize("mutate,code", [
    (lambda c: setattr(c, "d", 96), 2),
    (lambda c: setattr(c, "cap", 0), 1),
    (lambda c: setattr(c, "B", 300), 2),
    (lambda c: setattr(c, "k", None), 1),
    (lambda c: setattr(c, "v", (1 << 21) + 8), 3),
    (lambda c: setattr(c, "count", (1 << 23) + 2), 3),
    (lambda c: setattr(c, "seen", 1 << 23), 1),        # count and seen alias
    (lambda c: setattr(c, "stride_l", 60), 1),
    (lambda c: setattr(c, "stride_l", 68), 3),
    (lambda c: setattr(c, "gate_tau", -1.0), 1),
    (lambda c: setattr(c, "gate_sink", -1), 1),
])
def test_cache_validation_before_launch(lib, mutate, code):
    """Every cache entry point validates the cache description first and enqueues nothing
    on error (fake device pointers)."""
    c = _cache()
    mutate(c)
    vp = ctypes.c_void_p
    bias = (ctypes.c_float * 2)(-1.0, -2.0)
    assert lib.sigattn_decode(ctypes.byref(c), vp(1 << 24), 3 * 64, 64, bias, 0.0,
                              vp(1 << 25), 0, vp(1 << 26), 1 << 20, None) == code
    assert lib.sigattn_cache_append(ctypes.byref(c), vp(1 << 24), vp(1 << 25), 3 * 64, 64,
                                    vp(1 << 26), None, None) == code


def test_decode_argument_checks(lib):
    c = _cache()
    vp = ctypes.c_void_p
    bias = (ctypes.c_float * 2)(-1.0, -2.0)
    q, o, ws = vp(1 << 24), vp(1 << 25), vp(1 << 26)
    args = lambda **kw: dict(dict(q=q, sb=3 * 64, sh=64, bias=bias, scale=0.0, o=o, dt=0,
                                  ws=ws, wsb=1 << 20), **kw)

    def call(a):
        return lib.sigattn_decode(ctypes.byref(c), a["q"], a["sb"], a["sh"], a["bias"],
                                  a["scale"], a["o"], a["dt"], a["ws"], a["wsb"], None)
    assert call(args(bias=None)) == 1
    assert call(args(bias=(ctypes.c_float * 2)(float("nan"), 0.0))) == 1
    assert call(args(wsb=100)) == 1                  # workspace too small
    assert call(args(o=q)) == 1                      # output aliases the query
    assert call(args(ws=o)) == 1                     # workspace aliases the output
    assert call(args(dt=3)) == 2
    assert call(args(q=vp((1 << 24) + 4))) == 3
    assert call(args(sh=63)) == 3
    assert call(args(scale=-1.0)) == 1


def test_cache_build_checks(lib):
    c = _cache()
    vp = ctypes.c_void_p
    p, keep = S.make_problem(2, 3, 512, 64, [512, 100], gate_ptr=1 << 27)
    k, v = vp(1 << 28), vp(1 << 29)
    f = lib.sigattn_cache_build
    p.H = 4                                           # shape mismatch with the cache
    assert f(ctypes.byref(c), ctypes.byref(p), k, v, None) == 1
    p.H = 3
    c.cap = 300                                       # a prefill longer than the cache
    assert f(ctypes.byref(c), ctypes.byref(p), k, v, None) == 1
    c.cap = 1000
    c.gate = None                                     # gated prefill, ungated cache
    assert f(ctypes.byref(c), ctypes.byref(p), k, v, None) == 1
    c.gate = 1 << 22
    p.dtype = 1
    p.out_dtype = 1
    assert f(ctypes.byref(c), ctypes.byref(p), k, v, None) == 2


def _varlen(**kw):
    p = S.VarlenDesc()
    p.struct_size = ctypes.sizeof(S.VarlenDesc)
    p.B, p.H, p.d = 3, 2, 64
    p.max_seqlen_q, p.max_seqlen_k = 100, 200
    p.out_dtype, p.fast_math = 0, 0
    p.stride_t, p.stride_h = 128, 64
    p.cu_seqlens_q, p.cu_seqlens_k = 1 << 20, (1 << 20) + 64
    p.causal, p.scale = 0, 0.0
    p.gate_eps, p.gate_tau, p.gate_sink = 1e-8, 0.0, 4
    for key, val in kw.items():
        setattr(p, key, val)
    return p


@pytest.mark.parametrize("mutate,code", [
    (lambda p: setattr(p, "d", 80), 2),
    (lambda p: setattr(p, "H", 0), 1),
    (lambda p: setattr(p, "max_seqlen_q", -1), 1),
    (lambda p: setattr(p, "out_dtype", 4), 2),
    (lambda p: setattr(p, "causal", 3), 1),
    (lambda p: setattr(p, "stride_t", 100), 3),
    (lambda p: setattr(p, "stride_t", (1 << 22) + 8), 2),
    (lambda p: setattr(p, "cu_seqlens_q", None), 1),
    (lambda p: setattr(p, "cu_seqlens_k", (1 << 20) + 2), 3),
    (lambda p: setattr(p, "scale", -2.0), 1),
    (lambda p: (setattr(p, "gate", 1 << 24), setattr(p, "gate_tau", -1.0)), 1),
    (lambda p: (setattr(p, "B", 1 << 20), setattr(p, "H", 64), setattr(p, "stride_t", 64 * 64),
                setattr(p, "max_seqlen_k", 1 << 20)), 2),
    # B * H * ceil(max rows / 128) one past the work-item cap (2^23 - 1)
    (lambda p: (setattr(p, "B", 1 << 16), setattr(p, "H", 128), setattr(p, "stride_t", 128 * 64),
                setattr(p, "max_seqlen_q", 100)), 2),
    # rows of different heads overlap: stride_h below d, or heads wider than the row stride
    (lambda p: setattr(p, "stride_h", 32), 1),
    (lambda p: setattr(p, "H", 3), 1),
    (lambda p: setattr(p, "struct_size", 8), 1),
])
def test_varlen_validation_before_launch(lib, mutate, code):
    """Packed-batch entry points validate the description first (fake device pointers:
    nothing may be enqueued)."""
    p = _varlen()
    mutate(p)
    vp = ctypes.c_void_p
    t = [vp((1 << 21) * (i + 1)) for i in range(6)]
    assert lib.sigattn_fwd_varlen(ctypes.byref(p), t[0], t[1], t[2], t[3], None) == code
    assert lib.sigattn_bwd_dq_varlen(ctypes.byref(p), t[0], t[1], t[2], t[3], t[4], None) == code
    assert lib.sigattn_bwd_dkdv_varlen(ctypes.byref(p), t[0], t[1], t[2], t[3], t[4], t[5],
                                       None) == code
    assert lib.sigattn_bwd_varlen(ctypes.byref(p), t[0], t[1], t[2], t[3], t[4], t[5],
                                  vp(1 << 24), None) == code


def test_varlen_output_checks(lib):
    p = _varlen()
    vp = ctypes.c_void_p
    q, k, v = vp(1 << 21), vp(1 << 22), vp(1 << 23)
    assert lib.sigattn_fwd_varlen(ctypes.byref(p), q, k, v, q, None) == 1       # o aliases q
    assert lib.sigattn_fwd_varlen(ctypes.byref(p), q, k, v, None, None) == 1
    assert lib.sigattn_fwd_varlen(ctypes.byref(p), vp((1 << 21) + 4), k, v, vp(1 << 24), None) == 3
    two = vp(1 << 25)
    assert lib.sigattn_bwd_dkdv_varlen(ctypes.byref(p), q, k, v, q, two, two, None) == 1
    three, four = vp(1 << 26), vp(1 << 27)
    assert lib.sigattn_bwd_varlen(ctypes.byref(p), q, k, v, q, two, two, three, None) == 1
    assert lib.sigattn_bwd_varlen(ctypes.byref(p), q, k, v, q, two, three, k, None) == 1
    assert lib.sigattn_bwd_varlen(ctypes.byref(p), q, k, v, q, None, three, four, None) == 1
    assert lib.sigattn_bwd_varlen(ctypes.byref(p), q, k, v, q, vp((1 << 25) + 8), three, four,
                                  None) == 3


def test_noalloc_decode_checks_before_launch(lib):
    """sigattn_decode_noalloc validates like sigattn_decode and refuses a cache whose
    partial sums would not fit the library's 16 MiB static workspace; nothing is enqueued
    (fake device pointers)."""
    vp = ctypes.c_void_p
    q, o = vp(1 << 24), vp(1 << 25)
    f = lib.sigattn_decode_noalloc
    c = _cache()
    bias = (ctypes.c_float * 2)(-1.0, -2.0)
    assert f(ctypes.byref(c), q, 3 * 64, 64, None, 0.0, o, 0, None) == 1       # no bias
    assert f(ctypes.byref(c), q, 3 * 64, 64, bias, 0.0, q, 0, None) == 1       # o aliases q
    assert f(ctypes.byref(c), vp((1 << 24) + 4), 3 * 64, 64, bias, 0.0, o, 0, None) == 3
    assert f(ctypes.byref(c), q, 3 * 64, 64, bias, 0.0, o, 7, None) == 2
    # B * H * ceil(cap / 512) * d floats: 32 * 16 * 70 * 128 * 4 bytes > 16 MiB
    big = _cache(B=32, H=16, d=128, cap=70 * 512, stride_b=16 * 70 * 512 * 128,
                 stride_h=70 * 512 * 128, stride_l=128)
    assert lib.sigattn_decode_workspace_size(ctypes.byref(big)) > S.NOALLOC_WORKSPACE_BYTES
    b32 = (ctypes.c_float * 32)(*([-1.0] * 32))
    assert f(ctypes.byref(big), q, 16 * 128, 128, b32, 0.0, o, 0, None) == 2
    # one chunk fewer per (sequence, head) fits exactly: 32 * 16 * 64 * 128 * 4 = 16 MiB
    fits = _cache(B=32, H=16, d=128, cap=64 * 512, stride_b=16 * 64 * 512 * 128,
                  stride_h=64 * 512 * 128, stride_l=128)
    assert lib.sigattn_decode_workspace_size(ctypes.byref(fits)) == S.NOALLOC_WORKSPACE_BYTES

"""GPU parity of the KV cache with threshold eviction and of single-query decode,
through the C ABI, against the fp64 oracle ("Sigmoid Attention as a Better Substrate for
Learned KV Cache Eviction", gate paragraphs: removal after prefill, the same rule for
every newly written entry, kept entries keep their logit and value scaling).

Cache contents, counters and the overflow flag are integer / byte work: bit-exact.
Decode outputs meet the stated bar, max |gpu - ref| / rms(ref) <= 2e-2 (float outputs;
in practice float rounding only), and sequences with an empty cache give exactly 0.
"""

import math

import numpy as np
import pytest

import oracle as O
import sigmoid_attention_amd as S
import workloads as W
from gpu_util import BF16_TOL, err_ratio, need_gpu, note

pytestmark = pytest.mark.gpu


def _dev(torch, x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype).cuda() if dtype is not None else t.cuda()


def _oracle_cache(data, cap):
    return O.cache_compact(data["k"], data["v"], data["seqlens"], cap, gate=data["gate"],
                           tau=data["tau"], sink=data["sink"])


def _gpu_cache_state(cache):
    import torch
    torch.cuda.synchronize()
    return (cache.k.float().cpu().numpy(), cache.v.float().cpu().numpy(),
            None if cache.gate is None else cache.gate.cpu().numpy(),
            cache.count.cpu().numpy().astype(np.int64), cache.seen.cpu().numpy().astype(np.int64))


def _assert_same_cache(gpu, ref, label):
    gk, gv, gg, gc, gs = gpu
    rk, rv, rg, rc, rs = ref
    np.testing.assert_array_equal(gc, rc, err_msg=f"{label}: count")
    np.testing.assert_array_equal(gs, rs, err_msg=f"{label}: seen")
    for b in range(len(rc)):
        m = int(rc[b])
        np.testing.assert_array_equal(gk[b, :, :m], rk[b, :, :m], err_msg=f"{label}: K b={b}")
        np.testing.assert_array_equal(gv[b, :, :m], rv[b, :, :m], err_msg=f"{label}: V b={b}")
        if rg is not None:
            np.testing.assert_array_equal(gg[b, :m], rg[b, :m], err_msg=f"{label}: gate b={b}")


def _small(d, gated, lens=(300, 0, 1, 3, 257, 512), cap=600, seed=0):
    gate = ("logistic_normal", 1.0, 2.0, 0.3, 0.01) if gated else None
    w = W.Workload(f"dec_small_{d}_{int(gated)}", "bf16", len(lens), 3, d, max(512, max(lens)),
                   ("fixed", list(lens)), seed=300 + d + seed, gate=gate,
                   tau=0.05 if gated else 0.0, sink=4, extra={"cap": cap})
    return W.generate_decode(w)


def _make_cache(torch, data, d):
    B, H = data["k"].shape[:2]
    return S.KVCache(B, H, d, data["cap"], gated=data["gate"] is not None, tau=data["tau"],
                     sink=data["sink"])


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_cache_build_append_decode_small(d, gated):
    """Prefill compaction (ragged lengths, an empty and a one-token sequence, a sequence
    shorter than the sink), one append per sequence, decode before and after."""
    torch = need_gpu()
    data = _small(d, gated)
    cap = data["cap"]
    cache = _make_cache(torch, data, d)
    gate_t = None if data["gate"] is None else _dev(torch, data["gate"])
    note(f"cache build d={d} gated={gated}")
    cache.build(_dev(torch, data["k"], torch.bfloat16), _dev(torch, data["v"], torch.bfloat16),
                data["seqlens"], gate=gate_t)
    ref = _oracle_cache(data, cap)
    _assert_same_cache(_gpu_cache_state(cache), ref, "build")
    bias = [-math.log(max(int(n), 1)) for n in data["seqlens"]]
    q = _dev(torch, data["q"], torch.bfloat16)
    for step in range(2):
        note(f"decode d={d} gated={gated} step={step}")
        out = cache.decode(q, bias, out_dtype=torch.float32)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = O.decode(data["q"], ref[0], ref[1], ref[2], ref[3], bias)
        empty = ref[3] == 0
        assert np.all(got[empty] == 0.0)
        e = err_ratio(got, want, np.broadcast_to(~empty[:, None, None], got.shape))
        print(f"decode step {step}: ratio {e:.3e}")
        assert e <= BF16_TOL
        if step == 0:
            note(f"cache append d={d} gated={gated}")
            g_new = None if data["g_new"] is None else _dev(torch, data["g_new"])
            cache.append(_dev(torch, data["k_new"], torch.bfloat16),
                         _dev(torch, data["v_new"], torch.bfloat16), g_new)
            ref = O.cache_append(*ref, data["k_new"], data["v_new"], data["g_new"],
                                 tau=data["tau"], sink=data["sink"])
            _assert_same_cache(_gpu_cache_state(cache), ref, "append")
    # bf16 output of the same decode
    out16 = cache.decode(q, bias)
    torch.cuda.synchronize()
    got16 = out16.float().cpu().numpy()
    want = O.decode(data["q"], ref[0], ref[1], ref[2], ref[3], bias)
    assert np.all(np.abs(got16 - want) <= 2.0 ** -8 * np.abs(want) + 1e-6 * np.abs(want).max())


def test_decode_token_by_token_matches_oracle_forward():
    """40 tokens written one at a time into an empty gated cache (threshold rule at
    every write), decoding each token's query after its write: every step equals row i
    of the oracle's causal forward with hard dropping at the sequence bias."""
    torch = need_gpu()
    B, H, L, d = 3, 2, 40, 64
    rng = np.random.default_rng(77)
    q, k, v = (W.round_to_bf16(rng.standard_normal((B, H, L, d), dtype=np.float32))
               for _ in range(3))
    g = rng.uniform(0.0, 1.0, (B, L)).astype(np.float32)
    tau, sink = 0.3, 4
    bias = [-math.log(L)] * B
    ref = O.forward(q, k, v, [L] * B, causal=True, gate=g, tau=tau, sink=sink,
                    bias=np.array(bias))
    cache = S.KVCache(B, H, d, 64, gated=True, tau=tau, sink=sink)
    outs = []
    for i in range(L):
        cache.append(_dev(torch, k[:, :, i], torch.bfloat16), _dev(torch, v[:, :, i], torch.bfloat16),
                     _dev(torch, np.ascontiguousarray(g[:, i])))
        outs.append(cache.decode(_dev(torch, q[:, :, i], torch.bfloat16), bias,
                                 out_dtype=torch.float32))
    note("token-by-token decode, 40 steps")
    torch.cuda.synchronize()
    got = np.stack([o.cpu().numpy() for o in outs], axis=2)
    e = err_ratio(got, ref, np.ones(got.shape, bool))
    print("token-by-token ratio", e)
    assert e <= BF16_TOL
    kept = [sum(1 for j in range(L) if j < sink or g[b, j] >= tau) for b in range(B)]
    np.testing.assert_array_equal(cache.count.cpu().numpy(), kept)
    np.testing.assert_array_equal(cache.seen.cpu().numpy(), [L] * B)


def test_cache_append_overflow_sets_status():
    """A kept entry that finds its cache full is not stored, the status word is set, and
    the position counter still advances; a dropped entry never overflows."""
    torch = need_gpu()
    B, H, d, cap = 2, 2, 64, 8
    rng = np.random.default_rng(78)
    k = W.round_to_bf16(rng.standard_normal((B, H, cap, d), dtype=np.float32))
    g = np.full((B, cap), 0.9, np.float32)
    cache = S.KVCache(B, H, d, cap, gated=True, tau=0.05, sink=4)
    note("cache overflow")
    kt = _dev(torch, k, torch.bfloat16)
    cache.build(kt, kt.clone(), [cap, 3], gate=_dev(torch, g))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    new = _dev(torch, k[:, :, 0], torch.bfloat16)
    cache.append(new, new.clone(), _dev(torch, np.array([0.01, 0.9], np.float32)), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0                     # b=0 dropped (no overflow), b=1 fits
    assert cache.count.cpu().tolist() == [cap, 4] and cache.seen.cpu().tolist() == [cap + 1, 4]
    cache.append(new, new.clone(), _dev(torch, np.array([0.9, 0.9], np.float32)), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    assert cache.count.cpu().tolist() == [cap, 5] and cache.seen.cpu().tolist() == [cap + 2, 5]


@pytest.mark.parametrize("name", ["decode_gpt2_512", "decode_long", "decode_long_64"])
def test_decode_workloads(name):
    """The decode workloads at full size: cache contents bit-exact for sampled sequences
    and decode outputs of sampled (b, h) against the oracle."""
    torch = need_gpu()
    data = W.generate_decode(name)
    B, H, L, d = data["k"].shape
    cap = data["cap"]
    note(f"{name}: build, append, decode at full size")
    cache = S.KVCache(B, H, d, cap, gated=True, tau=data["tau"], sink=data["sink"])
    cache.build(_dev(torch, data["k"], torch.bfloat16), _dev(torch, data["v"], torch.bfloat16),
                data["seqlens"], gate=_dev(torch, data["gate"]))
    cache.append(_dev(torch, data["k_new"], torch.bfloat16), _dev(torch, data["v_new"], torch.bfloat16),
                 _dev(torch, data["g_new"]))
    bias = [-math.log(int(n)) for n in data["seqlens"]]
    out = cache.decode(_dev(torch, data["q"], torch.bfloat16), bias, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    counts = cache.count.cpu().numpy()
    sl = data["seqlens"]
    picks = sorted({int(np.argmin(sl)), int(np.argmax(sl)), B // 2})
    refs, gots = [], []
    for b in picks:
        sub = {key: data[key][b:b + 1] for key in ("k", "v", "gate", "k_new", "v_new", "g_new", "q")}
        st = O.cache_compact(sub["k"], sub["v"], sl[b:b + 1], cap, gate=sub["gate"],
                             tau=data["tau"], sink=data["sink"])
        st = O.cache_append(*st, sub["k_new"], sub["v_new"], sub["g_new"], tau=data["tau"],
                            sink=data["sink"])
        assert counts[b] == st[3][0]
        m = int(st[3][0])
        np.testing.assert_array_equal(cache.k[b, :, :m].float().cpu().numpy(), st[0][0, :, :m])
        np.testing.assert_array_equal(cache.gate[b, :m].cpu().numpy(), st[2][0, :m])
        want = O.decode(sub["q"], *st[:4], bias[b:b + 1])
        refs.append(want[0])
        gots.append(got[b])
    e = err_ratio(np.stack(gots), np.stack(refs), np.ones((len(picks), H, d), bool))
    print(f"{name}: ratio {e:.3e}, live fraction {counts.sum() / (sl.sum() + B):.3f}")
    assert e <= BF16_TOL


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_counts_around_chunk_edges(d, gated):
    """Cache lengths around the decode's 16-row steps, 128-row wave slices and 512-row
    chunks (1, 15, 16, 17, 127, 128, 129, 511, 512, 513, 1000, 1024 prefill positions)."""
    torch = need_gpu()
    data = _small(d, gated, lens=(1, 15, 16, 17, 127, 128, 129, 511, 512, 513, 1000, 1024),
                  cap=1100, seed=7)
    cache = _make_cache(torch, data, d)
    gate_t = None if data["gate"] is None else _dev(torch, data["gate"])
    note(f"decode chunk edges d={d} gated={gated}")
    cache.build(_dev(torch, data["k"], torch.bfloat16), _dev(torch, data["v"], torch.bfloat16),
                data["seqlens"], gate=gate_t)
    ref = _oracle_cache(data, data["cap"])
    _assert_same_cache(_gpu_cache_state(cache), ref, "build")
    bias = [-math.log(int(n)) for n in data["seqlens"]]
    out = cache.decode(_dev(torch, data["q"], torch.bfloat16), bias, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = O.decode(data["q"], ref[0], ref[1], ref[2], ref[3], bias)
    e = err_ratio(got, want, np.ones(got.shape, bool))
    print(f"decode chunk edges ratio {e:.3e}")
    assert e <= BF16_TOL

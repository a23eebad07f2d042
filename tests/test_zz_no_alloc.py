"""The allocation-free decode entry point (sigattn_decode_noalloc) against the decode that
takes a caller workspace (sigattn_decode), through the C ABI: the same kernels, so the
outputs must be bitwise equal. Two calls in a row, the second on a smaller cache, show
that the static workspace left by one call does not leak into the next. (A cache whose
workspace would exceed the static array is refused on the host: tests/test_abi.py.)
"""

import math

import numpy as np
import pytest

import sigmoid_attention_amd as S
import workloads as W
from gpu_util import need_gpu, note

pytestmark = pytest.mark.gpu


def _cache_and_query(torch, d, lens, cap, H, seed, gated):
    gate = ("logistic_normal", 1.0, 2.0, 0.3, 0.01) if gated else None
    w = W.Workload(f"noalloc_{d}_{seed}", "bf16", len(lens), H, d, max(512, max(lens)),
                   ("fixed", list(lens)), seed=seed, gate=gate, tau=0.05 if gated else 0.0,
                   sink=4, extra={"cap": cap})
    data = W.generate_decode(w)
    B = len(lens)
    cache = S.KVCache(B, H, d, cap, gated=gated, tau=data["tau"], sink=data["sink"])
    dev = lambda x, dt=None: (torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()
                              if dt is not None else torch.from_numpy(np.ascontiguousarray(x)).cuda())
    cache.build(dev(data["k"], torch.bfloat16), dev(data["v"], torch.bfloat16), data["seqlens"],
                gate=None if data["gate"] is None else dev(data["gate"]))
    q = dev(data["q"], torch.bfloat16)
    bias = [-math.log(max(int(n), 1)) for n in data["seqlens"]]
    return cache, q, bias


def test_noalloc_decode_matches_workspace_decode():
    torch = need_gpu()
    cases = [
        # (d, prefill lengths, cap, H, seed, gated, out dtype)
        (128, (2000, 0, 1, 1537, 700), 2048, 4, 401, True, torch.float32),
        (64, (300, 5, 64), 600, 2, 402, False, torch.bfloat16),
    ]
    for d, lens, cap, H, seed, gated, odt in cases:
        note(f"noalloc decode d={d} lens={lens} cap={cap} H={H} gated={gated} out={odt}")
        cache, q, bias = _cache_and_query(torch, d, lens, cap, H, seed, gated)
        assert cache.workspace_size() <= S.NOALLOC_WORKSPACE_BYTES
        ref = cache.decode(q, bias, out_dtype=odt)
        out = torch.full_like(ref, float("nan"))
        cache.decode_noalloc(q, bias, out=out, out_dtype=odt)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"d={d} lens={lens}: noalloc decode differs"
        # a second call into the same output, after the cache grew by one appended entry
        B = len(lens)
        g = torch.rand(B, generator=torch.Generator().manual_seed(seed)).cuda() if gated else None
        k1 = torch.randn((B, H, d), generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16).cuda()
        v1 = torch.randn((B, H, d), generator=torch.Generator().manual_seed(seed + 2)).to(torch.bfloat16).cuda()
        cache.append(k1, v1, g)
        ref2 = cache.decode(q, bias, out_dtype=odt)
        cache.decode_noalloc(q, bias, out=out, out_dtype=odt)
        torch.cuda.synchronize()
        assert torch.equal(out, ref2), f"d={d} lens={lens}: noalloc decode after append differs"

"""Benchmark: effective TFLOPS of padded bf16 sigmoid attention (forward + backward) on
one MI355X, the fp64 CPU oracle timed beside it.

One step = one pass of the whole hot path over one batch: sigattn_fwd, then sigattn_bwd
(the dQ and dK/dV kernels; at d = 64 their work items share one launch). FLOPs are counted over valid tokens only: 4 d per valid
(query, key) pair forward, 2.5x that backward (the FLOP appendix of "Better Models,
Faster Training: Sigmoid Attention for single-cell Foundation Models"), n^2 pairs per
head bidirectional, n(n+1)/2 causal. Inputs are resident in HBM before timing starts.
The two backward passes are also timed alone, outside the timed step (sigattn_bwd_dq and
sigattn_bwd_dkdv under "kernels"). `ms_per_step` and `value` come from K steps between two
events with nothing else in the stream; each call's duration (the per-kernel figures and
`roofline`) from a second run of the same K steps with an event before and after each call.
The host enqueues each timed loop while a spin kernel, ahead of the loop's first event,
holds the GPU, so that short launches run back to back instead of at the host's pace.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_8k_s1]
                    [--no-cpu-baseline]

Prints one JSON line. With a decode workload (--workload decode_long, decode_long_64,
decode_gpt2_512) a step is one sigattn_decode of one query per (sequence, head) against a
KV cache built by threshold eviction from a synthetic prefill, and the metric is the
algorithmic HBM bandwidth of that decode (live cached K and V rows and their gates, the
query and the output, per second) against the 8 TB/s of HBM3E.
"""

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective fwd/bwd TFLOPS, bf16 padded sigmoid attn, L=8K; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
# algorithmic MFMA FLOPs per valid pair, per launch: forward S and P.V (2 x 2d); the
# backward's dQ kernel recomputes S, forms dP and dQ (3 x 2d) and its dK/dV kernel
# recomputes S, forms dP, dV, dK (4 x 2d): 14 d per pair for the one-call backward. The
# credited backward (2.5 x forward = 10 d) counts S and dP once.
PASS_FLOPS_PER_PAIR = {"fwd": 4, "bwd": 14, "bwd_dq": 6, "bwd_dkdv": 8}
TIMING = ("step: K steps between two HIP events, no other events in the stream; per call: "
          "a second run of K steps with a HIP event before and after each call; each loop "
          "is enqueued while a spin kernel ahead of its first event holds the GPU")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long_8k_s1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-padding-line", action="store_true",
                    help="skip the 0 %% / 25 %% padding pair reported beside the headline")
    ap.add_argument("--fast-math", action="store_true",
                    help="time the single-bf16 operand mode instead of the default hi+lo split")
    ap.add_argument("--f16-forward", action="store_true",
                    help="time fast_math = 2 (P V on f16 operands in the forward, hi+lo "
                         "backward) instead of the default")
    ap.add_argument("--bf16-out", action="store_true", help="bf16 outputs instead of float")
    ap.add_argument("--also-fast", action="store_true",
                    help="also time fast math with bf16 outputs and report it beside the default")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run a plain copy kernel of known size and 3 launches of each pass, for "
                         "a rocprofv3 --pmc run (prints nothing else)")
    ap.add_argument("--pmc-collect", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter_collection.csv files of a FETCH_SIZE run and a "
                         "WRITE_SIZE run of --pmc-pass into profiles/traffic_<workload>.json")
    ap.add_argument("--sweep", action="store_true",
                    help="the pages' kernel sweep: L = 512..16384 at B*L = 16384 tokens, d = 64 "
                         "(32 heads) and 128 (16 heads), 0 %% and 25 %% padding; forward and "
                         "backward TFLOPS, mean and 99 %% interval over 250 iterations")
    ap.add_argument("--causal", action="store_true",
                    help="with --sweep: causal attention, every sequence at full length "
                         "(no padding)")
    ap.add_argument("--packed", action="store_true",
                    help="run the workload's sequences packed (device cu_seqlens, no padding) "
                         "through sigattn_fwd_varlen and sigattn_bwd_varlen")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="lower bound on the oracle time of the CPU baseline sample")
    return ap.parse_args()


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), else the platform's description."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(data, w, min_seconds):
    """Time the oracle, as it stands, on a bounded sample of the same workload: full
    forward + backward of whole (batch entry, head) pairs, starting with the entry of
    median length and going on to the entries closest to it, one head after another
    until at least `min_seconds` have passed (or the workload is done), on the host
    cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    sl = [int(x) for x in data["seqlens"]]
    med = sorted(sl)[len(sl) // 2]
    order = sorted((b for b in range(len(sl)) if sl[b] > 0), key=lambda b: (abs(sl[b] - med), b))
    kw = dict(causal=w.causal)
    t_fwd = t_bwd = 0.0
    pairs = 0
    done = []   # (batch entry, heads done)
    for b in order:
        n = sl[b]
        for h in range(w.H):
            q = data["q"][b:b + 1, h:h + 1].astype(np.float64)
            k = data["k"][b:b + 1, h:h + 1].astype(np.float64)
            v = data["v"][b:b + 1, h:h + 1].astype(np.float64)
            do = data["do"][b:b + 1, h:h + 1].astype(np.float64)
            t0 = time.perf_counter()
            oracle.forward(q, k, v, [n], **kw)
            t1 = time.perf_counter()
            oracle.backward(q, k, v, do, [n], **kw)
            t2 = time.perf_counter()
            t_fwd += t1 - t0
            t_bwd += t2 - t1
            pairs += n * (n + 1) // 2 if w.causal else n * n
            if done and done[-1][0] == b:
                done[-1] = (b, done[-1][1] + 1)
            else:
                done.append((b, 1))
            if t_fwd + t_bwd >= min_seconds:
                break
        if t_fwd + t_bwd >= min_seconds:
            break
    flops = 4.0 * w.d * pairs * 3.5   # forward + credited backward (2.5x forward)
    parts = ", ".join(f"{hd} of {w.H} heads of entry {b} (n={sl[b]})" for b, hd in done)
    return {
        "value": flops / (t_fwd + t_bwd) / 1e12,
        "unit": "TFLOPS",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle, forward+backward of {parts} of {w.name}; "
                  f"fwd {t_fwd:.2f} s, bwd {t_bwd:.2f} s",
        "host": cpu_model(),
        "host_cpus": os.cpu_count(),
    }


def cpu_baseline_decode(data, w, bias, min_seconds):
    """The oracle's cache compaction + decode, timed per sequence until `min_seconds`
    have passed, as algorithmic bytes per second (the GPU metric's unit)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    t_dec, nbytes, seqs = 0.0, 0, 0
    for b in range(w.B):
        sub = {key: data[key][b:b + 1] for key in ("k", "v", "gate", "q")}
        st = oracle.cache_compact(sub["k"], sub["v"], data["seqlens"][b:b + 1], data["cap"],
                                  gate=sub["gate"], tau=w.tau, sink=w.sink)
        t0 = time.perf_counter()
        oracle.decode(sub["q"], *st[:4], bias[b:b + 1])
        t_dec += time.perf_counter() - t0
        nbytes += decode_bytes(st[3], w.H, w.d, 4)
        seqs += 1
        if t_dec >= min_seconds:
            break
    return {"value": nbytes / t_dec / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle decode of {seqs} of the {w.B} sequences of {w.name} "
                      f"(all heads), {t_dec:.2f} s; cache compaction untimed",
            "host": cpu_model(), "host_cpus": os.cpu_count()}


def decode_bytes(counts, H, d, out_bytes):
    """Algorithmic bytes of one decode: every live cached K and V row (bf16) and its gate
    (float, read once per head), the bf16 query and the output of every (b, h)."""
    live = int(np.sum(counts))
    return live * H * (2 * d * 2 + 4) + len(counts) * H * d * (2 + out_bytes)


def hold_gpu(stream, steps):
    """Keep the GPU busy (a spin kernel, before the first event) while the host enqueues a
    timed loop, so that the loop's launches run back to back. Otherwise a loop of short
    launches is paced by the host's launch path, and host time lands between events."""
    import torch
    spin = getattr(torch.cuda, "_sleep", None)   # torch's spin kernel (a private helper)
    if spin is None:
        return
    with torch.cuda.stream(stream):
        spin(int(min(steps, 400) * 1_000_000))   # about 0.5 ms per step at 2 GHz


def time_steps(stream, steps, calls, step_time=True):
    """K steps of `calls` (name -> function, run in order) on `stream`, timed twice: first
    between two events with nothing else in the stream (the step time; skipped when
    step_time is False), then again with an event before and after each call (each call's
    duration, per step). The host enqueues each loop while the GPU is held busy."""
    import torch

    def ev():
        return torch.cuda.Event(enable_timing=True)

    ms_step = None
    if step_time:
        start, end = ev(), ev()
        torch.cuda.synchronize()
        hold_gpu(stream, steps)
        start.record(stream)
        for _ in range(steps):
            for fn in calls.values():
                fn()
        end.record(stream)
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(end) / steps
    evs = [[ev() for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    hold_gpu(stream, steps)
    for e in evs:
        for i, fn in enumerate(calls.values()):
            e[i].record(stream)
            fn()
        e[-1].record(stream)
    torch.cuda.synchronize()
    per = {name: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, name in enumerate(calls)}
    return ms_step, per


def measure_decode(S, W, w, steps, warmup, no_cpu, cpu_seconds):
    import math

    import torch
    data = W.generate_decode(w)
    dev = torch.device("cuda:0")
    B, H, L, d = data["k"].shape
    cache = S.KVCache(B, H, d, data["cap"], gated=data["gate"] is not None, tau=w.tau,
                      sink=w.sink)
    cache.build(torch.from_numpy(data["k"]).to(torch.bfloat16).to(dev),
                torch.from_numpy(data["v"]).to(torch.bfloat16).to(dev), data["seqlens"],
                gate=None if data["gate"] is None else torch.from_numpy(data["gate"]).to(dev))
    q = torch.from_numpy(data["q"]).to(torch.bfloat16).to(dev)
    bias = np.array([-math.log(max(int(n), 1)) for n in data["seqlens"]])
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, cache.workspace_size() // 4), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        cache.decode(q, bias, out=out, out_dtype=torch.float32, workspace=ws)
    ms_step, per = time_steps(stream, steps, {"decode": lambda: cache.decode(
        q, bias, out=out, out_dtype=torch.float32, workspace=ws)})
    ms_dec = float(np.mean(per["decode"]))
    counts = cache.count.cpu().numpy()
    nbytes = decode_bytes(counts, H, d, 4)
    res = {
        "metric": "decode HBM bandwidth, bf16 sigmoid attention against a KV cache with "
                  "threshold eviction (GB/s of algorithmic bytes)",
        "value": nbytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "timing": TIMING,
        "config": {"workload": w.name, "B": B, "H": H, "d": d, "cap": data["cap"],
                   "prefill_lengths": [int(x) for x in data["seqlens"]],
                   "live_entries": [int(x) for x in counts], "tau": w.tau, "sink": w.sink,
                   "step": "sigattn_decode (decode kernel + chunk reduction)"},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel + decode_reduce_kernel",
                     "achieved": nbytes / (ms_dec * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": nbytes / (ms_dec * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": traffic_for(w.name, "decode")},
        "algorithmic_bytes": nbytes,
    }
    # a plain streaming read + write of the same order of size (torch's float32 multiply,
    # the kernel the traffic counters are calibrated on): the measured counterpart of the
    # published HBM peak
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2.0, out=dst)
    cp = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(20)]
    torch.cuda.synchronize()
    hold_gpu(stream, 20)
    for e0, e1 in cp:
        e0.record(stream)
        torch.mul(src, 2.0, out=dst)
        e1.record(stream)
    torch.cuda.synchronize()
    ms_cp = float(np.median([e0.elapsed_time(e1) for e0, e1 in cp]))
    cp_gbs = 2 * COPY_ELEMS * 4 / (ms_cp * 1e-3) / 1e9
    res["hbm_stream_measured"] = {
        "gbs": cp_gbs, "kernel": "torch float32 multiply, 256 MiB read + 256 MiB written",
        "decode_frac": res["roofline"]["achieved"] / cp_gbs}
    del src, dst
    if not no_cpu:
        res["cpu_baseline"] = cpu_baseline_decode(data, w, bias, cpu_seconds)
    return res


# kernel names in rocprofv3 output (bwd_kernel: the one-call backward at d = 64)
PASS_KERNELS = {"fwd": "fwd_kernel", "bwd": "bwd_kernel"}
DECODE_KERNELS = {"decode": "decode_kernel"}
COPY_ELEMS = 64 << 20          # float32 elements read and written by the calibration copy


def source_hash():
    """sha256 of the library's kernel and host sources: traffic figures are tied to it."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sigmoid_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def pmc_collect(workload, fetch_csv, write_csv):
    """HBM bytes per launch of each pass from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by the factor that maps the same counter onto the known bytes of a plain
    copy (COPY_ELEMS float32 read and written)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                vals.setdefault(name, []).append(float(row["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = COPY_ELEMS * 4

    def pick(vals, key):
        rows = [v for k, vs in vals.items() if key in k for v in vs]
        if not rows:
            raise SystemExit(f"no dispatch of {key} in the counter file")
        return sum(rows) / len(rows)

    copy_key = "MulFunctor"    # torch's kernel for the calibration multiply
    f_copy, w_copy = pick(fetch, copy_key), pick(write, copy_key)
    out = {
        "workload": workload,
        "source_hash": source_hash(),
        "calibration": {"kernel": "torch elementwise multiply (float32, out of place)",
                        "bytes_read": copy_bytes, "bytes_written": copy_bytes,
                        "fetch_kib": f_copy, "write_kib": w_copy,
                        "fetch_factor": copy_bytes / (f_copy * 1024.0),
                        "write_factor": copy_bytes / (w_copy * 1024.0)},
        "kernels": {},
        "command": "rocprofv3 --pmc FETCH_SIZE -d <dir> -o p -f csv -- python3 bench.py --pmc-pass "
                   f"--workload {workload}; the same with WRITE_SIZE; then python bench.py "
                   f"--workload {workload} --pmc-collect <fetch csv> <write csv>",
    }
    keys = DECODE_KERNELS if workload.startswith("decode") else PASS_KERNELS
    for name, key in keys.items():
        fk, wk = pick(fetch, key), pick(write, key)
        hbm = fk * 1024.0 * out["calibration"]["fetch_factor"] + wk * 1024.0 * out["calibration"]["write_factor"]
        out["kernels"][name] = {"fetch_kib": fk, "write_kib": wk, "hbm_bytes": hbm}
    os.makedirs(os.path.dirname(traffic_path(workload)), exist_ok=True)
    with open(traffic_path(workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def traffic_for(workload, kernel):
    """Calibrated HBM bytes per launch of `kernel`, or None when no counters were taken for
    the current sources."""
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    return t["kernels"].get(kernel, {}).get("hbm_bytes")


def pmc_pass_decode(S, W, w):
    import math

    import torch
    data = W.generate_decode(w)
    B, H, L, d = data["k"].shape
    cache = S.KVCache(B, H, d, data["cap"], gated=True, tau=w.tau, sink=w.sink)
    cache.build(torch.from_numpy(data["k"]).to(torch.bfloat16).cuda(),
                torch.from_numpy(data["v"]).to(torch.bfloat16).cuda(), data["seqlens"],
                gate=torch.from_numpy(data["gate"]).cuda())
    q = torch.from_numpy(data["q"]).to(torch.bfloat16).cuda()
    bias = [-math.log(max(int(n), 1)) for n in data["seqlens"]]
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 2.0, out=dst)
    for _ in range(3):
        cache.decode(q, bias, out_dtype=torch.float32)
    torch.cuda.synchronize()


def pmc_pass(S, w, t, gate, sl, out_dtype, fast_math):
    import torch
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=t["q"].device)
    dst = torch.empty_like(src)
    torch.mul(src, 2.0, out=dst)
    kw = dict(causal=w.causal, gate=gate, tau=w.tau, sink=w.sink, out_dtype=out_dtype,
              fast_math=fast_math)
    for _ in range(3):
        S.fwd(t["q"], t["k"], t["v"], sl, **kw)
        S.bwd(t["q"], t["k"], t["v"], t["do"], sl, **kw)
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path needs no "
              "collectives and every (batch, head) is independent; run one process per GPU "
              "with its own share of the batch.", file=sys.stderr)
        sys.exit(2)

    if args.pmc_collect:
        pmc_collect(args.workload, *args.pmc_collect)
        return

    import torch

    import sigmoid_attention_amd as S
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    S.load()
    if args.sweep:
        print(json.dumps(sweep(S, W, iters=250,
                               fast_math=1 if args.fast_math else (2 if args.f16_forward else 0),
                               causal=args.causal)))
        return
    w = W.WORKLOADS[args.workload]
    if w.name.startswith("decode"):
        if args.pmc_pass:
            pmc_pass_decode(S, W, w)
            return
        print(json.dumps(measure_decode(S, W, w, args.steps, args.warmup, args.no_cpu_baseline,
                                        args.cpu_seconds)))
        return
    data = W.generate(w)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(data[k]).to(torch.bfloat16).to(dev) for k in ("q", "k", "v", "do")}
    gate = None if data["gate"] is None else torch.from_numpy(data["gate"]).to(dev)
    sl = data["seqlens"]
    stream = torch.cuda.current_stream(dev)
    out_dtype = torch.bfloat16 if args.bf16_out else torch.float32
    fast_math = 1 if args.fast_math else (2 if args.f16_forward else 0)
    mode = {"inputs": "bf16", "outputs": "bf16" if args.bf16_out else "float32",
            "operands": ["bf16 hi+lo split", "bf16",
                         "forward P V in f16, backward bf16 hi+lo split"][fast_math]}
    if args.pmc_pass:
        pmc_pass(S, w, t, gate, sl, out_dtype, fast_math)
        return
    if args.packed:
        res = measure_packed(S, W, w, data, stream, args.steps, args.warmup, out_dtype,
                             fast_math)
        res["mode"] = mode
        print(json.dumps(res))
        return
    res = measure(S, W, w, t, gate, sl, stream, args.steps, args.warmup, out_dtype,
                  fast_math)
    res["mode"] = mode
    # the bf16 MFMA rate and shader clock this GPU sustains in a register-only MFMA loop:
    # the measured counterpart of the published peak (the attention kernels run at their
    # own, lower clock under load)
    cal = S.calibrate_mfma()
    res["mfma_peak_measured"] = {
        "tflops": cal["tflops"], "sclk_mhz": cal["sclk_mhz"],
        "kernel": "sigattn_calibrate_mfma: v_mfma_f32_32x32x16_bf16 loop, 4 accumulators",
        "dominant_frac": res["roofline"]["achieved"] / cal["tflops"],
        "fwd_frac": res["fwd_tflops"] / cal["tflops"]}
    if fast_math == 0:
        # the opt-in f16 forward beside the default (same step, same inputs)
        f16 = measure(S, W, w, t, gate, sl, stream, args.steps, args.warmup, out_dtype, 2)
        res["f16_forward_mode"] = {
            "fast_math": 2, "value": f16["value"], "ms_per_step": f16["ms_per_step"],
            "fwd_tflops": f16["fwd_tflops"], "fwd_pct_peak": f16["fwd_pct_peak"],
            "fwd_ms": f16["kernels"]["fwd"]["avg_ms"],
            "note": "P V on f16 operands in the forward (P rounded to f16, 2^-11); meets "
                    "the stated bar when the batch's output rows are of similar size"}
    if not args.no_padding_line:
        res["padding_loss"] = padding_loss(S, W, stream, 20, 5, out_dtype, fast_math)
    if args.also_fast:
        fast = measure(S, W, w, t, gate, sl, stream, args.steps, args.warmup,
                       torch.bfloat16, True)
        res["fast_math_bf16_out"] = {k_: fast[k_] for k_ in ("value", "ms_per_step", "fwd_tflops",
                                                             "bwd_tflops", "fwd_pct_peak", "kernels")}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(data, w, args.cpu_seconds)
    print(json.dumps(res))


def padding_loss(S, W, stream, steps, warmup, out_dtype, fast_math):
    """The padding target's workload pair (B = 16, H = 16, d = 128, Lmax = 4096, mean
    padding 0 % and 25 %; the valid lengths of pad_sweep_0 and pad_sweep_25), one step =
    sigattn_fwd + sigattn_bwd as in the headline line, effective TFLOPS over valid tokens
    and the loss from 0 % to 25 %. Timing only: the values are standard normals drawn on
    the GPU with torch's seeded generator (the kernels' work does not depend on them)."""
    import torch
    dev = torch.device("cuda:0")
    out = {}
    for name in ("pad_sweep_0", "pad_sweep_25"):
        w = W.WORKLOADS[name]
        sl = W.seqlens_of(w)
        g = torch.Generator(device=dev).manual_seed(w.seed)
        t = {k_: torch.randn((w.B, w.H, w.L, w.d), generator=g, device=dev).to(torch.bfloat16)
             for k_ in ("q", "k", "v", "do")}
        m = measure(S, W, w, t, None, sl, stream, steps, warmup, out_dtype, fast_math,
                    separate=False)
        out[name] = {"padding": float(1.0 - np.mean(sl) / w.L), "value": m["value"],
                     "ms_per_step": m["ms_per_step"], "fwd_tflops": m["fwd_tflops"],
                     "bwd_tflops": m["bwd_tflops"]}
        del t
        torch.cuda.empty_cache()
    a, b = out["pad_sweep_0"], out["pad_sweep_25"]
    out["loss_pct"] = {k_: 100.0 * (1.0 - b[k_] / a[k_])
                       for k_ in ("value", "fwd_tflops", "bwd_tflops")}
    out["target"] = "effective TFLOPS loss from 0 % to 25 % padding below 10 %"
    return out


def sweep(S, W, iters=250, warmup_ms=100.0, fast_math=False, causal=False):
    """The kernel sweep of the sigmoid-attention paper's section 4.1 ("Kernel
    Performance"): sequence length 512..16384 with the batch set so that B * L = 16384
    tokens, head dimension 64 (32 heads) and 128 (16 heads) of a 2048-wide model, 0 % and
    25 % padding; bidirectional. Per configuration the forward and the backward
    (sigattn_bwd: dQ and dK/dV kernels) are timed separately, each for `iters` iterations after about
    `warmup_ms` of warm-up, with a pair of HIP events per iteration on the launch stream;
    TFLOPS count valid tokens only. causal: the same grid with the causal mask and every
    sequence at full length (FLOPs over the n(n+1)/2 allowed pairs)."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []
    for d, H in ((64, 32), (128, 16)):
        for pad in ((0.0,) if causal else (0.0, 0.25)):
            for L in (512, 1024, 2048, 4096, 8192, 16384):
                B = 16384 // L
                w = W.Workload(f"sweep_L{L}_d{d}_p{int(pad * 100)}", "bf16", B, H, d, L,
                               ("mean_pad", pad), seed=1000 + L + d + int(pad * 100),
                               causal=causal)
                data = W.generate(w)
                t = {k: torch.from_numpy(data[k]).to(torch.bfloat16).to(dev)
                     for k in ("q", "k", "v", "do")}
                sl = data["seqlens"]
                kw = dict(out_dtype=torch.float32, fast_math=fast_math, causal=causal)
                o = torch.empty(t["q"].shape, dtype=torch.float32, device=dev)
                dq, dk, dv = torch.empty_like(o), torch.empty_like(o), torch.empty_like(o)

                def fwd():
                    S.fwd(t["q"], t["k"], t["v"], sl, out=o, **kw)

                def bwd():
                    S.bwd(t["q"], t["k"], t["v"], t["do"], sl, out=(dq, dk, dv), **kw)

                res = {"L": L, "B": B, "H": H, "d": d, "padding": pad,
                       "seqlens": [int(x) for x in sl]}
                for name, fn, flops in (("fwd", fwd, W.flops_forward(sl, H, d, causal)),
                                        ("bwd", bwd, W.flops_backward(sl, H, d, causal))):
                    t0 = time.perf_counter()
                    while time.perf_counter() - t0 < warmup_ms * 1e-3:
                        fn()
                        torch.cuda.synchronize()
                    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                           for _ in range(iters)]
                    hold_gpu(stream, iters)
                    for e0, e1 in evs:
                        e0.record(stream)
                        fn()
                        e1.record(stream)
                    torch.cuda.synchronize()
                    ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
                    tf = flops / (ms * 1e-3) / 1e12
                    half = 2.576 * float(np.std(tf, ddof=1)) / np.sqrt(len(tf))
                    res[name] = {"ms": float(ms.mean()), "tflops": float(tf.mean()),
                                 "ci99": half, "pct_peak": 100.0 * float(tf.mean()) / PEAK_BF16_TFLOPS}
                rows.append(res)
                print(f"[sweep] d={d} pad={pad} L={L} B={B}: fwd {res['fwd']['tflops']:.1f} "
                      f"bwd {res['bwd']['tflops']:.1f} TFLOPS", file=sys.stderr, flush=True)
    return {"sweep": "kernel sweep, B*L = 16384 tokens, "
                     + ("causal, full-length sequences" if causal else "bidirectional")
                     + ", bf16 inputs, float "
                     "outputs, " + ["hi+lo operands", "single bf16 operands",
                                    "f16 forward P V, hi+lo backward"][int(fast_math)],
            "iters": iters, "rows": rows}


def measure_packed(S, W, w, data, stream, steps, warmup, out_dtype, fast_math):
    """The workload's valid rows packed back to back ([rows, H, d], device cu_seqlens),
    one step = sigattn_fwd_varlen + sigattn_bwd_varlen; the same FLOP count as the padded
    layout. The two backward passes are also timed alone."""
    import torch
    dev = torch.device("cuda:0")
    sl = [int(x) for x in data["seqlens"]]

    def pack(x):   # [B, H, L, d] -> [sum n, H, d]
        return np.concatenate([x[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(sl)], axis=0)

    t = {k: torch.from_numpy(np.ascontiguousarray(pack(data[k]))).to(torch.bfloat16).to(dev)
         for k in ("q", "k", "v", "do")}
    gate = None
    if data["gate"] is not None:
        gate = torch.from_numpy(np.concatenate([data["gate"][b, :n] for b, n in enumerate(sl)])).to(dev)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(sl)]).astype(np.int32), device=dev)
    mx = max(sl)
    kw = dict(causal=w.causal, gate=gate, tau=w.tau, sink=w.sink, out_dtype=out_dtype,
              fast_math=fast_math)
    o = torch.empty(t["q"].shape, dtype=out_dtype, device=dev)
    dq, dk, dv = torch.empty_like(o), torch.empty_like(o), torch.empty_like(o)
    args = (t["q"], t["k"], t["v"], t["do"], cu, cu, mx, mx)
    calls = {"fwd": lambda: S.fwd_varlen(t["q"], t["k"], t["v"], cu, cu, mx, mx, out=o, **kw),
             "bwd": lambda: S.bwd_varlen(*args, out=(dq, dk, dv), **kw)}
    alone = {"bwd_dq": lambda: S.bwd_dq_varlen(*args, out=dq, **kw),
             "bwd_dkdv": lambda: S.bwd_dkdv_varlen(*args, out=(dk, dv), **kw)}
    for _ in range(warmup):
        for fn in list(calls.values()) + list(alone.values()):
            fn()
    torch.cuda.synchronize()
    ms_step, per_steps = time_steps(stream, steps, calls)
    per = {name: float(np.mean(times)) for name, times in per_steps.items()}
    for name, fn in alone.items():
        per[name] = float(np.mean(time_steps(stream, steps, {name: fn}, step_time=False)[1][name]))
    f_fwd = W.flops_forward(data["seqlens"], w.H, w.d, w.causal)
    f_bwd = W.flops_backward(data["seqlens"], w.H, w.d, w.causal)
    pairs = W.valid_pairs(data["seqlens"], w.causal) * w.H
    kernels = {}
    for name, ms in per.items():
        algo = PASS_FLOPS_PER_PAIR[name] * w.d * pairs
        kernels[name] = {"avg_ms": ms, "algorithmic_tflop": algo / 1e12,
                         "achieved_tflops": algo / (ms * 1e-3) / 1e12,
                         "frac_of_peak": algo / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    dom = max(("fwd", "bwd"), key=lambda k_: kernels[k_]["avg_ms"])
    bwd_ms = per["bwd"]
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    return {
        "metric": METRIC, "value": value, "unit": "TFLOPS", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "timing": TIMING,
        "config": {"workload": w.name, "layout": "packed rows, device cu_seqlens", "B": w.B,
                   "H": w.H, "d": w.d, "rows": int(sum(sl)), "seqlens": sl, "causal": w.causal,
                   "gated": w.gate is not None, "seed": w.seed,
                   "step": "sigattn_fwd_varlen + sigattn_bwd_varlen"},
        "fwd_tflops": f_fwd / (per["fwd"] * 1e-3) / 1e12,
        "bwd_tflops": f_bwd / (bwd_ms * 1e-3) / 1e12,
        "pct_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma",
                     "kernel": {"fwd": "fwd_kernel",
                                "bwd": "bwd_kernel" if w.d == 64 else "dkdv_kernel + dq_kernel"}[dom],
                     "achieved": kernels[dom]["achieved_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": kernels[dom]["frac_of_peak"], "traffic": None},
        "kernels": kernels,
    }


def measure(S, W, w, t, gate, sl, stream, steps, warmup, out_dtype, fast_math, separate=True):
    import torch
    kw = dict(causal=w.causal, gate=gate, tau=w.tau, sink=w.sink, out_dtype=out_dtype,
              fast_math=fast_math)
    o = torch.empty(t["q"].shape, dtype=out_dtype, device=t["q"].device)
    dq = torch.empty_like(o)
    dk = torch.empty_like(o)
    dv = torch.empty_like(o)

    calls = {"fwd": lambda: S.fwd(t["q"], t["k"], t["v"], sl, out=o, **kw),
             "bwd": lambda: S.bwd(t["q"], t["k"], t["v"], t["do"], sl, out=(dq, dk, dv), **kw)}
    for _ in range(warmup):
        for fn in calls.values():
            fn()
    ms_step, per = time_steps(stream, steps, calls)

    # each backward pass alone as well (outside the timed step): the two kernels that the
    # one-call backward runs in one launch
    sep = {"bwd_dq": lambda: S.bwd_dq(t["q"], t["k"], t["v"], t["do"], sl, out=dq, **kw),
           "bwd_dkdv": lambda: S.bwd_dkdv(t["q"], t["k"], t["v"], t["do"], sl, out=(dk, dv), **kw)}
    for name, fn in (sep.items() if separate else ()):
        for _ in range(max(2, warmup // 4)):
            fn()
        per[name] = time_steps(stream, steps, {name: fn}, step_time=False)[1][name]

    f_fwd = W.flops_forward(sl, w.H, w.d, w.causal)
    f_bwd = W.flops_backward(sl, w.H, w.d, w.causal)
    pairs = W.valid_pairs(sl, w.causal) * w.H
    fwd_ms = float(np.mean(per["fwd"]))
    bwd_ms = float(np.mean(per["bwd"]))
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    kernels = {}
    for name, times in per.items():
        ms = float(np.mean(times))
        algo = PASS_FLOPS_PER_PAIR[name] * w.d * pairs
        kernels[name] = {"avg_ms": ms, "algorithmic_tflop": algo / 1e12,
                         "achieved_tflops": algo / (ms * 1e-3) / 1e12,
                         "frac_of_peak": algo / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    dom = max(("fwd", "bwd"), key=lambda k_: kernels[k_]["avg_ms"])   # launches of the step
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic", "timing": TIMING,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "d": w.d, "Lmax": w.L,
                   "seqlens": [int(x) for x in sl], "causal": w.causal,
                   "gated": w.gate is not None, "seed": w.seed,
                   "step": "sigattn_fwd + sigattn_bwd"},
        "fwd_tflops": f_fwd / (fwd_ms * 1e-3) / 1e12,
        "bwd_tflops": f_bwd / (bwd_ms * 1e-3) / 1e12,
        "fwd_pct_peak": 100.0 * f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "bwd_pct_peak": 100.0 * f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "pct_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma",
                     "kernel": {"fwd": "fwd_kernel",
                                "bwd": "bwd_kernel" if w.d == 64 else "dkdv_kernel + dq_kernel"}[dom],
                     "achieved": kernels[dom]["achieved_tflops"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": kernels[dom]["frac_of_peak"],
                     "traffic": traffic_for(w.name, dom)},
        "kernels": kernels,
    }
    return res


if __name__ == "__main__":
    main()

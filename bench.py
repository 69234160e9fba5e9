"""Benchmark of the KDA forward prefill on one MI355X.

One step = one kda_prefill call over the whole packed batch (every kernel of
the path: K1 + K2, or K1 + pre_scan + merge + segment-K2), inputs resident in
HBM. Prints one JSON line: tokens/s, the roofline of the path's kernels
measured with HIP events on the launch stream, and the CPU oracle timed on the
host cores as a reported baseline.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload varlen8_h32]

After the warm-up steps, untimed steps run until the GPU has worked
--settle-ms milliseconds at a stable step time (the clocks take tens of
milliseconds of work to settle). The timed region is --steps steps back to
back; a second pass of as many steps brackets every launch with HIP events
for the per-kernel times of the roofline.

With --workload decode_n256_h32 a step is instead one kda_decode call: one
token for each of 256 sequences x 32 heads, the fp32 states advanced in place.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/sec (H=32, D=128, bf16) + % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
# Algorithmic work per token-head of the path (D = 128, chunk 16):
#   bytes: q 256 + k 256 + v 256 (bf16) + g 512 (fp32) + beta 4 + o 256 (bf16)
#   flops of the chunked WY form, per 16-token chunk: the Grams A_kk and A_qk,
#          W = T diag(beta)(K Gamma) and U~ = T diag(beta) V (16x16x128
#          each), W S0, Qt S0 and Kt^T U (16x128x128 each) and A_qk U
#          (16x16x128): 2 * (3 * 262144 + 5 * 32768) / 16 per token. The
#          kernels regroup U = U~ - W S0 as T'(V - X S0), which needs one
#          16x16x128 product fewer: 2 * (3 * 262144 + 4 * 32768) / 16.
BYTES_PER_TOKEN_HEAD = 1540
FLOPS_PER_TOKEN_HEAD = 118784           # the method's count (the MFMA roofline's numerator)
FLOPS_PER_TOKEN_HEAD_EXECUTED = 114688  # what the regrouped kernels issue
STATE_BYTES = 128 * 128 * 4

WORKLOAD_TEXT = {
    "varlen8_h32": "8 packed sequences, lengths uniform in [512, 4096] (seed 1002), H=32, D=128, "
                   "bf16 q/k/v, fp32 g=-softplus(N(0,1)) and beta=sigmoid(N(0,1)), fp32 initial "
                   "state N(0, 0.1), fp32 final state",
    "long65536_h8": "one 65536-token sequence, H=8, D=128, initial state N(0, 0.1)",
    "batch16x8192_h64": "16 sequences x 8192 tokens, H=64, D=128, g=-softplus(2 N(0,1)), zero "
                        "initial state",
}


DECODE_METRIC = "KDA decode tokens/sec (one token per sequence, H=32, D=128, fp32 state in place) + % of HBM roofline"
# Algorithmic bytes of one decode step per (sequence, head): the fp32 state
# read and written (2 x 65536), q, k, v (bf16, 3 x 256), g (fp32, 512),
# beta (4) and o (bf16, 256).
DECODE_BYTES_PER_SEQ_HEAD = 2 * STATE_BYTES + 3 * 256 + 512 + 4 + 256
DECODE_TEXT = {
    "decode_n256_h32": "decode step: 256 sequences x 32 heads, one token each, D=128, bf16 q/k/v, "
                       "fp32 g=-softplus(N(0,1)) and beta=sigmoid(N(0,1)), fp32 state N(0, 0.1) "
                       "updated in place",
}


def source_digest(files=("kda_device.hpp", "kda_kernels.hip", "kda_launch.h")):
    """Digest of the kernel sources with comments and blank lines removed, so
    that it changes with the code and not with its commentary."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "kda_chunked_delta_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines()]
        h.update("\n".join(l for l in lines if l.strip()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, digest, workload_name):
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, each scaled by its reading on a copy of known size), if the
    committed measurement was taken on the current kernel sources and on this
    workload."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    # one entry per launch sequence, or per (launch sequence, workload) when
    # it is measured on several workloads
    ent = data.get(f"{kernel}@{workload_name}") or data.get(kernel)
    if not ent or ent.get("source_digest") != digest or ent.get("workload") != workload_name:
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(d, max_seconds):
    """The fp64 C oracle (plain per-token recurrence, OpenMP) on a bounded
    sample: whole sequences, all heads, added in order until the estimated
    time reaches max_seconds."""
    from oracle import reference as ref
    cu = d["cu_seqlens_host"]
    H = d["H"]
    threads = ref.c_max_threads()
    # probe speed on the first 256 tokens of sequence 0 (all heads)
    n_probe = min(256, cu[1] - cu[0])
    sl = lambda x, a, b: x[a:b]
    probe = [sl(d[k], 0, n_probe) for k in ("q", "k", "v", "g", "beta")]
    t = time.time()
    ref.recurrent_c(*probe, [0, n_probe], None)
    rate = n_probe * H / max(time.time() - t, 1e-6)  # token-heads / s
    budget = max_seconds * rate
    nseq = 0
    while nseq < len(cu) - 1 and (cu[nseq + 1] - cu[0]) * H <= budget:
        nseq += 1
    nseq = max(nseq, 1)
    T = cu[nseq]
    args = [sl(d[k], 0, T) for k in ("q", "k", "v", "g", "beta")]
    s0 = d["initial_state"][:nseq] if d["initial_state"] is not None else None
    # repeat the sample until half the budget, but at least 10 s (within the
    # budget), is spent, so that a short sample is still timed over seconds
    target = min(max_seconds, max(10.0, 0.5 * max_seconds))
    reps, dt = 0, 0.0
    while reps == 0 or dt < target:
        t = time.time()
        ref.recurrent_c(*args, cu[:nseq + 1], s0)
        dt += time.time() - t
        reps += 1
    return {"value": reps * T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "first %d of %d sequences (%d tokens), all %d heads, run %d times; per-token fp64 "
                      "recurrence in C, OpenMP over (sequence, head, 32-column block); %.1f s"
                      % (nseq, len(cu) - 1, T, H, reps, dt)}


def cold_steps(step, tokens, n):
    """Per-step times with the caches cold: before each step a 512 MiB write
    (twice the 256 MiB Infinity Cache) evicts the inputs; HIP events bracket
    the step alone, after a synchronisation. The same one-step-at-a-time
    timing without the flush is reported beside it, so the difference is the
    caches' share, not the launch from an idle queue."""
    import torch
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda:0")

    def one_by_one(cold):
        times = []
        for i in range(n):
            if cold:
                flush.fill_(float(i))
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        times.sort()
        return times

    warm = one_by_one(False)
    cold = one_by_one(True)
    med, wmed = cold[len(cold) // 2], warm[len(warm) // 2]
    return {"steps": n, "flush_bytes": flush.numel() * 4, "ms_per_step_median": round(med, 5),
            "ms_per_step_min": round(cold[0], 5), "ms_per_step_max": round(cold[-1], 5),
            "value_median": round(tokens / (med * 1e-3), 1),
            "warm_one_by_one_ms_median": round(wmed, 5)}


def plan_kind(info):
    if info.get("warm_cp", 0):
        return "warm-start cp(segments of %d chunks, warm-up %d chunks)" % (info["warm_cp_seg_chunks"],
                                                                            info["split_warm_chunks"])
    if info["uses_cp"]:
        return "cp"
    if info.get("n_split_seqs", 0) > 0:
        return "split(%d sequences, warm-up %d chunks)" % (info["n_split_seqs"], info["split_warm_chunks"])
    return "serial"


def settle_clocks(step, stream, min_ms, max_ms):
    """Untimed steps until the GPU has worked at least min_ms and the step
    time has stopped falling (two batches in a row within 1%), or max_ms has
    passed. The shader clock needs tens of milliseconds of work to reach its
    steady level; without this a short run times the ramp."""
    import torch
    total, steps, prev, batch = 0.0, 0, None, 8
    while True:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(batch):
            step()
        b.record(stream)
        b.synchronize()
        ms = a.elapsed_time(b)
        total += ms
        steps += batch
        per = ms / batch
        stable = prev is not None and abs(per - prev) <= 0.01 * prev
        prev = per
        if (total >= min_ms and stable) or total >= max_ms:
            return {"ms": round(total, 1), "steps": steps, "last_ms_per_step": round(per, 5)}
        batch = max(4, min(4000, int(25.0 / max(per, 1e-3))))  # about 25 ms per batch


def timed_steps(step, stream, n):
    """n steps back to back with an event after each on the launch stream:
    (total ms / n, median of the per-step intervals)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n))
    return evs[0].elapsed_time(evs[n]) / n, per[len(per) // 2]


def host_cost(call_py, call_c, n=200):
    """Host microseconds per prefill call, while the GPU works through the
    queued calls: through the Python binding, and through the C ABI alone
    (the same ctypes call with prepared arguments, less the cost of a ctypes
    call into the library that does nothing)."""
    import ctypes
    import torch
    import kda_chunked_delta_amd as kda

    def per_call(f, reps):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            f()
        dt = time.perf_counter() - t
        torch.cuda.synchronize()
        return dt / reps * 1e6

    py = per_call(call_py, n)
    raw = per_call(call_c, n)
    noop = kda.lib().kda_version
    t = time.perf_counter()
    for _ in range(n):
        noop()
    ctypes_us = (time.perf_counter() - t) / n * 1e6
    return {"python_us": round(py, 2), "c_abi_us": round(max(raw - ctypes_us, 0.0), 2),
            "ctypes_call_us": round(ctypes_us, 2), "calls": n,
            "note": "host time per kda_prefill call with the plan given, measured over back-to-back calls "
                    "while the GPU works through them; c_abi_us is the ctypes call with prepared arguments "
                    "less a no-op ctypes call"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="after the warm-up steps, run untimed steps until the GPU has worked this many "
                         "milliseconds and the step time is stable, so that the timed steps run at steady "
                         "clocks whatever --warmup is (reported as clock_settle; 0: no settling)")
    ap.add_argument("--host-calls", type=int, default=200,
                    help="calls over which the host cost of one prefill call is measured (0: skip)")
    ap.add_argument("--workload", default="varlen8_h32", choices=sorted(WORKLOAD_TEXT) + sorted(DECODE_TEXT))
    ap.add_argument("--cp", default="auto", choices=["auto", "on", "off"])
    ap.add_argument("--cold-steps", type=int, default=50,
                    help="after the timed steps, time this many more one by one with the caches "
                         "flushed before each (reported as \"cold\"; 0: skip)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target duration of the CPU-oracle baseline sample (0 disables it)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run `steps` launches of a plain elementwise copy of "
                         "MIB MiB (fp32 negation: MIB MiB read, MIB MiB written); the reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    ap.add_argument("--g-scale", type=float, default=None,
                    help="multiply g by this factor after drawing it (0.05: weak decay, the case in which "
                         "the carried-in state is not forgotten within a segment)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: measures one GPU only; --gpus %d is not supported (the prefill shards by "
              "sequence or head with no communication, so N GPUs each run this on their share)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kda_chunked_delta_amd as kda
    from kda_inputs import workload

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                          "launches": max(1, args.steps)}), flush=True)
        return
    if args.workload in DECODE_TEXT:
        bench_decode(args, dev)
        return
    d = workload(args.workload, device=dev)
    if args.g_scale is not None:
        d["g"].mul_(args.g_scale)
    H, cu = d["H"], d["cu_seqlens_host"]
    Tt, N = cu[-1], len(cu) - 1
    mode = {"auto": "auto", "on": True, "off": False}[args.cp]
    plan = kda.plan(cu, H, mode, device=dev)
    info = plan.info()
    s0 = d["initial_state"]
    s_out = torch.empty(N, H, 128, 128, dtype=torch.float32, device=dev)
    o = torch.empty_like(d["q"])

    def step():
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                    cu_seqlens_host=cu, initial_state=s0, final_state=s_out, out=o, plan=plan)

    print("bench: workload %s Tt=%d H=%d plan=%s units=%d" % (args.workload, Tt, H,
          plan_kind(info), info["n_units"]), file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settle = settle_clocks(step, stream, args.settle_ms, max(3000.0, 4 * args.settle_ms)) if args.settle_ms > 0 \
        else None
    print("bench: clocks settled after %s" % settle, file=sys.stderr, flush=True)

    # the timed region: `steps` steps back to back, one event after each on
    # the launch stream
    ms_step, ms_median = timed_steps(step, stream, args.steps)
    # the roofline's kernel times: the same number of steps again, each launch
    # bracketed by HIP events on the launch stream (those events add a gap
    # before and after every launch, so this pass is not the headline)
    ctx = kda.context(dev)
    ctx.set_timing(True)
    ms_ev, ms_ev_median = timed_steps(step, stream, args.steps)
    per_kernel = ctx.timing()
    ctx.set_timing(False)
    print("bench: %.4f ms/step (median %.4f); with per-launch events %.4f ms/step, kernels %s" % (
        ms_step, ms_median, ms_ev, {k: round(v[0] / v[1], 4) for k, v in per_kernel.items()}),
        file=sys.stderr, flush=True)

    token_heads = Tt * H
    alg_bytes = token_heads * BYTES_PER_TOKEN_HEAD + N * H * STATE_BYTES * (2 if s0 is not None else 1)
    alg_flops = token_heads * FLOPS_PER_TOKEN_HEAD
    kern_ms = {k: v[0] / v[1] for k, v in per_kernel.items()}
    path_ms = sum(v[0] for v in per_kernel.values()) / args.steps  # all kernels of one step
    dominant = max(kern_ms, key=lambda k: per_kernel[k][0])
    names = "+".join(per_kernel.keys())
    achieved = alg_bytes / (path_ms * 1e-3) / 1e9
    digest = source_digest()
    wl_key = args.workload if args.g_scale is None else "%s@g%g" % (args.workload, args.g_scale)
    traffic = traffic_from_profiles(names, digest, wl_key)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "frac_of_step": round(alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "frac_of_median_step": round(alg_bytes / (ms_median * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "basis": "frac: algorithmic bytes over the summed HIP-event time of the step's kernels (the "
                         "dominant one and the rest), from a pass of the same steps with every launch "
                         "bracketed by events; frac_of_step: over the headline ms_per_step, launch gaps "
                         "included",
                "kernel": names, "dominant": dominant, "kernel_ms": {k: round(v, 4) for k, v in kern_ms.items()},
                "alg_bytes_per_step": alg_bytes, "source_digest": digest}
    mfma_frac = alg_flops / (path_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)

    def call_py():
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                    cu_seqlens_host=cu, initial_state=s0, final_state=s_out, out=o, plan=plan)

    import ctypes
    opts = kda.PrefillOpts(H, 0, 0)
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    c_args = (ctx.handle, plan.handle, ctypes.byref(opts), p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]),
              p(d["beta"]), p(d["cu_seqlens"]), 1.0, p(s0), p(s_out), p(o), ctypes.c_void_p(stream.cuda_stream))
    fn = kda.lib().kda_prefill_ex

    def call_c():
        if fn(*c_args) != 0:
            raise RuntimeError("kda_prefill_ex: " + kda.lib().kda_last_error().decode())

    line = {
        "metric": METRIC,
        "value": round(Tt / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_median": round(ms_median, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (args.workload, WORKLOAD_TEXT[args.workload]), "tokens": Tt,
                   "heads": H, "head_dim": 128, "sequences": N, "lengths": d["lengths"],
                   "plan": plan_kind(info), "cp_mode": args.cp},
        "clock_settle": settle,
        "kernel_timing_pass": {"ms_per_step": round(ms_ev, 5), "ms_per_step_median": round(ms_ev_median, 5),
                               "steps": args.steps},
        "roofline": roofline,
        "mfma_roofline": {"bound": "mfma", "achieved": round(alg_flops / (path_ms * 1e-3) / 1e12, 2),
                          "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(mfma_frac, 4),
                          "flops_per_token_head": FLOPS_PER_TOKEN_HEAD,
                          "flops_per_token_head_executed": FLOPS_PER_TOKEN_HEAD_EXECUTED},
    }
    if args.g_scale is not None:
        line["config"]["g_scale"] = args.g_scale
    if args.host_calls > 0:
        line["host_per_call"] = host_cost(call_py, call_c, args.host_calls)
        print("bench: host per call %s" % line["host_per_call"], file=sys.stderr, flush=True)
    if args.cold_steps > 0:
        line["cold"] = cold_steps(step, Tt, args.cold_steps)
        print("bench: cold %s" % line["cold"], file=sys.stderr, flush=True)
    if args.cpu_seconds > 0:
        print("bench: timing the CPU oracle (~%.0f s)" % args.cpu_seconds, file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def cpu_baseline_decode(d, max_seconds):
    """The fp64 oracle decode step (numpy, one BLAS thread) on a bounded
    sample: whole sequences, all heads, added until the estimated time
    reaches max_seconds."""
    from threadpoolctl import threadpool_limits
    from oracle import reference as ref
    N, H = d["N"], d["H"]
    cpu = {k: d[k].cpu() for k in ("q", "k", "v", "g", "beta", "state")}
    with threadpool_limits(limits=1):
        t = time.time()
        ref.decode_step(*(cpu[k][:1] for k in ("q", "k", "v", "g", "beta", "state")))
        per_seq = max(time.time() - t, 1e-6)
        n = max(1, min(N, int(max_seconds / per_seq)))
        t = time.time()
        ref.decode_step(*(cpu[k][:n] for k in ("q", "k", "v", "g", "beta", "state")))
        dt = time.time() - t
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "first %d of %d sequences, all %d heads, one decode step; fp64 matrix-form update "
                      "in numpy with one BLAS thread; %.1f s" % (n, N, H, dt)}


def bench_decode(args, dev):
    import torch
    import kda_chunked_delta_amd as kda
    from kda_inputs import decode_workload

    d = decode_workload(args.workload, device=dev)
    N, H = d["N"], d["H"]
    state = d["state"].clone()
    o = torch.empty_like(d["q"])

    def step():
        kda.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=o)

    print("bench: workload %s N=%d H=%d" % (args.workload, N, H), file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settle = settle_clocks(step, stream, args.settle_ms, max(3000.0, 4 * args.settle_ms)) if args.settle_ms > 0 \
        else None
    ms_step, ms_median = timed_steps(step, stream, args.steps)
    ctx = kda.context(dev)
    ctx.set_timing(True)
    timed_steps(step, stream, args.steps)
    per_kernel = ctx.timing()
    ctx.set_timing(False)
    kern_ms = per_kernel["decode"][0] / per_kernel["decode"][1]
    print("bench: %.4f ms/step; decode kernel %.4f ms" % (ms_step, kern_ms), file=sys.stderr, flush=True)
    alg_bytes = N * H * DECODE_BYTES_PER_SEQ_HEAD
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    digest = source_digest(("kda_decode.hip", "kda_decode_launch.h"))
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profiles("decode", digest, args.workload),
                "kernel": "decode", "dominant": "decode", "kernel_ms": {"decode": round(kern_ms, 4)},
                "alg_bytes_per_step": alg_bytes, "source_digest": digest}
    line = {
        "metric": DECODE_METRIC,
        "value": round(N / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_median": round(ms_median, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (args.workload, DECODE_TEXT[args.workload]), "sequences": N,
                   "heads": H, "head_dim": 128},
        "clock_settle": settle,
        "roofline": roofline,
    }
    if args.cpu_seconds > 0:
        print("bench: timing the CPU oracle (~%.0f s)" % min(args.cpu_seconds, 10.0), file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_decode(d, min(args.cpu_seconds, 10.0))
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

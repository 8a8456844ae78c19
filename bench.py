"""Benchmark of one paged-decode step on one MI355X.

A step is the whole hot path on one batch: the split-KV plan (host, copied
into the fixed plan buffer), dynamic e4m3 Q quantization, the paged decode
and the LSE merge (when the plan splits), enqueued back to back on one
stream.  Inputs are seeded synthetic tensors already resident in HBM.  The
Infinity Cache is flushed (a 1 GiB write) before every step, outside that
step's event pair, so KV bytes come from HBM.

Prints one JSON line.  ``value`` is the achieved KV-read bandwidth of the
step (KV bytes / step time) with the step replayed as one hipGraph (device
planner + quantize + decode + merge); the eager step with the host planner
is reported in ``detail``.  The decode kernel's own bandwidth against the
8 TB/s HBM peak is the ``roofline`` object.  ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg2] [--extra 32k,cfg3,...]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# HBM traffic of the decode kernel from rocprofv3 --pmc (FETCH_SIZE and
# WRITE_SIZE per dispatch, KiB), scaled by the same counters on a plain copy
# kernel of known size.  Filled in from the committed profile summaries when
# they describe the kernel as it is now; None otherwise.
TRAFFIC = {}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="cfg2")
    ap.add_argument("--extra", default="32k", help="comma list of extra workloads reported under 'extra' ('' = none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--variant", type=int, default=0,
                    help="decode kernel: 0 automatic, 1 generic, 2 VALU-PV streaming (A/B runs)")
    ap.add_argument("--no-nt", action="store_true", help="plain (not non-temporal) KV loads (A/B runs)")
    ap.add_argument("--wgs-per-cu", type=int, default=0, help="planner workgroups per CU (0 = library default)")
    ap.add_argument("--stream-read", action="store_true", help="also time a plain streaming read of the KV pool")
    return ap.parse_args()


def measure(key, steps, warmup, flush_buf, wgs_per_cu=0, stream_read=False):
    import torch
    import synth
    from paged_fp8_decode_amd.runner import DecodeStep, new_output

    t0 = time.time()
    wl = synth.build(synth.spec_for(key), "cuda")
    torch.cuda.synchronize()
    log(f"[bench] {key}: built {wl.spec.name} in {time.time() - t0:.1f}s, kv_bytes={wl.kv_bytes()}")
    step = DecodeStep.for_workload(wl, wgs_per_cu=wgs_per_cu)
    out, lse = new_output(wl)
    stream = torch.cuda.current_stream()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [(E(), E(), E(), E(), E()) for _ in range(steps)]

    def one(e=None):
        if e:
            e[0].record(stream)
        info = step.plan_workload(wl, stream=stream)
        if e:
            e[1].record(stream)
        step.run_workload(wl, out, lse, info=info, stream=stream, events=(e[2], e[3]) if e else None)
        if e:
            e[4].record(stream)
        return info

    for _ in range(warmup):
        flush_buf.add_(1)
        one()
    torch.cuda.synchronize()
    t_wall = time.time()
    for k in range(steps):
        flush_buf.add_(1)  # 1 GiB read + write: evicts the 256 MB Infinity Cache
        one(ev[k])
    torch.cuda.synchronize()
    t_wall = time.time() - t_wall
    info = step.info

    # the same step as one hipGraph: device-side plan + quantize + decode + merge
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step.plan_workload_device(wl, stream=side)
        step.run_workload(wl, out, lse, stream=side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gs = torch.cuda.current_stream()
        ginfo = step.plan_workload_device(wl, stream=gs)
        step.run_workload(wl, out, lse, info=ginfo, stream=gs)
    torch.cuda.synchronize()
    gev = [(E(), E()) for _ in range(steps)]
    for _ in range(warmup):
        flush_buf.add_(1)
        graph.replay()
    for k in range(steps):
        flush_buf.add_(1)
        gev[k][0].record(stream)
        graph.replay()
        gev[k][1].record(stream)
    torch.cuda.synchronize()
    graph_ms = np.array([a.elapsed_time(b) for a, b in gev])
    del graph
    step_ms = np.array([e[0].elapsed_time(e[4]) for e in ev])
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    plan_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    kvb = wl.kv_bytes()
    res = dict(
        workload=wl.spec.name, kv_bytes=kvb, steps=steps,
        us_per_step_median=float(np.median(step_ms) * 1e3), us_per_step_mean=float(step_ms.mean() * 1e3),
        us_per_step_p10=float(np.percentile(step_ms, 10) * 1e3),
        us_per_step_p90=float(np.percentile(step_ms, 90) * 1e3),
        decode_us_mean=float(dec_ms.mean() * 1e3), decode_us_median=float(np.median(dec_ms) * 1e3),
        plan_us_median=float(np.median(plan_ms) * 1e3),
        graph_us_per_step_median=float(np.median(graph_ms) * 1e3),
        graph_us_per_step_mean=float(graph_ms.mean() * 1e3),
        graph_step_kv_gbs=kvb / (graph_ms.mean() * 1e-3) / 1e9,
        step_kv_gbs=kvb / (step_ms.mean() * 1e-3) / 1e9,
        decode_kv_gbs=kvb / (dec_ms.mean() * 1e-3) / 1e9,
        plan=dict(num_work=info.num_work, slots=info.slots, chunk_tiles=info.chunk_tiles,
                  with_reduction=info.with_reduction),
        timed_wall_s=t_wall,
    )
    res["decode_frac_of_hbm_peak"] = res["decode_kv_gbs"] / HBM_PEAK_GBS
    if stream_read:
        # plain non-temporal streaming read of as many bytes as the KV the step reads
        import paged_fp8_decode_amd as mjlib
        nbytes = min(kvb, wl.k_pool.numel()) // 16 * 16
        src = wl.k_pool.view(-1)[:nbytes]
        chk = torch.empty(4096, dtype=torch.int32, device="cuda")
        ms = []
        for k in range(10):
            flush_buf.add_(1)
            e0, e1 = E(), E()
            e0.record(stream)
            mjlib.mj_debug_stream_read(src, chk, 2048, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        res["stream_read_gbs"] = nbytes / (np.median(ms[2:]) * 1e-3) / 1e9
        log(f"[bench] {key}: plain streaming read of {nbytes} B: {res['stream_read_gbs']:.0f} GB/s")
    log(f"[bench] {key}: step {res['us_per_step_median']:.1f} us eager / {res['graph_us_per_step_median']:.1f} us graph "
        f"(median), decode {res['decode_us_mean']:.1f} us, "
        f"decode KV {res['decode_kv_gbs']:.0f} GB/s ({100 * res['decode_frac_of_hbm_peak']:.1f}% of 8 TB/s)")
    del wl
    torch.cuda.empty_cache()
    return res


def cpu_baseline(key, budget_s):
    """The oracle as it stands, single-threaded BLAS, on whole (sequence, KV
    head) pairs of the same workload until ~budget_s seconds of CPU work."""
    import torch
    import synth
    from oracle.attention import decode_step
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None

    spec = synth.spec_for(key)
    wl = synth.build(spec, "cuda")
    s = wl.spec
    order = [(i, g) for i in range(s.b) for g in range(s.h_k)]
    done, nbytes, t_used = 0, 0, 0.0
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        for i in np.random.default_rng(0).permutation(s.b).tolist():
            h = wl.host([i])
            for g in range(s.h_k):
                t0 = time.perf_counter()
                decode_step(h, q_len=s.q_len, h_q=s.h_q, h_k=s.h_k, d=s.d, page_size=s.page_size,
                            kv_format=s.kv_format, causal=s.causal, pairs=[(0, g)])
                t_used += time.perf_counter() - t0
                done += 1
                nbytes += wl.seq_lens[i] * 2 * s.row_bytes
                if t_used >= budget_s:
                    break
            if t_used >= budget_s:
                break
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    del wl
    torch.cuda.empty_cache()
    return dict(value=nbytes / t_used / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample=f"{done} of {len(order)} (sequence, KV head) pairs of {spec.name} "
                       f"(each a full Q quantization + gather + fp64 attention), {t_used:.1f} s of CPU time, "
                       f"single-threaded NumPy/BLAS",
                seconds_per_step_extrapolated=t_used * len(order) / done)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import paged_fp8_decode_amd

    paged_fp8_decode_amd.mj_debug_set_decode_variant(args.variant, 0 if args.no_nt else 1)

    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    main_res = measure(args.workload, args.steps, args.warmup, flush_buf, args.wgs_per_cu, args.stream_read)
    extra = {}
    for k in [x for x in args.extra.split(",") if x]:
        extra[k] = measure(k, max(10, args.steps // 2), max(3, args.warmup // 2), flush_buf, args.wgs_per_cu,
                           args.stream_read)
    cpu = None if args.no_cpu else cpu_baseline(args.workload, args.cpu_seconds)
    kvb = main_res["kv_bytes"]
    dec_s = main_res["decode_us_mean"] * 1e-6
    roof = dict(bound="hbm", achieved=round(kvb / dec_s / 1e9, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(kvb / dec_s / 1e9 / HBM_PEAK_GBS, 4), traffic=TRAFFIC.get(args.workload),
                kernel="mj_paged_decode", algorithmic_bytes_per_launch=kvb)
    line = dict(
        metric="paged decode us/step and achieved KV-read HBM GB/s (% of MI355X peak)",
        value=round(main_res["graph_step_kv_gbs"], 1),
        unit="GB/s",
        n_gpus=1,
        steps=args.steps,
        warmup=args.warmup,
        ms_per_step=round(main_res["graph_us_per_step_mean"] / 1e3, 5),
        us_per_step_median=round(main_res["graph_us_per_step_median"], 2),
        higher_is_better=True,
        scaling="weak",
        vs_baseline=None,
        dtype="e4m3" if "e2m3" not in main_res["workload"] else "e2m3",
        data="synthetic",
        config=dict(workload=main_res["workload"], kv_bytes=kvb, plan=main_res["plan"], kernel_variant=args.variant,
                    nontemporal=not args.no_nt),
        roofline=roof,
        cpu_baseline=cpu,
        detail=main_res,
        extra=extra,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

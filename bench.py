"""Benchmark of one paged-decode step on one MI355X.

A step is the whole hot path on one batch: the split-KV plan, dynamic e4m3
Q quantization, the paged decode and the LSE merge of split partials.  The
timed step is a hipGraph of ``mj_decode_step`` planning from the device
lengths itself: the decode kernel (each workgroup derives its plan item and
quantizes its Q rows) and, when the plan splits, the merge kernel.
Inputs are seeded synthetic tensors already resident in HBM.  Before every
step, outside that step's event pair, a 1 GiB read evicts the 256 MB
Infinity Cache, so KV bytes come from HBM.  (A 1 GiB write would evict it
too but leave it full of dirty lines whose write-back then competes with the
step's loads -- a state no serving step starts from; the graph step after
such a write is reported as well, ``graph_us_per_step_median_after_write``.)

The headline workload is 64 sequences of 32768 tokens each (32/8 heads,
token-major pages of 64, e4m3 KV); every other workload is measured the
same way under ``extra`` and summarised under ``configs``.  Before any
timing, one replay of each captured graph must give the eager step's output
(host planner, same kernels) bit for bit, or the run stops.

Prints one JSON line.  ``value`` is the achieved KV-read bandwidth of the
step (KV bytes / mean graph step time); ``detail`` also has the eager step
(host planner + fused step) and the eager three-call step (quantize, decode,
merge as separate launches).  The ``roofline`` object is the decode
kernel's own bandwidth against the 8 TB/s HBM peak: one event pair around
back-to-back steps that rotate over copies of the KV pools (no launch reads
KV the Infinity Cache still holds), minus one event pair around as many
back-to-back launches of the merge kernel alone, per launch.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload.  ``bf16_q`` measures the same step in the bf16-Q mode (Q used as
given, no quantization; the KV codes converted to bf16 in the kernel) on the
workloads ``--bf16q`` names.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 32k] [--extra cfg2,cfg3,...]
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
# kernel selection of every measured step (mj_config fields; --variant,
# --cache-policy, --step-merge): 0 = the library's choice
KSEL = dict(decode_kernel=0, kv_cache_policy=0, step_merge=0)
ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# HBM traffic of the decode kernel per launch from rocprofv3 --pmc
# (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by what the same counters
# read for a 256 MiB copy: fetch x 1.99980, write x 1.000), as recorded in
# profiles/decode_mfma_kernel_hbm_traffic.md.  Reported only while the
# kernel sources hash to the value the counters were taken with.
TRAFFIC_SOURCES = ("mj_decode_mfma.hip", "mj_merge.h", "mj_device.h", "mj_internal.h")
TRAFFIC = {
    "sources_sha256_16": "00a425ce9c4ef621",
    "32k": dict(fetch_bytes=4298008181, write_bytes=4325676),
    "cfg2": dict(fetch_bytes=269040771, write_bytes=266786),
    "cfg3": dict(fetch_bytes=1284662197, write_bytes=4182779),
    "cfg4c": dict(fetch_bytes=270878984, write_bytes=4259977),
    "cfg5": dict(fetch_bytes=806196733, write_bytes=540681),
    "cfg5_e2m1": dict(fetch_bytes=538387600, write_bytes=1081363),
    "cfg5_nvfp4": dict(fetch_bytes=604680679, write_bytes=1081362),
    "cfg3_e2m3": dict(fetch_bytes=861220086, write_bytes=4011291),
    "cfg3_e2m1": dict(fetch_bytes=653061632, write_bytes=4102751),
    "cfg3_nvfp4": dict(fetch_bytes=708577277, write_bytes=4094649),
}


def kernel_sources_hash():
    """sha256[:16] of the decode kernel's sources with // comments and blank
    lines removed (a comment edit does not change the kernel)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "paged_fp8_decode_amd", "csrc", f)) as fh:
            for line in fh:
                line = re.sub(r"//.*", "", line).strip()
                if line:
                    h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_for(key):
    if kernel_sources_hash() != TRAFFIC["sources_sha256_16"] or key not in TRAFFIC:
        return None
    t = TRAFFIC[key]
    return t["fetch_bytes"] + t["write_bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="32k",
                    help="the headline workload: 64 sequences of 32768 tokens, token-major pages of 64, e4m3 KV")
    ap.add_argument("--extra", default="cfg1,cfg2,cfg3,cfg4c,cfg4n,cfg5,32k_b16,cfg5_e3m2,cfg5_e2m1,cfg5_nvfp4,cfg3_e2m3,cfg3_e2m1,cfg3_nvfp4",
                    help="comma list of extra workloads reported under 'extra' ('' = none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--bf16q", default="cfg2,32k",
                    help="comma-separated workloads also measured in the bf16-Q mode ('' = none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--variant", type=int, default=0,
                    help="mj_config.decode_kernel: 0 automatic, 1 generic, 10..17 matrix-core tuning (A/B runs)")
    ap.add_argument("--cache-policy", type=int, default=0,
                    help="mj_config.kv_cache_policy: 0 the library's choice, 1..4 (A/B runs)")
    ap.add_argument("--wgs-per-cu", type=int, default=0, help="planner workgroups per CU (0 = library default)")
    ap.add_argument("--no-stream-read", action="store_true",
                    help="skip the plain streaming read of the main workload's KV pool (HBM context figure)")
    ap.add_argument("--step-merge", type=int, default=0,
                    help="mj_config.step_merge: 0 automatic, 1 in the decode kernel, 2 separate launch (A/B runs)")
    ap.add_argument("--no-write", action="store_true", help="skip the KV-cache write measurement")
    ap.add_argument("--cp", default="cfg3:8",
                    help="context-parallel share measured as WORKLOAD:G (one GPU's slice of each context, "
                         "and the combine of G slices); '' = skip")
    ap.add_argument("--draft", type=int, default=4,
                    help="draft steps of the multi-step draft loop (0 = skip)")
    ap.add_argument("--draft-workload", default="cfg2", help="workload of the draft loop")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run the HBM-counter calibration kernels (256 MiB streaming read, 256 MiB copy) and exit")
    return ap.parse_args()


def calibrate():
    """Kernels of known traffic for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE:
    the library's plain streaming read of 256 MiB (reads 256 MiB, writes one
    word per workgroup) and a torch copy of 256 MiB (reads and writes 256 MiB
    each)."""
    import torch
    import paged_fp8_decode_amd as mjlib
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    chk = torch.empty(4096, dtype=torch.int32, device="cuda")
    for _ in range(3):
        mjlib.mj_debug_stream_read(src, chk, 2048)
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(calibration=True, stream_read_bytes=n, copy_bytes=n)), flush=True)


class Flusher:
    """Evicts the Infinity Cache between steps: reads 1 GiB (``__call__``), or
    writes it (``dirty``) for the secondary after-write figure."""

    def __init__(self):
        import torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        self.acc = torch.zeros((), dtype=torch.float32, device="cuda")

    def __call__(self):
        import torch
        torch.sum(self.buf, 0, out=self.acc)

    def dirty(self):
        self.buf.add_(1)


def measure(key, steps, warmup, flush, wgs_per_cu=0, stream_read=False, q_mode="fp8"):
    import torch
    import synth
    from paged_fp8_decode_amd.runner import DecodeStep, new_output

    t0 = time.time()
    wl = synth.build(synth.spec_for(key), "cuda")
    torch.cuda.synchronize()
    log(f"[bench] {key}: built {wl.spec.name} in {time.time() - t0:.1f}s, kv_bytes={wl.kv_bytes()}")
    step = DecodeStep.for_workload(wl, wgs_per_cu=wgs_per_cu, q_mode=q_mode, **KSEL)
    out, lse = new_output(wl)
    stream = torch.cuda.current_stream()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def eager(n, fused, with_events):
        ev = [(E(), E(), E(), E()) for _ in range(n)] if with_events else None
        for k in range(n):
            flush()
            e = ev[k] if ev else None
            if e:
                e[0].record(stream)
            info = step.plan_workload(wl, stream=stream)
            step.run_workload(wl, out, lse, info=info, stream=stream, events=(e[1], e[2]) if e else None,
                              fused=fused)
            if e:
                e[3].record(stream)
        torch.cuda.synchronize()
        return ev

    # eager steps: host plan (async copy) + the fused step (one kernel)
    eager(warmup, True, False)
    t_wall = time.time()
    ev = eager(steps, True, True)
    t_wall = time.time() - t_wall
    info = step.info
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in ev])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    # the same step as the pages' three calls (quantize, decode, merge), for comparison
    eager(max(3, warmup // 2), False, False)
    ev3 = eager(max(5, steps // 2), False, True)
    step3_ms = np.array([e[0].elapsed_time(e[3]) for e in ev3])
    dec3_ms = np.array([e[1].elapsed_time(e[2]) for e in ev3])

    # the step as one hipGraph of mj_decode_step planning from the device
    # lengths itself; for comparison, a graph of the device planner kernel
    # followed by the step on its plan
    def capture(planner_kernel):
        def body(st):
            if planner_kernel:
                gi = step.plan_workload_device(wl, stream=st)
                step.run_workload(wl, out, lse, info=gi, stream=st, fused=True)
            else:
                gi = step.plan_workload_shape(wl)
                step.run_workload(wl, out, lse, info=gi, stream=st, fused=True, plan_on_device=True)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            body(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            body(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return gr

    def time_graph(gr, n, evict=flush):
        gev = [(E(), E()) for _ in range(n)]
        for _ in range(warmup):
            evict()
            gr.replay()
        for k in range(n):
            evict()
            gev[k][0].record(stream)
            gr.replay()
            gev[k][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in gev])

    # the timed graph's result, before any timing: bit for bit the eager
    # step on the host planner's plan (same kernels, same plan)
    graph = capture(False)
    graph_pk = capture(True)
    ref_out, ref_lse = torch.empty_like(out), torch.empty_like(lse)
    step.plan_workload(wl, stream=stream)
    step.run_workload(wl, ref_out, ref_lse, info=step.info, stream=stream, fused=True)
    torch.cuda.synchronize()
    for gr_chk in (graph, graph_pk):
        out.fill_(float("nan"))
        gr_chk.replay()
        torch.cuda.synchronize()
        if not (torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                            ref_out.view(torch.int16) if out.dtype == torch.bfloat16 else ref_out)
                and torch.equal(lse, ref_lse)):
            raise RuntimeError(f"{key}: the graph step's output differs from the eager host-plan step")
    del ref_out, ref_lse
    # the two graphs timed in alternating chunks, so that neither gains or
    # loses from its place in the run
    chunks = 4
    parts, parts_pk = [], []
    for i in range(chunks):
        parts.append(time_graph(graph, max(2, steps // chunks)))
        parts_pk.append(time_graph(graph_pk, max(2, steps // (2 * chunks))))
    graph_ms, graph_pk_ms = np.concatenate(parts), np.concatenate(parts_pk)
    graph_dirty_ms = time_graph(graph, max(5, steps // 2), flush.dirty)
    del graph, graph_pk

    # decode kernel duration for the roofline: steps (decode + merge
    # launch) back to back, rotating over copies of the KV pools so that no
    # launch finds the previous one's KV in the 256 MB Infinity Cache (>= 1 GiB
    # of distinct KV between reuses), one event pair over all of them; minus
    # the same number of merge launches alone, one event pair over those
    kvb = wl.kv_bytes()
    n_copies = max(1, -(-(1 << 30) // kvb))
    # (nvfp4: the block-scale pools rotate with the codes)
    srcs = (wl.k_pool, wl.v_pool, wl.k_bs_pool, wl.v_bs_pool)
    pools = [srcs] + [tuple(None if t is None else t.clone() for t in srcs) for _ in range(n_copies - 1)]
    reps = max(8, 2 * n_copies, steps)
    ks, vs = wl.kv_strides()
    bss = wl.bs_strides() if wl.k_bs_pool is not None else (None, None)

    # the same step with the merge as a launch of its own (step_merge 2), so
    # that the merge launches can be timed alone and subtracted
    step2 = DecodeStep.for_workload(wl, wgs_per_cu=wgs_per_cu, q_mode=q_mode, **dict(KSEL, step_merge=2))

    def launch(i):
        kp, vp, kb, vb = pools[i % len(pools)]
        step2.run(k_block_scale=kb, v_block_scale=vb, k_bs_strides=bss[0], v_bs_strides=bss[1],
                 q=wl.q, k_cache=kp, v_cache=vp, k_strides=ks, v_strides=vs, num_pages=wl.num_pages,
                 block_table=wl.block_table, seq_lens=wl.seq_lens_dev, k_descale=wl.k_descale,
                 v_descale=wl.v_descale, descale_kind=wl.descale_kind, softmax_scale=wl.softmax_scale, out=out,
                 lse=lse, q_mul=wl.q_mul, o_mul=wl.o_mul, causal=wl.spec.causal, info=info, stream=stream,
                 fused=True)

    info = step2.plan_workload(wl, stream=stream)
    torch.cuda.synchronize()
    for i in range(len(pools)):
        launch(i)
    torch.cuda.synchronize()
    # three series of each, medians: one stalled series (seen under the
    # profiler: a merge series at 5x its usual time) moves nothing
    step_series, merge_series = [], []
    for _ in range(3):
        k0, k1 = E(), E()
        k0.record(stream)
        for i in range(reps):
            launch(i)
        k1.record(stream)
        if info.with_reduction:
            m0, m1 = E(), E()
            m0.record(stream)
            for i in range(reps):
                step2.merge(out, lse, info, stream)
            m1.record(stream)
        torch.cuda.synchronize()
        step_series.append(k0.elapsed_time(k1) * 1e3 / reps)
        merge_series.append(m0.elapsed_time(m1) * 1e3 / reps if info.with_reduction else 0.0)
    merge_us = float(np.median(merge_series))
    step_us_b2b = float(np.median(step_series))
    kernel_us = step_us_b2b - merge_us
    del pools

    res = dict(
        workload=wl.spec.name, kv_format=wl.spec.kv_format, q_mode=q_mode, kv_bytes=kvb, steps=steps,
        us_per_step_median=float(np.median(step_ms) * 1e3), us_per_step_mean=float(step_ms.mean() * 1e3),
        us_per_step_p10=float(np.percentile(step_ms, 10) * 1e3),
        us_per_step_p90=float(np.percentile(step_ms, 90) * 1e3),
        step_decode_us_mean=float(dec_ms.mean() * 1e3), step_decode_us_median=float(np.median(dec_ms) * 1e3),
        three_call_us_per_step_median=float(np.median(step3_ms) * 1e3),
        three_call_decode_us_median=float(np.median(dec3_ms) * 1e3),
        graph_us_per_step_median=float(np.median(graph_ms) * 1e3),
        graph_us_per_step_mean=float(graph_ms.mean() * 1e3),
        graph_us_per_step_p10=float(np.percentile(graph_ms, 10) * 1e3),
        graph_us_per_step_p90=float(np.percentile(graph_ms, 90) * 1e3),
        graph_step_kv_gbs=kvb / (graph_ms.mean() * 1e-3) / 1e9,
        graph_with_planner_kernel_us_per_step_median=float(np.median(graph_pk_ms) * 1e3),
        graph_us_per_step_median_after_write=float(np.median(graph_dirty_ms) * 1e3),
        step_kv_gbs=kvb / (step_ms.mean() * 1e-3) / 1e9,
        kernel_us_back_to_back=kernel_us, step_us_back_to_back=step_us_b2b, merge_us_back_to_back=merge_us,
        back_to_back_series_us=dict(step=[round(x, 2) for x in step_series], merge=[round(x, 2) for x in merge_series]),
        kernel_launches=reps, kv_pool_copies=n_copies,
        kernel_kv_gbs=kvb / (kernel_us * 1e-6) / 1e9,
        plan=dict(num_work=info.num_work, slots=info.slots, chunk_tiles=info.chunk_tiles,
                  min_chunk_tiles=info.min_chunk_tiles, wgs_per_cu=info.wgs_per_cu,
                  with_reduction=info.with_reduction),
        graph_step_equals_host_plan_step=True,
        timed_wall_s=t_wall,
    )
    res["kernel_frac_of_hbm_peak"] = res["kernel_kv_gbs"] / HBM_PEAK_GBS
    if stream_read:
        # plain non-temporal streaming read of as many bytes as the KV the step reads
        import paged_fp8_decode_amd as mjlib
        nbytes = min(kvb, wl.k_pool.numel()) // 16 * 16
        src = wl.k_pool.view(-1)[:nbytes]
        chk = torch.empty(4096, dtype=torch.int32, device="cuda")
        ms = []
        for k in range(10):
            flush()
            e0, e1 = E(), E()
            e0.record(stream)
            mjlib.mj_debug_stream_read(src, chk, 2048, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        res["stream_read_gbs"] = nbytes / (np.median(ms[2:]) * 1e-3) / 1e9
        log(f"[bench] {key}: plain streaming read of {nbytes} B: {res['stream_read_gbs']:.0f} GB/s")
    log(f"[bench] {key} ({q_mode} Q): step {res['graph_us_per_step_median']:.1f} us graph "
        f"({res['graph_with_planner_kernel_us_per_step_median']:.1f} with the planner kernel) / "
        f"{res['us_per_step_median']:.1f} us "
        f"eager / {res['three_call_us_per_step_median']:.1f} us three calls (median); decode kernel "
        f"{kernel_us:.1f} us = {res['kernel_kv_gbs']:.0f} GB/s KV ({100 * res['kernel_frac_of_hbm_peak']:.1f}% "
        f"of 8 TB/s); in-step decode {res['step_decode_us_mean']:.1f} us fused / "
        f"{res['three_call_decode_us_median']:.1f} us unfused; graph step after a 1 GiB write "
        f"{res['graph_us_per_step_median_after_write']:.1f} us; back-to-back step {step_us_b2b:.1f} us, "
        f"merge alone {merge_us:.1f} us")
    del wl
    torch.cuda.empty_cache()
    return res


def measure_launch_floor(steps, warmup, flush):
    """What launching costs by itself, timed like the steps (events around
    the launch after the same Infinity Cache eviction): a hipGraph holding
    one trivial kernel (torch's add on one element), and that kernel
    launched alone.  A graph step can be no faster than the first."""
    import torch
    stream = torch.cuda.current_stream()
    x = torch.zeros(1, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        x.add_(1)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        x.add_(1)
    torch.cuda.synchronize()

    def timed(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for _ in range(warmup):
            flush()
            fn()
        for a, b in ev:
            flush()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]) * 1e3)

    res = dict(one_kernel_graph_us_median=round(timed(gr.replay), 2),
               one_kernel_eager_us_median=round(timed(lambda: x.add_(1)), 2))
    log(f"[bench] launch floor after eviction: graph of one trivial kernel {res['one_kernel_graph_us_median']} us, "
        f"the kernel launched alone {res['one_kernel_eager_us_median']} us")
    del gr
    return res


def measure_write(kv_format, n_tokens, reps, flush, h_k=8, page_size=64):
    """mj_write_kv of n_tokens new rows (bf16 K and V, h_k heads) into a paged
    cache at scattered slots: time per call (one event pair around reps
    back-to-back calls, cache flushed first) and algorithmic bytes (bf16 in,
    codes out, 8-byte slots) against the HBM peak."""
    import torch
    import paged_fp8_decode_amd as mjlib
    row = {"e4m3": 128, "e2m3": 96, "e3m2": 96, "e2m1": 64, "nvfp4": 64}[kv_format]
    srow = 8 if kv_format == "nvfp4" else 0  # nvfp4 block-scale bytes per row
    pages = max(16, -(-2 * n_tokens // page_size))
    g = torch.Generator(device="cuda").manual_seed(77)
    key = torch.randn(n_tokens, h_k, 128, generator=g, device="cuda").to(torch.bfloat16)
    value = torch.randn(n_tokens, h_k, 128, generator=g, device="cuda").to(torch.bfloat16)
    slots = torch.randperm(pages * page_size, generator=g, device="cuda")[:n_tokens].to(torch.int64)
    k_pool = torch.zeros(pages * page_size * h_k * row, dtype=torch.uint8, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    st = (h_k * page_size * row, row, page_size * row)  # HND
    kind = "head" if kv_format in ("e4m3", "nvfp4") else "channel"
    n_sc = h_k if kind == "head" else h_k * 128
    fmax = {"e4m3": 448.0, "e2m3": 7.5, "e3m2": 28.0, "e2m1": 6.0, "nvfp4": 6.0 * 448.0}[kv_format]
    k_sc = torch.full((n_sc,), 4.0 / fmax, device="cuda")
    v_sc = k_sc.clone()
    cfg = mjlib.mj_config(h_q=h_k, h_k=h_k, page_size=page_size, max_num_seqs=1, kv_format=kv_format)
    kk = mjlib.SCALE_KINDS[kind]
    a = mjlib.WriteArgs(key=key.data_ptr(), key_tok_stride=key.stride(0), key_head_stride=key.stride(1),
                        value=value.data_ptr(), value_tok_stride=value.stride(0),
                        value_head_stride=value.stride(1), num_tokens=n_tokens, slot_mapping=slots.data_ptr(),
                        k_cache=k_pool.data_ptr(), k_page_stride=st[0], k_slot_stride=st[1], k_head_stride=st[2],
                        v_cache=v_pool.data_ptr(), v_page_stride=st[0], v_slot_stride=st[1], v_head_stride=st[2],
                        num_pages=pages, k_scale=k_sc.data_ptr(), k_scale_kind=kk, v_scale=v_sc.data_ptr(),
                        v_scale_kind=kk)
    if srow:
        k_bs = torch.zeros(pages * page_size * h_k * srow, dtype=torch.uint8, device="cuda")
        v_bs = torch.zeros_like(k_bs)
        bst = (h_k * page_size * srow, srow, page_size * srow)
        a.k_block_scale, a.v_block_scale = k_bs.data_ptr(), v_bs.data_ptr()
        a.k_bs_page_stride, a.k_bs_slot_stride, a.k_bs_head_stride = bst
        a.v_bs_page_stride, a.v_bs_slot_stride, a.v_bs_head_stride = bst
    stream = torch.cuda.current_stream()
    for _ in range(3):
        mjlib.mj_write_kv(cfg, a, stream)
    flush()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        mjlib.mj_write_kv(cfg, a, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = n_tokens * h_k * 2 * (2 * 128 + row + srow) + 8 * n_tokens
    return dict(kv_format=kv_format, tokens=n_tokens, h_k=h_k, us_per_call=round(us, 2),
                algorithmic_bytes=nbytes, gbs=round(nbytes / us / 1e3, 1),
                frac_of_hbm_peak=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4))


def host_cpu():
    """(cores this process may run on, CPU model name) of the host."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def cpu_baseline(key, budget_s):
    """The oracle as it stands on whole (sequence, KV head) pairs of the same
    workload until ~budget_s seconds of wall time, with BLAS threads = the
    cores this process may use."""
    import torch
    import synth
    from oracle.attention import decode_step
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None

    cores, model = host_cpu()
    spec = synth.spec_for(key)
    wl = synth.build(spec, "cuda")
    s = wl.spec
    order = [(i, g) for i in range(s.b) for g in range(s.h_k)]
    done, nbytes, t_used = 0, 0, 0.0
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        for i in np.random.default_rng(0).permutation(s.b).tolist():
            h = wl.host([i])
            for g in range(s.h_k):
                t0 = time.perf_counter()
                decode_step(h, q_len=s.q_len, h_q=s.h_q, h_k=s.h_k, d=s.d, page_size=s.page_size,
                            kv_format=s.kv_format, causal=s.causal, pairs=[(0, g)])
                t_used += time.perf_counter() - t0
                done += 1
                nbytes += wl.seq_lens[i] * 2 * (s.row_bytes + s.scale_row_bytes)
                if t_used >= budget_s:
                    break
            if t_used >= budget_s:
                break
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    del wl
    torch.cuda.empty_cache()
    return dict(value=nbytes / t_used / 1e9, unit="GB/s", cores=cores, cpu_model=model, kind="oracle",
                blas_threads=cores,
                sample=f"{done} of {len(order)} (sequence, KV head) pairs of {spec.name} "
                       f"(each a full Q quantization + gather + fp64 attention), {t_used:.1f} s wall, "
                       f"NumPy with {cores} BLAS threads on {model}",
                seconds_per_step_extrapolated=t_used * len(order) / done)


def measure_cp(key, G, reps, flush):
    """Context parallelism on one GPU: the workload's pages cut into G
    end-aligned slices (rank r's share of each context), each slice's fused
    step (fp32 output and LSE) timed after the cache eviction, and
    mj_combine_lse over the G results; the all-gather between them (RCCL)
    is not run here: its bytes per GPU are reported."""
    import torch
    import synth
    import paged_fp8_decode_amd as mjlib
    from paged_fp8_decode_amd.runner import DecodeStep, new_output

    wl = synth.build(synth.spec_for(key), "cuda")
    s = wl.spec
    P = s.page_size
    bt = wl.block_table.cpu().numpy()
    lens = list(wl.seq_lens)
    pages = [max(1, -(-L // P)) if L else 0 for L in lens]
    chunk = [max(1, -(-p // G)) if p else 0 for p in pages]
    cols = max(1, max(chunk))
    rows = s.b * s.q_len
    part_o = torch.empty((G, rows, s.h_q, 128), dtype=torch.float32, device="cuda")
    part_l = torch.empty((G, rows, s.h_q), dtype=torch.float32, device="cuda")
    step = DecodeStep.for_workload(wl, out_f32=True)
    ks, vs = wl.kv_strides()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    stream = torch.cuda.current_stream()
    rank_us, rank_kv = [], []
    for r in range(G):
        bt_r = np.tile(bt[:, :1], (1, cols)).astype(np.int32)
        lens_r = np.zeros(s.b, dtype=np.int32)
        for i, L in enumerate(lens):
            hi = max(0, pages[i] - (G - 1 - r) * chunk[i]) if L else 0
            lo = max(0, hi - chunk[i])
            if hi > lo:
                bt_r[i, :hi - lo] = bt[i, lo:hi]
                lens_r[i] = min(hi * P, L) - lo * P
        bt_d = torch.from_numpy(bt_r).to("cuda")
        lens_d = torch.from_numpy(lens_r).to("cuda")
        info = step.plan(lens_r.tolist(), s.q_len, cols)

        def run():
            step.run(q=wl.q, k_cache=wl.k_pool, v_cache=wl.v_pool, k_strides=ks, v_strides=vs, num_pages=wl.num_pages,
                     block_table=bt_d, seq_lens=lens_d, k_descale=wl.k_descale, v_descale=wl.v_descale,
                     descale_kind=wl.descale_kind, softmax_scale=wl.softmax_scale, out=part_o[r], lse=part_l[r],
                     q_mul=wl.q_mul, o_mul=wl.o_mul, causal=s.causal and r == G - 1, info=info, stream=stream,
                     fused=True)
        ms = []
        for k in range(reps + 2):
            flush()
            e0, e1 = E(), E()
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            if k >= 2:
                ms.append(e0.elapsed_time(e1))
        rank_us.append(float(np.median(ms) * 1e3))
        rank_kv.append(int(lens_r.sum()) * s.h_k * 2 * (s.row_bytes + s.scale_row_bytes))
    cfg = mjlib.mj_config(h_q=s.h_q, h_k=s.h_k, page_size=P, max_num_seqs=s.b)
    out, lse = new_output(wl)
    ms = []
    for k in range(reps + 2):
        flush()
        e0, e1 = E(), E()
        e0.record(stream)
        mjlib.mj_combine_lse(cfg, part_o, part_l, out, lse, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if k >= 2:
            ms.append(e0.elapsed_time(e1))
    comb = float(np.median(ms) * 1e3)
    res = dict(workload=s.name, G=G, slice_step_us=[round(x, 1) for x in rank_us],
               slice_step_us_max=round(max(rank_us), 1), slice_kv_bytes=rank_kv,
               slice_kv_gbs_of_slowest=round(rank_kv[int(np.argmax(rank_us))] / max(rank_us) / 1e3, 1),
               combine_us=round(comb, 1), allgather_bytes_per_gpu=rows * s.h_q * (128 + 1) * 4,
               note="one GPU's share and the combine; the RCCL all-gather between them is not run")
    log(f"[bench] {key} context-parallel share G={G}: slice steps {min(rank_us):.1f}-{max(rank_us):.1f} us "
        f"(KV {min(rank_kv) / 1e6:.0f}-{max(rank_kv) / 1e6:.0f} MB per slice), combine of {G} slices "
        f"{comb:.1f} us, all-gather {res['allgather_bytes_per_gpu'] / 1e6:.2f} MB per GPU")
    del wl
    torch.cuda.empty_cache()
    return res


def measure_draft(key, k, reps, flush):
    """Multi-step draft decode on the workload's shape: k steps of
    (mj_draft_advance, mj_write_kv of one new K/V row per sequence,
    mj_decode_step) captured as one hipGraph, timed per replay after the
    cache eviction (the lengths reset outside the event pair).  Two plans:
    the pages' host plan made k tokens long once, and each step planning
    from the live lengths in its own decode launch."""
    import torch
    import synth
    import paged_fp8_decode_amd as mjlib
    from paged_fp8_decode_amd.runner import DecodeStep, new_output

    wl = synth.build(synth.spec_for(key), "cuda")
    s = wl.spec
    # real pages for the k new positions (the spare block-table columns point at the poison page)
    bt = wl.block_table.cpu().numpy()
    used = set(int(x) for x in bt.reshape(-1))
    free = [p for p in range(wl.num_pages) if p not in used]
    for i, L in enumerate(wl.seq_lens):
        for c in range(-(-L // s.page_size), -(-(L + k * s.q_len) // s.page_size)):
            bt[i, c] = free.pop()
    wl.block_table.copy_(torch.from_numpy(bt))
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    n = s.b * s.q_len
    kn = torch.randn((k, n, s.h_k, 128), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((k, n, s.h_k, 128), generator=g, device="cuda").to(torch.bfloat16)
    qn = torch.randn((k, n, s.h_q, 128), generator=g, device="cuda").to(torch.bfloat16)
    slots = torch.zeros((k, n), dtype=torch.int64, device="cuda")
    step = DecodeStep.for_workload(wl)
    out, lse = new_output(wl)
    lens0 = wl.seq_lens_dev.clone()
    ks, vs = wl.kv_strides()
    if s.kv_format in ("e4m3", "nvfp4"):
        kind, k_sc, v_sc = wl.descale_kind, wl.k_descale, wl.v_descale
    else:
        kind, k_sc, v_sc = "channel", wl.k_channel_scale, wl.v_channel_scale
    wa = []
    for i in range(k):
        a = mjlib.WriteArgs(key=kn[i].data_ptr(), key_tok_stride=kn[i].stride(0), key_head_stride=kn[i].stride(1),
                            value=vn[i].data_ptr(), value_tok_stride=vn[i].stride(0),
                            value_head_stride=vn[i].stride(1), num_tokens=n, slot_mapping=slots[i].data_ptr(),
                            k_cache=wl.k_pool.data_ptr(), k_page_stride=ks[0], k_slot_stride=ks[1],
                            k_head_stride=ks[2], v_cache=wl.v_pool.data_ptr(), v_page_stride=vs[0],
                            v_slot_stride=vs[1], v_head_stride=vs[2], num_pages=wl.num_pages,
                            k_scale=k_sc.data_ptr(), k_scale_kind=mjlib.SCALE_KINDS[kind], v_scale=v_sc.data_ptr(),
                            v_scale_kind=mjlib.SCALE_KINDS[kind])
        if wl.k_bs_pool is not None:
            kb, vb = wl.bs_strides()
            a.k_block_scale, a.v_block_scale = wl.k_bs_pool.data_ptr(), wl.v_bs_pool.data_ptr()
            a.k_bs_page_stride, a.k_bs_slot_stride, a.k_bs_head_stride = kb
            a.v_bs_page_stride, a.v_bs_slot_stride, a.v_bs_head_stride = vb
        wa.append(a)

    def loop(st, in_kernel):
        for i in range(k):
            mjlib.mj_draft_advance(step.cfg, wl.block_table, wl.seq_lens_dev, s.b, s.q_len, slots[i], st)
            mjlib.mj_write_kv(step.cfg, wa[i], st)
            wl.q = qn[i]
            info = step.plan_workload_shape(wl) if in_kernel else step.info
            step.run_workload(wl, out, lse, info=info, stream=st, fused=True, plan_on_device=in_kernel)

    res = dict(k=k, workload=s.name)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for name, in_kernel in (("margin_plan", False), ("in_kernel_plan", True)):
        if not in_kernel:
            step.plan(list(wl.seq_lens), s.q_len, wl.block_table.shape[1], margin=k * s.q_len)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            loop(side, in_kernel)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            loop(torch.cuda.current_stream(), in_kernel)
        stream = torch.cuda.current_stream()
        ms = []
        for r in range(reps + 3):
            wl.seq_lens_dev.copy_(lens0)
            flush()
            e0, e1 = E(), E()
            e0.record(stream)
            gr.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            if r >= 3:
                ms.append(e0.elapsed_time(e1))
        us = float(np.median(ms) * 1e3)
        res[name] = dict(us_per_graph=round(us, 2), us_per_draft_step=round(us / k, 2))
        del gr
    log(f"[bench] {key}: {k}-step draft loop (advance + KV write + decode step per draft step) in one hipGraph: "
        f"{res['margin_plan']['us_per_draft_step']:.1f} us per draft step on one margin plan, "
        f"{res['in_kernel_plan']['us_per_draft_step']:.1f} us planning in the decode launch")
    del wl
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import paged_fp8_decode_amd

    if args.calibrate:
        calibrate()
        return

    KSEL.update(decode_kernel=args.variant, kv_cache_policy=args.cache_policy, step_merge=args.step_merge)

    flush = Flusher()
    floor = measure_launch_floor(max(20, args.steps), max(5, args.warmup), flush)
    main_res = measure(args.workload, args.steps, args.warmup, flush, args.wgs_per_cu, not args.no_stream_read)
    extra = {}
    for k in [x for x in args.extra.split(",") if x]:
        extra[k] = measure(k, max(10, args.steps // 2), max(3, args.warmup // 2), flush, args.wgs_per_cu, False)
    bf16q = {}
    for k in [x for x in args.bf16q.split(",") if x]:
        bf16q[k] = measure(k, max(10, args.steps // 2), max(3, args.warmup // 2), flush, args.wgs_per_cu, False,
                           q_mode="bf16")
    writes = []
    if not args.no_write:
        for fmt in ("e4m3", "e2m3", "e3m2", "e2m1", "nvfp4"):
            for n_tok, reps in ((16384, 20), (32, 200)):
                w = measure_write(fmt, n_tok, reps, flush)
                log(f"[bench] mj_write_kv {fmt} {n_tok} tokens x 8 heads: {w['us_per_call']} us, {w['gbs']} GB/s")
                writes.append(w)
    cp = None
    if args.cp:
        cp_key, cp_g = args.cp.split(":")
        cp = measure_cp(cp_key, int(cp_g), max(10, args.steps // 2), flush)
    draft = None
    if args.draft > 0:
        draft = measure_draft(args.draft_workload, args.draft, max(10, args.steps // 2), flush)
    cpu = None if args.no_cpu else cpu_baseline(args.workload, args.cpu_seconds)
    kvb = main_res["kv_bytes"]
    dec_s = main_res["kernel_us_back_to_back"] * 1e-6
    roof = dict(bound="hbm", achieved=round(kvb / dec_s / 1e9, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(kvb / dec_s / 1e9 / HBM_PEAK_GBS, 4), traffic=traffic_for(args.workload),
                kernel="decode_mfma_kernel (fused Q quantization + paged decode; its steps' merge launches timed apart "
                       "and subtracted)",
                algorithmic_bytes_per_launch=kvb, kernel_us=round(main_res["kernel_us_back_to_back"], 2),
                traffic_unit="bytes per launch (scaled FETCH_SIZE + WRITE_SIZE)")
    # every workload at a glance: graph step, decode kernel and its share of the HBM peak
    configs = {k: dict(workload=r["workload"], kv_bytes=r["kv_bytes"],
                       graph_us_per_step_median=round(r["graph_us_per_step_median"], 2),
                       decode_kernel_us=round(r["kernel_us_back_to_back"], 2),
                       kernel_frac_of_hbm_peak=round(r["kernel_frac_of_hbm_peak"], 4),
                       graph_step_over_kernel_us=round(r["graph_us_per_step_median"] - r["kernel_us_back_to_back"], 2),
                       with_reduction=r["plan"]["with_reduction"])
               for k, r in [(args.workload, main_res)] + list(extra.items())}
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
        dtype=main_res["kv_format"],
        data="synthetic",
        config=dict(workload=main_res["workload"], kv_bytes=kvb, plan=main_res["plan"], kernel_variant=args.variant,
                    kv_cache_policy=args.cache_policy, step_merge=args.step_merge,
                    step="hipGraph: mj_decode_step with plan_on_device (decode + merge launches)"),
        roofline=roof,
        cpu_baseline=cpu,
        configs=configs,
        launch_floor=floor,
        detail=main_res,
        extra=extra,
        bf16_q=bf16q,
        write_kv=writes,
        draft=draft,
        context_parallel=cp,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

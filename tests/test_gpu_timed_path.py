"""The step bench.py times, checked at full size on every workload: a hipGraph
of mj_decode_step planning from the device lengths inside the decode launch
(plus the merge launch when the plan splits), in both Q modes.  One replay
must give the eager fused step on the host planner's plan bit for bit, leave
the host plan's n_splits / split_begin in the plan buffer, and match the fp64
oracle on sampled (sequence, KV head) pairs within the stated tolerance
(mjolnir-kernel README "What it does", step 1: a captured step replays later
plans with no re-capture)."""

import numpy as np
import pytest
import torch

import synth
from helpers import compare_lse, compare_out, oracle_step, say

pytestmark = pytest.mark.gpu

KEYS = ["cfg1", "cfg2", "cfg3", "cfg4c", "cfg4n", "cfg5", "32k", "32k_b16", "cfg5_e3m2", "cfg5_e2m1", "cfg5_nvfp4",
        "cfg3_nvfp4", "cfg3_e2m3", "cfg3_e2m1"]
# bf16 Q is the runner's other mode for the e4m3 and nvfp4 caches (the packed
# fp6 / fp4 caches take fp8 Q only)
CASES = [(k, "fp8") for k in KEYS] + [(k, "bf16") for k in KEYS
                                      if synth.spec_for(k).kv_format in ("e4m3", "nvfp4")]


@pytest.fixture(scope="module")
def mj(gpu):
    import paged_fp8_decode_amd as m
    return m


@pytest.mark.parametrize("key,q_mode", CASES)
def test_timed_step_full_size(mj, gpu, key, q_mode):
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for(key), gpu)
    s = wl.spec
    say(f"timed path {s.name} q_mode={q_mode}: b={s.b} kv_bytes={wl.kv_bytes()}")
    step = DecodeStep.for_workload(wl, q_mode=q_mode)
    out, lse = new_output(wl)
    info = step.plan_workload_shape(wl)

    def body():
        step.run_workload(wl, out, lse, info=info, fused=True, plan_on_device=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()
    step.plan_dev.fill_(-3)
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    plan_graph = step.plan_dev.cpu().numpy()

    # the eager step on the host planner's plan
    hinfo = step.plan_workload(wl)
    assert (hinfo.num_work, hinfo.with_reduction) == (info.num_work, info.with_reduction)
    ref_o, ref_l = new_output(wl)
    step.run_workload(wl, ref_o, ref_l, info=hinfo, fused=True)
    torch.cuda.synchronize()
    say(f"  plan: work={hinfo.num_work} slots={hinfo.slots} chunk_tiles={hinfo.chunk_tiles} "
        f"reduction={hinfo.with_reduction} wgs_per_cu={hinfo.wgs_per_cu}")
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), "graph step != host-plan step"
    assert torch.equal(lse, ref_l), "graph step LSE != host-plan step LSE"

    # the split counts and first items the graph's decode launch published
    img, _ = mj.mj_plan_compute(step.cfg, np.array(wl.seq_lens, np.int32), s.q_len, 0, wl.block_table.shape[1])
    cap_max = (img.size - 2 * step.cfg.max_num_seqs) // 4
    ns = slice(4 * cap_max, 4 * cap_max + s.b)
    sb = slice(4 * cap_max + step.cfg.max_num_seqs, 4 * cap_max + step.cfg.max_num_seqs + s.b)
    assert np.array_equal(plan_graph[ns], img[ns]) and np.array_equal(plan_graph[sb], img[sb])

    # the oracle on the longest and shortest sequences and one more, first and last KV head
    lens = np.array(wl.seq_lens)
    rng = np.random.default_rng(5)
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), int(rng.integers(0, s.b))})
    heads = sorted({0, s.h_k - 1})
    O, LSE = oracle_step(wl, seqs=seqs, heads=heads, quantize=q_mode == "fp8")
    compare_out(out, O, f"{s.name} {q_mode} seqs={seqs} heads={heads}")
    compare_lse(lse, LSE, f"{s.name} {q_mode}")
    del wl, graph
    torch.cuda.empty_cache()

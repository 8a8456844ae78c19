"""GPU parity of the context-parallel path on one GPU: each sequence's pages
are cut into G contiguous slices (one per rank of a context-parallel group),
every slice is decoded through the C ABI with fp32 output (config out_f32)
and its LSE, the G results stand side by side as an all-gather would leave
them, and mj_combine_lse merges them; the result is compared with the
oracle's attention over the whole context.  The last slice holds each
sequence's tail and runs causal; the others run non-causal."""

import numpy as np
import pytest
import torch

import synth
from helpers import compare_lse, compare_out, oracle_step, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mj(gpu):
    import paged_fp8_decode_amd as m
    return m


def slices(block_table, lens, page_size, G):
    """Per rank r: (block table rows (b, cols), lengths): page chunks of
    C_i = ceil(pages_i / G) pages aligned to the end of each sequence, so the
    last rank holds the tail; earlier ranks may hold nothing."""
    bt = block_table.cpu().numpy()
    b = len(lens)
    pages = [max(1, -(-L // page_size)) if L else 0 for L in lens]
    chunk = [max(1, -(-p // G)) if p else 0 for p in pages]
    cols = max(1, max(chunk))
    out = []
    for r in range(G):
        bt_r = np.tile(bt[:, :1], (1, cols)).astype(np.int32)  # unused columns: a valid page, never read
        lens_r = np.zeros(b, dtype=np.int32)
        for i, L in enumerate(lens):
            if not L:
                continue
            hi = max(0, pages[i] - (G - 1 - r) * chunk[i])
            lo = max(0, hi - chunk[i])
            if hi > lo:
                bt_r[i, :hi - lo] = bt[i, lo:hi]
                lens_r[i] = min(hi * page_size, L) - lo * page_size
        out.append((bt_r, lens_r))
    assert all(sum(int(x[1][i]) for x in out) == L for i, L in enumerate(lens))
    return out


def run_cp(mj, wl, G, gpu, **kw):
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    s = wl.spec
    rows = s.b * s.q_len
    part_o = torch.full((G, rows, s.h_q, 128), float("nan"), dtype=torch.float32, device=gpu)
    part_l = torch.full((G, rows, s.h_q), float("nan"), dtype=torch.float32, device=gpu)
    step = DecodeStep.for_workload(wl, out_f32=True, **kw)
    ks, vs = wl.kv_strides()
    bs = {}
    if wl.k_bs_pool is not None:
        kb, vb = wl.bs_strides()
        bs = dict(k_block_scale=wl.k_bs_pool, v_block_scale=wl.v_bs_pool, k_bs_strides=kb, v_bs_strides=vb)
    for r, (bt_r, lens_r) in enumerate(slices(wl.block_table, wl.seq_lens, s.page_size, G)):
        bt_d = torch.from_numpy(bt_r).to(gpu)
        lens_d = torch.from_numpy(lens_r).to(gpu)
        info = step.plan(lens_r.tolist(), s.q_len, bt_r.shape[1])
        step.run(**bs, q=wl.q, k_cache=wl.k_pool, v_cache=wl.v_pool, k_strides=ks, v_strides=vs,
                 num_pages=wl.num_pages, block_table=bt_d, seq_lens=lens_d, k_descale=wl.k_descale,
                 v_descale=wl.v_descale, descale_kind=wl.descale_kind, softmax_scale=wl.softmax_scale, out=part_o[r],
                 lse=part_l[r], q_mul=wl.q_mul, o_mul=wl.o_mul, causal=s.causal and r == G - 1, info=info, fused=True)
        torch.cuda.synchronize()
    cfg = mj.mj_config(h_q=s.h_q, h_k=s.h_k, page_size=s.page_size, max_num_seqs=s.b)
    out, lse = new_output(wl)
    out.fill_(float("nan"))
    mj.mj_combine_lse(cfg, part_o, part_l, out, lse)
    torch.cuda.synchronize()
    return out, lse, part_o, part_l


@pytest.mark.parametrize("G", [2, 4, 8])
@pytest.mark.parametrize("key", ["cfg2", "cfg3", "cfg4c", "cfg4n", "cfg5", "cfg5_nvfp4"])
def test_context_parallel_slices_combine_to_full_attention(mj, gpu, key, G):
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    say(f"context parallel {wl.spec.name} G={G} lens={wl.seq_lens}")
    out, lse, _, _ = run_cp(mj, wl, G, gpu, min_chunk_tokens=1)
    O, LSE = oracle_step(wl)
    compare_out(out, O, f"{key} G={G}")
    compare_lse(lse, LSE, f"{key} G={G}")


@pytest.mark.parametrize("key", ["cfg2", "cfg4c", "cfg5_nvfp4"])
def test_context_parallel_with_bf16_q(mj, gpu, key):
    """The slices decoded in bf16-Q mode (Q as given, KV converted in the
    kernel), fp32 output, combined."""
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    say(f"context parallel bf16 Q {wl.spec.name} G=4")
    out, lse, _, _ = run_cp(mj, wl, 4, gpu, q_mode="bf16", min_chunk_tokens=1)
    O, LSE = oracle_step(wl, quantize=False)
    compare_out(out, O, f"{key} bf16 Q G=4")
    compare_lse(lse, LSE, f"{key} bf16 Q G=4")


@pytest.mark.parametrize("key", ["cfg3", "cfg4c"])
def test_more_slices_than_one_combine_batch(mj, gpu, key):
    """11 slices: the combine takes them in two batches with a running
    maximum between (several slices of a short sequence are empty)."""
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    say(f"context parallel {wl.spec.name} G=11")
    out, lse, _, _ = run_cp(mj, wl, 11, gpu, min_chunk_tokens=1)
    O, LSE = oracle_step(wl)
    compare_out(out, O, f"{key} G=11")
    compare_lse(lse, LSE, f"{key} G=11")


def test_fp32_output_matches_bf16_output(mj, gpu):
    """out_f32 changes only the output rounding: the fp32 result rounded to
    bf16 is the bf16 result, on the matrix-core and generic kernels, split
    and unsplit."""
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for("cfg4c", small=True), gpu)
    for variant in (0, 1):
        for ms in (1, 16):
            res = []
            for f32 in (False, True):
                step = DecodeStep.for_workload(wl, out_f32=f32, max_splits=ms, min_chunk_tokens=1,
                                               decode_kernel=variant)
                info = step.plan_workload(wl)
                out, lse = new_output(wl, out_f32=f32)
                step.run_workload(wl, out, lse, info=info, fused=True)
                torch.cuda.synchronize()
                res.append((out, lse))
            assert torch.equal(res[1][0].to(torch.bfloat16).view(torch.int16), res[0][0].view(torch.int16))
            assert torch.equal(res[1][1], res[0][1])


def test_context_parallel_full_size_sampled(mj, gpu):
    """cfg3's full batch (64 ragged sequences up to 32K) over 8 slices, the
    per-GPU share of an 8-GPU context-parallel group."""
    wl = synth.build(synth.spec_for("cfg3"), gpu)
    say(f"context parallel full {wl.spec.name} G=8")
    out, lse, _, _ = run_cp(mj, wl, 8, gpu)
    lens = np.array(wl.seq_lens)
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 7})
    O, LSE = oracle_step(wl, seqs=seqs, heads=[0, wl.spec.h_k - 1])
    compare_out(out, O, "cfg3 G=8")
    compare_lse(lse, LSE, "cfg3 G=8")

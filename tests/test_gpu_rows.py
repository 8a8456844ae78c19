"""GPU parity for GQA groups of more than 32 query rows (q_len * h_q / h_k
> 32: long speculative blocks, wide groups).  The matrix-core kernel serves
them as tiles of 32 rows, one workgroup per (item, KV head, tile), all tiles
reading the same KV rows; the fused step's Q scale still covers every row of
the (sequence, KV head) pair, as the stand-alone quantization does.

* outputs and LSE of every format (and the token-major layout) against the
  oracle at 40 (two tiles, the second partial), 66, 128, 576 and 1024 rows,
  with causal blocks longer than some sequences, empty sequences and forced
  splits;
* the fused step (in-kernel quantization) equals the three-call path bit for
  bit, also with the in-kernel merge asked for (which such groups leave to
  the merge launch) and with the plan made in the kernel;
* the grid numberings and prefetch depths give the same bits;
* bf16-Q mode.
"""

import numpy as np
import pytest
import torch

import synth
from helpers import compare_lse, compare_out, oracle_step, say

pytestmark = pytest.mark.gpu

LENS = (0, 1, 2, 3, 31, 32, 33, 127, 128, 129, 1000)
# (q_len, h_q, h_k, causal): 40, 66, 128, 576 and 1024 rows per group (the
# library's largest)
SHAPES = [(5, 64, 8, True), (11, 48, 8, True), (16, 64, 8, False), (9, 64, 1, True), (16, 64, 1, True)]
KEYS = ["cfg2", "cfg3", "cfg5", "cfg5_e3m2", "cfg5_e2m1", "cfg5_nvfp4"]


@pytest.fixture(scope="module")
def mj(gpu):
    import paged_fp8_decode_amd as m
    return m


def _wl(key, shape, gpu, lens=LENS):
    q_len, h_q, h_k, causal = shape
    over = dict(b=len(lens), lens=lens, q_len=q_len, h_q=h_q, h_k=h_k, causal=causal, k_outliers=0,
                slots_override=0)
    if synth.SPECS[key].lens_loguniform:
        over["lens_loguniform"] = ()
    return synth.build(synth.spec_for(key, small=True, **over), gpu)


def _run(mj, wl, fused, q_mode="fp8", plan_on_device=False, **overrides):
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    step = DecodeStep.for_workload(wl, q_mode=q_mode, **overrides)
    info = step.plan_workload_shape(wl) if plan_on_device else step.plan_workload(wl)
    out, lse = new_output(wl)
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    step.run_workload(wl, out, lse, info=info, fused=fused, plan_on_device=plan_on_device)
    torch.cuda.synchronize()
    return out, lse, info


def _same(a, b, what):
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), what
    assert torch.equal(a[1], b[1]), what


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"q{s[0]}_h{s[1]}_{s[2]}")
@pytest.mark.parametrize("key", KEYS)
def test_many_rows_parity(mj, gpu, key, shape):
    wl = _wl(key, shape, gpu)
    n_q = shape[0] * shape[1] // shape[2]
    O, LSE = oracle_step(wl)
    for mct in (0, 1):
        say(f"rows {wl.spec.name} n_q={n_q} min_chunk_tokens={mct}")
        three = _run(mj, wl, fused=False, min_chunk_tokens=mct)
        say(f"  plan: work={three[2].num_work} reduction={three[2].with_reduction}")
        compare_out(three[0], O, f"{key} n_q={n_q} three-call")
        compare_lse(three[1], LSE, f"{key} n_q={n_q} three-call")
        fused = _run(mj, wl, fused=True, min_chunk_tokens=mct)
        _same(fused, three[:2], f"{key} n_q={n_q} fused vs three-call mct={mct}")


@pytest.mark.parametrize("key", ["cfg2", "cfg5_nvfp4"])
def test_many_rows_in_kernel_merge_request_and_plan(mj, gpu, key):
    """With the in-kernel merge switched on, groups of several row tiles
    still merge in the merge launch (the arrival counter covers one tile), and
    the in-kernel plan gives the host plan's bits."""
    wl = _wl(key, (5, 64, 8, True), gpu)
    ref = _run(mj, wl, fused=False, min_chunk_tokens=1)
    for rep in range(3):
        say(f"rows {wl.spec.name} step_merge=1 rep={rep}")
        _same(_run(mj, wl, fused=True, min_chunk_tokens=1, step_merge=1), ref[:2], f"merge request rep={rep}")
    for mct in (0, 1):
        host = _run(mj, wl, fused=True, min_chunk_tokens=mct)
        say(f"rows {wl.spec.name} plan in kernel mct={mct}")
        _same(_run(mj, wl, fused=True, plan_on_device=True, min_chunk_tokens=mct), host[:2], f"plan mct={mct}")


@pytest.mark.parametrize("key", ["cfg2", "cfg5_e2m1"])
def test_many_rows_grid_orders_bit_identical(mj, gpu, key):
    wl = _wl(key, (11, 48, 8, True), gpu)
    ref = None
    for v in (10, 11, 12, 14, 15):
        say(f"rows grid order {wl.spec.name} variant={v}")
        got = _run(mj, wl, fused=True, min_chunk_tokens=1, decode_kernel=v)
        if ref is None:
            ref = got
            O, LSE = oracle_step(wl)
            compare_out(got[0], O, f"{key} variant {v}")
            compare_lse(got[1], LSE, f"{key} variant {v}")
        else:
            _same(got, ref[:2], f"variant {v}")


@pytest.mark.parametrize("shape", [(5, 64, 8, True), (16, 64, 8, False)], ids=lambda s: f"q{s[0]}_h{s[1]}_{s[2]}")
@pytest.mark.parametrize("key", ["cfg2", "cfg5_nvfp4"])
def test_many_rows_bf16q(mj, gpu, key, shape):
    wl = _wl(key, shape, gpu)
    O, LSE = oracle_step(wl, quantize=False)
    for mct in (0, 1):
        say(f"rows bf16-Q {wl.spec.name} n_q={shape[0] * shape[1] // shape[2]} mct={mct}")
        out, lse, _ = _run(mj, wl, fused=True, q_mode="bf16", min_chunk_tokens=mct)
        compare_out(out, O, f"{key} bf16-Q")
        compare_lse(lse, LSE, f"{key} bf16-Q")

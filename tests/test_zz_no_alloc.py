"""mj_decode_step_noalloc (the step with the library's static per-GPU plan
buffer and workspace) against mj_decode_step on caller-owned buffers: the
same kernels on the same plan, so the outputs must agree bit for bit.  Two
calls in a row, the second on a smaller input, then a third on another
format: each call finds the previous call's contents in the shared array and
must not depend on them."""

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


def _both(mj, wl, **overrides):
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    step = DecodeStep.for_workload(wl, **overrides)
    info = step.plan_workload_shape(wl)
    ref_o, ref_l = new_output(wl)
    step.run_workload(wl, ref_o, ref_l, info=info, fused=True, plan_on_device=True)
    out, lse = new_output(wl)
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    assert mj.mj_noalloc_scratch_bytes(step.cfg) <= 32 << 20
    step.run_workload(wl, out, lse, info=info, fused=True, plan_on_device=True, noalloc=True)
    torch.cuda.synchronize()
    return info, (out, lse), (ref_o, ref_l)


def _same(a, b, what):
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), what
    assert torch.equal(a[1], b[1]), what


def test_noalloc_matches_decode_step_two_calls(mj, gpu):
    # call 1: the ragged batch at full size (64 sequences up to 32K tokens,
    # several splits per sequence)
    big = synth.build(synth.spec_for("cfg3"), gpu)
    say(f"noalloc call 1: {big.spec.name} b={big.spec.b}")
    info, got, ref = _both(mj, big)
    assert info.with_reduction
    _same(got, ref, "call 1")
    seqs = [int(np.argmax(big.seq_lens)), int(np.argmin(big.seq_lens))]
    O, LSE = oracle_step(big, seqs=seqs, heads=[0, big.spec.h_k - 1])
    compare_out(got[0], O, "noalloc call 1 (sampled)")
    compare_lse(got[1], LSE, "noalloc call 1 (sampled)")
    del big
    # call 2: a smaller input (the speculative-verification shape, reduced)
    small = synth.build(synth.spec_for("cfg4c", small=True), gpu)
    say(f"noalloc call 2: {small.spec.name} b={small.spec.b}")
    info, got, ref = _both(mj, small, min_chunk_tokens=1)
    _same(got, ref, "call 2")
    O, LSE = oracle_step(small)
    compare_out(got[0], O, "noalloc call 2")
    compare_lse(got[1], LSE, "noalloc call 2")
    # call 3: another format and a batch that cannot split
    tiny = synth.build(synth.spec_for("cfg5_nvfp4", small=True), gpu)
    say(f"noalloc call 3: {tiny.spec.name} b={tiny.spec.b}")
    info, got, ref = _both(mj, tiny)
    _same(got, ref, "call 3")

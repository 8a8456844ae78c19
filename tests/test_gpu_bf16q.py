"""GPU parity of the bf16-Q mode (config q_mode = bf16: Q used as given, the
e4m3 or nvfp4 KV codes converted to bf16 in the kernel) against the oracle's
unquantized-Q attention, through the C ABI:

* the in-kernel e4m3 -> bf16 operand converter on every code (bit-exact);
* every output of the reduced workloads, on the matrix-core kernel and the
  generic kernel, as four calls and as one mj_decode_step (with a host plan
  and planning from the device lengths);
* edge lengths and speculative shapes (replicated rows, 32 rows, > 32 rows as
  32-row tiles), forced splits, a strided Q view;
* sampled rows of the full-size workloads in the step the bench times.
"""

import numpy as np
import pytest
import torch

import synth
from helpers import compare_lse, compare_out, oracle_step, say, step_overrides

pytestmark = pytest.mark.gpu

E4M3_KEYS = ["cfg1", "cfg2", "cfg3", "cfg4c", "cfg4n", "32k", "32k_b16", "cfg5_nvfp4", "cfg3_nvfp4"]
FINE = dict(min_chunk_tokens=1)


@pytest.fixture(scope="module")
def mj(gpu):
    import paged_fp8_decode_amd as m
    return m


@pytest.fixture
def variant(mj, request):
    v = getattr(request, "param", 0)
    with step_overrides(decode_kernel=v):
        yield v


def _run(wl, fused=False, plan_on_device=False, **overrides):
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    step = DecodeStep.for_workload(wl, q_mode="bf16", **overrides)
    info = step.plan_workload_shape(wl) if plan_on_device else step.plan_workload(wl)
    out, lse = new_output(wl)
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    step.run_workload(wl, out, lse, info=info, fused=fused, plan_on_device=plan_on_device)
    torch.cuda.synchronize()
    return out, lse, info


def _check(wl, out, lse, what, **kw):
    O, LSE = oracle_step(wl, quantize=False, **kw)
    compare_out(out, O, what)
    compare_lse(lse, LSE, what)


def test_bf16_operand_converter_exhaustive(mj, gpu):
    from oracle.formats import E4M3_TABLE
    codes = torch.arange(256, dtype=torch.uint8, device=gpu)
    out = torch.empty(256, dtype=torch.float32, device=gpu)
    mj.mj_debug_decode_codes("e4m3_bf16", codes, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    fin = ~np.isnan(E4M3_TABLE)
    assert np.array_equal(got[fin], E4M3_TABLE[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(E4M3_TABLE[fin]))
    assert np.all(np.isnan(got[~fin]))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("variant", [0, 1], indirect=True)
@pytest.mark.parametrize("key", E4M3_KEYS)
def test_parity_small_all_outputs(mj, gpu, key, variant, fused):
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    say(f"bf16-Q parity {wl.spec.name} variant={variant} fused={fused} lens={wl.seq_lens}")
    out, lse, info = _run(wl, fused=fused, **FINE)
    say(f"  plan: work={info.num_work} chunk_tiles={info.chunk_tiles} reduction={info.with_reduction}")
    _check(wl, out, lse, wl.spec.name)


@pytest.mark.parametrize("key", ["cfg1", "cfg2", "cfg4c", "32k_b16"])
def test_plan_on_device_matches_host_plan(mj, gpu, key):
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    say(f"bf16-Q plan on device {wl.spec.name}")
    out1, lse1, _ = _run(wl, fused=True, **FINE)
    out2, lse2, _ = _run(wl, fused=True, plan_on_device=True, **FINE)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)
    _check(wl, out2, lse2, f"{wl.spec.name} plan on device")


@pytest.mark.parametrize("variant", [0, 1], indirect=True)
def test_split_and_unsplit_agree(mj, gpu, variant):
    wl = synth.build(synth.spec_for("cfg4c", small=True), gpu)
    say(f"bf16-Q splits {wl.spec.name}")
    O, LSE = oracle_step(wl, quantize=False)
    for ms, ovr in ((1, 0), (16, 0), (16, 64), (4, 200)):
        out, lse, info = _run(wl, max_splits=ms, slots_override=ovr, **FINE)
        say(f"  max_splits={ms} slots_override={ovr}: reduction={info.with_reduction}")
        compare_out(out, O, f"ms={ms}")
        compare_lse(lse, LSE, f"ms={ms}")


@pytest.mark.parametrize("variant", [0, 1], indirect=True)
def test_edge_lengths_and_shapes(mj, gpu, variant):
    wl = synth.build(synth.spec_for("cfg4c", small=True, b=7, lens=(0, 1, 2, 127, 128, 129, 3001)), gpu)
    say(f"bf16-Q edges {wl.spec.name} lens={wl.seq_lens}")
    out, lse, _ = _run(wl, **FINE)
    _check(wl, out, lse, "edges")
    assert torch.all(out[:4].float() == 0)
    lens = (0, 1, 2, 3, 31, 32, 33, 127, 128, 129, 1000)
    for q_len, h_q, h_k, causal in ((2, 16, 8, True), (4, 8, 8, True), (4, 8, 8, False), (2, 4, 2, False),
                                    (2, 32, 8, True), (4, 32, 8, True), (3, 40, 8, True), (4, 64, 8, False)):
        wl = synth.build(synth.spec_for("cfg2", small=True, b=len(lens), lens=lens, q_len=q_len, h_q=h_q, h_k=h_k,
                                        causal=causal, k_outliers=0), gpu)
        say(f"  edges q_len={q_len} h_q={h_q} h_k={h_k} causal={causal}")
        out, lse, _ = _run(wl, fused=True, **FINE)
        _check(wl, out, lse, f"edges q_len={q_len} h_q={h_q} causal={causal}")


def test_strided_q_view(mj, gpu):
    wl = synth.build(synth.spec_for("cfg2", small=True, q_extra_heads=16), gpu)
    say(f"bf16-Q strided Q {wl.spec.name} q.stride={wl.q.stride()}")
    for fused in (False, True):
        out, lse, _ = _run(wl, fused=fused, **FINE)
        _check(wl, out, lse, f"strided q fused={fused}")


FULL = {"cfg2": 2, "cfg3": 2, "cfg4c": 2, "32k": 2, "cfg5_nvfp4": 1}


@pytest.mark.parametrize("key", list(FULL))
def test_parity_full_size_sampled(mj, gpu, key):
    """Full-size workloads in the bench's launch configuration (default plan,
    one mj_decode_step planning from the device lengths)."""
    wl = synth.build(synth.spec_for(key), gpu)
    s = wl.spec
    say(f"bf16-Q full {s.name}: b={s.b}")
    out, lse, info = _run(wl, fused=True, plan_on_device=True)
    rng = np.random.default_rng(23)
    lens = np.array(wl.seq_lens)
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)),
                   *rng.choice(s.b, size=min(s.b, FULL[key]), replace=False).tolist()})
    heads = sorted({0, s.h_k - 1})
    _check(wl, out, lse, f"{s.name} seqs={seqs} heads={heads}", seqs=seqs, heads=heads)

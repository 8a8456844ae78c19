"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

* integer / byte work is bit-exact: the kernels' code decoders (all codes),
  the Q codes and descales, the gather through block table and strides;
* outputs match the fp64 oracle per element within 1e-2 + 2e-2*|ref| on all
  five workloads (reduced sizes: every output; full sizes: sampled
  (sequence, KV head) pairs, in the launch configuration bench.py times);
* physical page permutation gives bit-identical outputs; forced splits and no
  splits both match; hipGraph replay after re-planning new lengths is correct.
"""

import numpy as np
import pytest
import torch

import synth
from helpers import compare_lse, compare_out, oracle_step, say, step_overrides

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mj(gpu):
    import paged_fp8_decode_amd as m
    return m


def _run(mj, wl, fused=False, **overrides):
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    step = DecodeStep.for_workload(wl, **overrides)
    info = step.plan_workload(wl)
    out, lse = new_output(wl)
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    step.run_workload(wl, out, lse, info=info, fused=fused)
    torch.cuda.synchronize()
    return out, lse, info


# small workloads: KV-tile chunks (min_chunk_tokens=1) so that their short
# sequences still split and every path of the merge runs
FINE = dict(min_chunk_tokens=1)


def test_code_decoders_exhaustive(mj, gpu):
    from oracle.formats import E2M1_TABLE, E2M3_TABLE, E3M2_TABLE, E4M3_TABLE
    codes = torch.arange(256, dtype=torch.uint8, device=gpu)
    out = torch.empty(256, dtype=torch.float32, device=gpu)
    mj.mj_debug_decode_codes("e4m3", codes, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    fin = ~np.isnan(E4M3_TABLE)
    assert np.array_equal(got[fin], E4M3_TABLE[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(E4M3_TABLE[fin]))
    codes = torch.arange(64, dtype=torch.uint8, device=gpu)
    out = torch.empty(64, dtype=torch.float32, device=gpu)
    mj.mj_debug_decode_codes("e2m3", codes, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), E2M3_TABLE)
    for fmt, table in (("e3m2", E3M2_TABLE), ("e2m1", E2M1_TABLE)):
        codes = torch.arange(len(table), dtype=torch.uint8, device=gpu)
        out = torch.empty(len(table), dtype=torch.float32, device=gpu)
        mj.mj_debug_decode_codes(fmt, codes, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, table), fmt
        assert np.array_equal(np.signbit(got), np.signbit(table)), fmt


@pytest.mark.parametrize("b,q_len,h_q,h_k,mul,extra", [(1, 1, 8, 2, False, 0), (32, 1, 32, 8, False, 0),
                                                       (16, 4, 64, 8, False, 16), (4, 1, 32, 8, True, 0),
                                                       (3, 3, 16, 2, True, 4), (64, 1, 32, 8, False, 0)])
def test_quantize_q_bit_exact(mj, gpu, b, q_len, h_q, h_k, mul, extra):
    from oracle.qquant import quantize_q
    say(f"qquant b={b} q_len={q_len} h_q={h_q} h_k={h_k} mul={mul} extra_heads={extra}")
    g = torch.Generator().manual_seed(b + 7 * q_len)
    full = (torch.randn(b * q_len, h_q + extra, 128, generator=g) * 3).to(torch.bfloat16)
    full[0, 0, :5] = 0  # exact zeros and a tiny group
    q = full.to(gpu)[:, :h_q]
    q_mul = (torch.rand(h_q, 128, generator=g) * 2 + 0.05) if mul else None
    cfg = mj.mj_config(h_q=h_q, h_k=h_k, page_size=16, max_num_seqs=b, max_q_len=q_len, num_cus=256)
    q8 = torch.empty(b * h_k * q_len * (h_q // h_k) * 128, dtype=torch.uint8, device=gpu)
    qd = torch.empty(b * h_k, dtype=torch.float32, device=gpu)
    mj.mj_quantize_q(cfg, q, None if q_mul is None else q_mul.to(gpu), b, q_len, q8, qd)
    torch.cuda.synchronize()
    ref_c, ref_s = quantize_q(full[:, :h_q].float().numpy(), b, q_len, h_k, None if q_mul is None else q_mul.numpy())
    assert np.array_equal(qd.cpu().numpy().reshape(b, h_k), ref_s)
    assert np.array_equal(q8.cpu().numpy().reshape(ref_c.shape), ref_c)


def test_quantize_q_ties(mj, gpu):
    """Q rows holding every e4m3 grid value and every midpoint between
    neighbours (both signs), with 448 in each (sequence, KV head) group so the
    scale is exactly 1: the stand-alone kernel's codes (ties to even) and
    descales equal the oracle's.  (The fused step's prologue repeats this
    arithmetic; its outputs equal the three-call path's bit for bit.)"""
    from oracle.formats import E4M3_TABLE
    from oracle.qquant import quantize_q
    grid = np.unique(E4M3_TABLE[:0x7F])
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([grid, mids])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    b, q_len, h_q, h_k = 2, 1, 8, 2
    n_grp = q_len * (h_q // h_k) * 128
    q = np.zeros((b * q_len, h_q, 128), np.float32)
    for i in range(b):
        for g in range(h_k):
            blk = np.resize(np.roll(vals, 37 * (2 * i + g)), n_grp)
            blk[0] = 448.0
            q[i * q_len:(i + 1) * q_len, g * (h_q // h_k):(g + 1) * (h_q // h_k)] = blk.reshape(q_len, h_q // h_k, 128)
    qt = torch.from_numpy(q).to(torch.bfloat16)
    assert torch.equal(qt.float(), torch.from_numpy(q))
    cfg = mj.mj_config(h_q=h_q, h_k=h_k, page_size=16, max_num_seqs=b, max_q_len=q_len, num_cus=256)
    q8 = torch.empty(b * h_k * n_grp, dtype=torch.uint8, device=gpu)
    qd = torch.empty(b * h_k, dtype=torch.float32, device=gpu)
    mj.mj_quantize_q(cfg, qt.to(gpu), None, b, q_len, q8, qd)
    torch.cuda.synchronize()
    ref_c, ref_s = quantize_q(q, b, q_len, h_k, None)
    assert np.all(ref_s == 1.0)
    assert np.array_equal(qd.cpu().numpy().reshape(b, h_k), ref_s)
    assert np.array_equal(q8.cpu().numpy().reshape(ref_c.shape), ref_c)


@pytest.mark.parametrize("key", ["cfg2", "cfg4c"])
def test_fused_quantization_ties(mj, gpu, key):
    """The fused step's in-kernel Q quantization on tie values (every e4m3
    midpoint at unit scale, 448 in each group) gives the stand-alone kernel's
    codes: the fused step's outputs equal the three-call path's bit for bit."""
    from oracle.formats import E4M3_TABLE
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    s = wl.spec
    grid = np.unique(E4M3_TABLE[:0x7F])
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([mids, -mids]).astype(np.float32)
    h_r = s.h_q // s.h_k
    n_grp = s.q_len * h_r * 128
    q = np.zeros((s.b * s.q_len, s.h_q, 128), np.float32)
    for i in range(s.b):
        for g in range(s.h_k):
            blk = np.resize(np.roll(vals, 29 * (i + 3 * g)), n_grp) / 64.0  # midpoints / 64: still ties after x / s
            blk[0] = 448.0 / 64.0
            q[i * s.q_len:(i + 1) * s.q_len, g * h_r:(g + 1) * h_r] = blk.reshape(s.q_len, h_r, 128)
    wl.q.copy_(torch.from_numpy(q).to(torch.bfloat16).to(gpu))
    say(f"fused quantization ties {wl.spec.name}")
    step = DecodeStep.for_workload(wl, **FINE)
    info = step.plan_workload(wl)
    ref_o, ref_l = new_output(wl)
    step.run_workload(wl, ref_o, ref_l, info=info)
    out, lse = new_output(wl)
    step.run_workload(wl, out, lse, info=info, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(lse, ref_l)
    O, LSE = oracle_step(wl)
    compare_out(out, O, f"{key} Q ties")
    compare_lse(lse, LSE, f"{key} Q ties")


@pytest.mark.parametrize("key", ["cfg1", "cfg2", "cfg3", "cfg4c", "cfg5", "cfg5_e3m2", "cfg5_e2m1", "cfg5_nvfp4",
                                 "cfg3_nvfp4", "cfg3_e2m3", "cfg3_e2m1"])
def test_gather_probe_bit_exact(mj, gpu, key):
    from oracle.attention import gather_codes
    from paged_fp8_decode_amd.runner import DecodeStep
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    s = wl.spec
    say(f"gather {s.name}")
    step = DecodeStep.for_workload(wl)
    ks, vs = wl.kv_strides()
    a = mj.DecodeArgs(k_cache=wl.k_pool.data_ptr(), k_page_stride=ks[0], k_slot_stride=ks[1], k_head_stride=ks[2],
                      v_cache=wl.v_pool.data_ptr(), v_page_stride=vs[0], v_slot_stride=vs[1], v_head_stride=vs[2],
                      num_pages=wl.num_pages, block_table=wl.block_table.data_ptr(),
                      bt_row_stride=wl.block_table.stride(0), max_blocks_per_seq=wl.block_table.shape[1])
    h = wl.host()
    pools = [(0, h["k_pool"], h["k_strides"], s.row_bytes), (1, h["v_pool"], h["v_strides"], s.row_bytes)]
    if s.kv_format == "nvfp4":
        kb, vb = wl.bs_strides()
        a.k_block_scale, a.v_block_scale = wl.k_bs_pool.data_ptr(), wl.v_bs_pool.data_ptr()
        a.k_bs_page_stride, a.k_bs_slot_stride, a.k_bs_head_stride = kb
        a.v_bs_page_stride, a.v_bs_slot_stride, a.v_bs_head_stride = vb
        pools += [(2, h["k_bs_pool"], h["k_bs_strides"], s.scale_row_bytes),
                  (3, h["v_bs_pool"], h["v_bs_strides"], s.scale_row_bytes)]
    for i in range(s.b):
        L = wl.seq_lens[i]
        for g in {0, s.h_k - 1}:
            for which, pool, st, row in pools:
                dense = torch.empty(max(1, L * row), dtype=torch.uint8, device=gpu)
                mj.mj_debug_gather_kv(step.cfg, a, i, g, L, which, dense)
                torch.cuda.synchronize()
                ref = gather_codes(pool, st, s.page_size, h["block_table"][i], L, g, row)
                assert np.array_equal(dense.cpu().numpy()[: L * row].reshape(L, row), ref)


SMALL_KEYS = ["cfg1", "cfg2", "cfg3", "cfg4c", "cfg4n", "cfg5", "cfg5_e3m2", "cfg5_e2m1", "cfg5_nvfp4", "cfg3_nvfp4",
              "cfg3_e2m3", "cfg3_e2m1", "32k", "32k_b16"]
# mj_config.decode_kernel: 0 = automatic choice, 1 = generic LDS kernel, 18 =
# the matrix-core kernel with four waves where the default runs eight, 58 =
# four KV heads per workgroup and 46 = two on the XCD-grouped grid (packed
# formats; the small workloads have too few items for the automatic choice
# to take head groups)
VARIANTS = [0, 1, 18, 58, 46]


@pytest.fixture
def variant(mj, request):
    v = getattr(request, "param", 0)
    with step_overrides(decode_kernel=v):
        yield v


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("key", SMALL_KEYS)
def test_parity_small_all_outputs(mj, gpu, key, variant):
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    say(f"parity {wl.spec.name} variant={variant} lens={wl.seq_lens}")
    out, lse, info = _run(mj, wl, **FINE)
    say(f"  plan: work={info.num_work} slots={info.slots} chunk_tiles={info.chunk_tiles} "
        f"reduction={info.with_reduction}")
    O, LSE = oracle_step(wl)
    compare_out(out, O, wl.spec.name)
    compare_lse(lse, LSE, wl.spec.name)


@pytest.mark.parametrize("key", ["cfg2", "cfg4c", "cfg5", "cfg5_e3m2", "cfg5_e2m1", "cfg5_nvfp4", "cfg3_e2m3"])
@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
def test_split_and_unsplit_agree(mj, gpu, key, variant):
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    say(f"splits {wl.spec.name}")
    O, LSE = oracle_step(wl)
    for ms, ovr in ((1, 0), (16, 0), (16, 64), (4, 200)):
        out, lse, info = _run(mj, wl, max_splits=ms, slots_override=ovr, **FINE)
        say(f"  max_splits={ms} slots_override={ovr}: reduction={info.with_reduction} chunks={info.num_chunks}")
        compare_out(out, O, f"{wl.spec.name} ms={ms}")
        compare_lse(lse, LSE, f"{wl.spec.name} ms={ms}")


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
def test_page_permutation_bit_identical(mj, gpu, variant):
    wl = synth.build(synth.spec_for("cfg3", small=True), gpu)
    say(f"permutation {wl.spec.name}")
    out1, lse1, _ = _run(mj, wl, **FINE)
    perm = torch.randperm(wl.num_pages, generator=torch.Generator().manual_seed(3)).to(gpu)
    inv = torch.argsort(perm)
    wl.k_pool = wl.k_pool[perm].contiguous()
    wl.v_pool = wl.v_pool[perm].contiguous()
    wl.block_table = inv[wl.block_table.long()].to(torch.int32).contiguous()
    out2, lse2, _ = _run(mj, wl, **FINE)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)


@pytest.mark.parametrize("variant", [0, 1, 46, 58], indirect=True)
@pytest.mark.parametrize("key", ["cfg5_e2m1", "cfg5_nvfp4", "cfg3_nvfp4", "cfg3_e2m3", "cfg3_e2m1"])
def test_sub_byte_edge_lengths_and_shapes(mj, gpu, key, variant):
    """The packed formats at empty, single-token and tile-boundary lengths,
    and in the speculative row shapes (replicated rows, 8, 16, 32 rows; 40
    rows as two 32-row tiles, or on the generic kernel as variant 1), with
    one, two (46) and four (58) KV heads per workgroup where the shape
    allows it (up to 16 rows, h_k a multiple)."""
    lens = (0, 1, 2, 3, 31, 32, 33, 127, 128, 129, 1000)
    for q_len, h_q, h_k, causal in ((1, 32, 8, True), (2, 16, 8, True), (4, 8, 8, True), (2, 4, 2, False),
                                    (2, 32, 8, True), (4, 32, 8, True), (3, 40, 8, True), (5, 64, 8, True)):
        wl = synth.build(synth.spec_for(key, small=True, b=len(lens), lens=lens, lens_loguniform=(), q_len=q_len,
                                        h_q=h_q, h_k=h_k, causal=causal, k_outliers=0, slots_override=0), gpu)
        say(f"  {key} edges q_len={q_len} h_q={h_q} h_k={h_k} causal={causal} variant={variant}")
        out, lse, _ = _run(mj, wl, **FINE)
        O, LSE = oracle_step(wl)
        compare_out(out, O, f"{key} edges q_len={q_len} h_q={h_q}")
        compare_lse(lse, LSE, f"{key} edges q_len={q_len} h_q={h_q}")
        if q_len == 1:
            assert torch.all(out[:1].float() == 0)  # L = 0


def test_e2m1_eight_head_groups(mj, gpu):
    """e2m1 in token-major pages takes eight KV heads per workgroup when h_k
    is a multiple of 8 and the grid still gives every CU a workgroup (a small
    CU count in the config reaches that at these sizes).  Each head is one
    wave over the same granules in the same order as in the four-head groups
    (decode_kernel 58), so the outputs match those bit for bit, and the
    oracle within the usual bounds; edge lengths as above."""
    lens = (0, 1, 2, 3, 31, 32, 33, 127, 128, 129, 1000)
    for q_len, h_q, h_k in ((1, 32, 8), (2, 16, 8), (4, 8, 8), (2, 32, 8), (4, 32, 8), (1, 64, 16)):
        wl = synth.build(synth.spec_for("cfg3_e2m1", small=True, b=len(lens), lens=lens, lens_loguniform=(),
                                        q_len=q_len, h_q=h_q, h_k=h_k, causal=True, k_outliers=0,
                                        slots_override=0), gpu)
        say(f"  e2m1 eight-head groups q_len={q_len} h_q={h_q} h_k={h_k}")
        out8, lse8, _ = _run(mj, wl, num_cus=2, **FINE)
        out4, lse4, _ = _run(mj, wl, num_cus=2, decode_kernel=58, **FINE)
        O, LSE = oracle_step(wl)
        compare_out(out8, O, f"e2m1 eight-head q_len={q_len} h_q={h_q} h_k={h_k}")
        compare_lse(lse8, LSE, f"e2m1 eight-head q_len={q_len} h_q={h_q} h_k={h_k}")
        assert torch.equal(out8.view(torch.int16), out4.view(torch.int16))
        assert torch.equal(lse8, lse4)


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
def test_edge_lengths(mj, gpu, variant):
    # empty (padding) request, a single token, a length inside the first
    # page, tile boundaries +-1, and causal rows that see no key (L < q_len)
    wl = synth.build(synth.spec_for("cfg4c", small=True, b=7, lens=(0, 1, 2, 127, 128, 129, 3001)), gpu)
    say(f"edges {wl.spec.name} lens={wl.seq_lens}")
    out, lse, _ = _run(mj, wl, **FINE)
    O, LSE = oracle_step(wl)
    compare_out(out, O, "edges")
    compare_lse(lse, LSE, "edges")
    assert torch.all(out[:4].float() == 0)  # L = 0: every row empty
    wl = synth.build(synth.spec_for("cfg2", small=True, b=3, lens=(0, 1, 17)), gpu)
    out, lse, _ = _run(mj, wl, **FINE)
    O, LSE = oracle_step(wl)
    compare_out(out, O, "edges q_len=1")
    compare_lse(lse, LSE, "edges q_len=1")
    # speculative blocks: q_len*h_r of 4 (replicated rows), 8, 16, 15 and 32
    lens = (0, 1, 2, 3, 31, 32, 33, 127, 128, 129, 1000)
    for q_len, h_q, h_k, causal in ((2, 16, 8, True), (4, 8, 8, True), (4, 8, 8, False), (2, 4, 2, False),
                                    (2, 32, 8, True), (4, 32, 8, True), (3, 40, 8, True), (4, 64, 8, False)):
        wl = synth.build(synth.spec_for("cfg2", small=True, b=len(lens), lens=lens, q_len=q_len, h_q=h_q, h_k=h_k,
                                        causal=causal, k_outliers=0), gpu)
        say(f"  edges q_len={q_len} h_q={h_q} h_k={h_k} causal={causal}")
        out, lse, _ = _run(mj, wl, **FINE)
        O, LSE = oracle_step(wl)
        compare_out(out, O, f"edges q_len={q_len} causal={causal}")
        compare_lse(lse, LSE, f"edges q_len={q_len} causal={causal}")


def test_strided_q_view(mj, gpu):
    wl = synth.build(synth.spec_for("cfg2", small=True, q_extra_heads=16), gpu)
    say(f"strided Q {wl.spec.name} q.stride={wl.q.stride()}")
    out, lse, _ = _run(mj, wl, **FINE)
    O, LSE = oracle_step(wl)
    compare_out(out, O, "strided q")
    out, lse, _ = _run(mj, wl, fused=True, **FINE)
    O, LSE = oracle_step(wl)
    compare_out(out, O, "strided q")


def test_graph_replay_after_replanning(mj, gpu):
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for("cfg4c", small=True), gpu)
    say(f"graph replay {wl.spec.name}")
    step = DecodeStep.for_workload(wl, **FINE)
    info = step.plan_workload(wl)
    out, lse = new_output(wl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run_workload(wl, out, lse, info=info)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run_workload(wl, out, lse, info=info)
    torch.cuda.synchronize()
    orig = list(wl.seq_lens)
    rng = np.random.default_rng(5)
    for trial in range(4):
        lens = [int(x) for x in rng.integers(1, np.array(orig) + 1)]
        wl.seq_lens = lens
        wl.seq_lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        new_info = step.plan_workload(wl)
        assert new_info.num_work == info.num_work and new_info.with_reduction == info.with_reduction
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        O, LSE = oracle_step(wl)
        compare_out(out, O, f"replay {trial} lens={lens}")
        compare_lse(lse, LSE, f"replay {trial}")


FULL = {"cfg1": 1, "cfg2": 2, "cfg3": 2, "cfg4c": 2, "cfg4n": 2, "cfg5": 2, "cfg5_e3m2": 1, "cfg5_e2m1": 1,
        "cfg5_nvfp4": 1, "cfg3_nvfp4": 2, "cfg3_e2m3": 2, "cfg3_e2m1": 2, "32k": 2, "32k_b16": 2}


@pytest.mark.parametrize("key", list(FULL))
def test_parity_full_size_sampled(mj, gpu, key, variant):
    """Full-size workloads in the bench's launch configuration (default plan,
    fused step); the oracle checks every output row of a few sampled
    (sequence, KV head) pairs."""
    wl = synth.build(synth.spec_for(key), gpu)
    s = wl.spec
    say(f"full {s.name}: b={s.b} kv_bytes={wl.kv_bytes()}")
    out, lse, info = _run(mj, wl, fused=True)
    say(f"  plan: work={info.num_work} slots={info.slots} chunk_tiles={info.chunk_tiles} "
        f"reduction={info.with_reduction}")
    rng = np.random.default_rng(17)
    lens = np.array(wl.seq_lens)
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), *rng.choice(s.b, size=min(s.b, FULL[key]) , replace=False).tolist()})
    heads = sorted({0, s.h_k - 1})
    O, LSE = oracle_step(wl, seqs=seqs, heads=heads)
    compare_out(out, O, f"{s.name} seqs={seqs} heads={heads}")
    compare_lse(lse, LSE, s.name)


def test_device_plan_bit_exact(mj, gpu):
    """The device planner writes the same plan image as the host planner."""
    rng = np.random.default_rng(21)
    cases = 0
    for trial in range(40):
        h_k = int(rng.choice([1, 2, 4, 8]))
        h_q = h_k * int(rng.choice([1, 4, 8]))
        mns = int(rng.choice([1, 8, 64, 300, 1500]))
        cfg = mj.mj_config(h_q=h_q, h_k=h_k, page_size=int(rng.choice([16, 32, 64, 128])), max_num_seqs=mns,
                           max_q_len=int(rng.integers(1, 5)), max_splits=int(rng.choice([1, 4, 16, 64])),
                           num_cus=256, wgs_per_cu=int(rng.integers(1, 9)),
                           kv_tile_tokens=int(rng.choice([16, 64, 128, 256])),
                           slots_override=int(rng.choice([0, 0, 24, 700])))
        b = int(rng.integers(1, mns + 1))
        q_len = int(rng.integers(1, cfg.max_q_len + 1))
        lens = rng.integers(0, int(rng.choice([50, 5000, 140000])), size=b).astype(np.int32)
        if trial % 7 == 0:
            lens[:] = 0
        margin = int(rng.integers(0, 6))
        max_blocks = int(-(-int(lens.max()) // cfg.page_size)) + 1
        img, hinfo = mj.mj_plan_compute(cfg, lens, q_len, margin, max_blocks)
        plan = torch.full((img.size,), -7, dtype=torch.int32, device=gpu)
        dinfo = mj.mj_plan_split_kv_device(cfg, torch.from_numpy(lens).to(gpu), b, q_len, margin, max_blocks, plan)
        torch.cuda.synchronize()
        assert np.array_equal(plan.cpu().numpy(), img), f"trial {trial}: b={b} split={hinfo.with_reduction}"
        assert (dinfo.num_work, dinfo.with_reduction, dinfo.slots) == (hinfo.num_work, hinfo.with_reduction,
                                                                       hinfo.slots)
        cases += hinfo.with_reduction
    assert cases > 5


def test_graph_replay_with_device_plan(mj, gpu):
    """One graph holds plan + quantize + decode + merge; replays follow new
    device lengths with no host planning."""
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for("cfg2", small=True), gpu)
    say(f"graph+device plan {wl.spec.name}")
    step = DecodeStep.for_workload(wl, **FINE)
    out, lse = new_output(wl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        info = step.plan_workload_device(wl)
        step.run_workload(wl, out, lse, info=info)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        info = step.plan_workload_device(wl)
        step.run_workload(wl, out, lse, info=info)
    torch.cuda.synchronize()
    orig = list(wl.seq_lens)
    rng = np.random.default_rng(8)
    for trial in range(4):
        lens = [int(x) for x in rng.integers(0, np.array(orig) + 1)]
        wl.seq_lens = lens
        wl.seq_lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        O, LSE = oracle_step(wl)
        compare_out(out, O, f"device-plan replay {trial} lens={lens}")
        compare_lse(lse, LSE, f"device-plan replay {trial}")


@pytest.fixture
def step_merge(mj, request):
    m = getattr(request, "param", 0)
    with step_overrides(step_merge=m):
        yield m


@pytest.mark.parametrize("step_merge", [1, 2], indirect=True)
@pytest.mark.parametrize("variant", [0, 1], indirect=True)
@pytest.mark.parametrize("key", SMALL_KEYS)
def test_fused_step_matches_three_calls(mj, gpu, key, variant, step_merge):
    """mj_decode_step (one launch: in-kernel Q quantization, last-split merge)
    gives the three-call path's outputs bit for bit, call after call (a
    counter left non-zero would skip the next call's merge and leave NaN
    rows), with default and fine splits; with the
    generic kernel (variant 1) it is the three-call fallback."""
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    say(f"fused {wl.spec.name} variant={variant} step_merge={step_merge} lens={wl.seq_lens}")
    for mct in (0, 1):
        step = DecodeStep.for_workload(wl, min_chunk_tokens=mct)
        info = step.plan_workload(wl)
        say(f"  min_chunk_tokens={mct}: chunks={info.num_chunks} reduction={info.with_reduction}")
        ref_o, ref_l = new_output(wl)
        step.run_workload(wl, ref_o, ref_l, info=info)
        out, lse = new_output(wl)
        for rep in range(3):
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            step.run_workload(wl, out, lse, info=info, fused=True)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"mct={mct} rep={rep}"
            assert torch.equal(lse, ref_l), f"mct={mct} rep={rep}"
    O, LSE = oracle_step(wl)
    compare_out(out, O, f"fused {wl.spec.name}")
    compare_lse(lse, LSE, f"fused {wl.spec.name}")


@pytest.mark.parametrize("step_merge", [1, 2], indirect=True)
def test_fused_step_graph_replay(mj, gpu, step_merge):
    """plan (device) + fused step captured once; replays with new device
    lengths match the oracle and the eager fused step, replay after replay."""
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for("cfg3", small=True), gpu)
    say(f"fused graph {wl.spec.name}")
    step = DecodeStep.for_workload(wl, **FINE)
    out, lse = new_output(wl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        info = step.plan_workload_device(wl)
        step.run_workload(wl, out, lse, info=info, fused=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        info = step.plan_workload_device(wl)
        step.run_workload(wl, out, lse, info=info, fused=True)
    torch.cuda.synchronize()
    orig = list(wl.seq_lens)
    rng = np.random.default_rng(12)
    eager_o, eager_l = new_output(wl)
    for trial in range(5):
        lens = [int(x) for x in rng.integers(0, np.array(orig) + 1)]
        wl.seq_lens = lens
        wl.seq_lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step.plan_workload_device(wl)
        step.run_workload(wl, eager_o, eager_l, info=info, fused=True)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_o.view(torch.int16)), f"replay {trial}"
        assert torch.equal(lse, eager_l), f"replay {trial}"
        O, LSE = oracle_step(wl)
        compare_out(out, O, f"fused replay {trial} lens={lens}")
        compare_lse(lse, LSE, f"fused replay {trial}")


@pytest.mark.parametrize("shape", [dict(h_q=32, h_k=8, q_len=1), dict(h_q=64, h_k=8, q_len=4),
                                   dict(h_q=8, h_k=2, q_len=1, kv_format="e2m3"),
                                   dict(h_q=32, h_k=8, q_len=1, kv_format="e2m1")])
def test_plan_in_kernel_matches_host_plan(mj, gpu, shape):
    """mj_decode_step with plan_on_device: the decode workgroups derive their
    items from the device lengths.  Outputs are bit-identical to the step on
    the host plan, and n_splits / split_begin in the plan buffer equal the
    host plan's; batches beyond the in-kernel limit take the device
    planner."""
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    key = {"e2m3": "cfg5", "e2m1": "cfg5_e2m1"}.get(shape.get("kv_format"), "cfg2")
    rng = np.random.default_rng(31 + shape["q_len"])
    for trial, b in enumerate([1, 3, 17, 64, 130, 256, 260]):
        lens = tuple(int(x) for x in rng.integers(0, 700, size=b))
        if trial == 2:
            lens = (0,) * b
        over = dict(b=b, lens=lens, h_q=shape["h_q"], h_k=shape["h_k"], q_len=shape["q_len"], k_outliers=0)
        wl = synth.build(synth.spec_for(key, small=True, **over), gpu)
        for mct in (0, 1):
            step = DecodeStep.for_workload(wl, min_chunk_tokens=mct)
            info = step.plan_workload(wl)
            img, _ = mj.mj_plan_compute(step.cfg, np.array(wl.seq_lens, np.int32), shape["q_len"], 0,
                                        wl.block_table.shape[1])
            ref_o, ref_l = new_output(wl)
            step.run_workload(wl, ref_o, ref_l, info=info, fused=True)
            step.plan_dev.fill_(-5)
            sinfo = step.plan_workload_shape(wl)
            assert (sinfo.num_work, sinfo.with_reduction) == (info.num_work, info.with_reduction)
            out, lse = new_output(wl)
            out.fill_(float("nan"))
            step.run_workload(wl, out, lse, info=sinfo, fused=True, plan_on_device=True)
            torch.cuda.synchronize()
            say(f"  plan-in-kernel {shape} b={b} mct={mct} splits={info.with_reduction} chunk={info.chunk_tiles}")
            assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"b={b} mct={mct}"
            assert torch.equal(lse, ref_l), f"b={b} mct={mct}"
            if info.with_reduction:
                cap_max = (img.size - 2 * step.cfg.max_num_seqs) // 4
                got = step.plan_dev.cpu().numpy()
                ns = slice(4 * cap_max, 4 * cap_max + b)
                sb = slice(4 * cap_max + step.cfg.max_num_seqs, 4 * cap_max + step.cfg.max_num_seqs + b)
                assert np.array_equal(got[ns], img[ns]) and np.array_equal(got[sb], img[sb]), f"b={b}"


def test_plan_in_kernel_graph_replay(mj, gpu):
    """One graph of just the step (planning included) follows new device
    lengths replay after replay."""
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for("cfg3", small=True), gpu)
    say(f"plan-in-kernel graph {wl.spec.name}")
    step = DecodeStep.for_workload(wl, **FINE)
    out, lse = new_output(wl)
    info = step.plan_workload_shape(wl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run_workload(wl, out, lse, info=info, fused=True, plan_on_device=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run_workload(wl, out, lse, info=info, fused=True, plan_on_device=True)
    torch.cuda.synchronize()
    orig = list(wl.seq_lens)
    rng = np.random.default_rng(19)
    for trial in range(5):
        lens = [int(x) for x in rng.integers(0, np.array(orig) + 1)]
        wl.seq_lens = lens
        wl.seq_lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        O, LSE = oracle_step(wl)
        compare_out(out, O, f"plan-in-kernel replay {trial} lens={lens}")
        compare_lse(lse, LSE, f"plan-in-kernel replay {trial}")


@pytest.mark.parametrize("key", ["cfg2", "cfg3", "cfg4c", "cfg5", "cfg5_e2m1", "cfg3_nvfp4"])
def test_grid_orders_bit_identical(mj, gpu, key):
    """The matrix-core kernel's three grid numberings (item-major, head-major,
    XCD-grouped with a padded last group) and both prefetch depths give the
    same bits: the order of workgroups changes no arithmetic.  Variants are
    compared within a wave count (the waves of a workgroup share its
    granules, so their number sets the summation order): the default waves
    (10, 12, 14), and four waves (18, 20, 22, and the two-granule prefetch
    11, 15, which runs four)."""
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    O, LSE = oracle_step(wl)
    for family in ((10, 12, 14), (18, 11, 15, 20, 22)):
        ref = None
        for v in family:
            say(f"grid order {wl.spec.name} variant={v}")
            out, lse, info = _run(mj, wl, fused=True, decode_kernel=v, **FINE)
            if ref is None:
                ref = (out, lse)
                compare_out(out, O, f"{key} variant {v}")
                compare_lse(lse, LSE, f"{key} variant {v}")
            else:
                assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), v
                assert torch.equal(lse, ref[1]), v


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("key,q_mode", [("cfg2", "fp8"), ("cfg2", "bf16"), ("cfg4c", "fp8"), ("cfg3", "fp8"),
                                        ("32k_b16", "fp8"), ("cfg5_nvfp4", "fp8"), ("cfg5_nvfp4", "bf16")])
def test_nan_codes_past_the_sequence_end(mj, gpu, key, q_mode, variant):
    """The unused slots of each sequence's last page hold NaN codes (e4m3
    S.1111.111, NaN nvfp4 block scales): a tile that crosses the end must not
    let them into the output (zero probabilities times NaN are NaN)."""
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for(key, small=True, tail_nan=True), gpu)
    say(f"NaN tails {wl.spec.name} q_mode={q_mode} variant={variant} lens={wl.seq_lens}")
    step = DecodeStep.for_workload(wl, q_mode=q_mode, **FINE)
    info = step.plan_workload(wl)
    out, lse = new_output(wl)
    out.fill_(float("nan"))
    step.run_workload(wl, out, lse, info=info, fused=True)
    torch.cuda.synchronize()
    O, LSE = oracle_step(wl, quantize=q_mode == "fp8")
    compare_out(out, O, f"{key} NaN tails")
    compare_lse(lse, LSE, f"{key} NaN tails")


@pytest.mark.parametrize("variant", [0, 1], indirect=True)
@pytest.mark.parametrize("key,q_mode", [("cfg5_nvfp4", "fp8"), ("cfg5_nvfp4", "bf16"), ("cfg3_nvfp4", "fp8")])
def test_nvfp4_full_scale_range(mj, gpu, key, q_mode, variant):
    """Block scales drawn over every finite non-negative e4m3 code (the
    subnormals 2^-9 .. 7 * 2^-9 up to 448) and codes over all 16 e2m1 values
    of both signs: the kernel's fp16 products code x scale must be exact over
    the whole range (smallest 2^-10, largest 2688).  The fp32 descales bring
    logits and outputs back to O(1)."""
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    g = torch.Generator().manual_seed(91)
    for pool in (wl.k_bs_pool, wl.v_bs_pool):
        pool.copy_(torch.randint(0, 0x7F, pool.shape, generator=g, dtype=torch.uint8))
    for pool in (wl.k_pool, wl.v_pool):
        pool.copy_(torch.randint(0, 256, pool.shape, generator=g, dtype=torch.uint8))
    wl.k_descale.fill_(1.0 / 300.0)
    wl.v_descale.fill_(1.0 / 200.0)
    say(f"nvfp4 full scale range {wl.spec.name} q_mode={q_mode} variant={variant}")
    step = DecodeStep.for_workload(wl, q_mode=q_mode, **FINE)
    info = step.plan_workload(wl)
    out, lse = new_output(wl)
    out.fill_(float("nan"))
    step.run_workload(wl, out, lse, info=info, fused=True)
    torch.cuda.synchronize()
    O, LSE = oracle_step(wl, quantize=q_mode == "fp8")
    compare_out(out, O, f"{key} full scale range")
    compare_lse(lse, LSE, f"{key} full scale range")


@pytest.mark.parametrize("variant", [0, 1], indirect=True)
@pytest.mark.parametrize("key", ["cfg5", "cfg5_e3m2", "cfg5_e2m1"])
def test_packed_codes_full_range(mj, gpu, key, variant):
    """Every 6-bit (e2m3, e3m2) or 4-bit (e2m1) code, both signs and the
    largest magnitudes (7.5, 28, 6), as random cache bytes through the
    matrix-core operands and the generic kernel's decoders; the K descale
    keeps the logits moderate."""
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    g = torch.Generator().manual_seed(92)
    for pool in (wl.k_pool, wl.v_pool):
        pool.copy_(torch.randint(0, 256, pool.shape, generator=g, dtype=torch.uint8))
    wl.k_descale.fill_(0.25)
    say(f"full code range {wl.spec.name} variant={variant}")
    out, lse, _ = _run(mj, wl, fused=True, **FINE)
    O, LSE = oracle_step(wl)
    compare_out(out, O, f"{key} full code range")
    compare_lse(lse, LSE, f"{key} full code range")


@pytest.mark.parametrize("variant", VARIANTS, indirect=True)
@pytest.mark.parametrize("key,q_mode", [("cfg2", "fp8"), ("cfg2", "bf16"), ("cfg4c", "fp8")])
def test_e4m3_codes_full_range(mj, gpu, key, q_mode, variant):
    """Every finite e4m3 code (subnormals, both signs, +-448) as random cache
    bytes (the NaN codes replaced by zero), through every decode kernel."""
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    g = torch.Generator().manual_seed(93)
    for pool in (wl.k_pool, wl.v_pool):
        r = torch.randint(0, 256, pool.shape, generator=g, dtype=torch.uint8)
        r[(r & 0x7F) == 0x7F] = 0
        pool.copy_(r)
    wl.k_descale.fill_(0.01)
    wl.v_descale.fill_(0.01)
    say(f"e4m3 full code range {wl.spec.name} q_mode={q_mode} variant={variant}")
    step = DecodeStep.for_workload(wl, q_mode=q_mode, **FINE)
    info = step.plan_workload(wl)
    out, lse = new_output(wl)
    out.fill_(float("nan"))
    step.run_workload(wl, out, lse, info=info, fused=True)
    torch.cuda.synchronize()
    O, LSE = oracle_step(wl, quantize=q_mode == "fp8")
    compare_out(out, O, f"{key} e4m3 full code range")
    compare_lse(lse, LSE, f"{key} e4m3 full code range")

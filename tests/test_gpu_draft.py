"""GPU parity of multi-step draft decoding through the C ABI: the device
advance (mj_draft_advance) bit-exact against the oracle, and a k-step draft
loop -- advance, mj_write_kv of the draft token's K/V rows, mj_decode_step on
one plan made k tokens long -- captured as one hipGraph and replayed: every
step's outputs against the oracle on the grown cache, against the same loop
run eagerly with an exact plan per step, and bit-identical across replays."""

import numpy as np
import pytest
import torch

import synth
from helpers import compare_lse, compare_out, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mj(gpu):
    import paged_fp8_decode_amd as m
    return m


def test_draft_advance_bit_exact(mj, gpu):
    from oracle.draft import draft_advance
    rng = np.random.default_rng(41)
    for P, b, cols, q_len in ((16, 5, 6, 1), (16, 7, 4, 3), (128, 300, 3, 2), (64, 1, 1, 4)):
        bt = rng.permutation(4096)[:b * cols].reshape(b, cols).astype(np.int32)
        cap = cols * P
        lens = rng.integers(0, cap + 1, size=b)
        lens[0] = 0
        if b > 2:
            lens[1], lens[2] = cap, cap - 1
        cfg = mj.mj_config(h_q=8, h_k=2, page_size=P, max_num_seqs=b, max_q_len=q_len, num_cus=256)
        bt_d = torch.from_numpy(bt).to(gpu)
        lens_d = torch.from_numpy(lens.astype(np.int32)).to(gpu)
        slots_d = torch.full((b * q_len,), 12345, dtype=torch.int64, device=gpu)
        say(f"draft advance P={P} b={b} cols={cols} q_len={q_len}")
        mj.mj_draft_advance(cfg, bt_d, lens_d, b, q_len, slots_d)
        torch.cuda.synchronize()
        ref_slots, ref_lens = draft_advance(bt, lens, q_len, P)
        assert np.array_equal(slots_d.cpu().numpy(), ref_slots)
        assert np.array_equal(lens_d.cpu().numpy(), ref_lens)


def _grow_block_table(wl, k):
    """Give every sequence real pages for k more tokens (the workload's spare
    block-table columns point at the shared poison page)."""
    s = wl.spec
    bt = wl.block_table.cpu().numpy()
    used = set(int(x) for x in bt.reshape(-1))
    free = [p for p in range(wl.num_pages) if p not in used]
    for i, L in enumerate(wl.seq_lens):
        if L == 0:
            continue
        have = -(-L // s.page_size)
        need = -(-(L + k) // s.page_size)
        assert need <= bt.shape[1], "the block table needs more spare columns"
        for c in range(have, need):
            bt[i, c] = free.pop()
    wl.block_table.copy_(torch.from_numpy(bt))


def _write_args(mj, wl, key, value, slots):
    ks, vs = wl.kv_strides()
    s = wl.spec
    if s.kv_format in ("e4m3", "nvfp4"):
        kind = wl.descale_kind
        k_sc, v_sc = wl.k_descale, wl.v_descale
    else:
        kind = "channel"
        k_sc, v_sc = wl.k_channel_scale, wl.v_channel_scale
    kk = mj.SCALE_KINDS[kind]
    a = mj.WriteArgs(key=key.data_ptr(), key_tok_stride=key.stride(0), key_head_stride=key.stride(1),
                     value=value.data_ptr(), value_tok_stride=value.stride(0), value_head_stride=value.stride(1),
                     num_tokens=key.shape[0], slot_mapping=slots.data_ptr(),
                     k_cache=wl.k_pool.data_ptr(), k_page_stride=ks[0], k_slot_stride=ks[1], k_head_stride=ks[2],
                     v_cache=wl.v_pool.data_ptr(), v_page_stride=vs[0], v_slot_stride=vs[1], v_head_stride=vs[2],
                     num_pages=wl.num_pages, k_scale=k_sc.data_ptr(), k_scale_kind=kk, v_scale=v_sc.data_ptr(),
                     v_scale_kind=kk)
    if wl.k_bs_pool is not None:
        kb, vb = wl.bs_strides()
        a.k_block_scale, a.v_block_scale = wl.k_bs_pool.data_ptr(), wl.v_bs_pool.data_ptr()
        a.k_bs_page_stride, a.k_bs_slot_stride, a.k_bs_head_stride = kb
        a.v_bs_page_stride, a.v_bs_slot_stride, a.v_bs_head_stride = vb
    return a


@pytest.mark.parametrize("key,q_len", [("cfg2", 1), ("cfg5", 1), ("cfg5_nvfp4", 1), ("cfg2", 4)])
def test_draft_loop_graph_on_one_margin_plan(mj, gpu, key, q_len):
    """q_len = 4: each draft step appends a causal block of four tokens."""
    from oracle.attention import decode_step
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    k = 4
    lens0 = (1000, 2048, 0, 777)  # a padding request stays empty
    wl = synth.build(synth.spec_for(key, small=True, b=4, lens=lens0, extra_bt_cols=2, q_len=q_len), gpu)
    s = wl.spec
    n = s.b * q_len
    _grow_block_table(wl, k * q_len)
    g = torch.Generator(device=gpu)
    g.manual_seed(20260 + len(key))
    kn = (torch.randn((k, n, s.h_k, 128), generator=g, device=gpu) * 1.5).to(torch.bfloat16)
    vn = torch.randn((k, n, s.h_k, 128), generator=g, device=gpu).to(torch.bfloat16)
    qn = torch.randn((k, n, s.h_q, 128), generator=g, device=gpu).to(torch.bfloat16)
    slots = torch.zeros((k, n), dtype=torch.int64, device=gpu)
    step = DecodeStep.for_workload(wl, min_chunk_tokens=1)
    pools0 = [t.clone() for t in (wl.k_pool, wl.v_pool, wl.k_bs_pool, wl.v_bs_pool) if t is not None]
    lens0_d = wl.seq_lens_dev.clone()

    def restore():
        for t, t0 in zip([t for t in (wl.k_pool, wl.v_pool, wl.k_bs_pool, wl.v_bs_pool) if t is not None], pools0):
            t.copy_(t0)
        wl.seq_lens_dev.copy_(lens0_d)

    outs = [new_output(wl) for _ in range(k)]

    def loop(stream, info_per_step=None):
        for st_i in range(k):
            mj.mj_draft_advance(step.cfg, wl.block_table, wl.seq_lens_dev, s.b, q_len, slots[st_i], stream)
            mj.mj_write_kv(step.cfg, _write_args(mj, wl, kn[st_i], vn[st_i], slots[st_i]), stream)
            wl.q = qn[st_i]
            info = info_per_step[st_i] if info_per_step else None
            step.run_workload(wl, outs[st_i][0], outs[st_i][1], info=info, stream=stream, fused=True)

    # one plan, k tokens long, before capture
    margin_info = step.plan(list(lens0), q_len, wl.block_table.shape[1], margin=k * q_len)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop(side)  # warm-up (library and allocator state) outside the capture
    torch.cuda.synchronize()
    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop(torch.cuda.current_stream())
    torch.cuda.synchronize()

    replays = []
    for r in range(3):
        restore()
        for o, l in outs:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replays.append([(o.clone(), l.clone()) for o, l in outs])
        assert wl.seq_lens_dev.cpu().tolist() == [L + k * q_len if L else 0 for L in lens0]
    for r in (1, 2):
        for st_i in range(k):
            assert torch.equal(replays[r][st_i][0].view(torch.int16), replays[0][st_i][0].view(torch.int16))
            assert torch.equal(replays[r][st_i][1], replays[0][st_i][1])

    # oracle: the cache after all k writes holds every step's rows; step i
    # sees lengths L + i + 1, so later rows are masked
    h = wl.host()
    for st_i in range(k):
        hi = dict(h)
        hi["seq_lens"] = np.array([L + (st_i + 1) * q_len if L else 0 for L in lens0], dtype=np.int64)
        hi["q"] = qn[st_i].float().cpu().numpy()
        O, LSE = decode_step(hi, q_len=q_len, h_q=s.h_q, h_k=s.h_k, d=s.d, page_size=s.page_size, kv_format=s.kv_format,
                             causal=s.causal)
        say(f"draft {key} step {st_i}: lens={hi['seq_lens'].tolist()} plan work={margin_info.num_work}")
        compare_out(replays[0][st_i][0], O, f"{key} graph step {st_i}")
        compare_lse(replays[0][st_i][1], LSE, f"{key} graph step {st_i}")

    # the same loop eagerly, planned exactly at every step
    restore()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    for st_i in range(k):
        mj.mj_draft_advance(step.cfg, wl.block_table, wl.seq_lens_dev, s.b, q_len, slots[st_i], st)
        mj.mj_write_kv(step.cfg, _write_args(mj, wl, kn[st_i], vn[st_i], slots[st_i]), st)
        wl.q = qn[st_i]
        info = step.plan([L + (st_i + 1) * q_len if L else 0 for L in lens0], q_len, wl.block_table.shape[1],
                         stream=st)
        step.run_workload(wl, outs[st_i][0], outs[st_i][1], info=info, stream=st, fused=True)
        torch.cuda.synchronize()
        compare_out(outs[st_i][0], replays[0][st_i][0].float().cpu().numpy().astype(np.float64),
                    f"{key} eager exact plan vs graph step {st_i}")

"""Host-side tests of the C-ABI library (no GPU needed): it loads and exports
every symbol include/mj.h declares; the C++ planner equals the oracle's plan
bit for bit; argument validation rejects bad calls before any device work."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import paged_fp8_decode_amd as mj
from oracle import plan as oplan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="fake device pointers: host-validation tests run where no GPU is visible")


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "mj.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:[\w\*\s]+?)\b(mj_\w+)\(", hdr, flags=re.M)))
    assert len(names) >= 12, names
    lib = ctypes.CDLL(mj.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert mj.lib().mj_abi_version() == 9


def _cfg(**kw):
    base = dict(h_q=32, h_k=8, page_size=16, max_num_seqs=64, max_q_len=1, max_splits=16, num_cus=256,
                wgs_per_cu=2, kv_tile_tokens=128)
    base.update(kw)
    return mj.mj_config(**base)


def _oracle(cfg, lens, q_len, margin, max_blocks, info):
    """The oracle's plan rule with the parameters the library reports for
    this plan (workgroups per CU, chunk floor): the rule is the pages', the
    two parameters are the library's tuning, checked on their own below."""
    kv_tile = cfg.kv_tile_tokens or 128
    return oplan.plan_split_kv(lens, q_len=q_len, h_q=cfg.h_q, h_k=cfg.h_k, num_cus=cfg.num_cus,
                               wgs_per_cu=info.wgs_per_cu, kv_tile=kv_tile,
                               max_splits=cfg.max_splits, max_num_seqs=cfg.max_num_seqs,
                               slots_override=cfg.slots_override, margin=margin,
                               min_chunk_tiles=info.min_chunk_tiles, max_len=max_blocks * cfg.page_size)


def _unpack(cfg, img, q_len):
    cap_max = max(mj.mj_plan_capacity(cfg, ql) for ql in range(1, cfg.max_q_len + 1))
    work = img[: 4 * cap_max].reshape(cap_max, 4)
    ns = img[4 * cap_max: 4 * cap_max + cfg.max_num_seqs]
    sb = img[4 * cap_max + cfg.max_num_seqs:]
    return work, ns, sb


def _compare(cfg, lens, q_len, margin=0, max_blocks=1 << 24):
    img, info = mj.mj_plan_compute(cfg, lens, q_len, margin, max_blocks)
    if cfg.wgs_per_cu:
        assert info.wgs_per_cu == cfg.wgs_per_cu
    if cfg.min_chunk_tokens:
        assert info.min_chunk_tiles == -(-cfg.min_chunk_tokens // (cfg.kv_tile_tokens or 128))
    ref = _oracle(cfg, lens, q_len, margin, max_blocks, info)
    work, ns, sb = _unpack(cfg, img, q_len)
    cap = ref["num_work"]
    assert info.num_work == cap
    assert [tuple(int(x) for x in w) for w in work[:cap]] == [tuple(w) for w in ref["work"]]
    assert np.all(work[cap:] == [-1, 0, 0, 0])
    assert ns[: len(lens)].tolist() == ref["n_splits"]
    assert sb[: len(lens)].tolist() == ref["split_begin"]
    assert info.chunk_tiles == ref["chunk_tiles"]
    assert info.slots == ref["slots"]
    assert info.num_chunks == ref["num_chunks"]
    assert bool(info.with_reduction) == ref["with_reduction"]
    # the plan's size fields, known before any length
    shp = mj.mj_plan_shape(cfg, len(lens), q_len, max_blocks)
    assert (shp.num_work, shp.slots, shp.with_reduction, shp.min_chunk_tiles, shp.wgs_per_cu) == \
        (info.num_work, info.slots, info.with_reduction, info.min_chunk_tiles, info.wgs_per_cu)
    return info


@pytest.mark.parametrize("key", ["cfg1", "cfg2", "cfg3", "cfg4c", "cfg5", "32k", "32k_b16"])
def test_planner_matches_oracle_on_workloads(key):
    import synth
    s = synth.spec_for(key)
    lens = synth.workloads._lens(s, np.random.default_rng(s.seed))
    mb = -(-max(lens) // s.page_size) + 3  # a block table a little wider than the longest sequence
    cfg = _cfg(h_q=s.h_q, h_k=s.h_k, page_size=s.page_size, max_num_seqs=s.b, max_q_len=s.q_len,
               slots_override=s.slots_override)
    _compare(cfg, lens, s.q_len, max_blocks=mb)
    # the library's defaults (wgs_per_cu = min_chunk_tokens = 0)
    cfg = _cfg(h_q=s.h_q, h_k=s.h_k, page_size=s.page_size, max_num_seqs=s.b, max_q_len=s.q_len,
               slots_override=s.slots_override, wgs_per_cu=0, kv_format=s.kv_format)
    _compare(cfg, lens, s.q_len, max_blocks=mb)


def test_planner_matches_oracle_random():
    rng = np.random.default_rng(11)
    for _ in range(300):
        h_k = int(rng.choice([1, 2, 4, 8]))
        h_q = h_k * int(rng.choice([1, 2, 4, 8, 16]))
        mq = int(rng.integers(1, 6))
        cfg = _cfg(h_q=h_q, h_k=h_k, max_num_seqs=int(rng.integers(1, 100)), max_q_len=mq,
                   max_splits=int(rng.choice([1, 2, 4, 16, 32])), num_cus=int(rng.choice([20, 80, 256, 304])),
                   wgs_per_cu=int(rng.integers(0, 5)), kv_tile_tokens=int(rng.choice([16, 64, 128, 256])),
                   slots_override=int(rng.choice([0, 0, 0, 7, 300])),
                   min_chunk_tokens=int(rng.choice([0, 0, 1, 100, 2048, 9000])),
                   kv_format=str(rng.choice(["e4m3", "e2m3", "e3m2", "e2m1", "nvfp4"])))
        b = int(rng.integers(1, cfg.max_num_seqs + 1))
        lens = rng.integers(0, int(rng.choice([100, 5000, 200000])), size=b).tolist()
        # block tables from exactly the longest sequence's pages (the margin
        # then reaches past the row) to far wider than any sequence
        need = max(1, -(-max(lens) // cfg.page_size))
        mb = need + int(rng.choice([0, 0, 1, 7, 1000, 1 << 20]))
        _compare(cfg, lens, int(rng.integers(1, mq + 1)), int(rng.integers(0, 300)), mb)


def test_config_errors():
    assert mj.mj_config_check(_cfg()) == mj.MJ_OK
    assert mj.mj_config_check(_cfg(head_dim=64)) == mj.MJ_EUNSUPPORTED
    assert mj.mj_config_check(_cfg(page_size=24)) == mj.MJ_EUNSUPPORTED
    assert mj.mj_config_check(_cfg(page_size=256)) == mj.MJ_EUNSUPPORTED
    assert mj.mj_config_check(_cfg(h_q=30, h_k=8)) == mj.MJ_EUNSUPPORTED
    assert mj.mj_config_check(_cfg(kv_format=5)) == mj.MJ_EUNSUPPORTED
    assert mj.mj_config_check(_cfg(kv_format=-1)) == mj.MJ_EUNSUPPORTED
    for f in ("e2m3", "e3m2", "e2m1", "nvfp4"):
        assert mj.mj_config_check(_cfg(kv_format=f)) == mj.MJ_OK
    assert mj.mj_config_check(_cfg(kv_format="nvfp4", q_mode="bf16")) == mj.MJ_OK
    assert mj.mj_config_check(_cfg(max_num_seqs=0)) == mj.MJ_EINVAL
    assert mj.mj_config_check(_cfg(kv_tile_tokens=100)) == mj.MJ_EINVAL
    assert mj.mj_config_check(_cfg(q_mode="bf16")) == mj.MJ_OK
    assert mj.mj_config_check(_cfg(q_mode=2)) == mj.MJ_EINVAL
    # the packed sub-byte caches take fp8 Q only
    for f in ("e2m3", "e3m2", "e2m1"):
        assert mj.mj_config_check(_cfg(q_mode="bf16", kv_format=f)) == mj.MJ_EUNSUPPORTED
    assert mj.mj_plan_buffer_bytes(_cfg(head_dim=64)) == 0
    assert mj.mj_workspace_bytes(_cfg(page_size=8)) == 0


def test_plan_errors():
    cfg = _cfg(max_num_seqs=4, max_q_len=2)
    with pytest.raises(mj.MjError) as e:
        mj.mj_plan_compute(cfg, [10] * 5, 1)
    assert e.value.status == mj.MJ_ECAPACITY
    with pytest.raises(mj.MjError) as e:
        mj.mj_plan_compute(cfg, [10], 3)
    assert e.value.status == mj.MJ_ECAPACITY
    with pytest.raises(mj.MjError) as e:
        mj.mj_plan_compute(cfg, [10, -1], 1)
    assert e.value.status == mj.MJ_EINVAL
    with pytest.raises(mj.MjError) as e:  # 33 tokens need 3 pages of 16
        mj.mj_plan_compute(cfg, [33], 1, max_blocks_per_seq=2)
    assert e.value.status == mj.MJ_ECAPACITY
    mj.mj_plan_compute(cfg, [32], 1, max_blocks_per_seq=2)


FAKE = 1 << 20  # a 16-byte (and 256-byte) aligned, never dereferenced address


def _args(cfg, **kw):
    # rows of 256 pages (4096 tokens): long enough for a split plan (an
    # invalid config has no plan: any grid, the config check comes first)
    shp = mj.mj_plan_shape(cfg, 4, 1, 256) if mj.mj_config_check(cfg) == mj.MJ_OK else mj.PlanInfo(num_work=1)
    a = dict(q8=FAKE, q_descale=FAKE, num_seqs=4, q_len=1, causal=1, k_cache=FAKE, k_page_stride=16 * 8 * 128,
             k_slot_stride=128, k_head_stride=16 * 128, v_cache=FAKE, v_page_stride=16 * 8 * 128, v_slot_stride=128,
             v_head_stride=16 * 128, num_pages=100, k_descale=FAKE, k_descale_kind=0, v_descale=FAKE,
             v_descale_kind=0, block_table=FAKE, bt_row_stride=256, max_blocks_per_seq=256, seq_lens=FAKE, plan=FAKE,
             num_work=shp.num_work, with_reduction=1, workspace=FAKE, workspace_bytes=mj.mj_workspace_bytes(cfg),
             softmax_scale=0.088, o_mul=None, out=FAKE, out_tok_stride=32 * 128, out_head_stride=128, lse=None)
    a.update(kw)
    return mj.DecodeArgs(**a)


def _decode_status(cfg, **kw):
    return mj.lib().mj_paged_decode(ctypes.byref(cfg), ctypes.byref(_args(cfg, **kw)), None)


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(q8=None), mj.MJ_EINVAL),
    (dict(out=None), mj.MJ_EINVAL),
    (dict(plan=None), mj.MJ_EINVAL),
    (dict(num_seqs=0), mj.MJ_EINVAL),
    (dict(num_seqs=65), mj.MJ_ECAPACITY),
    (dict(q_len=2), mj.MJ_ECAPACITY),
    (dict(num_work=5), mj.MJ_EINVAL),
    (dict(with_reduction=0), mj.MJ_EINVAL),
    (dict(workspace_bytes=1024), mj.MJ_ECAPACITY),
    (dict(workspace=None), mj.MJ_ECAPACITY),
    (dict(k_cache=FAKE + 8), mj.MJ_EALIGN),
    (dict(v_slot_stride=120), mj.MJ_EALIGN),
    (dict(out=FAKE + 2), mj.MJ_EALIGN),
    (dict(out_head_stride=129), mj.MJ_EALIGN),
    (dict(k_descale_kind=3), mj.MJ_EINVAL),
    (dict(num_pages=0), mj.MJ_EINVAL),
    (dict(bt_row_stride=4), mj.MJ_EINVAL),
    (dict(softmax_scale=float("nan")), mj.MJ_EINVAL),
])
def test_decode_argument_errors(kw, status):
    assert _decode_status(_cfg(), **kw) == status


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(q_bf16=None), mj.MJ_EINVAL),
    (dict(q_head_stride=-128), mj.MJ_EINVAL),
    (dict(q_bf16=FAKE + 2), mj.MJ_EALIGN),
    (dict(q_tok_stride=4100), mj.MJ_EALIGN),
    (dict(q_head_stride=130), mj.MJ_EALIGN),
    (dict(out=None), mj.MJ_EINVAL),
])
def test_decode_bf16_q_argument_errors(kw, status):
    base = dict(q8=None, q_descale=None, q_bf16=FAKE, q_tok_stride=32 * 128, q_head_stride=128)
    base.update(kw)
    assert _decode_status(_cfg(q_mode="bf16"), **base) == status


_NV = dict(k_block_scale=FAKE, k_bs_page_stride=16 * 8 * 8, k_bs_slot_stride=8, k_bs_head_stride=16 * 8,
           v_block_scale=FAKE, v_bs_page_stride=16 * 8 * 8, v_bs_slot_stride=8, v_bs_head_stride=16 * 8)


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(k_block_scale=None), mj.MJ_EINVAL),
    (dict(v_block_scale=None), mj.MJ_EINVAL),
    (dict(k_bs_slot_stride=-8), mj.MJ_EINVAL),
    (dict(k_block_scale=FAKE + 4), mj.MJ_EALIGN),
    (dict(v_bs_head_stride=12), mj.MJ_EALIGN),
    (dict(v_bs_page_stride=1020), mj.MJ_EALIGN),
])
def test_decode_nvfp4_block_scale_errors(kw, status):
    a = dict(_NV, k_page_stride=16 * 8 * 64, k_slot_stride=64, k_head_stride=16 * 64, v_page_stride=16 * 8 * 64,
             v_slot_stride=64, v_head_stride=16 * 64)
    a.update(kw)
    assert _decode_status(_cfg(kv_format="nvfp4"), **a) == status


@no_gpu
def test_block_scales_are_not_read_for_other_formats():
    # null block-scale pools are fine outside nvfp4 (the decode then proceeds
    # to its other checks: here a deliberately short workspace)
    assert _decode_status(_cfg(kv_format="e2m1"), k_block_scale=None, workspace_bytes=16) == mj.MJ_ECAPACITY
    assert _decode_status(_cfg(kv_format="nvfp4"), **_NV, workspace_bytes=16) == mj.MJ_ECAPACITY


@no_gpu
def test_step_rejects_q_mul_in_bf16_q_mode():
    cfg = _cfg(q_mode="bf16")
    sa = mj.StepArgs(decode=_args(cfg, q8=None, q_descale=None), q=FAKE, q_tok_stride=32 * 128, q_head_stride=128,
                     q_mul=FAKE)
    assert mj.lib().mj_decode_step(ctypes.byref(cfg), ctypes.byref(sa), None) == mj.MJ_EUNSUPPORTED


@no_gpu
def test_decode_config_errors_come_first():
    assert _decode_status(_cfg(page_size=12)) == mj.MJ_EUNSUPPORTED
    assert mj.lib().mj_paged_decode(ctypes.byref(_cfg()), None, None) == mj.MJ_EINVAL


@no_gpu
def test_quantize_and_merge_errors():
    cfg = _cfg()
    L = mj.lib()
    assert L.mj_quantize_q(ctypes.byref(cfg), None, 4096, 128, None, 4, 1, FAKE, FAKE, None) == mj.MJ_EINVAL
    assert L.mj_quantize_q(ctypes.byref(cfg), FAKE + 2, 4096, 128, None, 4, 1, FAKE, FAKE, None) == mj.MJ_EALIGN
    assert L.mj_quantize_q(ctypes.byref(cfg), FAKE, 4096, 100, None, 4, 1, FAKE, FAKE, None) == mj.MJ_EALIGN
    assert L.mj_quantize_q(ctypes.byref(cfg), FAKE, 4096, 128, None, 65, 1, FAKE, FAKE, None) == mj.MJ_ECAPACITY
    assert L.mj_quantize_q(ctypes.byref(cfg), FAKE, 4096, 128, None, 4, 2, FAKE, FAKE, None) == mj.MJ_ECAPACITY
    m = mj.MergeArgs(plan=FAKE, num_seqs=4, q_len=1, workspace=FAKE, workspace_bytes=10, out=FAKE,
                     out_tok_stride=4096, out_head_stride=128, lse=None)
    assert L.mj_merge_lse(ctypes.byref(cfg), ctypes.byref(m), None) == mj.MJ_ECAPACITY
    m.workspace_bytes = mj.mj_workspace_bytes(cfg)
    m.out = FAKE + 4
    assert L.mj_merge_lse(ctypes.byref(cfg), ctypes.byref(m), None) == mj.MJ_EALIGN
    m.out = FAKE
    m.num_seqs = 0
    assert L.mj_merge_lse(ctypes.byref(cfg), ctypes.byref(m), None) == mj.MJ_EINVAL
    for fmt in (-1, 4, 7, 15, 17):
        assert L.mj_debug_decode_codes(fmt, FAKE, 4, FAKE, None) == mj.MJ_EINVAL
    assert L.mj_debug_decode_codes(0, FAKE, -1, FAKE, None) == mj.MJ_EINVAL


def _wargs(**kw):
    a = dict(key=FAKE, key_tok_stride=8 * 128, key_head_stride=128, value=FAKE, value_tok_stride=8 * 128,
             value_head_stride=128, num_tokens=4, slot_mapping=FAKE, k_cache=FAKE, k_page_stride=16 * 8 * 128,
             k_slot_stride=128, k_head_stride=16 * 128, v_cache=FAKE, v_page_stride=16 * 8 * 128, v_slot_stride=128,
             v_head_stride=16 * 128, num_pages=10, k_scale=FAKE, k_scale_kind=0, v_scale=FAKE, v_scale_kind=0)
    a.update(kw)
    return mj.WriteArgs(**a)


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(key=None), mj.MJ_EINVAL),
    (dict(slot_mapping=None), mj.MJ_EINVAL),
    (dict(num_tokens=-1), mj.MJ_EINVAL),
    (dict(num_pages=0), mj.MJ_EINVAL),
    (dict(k_scale_kind=7), mj.MJ_EINVAL),
    (dict(v_scale_kind=2), mj.MJ_EUNSUPPORTED),
    (dict(key=FAKE + 2), mj.MJ_EALIGN),
    (dict(value_head_stride=100), mj.MJ_EALIGN),
    (dict(k_slot_stride=120), mj.MJ_EALIGN),
    (dict(v_cache=FAKE + 4), mj.MJ_EALIGN),
    (dict(k_head_stride=-16), mj.MJ_EINVAL),
])
def test_write_argument_errors(kw, status):
    cfg = _cfg(max_num_seqs=64)
    assert mj.lib().mj_write_kv(ctypes.byref(cfg), ctypes.byref(_wargs(**kw)), None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(k_block_scale=None), mj.MJ_EINVAL),
    (dict(v_bs_slot_stride=-8), mj.MJ_EINVAL),
    (dict(v_block_scale=FAKE + 2), mj.MJ_EALIGN),
    (dict(k_bs_head_stride=4), mj.MJ_EALIGN),
])
def test_write_nvfp4_block_scale_errors(kw, status):
    cfg = _cfg(max_num_seqs=64, kv_format="nvfp4")
    a = dict(_NV)
    a.update(kw)
    assert mj.lib().mj_write_kv(ctypes.byref(cfg), ctypes.byref(_wargs(**a)), None) == status


def test_write_zero_tokens_needs_no_buffers():
    cfg = _cfg()
    assert mj.lib().mj_write_kv(ctypes.byref(cfg), ctypes.byref(mj.WriteArgs(num_tokens=0)), None) == mj.MJ_OK


def test_kernel_selection_config_values():
    for kw, status in ((dict(decode_kernel=0), mj.MJ_OK), (dict(decode_kernel=1), mj.MJ_OK),
                       (dict(decode_kernel=2), mj.MJ_EINVAL), (dict(decode_kernel=9), mj.MJ_EINVAL),
                       (dict(decode_kernel=10), mj.MJ_OK), (dict(decode_kernel=25), mj.MJ_OK), (dict(decode_kernel=73), mj.MJ_OK),
                       (dict(decode_kernel=74), mj.MJ_EINVAL), (dict(decode_kernel=-1), mj.MJ_EINVAL),
                       (dict(kv_cache_policy=4), mj.MJ_OK), (dict(kv_cache_policy=5), mj.MJ_EINVAL),
                       (dict(kv_cache_policy=-1), mj.MJ_EINVAL), (dict(step_merge=2), mj.MJ_OK),
                       (dict(step_merge=3), mj.MJ_EINVAL), (dict(step_merge=-1), mj.MJ_EINVAL)):
        assert mj.mj_config_check(_cfg(**kw)) == status, kw


@no_gpu
def test_gather_probe_scale_pools_need_nvfp4():
    L = mj.lib()
    for fmt, which, status in (("e4m3", 2, mj.MJ_EINVAL), ("e2m1", 3, mj.MJ_EINVAL), ("nvfp4", 4, mj.MJ_EINVAL),
                               ("e4m3", -1, mj.MJ_EINVAL)):
        cfg = _cfg(kv_format=fmt)
        a = _args(cfg, **_NV)
        assert L.mj_debug_gather_kv(ctypes.byref(cfg), ctypes.byref(a), 0, 0, 16, which, FAKE, None) == status
    cfg = _cfg(kv_format="nvfp4")
    a = _args(cfg, **dict(_NV, k_block_scale=None))
    assert L.mj_debug_gather_kv(ctypes.byref(cfg), ctypes.byref(a), 0, 0, 16, 2, FAKE, None) == mj.MJ_EINVAL


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(block_table=None), mj.MJ_EINVAL),
    (dict(seq_lens=None), mj.MJ_EINVAL),
    (dict(slot_mapping=None), mj.MJ_EINVAL),
    (dict(num_seqs=0), mj.MJ_EINVAL),
    (dict(q_len=0), mj.MJ_EINVAL),
    (dict(bt_row_stride=4), mj.MJ_EINVAL),
    (dict(max_blocks_per_seq=0, bt_row_stride=0), mj.MJ_EINVAL),
    (dict(num_seqs=65), mj.MJ_ECAPACITY),
    (dict(q_len=3), mj.MJ_ECAPACITY),
    (dict(slot_mapping=FAKE + 4), mj.MJ_EALIGN),
])
def test_draft_advance_errors(kw, status):
    cfg = _cfg(max_q_len=2)
    a = dict(block_table=FAKE, bt_row_stride=8, max_blocks_per_seq=8, seq_lens=FAKE, num_seqs=4, q_len=1,
             slot_mapping=FAKE)
    a.update(kw)
    assert mj.lib().mj_draft_advance(ctypes.byref(cfg), ctypes.byref(mj.DraftArgs(**a)), None) == status


@no_gpu
@pytest.mark.parametrize("kw,status,f32", [
    (dict(part_out=None), mj.MJ_EINVAL, 0),
    (dict(part_lse=None), mj.MJ_EINVAL, 0),
    (dict(out=None), mj.MJ_EINVAL, 0),
    (dict(num_parts=0), mj.MJ_EINVAL, 0),
    (dict(num_rows=0), mj.MJ_EINVAL, 0),
    (dict(part_tok_stride=-4), mj.MJ_EINVAL, 0),
    (dict(part_out=FAKE + 4), mj.MJ_EALIGN, 0),
    (dict(part_head_stride=130), mj.MJ_EALIGN, 0),
    (dict(out_head_stride=132), mj.MJ_EALIGN, 0),
    (dict(out_head_stride=130), mj.MJ_EALIGN, 1),
])
def test_combine_errors(kw, status, f32):
    cfg = _cfg(out_f32=f32)
    a = dict(num_parts=8, num_rows=4, part_out=FAKE, part_stride=4 * 32 * 128, part_tok_stride=32 * 128,
             part_head_stride=128, part_lse=FAKE, out=FAKE, out_tok_stride=32 * 128, out_head_stride=128, lse=None)
    a.update(kw)
    assert mj.lib().mj_combine_lse(ctypes.byref(cfg), ctypes.byref(mj.CombineArgs(**a)), None) == status


def test_out_f32_config_values():
    assert mj.mj_config_check(_cfg(out_f32=1)) == mj.MJ_OK
    c = _cfg()
    c.out_f32 = 2
    assert mj.mj_config_check(c) == mj.MJ_EINVAL


# The library's plan parameters when the config leaves wgs_per_cu and
# min_chunk_tokens at 0 (the defaults documented under mj_config in
# include/mj.h).  A tuning choice of the library, not part of the pages'
# method: checked here as a regression of that table, never through the oracle.
@pytest.mark.parametrize("fmt,n_q,wgs,floor_tiles", [
    ("e4m3", 1, 8, 16), ("e4m3", 4, 8, 16), ("e4m3", 16, 8, 16), ("e4m3", 32, 1, 1), ("e4m3", 64, 1, 1),
    ("e2m3", 4, 1, 1), ("e3m2", 16, 1, 1), ("e2m1", 4, 2, 1), ("e2m1", 32, 2, 1), ("e2m1", 40, 1, 1),
    ("nvfp4", 8, 2, 1), ("nvfp4", 64, 1, 1),
])
def test_library_default_plan_parameters(fmt, n_q, wgs, floor_tiles):
    h_k = 8
    q_len = 4 if n_q % 4 == 0 and n_q >= 16 else 1
    cfg = _cfg(h_q=h_k * n_q // q_len, h_k=h_k, max_q_len=q_len, wgs_per_cu=0, kv_format=fmt)
    info = mj.mj_plan_shape(cfg, 1, q_len, 4096)
    assert (info.wgs_per_cu, info.min_chunk_tiles) == (wgs, floor_tiles)


# The default plans of the workloads, worked by hand from the table above
# (256 CUs, 128-token tiles, max 16 splits, block-table rows exactly as long
# as the sequences):
#   cfg1: e4m3 4 rows: S = 256*8/2 = 1024; the 32-page row is 4 tiles <= the
#         16-tile floor: never split, one item, no merge, grid max_num_seqs = 1.
#   cfg2: 32 x 8 workgroups reach all 256 CUs, and the 256-page row (32
#         tiles, 2 chunks of the 16-tile floor) could make at most 64 items
#         x 8 = 512 = two workgroups per CU: one workgroup per CU, S =
#         256/8 = 32 = b: no split, no merge, grid 32.
#   cfg4: 32 rows: S = 256/8 = 32; 64 tiles; 16*ceil(64/c) <= 32 -> c = 32,
#         2 x 16 = 32 items; grid 32.
#   cfg5: e2m3: S = 32; 1024 tiles; 4*ceil(1024/c) <= 32 -> c = 128, 8 x 4.
#   32k:  S = 256; 256 tiles; 64*ceil(256/c) <= 256 -> c = 64, 4 x 64 = 256.
@pytest.mark.parametrize("b,h_q,h_k,q_len,L,P_,fmt,expect", [
    (1, 8, 2, 1, 512, 16, "e4m3", (1024, 4, 1, 1, 0, 1)),
    (32, 32, 8, 1, 4096, 16, "e4m3", (32, 32, 1, 32, 0, 32)),
    (16, 64, 8, 4, 8192, 32, "e4m3", (32, 32, 2, 32, 1, 32)),
    (4, 32, 8, 1, 131072, 128, "e2m3", (32, 128, 8, 32, 1, 32)),
    (64, 32, 8, 1, 32768, 64, "e4m3", (256, 64, 4, 256, 1, 256)),
])
def test_library_default_workload_plans(b, h_q, h_k, q_len, L, P_, fmt, expect):
    cfg = _cfg(h_q=h_q, h_k=h_k, page_size=P_, max_num_seqs=b, max_q_len=q_len, wgs_per_cu=0, kv_format=fmt)
    img, info = mj.mj_plan_compute(cfg, [L] * b, q_len, 0, L // P_)
    work, ns, _ = _unpack(cfg, img, q_len)
    items = int(np.sum(work[:, 0] >= 0))
    assert (info.slots, info.chunk_tiles, int(ns[0]), items, info.with_reduction, info.num_work) == expect


# Batches that already reach every CU plan one workgroup per CU when no split
# their block-table rows allow could make more than two workgroups per CU (a
# split would only add the merge); wider rows, smaller batches and explicit
# settings keep the format's default.
@pytest.mark.parametrize("b,max_blocks,wgs_cfg,expect", [
    # (workgroups per CU, slots, with_reduction, num_work); max_num_seqs 64
    (32, 256, 0, (1, 32, 0, 64)),      # cfg2's shape: 32 x 8 pairs, rows of 4K tokens
    (32, 258, 0, (1, 32, 0, 64)),      # two pages more: a 33rd tile is no third chunk
    (32, 384, 0, (8, 256, 1, 256)),    # rows of 6K tokens: three chunks of the floor
    (32, 2048, 0, (8, 256, 1, 256)),   # rows of 32K tokens: splits can add rounds
    (16, 256, 0, (8, 256, 1, 256)),    # 16 x 8 pairs leave CUs idle
    (64, 256, 0, (8, 256, 1, 256)),    # 64 x 8 pairs in two chunks: four per CU
    (32, 256, 8, (8, 256, 1, 256)),    # wgs_per_cu given: kept
    (32, 16, 0, (1, 32, 0, 64)),       # rows within the chunk floor: never split
])
def test_one_round_batches_do_not_split(b, max_blocks, wgs_cfg, expect):
    cfg = _cfg(h_q=32, h_k=8, page_size=16, max_num_seqs=64, max_q_len=1, wgs_per_cu=wgs_cfg, kv_format="e4m3")
    shp = mj.mj_plan_shape(cfg, b, 1, max_blocks)
    _, info = mj.mj_plan_compute(cfg, [max_blocks * 16] * b, 1, 0, max_blocks)
    got = (info.wgs_per_cu, info.slots, info.with_reduction, info.num_work)
    assert got == (shp.wgs_per_cu, shp.slots, shp.with_reduction, shp.num_work) == expect


@no_gpu
def test_noalloc_step_errors_come_before_any_device_work():
    """mj_decode_step_noalloc rejects caller buffers, a host plan, the
    in-kernel merge and configs beyond its static array on the host."""
    L = mj.lib()
    cfg = _cfg()
    need = mj.mj_noalloc_scratch_bytes(cfg)
    assert 0 < need == -(-mj.mj_plan_buffer_bytes(cfg) // 256) * 256 + mj.mj_workspace_bytes(cfg)
    assert need <= 32 << 20
    ok = dict(plan_on_device=1)
    for kw, status in ((dict(plan_on_device=0), mj.MJ_EINVAL),
                       (dict(ok, decode=mj.DecodeArgs(plan=FAKE)), mj.MJ_EINVAL),
                       (dict(ok, decode=mj.DecodeArgs(workspace=FAKE)), mj.MJ_EINVAL)):
        assert L.mj_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(mj.StepArgs(**kw)), None) == status, kw
    assert L.mj_decode_step_noalloc(ctypes.byref(_cfg(step_merge=1)), ctypes.byref(mj.StepArgs(**ok)),
                                    None) == mj.MJ_EUNSUPPORTED
    big = _cfg(h_q=64, h_k=1, max_num_seqs=4096, max_q_len=16)
    assert mj.mj_noalloc_scratch_bytes(big) > 32 << 20
    assert L.mj_decode_step_noalloc(ctypes.byref(big), ctypes.byref(mj.StepArgs(**ok)), None) == mj.MJ_ECAPACITY
    assert L.mj_decode_step_noalloc(ctypes.byref(_cfg(head_dim=64)), ctypes.byref(mj.StepArgs(**ok)),
                                    None) == mj.MJ_EUNSUPPORTED

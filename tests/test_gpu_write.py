"""GPU parity of the KV-cache write (mj_write_kv) against the oracle: whole
pools compared byte for byte after the write (every KV format, every scale
kind, HND and NHD, strided K/V views, padding and out-of-pool slots,
saturating values), and a written cache decoded end to end."""

import zlib

import numpy as np
import pytest
import torch

from helpers import compare_lse, compare_out, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mj(gpu):
    import paged_fp8_decode_amd as m
    return m


def _strides(layout, P, h_k, row):
    if layout == "HND":
        return (h_k * P * row, row, P * row)
    return (P * h_k * row, h_k * row, row)


def _write(mj, gpu, cfg, key, value, slots, k_pool, v_pool, ks, vs, k_scale, v_scale, kind, num_pages, bs=None):
    # the kernel trusts these sizes: check them before the launch
    assert slots.numel() == key.shape[0] == value.shape[0]
    assert key.shape[1:] == value.shape[1:] == (cfg.h_k, 128)
    row = (128, 96, 96, 64, 64)[cfg.kv_format]
    last = (num_pages - 1) * ks[0] + (cfg.page_size - 1) * ks[1] + (cfg.h_k - 1) * ks[2] + row
    assert last <= k_pool.numel() and last <= v_pool.numel()
    assert (bs is not None) == (cfg.kv_format == mj.KV_FORMATS["nvfp4"])
    if bs is not None:  # (k pool, v pool, k strides, v strides) of the block scales
        for pool, st in ((bs[0], bs[2]), (bs[1], bs[3])):
            assert (num_pages - 1) * st[0] + (cfg.page_size - 1) * st[1] + (cfg.h_k - 1) * st[2] + 8 <= pool.numel()
    need = {"tensor": 1, "head": cfg.h_k, "channel": cfg.h_k * 128}[kind]
    assert k_scale.numel() >= need and v_scale.numel() >= need
    kk = mj.SCALE_KINDS[kind]
    a = mj.WriteArgs(key=key.data_ptr(), key_tok_stride=key.stride(0), key_head_stride=key.stride(1),
                     value=value.data_ptr(), value_tok_stride=value.stride(0), value_head_stride=value.stride(1),
                     num_tokens=key.shape[0], slot_mapping=slots.data_ptr(),
                     k_cache=k_pool.data_ptr(), k_page_stride=ks[0], k_slot_stride=ks[1], k_head_stride=ks[2],
                     v_cache=v_pool.data_ptr(), v_page_stride=vs[0], v_slot_stride=vs[1], v_head_stride=vs[2],
                     num_pages=num_pages, k_scale=k_scale.data_ptr(), k_scale_kind=kk, v_scale=v_scale.data_ptr(),
                     v_scale_kind=kk)
    if bs is not None:
        a.k_block_scale, a.v_block_scale = bs[0].data_ptr(), bs[1].data_ptr()
        a.k_bs_page_stride, a.k_bs_slot_stride, a.k_bs_head_stride = bs[2]
        a.v_bs_page_stride, a.v_bs_slot_stride, a.v_bs_head_stride = bs[3]
    mj.mj_write_kv(cfg, a)
    torch.cuda.synchronize()


@pytest.mark.parametrize("kv_format,kind", [("e4m3", "tensor"), ("e4m3", "head"), ("e4m3", "channel"),
                                            ("e2m3", "channel"), ("e2m3", "head"), ("e3m2", "channel"),
                                            ("e3m2", "tensor"), ("e2m1", "channel"), ("e2m1", "head"),
                                            ("nvfp4", "tensor"), ("nvfp4", "head"), ("nvfp4", "channel")])
@pytest.mark.parametrize("layout", ["HND", "NHD"])
@pytest.mark.parametrize("P", [16, 128])
def test_write_bytes_match_oracle(mj, gpu, kv_format, kind, layout, P):
    from oracle.formats import FMT_MAX, ROW_BYTES
    from oracle.kvwrite import write_kv
    say(f"write {kv_format} {kind} {layout} P={P}")
    rng = np.random.default_rng(zlib.crc32(f"{kv_format}{kind}{layout}{P}".encode()))
    h_k, n = 4, 300
    pages = max(9, -(-2 * n // P))  # at least two slots per token
    row = ROW_BYTES[kv_format]
    ks = vs = _strides(layout, P, h_k, row)
    size = pages * P * h_k * row
    init_k = rng.integers(0, 256, size, dtype=np.uint8)
    init_v = rng.integers(0, 256, size, dtype=np.uint8)
    # K and V as strided views of one fused buffer (token stride 3 heads wider)
    fused = torch.from_numpy(rng.standard_normal((n, 2 * h_k + 2, 128)).astype(np.float32) * 2).to(torch.bfloat16)
    special = torch.tensor([0, -0.0, 1e4, -1e4, 1e-30, -1e-30, 3.0, -2.5, 0.1, -0.0])  # zeros, saturation, tiny
    fused[1, 0, :10] = special  # token 1 of K and token 2 of V are written (not padding)
    fused[2, h_k + 1, 118:] = special
    key, value = fused[:, :h_k], fused[:, h_k + 1:2 * h_k + 1]
    fmax = FMT_MAX.get(kv_format, 6.0 * 448.0)  # nvfp4: e2m1 max times e4m3 max
    amax_k = key.float().abs().amax(dim=0).numpy()  # (h_k, 128); saturating rows stay rare
    amax_v = value.float().abs().amax(dim=0).numpy()
    if kind == "tensor":
        k_sc = np.array([np.median(amax_k) / fmax], np.float32)
        v_sc = np.array([np.median(amax_v) / fmax], np.float32)
    elif kind == "head":
        k_sc = (np.median(amax_k, axis=1) / fmax).astype(np.float32)
        v_sc = (np.median(amax_v, axis=1) / fmax).astype(np.float32)
    else:
        k_sc = (amax_k / fmax * 0.9).astype(np.float32)
        v_sc = (amax_v / fmax * 0.9).astype(np.float32)
    slots = rng.permutation(pages * P)[:n].astype(np.int64)
    assert slots.shape == (n,)  # one slot per token: the kernel reads num_tokens entries
    slots[::17] = -1  # padding tokens (not tokens 1 and 2)
    num_pages = pages - 1
    slots[3] = (pages - 1) * P + 2  # in the last page: past num_pages, skipped
    k_pool = torch.from_numpy(init_k.copy()).to(gpu)
    v_pool = torch.from_numpy(init_v.copy()).to(gpu)
    bs = bs_np = None
    if kv_format == "nvfp4":
        bst = _strides(layout, P, h_k, 8)
        init_kb = rng.integers(0, 256, pages * P * h_k * 8, dtype=np.uint8)
        init_vb = rng.integers(0, 256, pages * P * h_k * 8, dtype=np.uint8)
        bs = (torch.from_numpy(init_kb.copy()).to(gpu), torch.from_numpy(init_vb.copy()).to(gpu), bst, bst)
        bs_np = dict(bs_pools=(init_kb, init_vb), bs_strides=(bst, bst))
    cfg = mj.mj_config(h_q=h_k, h_k=h_k, page_size=P, max_num_seqs=1, kv_format=kv_format, num_cus=256)
    _write(mj, gpu, cfg, key.to(gpu), value.to(gpu), torch.from_numpy(slots).to(gpu), k_pool, v_pool, ks, vs,
           torch.from_numpy(k_sc).to(gpu), torch.from_numpy(v_sc).to(gpu), kind, num_pages, bs)
    ref = write_kv((init_k, init_v), (ks, vs), P, kv_format, key.float().numpy(), value.float().numpy(),
                   slots, k_sc, v_sc, kind, num_pages=num_pages, **(bs_np or {}))
    assert np.array_equal(k_pool.cpu().numpy(), ref[0])
    assert np.array_equal(v_pool.cpu().numpy(), ref[1])
    if bs is not None:
        assert np.array_equal(bs[0].cpu().numpy(), ref[2])
        assert np.array_equal(bs[1].cpu().numpy(), ref[3])


def test_write_zero_tokens_is_a_noop(mj, gpu):
    cfg = mj.mj_config(h_q=8, h_k=2, page_size=16, max_num_seqs=1, num_cus=256)
    a = mj.WriteArgs(num_tokens=0)
    mj.mj_write_kv(cfg, a)


@pytest.mark.parametrize("key", ["cfg2", "cfg3", "cfg5", "cfg5_e3m2", "cfg5_e2m1", "cfg5_nvfp4", "cfg3_nvfp4"])
def test_written_cache_decodes(mj, gpu, key):
    """Blank every token row of a seeded workload's cache, re-write them with
    mj_write_kv from the dequantized K/V (code * scale in bf16: dividing by
    the scale lands within 2^-9 of the code, which rounds back to it; an
    nvfp4 block holds a +-6 code, so its amax / 6 lands as close to its
    block scale), and check the pools are byte-identical to the generator's;
    then decode."""
    import synth
    from helpers import oracle_step
    from oracle import formats as F
    from oracle.attention import gather_codes
    from paged_fp8_decode_amd.runner import DecodeStep, new_output
    wl = synth.build(synth.spec_for(key, small=True), gpu)
    s = wl.spec
    say(f"write+decode {s.name}")
    h = wl.host()
    ks, vs = wl.kv_strides()
    row = s.row_bytes
    nv = s.kv_format == "nvfp4"
    if s.kv_format in ("e4m3", "nvfp4"):
        kind = "head" if wl.descale_kind == "head" else ("tensor" if wl.descale_kind == "tensor" else None)
        if kind is None:  # per-(sequence, head) descales have no slot-mapped write form
            pytest.skip("per-(sequence, head) scales are a decode-side shape only")
        k_sc = wl.k_descale.cpu().numpy().astype(np.float32).reshape(-1)
        v_sc = wl.v_descale.cpu().numpy().astype(np.float32).reshape(-1)
    else:
        kind = "channel"
        k_sc = wl.k_channel_scale.cpu().numpy().astype(np.float32).reshape(-1)
        v_sc = wl.v_channel_scale.cpu().numpy().astype(np.float32).reshape(-1)
    n = sum(wl.seq_lens)
    kx = np.zeros((n, s.h_k, 128), np.float32)
    vx = np.zeros((n, s.h_k, 128), np.float32)
    slots = np.zeros(n, np.int64)
    mask = torch.zeros(wl.k_pool.numel(), dtype=torch.bool)
    bmask = torch.zeros(wl.k_bs_pool.numel() if nv else 1, dtype=torch.bool)
    bss = wl.bs_strides() if nv else None
    base = 0
    for i in range(s.b):
        L = wl.seq_lens[i]
        bt = h["block_table"][i]
        for j in range(L):
            page = int(bt[j // s.page_size])
            slots[base + j] = page * s.page_size + j % s.page_size
            for g in range(s.h_k):
                b = page * ks[0] + (j % s.page_size) * ks[1] + g * ks[2]
                mask[b:b + row] = True
                if nv:
                    b = page * bss[0][0] + (j % s.page_size) * bss[0][1] + g * bss[0][2]
                    bmask[b:b + 8] = True
        for g in range(s.h_k):
            for side, pool, st, dst, sc in ((0, h["k_pool"], h["k_strides"], kx, k_sc),
                                            (1, h["v_pool"], h["v_strides"], vx, v_sc)):
                codes = gather_codes(pool, st, s.page_size, bt, L, g, row)
                if nv:
                    bp, bst = (h["k_bs_pool"], h["k_bs_strides"]) if side == 0 else (h["v_bs_pool"], h["v_bs_strides"])
                    vals = F.nvfp4_decode(codes, gather_codes(bp, bst, s.page_size, bt, L, g, 8))
                else:
                    vals = F.decode_row_codes(codes, s.kv_format)
                div = sc[0] if kind == "tensor" else (sc[g] if kind == "head" else sc.reshape(-1, 128)[g])
                dst[base:base + L, g] = vals * div
        base += L
    assert ks == vs
    before_k, before_v = wl.k_pool.clone(), wl.v_pool.clone()
    m = mask.to(gpu)
    wl.k_pool.view(-1)[m] = 0
    wl.v_pool.view(-1)[m] = 0
    bs = None
    if nv:
        assert bss[0] == bss[1]
        before_kb, before_vb = wl.k_bs_pool.clone(), wl.v_bs_pool.clone()
        bm = bmask.to(gpu)
        wl.k_bs_pool.view(-1)[bm] = 0
        wl.v_bs_pool.view(-1)[bm] = 0
        bs = (wl.k_bs_pool, wl.v_bs_pool, bss[0], bss[1])
    cfg = mj.mj_config(h_q=s.h_q, h_k=s.h_k, page_size=s.page_size, max_num_seqs=s.b, kv_format=s.kv_format,
                       num_cus=256)
    _write(mj, gpu, cfg, torch.from_numpy(kx).to(torch.bfloat16).to(gpu),
           torch.from_numpy(vx).to(torch.bfloat16).to(gpu), torch.from_numpy(slots).to(gpu), wl.k_pool, wl.v_pool,
           ks, vs, torch.from_numpy(k_sc).to(gpu), torch.from_numpy(v_sc).to(gpu), kind, wl.num_pages, bs)
    assert torch.equal(wl.k_pool, before_k) and torch.equal(wl.v_pool, before_v)
    if nv:
        assert torch.equal(wl.k_bs_pool, before_kb) and torch.equal(wl.v_bs_pool, before_vb)
    step = DecodeStep.for_workload(wl, min_chunk_tokens=1)
    info = step.plan_workload(wl)
    out, lse = new_output(wl)
    step.run_workload(wl, out, lse, info=info, fused=True)
    torch.cuda.synchronize()
    O, LSE = oracle_step(wl)
    compare_out(out, O, f"written {s.name}")
    compare_lse(lse, LSE, f"written {s.name}")


@pytest.mark.parametrize("kv_format", ["e4m3", "e2m3", "e3m2", "e2m1"])
def test_write_ties_and_grid_points(mj, gpu, kv_format):
    """Every value of the format's grid, every midpoint between neighbours
    (ties to even) and values just inside and outside each midpoint, both
    signs, through the write at unit scale: the stored bytes equal the
    oracle's (all these inputs are exact in bf16)."""
    from oracle import formats as F
    from oracle.kvwrite import write_kv
    table = {"e4m3": F.E4M3_TABLE[:0x7F], "e2m3": F.E2M3_TABLE[:0x20], "e3m2": F.E3M2_TABLE[:0x20],
             "e2m1": F.E2M1_TABLE[:0x8]}[kv_format]
    grid = np.unique(table)
    mids = (grid[:-1] + grid[1:]) / 2
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(np.inf))])
    vals = np.concatenate([grid, mids, grid[-1:] * 1.25])  # the last: saturates
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    bf = torch.from_numpy(vals).to(torch.bfloat16)
    assert torch.equal(bf.float(), torch.from_numpy(vals)), "grid points and midpoints are exact in bf16"
    # nextafter of a midpoint is not a bf16 value: round it to bf16 and keep the ones still off the midpoint
    nb = torch.from_numpy(near).to(torch.bfloat16).float().numpy()
    nb = nb[~np.isin(nb, mids)]
    allv = torch.cat([bf, torch.from_numpy(np.concatenate([nb, -nb])).to(torch.bfloat16)])
    h_k, d = 2, 128
    n = -(-allv.numel() // (h_k * d)) + 1
    flat = torch.zeros(n * h_k * d, dtype=torch.bfloat16)
    flat[: allv.numel()] = allv
    key = flat.view(n, h_k, d)
    value = flat.flip(0).view(n, h_k, d).contiguous()
    P, layout = 16, "HND"
    pages = -(-n // P) + 1
    row = F.ROW_BYTES[kv_format]
    ks = vs = _strides(layout, P, h_k, row)
    size = pages * P * h_k * row
    rng = np.random.default_rng(5)
    init_k = rng.integers(0, 256, size, dtype=np.uint8)
    init_v = rng.integers(0, 256, size, dtype=np.uint8)
    slots = np.arange(n, dtype=np.int64)
    ones = np.ones((h_k, d), np.float32)
    k_pool = torch.from_numpy(init_k.copy()).to(gpu)
    v_pool = torch.from_numpy(init_v.copy()).to(gpu)
    say(f"write ties {kv_format}: {allv.numel()} values over {n} tokens")
    cfg = mj.mj_config(h_q=h_k, h_k=h_k, page_size=P, max_num_seqs=1, kv_format=kv_format, num_cus=256)
    _write(mj, gpu, cfg, key.to(gpu), value.to(gpu), torch.from_numpy(slots).to(gpu), k_pool, v_pool, ks, vs,
           torch.from_numpy(ones).to(gpu), torch.from_numpy(ones).to(gpu), "channel", pages)
    ref = write_kv((init_k, init_v), (ks, vs), P, kv_format, key.float().numpy(), value.float().numpy(),
                   slots, ones, ones, "channel")
    assert np.array_equal(k_pool.cpu().numpy(), ref[0])
    assert np.array_equal(v_pool.cpu().numpy(), ref[1])


def test_write_nvfp4_ties(mj, gpu):
    """nvfp4 blocks whose amax is 6 (block scale exactly 1) holding every
    e2m1 grid value and every midpoint (ties to even), both signs, and blocks
    whose amax / 6 is itself an e4m3 midpoint (the scale's own tie): codes
    and scale bytes equal the oracle's."""
    from oracle import formats as F
    from oracle.kvwrite import write_kv
    grid = np.unique(F.E2M1_TABLE[:0x8])
    mids = (grid[:-1] + grid[1:]) / 2
    body = np.concatenate([grid, mids, -grid, -mids]).astype(np.float32)  # 28 values
    e4 = np.unique(F.E4M3_TABLE[:0x7F])
    e4mid = (e4[:-1] + e4[1:]) / 2  # amax = 6 * e4mid: the block scale ties
    h_k, d, P = 2, 128, 16
    blocks = []
    for k in range(0, len(body), 15):
        b = np.zeros(16, np.float32)
        b[0] = 6.0
        chunk = body[k:k + 15]
        b[1:1 + len(chunk)] = chunk
        blocks.append(b)
    for m in e4mid[::5]:
        b = np.zeros(16, np.float32)
        b[0] = 6.0 * m
        b[1:8] = np.float32(m) * grid[1:]
        blocks.append(b)
    flat = np.concatenate(blocks)
    n = -(-flat.size // (h_k * d)) + 1
    buf = np.zeros(n * h_k * d, np.float32)
    buf[:flat.size] = flat
    kt = torch.from_numpy(buf).to(torch.bfloat16)
    keep = kt.float().numpy() == buf  # values not exact in bf16 would not be ties: drop them
    buf[~keep] = 0.0
    key = torch.from_numpy(buf).to(torch.bfloat16).view(n, h_k, d)
    value = key.flip(0).contiguous()
    pages = -(-n // P) + 1
    row = F.ROW_BYTES["nvfp4"]
    ks = vs = _strides("HND", P, h_k, row)
    bst = _strides("HND", P, h_k, 8)
    rng = np.random.default_rng(6)
    init_k = rng.integers(0, 256, pages * P * h_k * row, dtype=np.uint8)
    init_v = rng.integers(0, 256, pages * P * h_k * row, dtype=np.uint8)
    init_kb = rng.integers(0, 256, pages * P * h_k * 8, dtype=np.uint8)
    init_vb = rng.integers(0, 256, pages * P * h_k * 8, dtype=np.uint8)
    k_pool = torch.from_numpy(init_k.copy()).to(gpu)
    v_pool = torch.from_numpy(init_v.copy()).to(gpu)
    bs = (torch.from_numpy(init_kb.copy()).to(gpu), torch.from_numpy(init_vb.copy()).to(gpu), bst, bst)
    slots = np.arange(n, dtype=np.int64)
    ones = np.ones((h_k, d), np.float32)
    say(f"write nvfp4 ties: {len(blocks)} blocks over {n} tokens")
    cfg = mj.mj_config(h_q=h_k, h_k=h_k, page_size=P, max_num_seqs=1, kv_format="nvfp4", num_cus=256)
    _write(mj, gpu, cfg, key.to(gpu), value.to(gpu), torch.from_numpy(slots).to(gpu), k_pool, v_pool, ks, vs,
           torch.from_numpy(ones).to(gpu), torch.from_numpy(ones).to(gpu), "channel", pages, bs)
    ref = write_kv((init_k, init_v), (ks, vs), P, "nvfp4", key.float().numpy(), value.float().numpy(), slots,
                   ones, ones, "channel", bs_pools=(init_kb, init_vb), bs_strides=(bst, bst))
    assert np.array_equal(k_pool.cpu().numpy(), ref[0])
    assert np.array_equal(v_pool.cpu().numpy(), ref[1])
    assert np.array_equal(bs[0].cpu().numpy(), ref[2])
    assert np.array_equal(bs[1].cpu().numpy(), ref[3])


@pytest.mark.parametrize("kv_format,kind,n", [("e2m3", "channel", 16387), ("e4m3", "channel", 16386),
                                              ("e2m1", "channel", 2049), ("nvfp4", "channel", 2051),
                                              ("e3m2", "head", 16385)])
def test_large_write_matches_oracle_on_sampled_tokens(mj, gpu, kv_format, kind, n):
    """A write large enough to give each thread several tokens (8 KV heads,
    thousands of tokens, a token count that leaves a ragged last group),
    with padding and out-of-pool slots: the rows of a sample of tokens (the
    first, the last group and random ones) equal the oracle's bytes, and
    every row no token maps to is untouched."""
    from oracle.formats import FMT_MAX, ROW_BYTES
    from oracle.kvwrite import write_kv
    say(f"large write {kv_format} {kind} n={n}")
    rng = np.random.default_rng(zlib.crc32(f"large{kv_format}{kind}{n}".encode()))
    h_k, P = 8, 16
    pages = -(-(n + n // 4) // P) + 1
    row = ROW_BYTES[kv_format]
    ks = vs = _strides("NHD", P, h_k, row)
    size = pages * P * h_k * row
    init_k = rng.integers(0, 256, size, dtype=np.uint8)
    init_v = rng.integers(0, 256, size, dtype=np.uint8)
    key = torch.from_numpy(rng.standard_normal((n, h_k, 128)).astype(np.float32)).to(torch.bfloat16)
    value = torch.from_numpy(rng.standard_normal((n, h_k, 128)).astype(np.float32) * 3).to(torch.bfloat16)
    fmax = FMT_MAX.get(kv_format, 6.0 * 448.0)
    if kind == "channel":
        k_sc = (rng.uniform(2.0, 4.0, (h_k, 128)) / fmax).astype(np.float32)
        v_sc = (rng.uniform(6.0, 12.0, (h_k, 128)) / fmax).astype(np.float32)
    else:
        k_sc = (rng.uniform(2.0, 4.0, h_k) / fmax).astype(np.float32)
        v_sc = (rng.uniform(6.0, 12.0, h_k) / fmax).astype(np.float32)
    slots = rng.permutation(pages * P)[:n].astype(np.int64)
    slots[5::23] = -1
    num_pages = pages - 1
    slots[n - 2] = (pages - 1) * P + 1  # in the last group, past num_pages: skipped
    bs = bs_np = None
    if kv_format == "nvfp4":
        bst = _strides("NHD", P, h_k, 8)
        init_kb = rng.integers(0, 256, pages * P * h_k * 8, dtype=np.uint8)
        init_vb = rng.integers(0, 256, pages * P * h_k * 8, dtype=np.uint8)
        bs = (torch.from_numpy(init_kb.copy()).to(gpu), torch.from_numpy(init_vb.copy()).to(gpu), bst, bst)
    k_pool = torch.from_numpy(init_k.copy()).to(gpu)
    v_pool = torch.from_numpy(init_v.copy()).to(gpu)
    cfg = mj.mj_config(h_q=h_k, h_k=h_k, page_size=P, max_num_seqs=1, kv_format=kv_format, num_cus=256)
    _write(mj, gpu, cfg, key.to(gpu), value.to(gpu), torch.from_numpy(slots).to(gpu), k_pool, v_pool, ks, vs,
           torch.from_numpy(k_sc).to(gpu), torch.from_numpy(v_sc).to(gpu), kind, num_pages, bs)
    got = [k_pool.cpu().numpy(), v_pool.cpu().numpy()]
    if bs is not None:
        got += [bs[0].cpu().numpy(), bs[1].cpu().numpy()]
    sample = np.unique(np.concatenate([np.arange(8), np.arange(n - 9, n), rng.choice(n, 120, replace=False)]))
    if bs is not None:
        bs_np = dict(bs_pools=(init_kb, init_vb), bs_strides=(bst, bst))
    ref = write_kv((init_k, init_v), (ks, vs), P, kv_format, key[sample].float().numpy(),
                   value[sample].float().numpy(), slots[sample], k_sc, v_sc, kind, num_pages=num_pages,
                   **(bs_np or {}))
    inits = [init_k, init_v] + ([init_kb, init_vb] if bs is not None else [])
    others = np.setdiff1d(np.arange(n), sample)
    others = others[(slots[others] >= 0) & (slots[others] // P < num_pages)]
    # the row bytes of the tokens outside the sample are not compared; every other byte is
    for which, (g_, r_, i_) in enumerate(zip(got, ref, inits)):
        st, nb = ((ks, row), (vs, row), (bs[2], 8) if bs else None, (bs[3], 8) if bs else None)[which]
        base = (slots[others] // P) * st[0] + (slots[others] % P) * st[1]
        idx = base[:, None, None] + np.arange(h_k)[None, :, None] * st[2] + np.arange(nb)[None, None, :]
        skip = np.zeros(g_.size, bool)
        skip[idx.reshape(-1)] = True
        assert np.array_equal(g_[~skip], r_[~skip]), f"pool {which}"
        assert not np.array_equal(g_[skip], i_[skip]), f"pool {which}: rows outside the sample were not written"

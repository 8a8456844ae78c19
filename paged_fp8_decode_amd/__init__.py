"""Python binding of the mj C ABI (paged decode attention over an e4m3 or
packed fp6 (e2m3 / e3m2) or fp4 (e2m1) KV cache on MI355X).

The functions below carry the C names and only marshal arguments: every step
of the decode path runs in the HIP kernels of ``libmj.so``.  PyTorch supplies
device memory and the current HIP stream.  Importing works without a GPU
(host-only entry points such as ``mj_plan_compute`` run on the CPU).  The
library is loaded on first use; a missing or stale ``libmj.so`` raises
ImportError there -- there is no fallback implementation.
"""

from __future__ import annotations

import ctypes

import numpy as np

from ._abi import (  # noqa: F401
    Config, PlanInfo, DecodeArgs, MergeArgs, StepArgs, WriteArgs, DraftArgs, CombineArgs, MjError, KV_FORMATS, Q_MODES,
    SCALE_KINDS,
    MJ_OK, MJ_EINVAL, MJ_EUNSUPPORTED, MJ_EALIGN, MJ_ECAPACITY, MJ_EHIP, lib, check, LIB_PATH,
)


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def mj_config(*, h_q, h_k, page_size, max_num_seqs, max_q_len=1, max_splits=16, num_cus=0, wgs_per_cu=0,
              kv_tile_tokens=0, slots_override=0, kv_format="e4m3", head_dim=128, min_chunk_tokens=0,
              q_mode="fp8", out_f32=False, decode_kernel=0, kv_cache_policy=0, step_merge=0) -> Config:
    c = Config(h_q=h_q, h_k=h_k, head_dim=head_dim, page_size=page_size, max_num_seqs=max_num_seqs,
               max_q_len=max_q_len, max_splits=max_splits, num_cus=num_cus, wgs_per_cu=wgs_per_cu,
               kv_tile_tokens=kv_tile_tokens, slots_override=slots_override, min_chunk_tokens=min_chunk_tokens,
               kv_format=KV_FORMATS[kv_format] if isinstance(kv_format, str) else kv_format,
               q_mode=Q_MODES[q_mode] if isinstance(q_mode, str) else q_mode, out_f32=int(bool(out_f32)),
               decode_kernel=decode_kernel, kv_cache_policy=kv_cache_policy, step_merge=step_merge)
    return c


def mj_config_check(cfg: Config) -> int:
    return lib().mj_config_check(ctypes.byref(cfg))


def mj_plan_buffer_bytes(cfg: Config) -> int:
    return lib().mj_plan_buffer_bytes(ctypes.byref(cfg))


def mj_workspace_bytes(cfg: Config) -> int:
    return lib().mj_workspace_bytes(ctypes.byref(cfg))


def mj_plan_capacity(cfg: Config, q_len: int) -> int:
    return lib().mj_plan_capacity(ctypes.byref(cfg), q_len)


def mj_plan_compute(cfg: Config, seq_lens, q_len: int, margin: int = 0, max_blocks_per_seq: int = 1 << 30):
    """Host-only plan: returns (plan image as int32 array, PlanInfo)."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    n = mj_plan_buffer_bytes(cfg) // 4
    if n == 0:
        check(mj_config_check(cfg) or MJ_EINVAL, "mj_plan_buffer_bytes")
    out = np.zeros(n, dtype=np.int32)
    info = PlanInfo()
    st = lib().mj_plan_compute(ctypes.byref(cfg), lens.ctypes.data_as(ctypes.c_void_p), len(lens), q_len, margin,
                               max_blocks_per_seq, out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(info))
    check(st, "mj_plan_compute")
    return out, info


def mj_plan_split_kv(cfg: Config, seq_lens, q_len: int, margin: int, max_blocks_per_seq: int, host_staging,
                     plan_dev, stream=None) -> PlanInfo:
    """Plan into pinned ``host_staging`` (torch int32, pinned) and enqueue its
    copy into ``plan_dev`` (torch int32 on the GPU) on ``stream``."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    info = PlanInfo()
    st = lib().mj_plan_split_kv(ctypes.byref(cfg), lens.ctypes.data_as(ctypes.c_void_p), len(lens), q_len, margin,
                                max_blocks_per_seq, _ptr(host_staging), _ptr(plan_dev), ctypes.byref(info),
                                _stream(stream))
    check(st, "mj_plan_split_kv")
    return info


def mj_plan_split_kv_device(cfg: Config, seq_lens_dev, num_seqs: int, q_len: int, margin: int,
                            max_blocks_per_seq: int, plan_dev, stream=None) -> PlanInfo:
    """Plan on the device from ``seq_lens_dev`` (torch int32 on the GPU) into ``plan_dev``."""
    info = PlanInfo()
    st = lib().mj_plan_split_kv_device(ctypes.byref(cfg), _ptr(seq_lens_dev), num_seqs, q_len, margin,
                                       max_blocks_per_seq, _ptr(plan_dev), ctypes.byref(info), _stream(stream))
    check(st, "mj_plan_split_kv_device")
    return info


def mj_plan_shape(cfg: Config, num_seqs: int, q_len: int, max_blocks_per_seq: int) -> PlanInfo:
    info = PlanInfo()
    check(lib().mj_plan_shape(ctypes.byref(cfg), num_seqs, q_len, max_blocks_per_seq, ctypes.byref(info)),
          "mj_plan_shape")
    return info


def mj_quantize_q(cfg: Config, q, q_mul, num_seqs: int, q_len: int, q8, q_descale, stream=None):
    """q: bf16 torch view (tokens, h_q, 128) with unit channel stride."""
    assert q.stride(2) == 1
    st = lib().mj_quantize_q(ctypes.byref(cfg), _ptr(q), q.stride(0), q.stride(1), _ptr(q_mul), num_seqs, q_len,
                             _ptr(q8), _ptr(q_descale), _stream(stream))
    check(st, "mj_quantize_q")


def mj_paged_decode(cfg: Config, args: DecodeArgs, stream=None):
    check(lib().mj_paged_decode(ctypes.byref(cfg), ctypes.byref(args), _stream(stream)), "mj_paged_decode")


def mj_merge_lse(cfg: Config, args: MergeArgs, stream=None):
    check(lib().mj_merge_lse(ctypes.byref(cfg), ctypes.byref(args), _stream(stream)), "mj_merge_lse")


def mj_decode_step(cfg: Config, args: StepArgs, stream=None):
    check(lib().mj_decode_step(ctypes.byref(cfg), ctypes.byref(args), _stream(stream)), "mj_decode_step")


def mj_decode_step_noalloc(cfg: Config, args: StepArgs, stream=None):
    """mj_decode_step with the library's static per-GPU plan buffer and
    workspace (args.decode.plan / .workspace None, plan_on_device 1)."""
    check(lib().mj_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(args), _stream(stream)),
          "mj_decode_step_noalloc")


def mj_noalloc_scratch_bytes(cfg: Config) -> int:
    return lib().mj_noalloc_scratch_bytes(ctypes.byref(cfg))


def mj_write_kv(cfg: Config, args: WriteArgs, stream=None):
    check(lib().mj_write_kv(ctypes.byref(cfg), ctypes.byref(args), _stream(stream)), "mj_write_kv")


def mj_draft_advance(cfg: Config, block_table, seq_lens, num_seqs: int, q_len: int, slot_mapping, stream=None):
    """Slots of the q_len tokens each sequence appends, then seq_lens += q_len
    (device tensors: int32 block table and lengths, int64 slot mapping)."""
    a = DraftArgs(block_table=block_table.data_ptr(), bt_row_stride=block_table.stride(0),
                  max_blocks_per_seq=block_table.shape[1], seq_lens=seq_lens.data_ptr(), num_seqs=num_seqs,
                  q_len=q_len, slot_mapping=slot_mapping.data_ptr())
    check(lib().mj_draft_advance(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)), "mj_draft_advance")


def mj_combine_lse(cfg: Config, part_out, part_lse, out, lse=None, stream=None):
    """Merge num_parts context slices: part_out fp32 (parts, rows, h_q, 128)
    view, part_lse fp32 (parts, rows, h_q) contiguous, out (rows, h_q, 128)
    in the config's output dtype."""
    assert part_lse.is_contiguous() and part_out.shape[:3] == part_lse.shape
    a = CombineArgs(num_parts=part_out.shape[0], num_rows=part_out.shape[1], part_out=part_out.data_ptr(),
                    part_stride=part_out.stride(0), part_tok_stride=part_out.stride(1),
                    part_head_stride=part_out.stride(2), part_lse=part_lse.data_ptr(), out=out.data_ptr(),
                    out_tok_stride=out.stride(0), out_head_stride=out.stride(1),
                    lse=lse.data_ptr() if lse is not None else None)
    check(lib().mj_combine_lse(ctypes.byref(cfg), ctypes.byref(a), _stream(stream)), "mj_combine_lse")


def mj_debug_gather_kv(cfg: Config, args: DecodeArgs, seq: int, head: int, seq_len: int, which: int, dense_out,
                       stream=None):
    st = lib().mj_debug_gather_kv(ctypes.byref(cfg), ctypes.byref(args), seq, head, seq_len, which, _ptr(dense_out),
                                  _stream(stream))
    check(st, "mj_debug_gather_kv")


def mj_debug_decode_codes(kv_format, codes, out, stream=None):
    fmt = {**KV_FORMATS, "e4m3_bf16": 16}[kv_format] if isinstance(kv_format, str) else kv_format
    check(lib().mj_debug_decode_codes(fmt, _ptr(codes), codes.numel(), _ptr(out), _stream(stream)),
          "mj_debug_decode_codes")


def mj_debug_stream_read(src, out, blocks: int, stream=None):
    """src: any contiguous device tensor; out: uint32/int32 device tensor with >= blocks elements."""
    nbytes = src.numel() * src.element_size()
    check(lib().mj_debug_stream_read(_ptr(src), nbytes, _ptr(out), blocks, _stream(stream)), "mj_debug_stream_read")


from .runner import DecodeStep  # noqa: E402,F401

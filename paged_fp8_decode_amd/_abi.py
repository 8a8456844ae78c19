"""ctypes declarations of the mj C ABI (include/mj.h).  Marshalling only."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAGED_FP8_DECODE_LIB names another build of the same library (the
# host-sanitizer build the CPU tests load); unset, the in-tree libmj.so
LIB_PATH = os.environ.get("PAGED_FP8_DECODE_LIB") or os.path.join(_HERE, "libmj.so")

ABI_VERSION = 9  # MJ_ABI_VERSION of include/mj.h this binding matches
MJ_OK, MJ_EINVAL, MJ_EUNSUPPORTED, MJ_EALIGN, MJ_ECAPACITY, MJ_EHIP = 0, -1, -2, -3, -4, -5
KV_FORMATS = {"e4m3": 0, "e2m3": 1, "e3m2": 2, "e2m1": 3, "nvfp4": 4}
Q_MODES = {"fp8": 0, "bf16": 1}
SCALE_KINDS = {"tensor": 0, "head": 1, "seq_head": 2, "channel": 3}


class MjError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.mj_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "h_q", "h_k", "head_dim", "page_size", "max_num_seqs", "max_q_len", "max_splits", "num_cus",
        "wgs_per_cu", "kv_tile_tokens", "slots_override", "kv_format", "min_chunk_tokens", "q_mode", "out_f32",
        "decode_kernel", "kv_cache_policy", "step_merge")]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_work", "slots", "chunk_tiles", "num_chunks", "with_reduction", "num_seqs", "q_len", "kv_tile_tokens",
        "min_chunk_tiles", "wgs_per_cu")]


_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q8", _p), ("q_descale", _p), ("num_seqs", _i32), ("q_len", _i32), ("causal", _i32),
        ("k_cache", _p), ("k_page_stride", _i64), ("k_slot_stride", _i64), ("k_head_stride", _i64),
        ("v_cache", _p), ("v_page_stride", _i64), ("v_slot_stride", _i64), ("v_head_stride", _i64),
        ("num_pages", _i64),
        ("k_descale", _p), ("k_descale_kind", _i32), ("v_descale", _p), ("v_descale_kind", _i32),
        ("block_table", _p), ("bt_row_stride", _i64), ("max_blocks_per_seq", _i32), ("seq_lens", _p),
        ("plan", _p), ("num_work", _i32), ("with_reduction", _i32), ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
        ("softmax_scale", ctypes.c_float), ("o_mul", _p),
        ("out", _p), ("out_tok_stride", _i64), ("out_head_stride", _i64), ("lse", _p),
        ("q_bf16", _p), ("q_tok_stride", _i64), ("q_head_stride", _i64),
        ("k_block_scale", _p), ("k_bs_page_stride", _i64), ("k_bs_slot_stride", _i64), ("k_bs_head_stride", _i64),
        ("v_block_scale", _p), ("v_bs_page_stride", _i64), ("v_bs_slot_stride", _i64), ("v_bs_head_stride", _i64),
    ]


class MergeArgs(ctypes.Structure):
    _fields_ = [
        ("plan", _p), ("num_seqs", _i32), ("q_len", _i32), ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
        ("out", _p), ("out_tok_stride", _i64), ("out_head_stride", _i64), ("lse", _p),
    ]


class WriteArgs(ctypes.Structure):
    _fields_ = [
        ("key", _p), ("key_tok_stride", _i64), ("key_head_stride", _i64),
        ("value", _p), ("value_tok_stride", _i64), ("value_head_stride", _i64),
        ("num_tokens", _i32), ("slot_mapping", _p),
        ("k_cache", _p), ("k_page_stride", _i64), ("k_slot_stride", _i64), ("k_head_stride", _i64),
        ("v_cache", _p), ("v_page_stride", _i64), ("v_slot_stride", _i64), ("v_head_stride", _i64),
        ("num_pages", _i64), ("k_scale", _p), ("k_scale_kind", _i32), ("v_scale", _p), ("v_scale_kind", _i32),
        ("k_block_scale", _p), ("k_bs_page_stride", _i64), ("k_bs_slot_stride", _i64), ("k_bs_head_stride", _i64),
        ("v_block_scale", _p), ("v_bs_page_stride", _i64), ("v_bs_slot_stride", _i64), ("v_bs_head_stride", _i64),
    ]


class StepArgs(ctypes.Structure):
    _fields_ = [
        ("decode", DecodeArgs), ("q", _p), ("q_tok_stride", _i64), ("q_head_stride", _i64), ("q_mul", _p),
        ("plan_on_device", _i32), ("margin", _i32),
    ]


class DraftArgs(ctypes.Structure):
    _fields_ = [
        ("block_table", _p), ("bt_row_stride", _i64), ("max_blocks_per_seq", _i32), ("seq_lens", _p),
        ("num_seqs", _i32), ("q_len", _i32), ("slot_mapping", _p),
    ]


class CombineArgs(ctypes.Structure):
    _fields_ = [
        ("num_parts", _i32), ("num_rows", _i32), ("part_out", _p), ("part_stride", _i64), ("part_tok_stride", _i64),
        ("part_head_stride", _i64), ("part_lse", _p), ("out", _p), ("out_tok_stride", _i64),
        ("out_head_stride", _i64), ("lse", _p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m paged_fp8_decode_amd.build, or __graft_entry__.build()). There is no fallback path.")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sigs = {
        "mj_status_string": (ctypes.c_char_p, [_i32]),
        "mj_abi_version": (_i32, []),
        "mj_config_check": (_i32, [P(Config)]),
        "mj_plan_buffer_bytes": (ctypes.c_size_t, [P(Config)]),
        "mj_workspace_bytes": (ctypes.c_size_t, [P(Config)]),
        "mj_plan_capacity": (_i32, [P(Config), _i32]),
        "mj_plan_compute": (_i32, [P(Config), _p, _i32, _i32, _i32, _i32, _p, P(PlanInfo)]),
        "mj_plan_split_kv": (_i32, [P(Config), _p, _i32, _i32, _i32, _i32, _p, _p, P(PlanInfo), _p]),
        "mj_plan_split_kv_device": (_i32, [P(Config), _p, _i32, _i32, _i32, _i32, _p, P(PlanInfo), _p]),
        "mj_plan_shape": (_i32, [P(Config), _i32, _i32, _i32, P(PlanInfo)]),
        "mj_noalloc_scratch_bytes": (ctypes.c_size_t, [P(Config)]),
        "mj_quantize_q": (_i32, [P(Config), _p, _i64, _i64, _p, _i32, _i32, _p, _p, _p]),
        "mj_paged_decode": (_i32, [P(Config), P(DecodeArgs), _p]),
        "mj_merge_lse": (_i32, [P(Config), P(MergeArgs), _p]),
        "mj_decode_step": (_i32, [P(Config), P(StepArgs), _p]),
        "mj_decode_step_noalloc": (_i32, [P(Config), P(StepArgs), _p]),
        "mj_write_kv": (_i32, [P(Config), P(WriteArgs), _p]),
        "mj_draft_advance": (_i32, [P(Config), P(DraftArgs), _p]),
        "mj_combine_lse": (_i32, [P(Config), P(CombineArgs), _p]),
        "mj_debug_gather_kv": (_i32, [P(Config), P(DecodeArgs), _i32, _i32, _i32, _i32, _p, _p]),
        "mj_debug_decode_codes": (_i32, [_i32, _p, _i32, _p, _p]),
        "mj_debug_stream_read": (_i32, [_p, _i64, _p, _i32, _p]),
    }
    for name, (res, args) in sigs.items():
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} is stale (no {name}): rebuild it (python paged_fp8_decode_amd/build.py)")
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.mj_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI {lib.mj_abi_version()}, this binding expects {ABI_VERSION}: rebuild it")
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def check(status: int, where: str):
    if status != MJ_OK:
        raise MjError(status, where)

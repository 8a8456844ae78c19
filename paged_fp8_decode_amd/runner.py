"""``DecodeStep``: one decode site's configuration, its persistent device
buffers, and the C-ABI calls of a step in order: plan -> quantize Q ->
decode -> merge, or plan -> ``mj_decode_step`` (the last three fused).  With
``q_mode="bf16"`` there is no quantize call: the decode reads bf16 Q.  Buffers are allocated once with torch (plumbing) at fixed
addresses, so a hipGraph that captured ``run`` replays any later ``plan``
(mjolnir-kernel wheel page mjolnir/runner.py, module docstring and
T5DecodeRunner.__init__: fixed-address plan buffers padded to a fixed grid).
"""

from __future__ import annotations

import torch

from . import (DecodeArgs, MergeArgs, PlanInfo, SCALE_KINDS, StepArgs, check, mj_config, mj_config_check,
               mj_decode_step, mj_decode_step_noalloc, mj_merge_lse, mj_paged_decode, mj_plan_shape, mj_plan_buffer_bytes, mj_plan_capacity, mj_plan_split_kv, mj_plan_split_kv_device,
               mj_quantize_q, mj_workspace_bytes)


class DecodeStep:
    def __init__(self, *, h_q, h_k, page_size, max_num_seqs, max_q_len=1, max_splits=16, kv_format="e4m3",
                 num_cus=0, wgs_per_cu=0, kv_tile_tokens=0, slots_override=0, min_chunk_tokens=0, q_mode="fp8",
                 out_f32=False, decode_kernel=0, kv_cache_policy=0, step_merge=0, device="cuda"):
        self.device = torch.device(device)
        if num_cus == 0:
            num_cus = torch.cuda.get_device_properties(self.device).multi_processor_count
        self.cfg = mj_config(h_q=h_q, h_k=h_k, page_size=page_size, max_num_seqs=max_num_seqs, max_q_len=max_q_len,
                             max_splits=max_splits, num_cus=num_cus, wgs_per_cu=wgs_per_cu,
                             kv_tile_tokens=kv_tile_tokens, slots_override=slots_override, kv_format=kv_format,
                             min_chunk_tokens=min_chunk_tokens, q_mode=q_mode, out_f32=out_f32,
                             decode_kernel=decode_kernel, kv_cache_policy=kv_cache_policy, step_merge=step_merge)
        check(mj_config_check(self.cfg), "mj_config_check")
        self.h_q, self.h_k, self.h_r = h_q, h_k, h_q // h_k
        self.max_q_len = max_q_len
        self.q_bf16 = q_mode == "bf16"
        n_plan = mj_plan_buffer_bytes(self.cfg) // 4
        self.plan_dev = torch.zeros(n_plan, dtype=torch.int32, device=self.device)
        # two pinned staging slots: a slot is rewritten only after its copy ran
        self._staging = [torch.zeros(n_plan, dtype=torch.int32).pin_memory() for _ in range(2)]
        self._staging_done = [None, None]
        self._slot = 0
        # zeroed once: mj_decode_step's arrival counters start (and stay) zero
        self.workspace = torch.zeros(max(256, mj_workspace_bytes(self.cfg)), dtype=torch.uint8, device=self.device)
        n_q_max = max_q_len * self.h_r
        self.q8 = torch.empty(max_num_seqs * h_k * n_q_max * 128, dtype=torch.uint8, device=self.device)
        self.q_descale = torch.empty(max_num_seqs * h_k, dtype=torch.float32, device=self.device)
        self.info: PlanInfo | None = None

    def capacity(self, q_len: int) -> int:
        return mj_plan_capacity(self.cfg, q_len)

    def plan(self, seq_lens_host, q_len: int, max_blocks_per_seq: int, margin: int = 0, stream=None) -> PlanInfo:
        """Host plan + async copy into the fixed plan buffer (outside capture)."""
        stream = stream or torch.cuda.current_stream(self.device)
        slot = self._slot
        if self._staging_done[slot] is not None:
            self._staging_done[slot].synchronize()
        info = mj_plan_split_kv(self.cfg, seq_lens_host, q_len, margin, max_blocks_per_seq, self._staging[slot],
                                self.plan_dev, stream)
        ev = torch.cuda.Event()
        ev.record(stream)
        self._staging_done[slot] = ev
        self._slot ^= 1
        self.info = info
        return info

    def plan_device(self, seq_lens_dev, num_seqs: int, q_len: int, max_blocks_per_seq: int, margin: int = 0,
                    stream=None) -> PlanInfo:
        """Plan on the device from device lengths (capture-safe)."""
        stream = stream or torch.cuda.current_stream(self.device)
        info = mj_plan_split_kv_device(self.cfg, seq_lens_dev, num_seqs, q_len, margin, max_blocks_per_seq,
                                       self.plan_dev, stream)
        self.info = info
        return info

    def plan_shape(self, num_seqs: int, q_len: int, max_blocks_per_seq: int) -> PlanInfo:
        """The plan's size fields for a batch (no planning, no device work)."""
        info = mj_plan_shape(self.cfg, num_seqs, q_len, max_blocks_per_seq)
        self.info = info
        return info

    def run(self, *, q, k_cache, v_cache, k_strides, v_strides, num_pages, block_table, seq_lens, k_descale,
            v_descale, descale_kind, softmax_scale, out, lse=None, q_mul=None, o_mul=None, causal=True,
            info: PlanInfo | None = None, stream=None, events=None, fused=False, plan_on_device=False, margin=0,
            k_block_scale=None, v_block_scale=None, k_bs_strides=None, v_bs_strides=None, noalloc=False):
        """quantize Q -> decode -> merge (iff the plan split), all on ``stream``;
        with ``fused`` one ``mj_decode_step`` call instead.

        q: bf16 (b*q_len, h_q, 128) view; out: bf16 (b*q_len, h_q, 128) view;
        k/v strides: bytes (page, slot, head); block_table: int32 (b, max_blocks).
        ``events``: optional pair of events recorded right before and right
        after the decode launch (the step call when fused).  ``plan_on_device``
        (fused only): the step plans from ``seq_lens`` itself (``info`` from
        ``plan_shape``).  nvfp4 caches also pass the two block-scale pools
        (uint8) and their byte strides (page, slot, head).  ``noalloc``
        (with ``fused`` and ``plan_on_device``): ``mj_decode_step_noalloc``,
        the library's own plan buffer and workspace instead of this object's.
        """
        assert fused or not plan_on_device
        assert not noalloc or (fused and plan_on_device)
        info = info or self.info
        assert info is not None, "plan() first"
        b, ql = info.num_seqs, info.q_len
        stream = stream or torch.cuda.current_stream(self.device)
        kind = SCALE_KINDS[descale_kind] if isinstance(descale_kind, str) else descale_kind
        a = DecodeArgs(
            q8=self.q8.data_ptr(), q_descale=self.q_descale.data_ptr(), num_seqs=b, q_len=ql, causal=int(causal),
            k_cache=k_cache.data_ptr(), k_page_stride=k_strides[0], k_slot_stride=k_strides[1],
            k_head_stride=k_strides[2],
            v_cache=v_cache.data_ptr(), v_page_stride=v_strides[0], v_slot_stride=v_strides[1],
            v_head_stride=v_strides[2], num_pages=num_pages,
            k_descale=k_descale.data_ptr(), k_descale_kind=kind, v_descale=v_descale.data_ptr(), v_descale_kind=kind,
            block_table=block_table.data_ptr(), bt_row_stride=block_table.stride(0),
            max_blocks_per_seq=block_table.shape[1], seq_lens=seq_lens.data_ptr(),
            plan=self.plan_dev.data_ptr(), num_work=info.num_work, with_reduction=info.with_reduction,
            workspace=self.workspace.data_ptr(), workspace_bytes=self.workspace.numel(),
            softmax_scale=float(softmax_scale), o_mul=o_mul.data_ptr() if o_mul is not None else None,
            out=out.data_ptr(), out_tok_stride=out.stride(0), out_head_stride=out.stride(1),
            lse=lse.data_ptr() if lse is not None else None,
        )
        if k_block_scale is not None:
            a.k_block_scale, a.v_block_scale = k_block_scale.data_ptr(), v_block_scale.data_ptr()
            a.k_bs_page_stride, a.k_bs_slot_stride, a.k_bs_head_stride = k_bs_strides
            a.v_bs_page_stride, a.v_bs_slot_stride, a.v_bs_head_stride = v_bs_strides
        if self.q_bf16:
            if q_mul is not None:
                raise ValueError("q_mul folds fp6 K scales into quantized Q; bf16-Q mode has no Q scale")
            assert q.stride(2) == 1
            a.q_bf16, a.q_tok_stride, a.q_head_stride = q.data_ptr(), q.stride(0), q.stride(1)
        if fused:
            assert q.stride(2) == 1
            a.q8 = None
            a.q_descale = None
            sa = StepArgs(decode=a, q=q.data_ptr(), q_tok_stride=q.stride(0), q_head_stride=q.stride(1),
                          q_mul=q_mul.data_ptr() if q_mul is not None else None,
                          plan_on_device=int(plan_on_device), margin=margin)
            if noalloc:
                sa.decode.plan = None
                sa.decode.workspace = None
                sa.decode.workspace_bytes = 0
            if events:
                events[0].record(stream)
            (mj_decode_step_noalloc if noalloc else mj_decode_step)(self.cfg, sa, stream)
            if events:
                events[1].record(stream)
            return out
        if not self.q_bf16:
            mj_quantize_q(self.cfg, q, q_mul, b, ql, self.q8, self.q_descale, stream)
        if events:
            events[0].record(stream)
        mj_paged_decode(self.cfg, a, stream)
        if events:
            events[1].record(stream)
        if info.with_reduction:
            self.merge(out, lse, info, stream)
        return out

    def merge(self, out, lse=None, info: PlanInfo | None = None, stream=None):
        """mj_merge_lse of the partials in the workspace under the current plan."""
        info = info or self.info
        stream = stream or torch.cuda.current_stream(self.device)
        m = MergeArgs(plan=self.plan_dev.data_ptr(), num_seqs=info.num_seqs, q_len=info.q_len,
                      workspace=self.workspace.data_ptr(), workspace_bytes=self.workspace.numel(), out=out.data_ptr(),
                      out_tok_stride=out.stride(0), out_head_stride=out.stride(1),
                      lse=lse.data_ptr() if lse is not None else None)
        mj_merge_lse(self.cfg, m, stream)
        return out

    # convenience for seeded workloads (tests, bench, smoke)
    @classmethod
    def for_workload(cls, wl, device=None, **overrides):
        s = wl.spec
        kw = dict(h_q=s.h_q, h_k=s.h_k, page_size=s.page_size, max_num_seqs=s.b, max_q_len=s.q_len,
                  kv_format=s.kv_format, slots_override=s.slots_override, device=device or wl.q.device)
        kw.update(overrides)
        return cls(**kw)

    def plan_workload(self, wl, margin=0, stream=None) -> PlanInfo:
        return self.plan(wl.seq_lens, wl.spec.q_len, wl.block_table.shape[1], margin, stream)

    def plan_workload_device(self, wl, margin=0, stream=None) -> PlanInfo:
        return self.plan_device(wl.seq_lens_dev, wl.spec.b, wl.spec.q_len, wl.block_table.shape[1], margin, stream)

    def plan_workload_shape(self, wl) -> PlanInfo:
        return self.plan_shape(wl.spec.b, wl.spec.q_len, wl.block_table.shape[1])

    def run_workload(self, wl, out, lse=None, info=None, stream=None, events=None, fused=False,
                     plan_on_device=False, noalloc=False):
        ks, vs = wl.kv_strides()
        bs = {}
        if wl.k_bs_pool is not None:
            kbs, vbs = wl.bs_strides()
            bs = dict(k_block_scale=wl.k_bs_pool, v_block_scale=wl.v_bs_pool, k_bs_strides=kbs, v_bs_strides=vbs)
        return self.run(**bs, q=wl.q, k_cache=wl.k_pool, v_cache=wl.v_pool, k_strides=ks, v_strides=vs,
                        num_pages=wl.num_pages, block_table=wl.block_table, seq_lens=wl.seq_lens_dev,
                        k_descale=wl.k_descale, v_descale=wl.v_descale, descale_kind=wl.descale_kind,
                        softmax_scale=wl.softmax_scale, out=out, lse=lse, q_mul=wl.q_mul, o_mul=wl.o_mul,
                        causal=wl.spec.causal, info=info, stream=stream, events=events, fused=fused,
                        plan_on_device=plan_on_device, noalloc=noalloc)


def new_output(wl, device=None, out_f32=False):
    s = wl.spec
    dev = device or wl.q.device
    out = torch.empty(s.b * s.q_len, s.h_q, 128, dtype=torch.float32 if out_f32 else torch.bfloat16, device=dev)
    lse = torch.empty(s.b * s.q_len, s.h_q, dtype=torch.float32, device=dev)
    return out, lse

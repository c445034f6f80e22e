"""One decode step of the path on device buffers: kv_write -> decode_partial
-> merge_lse -> value_gate, for a synthetic workload (see synth.py).

Variants of the same step: `use_fp8_query(q_scale)` quantises the bf16
query with concat_quant_fp8 each step and attends on the fp8 codes
(decode_partial with q_scale); `fused_post = True` runs merge_value_gate in
place of merge_lse + value_gate (the value heads must be the attention
heads); `fused_attend = True` runs decode_attend (the partials and their
merge in one launch, into self.latent) in place of decode_partial +
merge_lse; `fused_write = True` runs kv_write_decode_partial_hostplan (the
cache write of the new tokens inside the partials' launch) in place of
kv_write + decode_partial.  The partials come from the *_hostplan entry points (the split
partition built on the host from the request offsets) unless `host_plan` is
set to False, which calls mla_decode_partial(_fp8q); the two give the same
bits.

Buffers are allocated once by `DeviceStep.__init__` (torch, on the current
device) and reused by every `run()`, so a timed step enqueues the library
calls and nothing else.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (D_LATENT, D_QK, D_V, concat_quant_fp8, decode_attend, decode_attend_workspace_bytes, decode_partial,
               kv_write, kv_write_decode_partial_hostplan, merge_lse, merge_value_gate, value_gate)
from .synth import FP8_NAN, Workload


def _bf16_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


class DeviceStep:
    def __init__(self, w: Workload, device="cuda", num_workers: int | None = None,
                 split_min_tokens: int | None = None, fill_cache: bool = True):
        self.w = w
        dev = torch.device(device)
        self.dev = dev
        self.num_workers = num_workers or w.num_workers
        self.split_min = split_min_tokens if split_min_tokens is not None else w.split_min_tokens
        S, H, VH = w.S, w.heads, w.value_heads
        self.q = _bf16_dev(w.q, dev)
        self.q_scale = None  # set, with an fp8 self.q, for the fp8-query entry point
        self.q_bf16 = None   # set by use_fp8_query: the bf16 query each step quantises
        # run() merges and projects in one call (possible when the value heads
        # are the attention heads); off: mla_merge_lse, then mla_value_gate
        self.fused_post = False
        # run() attends and merges in one launch (decode_attend, bf16 query)
        self.fused_attend = False
        # run() writes the new tokens inside the partials' launch
        self.fused_write = False
        self.workspace = None  # decode_attend's workspace, allocated (zeroed) on first use
        self.kv_cache = torch.full((w.num_slots, D_QK), FP8_NAN, dtype=torch.uint8, device=dev)
        self.indptr = torch.from_numpy(w.indptr).to(dev)
        self.indptr_host = np.ascontiguousarray(w.indptr, dtype=np.int32)  # the same offsets, on the host
        self.host_plan = True
        self.indices = torch.from_numpy(w.indices).to(dev)
        self.lengths = torch.from_numpy(w.lengths).to(dev)
        if fill_cache and w.kv_rows is not None and w.total_tokens > 0:
            rows = _bf16_dev(w.kv_rows, dev)
            slots = torch.from_numpy(w.indices.astype(np.int64)).to(dev)
            kv_write(rows[:, :D_LATENT], rows[:, D_LATENT:], slots, self.kv_cache, w.kv_scale)
            del rows
        self.new_rows = _bf16_dev(w.new_rows, dev)
        self.slot_mapping = torch.from_numpy(w.slot_mapping).to(dev)
        self.o_part = torch.empty((w.num_splits, S, H, D_LATENT), dtype=torch.bfloat16, device=dev)
        self.lse_part = torch.empty((w.num_splits, S, H), dtype=torch.float32, device=dev)
        # the W_UV stage may run on more heads than the attention (the extra
        # heads' latent rows are synthetic)
        self.latent = torch.zeros((S, VH, D_LATENT), dtype=torch.bfloat16, device=dev)
        if VH > H:
            self.latent[:, H:, :] = _bf16_dev(w.extra_latent, dev)
        self.lse = torch.empty((S, H), dtype=torch.float32, device=dev)
        self.gate = _bf16_dev(w.gate, dev)
        self.out = torch.empty((S, VH * D_V), dtype=torch.bfloat16, device=dev)
        self.w_uv = _bf16_dev(w.w_uv, dev) if w.w_uv is not None else None
        self.w_fp4 = torch.from_numpy(w.w_fp4).to(dev) if w.w_fp4 is not None else None
        self.w_scale = torch.from_numpy(w.w_scale).to(dev) if w.w_scale is not None else None

    def use_fp8_query(self, q_scale: float):
        """Run the fp8-query path: every step first quantises the bf16 query
        (ql_nope = dims 0..511, q_pe = dims 512..575 of the real heads) into an
        fp8 query buffer with mla_concat_quant_fp8, and attends on that."""
        w = self.w
        self.q_bf16 = self.q
        self.q = torch.full((w.S, w.heads_pad, D_QK), 0x7F, dtype=torch.uint8, device=self.dev)
        self.q_scale = float(q_scale)

    def quantize_query(self):
        H = self.w.heads
        concat_quant_fp8(self.q_bf16[:, :H, :D_LATENT], self.q_bf16[:, :H, D_LATENT:], self.q_scale, self.q[:, :H])

    # the calls of one step -----------------------------------------------------
    def write_new_tokens(self):
        nr = self.new_rows
        kv_write(nr[:, :D_LATENT], nr[:, D_LATENT:], self.slot_mapping, self.kv_cache, self.w.kv_scale)

    def attend(self, write_new: bool = False):
        """The split-KV partials; write_new: with the new tokens' cache write
        in the same launch (host plan only)."""
        w = self.w
        if write_new:
            if not self.host_plan:
                raise ValueError("the fused cache write takes the host-built partition")
            nr = self.new_rows
            kv_write_decode_partial_hostplan(
                nr[:, :D_LATENT], nr[:, D_LATENT:], self.slot_mapping, self.q, self.kv_cache, self.indptr,
                self.indices, self.o_part, self.lse_part, self.indptr_host, qlen=w.qlen, heads=w.heads,
                sm_scale=w.sm_scale, kv_scale=w.kv_scale, num_workers=self.num_workers,
                split_min_tokens=self.split_min, q_scale=self.q_scale)
            return
        plan = self.indptr_host if self.host_plan else None
        decode_partial(self.q, self.kv_cache, self.indptr, self.indices, self.o_part, self.lse_part,
                       qlen=w.qlen, heads=w.heads, sm_scale=w.sm_scale, kv_scale=w.kv_scale,
                       num_workers=self.num_workers, split_min_tokens=self.split_min, q_scale=self.q_scale,
                       kv_indptr_host=plan)

    def partials(self):
        """The step's partial launch: with the new tokens' cache write in it
        when fused_write is set (run() then writes no rows before it)."""
        self.attend(write_new=self.fused_write and not self.fused_attend)

    def attend_merged(self):
        """The partials and their LSE merge in one launch: self.latent (the
        attention heads) and self.lse, as attend() + merge() give them."""
        w = self.w
        if self.workspace is None:
            n = decode_attend_workspace_bytes(w.batch, w.qlen, w.heads, self.num_workers)
            self.workspace = torch.zeros(n, dtype=torch.uint8, device=self.dev)
        decode_attend(self.q, self.kv_cache, self.indptr, self.indices, self.latent[:, :w.heads], self.lse,
                      self.workspace, self.indptr_host, qlen=w.qlen, heads=w.heads, sm_scale=w.sm_scale,
                      kv_scale=w.kv_scale, num_splits=w.num_splits, num_workers=self.num_workers,
                      split_min_tokens=self.split_min)

    def merge(self):
        merge_lse(self.o_part, self.lse_part, self.latent[:, :self.w.heads], self.lse)

    def value(self):
        w = self.w
        value_gate(self.latent, self.gate, self.lengths, self.out, qlen=w.qlen, w_uv=self.w_uv,
                   w_fp4=self.w_fp4, w_scale=self.w_scale)

    def merge_value(self):
        """The merge, W_UV and gate in one call (the value heads must be the
        attention heads); self.latent is not written."""
        w = self.w
        if w.value_heads != w.heads:
            raise ValueError("merge_value needs the value heads (%d) to be the attention heads (%d)"
                             % (w.value_heads, w.heads))
        merge_value_gate(self.o_part, self.lse_part, self.gate, self.lengths, self.out, qlen=w.qlen, w_uv=self.w_uv,
                         w_fp4=self.w_fp4, w_scale=self.w_scale, lse=self.lse)

    def run(self, write_new: bool = True):
        fused_write = write_new and self.fused_write and not self.fused_attend
        if write_new and not fused_write:
            self.write_new_tokens()
        if self.q_bf16 is not None:
            self.quantize_query()
        if self.fused_attend:
            if self.q_scale is not None:
                raise ValueError("decode_attend takes a bf16 query")
            self.attend_merged()
            self.value()
            return
        self.partials()
        if self.fused_post:
            self.merge_value()
        else:
            self.merge()
            self.value()

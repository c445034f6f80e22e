"""Seeded synthetic inputs shaped like the MLA decode workloads.

This module only draws random numbers and lays them out; it holds none of
the path's arithmetic (no fp8 encoding, no attention, no projection).  Real
values are stored as bf16 by truncating binary32 draws (keeping the high 16
bits), which is storage, not a rounding step of the method.  fp8 cache bytes
are NOT produced here: callers write the cache from these bf16 rows with a
cache-write (`kv_write`) of their own.  MXFP4 weights are drawn directly as
codes (uniform E2M1 nibbles, E8M0 scales near 2^-6), so no quantiser is
involved either.

Shapes follow the decode runtime of "vllm.models.kimi_k3.amd.
specialized_decode.runtime.mla" (sections ``attend``, ``m1c_inputs``,
``pre``, ``post``) and "...nvidia.specialized_decode.cutedsl.mla.value"
(``MlaValue``): absorbed queries [S, H, 576] (512 latent + 64 rope), one
576-wide cache row per token, W_UV [H, 128, 512] with the latent axis
contiguous, gate logits [S, H*128].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D_LATENT, D_ROPE, D_QK, D_V = 512, 64, 576, 128
BF16_NAN = 0x7FC0
FP8_NAN = 0x7F
SM_SCALE = 1.0 / np.sqrt(192.0)  # qk_nope 128 + rope 64


@dataclass
class Workload:
    name: str
    batch: int
    qlen: int
    heads: int            # heads computed
    heads_pad: int        # heads in the query buffer (pad rows are NaN)
    lengths: np.ndarray   # [batch] int32 context lengths (0 = empty request)
    kv_scale: float
    sm_scale: float
    num_splits: int       # split capacity of the partial buffers
    split_min_tokens: int
    num_workers: int
    w_format: str         # "bf16" or "mxfp4"
    value_heads: int      # heads of the W_UV stage
    seed: int
    # drawn arrays
    q: np.ndarray = field(repr=False, default=None)          # [S, heads_pad, 576] bf16 bits
    kv_rows: np.ndarray = field(repr=False, default=None)    # [sum L, 576] bf16 bits (x values)
    num_slots: int = 0
    indptr: np.ndarray = field(repr=False, default=None)     # [batch+1] int32
    indices: np.ndarray = field(repr=False, default=None)    # [sum L] int32 cache rows
    new_rows: np.ndarray = field(repr=False, default=None)   # [n_new, 576] bf16 bits
    slot_mapping: np.ndarray = field(repr=False, default=None)  # [n_new] int64 (-1: skip)
    w_uv: np.ndarray = field(repr=False, default=None)       # [value_heads, 128, 512] bf16 bits
    w_fp4: np.ndarray = field(repr=False, default=None)      # [value_heads, 128, 256] u8
    w_scale: np.ndarray = field(repr=False, default=None)    # [value_heads, 128, 16] u8
    gate: np.ndarray = field(repr=False, default=None)       # [S, value_heads*128] bf16 bits
    extra_latent: np.ndarray = field(repr=False, default=None)  # [S, value_heads-heads, 512]

    @property
    def S(self) -> int:
        return self.batch * self.qlen

    @property
    def total_tokens(self) -> int:
        return int(self.lengths.sum())


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 draws -> bf16 storage (high half of the binary32 word)."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _normal_bf16(rng, shape, std=1.0):
    return to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


# The workloads: name -> parameters.  Context lengths are drawn uniformly on
# the stated closed ranges; "empty" requests have length 0.
SPECS = {
    "tiny": dict(batch=2, qlen=1, heads=16, heads_pad=16, fixed_lengths=[37, 64], kv_scale=1.0,
                 num_splits=2, split_min_tokens=1, num_workers=256, w_format="bf16", value_heads=16),
    "batch": dict(batch=64, qlen=1, heads=96, heads_pad=128, len_range=(1024, 8192), empty=4,
                  kv_scale=0.05, num_splits=16, split_min_tokens=256, num_workers=128,
                  w_format="bf16", value_heads=96),
    "batch_8k": dict(batch=64, qlen=1, heads=96, heads_pad=128, fixed_lengths=[8192] * 64,
                     kv_scale=0.05, num_splits=16, split_min_tokens=256, num_workers=128,
                     w_format="bf16", value_heads=96),
    "spec_q4": dict(batch=32, qlen=4, heads=96, heads_pad=96, len_range=(2048, 16384), kv_scale=0.05,
                    num_splits=16, split_min_tokens=256, num_workers=32, w_format="bf16",
                    value_heads=96, new_tokens=True),
    "spec_q8": dict(batch=32, qlen=8, heads=96, heads_pad=96, len_range=(2048, 16384), kv_scale=0.05,
                    num_splits=16, split_min_tokens=256, num_workers=16, w_format="bf16",
                    value_heads=96, new_tokens=True),
    "long": dict(batch=16, qlen=1, heads=96, heads_pad=96, len_range=(32768, 131072), kv_scale=0.05,
                 num_splits=64, split_min_tokens=256, num_workers=128, w_format="bf16",
                 value_heads=96),
    "rank_share": dict(batch=64, qlen=4, heads=12, heads_pad=12, len_range=(2048, 16384),
                       kv_scale=0.05, num_splits=16, split_min_tokens=256, num_workers=256,
                       w_format="mxfp4", value_heads=96),
}

# index of each workload in the list of configurations it stands for
SEED_BASE = {"tiny": 0, "batch": 1, "batch_8k": 1, "spec_q4": 2, "spec_q8": 2, "long": 3,
             "rank_share": 4}


def make(name: str, seed: int | None = None, batch: int | None = None,
         len_range: tuple[int, int] | None = None, draw_kv: bool = True) -> Workload:
    """Draw one workload.  `batch` / `len_range` shrink it for quick tests
    (the structure is kept); `draw_kv=False` skips the cache rows."""
    spec = dict(SPECS[name])
    if seed is None:
        seed = 1000 + SEED_BASE[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    B = batch if batch is not None else spec["batch"]
    qlen, H, Hp = spec["qlen"], spec["heads"], spec["heads_pad"]
    if "fixed_lengths" in spec and batch is None and len_range is None:
        lengths = np.array(spec["fixed_lengths"], dtype=np.int64)
    else:
        lo, hi = len_range if len_range is not None else spec.get("len_range", (1, 64))
        lengths = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    n_empty = spec.get("empty", 0)
    if n_empty and B > n_empty:
        empty = rng.choice(B, size=n_empty, replace=False)
        lengths[empty] = 0
    # a speculative window needs at least qlen tokens in every non-empty request
    lengths = np.where((lengths > 0) & (lengths < qlen), qlen, lengths)
    total = int(lengths.sum())
    indptr = np.zeros(B + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(lengths)
    num_slots = max(1, int(np.ceil(total * 1.25)))
    perm = rng.permutation(num_slots)
    indices = perm[:total].astype(np.int32)

    S = B * qlen
    q = _normal_bf16(rng, (S, Hp, D_QK))
    if Hp > H:
        q[:, H:, :] = BF16_NAN  # pad heads: never read

    kv_rows = None
    if draw_kv:
        # real values x ~ N(0,1) * 0.5 per cache row (512 latent + 64 rope)
        kv_rows = _normal_bf16(rng, (total, D_QK), std=0.5)

    new_rows = slot_mapping = None
    if spec.get("new_tokens"):
        # the qlen newest tokens of each request are written this step
        slot_mapping = np.full(S, -1, dtype=np.int64)
        for r in range(B):
            if lengths[r] > 0:
                slot_mapping[r * qlen:(r + 1) * qlen] = indices[indptr[r + 1] - qlen:indptr[r + 1]]
        new_rows = _normal_bf16(rng, (S, D_QK), std=0.5)
    else:
        # one new token per non-empty request (its last row)
        slot_mapping = np.full(B, -1, dtype=np.int64)
        for r in range(B):
            if lengths[r] > 0:
                slot_mapping[r] = indices[indptr[r + 1] - 1]
        new_rows = _normal_bf16(rng, (B, D_QK), std=0.5)

    VH = spec["value_heads"]
    w_uv = w_fp4 = w_scale = None
    if spec["w_format"] == "bf16":
        w_uv = _normal_bf16(rng, (VH, D_V, D_LATENT), std=np.sqrt(1.0 / 512.0))
    else:
        w_fp4 = rng.integers(0, 256, size=(VH, D_V, D_LATENT // 2), dtype=np.uint8)
        w_scale = rng.integers(120, 123, size=(VH, D_V, D_LATENT // 32), endpoint=True).astype(np.uint8)
    gate = _normal_bf16(rng, (S, VH * D_V))
    for r in range(B):
        if lengths[r] == 0:
            gate[r * qlen:(r + 1) * qlen, :] = BF16_NAN  # must come out as zero
    extra_latent = None
    if VH > H:
        extra_latent = _normal_bf16(rng, (S, VH - H, D_LATENT), std=0.3)

    return Workload(
        name=name, batch=B, qlen=qlen, heads=H, heads_pad=Hp, lengths=lengths.astype(np.int32),
        kv_scale=float(spec["kv_scale"]), sm_scale=float(SM_SCALE), num_splits=spec["num_splits"],
        split_min_tokens=spec["split_min_tokens"], num_workers=spec["num_workers"],
        w_format=spec["w_format"], value_heads=VH, seed=seed, q=q, kv_rows=kv_rows,
        num_slots=num_slots, indptr=indptr.astype(np.int32), indices=indices, new_rows=new_rows,
        slot_mapping=slot_mapping, w_uv=w_uv, w_fp4=w_fp4, w_scale=w_scale, gate=gate,
        extra_latent=extra_latent)


def fp8_query(rng, shape, heads: int, std: float = 16.0) -> tuple[np.ndarray, float]:
    """fp8 E4M3 query codes [S, H_pad, 576] of N(0, std^2) draws (torch's
    cast, far inside the format's range) and the per-tensor scale 1/std, so
    that the query stands for values ~ N(0, 1) like the bf16 one.  Pad heads
    (index >= heads) hold the NaN code 0x7F: they must never be read."""
    import torch

    x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))
    q8 = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    q8[:, heads:, :] = FP8_NAN
    return q8, 1.0 / std


def random_partials(rng, num_splits, rows, heads, p_empty=0.3):
    """Synthetic split partials for testing a merge on its own: bf16 o
    [splits, rows, heads, 512] and f32 LSE with some -inf (empty) splits,
    whose o is filled with NaN (it must never be read)."""
    o = _normal_bf16(rng, (num_splits, rows, heads, D_LATENT), std=0.5)
    lse = (rng.standard_normal((num_splits, rows, heads)) * 3.0).astype(np.float32)
    empty = rng.random((num_splits, rows, heads)) < p_empty
    lse[empty] = -np.inf
    o[empty] = BF16_NAN
    return o, lse

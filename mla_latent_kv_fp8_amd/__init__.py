"""MLA decode over an fp8 latent KV cache on MI355X (gfx950).

A thin Python binding of the C ABI in include/mla_fp8.h (libmla_fp8.so,
built by ``mla_latent_kv_fp8_amd.build``).  Functions here only check
arguments and marshal torch tensors into pointers, strides and the current
HIP stream; every step of the path runs in the library's HIP kernels.  There
is no fallback: if the library is missing, the first call raises.

The path (vLLM pages "vllm.models.kimi_k3.amd.specialized_decode.runtime.mla"
and "...nvidia.specialized_decode.cutedsl.mla.value"):
  kv_write -> decode_partial -> merge_lse -> value_gate.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

D_LATENT, D_ROPE, D_QK, D_V = 512, 64, 576, 128
W_BF16, W_MXFP4 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_FP8_LIBRARY names another build of the same library (the host-code
# sanitizer build of the CPU tests); the default is the in-tree build
LIB_PATH = os.environ.get("MLA_FP8_LIBRARY") or os.path.join(_HERE, "libmla_fp8.so")
_lib = None


class MlaError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libmla_fp8.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MlaError("libmla_fp8.so is not built (python -m mla_latent_kv_fp8_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.mla_status_string.argtypes = [ctypes.c_int]
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_kv_write.argtypes = [P, i64, P, i64, P, i32, P, i64, f32, P]
        L.mla_decode_partial.argtypes = [P, i64, i64, i32, i32, i32, P, i64, P, P, f32, f32, i32, i32,
                                         i32, P, i64, i64, i64, P, i64, i64, i64, P]
        L.mla_decode_partial_hostplan.argtypes = [P, i64, i64, i32, i32, i32, P, i64, P, P, f32, f32, i32,
                                                  i32, i32, P, i64, i64, i64, P, i64, i64, i64, P, P]
        L.mla_decode_partial_fp8q_hostplan.argtypes = [P, i64, i64, f32, i32, i32, i32, P, i64, P, P, f32,
                                                       f32, i32, i32, i32, P, i64, i64, i64, P, i64, i64,
                                                       i64, P, P]
        L.mla_kv_write_decode_partial_hostplan.argtypes = [P, i64, P, i64, P, i32] + \
            L.mla_decode_partial_hostplan.argtypes
        L.mla_kv_write_decode_partial_fp8q_hostplan.argtypes = [P, i64, P, i64, P, i32] + \
            L.mla_decode_partial_fp8q_hostplan.argtypes
        L.mla_concat_quant_fp8.argtypes = [P, i64, i64, P, i64, i64, f32, i32, i32, P, i64, i64, P]
        L.mla_absorb_query.argtypes = [P, i64, i64, P, i64, i64, P, i64, i64, P, i64, i64, i32, i32, i32, f32, P,
                                       i64, i64, P]
        L.mla_decode_partial_fp8q.argtypes = [P, i64, i64, f32, i32, i32, i32, P, i64, P, P, f32, f32,
                                              i32, i32, i32, P, i64, i64, i64, P, i64, i64, i64, P]
        L.mla_merge_value_gate.argtypes = [P, i64, i64, i64, P, i64, i64, i64, i32, i32, P, i64, i64, P, i64,
                                           i64, P, i64, P, i32, i32, i32, P, i64, P, i64, i64, P]
        L.mla_split_plan.argtypes = [P, i32, i32, i32, i32, P, P]
        L.mla_time_next_partial.argtypes = [P, P]
        L.mla_decode_attend.argtypes = [P, i64, i64, i32, i32, i32, P, i64, P, P, f32, f32, i32, i32, i32, P, P, i64,
                                        i64, P, i64, i64, P, i64, P]
        L.mla_decode_attend_noalloc.argtypes = [P, i64, i64, i32, i32, i32, P, i64, P, P, f32, f32, i32, i32, i32, P, P,
                                                i64, i64, P, i64, i64, P]
        L.mla_decode_attend_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.mla_decode_attend_workspace_bytes.restype = ctypes.c_int64
        L.mla_merge_lse.argtypes = [P, i64, i64, i64, P, i64, i64, i64, i32, i32, i32, P, i64, i64, P,
                                    i64, i64, P]
        L.mla_value_gate.argtypes = [P, i64, i64, i32, P, i64, i64, P, i64, i64, P, i64, P, i32, i32, i32,
                                     P, i64, P]
        for name in ("mla_kv_write", "mla_absorb_query", "mla_concat_quant_fp8", "mla_decode_partial", "mla_decode_partial_fp8q",
                     "mla_decode_partial_hostplan", "mla_decode_partial_fp8q_hostplan", "mla_split_plan", "mla_merge_lse", "mla_value_gate", "mla_merge_value_gate",
                     "mla_decode_attend", "mla_decode_attend_noalloc", "mla_time_next_partial",
                     "mla_kv_write_decode_partial_hostplan", "mla_kv_write_decode_partial_fp8q_hostplan"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def use_library(path: str) -> None:
    """Load another build of the same library on the first call into it (a
    measurement build such as libmla_fp8_timeline.so); call before that."""
    global LIB_PATH
    if _lib is not None:
        raise MlaError("the library is already loaded from %s" % LIB_PATH)
    LIB_PATH = path


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MlaError("%s: %s" % (what, lib().mla_status_string(status).decode()))


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise MlaError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype not in dtypes:
        raise MlaError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if t.numel() > 0 and t.stride(-1) != 1:
        raise MlaError("%s: the innermost axis must be contiguous" % name)
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8, torch.float8_e4m3fn)


def kv_write(kv_c: torch.Tensor, k_pe: torch.Tensor, slot_mapping: torch.Tensor, kv_cache: torch.Tensor,
             kv_scale: float) -> None:
    """Write n new tokens' rows E([kv_c | k_pe] / kv_scale) into kv_cache
    [num_slots, 576] at slot_mapping (int64; negative = skip)."""
    n = slot_mapping.shape[0]
    assert kv_c.shape[0] == n and k_pe.shape[0] == n
    assert kv_c.shape[-1] >= D_LATENT and k_pe.shape[-1] >= D_ROPE and kv_cache.shape[-1] == D_QK
    st = lib().mla_kv_write(_dev(kv_c, "kv_c", _BF16), kv_c.stride(0), _dev(k_pe, "k_pe", _BF16),
                            k_pe.stride(0), _dev(slot_mapping, "slot_mapping", (torch.int64,)), n,
                            _dev(kv_cache, "kv_cache", _U8), kv_cache.shape[0], float(kv_scale),
                            _stream())
    _check(st, "mla_kv_write")


def absorb_query(q_nope: torch.Tensor, q_pe: torch.Tensor, w_k: torch.Tensor, w_k_scale: torch.Tensor,
                 out: torch.Tensor, q_scale: float | None = None) -> None:
    """The absorbed query rows out [rows, >=H, 576] = [q_nope x W_UK | q_pe]:
    bf16 out (q_scale None) or fp8 codes E(. / q_scale) (uint8 or
    float8_e4m3fn out).  q_nope [rows, H, 128] and q_pe [rows, H, 64] bf16
    (strided views allowed); W_UK as MXFP4 codes w_k [H, 512, 64] u8 and
    E8M0 scales w_k_scale [H, 512, 4] u8."""
    rows, heads = q_nope.shape[0], q_nope.shape[1]
    if q_nope.shape[-1] != 128 or tuple(q_pe.shape) != (rows, heads, D_ROPE):
        raise MlaError("q_nope must be [rows, H, 128] and q_pe [rows, H, 64]")
    if tuple(w_k.shape) != (heads, D_LATENT, 64) or tuple(w_k_scale.shape) != (heads, D_LATENT, 4):
        raise MlaError("w_k must be [H, 512, 64] and w_k_scale [H, 512, 4]")
    if out.shape[0] != rows or out.shape[1] < heads or out.shape[2] != D_QK:
        raise MlaError("out must be [rows, >=H, 576]")
    fp8 = q_scale is not None
    st = lib().mla_absorb_query(
        _dev(q_nope, "q_nope", _BF16), q_nope.stride(0), q_nope.stride(1), _dev(q_pe, "q_pe", _BF16),
        q_pe.stride(0), q_pe.stride(1), _dev(w_k, "w_k", (torch.uint8,)), w_k.stride(0), w_k.stride(1),
        _dev(w_k_scale, "w_k_scale", (torch.uint8,)), w_k_scale.stride(0), w_k_scale.stride(1), rows, heads,
        1 if fp8 else 0, float(q_scale) if fp8 else 1.0, _dev(out, "out", _U8 if fp8 else _BF16), out.stride(0),
        out.stride(1), _stream())
    _check(st, "mla_absorb_query")


def concat_quant_fp8(ql_nope: torch.Tensor, q_pe: torch.Tensor, q_scale: float, q8: torch.Tensor) -> None:
    """fp8 query q8 [rows, H, 576] (uint8 or float8_e4m3fn) = E(cat(ql_nope, q_pe) / q_scale), with
    ql_nope [rows, H, 512] and q_pe [rows, H, 64] bf16 (strided views allowed)."""
    rows, heads = ql_nope.shape[0], ql_nope.shape[1]
    if ql_nope.shape[-1] != D_LATENT or tuple(q_pe.shape) != (rows, heads, D_ROPE):
        raise MlaError("ql_nope must be [rows, H, 512] and q_pe [rows, H, 64]")
    if q8.shape[0] != rows or q8.shape[1] < heads or q8.shape[2] != D_QK:
        raise MlaError("q8 must be [rows, >=H, 576]")
    st = lib().mla_concat_quant_fp8(
        _dev(ql_nope, "ql_nope", _BF16), ql_nope.stride(0), ql_nope.stride(1), _dev(q_pe, "q_pe", _BF16),
        q_pe.stride(0), q_pe.stride(1), float(q_scale), rows, heads, _dev(q8, "q8", _U8), q8.stride(0),
        q8.stride(1), _stream())
    _check(st, "mla_concat_quant_fp8")


def decode_partial(q: torch.Tensor, kv_cache: torch.Tensor, kv_indptr: torch.Tensor,
                   kv_indices: torch.Tensor, o_part: torch.Tensor, lse_part: torch.Tensor, *, qlen: int,
                   heads: int, sm_scale: float, kv_scale: float, num_workers: int = 256,
                   split_min_tokens: int = 256, q_scale: float | None = None,
                   kv_indptr_host: np.ndarray | None = None) -> None:
    """Split-KV partials: q [S, H_pad, 576] (first `heads` used) over
    kv_cache [num_slots, 576] u8 with CSR (kv_indptr [B+1], kv_indices) int32
    -> o_part [splits, S, heads, 512] bf16, lse_part [splits, S, heads] f32
    (strided views allowed).  q is bf16, or fp8 E4M3 codes (uint8 or
    float8_e4m3fn) standing for q_scale * fp8(q), which then must be given.
    kv_indptr_host: a host copy of kv_indptr, from which the *_hostplan entry
    points compute the split partition on the host."""
    S = q.shape[0]
    batch = kv_indptr.shape[0] - 1
    if S != batch * qlen:
        raise MlaError("q has %d rows, expected batch*qlen = %d" % (S, batch * qlen))
    ns = o_part.shape[0]
    if lse_part.shape[0] != ns or o_part.shape[1] < S or o_part.shape[2] < heads or o_part.shape[3] != D_LATENT:
        raise MlaError("bad partial buffer shapes")
    if q.shape[-1] != D_QK or q.shape[1] < heads:
        raise MlaError("q must be [S, >=heads, 576]")
    fp8_q = q.dtype in _U8
    if fp8_q != (q_scale is not None):
        raise MlaError("an fp8 query takes q_scale, a bf16 query does not")
    rest = (batch, qlen, heads, _dev(kv_cache, "kv_cache", _U8), kv_cache.shape[0],
            _dev(kv_indptr, "kv_indptr", (torch.int32,)), _dev(kv_indices, "kv_indices", (torch.int32,)),
            float(sm_scale), float(kv_scale), ns, int(num_workers), int(split_min_tokens),
            _dev(o_part, "o_part", _BF16), o_part.stride(0), o_part.stride(1), o_part.stride(2),
            _dev(lse_part, "lse_part", (torch.float32,)), lse_part.stride(0), lse_part.stride(1),
            lse_part.stride(2), _stream())
    ih = None
    if kv_indptr_host is not None:
        ih = np.ascontiguousarray(kv_indptr_host, dtype=np.int32)
        if ih.shape != (batch + 1,):
            raise MlaError("kv_indptr_host must hold batch+1 offsets")
    if fp8_q and ih is not None:
        st = lib().mla_decode_partial_fp8q_hostplan(_dev(q, "q", _U8), q.stride(0), q.stride(1), float(q_scale),
                                                    *rest[:-1], ih.ctypes.data_as(ctypes.c_void_p), rest[-1])
        _check(st, "mla_decode_partial_fp8q_hostplan")
    elif fp8_q:
        st = lib().mla_decode_partial_fp8q(_dev(q, "q", _U8), q.stride(0), q.stride(1), float(q_scale), *rest)
        _check(st, "mla_decode_partial_fp8q")
    elif ih is not None:
        st = lib().mla_decode_partial_hostplan(_dev(q, "q", _BF16), q.stride(0), q.stride(1), *rest[:-1],
                                               ih.ctypes.data_as(ctypes.c_void_p), rest[-1])
        _check(st, "mla_decode_partial_hostplan")
    else:
        st = lib().mla_decode_partial(_dev(q, "q", _BF16), q.stride(0), q.stride(1), *rest)
        _check(st, "mla_decode_partial")


def decode_partial_hostplan(q: torch.Tensor, kv_cache: torch.Tensor, kv_indptr: torch.Tensor,
                            kv_indices: torch.Tensor, o_part: torch.Tensor, lse_part: torch.Tensor,
                            kv_indptr_host: np.ndarray, **kw) -> None:
    """mla_decode_partial_hostplan / mla_decode_partial_fp8q_hostplan:
    decode_partial with the split partition computed on the host from
    kv_indptr_host."""
    decode_partial(q, kv_cache, kv_indptr, kv_indices, o_part, lse_part, kv_indptr_host=kv_indptr_host, **kw)


def kv_write_decode_partial_hostplan(kv_c: torch.Tensor, k_pe: torch.Tensor, slot_mapping: torch.Tensor,
                                     q: torch.Tensor, kv_cache: torch.Tensor, kv_indptr: torch.Tensor,
                                     kv_indices: torch.Tensor, o_part: torch.Tensor, lse_part: torch.Tensor,
                                     kv_indptr_host: np.ndarray, *, qlen: int, heads: int, sm_scale: float,
                                     kv_scale: float, num_workers: int = 256, split_min_tokens: int = 256,
                                     q_scale: float | None = None) -> None:
    """mla_kv_write_decode_partial_hostplan / _fp8q_hostplan: kv_write of
    the batch * k new tokens (the last k of each request, request-major:
    kv_c, k_pe [batch*k, .] bf16, slot_mapping [batch*k] int64) and
    decode_partial_hostplan over the updated cache, in one launch."""
    batch = kv_indptr.shape[0] - 1
    n = slot_mapping.shape[0]
    if batch < 1 or n % batch != 0:
        raise MlaError("slot_mapping must hold the same number of new tokens for each request")
    k = n // batch
    if kv_c.shape[0] != n or k_pe.shape[0] != n:
        raise MlaError("kv_c and k_pe must hold one row per new token")
    if kv_c.shape[-1] < D_LATENT or k_pe.shape[-1] < D_ROPE:
        raise MlaError("kv_c rows hold 512 values, k_pe rows 64")
    S = q.shape[0]
    if S != batch * qlen:
        raise MlaError("q has %d rows, expected batch*qlen = %d" % (S, batch * qlen))
    ns = o_part.shape[0]
    if lse_part.shape[0] != ns or o_part.shape[1] < S or o_part.shape[2] < heads or o_part.shape[3] != D_LATENT:
        raise MlaError("bad partial buffer shapes")
    if q.shape[-1] != D_QK or q.shape[1] < heads:
        raise MlaError("q must be [S, >=heads, 576]")
    fp8_q = q.dtype in _U8
    if fp8_q != (q_scale is not None):
        raise MlaError("an fp8 query takes q_scale, a bf16 query does not")
    ih = np.ascontiguousarray(kv_indptr_host, dtype=np.int32)
    if ih.shape != (batch + 1,):
        raise MlaError("kv_indptr_host must hold batch+1 offsets")
    new = (_dev(kv_c, "kv_c", _BF16), kv_c.stride(0), _dev(k_pe, "k_pe", _BF16), k_pe.stride(0),
           _dev(slot_mapping, "slot_mapping", (torch.int64,)), k)
    rest = (batch, qlen, heads, _dev(kv_cache, "kv_cache", _U8), kv_cache.shape[0],
            _dev(kv_indptr, "kv_indptr", (torch.int32,)), _dev(kv_indices, "kv_indices", (torch.int32,)),
            float(sm_scale), float(kv_scale), ns, int(num_workers), int(split_min_tokens),
            _dev(o_part, "o_part", _BF16), o_part.stride(0), o_part.stride(1), o_part.stride(2),
            _dev(lse_part, "lse_part", (torch.float32,)), lse_part.stride(0), lse_part.stride(1),
            lse_part.stride(2), ih.ctypes.data_as(ctypes.c_void_p), _stream())
    if fp8_q:
        st = lib().mla_kv_write_decode_partial_fp8q_hostplan(*new, _dev(q, "q", _U8), q.stride(0), q.stride(1),
                                                             float(q_scale), *rest)
        _check(st, "mla_kv_write_decode_partial_fp8q_hostplan")
    else:
        st = lib().mla_kv_write_decode_partial_hostplan(*new, _dev(q, "q", _BF16), q.stride(0), q.stride(1),
                                                        *rest)
        _check(st, "mla_kv_write_decode_partial_hostplan")


def decode_attend_workspace_bytes(batch: int, qlen: int, heads: int, num_workers: int) -> int:
    """mla_decode_attend_workspace_bytes: the workspace decode_attend needs."""
    n = lib().mla_decode_attend_workspace_bytes(int(batch), int(qlen), int(heads), int(num_workers))
    if n < 0:
        _check(-n, "mla_decode_attend_workspace_bytes")
    return int(n)


def _attend_args(q, kv_cache, kv_indptr, kv_indices, o, lse, *, qlen, heads, sm_scale, kv_scale, num_splits,
                 num_workers, split_min_tokens, kv_indptr_host):
    S = q.shape[0]
    batch = kv_indptr.shape[0] - 1
    if S != batch * qlen:
        raise MlaError("q has %d rows, expected batch*qlen = %d" % (S, batch * qlen))
    if q.shape[-1] != D_QK or q.shape[1] < heads:
        raise MlaError("q must be [S, >=heads, 576]")
    if o.shape[0] < S or o.shape[1] < heads or o.shape[2] != D_LATENT:
        raise MlaError("o must be [S, >=heads, 512]")
    if lse is not None and (lse.shape[0] < S or lse.shape[1] < heads):
        raise MlaError("lse must be [S, >=heads]")
    ih = np.ascontiguousarray(kv_indptr_host, dtype=np.int32)
    if ih.shape != (batch + 1,):
        raise MlaError("kv_indptr_host must hold batch+1 offsets")
    head = (_dev(q, "q", _BF16), q.stride(0), q.stride(1), batch, qlen, heads, _dev(kv_cache, "kv_cache", _U8),
            kv_cache.shape[0], _dev(kv_indptr, "kv_indptr", (torch.int32,)),
            _dev(kv_indices, "kv_indices", (torch.int32,)), float(sm_scale), float(kv_scale), int(num_splits),
            int(num_workers), int(split_min_tokens), ih.ctypes.data_as(ctypes.c_void_p),
            _dev(o, "o", _BF16), o.stride(0), o.stride(1))
    tail = ((_dev(lse, "lse", (torch.float32,)), lse.stride(0), lse.stride(1)) if lse is not None
            else (None, 0, 0))
    return head + tail, ih


def decode_attend(q: torch.Tensor, kv_cache: torch.Tensor, kv_indptr: torch.Tensor, kv_indices: torch.Tensor,
                  o: torch.Tensor, lse: torch.Tensor | None, workspace: torch.Tensor, kv_indptr_host: np.ndarray, *,
                  qlen: int, heads: int, sm_scale: float, kv_scale: float, num_splits: int,
                  num_workers: int = 256, split_min_tokens: int = 256) -> None:
    """mla_decode_attend: the partials and their LSE merge in one launch ->
    o [S, heads, 512] bf16 (the merged latent) and lse [S, heads] f32 (or
    None), bit for bit decode_partial (host plan) + merge_lse.  workspace: a
    uint8 device tensor of at least decode_attend_workspace_bytes bytes whose
    counter part is zero before its first use (torch.zeros)."""
    args, ih = _attend_args(q, kv_cache, kv_indptr, kv_indices, o, lse, qlen=qlen, heads=heads, sm_scale=sm_scale,
                            kv_scale=kv_scale, num_splits=num_splits, num_workers=num_workers,
                            split_min_tokens=split_min_tokens, kv_indptr_host=kv_indptr_host)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise MlaError("workspace must be a contiguous uint8 tensor")
    st = lib().mla_decode_attend(*args, _dev(workspace, "workspace", _U8), workspace.numel(), _stream())
    _check(st, "mla_decode_attend")


def decode_attend_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, kv_indptr: torch.Tensor,
                          kv_indices: torch.Tensor, o: torch.Tensor, lse: torch.Tensor | None,
                          kv_indptr_host: np.ndarray, *, qlen: int, heads: int, sm_scale: float, kv_scale: float,
                          num_splits: int, num_workers: int = 256, split_min_tokens: int = 256) -> None:
    """mla_decode_attend_noalloc: decode_attend on the library's own
    workspace (for callers that cannot allocate); same outputs."""
    args, ih = _attend_args(q, kv_cache, kv_indptr, kv_indices, o, lse, qlen=qlen, heads=heads, sm_scale=sm_scale,
                            kv_scale=kv_scale, num_splits=num_splits, num_workers=num_workers,
                            split_min_tokens=split_min_tokens, kv_indptr_host=kv_indptr_host)
    st = lib().mla_decode_attend_noalloc(*args, _stream())
    _check(st, "mla_decode_attend_noalloc")


def split_plan(kv_indptr, num_splits: int, num_workers: int, split_min_tokens: int):
    """Host-side split partition (no GPU): returns (bounds [B, splits+1] int32, chunk)."""
    indptr = np.ascontiguousarray(np.asarray(kv_indptr), dtype=np.int32)
    batch = indptr.shape[0] - 1
    bounds = np.zeros((batch, num_splits + 1), dtype=np.int32)
    chunk = ctypes.c_int64(0)
    st = lib().mla_split_plan(indptr.ctypes.data_as(ctypes.c_void_p), batch, num_splits, num_workers,
                              split_min_tokens, bounds.ctypes.data_as(ctypes.c_void_p), ctypes.byref(chunk))
    _check(st, "mla_split_plan")
    return bounds, int(chunk.value)


def time_next_partial(start: torch.cuda.Event | None, stop: torch.cuda.Event | None) -> None:
    """The next partial-kernel launch records `start` and `stop` (timing
    events, already created: recorded once) at its own start and end, so
    start.elapsed_time(stop) is the kernel's duration.  None, None clears."""
    handles = []
    for e in (start, stop):
        if e is not None and not e.cuda_event:
            raise MlaError("time_next_partial: record the event once first (it is created on first use)")
        handles.append(ctypes.c_void_p(e.cuda_event if e is not None else 0))
    _check(lib().mla_time_next_partial(*handles), "mla_time_next_partial")


def merge_lse(o_part: torch.Tensor, lse_part: torch.Tensor, o: torch.Tensor, lse: torch.Tensor | None = None) -> None:
    """LSE merge: o_part [splits, rows, heads, 512], lse_part [splits, rows, heads]
    -> o [rows, heads, 512] bf16 (+ lse [rows, heads] f32)."""
    ns, rows, heads = lse_part.shape
    if o.shape[0] < rows or o.shape[1] < heads:
        raise MlaError("bad output shape")
    lp = 0 if lse is None else _dev(lse, "lse", (torch.float32,))
    st = lib().mla_merge_lse(
        _dev(o_part, "o_part", _BF16), o_part.stride(0), o_part.stride(1), o_part.stride(2),
        _dev(lse_part, "lse_part", (torch.float32,)), lse_part.stride(0), lse_part.stride(1),
        lse_part.stride(2), ns, rows, heads, _dev(o, "o", _BF16), o.stride(0), o.stride(1),
        ctypes.c_void_p(lp), 0 if lse is None else lse.stride(0), 0 if lse is None else lse.stride(1),
        _stream())
    _check(st, "mla_merge_lse")


def value_gate(latent: torch.Tensor, gate: torch.Tensor, lengths: torch.Tensor, out: torch.Tensor, *,
               qlen: int, w_uv: torch.Tensor | None = None, w_fp4: torch.Tensor | None = None,
               w_scale: torch.Tensor | None = None) -> None:
    """W_UV + sigmoid gate: latent [rows, heads, 512] bf16 -> out [rows, heads*128] bf16.
    Weights: w_uv bf16 [heads, 128, 512], or w_fp4 u8 [heads, 128, 256] with
    w_scale u8 [heads, 128, 16]."""
    rows, heads = latent.shape[0], latent.shape[1]
    if w_uv is not None:
        fmt, wp, wh, wv = W_BF16, _dev(w_uv, "w_uv", _BF16), w_uv.stride(0), w_uv.stride(1)
        sp, sh, sv = 0, 0, 0
        if w_uv.shape[0] < heads or w_uv.shape[1] != D_V or w_uv.shape[2] != D_LATENT:
            raise MlaError("w_uv must be [heads, 128, 512]")
    else:
        fmt, wp, wh, wv = W_MXFP4, _dev(w_fp4, "w_fp4", (torch.uint8,)), w_fp4.stride(0), w_fp4.stride(1)
        sp, sh, sv = _dev(w_scale, "w_scale", (torch.uint8,)), w_scale.stride(0), w_scale.stride(1)
        if w_fp4.shape[0] < heads or w_fp4.shape[1] != D_V or w_fp4.shape[2] != D_LATENT // 2:
            raise MlaError("w_fp4 must be [heads, 128, 256]")
    st = lib().mla_value_gate(
        _dev(latent, "latent", _BF16), latent.stride(0), latent.stride(1), fmt, ctypes.c_void_p(wp), wh, wv,
        ctypes.c_void_p(sp), sh, sv, _dev(gate, "gate", _BF16), gate.stride(0),
        _dev(lengths, "lengths", (torch.int32,)), rows, qlen, heads, _dev(out, "out", _BF16), out.stride(0),
        _stream())
    _check(st, "mla_value_gate")


def _weights(heads, w_uv, w_fp4, w_scale):
    if w_uv is not None:
        if w_uv.shape[0] < heads or w_uv.shape[1] != D_V or w_uv.shape[2] != D_LATENT:
            raise MlaError("w_uv must be [heads, 128, 512]")
        return W_BF16, _dev(w_uv, "w_uv", _BF16), w_uv.stride(0), w_uv.stride(1), 0, 0, 0
    if w_fp4.shape[0] < heads or w_fp4.shape[1] != D_V or w_fp4.shape[2] != D_LATENT // 2:
        raise MlaError("w_fp4 must be [heads, 128, 256]")
    return (W_MXFP4, _dev(w_fp4, "w_fp4", (torch.uint8,)), w_fp4.stride(0), w_fp4.stride(1),
            _dev(w_scale, "w_scale", (torch.uint8,)), w_scale.stride(0), w_scale.stride(1))


def merge_value_gate(o_part: torch.Tensor, lse_part: torch.Tensor, gate: torch.Tensor, lengths: torch.Tensor,
                     out: torch.Tensor, *, qlen: int, w_uv: torch.Tensor | None = None,
                     w_fp4: torch.Tensor | None = None, w_scale: torch.Tensor | None = None,
                     lse: torch.Tensor | None = None) -> None:
    """Merge of the partials (o_part [splits, rows, heads, 512], lse_part
    [splits, rows, heads]) fused with W_UV + gate -> out [rows, heads*128]
    bf16 (+ the merged lse [rows, heads] f32); the latent is not written."""
    ns, rows, heads = lse_part.shape
    fmt, wp, wh, wv, sp, sh, sv = _weights(heads, w_uv, w_fp4, w_scale)
    lp = 0 if lse is None else _dev(lse, "lse", (torch.float32,))
    st = lib().mla_merge_value_gate(
        _dev(o_part, "o_part", _BF16), o_part.stride(0), o_part.stride(1), o_part.stride(2),
        _dev(lse_part, "lse_part", (torch.float32,)), lse_part.stride(0), lse_part.stride(1), lse_part.stride(2),
        ns, fmt, ctypes.c_void_p(wp), wh, wv, ctypes.c_void_p(sp), sh, sv, _dev(gate, "gate", _BF16),
        gate.stride(0), _dev(lengths, "lengths", (torch.int32,)), rows, qlen, heads, _dev(out, "out", _BF16),
        out.stride(0), ctypes.c_void_p(lp), 0 if lse is None else lse.stride(0),
        0 if lse is None else lse.stride(1), _stream())
    _check(st, "mla_merge_value_gate")

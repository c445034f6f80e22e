"""CPU oracle for MLA decode over an fp8 latent KV cache.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this
package.  The arithmetic lives in ``mla_oracle.c`` (plain C, IEEE double,
OpenMP over independent rows); this module builds it with gcc and marshals
numpy arrays.  It shares no code with the GPU library.

Sources: the vLLM API pages "vllm.models.kimi_k3.amd.specialized_decode.
runtime.mla" (sections ``attend``, ``m1c_inputs``, ``post``, ``pre``) and
"vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.mla.value"
(``MlaValue``, ``MlaGate``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_ASAN_LIB_PATH = os.path.join(_HERE, "liboracle_asan.so")
# MLA_ORACLE_LIBRARY names a prebuilt oracle to load instead (the
# AddressSanitizer + UndefinedBehaviorSanitizer build of the CPU tests)
_LIB_OVERRIDE = os.environ.get("MLA_ORACLE_LIBRARY")

D_LATENT, D_ROPE, D_QK, D_V = 512, 64, 576, 128


def build_sanitized() -> str:
    """The oracle built with gcc's AddressSanitizer and UndefinedBehaviorSanitizer
    (any finding aborts); load it into a process that preloads libasan."""
    tmp = _ASAN_LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _ASAN_LIB_PATH)
    return _ASAN_LIB_PATH


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            path = _LIB_OVERRIDE
        else:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            path = _LIB_PATH
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.orc_fp8_decode.argtypes = [ctypes.c_uint8]
        L.orc_fp8_decode.restype = f64
        L.orc_fp8_encode.argtypes = [f64]
        L.orc_fp8_encode.restype = ctypes.c_uint8
        L.orc_bf16_decode.argtypes = [ctypes.c_uint16]
        L.orc_bf16_decode.restype = f64
        L.orc_bf16_round.argtypes = [f64]
        L.orc_bf16_round.restype = ctypes.c_uint16
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_decode.restype = f64
        L.orc_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_decode.restype = f64
        L.orc_kv_write.argtypes = [P, i64, P, i64, P, i32, P, f32]
        L.orc_kv_write.restype = None
        L.orc_concat_quant_fp8.argtypes = [P, P, f32, i32, i32, P]
        L.orc_concat_quant_fp8.restype = None
        L.orc_split_bounds.argtypes = [P, i32, i32, i32, i32, P]
        L.orc_split_bounds.restype = i64
        L.orc_decode_partial.argtypes = [P, i32, i32, i32, P, P, P, P, i32, f64, f64, P, P]
        L.orc_decode_partial.restype = None
        L.orc_decode_partial_q8.argtypes = [P, f64, i32, i32, i32, P, P, P, P, i32, f64, f64, P, P]
        L.orc_decode_partial_q8.restype = None
        L.orc_merge_lse.argtypes = [P, P, i32, i64, i32, P, P]
        L.orc_merge_lse.restype = None
        L.orc_value_gate.argtypes = [P, P, P, P, P, P, i32, i32, i32, P, P]
        L.orc_value_gate.restype = None
        L.orc_mxfp4_block.argtypes = [P, P]
        L.orc_mxfp4_block.restype = None
        L.orc_absorb_query.argtypes = [P, P, P, P, i32, i32, i32, f32, P, P]
        L.orc_absorb_query.restype = None
        L.orc_bf16_round_array.argtypes = [P, P, i64]
        L.orc_bf16_round_array.restype = None
        L.orc_fp8_encode_array.argtypes = [P, P, i64]
        L.orc_fp8_encode_array.restype = None
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ codecs

def fp8_decode(codes) -> np.ndarray:
    """fp8 E4M3 (OCP fn) bytes -> float64, elementwise."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().orc_fp8_decode(b) for b in range(256)], dtype=np.float64)
    return table[codes]


def fp8_encode(values) -> np.ndarray:
    """float64 -> fp8 E4M3 bytes (nearest-even, saturating to +-448)."""
    v = _c(values, np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_fp8_encode_array(_p(v), _p(out), v.size)
    return out


def bf16_decode(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_round(values) -> np.ndarray:
    """float64 -> bf16 bits, nearest-even (the oracle's own rounding)."""
    v = _c(values, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_bf16_round_array(_p(v), _p(out), v.size)
    return out


def e2m1_decode(nibbles) -> np.ndarray:
    n = np.asarray(nibbles, dtype=np.uint8)
    table = np.array([lib().orc_e2m1_decode(b) for b in range(16)], dtype=np.float64)
    return table[n & 0xF]


def e8m0_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().orc_e8m0_decode(b) for b in range(256)], dtype=np.float64)
    return table[c]


# -------------------------------------------------------------- the path

def kv_write(kv_c, k_pe, slot_mapping, kv_cache, kv_scale: float) -> np.ndarray:
    """Scatter n new tokens' rows into (a copy of) kv_cache [slots, 576] u8.

    kv_c [n, 512] and k_pe [n, 64] are bf16 bits (uint16); returns the new cache."""
    kv_c = _c(kv_c, np.uint16)
    k_pe = _c(k_pe, np.uint16)
    slots = _c(slot_mapping, np.int64)
    out = np.array(kv_cache, dtype=np.uint8, copy=True, order="C")
    n = slots.shape[0]
    lib().orc_kv_write(_p(kv_c), D_LATENT, _p(k_pe), D_ROPE, _p(slots), n, _p(out),
                       ctypes.c_float(kv_scale))
    return out


def concat_quant_fp8(ql_nope, q_pe, q_scale: float) -> np.ndarray:
    """fp8 query codes [rows, H, 576] u8 of E(cat(ql_nope, q_pe) / q_scale);
    ql_nope [rows, H, 512] and q_pe [rows, H, 64] are bf16 bits (uint16)."""
    ql = _c(ql_nope, np.uint16)
    pe = _c(q_pe, np.uint16)
    rows, heads = ql.shape[0], ql.shape[1]
    assert ql.shape == (rows, heads, D_LATENT) and pe.shape == (rows, heads, D_ROPE)
    out = np.empty((rows, heads, D_QK), dtype=np.uint8)
    lib().orc_concat_quant_fp8(_p(ql), _p(pe), ctypes.c_float(q_scale), rows, heads, _p(out))
    return out


# stream positions each request takes before its tokens in the split
# partition (the C oracle's ORC_PIECE_TOKENS)
PIECE_TOKENS = 320


def split_bounds(indptr, num_splits: int, num_workers: int, split_min_tokens: int):
    """Split-KV partition: returns (bounds [batch, num_splits+1] int32, chunk)."""
    indptr = _c(indptr, np.int32)
    batch = indptr.shape[0] - 1
    b = np.zeros((batch, num_splits + 1), dtype=np.int32)
    chunk = lib().orc_split_bounds(_p(indptr), batch, num_splits, num_workers, split_min_tokens, _p(b))
    return b, int(chunk)


def decode_partial(q, kv_cache, indptr, indices, bounds, qlen: int, sm_scale: float, kv_scale: float,
                   q_scale: float | None = None):
    """Exact split partials.  q [S, H, 576]: bf16 bits (uint16), or fp8 E4M3
    codes (uint8) standing for q_scale * D(q8) when q_scale is given.
    Returns (o f64 [splits, S, H, 512], lse f64 [splits, S, H]); o is NOT
    rounded."""
    fp8_q = q_scale is not None
    q = _c(q, np.uint8 if fp8_q else np.uint16)
    S, H, D = q.shape
    assert D == D_QK
    kv = _c(kv_cache, np.uint8)
    indptr = _c(indptr, np.int32)
    indices = _c(indices, np.int32)
    bounds = _c(bounds, np.int32)
    batch = indptr.shape[0] - 1
    assert S == batch * qlen
    ns = bounds.shape[1] - 1
    o = np.empty((ns, S, H, D_LATENT), dtype=np.float64)
    lse = np.empty((ns, S, H), dtype=np.float64)
    if fp8_q:
        lib().orc_decode_partial_q8(_p(q), float(q_scale), batch, qlen, H, _p(kv), _p(indptr), _p(indices),
                                    _p(bounds), ns, float(sm_scale), float(kv_scale), _p(o), _p(lse))
    else:
        lib().orc_decode_partial(_p(q), batch, qlen, H, _p(kv), _p(indptr), _p(indices), _p(bounds), ns,
                                 float(sm_scale), float(kv_scale), _p(o), _p(lse))
    return o, lse


def merge_lse(o_part, lse_part):
    """LSE merge.  o_part [splits, S, H, 512] bf16 bits, lse_part f32.
    Returns (o f64 [S, H, 512], lse f64 [S, H]); o is NOT rounded."""
    o_part = _c(o_part, np.uint16)
    lse_part = _c(lse_part, np.float32)
    ns, S, H, D = o_part.shape
    o = np.empty((S, H, D), dtype=np.float64)
    lse = np.empty((S, H), dtype=np.float64)
    lib().orc_merge_lse(_p(o_part), _p(lse_part), ns, S, H, _p(o), _p(lse))
    return o, lse


def value_gate(latent, gate, lengths, qlen: int, w_bf16=None, w_fp4=None, w_scale=None):
    """W_UV + sigmoid gate.  latent [S, H, 512] bf16 bits; gate [S, H*128]
    bf16 bits; w_bf16 [H, 128, 512] bf16 bits or (w_fp4 [H, 128, 256] u8,
    w_scale [H, 128, 16] u8).  Returns (acc f64 [S, H*128], out bf16 bits)."""
    latent = _c(latent, np.uint16)
    S, H, D = latent.shape
    gate = _c(gate, np.uint16)
    lengths = _c(lengths, np.int32)
    batch = lengths.shape[0]
    assert S == batch * qlen
    if w_bf16 is not None:
        w_bf16 = _c(w_bf16, np.uint16)
    else:
        w_fp4 = _c(w_fp4, np.uint8)
        w_scale = _c(w_scale, np.uint8)
    acc = np.empty((S, H * D_V), dtype=np.float64)
    out = np.empty((S, H * D_V), dtype=np.uint16)
    lib().orc_value_gate(_p(latent), _p(w_bf16), _p(w_fp4), _p(w_scale), _p(gate), _p(lengths),
                         batch, qlen, H, _p(acc), _p(out))
    return acc, out


def mxfp4_block(values) -> np.ndarray:
    """One block of 32 values -> its MXFP4 quantisation, dequantised (f64)."""
    v = _c(np.asarray(values, np.float64).reshape(32), np.float64)
    out = np.empty(32, np.float64)
    lib().orc_mxfp4_block(_p(v), _p(out))
    return out


def absorb_query(q_nope, q_pe, w_k, w_scale, fp8: bool = False, q_scale: float = 1.0):
    """The absorbed query: q_nope [rows, H, 128] and q_pe [rows, H, 64] bf16
    bits, W_K codes [H, 512, 64] u8 and scales [H, 512, 4] u8.  Returns (y f64
    [rows, H, 512] exact products, out [rows, H, 576] bf16 bits or fp8 codes)."""
    q_nope = _c(q_nope, np.uint16)
    rows, heads, k = q_nope.shape
    assert k == 128
    q_pe = _c(q_pe, np.uint16)
    assert q_pe.shape == (rows, heads, D_ROPE)
    w_k = _c(w_k, np.uint8)
    w_scale = _c(w_scale, np.uint8)
    assert w_k.shape == (heads, D_LATENT, 64) and w_scale.shape == (heads, D_LATENT, 4)
    y = np.empty((rows, heads, D_LATENT), np.float64)
    out = np.empty((rows, heads, D_QK), np.uint8 if fp8 else np.uint16)
    lib().orc_absorb_query(_p(q_nope), _p(q_pe), _p(w_k), _p(w_scale), rows, heads, 1 if fp8 else 0,
                           float(q_scale), _p(out), _p(y))
    return y, out


def num_threads() -> int:
    return int(lib().orc_num_threads())

"""ctypes wrapper around the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product library or its binding.
It shares no code with the HIP path.

The oracle computes, in plain loops:
  * the OCP E4M3FN codec (decode, round-to-nearest-even saturating encode)
    and the symmetric INT8 codec (round half to even, clamp to +-127);
  * per-row quantization: s = fl32(amax/448), codes = encode(fl32(x/s))
    (INT8: s = fl32(amax/127));
  * decode attention in fp64 over the dequantized page-size-1 pool, for head
    dim 128 or 256, one or more causal query rows per request and an
    optional sliding window;
  * prefill reconstruction bf16_rne(fl32(decode(c)*s)) and fp64 causal
    prefill attention over [workspace prefix ; bf16 chunk];
  * KV byte accounting per token and for the shared bf16 workspace.
Page citations live in oracle.c next to each function.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_lib: Optional[ctypes.CDLL] = None
HEAD_DIM = 128        # prefill and the default everywhere
HEAD_DIMS = (128, 256)  # head dims of the pool, quantize and decode
FORMATS = {"e4m3": 0, "int8": 1}  # KV code formats

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_int8_encode.argtypes = [ctypes.c_float]
        L.oracle_int8_encode.restype = ctypes.c_int8
        L.oracle_int8_decode.argtypes = [ctypes.c_uint8]
        L.oracle_int8_decode.restype = ctypes.c_double
        L.oracle_quantize_rows.argtypes = [_u16p, _i64, _i32, _i32, _u8p, _f32p]
        L.oracle_quantize_rows.restype = _i32
        L.oracle_decode_attention.argtypes = [
            _u16p, _i32, _i32, _i32, _i32, _i32, _i32, _u8p, _u8p, _f32p, _f32p, _i64, _i64,
            _i32p, _i64, _i32p, _i32, ctypes.c_float, _f64p]
        L.oracle_decode_attention.restype = _i32
        L.oracle_reconstruct.argtypes = [_u8p, _f32p, _i64, _i64, _i32, _i32, _i32, _i32p, _i64, _u16p]
        L.oracle_reconstruct.restype = None
        L.oracle_prefill_attention.argtypes = [
            _u16p, _u16p, _u16p, _u16p, _u16p, _i32, _i32, _i32, _i32, ctypes.c_float,
            _i32p, _i32, _f64p]
        L.oracle_prefill_attention.restype = None
        for name in ("oracle_fp8_bytes_per_token", "oracle_bf16_bytes_per_token"):
            getattr(L, name).argtypes = [_i32, _i32, _i32]
            getattr(L, name).restype = _i64
        L.oracle_bf16_workspace_bytes.argtypes = [_i64, _i32, _i32]
        L.oracle_bf16_workspace_bytes.restype = _i64
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = _i32
        L.oracle_set_num_threads.argtypes = [_i32]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Host threads for later oracle calls from this thread (timing only)."""
    lib().oracle_set_num_threads(int(n))


# ------------------------------------------------------------------ codec --

def e4m3_decode(code: int) -> float:
    return float(lib().oracle_e4m3_decode(int(code) & 0xFF))


def e4m3_decode_table() -> np.ndarray:
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y: float) -> int:
    return int(lib().oracle_e4m3_encode(float(np.float32(y))))


def e4m3_encode_array(y: np.ndarray) -> np.ndarray:
    f = lib().oracle_e4m3_encode
    return np.array([f(float(v)) for v in np.asarray(y, np.float32).ravel()],
                    dtype=np.uint8).reshape(np.shape(y))


def int8_encode(y: float) -> int:
    return int(lib().oracle_int8_encode(float(np.float32(y))))


def int8_decode(code: int) -> float:
    return float(lib().oracle_int8_decode(int(code) & 0xFF))


def code_values(fmt: str = "e4m3") -> np.ndarray:
    """Value of every code byte in a format (fp64)."""
    f = e4m3_decode if fmt == "e4m3" else int8_decode
    return np.array([f(c) for c in range(256)], dtype=np.float64)


def f32_to_bf16(x: float) -> int:
    return int(lib().oracle_f32_to_bf16(float(np.float32(x))))


# --------------------------------------------------------------- quantize --

def quantize_rows(rows_bf16: np.ndarray, fmt: str = "e4m3"):
    """rows_bf16: [..., D] uint16 (D = 128 or 256) -> (codes uint8 [..., D], scales float32 [...]).
    fmt: "e4m3" (s = amax/448) or "int8" (s = amax/127)."""
    r = np.ascontiguousarray(rows_bf16, dtype=np.uint16)
    shape = r.shape[:-1]
    D = r.shape[-1]
    assert D in HEAD_DIMS
    n = int(np.prod(shape)) if shape else 1
    flat = r.reshape(n, D)
    codes = np.empty((n, D), np.uint8)
    scales = np.empty(n, np.float32)
    assert lib().oracle_quantize_rows(flat, n, D, FORMATS[fmt], codes, scales) == 0
    return codes.reshape(*shape, D), scales.reshape(shape)


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """decode(c) * s in fp64, broadcast over the last (head-dim) axis."""
    t = e4m3_decode_table() if fmt == "e4m3" else code_values("int8")
    return t[np.asarray(codes, np.uint8)] * np.asarray(scales, np.float64)[..., None]


# ------------------------------------------------------------- attention --

def decode_attention(q, k_codes, v_codes, k_scales, v_scales, table, seq_lens, sm_scale,
                     n_kv_heads: int, window: int = 0, fmt: str = "e4m3") -> np.ndarray:
    """fp64 decode attention.

    q: uint16 [B][Hq][D] (one query row per request) or [B][n_qrows][Hq][D]
    (the request's last n_qrows positions, each causal); D = 128 or 256.
    k_codes/v_codes: uint8 [R][Hkv][D]; k_scales/v_scales: float32 [R][Hkv];
    table: int32 [B][stride]; seq_lens int32 [B]; window > 0 limits the query
    at position p to positions p-window+1 .. p; fmt: the code format.
    Returns float64 with q's shape.
    """
    q = np.ascontiguousarray(q, np.uint16)
    single = q.ndim == 3
    q4 = q[:, None] if single else q
    B, NQ, Hq, D = q4.shape
    assert D in HEAD_DIMS
    kc = np.ascontiguousarray(k_codes, np.uint8)
    vc = np.ascontiguousarray(v_codes, np.uint8)
    assert kc.shape[-1] == D and vc.shape[-1] == D
    ks = np.ascontiguousarray(k_scales, np.float32)
    vs = np.ascontiguousarray(v_scales, np.float32)
    tb = np.ascontiguousarray(table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    out = np.zeros((B, NQ, Hq, D), np.float64)
    rc = lib().oracle_decode_attention(np.ascontiguousarray(q4), B, NQ, Hq, n_kv_heads, D, FORMATS[fmt],
                                       kc.reshape(-1), vc.reshape(-1), ks.reshape(-1), vs.reshape(-1),
                                       n_kv_heads * D, n_kv_heads, tb.reshape(-1), tb.shape[1], sl,
                                       int(window), float(sm_scale), out)
    assert rc == 0
    return out[:, 0] if single else out


def reconstruct(codes, scales, rows, n_kv_heads: int, fmt: str = "e4m3") -> np.ndarray:
    """bf16 workspace [P][Hkv][D] (uint16 bits) for pool rows `rows`."""
    c = np.ascontiguousarray(codes, np.uint8)
    D = c.shape[-1]
    s = np.ascontiguousarray(scales, np.float32)
    r = np.ascontiguousarray(rows, np.int32)
    ws = np.empty((r.size, n_kv_heads, D), np.uint16)
    lib().oracle_reconstruct(c.reshape(-1), s.reshape(-1), n_kv_heads * D, n_kv_heads,
                             n_kv_heads, D, FORMATS[fmt], r, r.size, ws)
    return ws


def prefill_attention(q, ws_k, ws_v, k_cur, v_cur, sm_scale, q_idx=None) -> np.ndarray:
    """fp64 causal prefill attention for the chunk queries in q_idx (default: all).

    q: [T][Hq][128]; ws_k/ws_v: [P][Hkv][128]; k_cur/v_cur: [T][Hkv][128] (uint16 bf16 bits).
    Returns float64 [len(q_idx)][Hq][128].
    """
    q = np.ascontiguousarray(q, np.uint16)
    T, Hq, _ = q.shape
    k_cur = np.ascontiguousarray(k_cur, np.uint16)
    v_cur = np.ascontiguousarray(v_cur, np.uint16)
    Hkv = k_cur.shape[1]
    P = 0 if ws_k is None else ws_k.shape[0]
    wk = np.zeros((max(P, 1), Hkv, HEAD_DIM), np.uint16) if P == 0 else np.ascontiguousarray(ws_k, np.uint16)
    wv = np.zeros((max(P, 1), Hkv, HEAD_DIM), np.uint16) if P == 0 else np.ascontiguousarray(ws_v, np.uint16)
    idx = np.arange(T, dtype=np.int32) if q_idx is None else np.ascontiguousarray(q_idx, np.int32)
    out = np.zeros((idx.size, Hq, HEAD_DIM), np.float64)
    lib().oracle_prefill_attention(q, wk, wv, k_cur, v_cur, P, T, Hq, Hkv, float(sm_scale),
                                   idx, idx.size, out)
    return out


# ------------------------------------------------------------- accounting --

def fp8_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int = HEAD_DIM) -> int:
    return int(lib().oracle_fp8_bytes_per_token(n_layers, n_kv_heads, head_dim))


def bf16_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int = HEAD_DIM) -> int:
    return int(lib().oracle_bf16_bytes_per_token(n_layers, n_kv_heads, head_dim))


def bf16_workspace_bytes(n_rows: int, n_kv_heads: int, head_dim: int = HEAD_DIM) -> int:
    return int(lib().oracle_bf16_workspace_bytes(n_rows, n_kv_heads, head_dim))

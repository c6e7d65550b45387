"""CPU oracle for the block-quantized KV cache and decode attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product package. It shares no code with
the HIP library. See kvq_oracle.cpp for the definitions and the pages they follow.

All arrays are numpy. fp16 data is passed as numpy float16 (bit patterns are read
by the oracle's own binary16 decoder).
"""
import ctypes
import os

import numpy as np

from . import build as _build

BLOCK = 64
INT4_SYM = 0
UINT8_ASYM = 1
FP8_E4M3 = 2

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_version.restype = ctypes.c_int
        L.oracle_half_to_float.argtypes = [P, P, i64]
        L.oracle_half_to_float.restype = None
        L.oracle_quantize_cache.argtypes = [i32] * 5 + [P, P, i64, i64, i64, P] + [P] * 6
        L.oracle_quantize_cache.restype = ctypes.c_int
        L.oracle_append.argtypes = [i32] * 5 + [P, P, i64, i64, i64, P] + [P] * 6
        L.oracle_append.restype = ctypes.c_int
        L.oracle_attention.argtypes = [i32] * 5 + [P] * 6 + [P, P, ctypes.c_double, i64,
                                                             i64, P]
        L.oracle_attention.restype = ctypes.c_int
        L.oracle_e4m3_code.argtypes = [P, P, i64]
        L.oracle_e4m3_code.restype = None
        L.oracle_e4m3_value.argtypes = [P, P, i64]
        L.oracle_e4m3_value.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def row_bytes(scheme, D):
    return D // 2 if scheme == INT4_SYM else D


def half_to_float(bits):
    """binary16 bit patterns (uint16 array) -> float32 values, by the oracle's decoder."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    lib().oracle_half_to_float(_ptr(bits), _ptr(out), bits.size)
    return out


def e4m3_code(x):
    """float32 array -> uint8 FP8 E4M3 codes (nearest, ties to even, saturating)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_e4m3_code(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_value(codes):
    """uint8 FP8 E4M3 codes -> float64 values."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    lib().oracle_e4m3_value(_ptr(codes), _ptr(out), codes.size)
    return out


def empty_cache(scheme, B, H, D, max_blocks):
    """Zero-filled cache arrays in the oracle's layout."""
    rb = row_bytes(scheme, D)
    return {
        "scheme": scheme, "B": B, "H": H, "D": D, "max_blocks": max_blocks,
        "k_codes": np.zeros((B, H, max_blocks, BLOCK, rb), np.uint8),
        "v_codes": np.zeros((B, H, max_blocks, BLOCK, rb), np.uint8),
        "k_scale": np.zeros((B, H, max_blocks), np.float32),
        "v_scale": np.zeros((B, H, max_blocks), np.float32),
        "k_zero": np.zeros((B, H, max_blocks), np.float32),
        "v_zero": np.zeros((B, H, max_blocks), np.float32),
    }


def _strides_elems(x):
    if x.dtype != np.float16 or x.ndim != 4 or x.strides[3] != 2:
        raise ValueError("expected float16 [B][S][H][D] with contiguous D")
    return [s // 2 for s in x.strides[:3]]


def quantize_cache(scheme, k, v, lens, max_blocks, cache=None):
    """Quantizes blocks [0, ceil(len_b/64)) of every row of k, v (float16 [B][S][H][D],
    any strides with D contiguous). Returns (or fills) a cache dict."""
    B, S, H, D = k.shape
    if v.shape != k.shape or v.strides != k.strides:
        raise ValueError("k and v must share shape and strides")
    sb, st, sh = _strides_elems(k)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    if lens.shape != (B,) or (lens > S).any():
        raise ValueError("bad lens")
    c = cache if cache is not None else empty_cache(scheme, B, H, D, max_blocks)
    rc = lib().oracle_quantize_cache(
        scheme, B, H, D, max_blocks, _ptr(k), _ptr(v), sb, st, sh, _ptr(lens),
        _ptr(c["k_codes"]), _ptr(c["v_codes"]), _ptr(c["k_scale"]), _ptr(c["v_scale"]),
        _ptr(c["k_zero"]), _ptr(c["v_zero"]))
    if rc != 0:
        raise ValueError("oracle_quantize_cache rejected its arguments")
    return c


def append(cache, k_hist, v_hist, new_lens):
    """Re-quantizes the tail block (new_len-1)//64 of every row from the fp16 history."""
    B, S, H, D = k_hist.shape
    sb, st, sh = _strides_elems(k_hist)
    new_lens = np.ascontiguousarray(new_lens, dtype=np.int32)
    if (new_lens > S).any():
        raise ValueError("history shorter than new_lens")
    c = cache
    rc = lib().oracle_append(
        c["scheme"], B, H, D, c["max_blocks"], _ptr(k_hist), _ptr(v_hist), sb, st, sh,
        _ptr(new_lens), _ptr(c["k_codes"]), _ptr(c["v_codes"]), _ptr(c["k_scale"]),
        _ptr(c["v_scale"]), _ptr(c["k_zero"]), _ptr(c["v_zero"]))
    if rc != 0:
        raise ValueError("oracle_append rejected its arguments")
    return c


def attention(cache, q, lens, sm_scale, rows=None):
    """fp64 decode attention over the dequantized cache. q: float16 [B][H][D].
    rows: optional (begin, end) over the flattened (b, h) index; other rows are NaN."""
    c = cache
    B, H, D = c["B"], c["H"], c["D"]
    q = np.ascontiguousarray(q, dtype=np.float16)
    if q.shape != (B, H, D):
        raise ValueError("q shape")
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    r0, r1 = (0, B * H) if rows is None else rows
    out = np.full((B, H, D), np.nan, dtype=np.float64)
    for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
        if not c[key].flags.c_contiguous:
            raise ValueError(key + " must be contiguous")
    rc = lib().oracle_attention(
        c["scheme"], B, H, D, c["max_blocks"], _ptr(c["k_codes"]), _ptr(c["v_codes"]),
        _ptr(c["k_scale"]), _ptr(c["v_scale"]), _ptr(c["k_zero"]), _ptr(c["v_zero"]),
        _ptr(lens), _ptr(q), float(sm_scale), r0, r1, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return out


def dequantize(cache, b, h, length):
    """Dequantized K^ and V^ (float64 [length][D]) of row (b, h), straight from the
    cache layout: int4 (nibble - 8)*s with offset-binary nibbles (low nibble = even
    channel), uint8 (c - zp)*s, FP8 E4M3 value(c)*s."""
    c = cache
    D = c["D"]
    nb = (length + BLOCK - 1) // BLOCK
    out = []
    for which in ("k", "v"):
        codes = c[which + "_codes"][b, h, :nb].reshape(nb * BLOCK, -1)[:length]
        s = np.repeat(c[which + "_scale"][b, h, :nb].astype(np.float64), BLOCK)[:length]
        if c["scheme"] == INT4_SYM:
            vals = np.empty((length, D), np.int64)
            vals[:, 0::2] = (codes & 0x0F).astype(np.int64) - 8
            vals[:, 1::2] = (codes >> 4).astype(np.int64) - 8
            out.append(vals.astype(np.float64) * s[:, None])
        elif c["scheme"] == FP8_E4M3:
            out.append(e4m3_value(codes) * s[:, None])
        else:
            z = np.repeat(c[which + "_zero"][b, h, :nb].astype(np.float64), BLOCK)[:length]
            out.append((codes.astype(np.float64) - z[:, None]) * s[:, None])
    return out[0], out[1]

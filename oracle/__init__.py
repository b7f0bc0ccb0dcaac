"""Python access to the plain C oracle of the Engram forward pass.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product library never uses it.

``build()`` compiles ``engram_oracle.c`` with gcc into ``liboracle.so`` next to
it.  The wrappers take numpy arrays and return numpy arrays; floating-point
results are float64.  See ``engram_oracle.c`` for the definitions and the
passages of "Conditional Memory via Scalable Lookup" they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "engram_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build() -> str:
    """Compile the oracle (gcc, -O2, one thread) and return the library path."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                           "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_compress.argtypes = [P, i64, P, i32, P]
        L.oracle_compress.restype = i64
        L.oracle_hash.argtypes = [P, i32, i64, i64, i64, P, i32, i32, i32, P, P, i32, P]
        L.oracle_hash.restype = None
        L.oracle_gather.argtypes = [P, i64, i32, P, i32, P]
        L.oracle_gather.restype = None
        L.oracle_gate.argtypes = [P, i64, i32, i32, P, P, P, P, P, ctypes.c_double, i32, i32, P, P, P]
        L.oracle_gate.restype = ctypes.c_int
        L.oracle_conv.argtypes = [P, i32, i64, i32, P, P, i32, i32, ctypes.c_double, i32, P, P]
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_quant_rows.argtypes = [P, i64, i32, P, P]
        L.oracle_gate_fp8.argtypes = [P, i64, i32, i32, P, P, P, P, P, ctypes.c_double, i32, i32, P, P]
        L.oracle_gate_fp8.restype = ctypes.c_int
        L.oracle_conv.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def compress(raw: np.ndarray, cmap: np.ndarray):
    """Canonical ids (int32, same shape as raw; -1 where out of range) and the bad-id count."""
    raw = np.ascontiguousarray(raw, dtype=np.int32)
    cmap = np.ascontiguousarray(cmap, dtype=np.int32)
    out = np.empty_like(raw)
    bad = lib().oracle_compress(_p(raw), raw.size, _p(cmap), cmap.size, _p(out))
    return out, int(bad)


def hash_ids(ids: np.ndarray, orders: Sequence[int], heads: int, mult: np.ndarray,
             rows: np.ndarray, pad_id: int, t_begin: int = 0, t_count: int | None = None):
    """Hash indices [batch * t_count, len(orders) * heads] (int32) of positions
    t_begin .. t_begin + t_count - 1 of every row of ids [batch, ld]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    batch, ld = ids.shape
    if t_count is None:
        t_count = ld - t_begin
    orders_a = np.ascontiguousarray(orders, dtype=np.int32)
    mult = np.ascontiguousarray(mult, dtype=np.uint64)
    rows = np.ascontiguousarray(rows, dtype=np.uint32)
    n_tables = len(orders) * heads
    assert mult.shape == (len(orders), heads, max(orders)) and rows.shape == (n_tables,)
    idx = np.empty((batch * t_count, n_tables), dtype=np.int32)
    lib().oracle_hash(_p(ids), batch, ld, t_begin, t_count, _p(orders_a), len(orders), heads,
                      max(orders), _p(mult), _p(rows), pad_id, _p(idx))
    return idx


def gather(idx: np.ndarray, tables: Sequence[np.ndarray]):
    """Concatenated rows [n_tok, n_tables * w] (dtype of the tables); bitwise copies."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n_tok, n_tables = idx.shape
    assert len(tables) == n_tables
    tables = [np.ascontiguousarray(t) for t in tables]
    row_bytes = tables[0].shape[1] * tables[0].itemsize
    ptrs = (ctypes.c_void_p * n_tables)(*[t.ctypes.data for t in tables])
    out = np.empty((n_tok, n_tables * tables[0].shape[1]), dtype=tables[0].dtype)
    lib().oracle_gather(_p(idx), n_tok, n_tables, ptrs, row_bytes, _p(out))
    return out


KEY_NORM_MEMORY = 0      # k = W_K RMSNorm_gk(e), gk over d_mem (the review page's pseudocode)
KEY_NORM_PROJECTED = 1   # k = RMSNorm_gk(W_K e), gk over d_model (the paper's Eq. (4) / Eq. (6))


def gate(mem: np.ndarray, h: np.ndarray, wk: np.ndarray, wv: np.ndarray, gq: np.ndarray,
         gk: np.ndarray, eps: float, dtype: int, with_value: bool = False,
         key_norm: int = KEY_NORM_MEMORY):
    """One gating branch: (out [n_tok, d_model] float64, alpha [n_tok] float64), and the
    gated value alpha * v [n_tok, d_model] float64 as a third element when with_value.

    Arrays hold float32 values (dtype F32) or raw bfloat16 bits as uint16 (dtype BF16).
    gk has d_mem entries for KEY_NORM_MEMORY and d_model for KEY_NORM_PROJECTED.
    """
    mem, h, wk, wv, gq, gk = (np.ascontiguousarray(a) for a in (mem, h, wk, wv, gq, gk))
    n_tok, d_mem = mem.shape
    d_model = h.shape[1]
    assert h.shape[0] == n_tok and wk.shape == (d_model, d_mem) and wv.shape == (d_model, d_mem)
    assert gq.shape == (d_model,)
    assert gk.shape == ((d_mem,) if key_norm == KEY_NORM_MEMORY else (d_model,))
    want = np.float32 if dtype == F32 else np.uint16
    for a in (mem, h, wk, wv, gq, gk):
        assert a.dtype == want, a.dtype
    out = np.empty((n_tok, d_model), dtype=np.float64)
    alpha = np.empty(n_tok, dtype=np.float64)
    value = np.empty((n_tok, d_model), dtype=np.float64) if with_value else None
    rc = lib().oracle_gate(_p(mem), n_tok, d_mem, d_model, _p(h), _p(wk), _p(wv), _p(gq), _p(gk),
                           float(eps), dtype, key_norm, _p(out), _p(alpha), _p(value) if with_value else None)
    assert rc == 0, rc
    return (out, alpha, value) if with_value else (out, alpha)


def conv(value: np.ndarray, batch: int, seq: int, w: np.ndarray, gamma: np.ndarray, dil: int,
         eps: float, dtype: int, base: np.ndarray):
    """Eq. (5) convolution: base + SiLU(Conv1D(RMSNorm(value))) as float64 [batch*seq, d_model].

    value, base: float64 [batch*seq, d_model] (tokens b*seq + t); w: [d_model, taps] and
    gamma: [d_model] as float32 (F32) or bfloat16 bits (BF16)."""
    value = np.ascontiguousarray(value, dtype=np.float64)
    base = np.ascontiguousarray(base, dtype=np.float64)
    w, gamma = np.ascontiguousarray(w), np.ascontiguousarray(gamma)
    n_tok, d_model = value.shape
    taps = w.shape[1]
    assert n_tok == batch * seq and base.shape == value.shape and w.shape == (d_model, taps)
    assert gamma.shape == (d_model,)
    want = np.float32 if dtype == F32 else np.uint16
    assert w.dtype == want and gamma.dtype == want
    out = np.empty_like(value)
    lib().oracle_conv(_p(value), batch, seq, d_model, _p(w), _p(gamma), taps, dil, float(eps), dtype,
                      _p(base), _p(out))
    return out


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) quantization and the gate with FP8 projections

def e4m3_decode(codes) -> np.ndarray:
    """Values (float64) of E4M3 codes (uint8 array-like); NaN for 0x7F and 0xFF."""
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib().oracle_e4m3_decode(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_encode(values) -> np.ndarray:
    """Nearest E4M3 codes (ties to even, saturating at +-448) of float32 values."""
    v = np.asarray(values, dtype=np.float32)
    return np.array([lib().oracle_e4m3_encode(float(x)) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)


def quant_rows(x: np.ndarray):
    """Per-row FP8 quantization of float32 x [rows, cols]: (codes uint8 [rows, cols],
    scales float32 [rows]) with scale = max|row| / 448 in fp32 (1 for a zero row)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    codes = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty(rows, dtype=np.float32)
    lib().oracle_quant_rows(_p(x), rows, cols, _p(codes), _p(scales))
    return codes, scales


def gate_fp8(mem, h, wk, wv, gq, gk, eps: float, dtype: int, key_norm: int = KEY_NORM_MEMORY):
    """oracle.gate with both projections in FP8 (per-token / per-row scales):
    (out [n_tok, d_model] float64, alpha [n_tok] float64)."""
    mem, h, wk, wv, gq, gk = (np.ascontiguousarray(a) for a in (mem, h, wk, wv, gq, gk))
    n_tok, d_mem = mem.shape
    d_model = h.shape[1]
    assert wk.shape == (d_model, d_mem) and wv.shape == (d_model, d_mem) and gq.shape == (d_model,)
    assert gk.shape == ((d_mem,) if key_norm == KEY_NORM_MEMORY else (d_model,))
    out = np.empty((n_tok, d_model), dtype=np.float64)
    alpha = np.empty(n_tok, dtype=np.float64)
    rc = lib().oracle_gate_fp8(_p(mem), n_tok, d_mem, d_model, _p(h), _p(wk), _p(wv), _p(gq), _p(gk), float(eps),
                               dtype, key_norm, _p(out), _p(alpha))
    assert rc == 0, rc
    return out, alpha

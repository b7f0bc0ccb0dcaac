"""Engram forward pass on AMD Instinct MI355X: Python binding of libengram.so.

The work happens in the HIP kernels behind the C ABI declared in
``include/engram.h``; this module only marshals arguments (torch tensors give
device memory and stream handles) and turns non-OK statuses into exceptions.
The functions carry the C names:

* ``engram_compress``  -- tokenizer compression lookup ("Conditional Memory via
  Scalable Lookup", section 2.2);
* ``engram_hash``      -- multi-head multiply-XOR hashing of suffix n-grams
  (section 2.2, Eq. 1);
* ``engram_compress_hash`` -- both of the above in one kernel;
* ``engram_gather``    -- table lookup and concatenation (Eq. 1-2);
* ``engram_lookup``    -- compression, hashing and the gather in one kernel;
* ``engram_gate_forward`` -- context-aware gating and residual update
  (section 2.3, Eq. 3-4; section 2.4, Eq. 6 for several branches);
  ``fp8=True`` runs both projections on E4M3 codes (section 2.4);
* ``engram_lookup_gate`` -- the lookup and the gate in one pass, the gate's
  matrix-core kernel loading the table rows itself (section 2.2 into 2.3);
* ``engram_lookup_fp8``, ``engram_gate_prepare_fp8``, ``engram_gate_forward_fp8q``
  -- the FP8 gate's operands made once: the lookup quantizing its memory vectors,
  the weights quantized ahead, and the gate on the codes;
* ``engram_conv_forward`` -- the short depthwise causal convolution over the
  gated values (section 2.3, Eq. 5);
* ``engram_prefetch_host`` -- the same gather from pinned host-memory tables
  over PCIe (section 2.5, Figure 2(b); section 6.4);
* ``engram_cache_select`` / ``engram_cache_build`` / ``engram_prefetch_host_cached``
  -- an HBM cache of the most frequent rows in front of those tables (section 2.5).

There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libengram.so")

F32 = 0
BF16 = 1
MAX_TABLES = 32
MAX_ORDER = 4
MAX_BRANCHES = 8
KEY_NORM_MEMORY = 0      # k = W_K RMSNorm_gk(e), gk over d_mem (the review page's pseudocode)
KEY_NORM_PROJECTED = 1   # k = RMSNorm_gk(W_K e), gk over d_model (the paper's Eq. 4 / Eq. 6)
CONV_MAX_TAPS = 8
CONV_MAX_DILATION = 16
NOALLOC_SCRATCH_BYTES = 128 << 20   # ENGRAM_NOALLOC_SCRATCH_BYTES

_STATUS = {0: "ENGRAM_OK", 1: "ENGRAM_ERR_INVALID_ARG", 2: "ENGRAM_ERR_UNSUPPORTED", 3: "ENGRAM_ERR_HIP"}

# names exported by include/engram.h
EXPORTS = (
    "engram_last_error", "engram_version", "engram_compress", "engram_hash", "engram_gather",
    "engram_gate_forward", "engram_conv_forward", "engram_prefetch_host", "engram_host_alloc",
    "engram_host_free", "engram_cache_select", "engram_cache_build", "engram_prefetch_host_cached",
    "engram_compress_hash", "engram_quantize_fp8", "engram_gate_forward_fp8", "engram_lookup",
    "engram_lookup_fp8", "engram_gate_prepare_fp8", "engram_gate_forward_fp8q", "engram_gate_prepare",
    "engram_gate_forward_prepared", "engram_gate_wait_timeouts", "engram_debug_force_gate_timeout",
    "engram_debug_gate_key_form",
    "engram_gate_forward_noalloc", "engram_lookup_gate",
)


class EngramError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libengram.so (built by ``build.build()``); raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m hashed_gram_embedding_hash_amd.build`")
        # torch first, so the library binds to the HIP runtime torch already loaded
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        st = ctypes.c_int
        L.engram_last_error.restype = ctypes.c_char_p
        L.engram_last_error.argtypes = []
        L.engram_version.restype = ctypes.c_char_p
        L.engram_version.argtypes = []
        L.engram_compress.argtypes = [P, i64, P, i32, P, P, P]
        L.engram_hash.argtypes = [P, i32, i64, i64, i64, P, i32, i32, P, P, i32, P, P]
        L.engram_compress_hash.argtypes = [P, i32, i64, i64, i64, P, i32, P, i32, i32, P, P, i32, P, P, P, P]
        L.engram_quantize_fp8.argtypes = [P, i64, i32, i32, P, P, P, P]
        L.engram_gather.argtypes = [P, i64, i32, P, P, i32, i32, P, P, P]
        L.engram_lookup.argtypes = [P, i32, i64, i64, i64, P, i32, P, i32, i32, P, P, i32, P, i32, i32, P, P, P, P,
                                    P]
        L.engram_gate_forward.argtypes = [P, i64, i32, i32, i32, P, P, P, P, P, ctypes.c_float, i32, i32,
                                          P, P, P, P]
        L.engram_gate_forward_fp8.argtypes = L.engram_gate_forward.argtypes
        L.engram_gate_forward_noalloc.argtypes = L.engram_gate_forward.argtypes
        L.engram_lookup_fp8.argtypes = [P, i32, i64, i64, i64, P, i32, P, i32, i32, P, P, i32, P, i32, P, P, P, P, P,
                                        P, P]
        L.engram_gate_prepare.argtypes = [i32, i32, i32, P, P, P, P, P]
        L.engram_gate_forward_prepared.argtypes = [P, i64, i32, i32, i32, P, P, P, ctypes.c_float, P, P, P, P]
        L.engram_gate_prepare_fp8.argtypes = [i32, i32, i32, P, P, P, P, i32, P, P, P, P, P]
        L.engram_gate_forward_fp8q.argtypes = [P, P, P, i64, i32, i32, i32, P, P, P, P, P, P, P, ctypes.c_float, i32,
                                               P, P, P, P]
        L.engram_conv_forward.argtypes = [P, i32, i64, i32, P, P, i32, i32, ctypes.c_float, i32, P, P]
        L.engram_prefetch_host.argtypes = [P, i64, i32, P, P, i32, i32, P, P, P]
        L.engram_host_alloc.argtypes = [ctypes.c_size_t, ctypes.POINTER(ctypes.c_void_p)]
        L.engram_host_free.argtypes = [P]
        L.engram_cache_select.argtypes = [P, i64, i32, i32, P]
        L.engram_cache_build.argtypes = [P, P, i32, i32, i32, P, i32, i32, P, P, P]
        L.engram_prefetch_host_cached.argtypes = [P, i64, i32, P, P, i32, i32, P, i32, P, P, P, P, P]
        L.engram_gate_wait_timeouts.argtypes = [ctypes.POINTER(i32), i32]
        L.engram_debug_force_gate_timeout.argtypes = [i32]
        L.engram_debug_gate_key_form.argtypes = [i32]
        L.engram_lookup_gate.argtypes = [P, i32, i64, i64, i64, P, i32, P, i32, i32, P, P, i32, P, i32, i32, i32,
                                         P, P, P, P, P, ctypes.c_float, i32, P, P, P, P, P, P]
        for f in ("engram_compress", "engram_hash", "engram_gather", "engram_gate_forward",
                  "engram_conv_forward", "engram_prefetch_host", "engram_host_alloc", "engram_host_free",
                  "engram_cache_select", "engram_cache_build", "engram_prefetch_host_cached",
                  "engram_compress_hash", "engram_quantize_fp8", "engram_gate_forward_fp8", "engram_lookup",
                  "engram_lookup_fp8", "engram_gate_prepare_fp8", "engram_gate_forward_fp8q",
                  "engram_gate_prepare", "engram_gate_forward_prepared", "engram_gate_wait_timeouts",
                  "engram_debug_force_gate_timeout", "engram_debug_gate_key_form", "engram_gate_forward_noalloc",
                  "engram_lookup_gate"):
            getattr(L, f).restype = st
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise EngramError(status, lib().engram_last_error().decode())


def _stream(stream) -> ctypes.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name: str, dtype=None):
    import torch
    if not torch.is_tensor(t) or not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _opt(t, name, dtype=None):
    return ctypes.c_void_p(0) if t is None else _dev(t, name, dtype)


def _edtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr_array(ptrs: Sequence[int]):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def version() -> str:
    return lib().engram_version().decode()


# ---------------------------------------------------------------------------
def engram_compress(raw, cmap, out=None, err_count=None, stream=None):
    """out[i] = cmap[raw[i]] (or -1 for an out-of-range id, counted in err_count)."""
    import torch
    if out is None:
        out = torch.empty_like(raw)
    _check(lib().engram_compress(_dev(raw, "raw", torch.int32), raw.numel(), _dev(cmap, "map", torch.int32),
                                 cmap.numel(), _dev(out, "out", torch.int32),
                                 _opt(err_count, "err_count", torch.int32), _stream(stream)))
    return out


def engram_hash(ids, orders: Sequence[int], heads: int, mult, rows, pad_id: int, t_begin: int = 0,
                t_count: Optional[int] = None, out=None, stream=None):
    """Hash indices [batch * t_count, len(orders) * heads] (int32) of ids [batch, ld].

    ``mult``: uint64 array-like [n_orders][heads][max(orders)] (host); ``rows``:
    per-table sizes (host)."""
    import numpy as np
    import torch
    batch, ld = ids.shape
    if t_count is None:
        t_count = ld - t_begin
    orders_a = np.ascontiguousarray(orders, dtype=np.int32)
    mult_a = np.ascontiguousarray(mult, dtype=np.uint64)
    rows_a = np.ascontiguousarray(rows, dtype=np.uint32)
    n_tables = len(orders) * heads
    if mult_a.shape != (len(orders), heads, max(orders)) or rows_a.shape != (n_tables,):
        raise ValueError("mult must be [n_orders][heads][max_order] and rows [n_tables]")
    if out is None:
        out = torch.empty((batch * t_count, n_tables), dtype=torch.int32, device=ids.device)
    _check(lib().engram_hash(_dev(ids, "ids", torch.int32), batch, ld, t_begin, t_count,
                             orders_a.ctypes.data, len(orders), heads, mult_a.ctypes.data,
                             rows_a.ctypes.data, pad_id, _dev(out, "idx", torch.int32), _stream(stream)))
    return out


def engram_compress_hash(raw, cmap, orders: Sequence[int], heads: int, mult, rows, pad_id: int, t_begin: int = 0,
                         t_count: Optional[int] = None, out=None, ids_out=None, err_count=None, stream=None):
    """engram_compress then engram_hash in one kernel: hash indices [batch * t_count,
    len(orders) * heads] of the raw ids [batch, ld]; ``ids_out`` [batch, ld] optionally
    receives the window's canonical ids."""
    import numpy as np
    import torch
    batch, ld = raw.shape
    if t_count is None:
        t_count = ld - t_begin
    orders_a = np.ascontiguousarray(orders, dtype=np.int32)
    mult_a = np.ascontiguousarray(mult, dtype=np.uint64)
    rows_a = np.ascontiguousarray(rows, dtype=np.uint32)
    n_tables = len(orders) * heads
    if mult_a.shape != (len(orders), heads, max(orders)) or rows_a.shape != (n_tables,):
        raise ValueError("mult must be [n_orders][heads][max_order] and rows [n_tables]")
    if ids_out is not None and tuple(ids_out.shape) != (batch, ld):
        raise ValueError("ids_out must be [batch, ld]")
    if out is None:
        out = torch.empty((batch * t_count, n_tables), dtype=torch.int32, device=raw.device)
    _check(lib().engram_compress_hash(_dev(raw, "raw", torch.int32), batch, ld, t_begin, t_count,
                                      _dev(cmap, "map", torch.int32), cmap.numel(), orders_a.ctypes.data,
                                      len(orders), heads, mult_a.ctypes.data, rows_a.ctypes.data, pad_id,
                                      _opt(ids_out, "ids_out", torch.int32), _dev(out, "idx", torch.int32),
                                      _opt(err_count, "err_count", torch.int32), _stream(stream)))
    return out


def engram_gather(idx, tables: Sequence, out=None, err_count=None, stream=None):
    """Concatenated rows [n_tok, n_tables * w]; tables: GPU tensors [rows_b, w] of one dtype."""
    import numpy as np
    import torch
    n_tok, n_tables = idx.shape
    w = tables[0].shape[1]
    dt = tables[0].dtype
    for t in tables:
        if t.shape[1] != w or t.dtype != dt:
            raise ValueError("all tables need the same width and dtype")
        _dev(t, "table")
    ptrs = _ptr_array([t.data_ptr() for t in tables])
    rows = np.array([t.shape[0] for t in tables], dtype=np.int64)
    if out is None:
        out = torch.empty((n_tok, n_tables * w), dtype=dt, device=idx.device)
    _check(lib().engram_gather(_dev(idx, "idx", torch.int32), n_tok, n_tables, ptrs, rows.ctypes.data, w,
                               _edtype(tables[0]), _dev(out, "out", dt), _opt(err_count, "err_count", torch.int32),
                               _stream(stream)))
    return out


def engram_lookup(raw, cmap, orders: Sequence[int], heads: int, mult, tables: Sequence, pad_id: int,
                  t_begin: int = 0, t_count: Optional[int] = None, out=None, ids_out=None, idx_out=None,
                  err_count=None, stream=None):
    """engram_compress_hash then engram_gather in one kernel: the memory vectors
    [batch * t_count, len(orders) * heads * w] of the raw ids [batch, ld].  ``cmap`` may be
    None (raw ids are canonical); each table's row count is its hash modulus.  ``idx_out``
    [batch * t_count, n_tables] and ``ids_out`` [batch, ld] optionally receive the indices
    and the canonical ids."""
    import numpy as np
    import torch
    batch, ld = raw.shape
    if t_count is None:
        t_count = ld - t_begin
    orders_a = np.ascontiguousarray(orders, dtype=np.int32)
    mult_a = np.ascontiguousarray(mult, dtype=np.uint64)
    n_tables = len(orders) * heads
    if mult_a.shape != (len(orders), heads, max(orders)) or len(tables) != n_tables:
        raise ValueError("mult must be [n_orders][heads][max_order], one table per (order, head)")
    w = tables[0].shape[1]
    dt = tables[0].dtype
    for t in tables:
        if t.shape[1] != w or t.dtype != dt:
            raise ValueError("all tables need the same width and dtype")
        _dev(t, "table")
    rows_a = np.array([t.shape[0] for t in tables], dtype=np.uint32)
    if ids_out is not None and tuple(ids_out.shape) != (batch, ld):
        raise ValueError("ids_out must be [batch, ld]")
    if idx_out is not None and tuple(idx_out.shape) != (batch * t_count, n_tables):
        raise ValueError("idx_out must be [batch * t_count, n_tables]")
    if out is None:
        out = torch.empty((batch * t_count, n_tables * w), dtype=dt, device=raw.device)
    ptrs = _ptr_array([t.data_ptr() for t in tables])
    _check(lib().engram_lookup(_dev(raw, "raw", torch.int32), batch, ld, t_begin, t_count,
                               _opt(cmap, "map", torch.int32), 0 if cmap is None else cmap.numel(),
                               orders_a.ctypes.data, len(orders), heads, mult_a.ctypes.data, rows_a.ctypes.data,
                               pad_id, ptrs, w, _edtype(tables[0]), _opt(ids_out, "ids_out", torch.int32),
                               _opt(idx_out, "idx_out", torch.int32), _dev(out, "out", dt),
                               _opt(err_count, "err_count", torch.int32), _stream(stream)))
    return out


def engram_lookup_gate(raw, cmap, orders: Sequence[int], heads: int, mult, tables: Sequence, pad_id: int,
                       h: Sequence, wk: Sequence, wv: Sequence, gq: Sequence, gk: Sequence, eps: float = 1e-6,
                       t_begin: int = 0, t_count: Optional[int] = None, out: Optional[Sequence] = None,
                       gate_out=None, value_out: Optional[Sequence] = None, key_norm: int = KEY_NORM_MEMORY,
                       ids_out=None, err_count=None, stream=None):
    """engram_lookup (bf16 tables) followed by engram_gate_forward, in one pass that never
    stores the memory vectors; the results are those of the two calls bit for bit.
    Arguments as for those two functions (h, out, value_out: [batch * t_count, d_model])."""
    import numpy as np
    import torch
    batch, ld = raw.shape
    if t_count is None:
        t_count = ld - t_begin
    orders_a = np.ascontiguousarray(orders, dtype=np.int32)
    mult_a = np.ascontiguousarray(mult, dtype=np.uint64)
    n_tables = len(orders) * heads
    if mult_a.shape != (len(orders), heads, max(orders)) or len(tables) != n_tables:
        raise ValueError("mult must be [n_orders][heads][max_order], one table per (order, head)")
    w = tables[0].shape[1]
    for t in tables:
        if t.shape[1] != w:
            raise ValueError("all tables need the same width")
        _dev(t, "table", torch.bfloat16)
    rows_a = np.array([t.shape[0] for t in tables], dtype=np.uint32)
    if ids_out is not None and tuple(ids_out.shape) != (batch, ld):
        raise ValueError("ids_out must be [batch, ld]")
    n_tok = batch * t_count
    d_mem = n_tables * w
    nb = len(h)
    d_model = h[0].shape[1]
    if out is None:
        out = [torch.empty_like(x) for x in h]
    if not (len(wk) == len(wv) == len(gq) == len(gk) == len(out) == nb):
        raise ValueError("one h/wk/wv/gq/gk/out per branch")
    if value_out is not None and len(value_out) != nb:
        raise ValueError("one value_out entry per branch")
    for name, seq in (("h", h), ("wk", wk), ("wv", wv), ("gq", gq), ("gk", gk), ("out", out)):
        for x in seq:
            _dev(x, name, torch.bfloat16)
    vals = [x for x in (value_out or []) if x is not None]
    for x in vals:
        _dev(x, "value_out", torch.bfloat16)
    for x in list(h) + list(out) + vals:
        if tuple(x.shape) != (n_tok, d_model):
            raise ValueError("h/out/value_out must be [batch * t_count, d_model]")
    for x in list(wk) + list(wv):
        if tuple(x.shape) != (d_model, d_mem):
            raise ValueError("weights must be [d_model, d_mem]")
    gk_len = d_mem if key_norm == KEY_NORM_MEMORY else d_model
    for x in gq:
        if tuple(x.shape) != (d_model,):
            raise ValueError("gq must be [d_model]")
    for x in gk:
        if tuple(x.shape) != (gk_len,):
            raise ValueError(f"gk must be [{gk_len}] for key_norm {key_norm}")
    arr = lambda seq: _ptr_array([x.data_ptr() for x in seq])
    varr = None if value_out is None else _ptr_array([0 if x is None else x.data_ptr() for x in value_out])
    _check(lib().engram_lookup_gate(_dev(raw, "raw", torch.int32), batch, ld, t_begin, t_count,
                                    _opt(cmap, "map", torch.int32), 0 if cmap is None else cmap.numel(),
                                    orders_a.ctypes.data, len(orders), heads, mult_a.ctypes.data,
                                    rows_a.ctypes.data, pad_id, arr(tables), w, d_model, nb, arr(h), arr(wk),
                                    arr(wv), arr(gq), arr(gk), float(eps), int(key_norm), arr(out),
                                    _opt(gate_out, "gate_out", torch.float32), varr,
                                    _opt(ids_out, "ids_out", torch.int32), _opt(err_count, "err_count", torch.int32),
                                    _stream(stream)))
    return out


def engram_lookup_fp8(raw, cmap, orders: Sequence[int], heads: int, mult, tables: Sequence, pad_id: int,
                      t_begin: int = 0, t_count: Optional[int] = None, codes=None, scales=None, sumsq=None,
                      with_sumsq: bool = True, ids_out=None, idx_out=None, err_count=None, stream=None):
    """engram_lookup on bf16 tables with the memory vectors quantized per row to E4M3:
    (codes uint8 [n, d_mem], scales float32 [n], sumsq float32 [n] or None), n = batch *
    t_count."""
    import numpy as np
    import torch
    batch, ld = raw.shape
    if t_count is None:
        t_count = ld - t_begin
    orders_a = np.ascontiguousarray(orders, dtype=np.int32)
    mult_a = np.ascontiguousarray(mult, dtype=np.uint64)
    n_tables = len(orders) * heads
    if mult_a.shape != (len(orders), heads, max(orders)) or len(tables) != n_tables:
        raise ValueError("mult must be [n_orders][heads][max_order], one table per (order, head)")
    w = tables[0].shape[1]
    for t in tables:
        if t.shape[1] != w:
            raise ValueError("all tables need the same width")
        _dev(t, "table", torch.bfloat16)
    rows_a = np.array([t.shape[0] for t in tables], dtype=np.uint32)
    n = batch * t_count
    dev = raw.device
    if codes is None:
        codes = torch.empty((n, n_tables * w), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(n, dtype=torch.float32, device=dev)
    if sumsq is None and with_sumsq:
        sumsq = torch.empty(n, dtype=torch.float32, device=dev)
    ptrs = _ptr_array([t.data_ptr() for t in tables])
    _check(lib().engram_lookup_fp8(_dev(raw, "raw", torch.int32), batch, ld, t_begin, t_count,
                                   _opt(cmap, "map", torch.int32), 0 if cmap is None else cmap.numel(),
                                   orders_a.ctypes.data, len(orders), heads, mult_a.ctypes.data, rows_a.ctypes.data,
                                   pad_id, ptrs, w, _opt(ids_out, "ids_out", torch.int32),
                                   _opt(idx_out, "idx_out", torch.int32), _dev(codes, "codes", torch.uint8),
                                   _dev(scales, "scales", torch.float32), _opt(sumsq, "sumsq", torch.float32),
                                   _opt(err_count, "err_count", torch.int32), _stream(stream)))
    return codes, scales, sumsq


def engram_gate_prepare_fp8(wk: Sequence, wv: Sequence, gq: Optional[Sequence] = None, gk: Optional[Sequence] = None,
                            key_norm: int = KEY_NORM_MEMORY, stream=None):
    """The FP8 gate's weights, quantized once: a dict of per-branch lists wk_codes,
    wk_scales, wv_codes, wv_scales.  Branches passing the same W_V tensor share one copy
    of its codes (the gate then computes W_V e once)."""
    import torch
    nb = len(wk)
    d_model, d_mem = wk[0].shape
    wk_codes = [torch.empty((d_model, d_mem), dtype=torch.uint8, device=w.device) for w in wk]
    wk_scales = [torch.empty(d_model, dtype=torch.float32, device=w.device) for w in wk]
    wv_codes, wv_scales, seen = [], [], {}
    for w in wv:
        if w.data_ptr() not in seen:
            seen[w.data_ptr()] = (torch.empty((d_model, d_mem), dtype=torch.uint8, device=w.device),
                                  torch.empty(d_model, dtype=torch.float32, device=w.device))
        wv_codes.append(seen[w.data_ptr()][0])
        wv_scales.append(seen[w.data_ptr()][1])
    arr = lambda seq: _ptr_array([0 if x is None else x.data_ptr() for x in seq])
    for x in list(wk) + list(wv):
        _dev(x, "weights", torch.bfloat16)
        if tuple(x.shape) != (d_model, d_mem):
            raise ValueError("weights must be [d_model, d_mem]")
    gq_a = arr(gq) if gq is not None else None
    gk_a = arr(gk) if gk is not None else None
    _check(lib().engram_gate_prepare_fp8(d_mem, d_model, nb, arr(wk), arr(wv), gq_a, gk_a, int(key_norm),
                                         arr(wk_codes), arr(wk_scales), arr(wv_codes), arr(wv_scales),
                                         _stream(stream)))
    return {"wk_codes": wk_codes, "wk_scales": wk_scales, "wv_codes": wv_codes, "wv_scales": wv_scales,
            "key_norm": int(key_norm)}


def engram_gate_forward_fp8q(codes, scales, sumsq, h: Sequence, prepared, gq: Sequence, gk: Sequence,
                             eps: float = 1e-6, out: Optional[Sequence] = None, gate_out=None,
                             value_out: Optional[Sequence] = None, stream=None):
    """engram_gate_forward(..., fp8=True) on operands quantized ahead: the memory vectors'
    (codes, scales, sumsq) from engram_lookup_fp8 or engram_quantize_fp8 and the weights
    from engram_gate_prepare_fp8 (its key_norm applies)."""
    import torch
    n_tok, d_mem = codes.shape
    nb = len(h)
    d_model = h[0].shape[1]
    if out is None:
        out = [torch.empty_like(x) for x in h]
    for name, seq in (("h", h), ("gq", gq), ("gk", gk), ("out", out)):
        for x in seq:
            _dev(x, name, torch.bfloat16)
    arr = lambda seq: _ptr_array([x.data_ptr() for x in seq])
    varr = None if value_out is None else _ptr_array([0 if x is None else x.data_ptr() for x in value_out])
    _check(lib().engram_gate_forward_fp8q(_dev(codes, "codes", torch.uint8), _dev(scales, "scales", torch.float32),
                                          _opt(sumsq, "sumsq", torch.float32), n_tok, d_mem, d_model, nb, arr(h),
                                          arr(prepared["wk_codes"]), arr(prepared["wk_scales"]),
                                          arr(prepared["wv_codes"]), arr(prepared["wv_scales"]), arr(gq), arr(gk),
                                          float(eps), prepared["key_norm"], arr(out),
                                          _opt(gate_out, "gate_out", torch.float32), varr, _stream(stream)))
    return out


def engram_gate_forward(mem, h: Sequence, wk: Sequence, wv: Sequence, gq: Sequence, gk: Sequence,
                        eps: float = 1e-6, out: Optional[Sequence] = None, gate_out=None,
                        value_out: Optional[Sequence] = None, key_norm: int = KEY_NORM_MEMORY, stream=None,
                        fp8: bool = False, noalloc: bool = False):
    """out[m] = h[m] + sigmoid(RMSNorm(h[m]) . k[m] / sqrt(d)) * W_V[m] mem, with
    k[m] = W_K[m] RMSNorm(mem) (KEY_NORM_MEMORY, gk over d_mem) or RMSNorm(W_K[m] mem)
    (KEY_NORM_PROJECTED, gk over d_model).

    ``fp8``: both projections on per-row E4M3 codes of the weights and of mem
    (engram_gate_forward_fp8; bf16 operands, d_mem % 128 == 0).
    ``noalloc``: engram_gate_forward_noalloc (no allocation; the library's fixed
    scratch array; the output tensors must be passed or are allocated here by torch).

    Lists hold one tensor per branch; ``out`` defaults to new tensors (pass ``h``
    for in-place).  ``gate_out``: optional float32 [n_branch, n_tok] for alpha.
    ``value_out``: optional list (entries may be None) of [n_tok, d_model] tensors
    receiving the gated values alpha * v."""
    import torch
    n_tok, d_mem = mem.shape
    nb = len(h)
    d_model = h[0].shape[1]
    dt = mem.dtype
    _dev(mem, "mem", dt)
    if out is None:
        out = [torch.empty_like(x) for x in h]
    if not (len(wk) == len(wv) == len(gq) == len(gk) == len(out) == nb):
        raise ValueError("one h/wk/wv/gq/gk/out per branch")
    if value_out is not None and len(value_out) != nb:
        raise ValueError("one value_out entry per branch")
    for name, seq in (("h", h), ("wk", wk), ("wv", wv), ("gq", gq), ("gk", gk), ("out", out)):
        for x in seq:
            _dev(x, name, dt)
    vals = [x for x in (value_out or []) if x is not None]
    for x in vals:
        _dev(x, "value_out", dt)
    for x in list(h) + list(out) + vals:
        if tuple(x.shape) != (n_tok, d_model):
            raise ValueError("h/out/value_out must be [n_tok, d_model]")
    for x in list(wk) + list(wv):
        if tuple(x.shape) != (d_model, d_mem):
            raise ValueError("weights must be [d_model, d_mem]")
    arr = lambda seq: _ptr_array([x.data_ptr() for x in seq])
    varr = None if value_out is None else _ptr_array([0 if x is None else x.data_ptr() for x in value_out])
    gk_len = d_mem if key_norm == KEY_NORM_MEMORY else d_model
    for x in gq:
        if tuple(x.shape) != (d_model,):
            raise ValueError("gq must be [d_model]")
    for x in gk:
        if tuple(x.shape) != (gk_len,):
            raise ValueError(f"gk must be [{gk_len}] for key_norm {key_norm}")
    if fp8 and noalloc:
        raise ValueError("the allocation-free gate has no FP8 form")
    fn = (lib().engram_gate_forward_fp8 if fp8 else
          lib().engram_gate_forward_noalloc if noalloc else lib().engram_gate_forward)
    _check(fn(mem.data_ptr(), n_tok, d_mem, d_model, nb, arr(h), arr(wk), arr(wv), arr(gq), arr(gk), float(eps),
              _edtype(mem), int(key_norm), arr(out), _opt(gate_out, "gate_out", torch.float32), varr,
              _stream(stream)))
    return out


def engram_gate_prepare(wk: Sequence, gq: Sequence, gk: Sequence, stream=None):
    """The bf16 gate's key weights with both RMSNorm gains folded in (memory-side key
    norm): one [d_model, d_mem] bf16 tensor per branch, for engram_gate_forward_prepared."""
    import torch
    nb = len(wk)
    d_model, d_mem = wk[0].shape
    if not (len(gq) == len(gk) == nb):
        raise ValueError("one wk/gq/gk per branch")
    for x in wk:
        _dev(x, "wk", torch.bfloat16)
        if tuple(x.shape) != (d_model, d_mem):
            raise ValueError("weights must be [d_model, d_mem]")
    for x in gq:
        _dev(x, "gq", torch.bfloat16)
        if tuple(x.shape) != (d_model,):
            raise ValueError("gq must be [d_model]")
    for x in gk:
        _dev(x, "gk", torch.bfloat16)
        if tuple(x.shape) != (d_mem,):
            raise ValueError("gk must be [d_mem]")
    folded = [torch.empty_like(x) for x in wk]
    arr = lambda seq: _ptr_array([x.data_ptr() for x in seq])
    _check(lib().engram_gate_prepare(d_mem, d_model, nb, arr(wk), arr(gq), arr(gk), arr(folded), _stream(stream)))
    return folded


def engram_gate_forward_prepared(mem, h: Sequence, wk_folded: Sequence, wv: Sequence, eps: float = 1e-6,
                                 out: Optional[Sequence] = None, gate_out=None, value_out: Optional[Sequence] = None,
                                 stream=None):
    """engram_gate_forward (bf16, KEY_NORM_MEMORY) on key weights from engram_gate_prepare;
    bit-identical to it."""
    import torch
    n_tok, d_mem = mem.shape
    nb = len(h)
    d_model = h[0].shape[1]
    _dev(mem, "mem", torch.bfloat16)
    if out is None:
        out = [torch.empty_like(x) for x in h]
    if not (len(wk_folded) == len(wv) == len(out) == nb):
        raise ValueError("one h/wk_folded/wv/out per branch")
    if value_out is not None and len(value_out) != nb:
        raise ValueError("one value_out entry per branch")
    vals = [x for x in (value_out or []) if x is not None]
    for name, seq in (("h", h), ("wk_folded", wk_folded), ("wv", wv), ("out", out), ("value_out", vals)):
        for x in seq:
            _dev(x, name, torch.bfloat16)
    for x in list(h) + list(out) + vals:
        if tuple(x.shape) != (n_tok, d_model):
            raise ValueError("h/out/value_out must be [n_tok, d_model]")
    for x in list(wk_folded) + list(wv):
        if tuple(x.shape) != (d_model, d_mem):
            raise ValueError("weights must be [d_model, d_mem]")
    arr = lambda seq: _ptr_array([x.data_ptr() for x in seq])
    varr = None if value_out is None else _ptr_array([0 if x is None else x.data_ptr() for x in value_out])
    _check(lib().engram_gate_forward_prepared(mem.data_ptr(), n_tok, d_mem, d_model, nb, arr(h), arr(wk_folded),
                                              arr(wv), float(eps), arr(out),
                                              _opt(gate_out, "gate_out", torch.float32), varr, _stream(stream)))
    return out


def engram_conv_forward(value, batch: int, seq: int, w, gamma, dilation: int, out, eps: float = 1e-6,
                        stream=None):
    """out += SiLU(Conv1D(RMSNorm_gamma(value))) per sequence, in place, and returns ``out``.

    value, out: [batch * seq, d_model] (token t of sequence b is row b * seq + t);
    w: [d_model, taps] depthwise kernel, tap j looking j * dilation tokens back;
    gamma: [d_model]."""
    n_tok, d_model = value.shape
    dt = value.dtype
    if n_tok != batch * seq or tuple(out.shape) != (n_tok, d_model):
        raise ValueError("value and out must be [batch * seq, d_model]")
    if w.dim() != 2 or w.shape[0] != d_model or tuple(gamma.shape) != (d_model,):
        raise ValueError("w must be [d_model, taps] and gamma [d_model]")
    _check(lib().engram_conv_forward(_dev(value, "value", dt), batch, seq, d_model, _dev(w, "w", dt),
                                     _dev(gamma, "gamma", dt), w.shape[1], dilation, float(eps), _edtype(value),
                                     _dev(out, "out", dt), _stream(stream)))
    return out


def engram_prefetch_host(idx, host_tables: Sequence, rows: Sequence[int], w: int, dtype, staging=None,
                         err_count=None, stream=None):
    """Gather from pinned host tables into the device buffer ``staging`` [n_tok, n_tables * w].

    ``host_tables``: pinned CPU tensors, or integer addresses from ``host_alloc``."""
    import numpy as np
    import torch
    n_tok, n_tables = idx.shape
    ptrs = []
    for t in host_tables:
        if torch.is_tensor(t):
            if t.is_cuda or not t.is_pinned():
                raise ValueError("host tables must be pinned host memory")
            ptrs.append(t.data_ptr())
        else:
            ptrs.append(int(t))
    rows_a = np.ascontiguousarray(rows, dtype=np.int64)
    if staging is None:
        staging = torch.empty((n_tok, n_tables * w), dtype=dtype, device=idx.device)
    _check(lib().engram_prefetch_host(_dev(idx, "idx", torch.int32), n_tok, n_tables, _ptr_array(ptrs),
                                      rows_a.ctypes.data, w, BF16 if dtype == torch.bfloat16 else F32,
                                      _dev(staging, "staging", dtype), _opt(err_count, "err_count", torch.int32),
                                      _stream(stream)))
    return staging


def _host_table_ptrs(host_tables):
    import torch
    ptrs = []
    for t in host_tables:
        if torch.is_tensor(t):
            if t.is_cuda or not t.is_pinned():
                raise ValueError("host tables must be pinned host memory")
            ptrs.append(t.data_ptr())
        else:
            ptrs.append(int(t))
    return ptrs


def engram_cache_select(idx, capacity: int):
    """Per table, the ``capacity`` most frequent rows of the sample ``idx`` [n, n_tables]
    (host array or tensor, int32); ties to the smaller row, -1 padding.  Returns a numpy
    int32 array [n_tables, capacity].  Pure host computation."""
    import numpy as np
    import torch
    if torch.is_tensor(idx):
        idx = idx.detach().cpu().numpy()
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n, n_tables = idx.shape
    hot = np.empty((n_tables, capacity), dtype=np.int32)
    _check(lib().engram_cache_select(idx.ctypes.data, n, n_tables, capacity, hot.ctypes.data))
    return hot


def engram_cache_build(host_tables: Sequence, rows: Sequence[int], w: int, dtype, hot, slots: Optional[int] = None,
                       stream=None):
    """Build the HBM row cache for the rows ``hot`` [n_tables, capacity] (from
    ``engram_cache_select``).  Returns (table int32 [n_tables, slots, 2], cache_rows
    [capacity, n_tables * w]) on the current device; the call waits for the build."""
    import numpy as np
    import torch
    hot = np.ascontiguousarray(hot, dtype=np.int32)
    n_tables, capacity = hot.shape
    if slots is None:
        slots = 1
        while slots < 2 * capacity:
            slots *= 2
    rows_a = np.ascontiguousarray(rows, dtype=np.int64)
    dev = torch.device("cuda", torch.cuda.current_device())
    table = torch.empty((n_tables, slots, 2), dtype=torch.int32, device=dev)
    cache_rows = torch.empty((capacity, n_tables * w), dtype=dtype, device=dev)
    _check(lib().engram_cache_build(_ptr_array(_host_table_ptrs(host_tables)), rows_a.ctypes.data, n_tables, w,
                                    BF16 if dtype == torch.bfloat16 else F32, hot.ctypes.data, capacity, slots,
                                    _dev(table, "table", torch.int32), _dev(cache_rows, "cache_rows", dtype),
                                    _stream(stream)))
    return table, cache_rows


def engram_prefetch_host_cached(idx, host_tables: Sequence, rows: Sequence[int], w: int, dtype, table, cache_rows,
                                staging=None, hits=None, err_count=None, stream=None):
    """``engram_prefetch_host`` through the HBM row cache of ``engram_cache_build``."""
    import numpy as np
    import torch
    n_tok, n_tables = idx.shape
    rows_a = np.ascontiguousarray(rows, dtype=np.int64)
    if staging is None:
        staging = torch.empty((n_tok, n_tables * w), dtype=dtype, device=idx.device)
    _check(lib().engram_prefetch_host_cached(
        _dev(idx, "idx", torch.int32), n_tok, n_tables, _ptr_array(_host_table_ptrs(host_tables)),
        rows_a.ctypes.data, w, BF16 if dtype == torch.bfloat16 else F32, _dev(table, "table", torch.int32),
        table.shape[1], _dev(cache_rows, "cache_rows", dtype), _dev(staging, "staging", dtype),
        _opt(hits, "hits", torch.int32), _opt(err_count, "err_count", torch.int32), _stream(stream)))
    return staging


def engram_quantize_fp8(x, with_sumsq: bool = False, stream=None):
    """Per-row FP8 (OCP E4M3) codes of x [rows, cols]: (codes uint8 [rows, cols], scales
    float32 [rows]) and, with_sumsq, the rows' sums of squares of the dequantized values."""
    import torch
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    sumsq = torch.empty(rows, dtype=torch.float32, device=x.device) if with_sumsq else None
    _check(lib().engram_quantize_fp8(_dev(x, "x"), rows, cols, _edtype(x), _dev(codes, "codes", torch.uint8),
                                     _dev(scales, "scales", torch.float32), _opt(sumsq, "sumsq", torch.float32),
                                     _stream(stream)))
    return (codes, scales, sumsq) if with_sumsq else (codes, scales)


def engram_gate_wait_timeouts(reset: bool = False) -> int:
    """Value-tile wavefronts of gate calls on the current device whose bounded wait for
    their gates ran out (they wrote NaN) since load or the last reset; synchronizes the
    device.  0 in normal operation."""
    n = ctypes.c_int32(0)
    _check(lib().engram_gate_wait_timeouts(ctypes.byref(n), 1 if reset else 0))
    return int(n.value)


def engram_debug_force_gate_timeout(on: bool):
    """Test hook: make every later gate launch's value-tile wait give up (see engram.h)."""
    _check(lib().engram_debug_force_gate_timeout(1 if on else 0))


GATE_KEY_FORMS = {"auto": 0, "feature": 1, "memory": 2}


def engram_debug_gate_key_form(form: str):
    """Test hook: the gate's key-tile form, "auto" (by shape, the default), "feature"
    (feature-major) or "memory" (memory-major where it applies); see engram.h."""
    _check(lib().engram_debug_gate_key_form(GATE_KEY_FORMS[form]))


def host_alloc(nbytes: int) -> int:
    """Pinned, device-mapped host allocation (hipHostMalloc); returns the address."""
    p = ctypes.c_void_p()
    _check(lib().engram_host_alloc(nbytes, ctypes.byref(p)))
    return p.value


def host_free(addr: int):
    _check(lib().engram_host_free(ctypes.c_void_p(addr)))

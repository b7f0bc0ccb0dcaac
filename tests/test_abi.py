"""The C ABI library: it loads, exports every entry point of include/engram.h,
and rejects bad arguments on the host (no GPU work is started by these calls)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import hashed_gram_embedding_hash_amd as eg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "engram.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("engram_compress", "engram_hash", "engram_gather", "engram_gate_forward", "engram_prefetch_host"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = eg.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(eg.EXPORTS)
    assert "gfx950" in eg.version()


def test_library_is_gfx950_code_object():
    data = open(eg.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def _dynamic_symbols(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_timeline_build_exports_the_api_and_its_two_calls():
    """libengram_timeline.so (the gate compiled with its per-tile stamps) carries every entry point
    of engram.h plus engram_gate_timeline_read / _clear; the normal library has neither of those."""
    from hashed_gram_embedding_hash_amd import build as hb
    timeline = _dynamic_symbols(hb.TIMELINE_LIB)
    normal = _dynamic_symbols(eg.LIB_PATH)
    extra = {"engram_gate_timeline_read", "engram_gate_timeline_clear"}
    assert set(declared_functions()) <= timeline
    assert extra <= timeline
    assert not (extra & normal)
    assert set(declared_functions()) <= normal


def _st(name):
    return {"ok": 0, "arg": 1, "unsup": 2, "hip": 3}[name]


def test_compress_argument_errors():
    L = eg.lib()
    assert L.engram_compress(None, -1, None, 10, None, None, None) == _st("arg")
    assert b"n < 0" in L.engram_last_error()
    assert L.engram_compress(None, 5, None, 10, None, None, None) == _st("arg")
    assert L.engram_compress(None, 0, ctypes.c_void_p(16), 0, None, None, None) == _st("arg")
    # n == 0 is a no-op and touches no device memory
    assert L.engram_compress(None, 0, ctypes.c_void_p(16), 10, None, None, None) == _st("ok")


def test_hash_argument_errors():
    L = eg.lib()
    orders = np.array([2, 3], np.int32)
    mult = np.ones((2, 2, 3), np.uint64)
    rows = np.array([7, 7, 7, 7], np.uint32)
    call = lambda **kw: L.engram_hash(
        kw.get("ids", ctypes.c_void_p(256)), kw.get("batch", 1), kw.get("ld", 10), kw.get("t_begin", 0),
        kw.get("t_count", 10), kw.get("orders", orders.ctypes.data), kw.get("n_orders", 2), kw.get("heads", 2),
        kw.get("mult", mult.ctypes.data), kw.get("rows", rows.ctypes.data), 0, kw.get("idx", ctypes.c_void_p(256)),
        None)
    assert call(t_begin=5, t_count=6) == _st("arg")
    assert b"exceeds" in L.engram_last_error()
    assert call(batch=-1) == _st("arg")
    bad_orders = np.array([2, 5], np.int32)
    assert call(orders=bad_orders.ctypes.data) == _st("arg")
    bad_rows = np.array([7, 0, 7, 7], np.uint32)
    assert call(rows=bad_rows.ctypes.data) == _st("arg")
    big_rows = np.array([7, 1 << 31, 7, 7], np.uint32)
    assert call(rows=big_rows.ctypes.data) == _st("arg")
    assert call(heads=17) == _st("arg")          # 2 * 17 tables > 32
    assert call(ids=None) == _st("arg")
    assert call(t_count=0) == _st("ok")          # empty window: no-op


def test_gather_argument_errors():
    L = eg.lib()
    tabs = (ctypes.c_void_p * 2)(256, 512)
    rows = np.array([10, 10], np.int64)
    g = lambda **kw: L.engram_gather(ctypes.c_void_p(256), kw.get("n", 4), kw.get("nt", 2), kw.get("tabs", tabs),
                                     kw.get("rows", rows.ctypes.data), kw.get("w", 8), kw.get("dt", eg.BF16),
                                     kw.get("out", ctypes.c_void_p(1024)), None, None)
    assert g(w=4) == _st("unsup")                 # 8-byte rows
    assert g(dt=7) == _st("arg")
    assert g(nt=0) == _st("arg")
    assert g(nt=33) == _st("arg")
    assert g(tabs=(ctypes.c_void_p * 2)(256, 513)) == _st("arg")   # misaligned table
    assert g(out=ctypes.c_void_p(1032)) == _st("arg")               # misaligned output
    assert g(rows=np.array([10, 0], np.int64).ctypes.data) == _st("arg")
    assert g(n=-1) == _st("arg")
    assert g(w=5120) == _st("unsup")              # 2 x 10240-byte rows exceed 16 KiB per token
    assert g(n=0) == _st("ok")


def test_gate_argument_errors():
    L = eg.lib()
    one = (ctypes.c_void_p * 1)(4096)
    gf = lambda **kw: L.engram_gate_forward(
        ctypes.c_void_p(4096), kw.get("n", 8), kw.get("dm", 1280), kw.get("dmod", 2560), kw.get("nb", 1),
        one, one, one, one, one, ctypes.c_float(kw.get("eps", 1e-6)), kw.get("dt", eg.BF16), kw.get("kn", 0),
        one, None, kw.get("vout"), None)
    assert gf(dm=1000) == _st("unsup")
    assert gf(dmod=2500) == _st("unsup")
    assert b"d_mem % 64" in L.engram_last_error()
    assert gf(nb=0) == _st("arg")
    assert gf(nb=9) == _st("arg")
    assert gf(eps=-1.0) == _st("arg")
    assert gf(n=-2) == _st("arg")
    assert gf(dt=5) == _st("arg")
    assert gf(vout=(ctypes.c_void_p * 1)(4104)) == _st("arg")   # misaligned gated-value output
    assert gf(kn=2) == _st("arg")                                 # unknown key placement
    assert b"key_norm" in L.engram_last_error()
    assert gf(n=0) == _st("ok")
    # shapes whose 32-bit weight offsets or int tile numbers would wrap are refused on the
    # host (the pointers are never dereferenced)
    assert gf(dm=65536, dmod=65536) == _st("unsup")               # d_model * d_mem = 2^32
    assert b"2^32" in L.engram_last_error()
    assert gf(dm=1 << 16, dmod=1 << 17) == _st("unsup")           # 2^33 weight elements
    assert gf(n=(1 << 31) - 1, dm=64, dmod=1 << 16, nb=8) == _st("unsup")   # 2^33 tiles
    assert b"tiles" in L.engram_last_error()
    assert gf(dm=65536 - 64, dmod=65504, n=0) == _st("ok")         # just below 2^32: accepted (no tokens)


def test_gate_wait_timeout_query_argument_errors():
    L = eg.lib()
    assert L.engram_gate_wait_timeouts(None, 0) == _st("arg")
    assert L.engram_debug_force_gate_timeout(0) == _st("ok")


def test_gate_key_form_hook_argument_errors():
    L = eg.lib()
    assert L.engram_debug_gate_key_form(3) == _st("arg")
    assert L.engram_debug_gate_key_form(-1) == _st("arg")
    assert b"form" in L.engram_last_error()
    for form in (1, 2, 0):  # ends on the default
        assert L.engram_debug_gate_key_form(form) == _st("ok")


def test_lookup_argument_errors():
    import numpy as np
    L = eg.lib()
    orders = np.array([2, 3], np.int32)
    mult = np.ones((2, 2, 3), np.uint64)
    rows = np.full(4, 1009, np.uint32)
    tabs = (ctypes.c_void_p * 4)(4096, 8192, 12288, 16384)
    lk = lambda **kw: L.engram_lookup(
        ctypes.c_void_p(kw.get("raw", 4096)), kw.get("batch", 2), kw.get("ld", 100), kw.get("tb", 0),
        kw.get("tc", 100), None, 0, kw.get("orders", orders).ctypes.data, kw.get("no", 2), 2, mult.ctypes.data,
        kw.get("rows", rows).ctypes.data, 7, kw.get("tabs", tabs), kw.get("w", 80), kw.get("dt", eg.BF16), None,
        ctypes.c_void_p(kw.get("idx", 0)), ctypes.c_void_p(kw.get("out", 1 << 20)), None, None)
    assert lk(w=12) == _st("unsup")                              # 24-byte bf16 rows
    assert lk(tb=50, tc=60) == _st("arg")                        # window past the row
    assert lk(orders=np.array([2, 5], np.int32)) == _st("arg")   # order above the maximum
    assert lk(rows=np.zeros(4, np.uint32)) == _st("arg")
    assert lk(tabs=(ctypes.c_void_p * 4)(4096, 8200, 12288, 16384)) == _st("arg")  # misaligned table
    assert lk(out=(1 << 20) + 8) == _st("arg")                   # misaligned output
    assert lk(idx=4098) == _st("arg")                            # misaligned index output
    assert lk(raw=0) == _st("arg")
    assert lk(dt=9) == _st("arg")
    assert lk(tc=0, raw=0, out=0) == _st("ok")
    assert lk(batch=0, raw=0, out=0) == _st("ok")


def test_fp8_operand_calls_argument_errors():
    import numpy as np
    L = eg.lib()
    one = (ctypes.c_void_p * 1)(4096)
    p1 = lambda **kw: L.engram_gate_prepare_fp8(
        kw.get("dm", 1280), kw.get("dmod", 2560), kw.get("nb", 1), one, one, kw.get("gq", one), kw.get("gk", one),
        kw.get("kn", 0), kw.get("codes", one), one, one, one, None)
    assert p1(dm=1216) == _st("unsup")
    assert p1(dmod=2500) == _st("unsup")
    assert p1(nb=0) == _st("arg")
    assert p1(kn=4) == _st("arg")
    assert p1(gq=None) == _st("arg")                                   # the memory-side key needs the gains
    assert p1(codes=(ctypes.c_void_p * 1)(4100)) == _st("arg")         # misaligned codes
    q = lambda **kw: L.engram_gate_forward_fp8q(
        ctypes.c_void_p(kw.get("codes", 4096)), ctypes.c_void_p(kw.get("scales", 8192)),
        ctypes.c_void_p(kw.get("ss", 8192)), kw.get("n", 8), kw.get("dm", 1280), 2560, 1, one, one, one, one, one, one,
        one, ctypes.c_float(1e-6), kw.get("kn", 0), one, None, None, None)
    assert q(dm=1216) == _st("unsup")
    assert q(ss=0) == _st("arg")                                       # sums of squares needed (memory key)
    assert q(scales=8194) == _st("arg")
    assert q(codes=4100) == _st("arg")
    assert q(n=0) == _st("ok")
    orders = np.array([2, 3], np.int32)
    mult = np.ones((2, 2, 3), np.uint64)
    rows = np.full(4, 1009, np.uint32)
    tabs = (ctypes.c_void_p * 4)(4096, 8192, 12288, 16384)
    lf = lambda **kw: L.engram_lookup_fp8(
        ctypes.c_void_p(4096), 2, 100, 0, kw.get("tc", 100), None, 0, orders.ctypes.data, 2, 2, mult.ctypes.data,
        rows.ctypes.data, 7, tabs, kw.get("w", 80), None, None, ctypes.c_void_p(kw.get("codes", 1 << 20)),
        ctypes.c_void_p(kw.get("scales", 1 << 21)), None, None, None)
    assert lf(w=12) == _st("unsup")
    assert lf(codes=(1 << 20) + 8) == _st("arg")
    assert lf(scales=0) == _st("arg")
    assert lf(tc=0) == _st("ok")


def test_gate_fp8_argument_errors():
    L = eg.lib()
    one = (ctypes.c_void_p * 1)(4096)
    gf = lambda **kw: L.engram_gate_forward_fp8(
        ctypes.c_void_p(4096), kw.get("n", 8), kw.get("dm", 1280), kw.get("dmod", 2560), kw.get("nb", 1),
        one, one, one, one, one, ctypes.c_float(1e-6), kw.get("dt", eg.BF16), kw.get("kn", 0), one, None, None,
        None)
    assert gf(dm=1216) == _st("unsup")             # a multiple of 64 but not of 128
    assert b"multiple of 128" in L.engram_last_error()
    assert gf(dt=eg.F32) == _st("unsup")
    assert gf(dmod=2500) == _st("unsup")
    assert gf(nb=0) == _st("arg")
    assert gf(kn=3) == _st("arg")
    assert gf(n=0) == _st("ok")


def test_conv_argument_errors():
    L = eg.lib()
    cf = lambda **kw: L.engram_conv_forward(
        ctypes.c_void_p(kw.get("value", 4096)), kw.get("batch", 2), kw.get("seq", 100), kw.get("dmod", 2560),
        ctypes.c_void_p(kw.get("w", 1 << 20)), ctypes.c_void_p(kw.get("g", 1 << 21)), kw.get("taps", 4),
        kw.get("dil", 3), ctypes.c_float(kw.get("eps", 1e-6)), kw.get("dt", eg.BF16),
        ctypes.c_void_p(kw.get("out", 1 << 30)), None)
    assert cf(taps=0) == _st("unsup")
    assert cf(taps=9) == _st("unsup")
    assert cf(dil=0) == _st("unsup")
    assert cf(dil=17) == _st("unsup")
    assert cf(dmod=12) == _st("unsup")                # 24-byte bf16 rows
    assert b"multiple of 16" in L.engram_last_error()
    assert cf(dmod=6, dt=eg.F32) == _st("unsup")      # 24-byte fp32 rows
    assert cf(batch=-1) == _st("arg")
    assert cf(seq=-1) == _st("arg")
    assert cf(dmod=0) == _st("arg")
    assert cf(eps=-1.0) == _st("arg")
    assert cf(dt=7) == _st("arg")
    assert cf(w=0) == _st("arg")
    assert cf(g=8) == _st("arg")                      # misaligned gamma
    assert cf(value=4100) == _st("arg")               # misaligned value
    assert cf(out=4096 + 5120 * 10) == _st("arg")     # out overlaps value
    assert b"overlaps" in L.engram_last_error()
    assert cf(batch=0) == _st("ok")
    assert cf(seq=0, value=0, out=0) == _st("ok")


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(eg, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(eg, "_lib", None)
    with pytest.raises(ImportError):
        eg.lib()


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "hashed_gram_embedding_hash_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_compress_hash_argument_errors():
    L = eg.lib()
    orders = np.array([2, 3], np.int32)
    mult = np.ones((2, 2, 3), np.uint64)
    rows = np.full(4, 1009, np.uint32)
    cmap = np.zeros(10, np.int32)
    ch = lambda **kw: L.engram_compress_hash(
        ctypes.c_void_p(4096), kw.get("batch", 2), kw.get("ld", 100), kw.get("tb", 0), kw.get("tc", 100),
        ctypes.c_void_p(kw.get("map", cmap.ctypes.data)), kw.get("vocab", 10), orders.ctypes.data, 2, 2,
        mult.ctypes.data, rows.ctypes.data, 10, None, ctypes.c_void_p(kw.get("idx", 8192)), None, None)
    assert ch(map=0) == _st("arg")
    assert ch(vocab=0) == _st("arg")
    assert ch(tb=50, tc=60) == _st("arg")       # window past the row
    assert ch(batch=-1) == _st("arg")
    assert ch(tc=0) == _st("ok")


def test_gate_prepared_argument_errors():
    L = eg.lib()
    one = (ctypes.c_void_p * 1)(4096)
    pr = lambda **kw: L.engram_gate_prepare(kw.get("dm", 1280), kw.get("dmod", 2560), kw.get("nb", 1), one, one, one,
                                            kw.get("out", one), None)
    assert pr(dm=1000) == _st("unsup")              # d_mem not a multiple of 64
    assert pr(dmod=2500) == _st("unsup")
    assert pr(nb=0) == _st("arg")
    assert pr(nb=9) == _st("arg")
    assert pr(out=None) == _st("arg")
    assert pr(out=(ctypes.c_void_p * 1)(4100)) == _st("arg")   # misaligned output
    fp = lambda **kw: L.engram_gate_forward_prepared(
        ctypes.c_void_p(kw.get("mem", 4096)), kw.get("n", 8), kw.get("dm", 1280), 2560, 1, one, one, one,
        ctypes.c_float(kw.get("eps", 1e-6)), one, None, None, None)
    assert fp(dm=1216 + 32) == _st("unsup")
    assert fp(eps=-1.0) == _st("arg")
    assert fp(mem=4100) == _st("arg")               # misaligned memory vectors
    assert fp(n=0, mem=0) == _st("ok")


def test_lookup_gate_argument_errors():
    L = eg.lib()
    orders = np.array([2, 3], np.int32)
    mult = np.ones((2, 2, 3), np.uint64)
    rows = np.full(4, 1009, np.uint32)
    tabs = (ctypes.c_void_p * 4)(4096, 8192, 12288, 16384)
    one = (ctypes.c_void_p * 1)(4096)
    lg = lambda **kw: L.engram_lookup_gate(
        ctypes.c_void_p(kw.get("raw", 4096)), kw.get("batch", 2), kw.get("ld", 100), kw.get("tb", 0),
        kw.get("tc", 100), None, 0, orders.ctypes.data, 2, 2, mult.ctypes.data, rows.ctypes.data, 7,
        kw.get("tabs", tabs), kw.get("w", 80), kw.get("dmod", 2560), kw.get("nb", 1), kw.get("h", one), one, one,
        one, one, ctypes.c_float(1e-6), kw.get("kn", eg.KEY_NORM_MEMORY), kw.get("out", one), None, None,
        ctypes.c_void_p(kw.get("ids", 0)), None, None)
    assert lg(w=32) == _st("unsup")           # rows under 64 values: a k-step would span three tables
    assert lg(w=12) == _st("unsup")           # 24-byte rows
    assert lg(w=72) == _st("unsup")           # d_mem = 288, not a multiple of 64
    assert lg(dmod=2500) == _st("unsup")      # d_model not a multiple of 32
    assert lg(tb=50, tc=60) == _st("arg")     # window past the row
    assert lg(tabs=(ctypes.c_void_p * 4)(4096, 8200, 12288, 16384)) == _st("arg")  # misaligned table
    assert lg(raw=0) == _st("arg")
    assert lg(nb=0) == _st("arg")
    assert lg(kn=5) == _st("arg")
    assert lg(ids=4098) == _st("arg")         # misaligned ids output
    assert lg(out=(ctypes.c_void_p * 1)(0)) == _st("arg")
    assert lg(tc=0, raw=0) == _st("ok")
    assert lg(batch=0, raw=0) == _st("ok")

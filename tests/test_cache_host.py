"""Host logic of the HBM row cache (no GPU): hot-row selection against a numpy brute
force, and argument checks that fail before any device work."""
import ctypes

import numpy as np
import pytest

import hashed_gram_embedding_hash_amd as eg

ARG, UNSUP = 1, 2


def brute_force_hot(idx, capacity):
    """Per column: rows by descending count, ties by ascending row; -1 padding."""
    n_tables = idx.shape[1]
    hot = np.full((n_tables, capacity), -1, np.int32)
    for b in range(n_tables):
        col = idx[:, b]
        rows, counts = np.unique(col[col >= 0], return_counts=True)
        order = np.lexsort((rows, -counts))[:capacity]
        hot[b, :len(order)] = rows[order]
    return hot


def test_cache_select_matches_brute_force_on_zipf_indices():
    rng = np.random.default_rng(0)
    n, n_tables = 20000, 5
    ranks = rng.zipf(1.3, size=(n, n_tables)) % 3000
    perm = rng.permutation(3000).astype(np.int32)    # hot rows are not the small ones
    idx = perm[ranks].astype(np.int32)
    for cap in (1, 17, 250, 5000):
        got = eg.engram_cache_select(idx, cap)
        assert np.array_equal(got, brute_force_hot(idx, cap)), cap


def test_cache_select_ties_padding_and_negative_entries():
    idx = np.array([[5, -1], [3, 7], [5, 7], [3, -3], [9, 7]], np.int32)
    got = eg.engram_cache_select(idx, 4)
    # column 0: 3 and 5 twice (tie -> 3 first), 9 once; column 1: 7 three times
    assert got.tolist() == [[3, 5, 9, -1], [7, -1, -1, -1]]
    assert np.array_equal(got, brute_force_hot(idx, 4))
    empty = eg.engram_cache_select(np.zeros((0, 3), np.int32), 2)
    assert (empty == -1).all()


def test_cache_argument_errors():
    L = eg.lib()
    hot = np.zeros((2, 4), np.int32)
    rows = np.array([100, 100], np.int64)
    tabs = (ctypes.c_void_p * 2)(1 << 20, 1 << 21)
    build = lambda **kw: L.engram_cache_build(
        tabs, rows.ctypes.data, 2, kw.get("w", 80), kw.get("dt", eg.BF16), kw.get("hot", hot).ctypes.data,
        kw.get("cap", 4), kw.get("slots", 8), ctypes.c_void_p(kw.get("table", 1 << 22)),
        ctypes.c_void_p(kw.get("cache", 1 << 23)), None)
    assert build(slots=6) == ARG            # not a power of two
    assert build(slots=4) == ARG            # not above capacity
    assert build(cap=0) == ARG
    assert build(w=5) == UNSUP              # 10-byte rows
    assert build(table=4) == ARG            # misaligned table
    bad = hot.copy()
    bad[1, 2] = 100                         # row 100 of a 100-row table
    assert build(hot=bad) == ARG
    assert b"out of range" in L.engram_last_error()
    sel = lambda **kw: L.engram_cache_select(hot.ctypes.data, kw.get("n", 2), kw.get("nt", 2),
                                             kw.get("cap", 4), hot.ctypes.data)
    assert sel(n=-1) == ARG and sel(nt=0) == ARG and sel(cap=0) == ARG
    idx = np.zeros((3, 2), np.int32)
    pc = lambda **kw: L.engram_prefetch_host_cached(
        idx.ctypes.data, 3, 2, tabs, rows.ctypes.data, 80, eg.BF16, ctypes.c_void_p(kw.get("table", 1 << 22)),
        kw.get("slots", 8), ctypes.c_void_p(1 << 23), ctypes.c_void_p(1 << 24), None, None, None)
    assert pc(slots=12) == ARG
    assert pc(table=12) == ARG

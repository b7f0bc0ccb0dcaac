"""Host-side pieces of the benchmark (no GPU): the one-GPU guard, the algorithmic work it
divides by, the offload sizing rule, and the source hash that keeps stale counter
summaries out of the JSON line."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.mark.parametrize("name,flops", [
    ("small", 4 * 1280 * 2560 * 1 * 16384),     # 4 d_mem d_model M T
    ("multi", 4 * 1280 * 4096 * 4 * 65536),
    ("large", 4 * 1280 * 4096 * 2 * 262144),
])
def test_gate_flops_are_the_closed_form(name, flops):
    assert bench.algorithmic(synth.CONFIGS[name])["gate"]["flops"] == flops


def test_shared_wv_counts_the_value_product_once():
    cfg = synth.CONFIGS["multi"]
    # W_K per branch (4) plus one W_V instead of four: 5/8 of the FLOPs
    assert bench.algorithmic(cfg, shared_wv=True)["gate"]["flops"] * 8 == bench.algorithmic(cfg)["gate"]["flops"] * 5


def test_lookup_bytes_are_ids_rows_and_vectors():
    cfg = synth.CONFIGS["large"]
    T = cfg.tokens
    # 4 B raw id in, 16 rows x 160 B read, the 2,560-B memory vector written
    assert bench.algorithmic(cfg)["lookup"]["bytes"] == T * (4 + 2560 + 2560)


def test_offload_sizing_caps_and_primes():
    cfg = synth.CONFIGS["offload"]
    row_bytes = cfg.w * 2
    # plenty of everything: the 48-GB pinned cap decides, rounded up to a prime
    rows = synth.offload_table_rows(cfg, 10 ** 15, 10 ** 15)
    assert rows == synth.next_prime(int(48e9 / (cfg.n_tables * row_bytes)))
    # a small HBM: 80 % of it holds the HBM-resident copy
    rows = synth.offload_table_rows(cfg, 10 ** 15, 10 * 10 ** 9)
    assert cfg.n_tables * rows * row_bytes <= 0.8 * 10 * 10 ** 9 + cfg.n_tables * row_bytes * 1000
    assert all(rows % p for p in range(2, 1000))


def test_code_hash_ignores_comments_and_whitespace_only():
    a = "int f(int x) {  // one\n  return x + 1; /* two */ }\n"
    b = "int f(int x){\n\treturn x+1;}"
    c = "int f(int x) { return x + 2; }"
    assert bench.code_sha(a) == bench.code_sha(b) != bench.code_sha(c)


def test_key_tile_form_reported_for_each_workload():
    """The form the JSON line names follows engram.h's rule: memory-major key tiles when
    d_mem < d_model, d_model % 64 == 0 and at least one key tile per compute unit."""
    import argparse
    a = argparse.Namespace(fp8=False, key_norm="memory", key_form="auto")
    got = {n: bench.gate_key_tiles(synth.CONFIGS[n], a) for n in ("tiny", "small", "multi", "large")}
    assert got == {"tiny": "feature-major", "small": "memory-major", "multi": "memory-major",
                   "large": "memory-major"}
    # a decode step: 256 tokens, 5 key tiles
    assert bench.gate_key_tiles(synth.CONFIGS["large"].replace(batch=1, seq=256), a) == "feature-major"
    assert bench.gate_key_tiles(synth.CONFIGS["large"], argparse.Namespace(
        fp8=False, key_norm="memory", key_form="feature")) == "feature-major (forced)"
    assert bench.gate_key_tiles(synth.CONFIGS["large"], argparse.Namespace(
        fp8=True, key_norm="memory", key_form="auto")) == "feature-major"

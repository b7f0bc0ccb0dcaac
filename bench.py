#!/usr/bin/env python3
"""Throughput of the Engram forward pass (compress -> hash -> gather -> gate) on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic input
already resident in HBM.  The default workload is the largest that fits one GPU,
"large": 8 x 32768 Zipf(1.05) tokens, 16 bf16 tables of 10,156,253 x 80 (26 GB),
memory dim 1280, d_model 4096, two gating branches; the step is two calls:
engram_lookup (compression, hashing and the gather in one kernel) and
engram_gate_forward.  Prints ONE JSON line with tokens/s, the per-call breakdown,
the roofline of the dominant kernel (the gate), the same step with the FP8 gate,
the short convolution beside it, the "small" workload (4 x 4096 tokens, 1,000,003-row
tables, d_model 2560, one branch) as a secondary line, and the CPU oracle's tokens/s
on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--config large|small|multi|tiny]
    python bench.py --calibrate-copy MIB     # plain device copy, for HBM counter scaling
    python bench.py --config offload         # decode steps: host-resident vs HBM-resident tables

Between timed steps (outside the timed events) a scratch buffer larger than the
last-level cache is rewritten, so every step starts with cold L2 and MALL.  Each
timed iteration runs the step twice, each time after the flush: launched call by
call (events between the calls give the per-call breakdown and the gate's
roofline), then as one replay of a HIP graph captured from it (the reported
value; --no-graph reports the eager step instead).  wall_s_timed covers both.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Engram tokens/s (hash+gather+gate); gather HBM GB/s & MFMA util vs peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # fp32 vector / matrix
PEAK_FP8_TFLOPS = 5000.0       # dense fp8 MFMA
GATE_SOURCE = os.path.join(ROOT, "hashed_gram_embedding_hash_amd", "csrc", "gate_bf16.hip")
PROFILES = os.path.join(ROOT, "profiles")


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"gate_persistent_kernel_{workload}_hbm_traffic.txt")


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    p.add_argument("--steps", type=int, default=30)
    # the GPU's clocks settle over the first ~10-20 steps of this workload
    p.add_argument("--warmup", type=int, default=20)
    # the largest single-GPU workload (262,144 tokens, 26 GB of tables, two branches); the
    # small one is measured after it as a secondary line (--no-secondary skips it)
    p.add_argument("--config", default="large")
    p.add_argument("--no-secondary", action="store_true",
                   help="with the large workload: skip the secondary measurement of the small one")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time of the CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--shared-wv", action="store_true",
                   help="every branch uses branch 0's W_V (the paper's Eq. 6): W_V e is computed once")
    p.add_argument("--key-norm", choices=("memory", "projected"), default="memory",
                   help="memory: k = W_K RMSNorm(e) (default); projected: k = RMSNorm(W_K e), Eq. 4")
    p.add_argument("--key-form", choices=("auto", "feature", "memory"), default="auto",
                   help="the bf16 gate's key tiles: chosen by shape (auto, the library's default), "
                        "feature-major, or memory-major where that form applies (A/B measurements)")
    p.add_argument("--fp8", action="store_true",
                   help="gate projections on E4M3 codes (engram_gate_forward_fp8; quantization inside the call)")
    p.add_argument("--no-fp8", action="store_true", help="skip the extra fp8-gate step measurement")
    p.add_argument("--probes", action="store_true",
                   help="run the probe library's measurements of what bounds the gate's main loop (operand "
                        "stream into LDS, the main loop with parts switched off, the MFMA rate and the clock), "
                        "print one JSON line and exit")
    p.add_argument("--timeline", action="store_true",
                   help="run one gate call of --config with libengram_timeline.so (the gate stamping each "
                        "tile's phase boundaries), print the per-tile breakdown as one JSON line and exit")
    p.add_argument("--no-fused", action="store_true",
                   help="skip the one-call step (engram_lookup_gate) measured beside the two-call step")
    p.add_argument("--no-graph", action="store_true",
                   help="time the eagerly launched step only (default: the step is also captured in a HIP graph "
                        "and the graph replay is the reported value)")
    p.add_argument("--no-conv", action="store_true",
                   help="skip the separate measurement of the short convolution (Eq. 5)")
    p.add_argument("--flush-mb", type=int, default=512, help="cache-flush buffer rewritten between steps (0: off)")
    p.add_argument("--offload-rows", type=int, default=0,
                   help="offload config: rows per table (default: 100B parameters, scaled to 60%% of free host RAM)")
    p.add_argument("--offload-reps", type=int, default=3)
    p.add_argument("--offload-fold-each-step", action="store_true",
                   help="offload config: call engram_gate_forward every step (it folds the key weights with "
                        "their gains on every call) instead of engram_gate_forward_prepared on weights folded once")
    p.add_argument("--offload-cache-gb", type=float, default=4.0,
                   help="HBM cache of the rows most frequent in the decode histories (0: off); 4 GB holds "
                        "every row the 256 x 4096-token histories use")
    p.add_argument("--offload-host-gb", type=float, default=48.0,  # synth.OFFLOAD_HOST_GB
                   help="offload config: cap on pinned host table bytes (the GPU's system-memory aperture is "
                        "shared with the runtime; on the measured host, pinning beyond ~64 GB fails)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB three times and exit")
    return p.parse_args()


def workload_desc(cfg, args=None):
    extra = {}
    if args is not None and (args.shared_wv or args.key_norm != "memory" or args.fp8):
        extra = {"key_norm": args.key_norm, "shared_wv": bool(args.shared_wv),
                 "gate_projections": "fp8 e4m3, per-row scales" if args.fp8 else "bf16"}
    if args is not None and getattr(args, "key_form", "auto") != "auto":
        extra["gate_key_tiles"] = args.key_form
    return {**extra,
        "workload": cfg.name,
        "tokens": cfg.tokens, "batch": cfg.batch, "seq_len": cfg.seq,
        "tables": f"{cfg.n_tables} x {cfg.rows} x {cfg.w} {cfg.dtype}",
        "orders": list(cfg.orders), "heads": cfg.heads, "d_mem": cfg.d_mem, "d_model": cfg.d_model,
        "branches": cfg.n_branch, "zipf_s": cfg.zipf_s, "parallelism": "single GPU",
    }


def algorithmic(cfg, shared_wv=False):
    """Algorithmic work of one step, per call (bytes moved to/from HBM, flops).  With a
    shared W_V the value product is counted once, not once per branch."""
    T, nt, dm, d, M = cfg.tokens, cfg.n_tables, cfg.d_mem, cfg.d_model, cfg.n_branch
    nv = 1 if shared_wv else M
    es = 4 if cfg.dtype == "f32" else 2
    return {
        # raw ids in, rows read and the memory vectors written (the indices stay on chip;
        # the 517-KB compression map stays in L2)
        "lookup": {"bytes": 4 * T + 2 * dm * es * T},
        # the same as two calls: raw ids in, indices out; indices in, rows read, vectors out
        "compress_hash": {"bytes": 4 * T + 4 * nt * T},
        "gather": {"bytes": 4 * nt * T + 2 * dm * es * T},
        # weights once, memory vector once, hidden read + output written per branch
        "gate": {"flops": 2 * dm * d * (M + nv) * T,
                 "bytes": dm * es * T + (M + nv) * d * dm * es + M * 2 * d * es * T},
    }


def code_sha(text: str) -> str:
    """sha256 of C++ source with its comments and whitespace removed: changes when the
    code does, not when a comment does (the source holds no string with a comment marker)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256("".join(text.split()).encode()).hexdigest()


def gate_source_sha():
    with open(GATE_SOURCE) as f:
        return code_sha(f.read())


def gate_key_tiles(cfg, args, n_cu=256):
    """The key-tile form engram_gate_forward takes for this workload, by the rule engram.h
    documents for engram_debug_gate_key_form (bf16, memory-side key norm, the weights folded
    by the call: memory-major when d_mem < d_model, d_model % 64 == 0 and there are at least as
    many memory-major key tiles as compute units; feature-major otherwise)."""
    if cfg.dtype != "bf16" or args.fp8 or args.key_norm != "memory":
        return "feature-major"
    if args.key_form != "auto":
        forced = args.key_form == "memory" and cfg.d_mem < cfg.d_model and cfg.d_model % 64 == 0
        return ("memory-major" if forced else "feature-major") + " (forced)"
    n_ttiles = -(-cfg.tokens // 256)
    n_ktiles = -(-cfg.d_mem // 256)
    mm = cfg.d_mem < cfg.d_model and cfg.d_model % 64 == 0 and n_ttiles * cfg.n_branch * n_ktiles >= n_cu
    return "memory-major" if mm else "feature-major"


def measured_traffic(cfg):
    """HBM bytes per launch of the gate's persistent kernel, from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE scaled by a plain copy of known size).  None when
    the summary is missing, covers another workload, or the kernel source has changed
    since the counters were taken."""
    path = traffic_file(cfg.name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("workload") != cfg.name or kv.get("source_sha256") != gate_source_sha():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def probes():
    """Measurements behind the gate's limiter (libengram_probe.so, not part of the path), each
    timed with events; one JSON line.
    operand_stream: one workgroup of 256 threads per CU moving 64 KB per iteration from a 2-MB
      L2-resident buffer into LDS, by direct global->LDS loads and through registers;
    mainloop: the gate's k-step alone (256 x 256 tile, 20 k-steps of 64, the five-slot ring)
      over synthetic operands, whole and with its operand loads, fragment reads or MFMAs
      switched off, four waves as in the gate and eight; with the clock the chip ran at
      (s_memtime cycles over s_memrealtime's 100-MHz ticks) and cycles per k-step;
    mainloop_fp8: the FP8 gate's k-step (128 E4M3 values per ring row, 32x32x64 MFMAs) the same way;
    mfma: back-to-back 32x32x16 bf16 MFMAs and 32x32x64 E4M3 MFMAs (the FP8 gate's scaled form),
      one wave per SIMD on every CU, with the clock."""
    import ctypes
    import torch
    from hashed_gram_embedding_hash_amd import build as hb
    L = ctypes.CDLL(hb.PROBE_LIB)
    P = ctypes.c_void_p
    for f in (L.engram_probe_lds_dma, L.engram_probe_lds_vgpr):
        f.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P]
        f.restype = ctypes.c_int
    L.engram_probe_mainloop.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_int32, P, P, P]
    L.engram_probe_mainloop.restype = ctypes.c_int
    L.engram_probe_mainloop_fp8.argtypes = [ctypes.c_int32, P, P, ctypes.c_int32, P, P, P]
    L.engram_probe_mainloop_fp8.restype = ctypes.c_int
    L.engram_probe_mainloop_tokens.argtypes = [ctypes.c_int32]
    L.engram_probe_mainloop_tokens.restype = ctypes.c_int64
    L.engram_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P]
    L.engram_probe_mfma.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = P(torch.cuda.current_stream().cuda_stream)

    def timed(run, reps=5):
        assert run() == 0
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            assert run() == 0
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        return sorted(x.elapsed_time(y) for x, y in ts)[reps // 2]

    def clock(clk, blocks):
        c = clk[: 2 * blocks].view(blocks, 2).double().cpu()
        cycles, ticks = c[:, 0].median().item(), c[:, 1].median().item()
        return cycles, cycles / (ticks / 100e6) / 1e9  # s_memrealtime ticks at 100 MHz

    out = {"probe": "libengram_probe.so (measurement only)", "cus": cus}
    n_bytes, iters = 2 << 20, 4000
    src = torch.arange(n_bytes // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    clk = torch.zeros(cus * 2, dtype=torch.int64, device=dev)
    o = {"bytes_per_workgroup_iteration": 65536, "iterations": iters, "source_bytes": n_bytes}
    for name, fn in (("direct_to_lds", L.engram_probe_lds_dma), ("through_registers", L.engram_probe_lds_vgpr)):
        ms = timed(lambda: fn(P(src.data_ptr()), n_bytes, cus, iters, P(sink.data_ptr()), stream))
        total = cus * iters * 65536
        o[name] = {"ms": round(ms, 4), "TB/s_all_CUs": round(total / (ms * 1e-3) / 1e12, 3),
                   "GB/s_per_CU": round(total / cus / (ms * 1e-3) / 1e9, 2)}
    out["operand_stream"] = o
    del src

    if cus == 256:  # the main-loop probe's tile schedule assumes 256 workgroups
        rounds = 8
        g = torch.Generator(device=dev).manual_seed(5)
        W = (torch.randn(4096 * 1280, device=dev, generator=g) * 0.05).to(torch.bfloat16)
        E = (torch.randn(L.engram_probe_mainloop_tokens(rounds) * 1280, device=dev, generator=g) * 0.05
             ).to(torch.bfloat16)
        ksteps = rounds * 20
        flops = cus * rounds * 2 * 256 * 256 * 1280
        o = {"tile": "256 x 256 outputs, 20 k-steps of 64 (d_mem 1280)", "tiles_per_workgroup": rounds}
        modes = [(4, 0, "whole"), (4, 1, "no operand loads"), (4, 2, "no fragment reads"),
                 (4, 3, "no loads, no reads"), (4, 4, "no MFMAs"), (4, 6, "operand loads only"),
                 (8, 0, "whole, eight waves"), (8, 3, "no loads, no reads, eight waves")]
        for waves, mode, name in modes:
            ms = timed(lambda: L.engram_probe_mainloop(mode, waves, P(W.data_ptr()), P(E.data_ptr()), rounds,
                                                       P(sink.data_ptr()), P(clk.data_ptr()), stream))
            cycles, ghz = clock(clk, 256)
            o[name] = {"us_per_kstep": round(ms * 1e3 / ksteps, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
                       "clock_GHz": round(ghz, 3), "cycles_per_kstep": round(cycles / ksteps, 1)}
        out["mainloop"] = o
        o = {"tile": "256 x 256 outputs, 20 k-steps of 128 E4M3 values (the same bytes as the bf16 probe)",
             "tiles_per_workgroup": rounds}
        for mode, name in ((0, "whole"), (1, "no operand loads"), (2, "no fragment reads"), (3, "no loads, no reads")):
            ms = timed(lambda: L.engram_probe_mainloop_fp8(mode, P(W.data_ptr()), P(E.data_ptr()), rounds,
                                                           P(sink.data_ptr()), P(clk.data_ptr()), stream))
            cycles, ghz = clock(clk, 256)
            o[name] = {"us_per_kstep": round(ms * 1e3 / ksteps, 3),
                       "TFLOP/s": round(2 * flops / (ms * 1e-3) / 1e12, 1),
                       "clock_GHz": round(ghz, 3), "cycles_per_kstep": round(cycles / ksteps, 1)}
        out["mainloop_fp8"] = o
        del W, E

    iters = 20000
    out["mfma"] = {}
    for kind, name, flop in ((0, "v_mfma_f32_32x32x16_bf16", 32 * 32 * 16 * 2),
                             (1, "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3)", 32 * 32 * 64 * 2)):
        ms = timed(lambda: L.engram_probe_mfma(kind, cus, iters, P(sink.data_ptr()), P(clk.data_ptr()), stream),
                   reps=3)
        cycles, ghz = clock(clk, cus)
        n_mfma = iters * 16
        out["mfma"][name] = {"mfma_per_wave": n_mfma, "ms": round(ms, 4),
                             "TFLOP/s": round(cus * 4 * n_mfma * flop / (ms * 1e-3) / 1e12, 1),
                             "clock_GHz": round(ghz, 3), "cycles_per_mfma": round(cycles / n_mfma, 2)}
    print(json.dumps(out), flush=True)


TIMELINE_PARTS = {
    # (from point, to point): name; points as the gate's timeline build numbers them
    "K": [((0, 1), "claim and decode"), ((1, 2), "first operands"), ((2, 3), "main loop"),
          ((3, 4), "h tile wait"), ((5, 8), "dot pass"), ((8, 9), "partial stores"), ((9, 10), "store ack"),
          ((10, 11), "count"), ((11, 6), "gates (last K tile)"), ((6, 7), "end barrier")],
    "V": [((0, 1), "claim and decode"), ((1, 2), "first operands"), ((2, 3), "main loop"),
          ((3, 4), "h tile wait"), ((4, 5), "gate wait"), ((5, 12), "output into LDS"), ((12, 13), "stream out"),
          ((13, 6), "rest"), ((6, 7), "end barrier")],
}


def timeline(args):
    """One engram_gate_forward call of the workload's step (bf16, or with --fp8 the FP8 gate) run with
    libengram_timeline.so, the library whose gate stamps s_memrealtime (100 MHz) at each tile's
    phase boundaries; after three warm-up calls.  Per phase (K, V): the mean, median and 90th
    percentile of each part of a tile in microseconds and its share of all workgroups' time;
    the workgroups' start skew and end spread.  One JSON line."""
    import ctypes
    import numpy as np
    import torch
    import synth
    import hashed_gram_embedding_hash_amd as eg
    from hashed_gram_embedding_hash_amd import build as hb
    eg.LIB_PATH = hb.TIMELINE_LIB  # before anything loads the library
    L = eg.lib()
    eg.engram_debug_gate_key_form(args.key_form)
    L.engram_gate_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    L.engram_gate_timeline_read.restype = ctypes.c_int
    L.engram_gate_timeline_clear.argtypes = []
    L.engram_gate_timeline_clear.restype = ctypes.c_int
    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    inp = synth.device_inputs(cfg, dev)
    mem = torch.empty((cfg.tokens, cfg.d_mem), dtype=torch.bfloat16, device=dev)
    eg.engram_lookup(inp["raw"], inp["map"], cfg.orders, cfg.heads, inp["mult"], inp["tables"], cfg.vocab_c,
                     out=mem)
    outs = [torch.empty_like(h) for h in inp["h"]]

    def gate():
        eg.engram_gate_forward(mem, inp["h"], inp["wk"], inp["wv"], inp["gq"], inp["gk"], cfg.eps, out=outs,
                               fp8=args.fp8)
    for _ in range(3):
        gate()
    torch.cuda.synchronize()
    assert L.engram_gate_timeline_clear() == 0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    gate()
    b.record()
    torch.cuda.synchronize()
    wgs, tiles, points = 256, 512, 16
    buf = np.zeros(wgs * tiles * points, dtype=np.uint64)
    assert L.engram_gate_timeline_read(buf.ctypes.data, buf.nbytes) == 0
    t = buf.reshape(wgs, tiles, points).astype(np.int64)
    done = t[:, :, 7] > 0
    used = done.any(axis=1)
    assert done.sum() > 0, "no tile stamped"
    t0 = t[:, :, 0][t[:, :, 0] > 0].min()
    us = 0.01  # one s_memrealtime tick is 10 ns
    starts = np.where(done, t[:, :, 0], np.iinfo(np.int64).max).min(axis=1)[used]
    ends = np.where(done, t[:, :, 7], 0).max(axis=1)[used]
    span = (ends.max() - t0) * us
    out = {"timeline": cfg.name, "gate": "fp8" if args.fp8 else "bf16", "key_tiles": args.key_form,
           "gate_call_ms_events": round(a.elapsed_time(b), 4),
           "workgroups": int(used.sum()), "tiles": int(done.sum()),
           "span_us": round(span, 1), "start_skew_us_max": round(float((starts - t0).max()) * us, 2),
           "end_us": {"min": round(float((ends - t0).min()) * us, 1), "median": round(float(np.median(ends - t0)) * us, 1),
                      "max": round(float((ends - t0).max()) * us, 1)}}
    phase = t[:, :, 15] & 1
    for ph, name in ((0, "K"), (1, "V")):
        sel = done & (phase == ph)
        if not sel.any():
            continue
        rows = {}
        for (p0, p1), part in TIMELINE_PARTS[name]:
            d = (t[:, :, p1] - t[:, :, p0])[sel] * us
            rows[part] = {"mean": round(float(d.mean()), 3), "median": round(float(np.median(d)), 3),
                          "p90": round(float(np.percentile(d, 90)), 3),
                          "share": round(float(d.sum()) / (int(used.sum()) * span), 4)}
        tot = (t[:, :, 7] - t[:, :, 0])[sel] * us
        rows["tile"] = {"mean": round(float(tot.mean()), 3), "share": round(float(tot.sum()) / (int(used.sum()) * span), 4)}
        out[name] = {"tiles": int(sel.sum()), "parts_us": rows}
    print(json.dumps(out), flush=True)


def calibrate_copy(mib):
    import torch
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy": "torch bf16 device copy", "bytes_read": 2 * n, "bytes_written": 2 * n,
                      "kib_read": 2 * n / 1024, "kib_written": 2 * n / 1024}), flush=True)


def run_offload(args):
    """Decode steps of the host-offload workload (256 sequences, one new token each):
    the rows of step s+1 are hashed and fetched on a side stream while step s gates.
    The same two-stream pipeline runs once with the tables in pinned host memory
    (engram_prefetch_host over PCIe) and once with the same tables in HBM
    (engram_gather); the overhead is the ratio of the steady-state step times.  A third
    run puts an HBM cache of the rows most frequent in the sequences' histories in front
    of the host tables (engram_prefetch_host_cached).  Step times come from a HIP graph
    of the whole pipeline, so that the GPU and not the host's per-call cost sets the
    pace; the host-issued (eager) times are reported beside them."""
    import ctypes
    import numpy as np
    import torch
    import synth
    import hashed_gram_embedding_hash_amd as eg

    cfg = synth.CONFIGS["offload"]
    dev = torch.device("cuda:0")
    say = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)
    avail = synth.mem_available_bytes()
    row_bytes = cfg.w * 2
    free_hbm, _ = torch.cuda.mem_get_info()
    rows = args.offload_rows or synth.offload_table_rows(cfg, avail, free_hbm, args.offload_host_gb)
    say(f"offload: target {cfg.n_tables} tables x {rows} rows = {cfg.n_tables * rows * row_bytes / 1e9:.1f} GB "
        f"(host MemAvailable {avail / 1e9 if avail else float('nan'):.0f} GB)")

    dtabs, haddr = [], []
    try:
        for b in range(cfg.n_tables):
            t = torch.empty((rows, cfg.w), dtype=torch.bfloat16, device=dev)
            dtabs.append(synth.fill_table(cfg, b, t))
        torch.cuda.synchronize()
        say("device tables filled")
        for b in range(cfg.n_tables):
            haddr.append(eg.host_alloc(rows * row_bytes))
        for b in range(cfg.n_tables):
            arr = np.ctypeslib.as_array((ctypes.c_int16 * (rows * cfg.w)).from_address(haddr[b]))
            torch.from_numpy(arr).view(torch.bfloat16).view(rows, cfg.w).copy_(dtabs[b])
        torch.cuda.synchronize()
        table_bytes = cfg.n_tables * rows * row_bytes
        say(f"host tables filled: {cfg.n_tables} x {rows} rows = {table_bytes / 1e9:.1f} GB")

        S, B, T0 = cfg.decode_steps, cfg.batch, cfg.seq
        raw = torch.from_numpy(synth.raw_ids(cfg)).to(dev)            # [B, T0 + S]
        ids = eg.engram_compress(raw, torch.from_numpy(synth.comp_map(cfg)).to(dev))
        mult, rows_u32 = synth.multipliers(cfg), np.full(cfg.n_tables, rows, dtype=np.uint32)
        wk, wv = synth.weights(cfg, 0, dev)
        gq, gk = synth.gains(cfg, 0, dev)
        tok = (torch.arange(B, dtype=torch.int64) * (T0 + S)).view(1, B) + (T0 + torch.arange(S)).view(S, 1)
        h = synth.hidden_rows(cfg, 0, tok.reshape(-1), dev).view(S, B, cfg.d_model)
        out = torch.empty((B, cfg.d_model), dtype=torch.bfloat16, device=dev)
        idx = [torch.empty((B, cfg.n_tables), dtype=torch.int32, device=dev) for _ in range(2)]
        stg = [torch.empty((B, cfg.n_tables * cfg.w), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        main, side = torch.cuda.current_stream(), torch.cuda.Stream()
        hrows = [rows] * cfg.n_tables

        # Per-step calls go straight to the C ABI with arguments prepared once, so the
        # host issues a step in a few microseconds and the GPU sets the pace.
        L = eg.lib()
        P = ctypes.c_void_p
        ms, ss = P(main.cuda_stream), P(side.cuda_stream)
        orders_a = np.ascontiguousarray(cfg.orders, dtype=np.int32)
        mult_a = np.ascontiguousarray(mult, dtype=np.uint64)
        rows64 = np.full(cfg.n_tables, rows, dtype=np.int64)
        dptrs = (P * cfg.n_tables)(*[t.data_ptr() for t in dtabs])
        hptrs = (P * cfg.n_tables)(*haddr)
        arr = lambda xs: (P * len(xs))(*[x.data_ptr() for x in xs])
        wk_a, wv_a, gq_a, gk_a, out_a = arr([wk]), arr([wv]), arr([gq]), arr([gk]), arr([out])
        h_a = [arr([h[s]]) for s in range(S)]
        chk = lambda st: st == 0 or eg._check(st)

        # the HBM row cache: the rows most frequent in the histories of the sequences
        cache = None
        modes = ("hbm", "host")
        if args.offload_cache_gb > 0:
            capacity = int(args.offload_cache_gb * 1e9 / (cfg.n_tables * row_bytes))
            t_sel = time.perf_counter()
            hist_idx = eg.engram_hash(ids, cfg.orders, cfg.heads, mult, rows_u32, cfg.vocab_c, t_begin=0, t_count=T0)
            hot = eg.engram_cache_select(hist_idx.cpu().numpy(), capacity)
            del hist_idx
            t_sel = time.perf_counter() - t_sel
            t_build = time.perf_counter()
            ctab, crows = eg.engram_cache_build(haddr, hrows, cfg.w, torch.bfloat16, hot)
            t_build = time.perf_counter() - t_build
            cache = {"capacity": capacity, "slots": ctab.shape[1], "table": ctab, "rows": crows,
                     "hits": torch.zeros(1, dtype=torch.int32, device=dev),
                     "select_s": round(t_sel, 2), "build_s": round(t_build, 2),
                     "hbm_bytes": ctab.numel() * 4 + crows.numel() * 2}
            modes = ("hbm", "host", "cached")
            say(f"row cache: {capacity} rows per table ({cache['hbm_bytes'] / 1e9:.2f} GB of HBM), "
                f"selected in {t_sel:.1f} s, built in {t_build:.1f} s")

        def cached_prefetch(buf, st, hits=None):
            chk(L.engram_prefetch_host_cached(idx[buf].data_ptr(), B, cfg.n_tables, hptrs, rows64.ctypes.data, cfg.w,
                                              eg.BF16, P(cache["table"].data_ptr()), cache["slots"],
                                              P(cache["rows"].data_ptr()), stg[buf].data_ptr(),
                                              None if hits is None else P(hits.data_ptr()), None, st))

        def fetch(mode, s, buf, stream):
            st = ss if stream is side else ms
            chk(L.engram_hash(ids.data_ptr(), B, ids.shape[1], T0 + s, 1, orders_a.ctypes.data, len(cfg.orders),
                              cfg.heads, mult_a.ctypes.data, rows_u32.ctypes.data, cfg.vocab_c, idx[buf].data_ptr(), st))
            if mode == "cached":
                cached_prefetch(buf, st)
                return
            fn = L.engram_prefetch_host if mode == "host" else L.engram_gather
            chk(fn(idx[buf].data_ptr(), B, cfg.n_tables, hptrs if mode == "host" else dptrs, rows64.ctypes.data,
                   cfg.w, eg.BF16, stg[buf].data_ptr(), None, st))

        # The decode loop's weights are constant: by default the key weights are folded with
        # their gains once (engram_gate_prepare) and every step calls engram_gate_forward_prepared
        # (the same results bit for bit); --offload-fold-each-step calls engram_gate_forward,
        # which folds them again on every call.
        folded = eg.engram_gate_prepare([wk], [gq], [gk])
        folded_a = arr(folded)

        def gate(s, buf, st=ms):
            if args.offload_fold_each_step:
                chk(L.engram_gate_forward(stg[buf].data_ptr(), B, cfg.d_mem, cfg.d_model, 1, h_a[s], wk_a, wv_a,
                                          gq_a, gk_a, cfg.eps, eg.BF16, eg.KEY_NORM_MEMORY, out_a, None, None, st))
            else:
                chk(L.engram_gate_forward_prepared(stg[buf].data_ptr(), B, cfg.d_mem, cfg.d_model, 1, h_a[s],
                                                   folded_a, wv_a, ctypes.c_float(cfg.eps), out_a, None, None, st))

        def enqueue(mode, mstream):
            """The S decode steps on `mstream` (gates) and `side` (hash + fetch of the next
            step), ordered by events; side joins mstream at the end."""
            mst = P(mstream.cuda_stream)
            ready = [torch.cuda.Event() for _ in range(2)]
            free = [torch.cuda.Event() for _ in range(2)]
            freed = [False, False]
            side.wait_stream(mstream)
            with torch.cuda.stream(side):
                fetch(mode, 0, 0, side)
                ready[0].record(side)
            for s in range(S):
                cur, nxt = s % 2, (s + 1) % 2
                if s + 1 < S:
                    with torch.cuda.stream(side):
                        if freed[nxt]:
                            side.wait_event(free[nxt])  # the gate of step s-1 has read that buffer
                        fetch(mode, s + 1, nxt, side)
                        ready[nxt].record(side)
                mstream.wait_event(ready[cur])
                gate(s, cur, mst)
                free[cur].record(mstream)
                freed[cur] = True
            mstream.wait_stream(side)

        def pipeline(mode):
            """us per step with the host issuing every call (eager)."""
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(main)
            host0 = time.perf_counter()
            enqueue(mode, main)
            t1.record(main)
            host_us.append((time.perf_counter() - host0) * 1e6 / S)
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) * 1e3 / S

        def capture(mode):
            """The same S steps captured once as a HIP graph (both streams), so that the GPU
            sets the pace rather than the host's per-call cost.  An eager pass on the capture
            stream comes first: the gate's scratch is then sized and last used there."""
            cs = torch.cuda.Stream()
            cs.wait_stream(main)
            with torch.cuda.stream(cs):
                enqueue(mode, cs)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                enqueue(mode, cs)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            return g

        def replay(g):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            g.replay()
            t1.record()
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) * 1e3 / S

        def serial(fn, n=S):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for s in range(n):
                fn(s)
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / n

        host_us = []
        for mode in modes:
            pipeline(mode)                             # warm-up
        graphs = {m: capture(m) for m in modes}
        steps = {m: [] for m in modes}
        eager = {m: [] for m in modes}
        for _ in range(args.offload_reps):
            for mode in modes:
                steps[mode].append(replay(graphs[mode]))
                eager[mode].append(pipeline(mode))
        del graphs
        med = {k: float(np.median(v)) for k, v in steps.items()}
        med_eager = {k: float(np.median(v)) for k, v in eager.items()}
        comp = {
            "hash_us": serial(lambda s: chk(L.engram_hash(ids.data_ptr(), B, ids.shape[1], T0 + s, 1,
                                                          orders_a.ctypes.data, len(cfg.orders), cfg.heads,
                                                          mult_a.ctypes.data, rows_u32.ctypes.data, cfg.vocab_c,
                                                          idx[0].data_ptr(), ms))),
            "gather_hbm_us": serial(lambda s: chk(L.engram_gather(idx[0].data_ptr(), B, cfg.n_tables, dptrs,
                                                                  rows64.ctypes.data, cfg.w, eg.BF16,
                                                                  stg[0].data_ptr(), None, ms))),
            "prefetch_host_us": serial(lambda s: chk(L.engram_prefetch_host(idx[0].data_ptr(), B, cfg.n_tables, hptrs,
                                                                         rows64.ctypes.data, cfg.w, eg.BF16,
                                                                         stg[0].data_ptr(), None, ms))),
            "gate_us": serial(lambda s: gate(s, 0)),
        }
        if cache is not None:
            # hit rate over every decode step's indices
            for s_ in range(S):
                chk(L.engram_hash(ids.data_ptr(), B, ids.shape[1], T0 + s_, 1, orders_a.ctypes.data, len(cfg.orders),
                                  cfg.heads, mult_a.ctypes.data, rows_u32.ctypes.data, cfg.vocab_c, idx[0].data_ptr(),
                                  ms))
                cached_prefetch(0, ms, cache["hits"])
            torch.cuda.synchronize()
            cache["hit_rate"] = int(cache["hits"].item()) / (S * B * cfg.n_tables)
            comp["prefetch_cached_us"] = serial(lambda s: cached_prefetch(0, ms))
        pcie_bytes = B * cfg.n_tables * row_bytes
        comp["prefetch_host_GBps"] = pcie_bytes / (comp["prefetch_host_us"] * 1e-6) / 1e9
        # What kernel loads get over PCIe for this access pattern (the probes of
        # libengram_probe.so, measurement only): the step's B x n_tables row indices read from
        # one host table (every table has the same rows), nothing written; and a contiguous
        # read of the same number of bytes from host memory.
        from hashed_gram_embedding_hash_amd import build as hb
        PL = ctypes.CDLL(hb.PROBE_LIB)
        PL.engram_probe_rows_sink_words.restype = ctypes.c_int64
        PL.engram_probe_rows_sink_words.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
        PL.engram_probe_row_reads.argtypes = [P, ctypes.c_int32, P, ctypes.c_int64, ctypes.c_int32, P, P]
        PL.engram_probe_stream_reads.argtypes = [P, ctypes.c_int64, P, P]
        sink = torch.empty(max(int(PL.engram_probe_rows_sink_words(B, row_bytes, cfg.n_tables)), 8192 * 256),
                           dtype=torch.int32, device=dev)
        assert all(r == rows for r in hrows)
        comp["probe_host_rows_us"] = serial(lambda s: chk(-1 if PL.engram_probe_row_reads(
            P(haddr[0]), row_bytes, P(idx[0].data_ptr()), B, cfg.n_tables, P(sink.data_ptr()), ms) else 0))
        comp["probe_host_rows_GBps"] = pcie_bytes / (comp["probe_host_rows_us"] * 1e-6) / 1e9
        comp["probe_host_stream_us"] = serial(lambda s: chk(-1 if PL.engram_probe_stream_reads(
            P(haddr[0]), pcie_bytes, P(sink.data_ptr()), ms) else 0))
        comp["probe_host_stream_GBps"] = pcie_bytes / (comp["probe_host_stream_us"] * 1e-6) / 1e9
        comp["prefetch_host_frac_of_row_probe"] = comp["probe_host_rows_us"] / comp["prefetch_host_us"]
        # reference: pinned host-to-device copy of one contiguous 256 MiB block
        nb = min(256 << 20, rows * row_bytes)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        src = torch.from_numpy(np.ctypeslib.as_array((ctypes.c_uint8 * nb).from_address(haddr[0])))
        comp["h2d_memcpy_GBps"] = nb / (serial(lambda s: dst.copy_(src, non_blocking=True), 5) * 1e-6) / 1e9
        res = {
            "metric": "host-offload overhead of an Engram decode step (tables in pinned host DRAM vs HBM)",
            "value": round(100.0 * (med["host"] / med["hbm"] - 1.0), 2), "unit": "%", "higher_is_better": False,
            "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "offload", "sequences": B, "history": T0, "decode_steps": S,
                       "tables": f"{cfg.n_tables} x {rows} x {cfg.w} bf16", "table_GB": round(table_bytes / 1e9, 2),
                       "host_mem_available_GB": round(avail / 1e9, 1) if avail else None,
                       "full_size_rows": cfg.rows,
                       "sizing": f"100B parameters scaled to min(60% of free host RAM, {args.offload_host_gb:g} GB "
                                 "of pinned host memory, 80% of free HBM)",
                       "d_mem": cfg.d_mem, "d_model": cfg.d_model, "branches": 1,
                       "pipeline": "side stream: hash + fetch of step s+1; main stream: gate of step s",
                       "gate_call": ("engram_gate_forward (key weights folded every step)" if args.offload_fold_each_step
                                     else "engram_gate_forward_prepared (key weights folded once)")},
            "step_us": {k: round(v, 2) for k, v in med.items()},
            "step_us_all": {k: [round(x, 2) for x in v] for k, v in steps.items()},
            "step_timing": "graph replay of the whole two-stream pipeline (GPU-paced)",
            "step_us_eager": {k: round(v, 2) for k, v in med_eager.items()},
            "overhead_pct_eager": round(100.0 * (med_eager["host"] / med_eager["hbm"] - 1.0), 2),
            "host_enqueue_us_per_step": round(float(np.median(host_us)), 2),
            "decode_tokens_per_s": {k: round(B / (v * 1e-6), 1) for k, v in med.items()},
            "components_serial": {k: round(v, 2) for k, v in comp.items()},
            "pcie_bytes_per_step": pcie_bytes,
        }
        if cache is not None:
            res["row_cache"] = {
                "overhead_pct": round(100.0 * (med["cached"] / med["hbm"] - 1.0), 2),
                "overhead_pct_eager": round(100.0 * (med_eager["cached"] / med_eager["hbm"] - 1.0), 2),
                "rows_per_table": cache["capacity"], "hash_slots_per_table": cache["slots"],
                "hbm_GB": round(cache["hbm_bytes"] / 1e9, 3),
                "selected_from": f"hash indices of the {B} x {T0}-token histories",
                "hit_rate": round(cache["hit_rate"], 4),
                "pcie_bytes_per_step": round(pcie_bytes * (1.0 - cache["hit_rate"])),
                "select_s": cache["select_s"], "build_s": cache["build_s"]}
        print(json.dumps(res), flush=True)
    finally:
        dtabs.clear()
        torch.cuda.synchronize()
        for a in haddr:
            eg.host_free(a)


def measure_conv(args, cfg, bufs, h, layer, outs, flush):
    """The short convolution of Eq. (5), measured beside the step (it is not part of the
    hash+gather+gate metric).  Each rep, with the cache flush before each timed piece:
    the plain gate; the gate writing the gated values as well, followed at once by
    engram_conv_forward on every branch (the layer's own order: the values the
    convolution reads were just written); and the convolution alone from cold caches.
    Every piece is bracketed by events."""
    import torch
    import synth
    import hashed_gram_embedding_hash_amd as eg
    dev = outs[0].device
    dil = synth.conv_dilation(cfg)
    vals = [torch.empty_like(x) for x in outs]
    params = [synth.conv_params(cfg, m, device=dev) for m in range(cfg.n_branch)]

    def gate(with_values):
        eg.engram_gate_forward(bufs["mem"], h, layer.wk, layer.wv, layer.gq, layer.gk, cfg.eps, out=outs,
                               value_out=vals if with_values else None, key_norm=layer.key_norm)

    def conv():
        for m in range(cfg.n_branch):
            eg.engram_conv_forward(vals[m], cfg.batch, cfg.seq, params[m][0], params[m][1], dil, outs[m], cfg.eps)

    for _ in range(3):
        gate(True)
        conv()
    torch.cuda.synchronize()
    reps = max(5, args.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(reps)]
    for i in range(reps):
        if flush is not None:
            flush.fill_(float(i))
        ev[i][0].record()
        gate(False)
        ev[i][1].record()
        if flush is not None:
            flush.fill_(float(i + 1))
        ev[i][2].record()
        gate(True)
        ev[i][3].record()
        conv()
        ev[i][4].record()
        if flush is not None:
            flush.fill_(float(i + 2))
        ev[i][5].record()
        conv()
        ev[i][6].record()
    torch.cuda.synchronize()
    avg = lambda a, b: sum(ev[i][a].elapsed_time(ev[i][b]) for i in range(reps)) / reps
    gate_ms, gate_v_ms, conv_ms, conv_cold_ms = avg(0, 1), avg(2, 3), avg(3, 4), avg(5, 6)
    es = 2 if cfg.dtype == "bf16" else 4
    unit = cfg.tokens * cfg.d_model * es * cfg.n_branch     # one [tokens, d_model] array per branch
    conv_bytes = 3 * unit          # read the gated values once, read and write out
    rate = lambda ms: conv_bytes / (ms * 1e-3) / 1e9
    return {"kernel": "engram_conv_forward: conv_rms_kernel + conv_apply_kernel",
            "taps": synth.CONV_TAPS, "dilation": dil, "branches": cfg.n_branch, "reps": reps,
            "bytes_algorithmic": conv_bytes,
            "ms_after_gate": round(conv_ms, 5), "GB/s_after_gate": round(rate(conv_ms), 1),
            "ms_cold": round(conv_cold_ms, 5), "GB/s_cold": round(rate(conv_cold_ms), 1),
            "hbm_frac_cold": round(rate(conv_cold_ms) / PEAK_HBM_GBS, 4),
            "gate_ms": round(gate_ms, 5), "gate_with_values_ms": round(gate_v_ms, 5),
            "values_write_GB/s": round(unit / max(1e-9, (gate_v_ms - gate_ms) * 1e-3) / 1e9, 1),
            "gate_with_values_plus_conv_ms": round(gate_v_ms + conv_ms, 5)}


def measure_ceiling(args, cfg, layer, bufs, sep_per, per, flush):
    """What the memory system delivers for the gather's access pattern, from the probes
    of libengram_probe.so (not part of the path): the same index matrix, read-only from
    one table (the rows' bytes, nothing written), a contiguous read of the same number of
    bytes, and a contiguous device copy of the memory vectors (read + write), each timed
    with events after the cache flush.  The gather (engram_gather) and the fused lookup
    are then stated against these as well as against the 8 TB/s spec."""
    import ctypes
    import torch
    from hashed_gram_embedding_hash_amd import build as hb
    L = ctypes.CDLL(hb.PROBE_LIB)
    P = ctypes.c_void_p
    L.engram_probe_rows_sink_words.restype = ctypes.c_int64
    L.engram_probe_rows_sink_words.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    L.engram_probe_row_reads.argtypes = [P, ctypes.c_int32, P, ctypes.c_int64, ctypes.c_int32, P, P]
    L.engram_probe_stream_reads.argtypes = [P, ctypes.c_int64, P, P]
    dev = bufs["mem"].device
    T, nt = cfg.tokens, cfg.n_tables
    row_bytes = cfg.w * (4 if cfg.dtype == "f32" else 2)
    idx = bufs["idx"]                      # [tokens, n_tables], written by engram_compress_hash
    table0 = layer.tables[0]
    sink = torch.empty(max(int(L.engram_probe_rows_sink_words(T, row_bytes, nt)), 8192 * 256), dtype=torch.int32,
                       device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    row_total = T * nt * row_bytes
    stream_bytes = min(row_total, table0.numel() * table0.element_size()) // 16 * 16
    copy_dst = torch.empty_like(bufs["mem"])

    def rows():
        assert L.engram_probe_row_reads(P(table0.data_ptr()), row_bytes, P(idx.data_ptr()), T, nt,
                                        P(sink.data_ptr()), stream) == 0

    def stream_read():
        assert L.engram_probe_stream_reads(P(table0.data_ptr()), stream_bytes, P(sink.data_ptr()), stream) == 0

    def copy():
        copy_dst.copy_(bufs["mem"])

    def timed(fn, reps):
        ts = []
        for i in range(reps):
            if flush is not None:
                flush.fill_(float(i))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ts) / reps
    for fn in (rows, stream_read, copy):
        fn()
    reps = max(5, args.steps)
    t_rows, t_stream, t_copy = timed(rows, reps), timed(stream_read, reps), timed(copy, reps)
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    ceil_rows = gbs(row_total, t_rows)
    g_ms, l_ms = sep_per["gather"], per["lookup"]
    return {
        "probe": "libengram_probe.so (measurement only): engram_probe_row_reads / engram_probe_stream_reads",
        "random_rows_read_only": {"ms": round(t_rows, 5), "row_GB/s": round(ceil_rows, 1),
                                  "note": f"the step's {T} x {nt} row indices, all read from table 0 "
                                          f"({row_bytes}-byte rows), nothing written"},
        "stream_read": {"ms": round(t_stream, 5), "GB/s": round(gbs(stream_bytes, t_stream), 1),
                        "bytes": stream_bytes},
        "device_copy_of_memory_vectors": {"ms": round(t_copy, 5),
                                          "GB/s_read_plus_write": round(gbs(2 * bufs["mem"].numel() *
                                                                            bufs["mem"].element_size(), t_copy), 1)},
        "gather": {"ms": round(g_ms, 5), "row_read_GB/s": round(gbs(row_total, g_ms), 1),
                   "row_read_frac_of_random_row_ceiling": round(t_rows / g_ms, 4)},
        "lookup": {"ms": round(l_ms, 5), "row_read_GB/s": round(gbs(row_total, l_ms), 1),
                   "row_read_frac_of_random_row_ceiling": round(t_rows / l_ms, 4)},
    }


def measure_gemm_reference(args, cfg, layer, bufs, per, flush):
    """The library's plain bf16 GEMM (torch.mm on ROCm: hipBLASLt) on the gate's contraction:
    the memory vectors [tokens, d_mem] times every projection matrix of the call at once
    ([d_mem, 2 * n_branch * d_model], contiguous), written out as bf16; no norms, gate or
    residual.  Timed with events after the cache flush, as the gate is.  A reference for the
    gate's matrix-core rate, not part of the path."""
    import torch
    mats = [w for m in range(cfg.n_branch) for w in (layer.wk[m], layer.wv[m])]
    w_t = torch.cat(mats, dim=0).t().contiguous()          # [d_mem, N]
    mem = bufs["mem"]
    out = torch.empty((mem.shape[0], w_t.shape[1]), dtype=mem.dtype, device=mem.device)
    for _ in range(2):
        torch.mm(mem, w_t, out=out)
    torch.cuda.synchronize()
    reps = max(5, args.steps // 2)
    ts = []
    for i in range(reps):
        if flush is not None:
            flush.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.mm(mem, w_t, out=out)
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ts) / reps
    flops = 2.0 * mem.shape[0] * mem.shape[1] * w_t.shape[1]
    tf = flops / (ms * 1e-3) / 1e12
    gate_tf = flops / (per["gate"] * 1e-3) / 1e12
    del out, w_t
    return {"call": "torch.mm (hipBLASLt), bf16 in and out, fp32 accumulation",
            "shape": [int(mem.shape[0]), int(mem.shape[1]), len(mats) * cfg.d_model],
            "ms": round(ms, 5), "TFLOP/s": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "gate_TFLOP/s": round(gate_tf, 2), "gate_vs_gemm": round(gate_tf / tf, 4),
            "note": "the same FLOPs as the gate's two projections per branch, as one plain GEMM that writes "
                    "its products to HBM (the gate never stores them and adds the norms, the gate and the "
                    "residual); a reference, not part of the path"}


def cpu_baseline(cfg, target_s, fp8=False):
    """The oracle (single thread) on the first tokens of sequence 0: compress, hash,
    gather and gate (its FP8 form with fp8).  Table rows are regenerated outside the
    timed region."""
    import numpy as np
    import torch
    import oracle
    import synth

    def host_view(t):
        t = t.contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    raw = synth.raw_ids(cfg)
    cmap = synth.comp_map(cfg)
    mult, rows = synth.multipliers(cfg), synth.table_rows_u32(cfg)
    wts = [synth.weights(cfg, m) for m in range(cfg.n_branch)]
    gns = [synth.gains(cfg, m) for m in range(cfg.n_branch)]
    wts = [(host_view(a), host_view(b)) for a, b in wts]
    gns = [(host_view(a), host_view(b)) for a, b in gns]
    dt = oracle.F32 if cfg.dtype == "f32" else oracle.BF16

    def run(n):
        seq = raw[:1, :n]
        t0 = time.perf_counter()
        ids, _ = oracle.compress(seq, cmap)
        idx = oracle.hash_ids(ids, cfg.orders, cfg.heads, mult, rows, cfg.vocab_c)
        t_int = time.perf_counter() - t0
        subs, remap = [], np.empty_like(idx)
        for b in range(cfg.n_tables):   # input generation: not timed
            uniq, inv = np.unique(idx[:, b], return_inverse=True)
            subs.append(host_view(synth.table_rows(cfg, b, torch.from_numpy(uniq.astype(np.int64)))))
            remap[:, b] = inv
        h = [host_view(synth.hidden_rows(cfg, m, torch.arange(n))) for m in range(cfg.n_branch)]
        t1 = time.perf_counter()
        e = oracle.gather(remap, subs)
        gate = oracle.gate_fp8 if fp8 else oracle.gate
        for m in range(cfg.n_branch):
            gate(e, h[m], wts[m][0], wts[m][1], gns[m][0], gns[m][1], cfg.eps, dt)
        return t_int + time.perf_counter() - t1

    # one thread, pinned to one core of those this process may use, for the timed runs
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})
    try:
        probe = 8
        t = run(probe)
        n = int(max(probe, min(cfg.seq, probe * target_s / max(t, 1e-9))))
        t = run(n)
    finally:
        os.sched_setaffinity(0, set(allowed))
    return {"value": n / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "pinned_core": core, "host_cores": os.cpu_count(), "cores_available": len(allowed),
            "cpu_model": cpu_model(),
            "sample": f"first {n} tokens of sequence 0 of the {cfg.name} workload: compress, hash, "
                      f"gather and all {cfg.n_branch} {'fp8 ' if fp8 else ''}gate branch(es), one thread pinned "
                      f"to core {core}, {t:.1f} s"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def run_workload(args, name, secondary=False):
    """One workload's measurement: the step (engram_lookup + engram_gate_forward) timed
    eagerly and as a graph replay, with the per-call breakdown and the gate's roofline;
    unless secondary, also the separate calls, the prepared-weight gate, the FP8 steps and
    the convolution.  Returns the result dict (without the CPU baseline)."""
    import torch
    import synth
    import hashed_gram_embedding_hash_amd as eg
    from hashed_gram_embedding_hash_amd.pipeline import EngramLayer

    cfg = synth.CONFIGS[name]
    dev = torch.device("cuda:0")
    print(f"[bench] building inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = synth.device_inputs(cfg, dev)
    if args.shared_wv:
        inp["wv"] = [inp["wv"][0]] * cfg.n_branch
    key_norm = eg.KEY_NORM_PROJECTED if args.key_norm == "projected" else eg.KEY_NORM_MEMORY
    if key_norm == eg.KEY_NORM_PROJECTED:
        inp["gk"] = [synth.gains(cfg, m, dev, projected_key=True)[1] for m in range(cfg.n_branch)]
    layer = EngramLayer(inp["map"], cfg.orders, cfg.heads, inp["mult"], inp["tables"], inp["wk"], inp["wv"],
                        inp["gq"], inp["gk"], cfg.eps, pad_id=cfg.vocab_c, key_norm=key_norm)
    outs = [torch.empty_like(h) for h in inp["h"]]
    bufs = layer.buffers(cfg.batch, cfg.seq)
    raw, h = inp["raw"], inp["h"]

    def make_step(fp8):
        def step(ev=None):
            # compression, hashing and the gather in one kernel (engram_lookup), then the gate
            if ev is not None:
                ev[0].record()
            eg.engram_lookup(raw, layer.cmap, layer.orders, layer.heads, layer.mult, layer.tables, layer.pad_id,
                             out=bufs["mem"])
            if ev is not None:
                ev[1].record()
            eg.engram_gate_forward(bufs["mem"], h, layer.wk, layer.wv, layer.gq, layer.gk, cfg.eps, out=outs,
                                   key_norm=layer.key_norm, fp8=fp8)
            if ev is not None:
                ev[2].record()
        return step

    flush = (torch.empty(args.flush_mb << 18, dtype=torch.float32, device=dev) if args.flush_mb > 0 else None)
    names = ["lookup", "gate"]

    def time_steps(step, n_steps, n_warm, use_graph, names=names):
        """Warm-up, then n_steps iterations of: the eager step (events between its calls give
        the per-call breakdown) and the graph replay, each after the cache flush, so both see
        the same clocks and the same cold caches.  Returns (ms per step, ms eager, per-call
        ms, wall seconds)."""
        print(f"[bench] warmup {n_warm}", file=sys.stderr, flush=True)
        for _ in range(n_warm):
            step()
        torch.cuda.synchronize()
        # The same step captured once in a HIP graph (a launch per step instead of one per
        # kernel).  Two eager steps on the capture stream come first, so the gate's scratch
        # is sized and last used on that stream (no allocation or cross-stream wait is
        # recorded).
        graph = None
        if use_graph:
            gs = torch.cuda.Stream()
            gs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(gs):
                step()
                step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=gs):
                step()
            torch.cuda.synchronize()
            for _ in range(5):
                graph.replay()
            torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(n_steps)]
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
        print(f"[bench] timing {n_steps} steps" + ("" if graph is None else " and graph replays"),
              file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        for i in range(n_steps):
            if flush is not None:
                flush.fill_(float(i))       # evicts L2 and MALL; outside the step's events
            step(evs[i])
            if graph is not None:
                if flush is not None:
                    flush.fill_(float(i) + 0.5)
                gev[i][0].record()
                graph.replay()
                gev[i][1].record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        # per-step time: first to last event of each step (the flush between steps excluded)
        ms_eager = sum(evs[i][0].elapsed_time(evs[i][-1]) for i in range(n_steps)) / n_steps
        ms_step = ms_eager if graph is None else sum(a.elapsed_time(b) for a, b in gev) / n_steps
        per = {n: sum(evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(n_steps)) / n_steps
               for k, n in enumerate(names)}
        return ms_step, ms_eager, per, t_wall

    ms_step, ms_eager, per, t_wall = time_steps(make_step(args.fp8), args.steps, args.warmup, not args.no_graph)

    # The same step as one call, engram_lookup_gate: the gate's kernel hashes each token and
    # loads the table rows itself (the memory vectors are never stored).  Its key tiles are
    # feature-major: bit-identical to the two calls with feature-major key tiles, and within
    # the fp32 rounding of the logit's sum of them with memory-major ones.
    fused_step = None
    if cfg.dtype == "bf16" and not args.fp8 and not args.no_fused:
        def fused(ev=None):
            if ev is not None:
                ev[0].record()
            eg.engram_lookup_gate(raw, layer.cmap, layer.orders, layer.heads, layer.mult, layer.tables,
                                  layer.pad_id, h, layer.wk, layer.wv, layer.gq, layer.gk, cfg.eps, out=outs,
                                  key_norm=layer.key_norm)
            if ev is not None:
                ev[1].record()
        ms_f, ms_fe, _, _ = time_steps(fused, args.steps, 3, not args.no_graph, names=["step"])
        fused_step = {"call": "engram_lookup_gate", "ms_per_step": round(ms_f, 5),
                      "ms_per_step_eager": round(ms_fe, 5), "tokens/s": round(cfg.tokens / (ms_f * 1e-3), 1),
                      "speedup_vs_two_calls": round(ms_step / ms_f, 4),
                      "note": "lookup and gate in one pass: the gate kernel hashes each token's n-grams and "
                              "loads the table rows into its operand tiles (no memory-vector array); timed "
                              "like the step, in the same run"}
    if secondary:
        work = algorithmic(cfg, args.shared_wv)
        gate_tf = work["gate"]["flops"] / (per["gate"] * 1e-3) / 1e12
        lk = work["lookup"]["bytes"] / (per["lookup"] * 1e-3) / 1e9
        return {"workload": cfg.name, "tokens": cfg.tokens, "value": round(cfg.tokens / (ms_step * 1e-3), 1),
                "unit": "tokens/s", "ms_per_step": round(ms_step, 5), "ms_per_step_eager": round(ms_eager, 5),
                "steps": args.steps, "warmup": args.warmup,
                "kernels": {"lookup": {"ms": round(per["lookup"], 5), "GB/s": round(lk, 1),
                                       "hbm_frac": round(lk / PEAK_HBM_GBS, 4)},
                            "gate": {"ms": round(per["gate"], 5), "TFLOP/s": round(gate_tf, 2),
                                     "frac": round(gate_tf / PEAK_BF16_TFLOPS, 4)}},
                "fused_step": fused_step,
                "config": workload_desc(cfg, args)}

    # the lookup as its separate calls (engram_compress_hash, then engram_gather), for each
    # call's own rate
    def separate(ev=None):
        if ev is not None:
            ev[0].record()
        eg.engram_compress_hash(raw, layer.cmap, layer.orders, layer.heads, layer.mult, layer.rows, layer.pad_id,
                                out=bufs["idx"])
        if ev is not None:
            ev[1].record()
        eg.engram_gather(bufs["idx"], layer.tables, out=bufs["mem"])
        if ev is not None:
            ev[2].record()
    sep_names = ["compress_hash", "gather"]
    _, _, sep_per, _ = time_steps(separate, args.steps, 3, False, names=sep_names)

    # the bf16 gate on key weights folded once (engram_gate_prepare): the same results, without
    # the per-call folding kernel
    prepared = None
    if cfg.dtype == "bf16" and layer.key_norm == eg.KEY_NORM_MEMORY and not args.fp8:
        folded = eg.engram_gate_prepare(layer.wk, layer.gq, layer.gk)
        def gate_prepared(ev=None):
            if ev is not None:
                ev[0].record()
            eg.engram_gate_forward_prepared(bufs["mem"], h, folded, layer.wv, cfg.eps, out=outs)
            if ev is not None:
                ev[1].record()
        _, _, prep_per, _ = time_steps(gate_prepared, args.steps, 3, False, names=["gate"])
        prepared = prep_per["gate"]

    work = algorithmic(cfg, args.shared_wv)
    def rates(n, ms):
        s = ms * 1e-3
        d = {"ms": round(ms, 5)}
        if "bytes" in work[n]:
            d["GB/s"] = round(work[n]["bytes"] / s / 1e9, 1)
            d["hbm_frac"] = round(work[n]["bytes"] / s / 1e9 / PEAK_HBM_GBS, 4)
        return d
    kernels = {}
    for n in names:
        d = rates(n, per[n])
        if "flops" in work[n]:
            d["TFLOP/s"] = round(work[n]["flops"] / (per[n] * 1e-3) / 1e12, 2)
        kernels[n] = d
    separate_calls = {n: rates(n, sep_per[n]) for n in sep_names}
    if prepared is not None:
        separate_calls["gate_prepared_weights"] = {
            "ms": round(prepared, 5), "TFLOP/s": round(work["gate"]["flops"] / (prepared * 1e-3) / 1e12, 2),
            "note": "engram_gate_forward_prepared on key weights folded once by engram_gate_prepare "
                    "(feature-major key tiles: bit-identical to engram_gate_forward's of that form; no "
                    "per-call folding kernel), timed eagerly after the cache flush"}
    gate_s = per["gate"] * 1e-3
    if cfg.dtype == "bf16" and args.fp8:
        peak, dtype = PEAK_FP8_TFLOPS, "fp8e4m3 projections, bf16 storage"
    elif cfg.dtype == "bf16":
        peak, dtype = PEAK_BF16_TFLOPS, "bf16"
    else:
        peak, dtype = PEAK_FP32_TFLOPS, "f32"
    achieved = work["gate"]["flops"] / gate_s / 1e12
    default_gate = not args.shared_wv and args.key_norm == "memory" and not args.fp8
    traffic = measured_traffic(cfg) if cfg.dtype == "bf16" and default_gate else None
    kernel = ("engram_gate_forward_fp8: gate_prep_projected_kernel + quant_rows_kernel (W_K, W_V, mem) + "
              "gate_persistent_kernel (events bracket all)" if args.fp8 else
              "engram_gate_forward: the key-weight fold (gate_prep_kernel, or gate_prep_t_kernel for "
              "memory-major key tiles) + gate_persistent_kernel (events bracket both; the fold is about "
              "3 % of the call)")
    roofline = {"kernel": kernel, "key_tiles": gate_key_tiles(cfg, args),
                "bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "traffic_algorithmic": work["gate"]["bytes"],
                "flops_per_launch": work["gate"]["flops"], "avg_ms": round(per["gate"], 5)}

    result = {
        "metric": METRIC,
        "value": round(cfg.tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_launch": "eager" if args.no_graph else "hip graph replay (one launch per step)",
        "ms_per_step_eager": round(ms_eager, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic (seeded Zipf ids, counter-generated tables/weights/hidden)",
        "config": workload_desc(cfg, args),
        "wall_s_timed": round(t_wall, 4),
        "cache_flush_mb_between_steps": args.flush_mb,
        "kernels": kernels,
        "fused_step": fused_step,
        "separate_calls": {**separate_calls, "note": "the lookup as engram_compress_hash + engram_gather, and the gate on prepared weights, "
                                                     "timed eagerly in the same run (not part of the step)"},
        "roofline": roofline,
    }
    if cfg.dtype == "bf16" and not args.fp8 and not args.no_fp8:
        # the same step with the gate's projections on E4M3 codes (engram_gate_forward_fp8,
        # quantization of W_K, W_V and the memory vectors inside the call)
        print("[bench] fp8 gate step", file=sys.stderr, flush=True)
        f_ms, f_eager, f_per, _ = time_steps(make_step(True), args.steps, max(3, args.warmup // 2), not args.no_graph)
        f_tf = work["gate"]["flops"] / (f_per["gate"] * 1e-3) / 1e12
        result["fp8_step"] = {
            "value": round(cfg.tokens / (f_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(f_ms, 5),
            "ms_per_step_eager": round(f_eager, 5),
            "dtype": "fp8e4m3 projections (per-row scales), bf16 storage",
            "kernels_ms": {n: round(f_per[n], 5) for n in names},
            "gate": {"TFLOP/s": round(f_tf, 2), "peak": PEAK_FP8_TFLOPS, "frac": round(f_tf / PEAK_FP8_TFLOPS, 4),
                     "frac_of_bf16_peak": round(f_tf / PEAK_BF16_TFLOPS, 4),
                     "note": "events bracket the whole call: counter clear, three quantization launches "
                             "and the persistent kernel"},
        }
        # the FP8 pipeline with its operands made once: the weights quantized before timing
        # (engram_gate_prepare_fp8), the lookup writing E4M3 memory vectors (engram_lookup_fp8),
        # the gate on the codes (engram_gate_forward_fp8q)
        print("[bench] fp8 step with prepared operands", file=sys.stderr, flush=True)
        prep = eg.engram_gate_prepare_fp8(layer.wk, layer.wv, layer.gq, layer.gk, key_norm=layer.key_norm)
        q_codes = torch.empty((cfg.tokens, cfg.d_mem), dtype=torch.uint8, device=dev)
        q_scales = torch.empty(cfg.tokens, dtype=torch.float32, device=dev)
        q_ss = torch.empty(cfg.tokens, dtype=torch.float32, device=dev)

        def step_q(ev=None):
            if ev is not None:
                ev[0].record()
            eg.engram_lookup_fp8(raw, layer.cmap, layer.orders, layer.heads, layer.mult, layer.tables, layer.pad_id,
                                 codes=q_codes, scales=q_scales, sumsq=q_ss)
            if ev is not None:
                ev[1].record()
            eg.engram_gate_forward_fp8q(q_codes, q_scales, q_ss, h, prep, layer.gq, layer.gk, cfg.eps, out=outs)
            if ev is not None:
                ev[2].record()
        q_ms, q_eager, q_per, _ = time_steps(step_q, args.steps, max(3, args.warmup // 2), not args.no_graph,
                                             names=["lookup_fp8", "gate"])
        q_tf = work["gate"]["flops"] / (q_per["gate"] * 1e-3) / 1e12
        result["fp8_step"]["with_prepared_operands"] = {
            "value": round(cfg.tokens / (q_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(q_ms, 5),
            "ms_per_step_eager": round(q_eager, 5), "kernels_ms": {n: round(q_per[n], 5) for n in q_per},
            "gate": {"TFLOP/s": round(q_tf, 2), "frac": round(q_tf / PEAK_FP8_TFLOPS, 4),
                     "frac_of_bf16_peak": round(q_tf / PEAK_BF16_TFLOPS, 4)},
            "note": "weights quantized once before timing (engram_gate_prepare_fp8); per step: engram_lookup_fp8 "
                    "(compress, hash, gather and per-token quantization) and engram_gate_forward_fp8q",
        }
    if not args.no_conv:
        print("[bench] short convolution", file=sys.stderr, flush=True)
        result["conv"] = measure_conv(args, cfg, bufs, h, layer, outs, flush)
    print("[bench] gather ceiling probes", file=sys.stderr, flush=True)
    result["gather_ceiling"] = measure_ceiling(args, cfg, layer, bufs, sep_per, per, flush)
    if cfg.dtype == "bf16" and not args.fp8 and not args.shared_wv:
        print("[bench] library GEMM reference", file=sys.stderr, flush=True)
        result["gemm_reference"] = measure_gemm_reference(args, cfg, layer, bufs, per, flush)
    return result


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on exactly one GPU; "
                                   "the Engram path here is single-GPU (no multi-GPU runs)"}))
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    if args.probes:
        probes()
        return

    if args.timeline:
        timeline(args)
        return

    if args.key_form != "auto":
        import hashed_gram_embedding_hash_amd as eg
        eg.engram_debug_gate_key_form(args.key_form)

    if args.config == "offload":
        run_offload(args)
        return

    result = run_workload(args, args.config)
    if args.config == "large" and not args.no_secondary:
        import torch
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        print("[bench] secondary workload: small", file=sys.stderr, flush=True)
        result["secondary"] = {"small": run_workload(args, "small", secondary=True),
                               "note": "the small workload (4 x 4096 tokens, d_model 2560, one branch), step "
                                       "timed by the same procedure after the main line"}
    if not args.no_cpu_baseline:
        import synth
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(synth.CONFIGS[args.config], args.cpu_seconds, fp8=args.fp8)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

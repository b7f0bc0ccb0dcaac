"""Build the HIP library libengram.so (gfx950) in-tree with hipcc.

Each csrc/*.hip file is compiled to an object in parallel, then linked into
hashed_gram_embedding_hash_amd/libengram.so.  The benchmark's measurement probes
(probe/*.hip, not part of the method) go to libengram_probe.so, and a diagnostic copy of the
library whose gate stamps a per-tile timeline (gate_bf16.hip compiled with ENGRAM_GATE_TIMELINE)
to libengram_timeline.so.  Always recompiles (the caller asked for a build); objects go to
_build/ at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "engram")
LIB = os.path.join(PKG, "libengram.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # atomics stay single atomics: the gate claims its next tile early and reads the
    # result late, which the wave-aggregating rewrite (it consumes the result at once)
    # would turn into a full memory round trip; the library's other atomics are
    # already one per wave or rare
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, timeline: bool = False) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + (".timeline.o" if timeline else ".o"))
    cmd = [HIPCC, *FLAGS, *(["-DENGRAM_GATE_TIMELINE"] if timeline else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


PROBE_DIR = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libengram_probe.so")
TIMELINE_LIB = os.path.join(PKG, "libengram_timeline.so")
TIMELINE_SRC = os.path.join(CSRC, "gate_bf16.hip")


def probe_sources():
    return sorted(os.path.join(PROBE_DIR, f) for f in os.listdir(PROBE_DIR) if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    """Build libengram.so, the benchmark's measurement probes (libengram_probe.so) and the
    timeline build (libengram_timeline.so)."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    psrcs = probe_sources()
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        timeline = ex.submit(_compile, TIMELINE_SRC, True)  # the slowest file: start it first
        probes = [ex.submit(_compile, p) for p in psrcs]
        objs = list(ex.map(_compile, srcs))
        probe_objs = [p.result() for p in probes]
        timeline_obj = timeline.result()
    timeline_objs = [timeline_obj if os.path.basename(o) == os.path.basename(TIMELINE_SRC) + ".o" else o for o in objs]
    assert timeline_obj in timeline_objs
    for out, parts in ((PROBE_LIB, probe_objs), (TIMELINE_LIB, timeline_objs), (LIB, objs)):
        tmp = out + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *parts]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, out)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

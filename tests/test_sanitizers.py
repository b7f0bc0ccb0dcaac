"""CPU-side tooling: the oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

- tests/sanitize/oracle_checks.c links the oracle built with gcc's sanitizers and runs
  every oracle function on small inputs with known values.
- tests/sanitize/host_checks.cpp links every csrc/*.hip object built with the
  sanitizers on the host code only (-Xarch_host; the gfx950 code is built as usual) and
  calls each C-ABI entry point with arguments that fail validation (nothing reaches the
  GPU), plus the row cache's host-side selection against a brute force.
Both abort on the first sanitizer report (halt_on_error)."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "hashed_gram_embedding_hash_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ENV = {**os.environ, "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_checks")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
          os.path.join(SAN, "oracle_checks.c"), os.path.join(ROOT, "oracle", "engram_oracle.c"), "-lm"])
    r = _run([exe], env=ENV)
    assert "oracle checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_library_host_code_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", *san, "-I", os.path.join(ROOT, "include")]
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    srcs.append(os.path.join(SAN, "host_checks.cpp"))

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        _run([HIPCC, *flags, *lang, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(OUT, "host_checks")
    _run([HIPCC, "--offload-arch=gfx950", *san, *objs, "-o", exe])
    r = _run([exe], env=ENV)
    assert "host checks passed" in r.stdout

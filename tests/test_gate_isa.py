"""The bf16 gate's main loop as compiled for gfx950 (CPU: hipcc cross-compiles).

The operand ring's direct global->LDS loads are issued from inline asm and waited for by
hand (s_waitcnt vmcnt(N) with N >= one chunk's 8 loads in flight).  The compiler does
not see those loads, but the hardware counts them with its own: a wait the compiler adds
inside the k-step loop for one of its own loads (a spill reload, say) would also wait for
the ring's refills and drain the prefetch on every k-step.  That happened once to the
memory-major instantiation (vmcnt(0) in the steady k-step, 15-20 % slower k-steps).  This
test compiles gate_bf16.hip as the build does and checks, for the two persistent kernels
the default gate launches (feature-major and memory-major key tiles), that no block of
the main loop (a basic block holding at least 16 MFMAs) waits for fewer than 8 vector
memory operations in flight.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "hashed_gram_embedding_hash_amd", "csrc", "gate_bf16.hip")
KERNELS = {
    "feature-major": "_ZN6engram12_GLOBAL__N_122gate_persistent_kernelILb0ELb0ELb0ELb0ELb0EEEvNS_8GateArgsE",
    "memory-major": "_ZN6engram12_GLOBAL__N_122gate_persistent_kernelILb0ELb0ELb0ELb0ELb1EEEvNS_8GateArgsE",
}
MIN_IN_FLIGHT = 8  # one operand chunk: G_INSTR direct loads per wave


def _blocks(asm: str, symbol: str):
    start = asm.index(symbol + ":")
    body = asm[start:asm.index(".Lfunc_end", start)]
    blocks, cur = {"entry": []}, "entry"
    for line in body.split("\n"):
        m = re.match(r"^(\.LBB\d+_\d+):", line)
        if m:
            cur = m.group(1)
            blocks[cur] = []
        elif line.startswith("\t") and not line.startswith(("\t.", "\t;")) and line.strip():
            blocks[cur].append(line.strip().split(";")[0].strip())
    return blocks


@pytest.fixture(scope="module")
def gate_asm(tmp_path_factory):
    from hashed_gram_embedding_hash_amd import build
    hipcc = build.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "gate_bf16.s"
    cmd = [hipcc, *build.FLAGS, "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


@pytest.mark.parametrize("form", sorted(KERNELS))
def test_main_loop_never_drains_the_operand_ring(gate_asm, form):
    blocks = _blocks(gate_asm, KERNELS[form])
    loop_blocks = {n: ops for n, ops in blocks.items() if sum("mfma" in o for o in ops) >= 16}
    assert len(loop_blocks) >= 8, f"{form}: main-loop blocks not found ({len(loop_blocks)})"
    bad = []
    for name, ops in loop_blocks.items():
        for o in ops:
            m = re.search(r"vmcnt\((\d+)\)", o)
            if o.startswith("s_waitcnt") and m and int(m.group(1)) < MIN_IN_FLIGHT:
                bad.append(f"{name}: {o}")
    assert not bad, f"{form}: waits inside the main loop drain the operand ring: {bad}"

"""engram_gate_forward_noalloc (the gate without any allocation, on the library's fixed
scratch array) against engram_gate_forward through the C ABI: bit-identical outputs and
gates on two calls in a row, the second with a smaller input, and the oversized-shape
refusal."""
import ctypes

import numpy as np
import pytest
import torch

import hashed_gram_embedding_hash_amd as eg
import synth
from gpu_helpers import sentinel_like

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(cfg, n_tok, n_branch, seed, shared=False):
    g = torch.Generator().manual_seed(seed)
    e = (torch.randn(n_tok, cfg.d_mem, generator=g) * 0.5).to(torch.bfloat16).to(DEV)
    hs = [torch.randn(n_tok, cfg.d_model, generator=g).to(torch.bfloat16).to(DEV) for _ in range(n_branch)]
    ws = [synth.weights(cfg, m, DEV) for m in range(n_branch)]
    wks = [w[0] for w in ws]
    wvs = [ws[0][1]] * n_branch if shared else [w[1] for w in ws]
    gs = [synth.gains(cfg.replace(gamma_jitter=0.2), m, DEV) for m in range(n_branch)]
    return e, hs, wks, wvs, [x[0] for x in gs], [x[1] for x in gs]


def _both(e, hs, wks, wvs, gqs, gks, eps=1e-6):
    nb, n = len(hs), e.shape[0]
    a_ref = sentinel_like(torch.empty((nb, n), dtype=torch.float32, device=DEV))
    a_na = sentinel_like(torch.empty((nb, n), dtype=torch.float32, device=DEV))
    ref = eg.engram_gate_forward(e, hs, wks, wvs, gqs, gks, eps, gate_out=a_ref,
                                 out=[sentinel_like(torch.empty_like(h)) for h in hs])
    na = eg.engram_gate_forward(e, hs, wks, wvs, gqs, gks, eps, gate_out=a_na, noalloc=True,
                                out=[sentinel_like(torch.empty_like(h)) for h in hs])
    torch.cuda.synchronize()
    return ref, a_ref, na, a_na


def test_noalloc_equals_gate_forward_two_calls_second_smaller():
    """Calls in a row, each smaller than the one before: 13,312 tokens x 2 branches (520
    key tiles: memory-major, the array holding the transposed folded weights), then 3,000
    x 2 and 300 x 1 (feature-major, the same array refilled)."""
    cfg = synth.CONFIGS["small"]
    print("noalloc gate: 13312 tokens x 2 branches, 3000 x 2, then 300 x 1", flush=True)
    for n_tok, nb, seed in ((13312, 2, 4), (3000, 2, 1), (300, 1, 2)):
        ref, a_ref, na, a_na = _both(*_case(cfg, n_tok, nb, seed))
        assert torch.equal(a_ref, a_na) and torch.isfinite(a_na).all()
        for m in range(nb):
            assert torch.equal(ref[m].view(torch.int16), na[m].view(torch.int16)), (n_tok, m)
    assert eg.engram_gate_wait_timeouts() == 0


def test_noalloc_shared_wv_and_decode_shape():
    """Three branches sharing W_V at the decode shape (256 tokens, d_model 4096)."""
    cfg = synth.CONFIGS["offload"]
    print("noalloc gate: decode shape, 3 branches sharing W_V", flush=True)
    ref, a_ref, na, a_na = _both(*_case(cfg, 256, 3, 3, shared=True))
    assert torch.equal(a_ref, a_na)
    for m in range(3):
        assert torch.equal(ref[m].view(torch.int16), na[m].view(torch.int16)), m


def test_noalloc_refuses_shapes_beyond_its_array():
    """A request whose scratch exceeds ENGRAM_NOALLOC_SCRATCH_BYTES is refused on the
    host before anything is enqueued (pointers are never dereferenced)."""
    L = eg.lib()
    one = (ctypes.c_void_p * 8)(*([4096] * 8))
    st = L.engram_gate_forward_noalloc(ctypes.c_void_p(4096), 1 << 20, 1280, 4096, 8, one, one, one, one, one,
                                       ctypes.c_float(1e-6), eg.BF16, 0, one, None, None, None)
    assert st == 2 and b"scratch" in L.engram_last_error()

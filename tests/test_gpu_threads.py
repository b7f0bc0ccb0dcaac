"""The library called from several host threads at once, each on its own stream.

engram.h states that calls are thread-safe and that calls on different streams may run
concurrently; the gate and the convolution share one scratch buffer per device, handed
from stream to stream with an event.  Here four threads issue lookup + gate calls and
engram_lookup_gate calls of different shapes on their own streams, interleaved; every
result must equal the same work done alone (the kernels' sums have a fixed order, so equal
means bit-identical).
"""
import threading

import pytest
import torch

import hashed_gram_embedding_hash_amd as eg
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def test_lookup_and_gate_calls_from_four_host_threads():
    cfg = synth.CONFIGS["small"].replace(batch=1, seq=1024)
    say("four host threads, each on its own stream")
    inp = synth.device_inputs(cfg, DEV, table_rows_override=65537)
    g = torch.Generator().manual_seed(11)
    wk, wv = inp["wk"][0], inp["wv"][0]
    gq, gk = inp["gq"][0], inp["gk"][0]
    # per thread: its own token count (so the scratch is used at several sizes) and inputs
    sizes = [(1, 1024), (1, 300), (1, 777), (1, 64)]
    work = []
    for b, t in sizes:
        raw = torch.randint(0, cfg.vocab, (b, t), generator=g, dtype=torch.int32).to(DEV)
        h = torch.randn(b * t, cfg.d_model, generator=g).to(torch.bfloat16).to(DEV)
        work.append((raw, h))
    args = lambda raw: (raw, inp["map"], cfg.orders, cfg.heads, inp["mult"], inp["tables"], cfg.vocab_c)

    def one(raw, h, mem, out, alpha, stream=None):
        eg.engram_lookup(*args(raw), out=mem, stream=stream)
        eg.engram_gate_forward(mem, [h], [wk], [wv], [gq], [gk], cfg.eps, out=[out], gate_out=alpha,
                               stream=stream)

    def buffers(raw, h):
        n = raw.numel()
        return (torch.empty((n, cfg.d_mem), dtype=torch.bfloat16, device=DEV), torch.empty_like(h),
                torch.empty((1, n), dtype=torch.float32, device=DEV))

    ref = []
    for raw, h in work:
        mem, out, alpha = buffers(raw, h)
        one(raw, h, mem, out, alpha)
        torch.cuda.synchronize()
        ref.append((out.clone(), alpha.clone()))

    reps = 6
    bufs = [[buffers(raw, h) for _ in range(reps)] for raw, h in work]
    streams = [torch.cuda.Stream() for _ in work]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            raw, h = work[i]
            for r in range(reps):
                mem, out, alpha = bufs[i][r]
                if r % 2 == 0:
                    one(raw, h, mem, out, alpha, stream=streams[i])
                else:  # the one-call form: its ids live in the same scratch
                    eg.engram_lookup_gate(*args(raw), [h], [wk], [wv], [gq], [gk], cfg.eps, out=[out],
                                          gate_out=alpha, stream=streams[i])
        except Exception as exc:  # reported by the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(work))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a host thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(work)):
        for r in range(reps):
            _, out, alpha = bufs[i][r]
            assert torch.equal(out.view(torch.int16), ref[i][0].view(torch.int16)), (i, r)
            assert torch.equal(alpha.view(torch.int32), ref[i][1].view(torch.int32)), (i, r)
    say(f"  {len(work)} threads x {reps} calls each: every result bit-identical to the call alone")

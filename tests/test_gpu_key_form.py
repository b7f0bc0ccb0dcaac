"""GPU parity of the bf16 gate's memory-major key tiles (memory-side key norm).

The logit's dot product q . k = sum_f h_f gq_f (W_K diag(gk) e)_f equals
sum_c e_c (W_K'^T (gq h))_c -- "Conditional Memory via Scalable Lookup", section 2.3,
Eq. (4) with the key normalised before W_K.  engram_gate_forward computes it either over
feature-major key tiles (256 features each, contracting over d_mem) or over memory-major
ones (256 memory dimensions each, contracting over d_model), chosen by shape;
engram_debug_gate_key_form forces one.  Bar: each form against the oracle with
gpu_helpers.check_gate's bars (out rel err <= 1e-2 on the kernel's operands, alpha within
1e-4 of them and within 2e-3 of the unrounded definition, and the update out - h where
|alpha v| is comparable to |h|); the two forms within the same bars of each other; and
the automatic choice equal bit for bit to the form it documents.  Outputs start as
sentinels.
"""
import numpy as np
import pytest
import torch

import hashed_gram_embedding_hash_amd as eg
import synth
from gpu_helpers import check_gate, check_gate_tokens, host_view, oracle_memory, rel_err, sentinel_like

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def _run(form, e, hs, wks, wvs, gqs, gks, inplace=False, values=False):
    """engram_gate_forward with the key tiles forced to `form` ("feature", "memory" or "auto")."""
    M = len(hs)
    n_tok, d_model = hs[0].shape
    alpha = sentinel_like(torch.empty((M, n_tok), dtype=torch.float32, device=DEV))
    h_in = [h.clone() for h in hs]
    outs = h_in if inplace else [sentinel_like(torch.empty_like(h)) for h in hs]
    vals = [sentinel_like(torch.empty_like(h)) for h in hs] if values else None
    eg.engram_debug_gate_key_form(form)
    try:
        out = eg.engram_gate_forward(e, h_in, wks, wvs, gqs, gks, 1e-6, out=outs, gate_out=alpha, value_out=vals)
        torch.cuda.synchronize()
    finally:
        eg.engram_debug_gate_key_form("auto")
    return out, alpha, vals


@pytest.mark.parametrize("d_mem,d_model,n_tok,M,shared,inplace,values", [
    (1280, 2560, 600, 1, False, False, False),   # 5 key tiles x 40 k-steps; ragged token tile
    (320, 1024, 333, 3, False, False, True),     # ragged last key tile (64 wide); branches past the first
    (1216, 2624, 300, 3, True, True, True),      # shared W_V in place with values; ragged tiles of both kinds
    (1280, 4096, 520, 2, False, True, False),    # the large workload's widths, 64 k-steps
    (640, 1024, 300, 8, False, True, False),     # the most branches (partials of branch 7), in place
    (64, 1024, 200, 2, False, False, True),      # one key tile, 64 wide (d_mem one k-step deep)
])
def test_gate_memory_major_against_oracle(d_mem, d_model, n_tok, M, shared, inplace, values):
    """Unit-scale memory and gains != 1 (so |alpha v| ~ |h| and the update bar applies);
    both forms against the oracle, and against each other."""
    say(f"key form: d_mem {d_mem} d_model {d_model} n_tok {n_tok} branches {M} shared {shared} "
        f"in place {inplace} values {values}")
    g = torch.Generator().manual_seed(7 * d_mem + d_model + n_tok)
    e = torch.randn(n_tok, d_mem, generator=g).to(torch.bfloat16)
    hs = [torch.randn(n_tok, d_model, generator=g).to(torch.bfloat16) for _ in range(M)]
    wks = [(torch.randn(d_model, d_mem, generator=g) / d_mem ** 0.5).to(torch.bfloat16) for _ in range(M)]
    wv0 = (torch.randn(d_model, d_mem, generator=g) / d_mem ** 0.5).to(torch.bfloat16)
    wvs = [wv0] * M if shared else [wv0] + [(torch.randn(d_model, d_mem, generator=g) / d_mem ** 0.5)
                                           .to(torch.bfloat16) for _ in range(M - 1)]
    gqs = [(1 + 0.2 * torch.randn(d_model, generator=g)).to(torch.bfloat16) for _ in range(M)]
    gks = [(1 + 0.2 * torch.randn(d_mem, generator=g)).to(torch.bfloat16) for _ in range(M)]
    dv = lambda xs: [x.to(DEV) for x in xs]
    wv_d = dv(wvs) if not shared else [wv0.to(DEV)] * M
    res = {}
    for form in ("memory", "feature"):
        out, alpha, vals = _run(form, e.to(DEV), dv(hs), dv(wks), wv_d, dv(gqs), dv(gks), inplace, values)
        res[form] = (out, alpha, vals)
        for m in range(M):
            check_gate(f"{form}-major, branch {m}", out[m].float().cpu().numpy(), alpha[m].cpu().numpy(),
                       host_view(e), host_view(hs[m]), host_view(wks[m]), host_view(wvs[m]), host_view(gqs[m]),
                       host_view(gks[m]), 1e-6, update=True,
                       vals=vals[m].float().cpu().numpy() if values else None, say=say)
    (om, am, _), (of, af, _) = res["memory"], res["feature"]
    da = float((am - af).abs().max())
    dout = max(rel_err(om[m].float().cpu().numpy(), of[m].float().cpu().numpy()) for m in range(M))
    say(f"  memory-major vs feature-major: alpha max abs diff {da:.2e}, out rel diff {dout:.2e}")
    assert da <= 1e-4 and dout <= 1e-2


def test_gate_key_form_auto_choice_and_oracle_at_scale():
    """The automatic choice: memory-major with at least one key tile per compute unit (here
    52 token tiles x 2 or 3 branches x 5 key tiles on the small workload's widths),
    feature-major for a decode step's 256 tokens (5 key tiles); each bit-identical to the
    form forced, and the memory-major run against the oracle on sampled tokens."""
    cfg = synth.CONFIGS["small"].replace(n_branch=2)
    n_tok = 52 * 256
    say(f"key form auto: {n_tok} tokens, d_mem {cfg.d_mem}, d_model {cfg.d_model}, 2 branches")
    rng = np.random.default_rng(91)
    idx = rng.integers(0, cfg.rows, (n_tok, cfg.n_tables)).astype(np.int32)
    e_o = oracle_memory(cfg, idx)
    tokens = rng.choice(1 << 20, n_tok, replace=False).astype(np.int64)
    e_d = torch.from_numpy(e_o.view(np.int16)).to(DEV).view(torch.bfloat16)
    hs = [synth.hidden_rows(cfg, m, torch.from_numpy(tokens)).to(DEV) for m in range(2)]
    ws = [synth.weights(cfg, m, DEV) for m in range(2)]
    gs = [synth.gains(cfg, m, DEV) for m in range(2)]
    args = ([w[0] for w in ws], [w[1] for w in ws], [x[0] for x in gs], [x[1] for x in gs])
    runs = {f: _run(f, e_d, hs, *args) for f in ("auto", "memory", "feature")}
    same = lambda a, b: (torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)) and
                         all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(a[0], b[0])))
    assert same(runs["auto"], runs["memory"]), "auto should have chosen memory-major tiles"
    assert not torch.equal(runs["memory"][1], runs["feature"][1]), "the two forms should round differently"
    sample = np.unique(np.concatenate([np.arange(4), rng.choice(n_tok, 60, replace=False), [n_tok - 1]]))
    for m in range(2):
        check_gate_tokens(f"memory-major branch {m}", cfg, m, runs["memory"][0][m][sample].float().cpu().numpy(),
                          runs["memory"][1][m][sample].cpu().numpy(), e_o[sample], tokens[sample], say=say)
    # a decode step: one token tile, 5 key tiles per branch, far below two per compute unit
    k = 256
    dec = {f: _run(f, e_d[:k], [h[:k].contiguous() for h in hs], *args) for f in ("auto", "feature")}
    assert same(dec["auto"], dec["feature"]), "auto should have chosen feature-major tiles"
    # three branches (the third reusing the first's inputs)
    a3 = tuple(x + x[:1] for x in args)
    h3 = hs + hs[:1]
    tri = {f: _run(f, e_d, h3, *a3) for f in ("auto", "feature", "memory")}
    assert same(tri["auto"], tri["memory"]), "auto should have chosen memory-major tiles for 3 branches"
    assert not torch.equal(tri["memory"][1], tri["feature"][1])
    say("  auto: memory-major at 52 token tiles (2 and 3 branches), feature-major at one token tile")

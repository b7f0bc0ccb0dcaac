"""GPU parity of engram_lookup_gate: the lookup and the gate in one pass, the gate's
matrix-core kernel hashing each token's n-grams and loading the table rows into its
operand tiles itself.

Bar: every output (the updated hidden states, the gates, the gated values, the canonical
ids and the error count) bit-identical to engram_lookup followed by engram_gate_forward
with feature-major key tiles (the fused call's form; set for every test here),
whose parity with the oracle the other GPU tests establish; and, independently, the gate
against the oracle (gpu_helpers.check_gate's bars) on memory vectors the oracle builds
from the same raw ids.  The cases span one to 25 k-steps, table rows of 8 to 25 16-byte
chunks (a k-step then covers up to two tables), orders 1 to 4, ragged token and feature
tiles, windows, out-of-vocabulary ids, several branches, a shared W_V and both key norms.
"""
import numpy as np
import pytest
import torch

import hashed_gram_embedding_hash_amd as eg
import oracle
import synth
from gpu_helpers import check_gate, host_view, sentinel_like

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def feature_major_key_tiles():
    """The gathering gate's key tiles are feature-major; engram_gate_forward chooses
    memory-major ones for some of these shapes (the small and large workloads), whose
    logits round differently.  The two-call references here take the same form as the
    fused call, so the comparison is bit for bit; the memory-major form has its own
    oracle tests (test_gpu_key_form.py)."""
    eg.engram_debug_gate_key_form("feature")
    yield
    eg.engram_debug_gate_key_form("auto")


MEM, PROJ = eg.KEY_NORM_MEMORY, eg.KEY_NORM_PROJECTED


def say(*a):
    print(*a, flush=True)


def _inputs(orders, heads, w, rows, batch, seq, d_model, n_branch, shared, key_norm, seed, table_std=0.5):
    """Seeded inputs of one case (tables of std 0.5, so that alpha * v is not small next to h;
    the gated values, checked on their own where a case asks for them, bound the update)."""
    g = torch.Generator().manual_seed(seed)
    vocab, vocab_c = 3000, 2200
    nt = len(orders) * heads
    d_mem = nt * w
    raw = torch.randint(0, vocab, (batch, seq), generator=g, dtype=torch.int32)
    bad = torch.rand((batch, seq), generator=g) < 0.01  # out-of-vocabulary raw ids
    raw[bad] = vocab + 7
    cmap = torch.randint(0, vocab_c, (vocab,), generator=g, dtype=torch.int32)
    mult = (torch.randint(0, 2 ** 62, (len(orders), heads, max(orders)), generator=g, dtype=torch.int64) * 2 + 1)
    tables = [(torch.randn((rows + b, w), generator=g) * table_std).to(torch.bfloat16) for b in range(nt)]
    n_tok = batch * seq
    h = [torch.randn((n_tok, d_model), generator=g).to(torch.bfloat16) for _ in range(n_branch)]
    wk = [(torch.randn((d_model, d_mem), generator=g) / d_mem ** 0.5).to(torch.bfloat16) for _ in range(n_branch)]
    wv0 = [(torch.randn((d_model, d_mem), generator=g) / d_mem ** 0.5).to(torch.bfloat16) for _ in range(n_branch)]
    gk_len = d_mem if key_norm == MEM else d_model
    gq = [(1 + 0.2 * torch.randn(d_model, generator=g)).to(torch.bfloat16) for _ in range(n_branch)]
    gk = [(1 + 0.2 * torch.randn(gk_len, generator=g)).to(torch.bfloat16) for _ in range(n_branch)]
    return dict(raw=raw, cmap=cmap, mult=mult.numpy().view(np.uint64), tables=tables, h=h, wk=wk, wv0=wv0, gq=gq,
                gk=gk, vocab_c=vocab_c)


def _dev(x):
    return [t.to(DEV) for t in x] if isinstance(x, list) else x.to(DEV)


CASES = [
    # orders, heads, w, rows, batch, seq, t_begin, d_model, n_branch, shared, key_norm, values
    ((2, 3), 8, 80, 4099, 3, 700, 0, 640, 1, False, MEM, False),      # 20 k-steps, ragged tiles
    ((2,), 2, 64, 1021, 2, 300, 5, 256, 3, True, MEM, True),          # 2 k-steps, shared W_V, window
    ((1, 2, 3, 4), 2, 72, 2003, 2, 257, 0, 320, 2, False, PROJ, True),  # 9 chunks a row, orders 1-4
    ((2,), 1, 64, 509, 1, 1, 0, 64, 1, False, MEM, False),            # one token, one k-step
    ((1, 2, 3), 1, 64, 509, 2, 129, 3, 128, 1, False, MEM, True),     # 3 k-steps
    ((2, 3), 2, 64, 2017, 1, 515, 0, 96, 2, False, MEM, False),       # 4 k-steps (one main-loop step)
    ((2, 3), 4, 128, 8191, 2, 1000, 0, 512, 2, True, PROJ, False),    # 16 chunks a row, shared, projected
    ((3,), 8, 200, 3001, 1, 513, 0, 256, 1, False, MEM, False),       # 25 chunks a row, 25 k-steps
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_lookup_gate_bit_identical_to_lookup_then_gate(case):
    orders, heads, w, rows, batch, ld, t_begin, d_model, nb, shared, key_norm, values = case
    t_count = ld - t_begin
    say(f"lookup_gate case: orders {orders} x {heads} heads, w {w}, {batch} x {t_count} tokens (t_begin "
        f"{t_begin}), d_model {d_model}, {nb} branches, shared W_V {shared}, key_norm {key_norm}")
    inp = _inputs(orders, heads, w, rows, batch, ld, d_model, nb, shared, key_norm, seed=CASES.index(case))
    raw, cmap, tables = _dev(inp["raw"]), _dev(inp["cmap"]), _dev(inp["tables"])
    n_tok = batch * t_count
    h = [x[: n_tok].contiguous() for x in _dev(inp["h"])]
    wk, gq, gk = _dev(inp["wk"]), _dev(inp["gq"]), _dev(inp["gk"])
    wv = [_dev(inp["wv0"][0])] * nb if shared else _dev(inp["wv0"])
    pad = inp["vocab_c"]

    def outputs():
        return dict(out=[sentinel_like(torch.empty_like(x)) for x in h],
                    alpha=sentinel_like(torch.empty((nb, n_tok), dtype=torch.float32, device=DEV)),
                    vals=[sentinel_like(torch.empty_like(x)) for x in h] if values else None,
                    ids=sentinel_like(torch.empty((batch, ld), dtype=torch.int32, device=DEV)),
                    err=torch.zeros(1, dtype=torch.int32, device=DEV))

    ref = outputs()
    mem = eg.engram_lookup(raw, cmap, orders, heads, inp["mult"], tables, pad, t_begin=t_begin, t_count=t_count,
                           ids_out=ref["ids"], err_count=ref["err"])
    eg.engram_gate_forward(mem, h, wk, wv, gq, gk, 1e-6, out=ref["out"], gate_out=ref["alpha"],
                           value_out=ref["vals"], key_norm=key_norm)
    got = outputs()
    eg.engram_lookup_gate(raw, cmap, orders, heads, inp["mult"], tables, pad, h, wk, wv, gq, gk, 1e-6,
                          t_begin=t_begin, t_count=t_count, out=got["out"], gate_out=got["alpha"],
                          value_out=got["vals"], key_norm=key_norm, ids_out=got["ids"], err_count=got["err"])
    torch.cuda.synchronize()
    say(f"  {int(got['err'].item())} out-of-vocabulary ids")
    assert int(got["err"].item()) == int(ref["err"].item())
    assert int(ref["err"].item()) > 0 or n_tok < 50
    # the window's ids are written; positions before t_begin keep their sentinel in both
    assert torch.equal(got["ids"], ref["ids"])
    assert torch.equal(got["alpha"].view(torch.int32), ref["alpha"].view(torch.int32))
    assert not torch.isnan(got["alpha"]).any()
    for m in range(nb):
        assert torch.equal(got["out"][m].view(torch.int16), ref["out"][m].view(torch.int16)), f"branch {m}"
        if values:
            assert torch.equal(got["vals"][m].view(torch.int16), ref["vals"][m].view(torch.int16)), f"values {m}"
    say("  bit-identical to engram_lookup + engram_gate_forward")

    # independently: the oracle's memory vectors from the same raw ids, then its gate
    if n_tok <= 2100:
        raw_h, cmap_h = inp["raw"].numpy(), inp["cmap"].numpy()
        ids_o, _ = oracle.compress(raw_h, cmap_h)
        rows_u32 = np.array([t.shape[0] for t in inp["tables"]], np.uint32)
        idx_o = oracle.hash_ids(ids_o, orders, heads, inp["mult"], rows_u32, pad, t_begin=t_begin, t_count=t_count)
        e_o = oracle.gather(idx_o, [host_view(t) for t in inp["tables"]])
        for m in range(nb):
            check_gate(f"branch {m}", got["out"][m].float().cpu().numpy(), got["alpha"][m].cpu().numpy(), e_o,
                       host_view(h[m]), host_view(inp["wk"][m]), host_view(inp["wv0"][0 if shared else m]),
                       host_view(inp["gq"][m]), host_view(inp["gk"][m]), 1e-6, key_norm=key_norm,
                       vals=got["vals"][m].float().cpu().numpy() if values else None, say=say)


def test_lookup_gate_small_config_against_oracle_sampled():
    """The small workload (16 tables x 1,000,003 rows, 16,384 tokens, d_model 2560): every
    output bit-identical to the two calls, and sampled tokens against the oracle."""
    from gpu_helpers import check_gate_tokens, oracle_ids_idx, oracle_memory, sample_tokens
    from hashed_gram_embedding_hash_amd.pipeline import EngramLayer
    cfg = synth.CONFIGS["small"]
    say(f"lookup_gate on the small workload: {cfg.tokens} tokens")
    inp = synth.device_inputs(cfg, DEV)
    layer = EngramLayer(inp["map"], cfg.orders, cfg.heads, inp["mult"], inp["tables"], inp["wk"], inp["wv"],
                        inp["gq"], inp["gk"], cfg.eps, pad_id=cfg.vocab_c)
    ref = [torch.empty_like(x) for x in inp["h"]]
    ref_a = torch.empty((cfg.n_branch, cfg.tokens), dtype=torch.float32, device=DEV)
    layer(inp["raw"], inp["h"], out=ref, gate_out=ref_a)
    got = [sentinel_like(torch.empty_like(x)) for x in inp["h"]]
    got_a = sentinel_like(torch.empty_like(ref_a))
    layer(inp["raw"], inp["h"], out=got, gate_out=got_a, fused=True)   # the layer's one-call form
    torch.cuda.synchronize()
    assert torch.equal(got_a.view(torch.int32), ref_a.view(torch.int32))
    for m in range(cfg.n_branch):
        assert torch.equal(got[m].view(torch.int16), ref[m].view(torch.int16))
    say("  bit-identical to the two calls")
    raw_h = inp["raw"].cpu().numpy()
    _, idx = oracle_ids_idx(cfg, raw_h)
    tokens = sample_tokens(cfg, 96, seed=3)
    e = oracle_memory(cfg, idx[tokens])
    for m in range(cfg.n_branch):
        check_gate_tokens(f"branch {m}", cfg, m, got[m][tokens].float().cpu().numpy(), got_a[m][tokens].cpu().numpy(),
                          e, tokens, say=say)


def test_lookup_gate_large_workload_bit_identical():
    """The large workload (26 GB of tables, 262,144 tokens, d_model 4096, two branches) in
    the benchmark's launch configuration: every output bit-identical to the two calls
    (feature-major key tiles, as throughout this module)."""
    from hashed_gram_embedding_hash_amd.pipeline import EngramLayer
    cfg = synth.CONFIGS["large"]
    say(f"lookup_gate on the large workload: {cfg.tokens} tokens, {cfg.n_tables} x {cfg.rows} rows")
    inp = synth.device_inputs(cfg, DEV)
    layer = EngramLayer(inp["map"], cfg.orders, cfg.heads, inp["mult"], inp["tables"], inp["wk"], inp["wv"],
                        inp["gq"], inp["gk"], cfg.eps, pad_id=cfg.vocab_c)
    ref = [torch.empty_like(x) for x in inp["h"]]
    ref_a = torch.empty((cfg.n_branch, cfg.tokens), dtype=torch.float32, device=DEV)
    layer(inp["raw"], inp["h"], out=ref, gate_out=ref_a)
    torch.cuda.synchronize()
    say("  two-call pass done (feature-major key tiles)")
    got = [sentinel_like(torch.empty_like(x)) for x in inp["h"]]
    got_a = sentinel_like(torch.empty_like(ref_a))
    eg.engram_lookup_gate(inp["raw"], inp["map"], cfg.orders, cfg.heads, inp["mult"], inp["tables"], cfg.vocab_c,
                          inp["h"], inp["wk"], inp["wv"], inp["gq"], inp["gk"], cfg.eps, out=got, gate_out=got_a)
    torch.cuda.synchronize()
    say("  fused pass done")
    assert torch.equal(got_a.view(torch.int32), ref_a.view(torch.int32))
    for m in range(cfg.n_branch):
        assert torch.equal(got[m].view(torch.int16), ref[m].view(torch.int16)), f"branch {m}"
    say("  bit-identical to the two calls")


def test_lookup_gate_graph_replay_equals_eager():
    """engram_lookup_gate (three kernels: ids, key-weight fold, gathering gate) captured in a
    HIP graph: every replay, with eager calls on other ids in between (they share the
    library's scratch), reproduces the eager result bit for bit, gates and gated values
    included."""
    orders, heads, w, rows, batch, ld, d_model, nb = (2, 3), 4, 80, 4099, 2, 600, 512, 2
    say("graph replay of engram_lookup_gate")
    inp = _inputs(orders, heads, w, rows, batch, ld, d_model, nb, False, MEM, seed=77)
    raw, cmap, tables = _dev(inp["raw"]), _dev(inp["cmap"]), _dev(inp["tables"])
    h, wk, wv = _dev(inp["h"]), _dev(inp["wk"]), _dev(inp["wv0"])
    gq, gk = _dev(inp["gq"]), _dev(inp["gk"])
    pad = inp["vocab_c"]
    n_tok = batch * ld

    def call(ids, out, alpha, vals):
        eg.engram_lookup_gate(ids, cmap, orders, heads, inp["mult"], tables, pad, h, wk, wv, gq, gk, 1e-6,
                              out=out, gate_out=alpha, value_out=vals)

    def bufs():
        return ([torch.empty_like(x) for x in h], torch.empty((nb, n_tok), dtype=torch.float32, device=DEV),
                [torch.empty_like(x) for x in h])

    want = bufs()
    call(raw, *want)
    raw2 = torch.roll(raw, 5, dims=1).contiguous()
    other = bufs()
    call(raw2, *other)
    torch.cuda.synchronize()
    assert not torch.equal(other[0][0], want[0][0])
    got = bufs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(raw, *got)                    # the scratch is sized on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(raw, *got)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in got[0] + got[2]:
            sentinel_like(x)
        sentinel_like(got[1])
        eager = bufs()
        call(raw2, *eager)                 # eager work on the same scratch in between
        torch.cuda.synchronize()
        assert torch.equal(eager[0][0].view(torch.int16), other[0][0].view(torch.int16)), rep
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got[1].view(torch.int32), want[1].view(torch.int32)), rep
        for m in range(nb):
            assert torch.equal(got[0][m].view(torch.int16), want[0][m].view(torch.int16)), (rep, m)
            assert torch.equal(got[2][m].view(torch.int16), want[2][m].view(torch.int16)), (rep, m)
    say("  three replays bit-identical to the eager call")


def test_lookup_gate_no_map_most_tables_and_branches():
    """Canonical ids passed straight in (no compression map), the most tables a call takes
    (32: orders 1-4 x 8 heads, 64-value rows, d_mem 2048) and the most branches (8, in place),
    against the two calls bit for bit."""
    orders, heads, w, rows, batch, ld, d_model, nb = (1, 2, 3, 4), 8, 64, 997, 3, 111, 64, 8
    say("lookup_gate: no map, 32 tables, 8 branches in place")
    inp = _inputs(orders, heads, w, rows, batch, ld, d_model, nb, False, MEM, seed=91)
    raw = (inp["raw"] % inp["vocab_c"]).to(DEV)           # canonical ids already
    tables = _dev(inp["tables"])
    wk, wv, gq, gk = _dev(inp["wk"]), _dev(inp["wv0"]), _dev(inp["gq"]), _dev(inp["gk"])
    pad = inp["vocab_c"]
    h_ref = _dev(inp["h"])
    h_got = [x.clone() for x in h_ref]
    a_ref = torch.empty((nb, batch * ld), dtype=torch.float32, device=DEV)
    a_got = sentinel_like(torch.empty_like(a_ref))
    mem = eg.engram_lookup(raw, None, orders, heads, inp["mult"], tables, pad)
    eg.engram_gate_forward(mem, h_ref, wk, wv, gq, gk, 1e-6, out=h_ref, gate_out=a_ref)
    eg.engram_lookup_gate(raw, None, orders, heads, inp["mult"], tables, pad, h_got, wk, wv, gq, gk, 1e-6,
                          out=h_got, gate_out=a_got)
    torch.cuda.synchronize()
    assert torch.equal(a_got.view(torch.int32), a_ref.view(torch.int32))
    for m in range(nb):
        assert torch.equal(h_got[m].view(torch.int16), h_ref[m].view(torch.int16)), m
    say("  bit-identical")

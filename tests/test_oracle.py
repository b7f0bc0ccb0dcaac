"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test ties the oracle to something other than its own code: the printed or
hand-derived values under tests/golden/, closed forms, special cases and
invariants of "Conditional Memory via Scalable Lookup" (section 2.2 Eq. (1)-(2),
section 2.3 Eq. (3)-(4)).  All run on the CPU.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden

MASK64 = (1 << 64) - 1


def bf16_bits(x):
    """Round float values to bfloat16 (RNE, via torch) and return the raw uint16 bits."""
    import torch
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# input generator pins (SplitMix64 draws the hash multipliers)
# ---------------------------------------------------------------------------
def test_splitmix64_published_vector():
    rows = read_golden("splitmix64.txt")
    assert rows[0][0] == "seed"
    seed = int(rows[0][1])
    want = [int(r[0]) for r in rows[1:]]
    assert synth.splitmix64(seed, len(want)) == want


def test_counter_generator_torch_equals_numpy():
    import torch
    rows = np.array([0, 1, 2, 4092, 999_999, 10_156_252, 78_125_040, (1 << 40) + 3])
    for stream in (0, 7, synth.STREAM_HIDDEN + 3):
        a = synth.counter_normal(11, stream, torch.as_tensor(rows), 80, 0.02)
        b = synth.counter_normal_numpy(11, stream, rows, 80, 0.02)
        assert np.array_equal(a.numpy(), b)
    big = synth.counter_normal(3, 1, torch.arange(20000), 64, 1.0).numpy().ravel()
    assert abs(big.mean()) < 0.01 and abs(big.std() - 1.0) < 0.01


def test_configs_sizes():
    c = synth.CONFIGS
    assert c["tiny"].d_mem == 128 and c["tiny"].n_tables == 4
    assert c["small"].d_mem == 1280 and c["small"].n_tables == 16
    assert synth.is_prime(c["small"].rows) and synth.is_prime(c["large"].rows)
    assert c["large"].rows == 10_156_253            # next prime >= 13e9 / (16 * 80)
    assert synth.ROWS_OFFLOAD == 78_125_041          # next prime >= 1e11 / 1280
    # 13e9 parameters over 16 tables, 100e9 for the offloaded table
    assert abs(c["large"].rows * 16 * 80 - 13e9) / 13e9 < 1e-5
    assert abs(synth.ROWS_OFFLOAD * 1280 - 1e11) / 1e11 < 1e-5


def test_compression_map_is_surjective():
    cfg = synth.CONFIGS["tiny"]
    m = synth.comp_map(cfg)
    assert m.shape == (cfg.vocab,) and m.min() == 0 and m.max() == cfg.vocab_c - 1
    assert len(np.unique(m)) == cfg.vocab_c


# ---------------------------------------------------------------------------
# compress (section 2.2, tokenizer compression)
# ---------------------------------------------------------------------------
def test_compress_is_the_lookup_and_flags_bad_ids():
    cmap = np.array([3, 0, 3, 1, 2], dtype=np.int32)
    raw = np.array([[0, 1, 2, 3, 4, 5, -1, 2]], dtype=np.int32)
    out, bad = oracle.compress(raw, cmap)
    assert out.tolist() == [[3, 0, 3, 1, 2, -1, -1, 3]]
    assert bad == 2


def test_compress_image_on_config():
    cfg = synth.CONFIGS["small"]
    raw = synth.raw_ids(cfg)
    cmap = synth.comp_map(cfg)
    out, bad = oracle.compress(raw, cmap)
    assert bad == 0 and out.min() >= 0 and out.max() < cfg.vocab_c
    # the value at each position is the map entry: spot-check by direct indexing
    i = np.random.default_rng(0).integers(0, raw.size, 100)
    assert np.array_equal(out.ravel()[i], cmap[raw.ravel()[i]])


# ---------------------------------------------------------------------------
# hash (section 2.2, Eq. (1))
# ---------------------------------------------------------------------------
def _golden_hash():
    mult = {}
    cases = []
    for r in read_golden("hash_worked.txt"):
        if r[0] == "mult":
            mult[(int(r[1]), int(r[2]))] = [int(x, 16) for x in r[3:]]
        else:
            cases.append(dict(name=r[1], n=int(r[2]), k=int(r[3]), gram=r[4].split(","), z=int(r[6])))
    return mult, cases


def test_hash_worked_values():
    mult_g, cases = _golden_hash()
    orders, heads, pad, M = (2, 3), 2, 770, 4093
    mult = synth.hash_multipliers(1, orders, heads)
    for (n, k), cs in mult_g.items():
        assert [int(x) for x in mult[orders.index(n), k, :n]] == cs
    rows = np.full(4, M, dtype=np.uint32)
    for c in cases:
        gram = c["gram"]
        if gram[0] == "pad":
            ids = np.array([[int(x) for x in gram[1:]]], dtype=np.int32)  # t = 0: older slot is padding
        else:
            ids = np.array([[int(x) for x in gram]], dtype=np.int32)
        idx = oracle.hash_ids(ids, orders, heads, mult, rows, pad)
        col = orders.index(c["n"]) * heads + c["k"]
        assert idx[-1, col] == c["z"], c["name"]


def test_hash_closed_forms_single_nonzero_id():
    """A gram whose only nonzero id is 1 at position j hashes to c[j] mod M; all-zero grams to 0."""
    orders, heads = (2, 3), 3
    mult = synth.hash_multipliers(99, orders, heads)
    rows = np.array([4093, 65521, 1_000_003, 7919, 104_729, 2_147_483_647], dtype=np.uint32)
    ids = np.array([[1, 0, 0, 0]], dtype=np.int32)     # t=0: (pad, 1); t=1: (1, 0); t=2: (1,0,0)
    idx = oracle.hash_ids(ids, orders, heads, mult, rows, pad_id=0)
    for k in range(heads):
        # order 2 at t=0: newest id 1 at j=0 (pad = 0) ; t=1: id 1 at j=1
        assert idx[0, k] == int(mult[0, k, 0]) % int(rows[k])
        assert idx[1, k] == int(mult[0, k, 1]) % int(rows[k])
        assert idx[3, k] == 0
        # order 3 at t=2: id 1 at j=2 ; t=3: all zero
        assert idx[2, heads + k] == int(mult[1, k, 2]) % int(rows[heads + k])
        assert idx[3, heads + k] == 0


def test_hash_power_of_two_id_is_a_shift():
    """x = 2^s at j = 0 with the other slot 0: h = (c0 << s) mod 2^64."""
    orders, heads = (2,), 1
    mult = synth.hash_multipliers(5, orders, heads)
    M = 2_147_483_647
    for s in (0, 1, 13, 30):
        ids = np.array([[0, 1 << s]], dtype=np.int32)
        idx = oracle.hash_ids(ids, orders, heads, mult, np.array([M], np.uint32), pad_id=0)
        assert idx[1, 0] == ((int(mult[0, 0, 0]) << s) & MASK64) % M


def test_hash_same_gram_same_slot_everywhere():
    """Determinism: an n-gram maps to the same slot at every position and in every sequence."""
    cfg = synth.CONFIGS["tiny"]
    rng = np.random.default_rng(1)
    ids = rng.integers(0, cfg.vocab_c, (4, 300)).astype(np.int32)
    ids[:, 50:53] = [11, 22, 33]
    ids[2, 200:203] = [11, 22, 33]
    ids[3, 0:3] = [11, 22, 33]
    mult = synth.multipliers(cfg)
    idx = oracle.hash_ids(ids, cfg.orders, cfg.heads, mult, synth.table_rows_u32(cfg), cfg.vocab_c)
    idx = idx.reshape(4, 300, -1)
    ref = idx[0, 52]
    for b in range(4):
        assert np.array_equal(idx[b, 52], ref)
    assert np.array_equal(idx[2, 202], ref) and np.array_equal(idx[3, 2], ref)
    # bigram part only needs the last two ids
    ids2 = ids.copy()
    ids2[1, 50] = 7
    idx2 = oracle.hash_ids(ids2, cfg.orders, cfg.heads, mult, synth.table_rows_u32(cfg), cfg.vocab_c)
    idx2 = idx2.reshape(4, 300, -1)
    assert np.array_equal(idx2[1, 52, :cfg.heads], ref[:cfg.heads])


def test_hash_range_and_uniformity():
    orders, heads = (2, 3), 4
    mult = synth.hash_multipliers(7, orders, heads)
    M = 1009
    rows = np.full(len(orders) * heads, M, dtype=np.uint32)
    rng = np.random.default_rng(2)
    ids = rng.integers(0, 99_546, (8, 40_000)).astype(np.int32)
    idx = oracle.hash_ids(ids, orders, heads, mult, rows, pad_id=99_546)
    assert idx.min() >= 0 and idx.max() < M
    # chi-square goodness of fit to uniform, per table: df = M-1, mean M-1, sd sqrt(2(M-1))
    for col in range(idx.shape[1]):
        cnt = np.bincount(idx[:, col], minlength=M)
        exp = idx.shape[0] / M
        chi2 = ((cnt - exp) ** 2 / exp).sum()
        assert abs(chi2 - (M - 1)) < 6 * math.sqrt(2 * (M - 1)), (col, chi2)


def test_hash_order_matters_and_heads_differ():
    mult_g, cases = _golden_hash()
    z = {c["name"]: c["z"] for c in cases}
    assert z["bigram_5_7"] != z["bigram_7_5"]
    cfg = synth.CONFIGS["tiny"]
    ids = np.random.default_rng(3).integers(0, 770, (1, 2000)).astype(np.int32)
    idx = oracle.hash_ids(ids, cfg.orders, cfg.heads, synth.multipliers(cfg), synth.table_rows_u32(cfg), 770)
    # distinct heads of one order are different functions
    assert (idx[:, 0] != idx[:, 1]).mean() > 0.99


def test_hash_window_equals_full():
    """Hashing a window of positions equals the same rows of a full-sequence hash."""
    cfg = synth.CONFIGS["tiny"]
    ids = np.random.default_rng(4).integers(0, 770, (3, 100)).astype(np.int32)
    args = (cfg.orders, cfg.heads, synth.multipliers(cfg), synth.table_rows_u32(cfg), 770)
    full = oracle.hash_ids(ids, *args).reshape(3, 100, -1)
    part = oracle.hash_ids(ids, *args, t_begin=40, t_count=7).reshape(3, 7, -1)
    assert np.array_equal(full[:, 40:47], part)


# ---------------------------------------------------------------------------
# gather + concatenation (section 2.2, Eq. (2))
# ---------------------------------------------------------------------------
def test_gather_concat_order_with_coded_tables():
    """Row r of table b holds the code (b, r, c); the output block b of token t must hold (b, idx[t,b], c)."""
    n_tables, rows, w = 6, 37, 8
    tables = [np.array([[b * 100_000 + r * 100 + c for c in range(w)] for r in range(rows)], np.float32)
              for b in range(n_tables)]
    idx = np.random.default_rng(5).integers(0, rows, (50, n_tables)).astype(np.int32)
    out = oracle.gather(idx, tables)
    for t in range(50):
        for b in range(n_tables):
            assert out[t, b * w:(b + 1) * w].tolist() == [b * 100_000 + idx[t, b] * 100 + c for c in range(w)]


def test_gather_is_bitwise_for_bf16_bits():
    tables = [np.random.default_rng(b).integers(0, 1 << 16, (11, 80)).astype(np.uint16) for b in range(16)]
    idx = np.random.default_rng(9).integers(0, 11, (30, 16)).astype(np.int32)
    out = oracle.gather(idx, tables)
    for t in range(30):
        for b in range(16):
            assert np.array_equal(out[t, b * 80:(b + 1) * 80], tables[b][idx[t, b]])


# ---------------------------------------------------------------------------
# gate (section 2.3, Eq. (3)-(4), gated value, residual)
# ---------------------------------------------------------------------------
def _golden_gate():
    ex, cur = {}, None
    for r in read_golden("gate_micro.txt"):
        if r[0] == "example":
            cur = ex.setdefault(r[1], {})
        else:
            cur[r[0]] = [float(x) for x in r[1:]]
    return ex


@pytest.mark.parametrize("name", ["A", "B", "C", "D", "E"])
def test_gate_hand_examples(name):
    """Hand-worked gate values (tests/golden/gate_micro.txt).  Examples marked fp8 have
    operands that E4M3 represents exactly with the per-row scales, so the FP8 gate must
    reproduce them too: D pins gq on the paper's key placement, E pins both gains with
    the key normalised before W_K (a gain applied twice or left out of the key moves the
    logit, see the fixture)."""
    g = _golden_gate()[name]
    dm, dmod = int(g["d_mem"][0]), int(g["d_model"][0])
    key_norm = int(g.get("key_norm", [0])[0])
    f = lambda k, shape: np.array(g[k], np.float32).reshape(shape)
    args = (f("e", (1, dm)), f("h", (1, dmod)), f("wk", (dmod, dm)), f("wv", (dmod, dm)),
            f("gq", (dmod,)), f("gk", (dm,) if key_norm == 0 else (dmod,)), g["eps"][0], oracle.F32)
    gates = [oracle.gate] + ([oracle.gate_fp8] if int(g.get("fp8", [0])[0]) else [])
    for gate in gates:
        out, alpha = gate(*args, key_norm=key_norm)
        # the inputs are not all exactly representable in float32; 1e-6 covers that rounding
        assert abs(alpha[0] - 1 / (1 + math.exp(-g["logit"][0]))) < 1e-6, gate
        assert abs(alpha[0] - g["alpha"][0]) < 1e-6, gate
        np.testing.assert_allclose(out[0], g["out"], rtol=0, atol=2e-6)


def _rand_gate(rng, n, dm, dmod, dtype=np.float32):
    e = (0.02 * rng.standard_normal((n, dm))).astype(dtype)
    h = rng.standard_normal((n, dmod)).astype(dtype)
    wk = (rng.standard_normal((dmod, dm)) / math.sqrt(dm)).astype(dtype)
    wv = (rng.standard_normal((dmod, dm)) / math.sqrt(dm)).astype(dtype)
    gq = (1 + 0.1 * rng.standard_normal(dmod)).astype(dtype)
    gk = (1 + 0.1 * rng.standard_normal(dm)).astype(dtype)
    return e, h, wk, wv, gq, gk


def test_gate_zero_value_projection_is_identity():
    e, h, wk, wv, gq, gk = _rand_gate(np.random.default_rng(0), 5, 24, 16)
    out, _ = oracle.gate(e, h, wk, np.zeros_like(wv), gq, gk, 1e-6, oracle.F32)
    assert np.array_equal(out, h.astype(np.float64))


def test_gate_zero_key_projection_gives_half():
    e, h, wk, wv, gq, gk = _rand_gate(np.random.default_rng(1), 5, 24, 16)
    out, alpha = oracle.gate(e, h, np.zeros_like(wk), wv, gq, gk, 1e-6, oracle.F32)
    assert np.all(alpha == 0.5)
    v = e.astype(np.float64) @ wv.astype(np.float64).T
    np.testing.assert_allclose(out, h + 0.5 * v, rtol=0, atol=1e-12)


def test_gate_saturates_to_residual_and_full_value():
    """h along -k with a huge query gain closes the gate (out == h); along +k opens it (out = h + v)."""
    rng = np.random.default_rng(2)
    d = 16
    e, _, wk, wv, _, gk = _rand_gate(rng, 1, d, d)
    gk[:] = 1
    en = e[0].astype(np.float64) / math.sqrt((e[0].astype(np.float64) ** 2).mean() + 1e-6)
    k = wk.astype(np.float64) @ en
    gq = np.full(d, 1e4, np.float32)
    for sign, want in ((-1, 0.0), (1, 1.0)):
        h = (sign * k).astype(np.float32)[None, :]
        out, alpha = oracle.gate(e, h, wk, wv, gq, gk, 1e-6, oracle.F32)
        assert alpha[0] == want
        v = wv.astype(np.float64) @ e[0].astype(np.float64)
        if want == 0.0:
            assert np.array_equal(out[0], h[0].astype(np.float64))
        else:
            np.testing.assert_allclose(out[0], h[0] + v, rtol=0, atol=1e-12)


def test_gate_identity_key_is_scaled_cosine():
    """W_K = I, unit gains, eps = 0: logit = sqrt(d) * cos(h, e) (RMSNorm is L2 normalisation times sqrt(d))."""
    rng = np.random.default_rng(3)
    d = 32
    e, h, _, wv, _, _ = _rand_gate(rng, 4, d, d)
    ones = np.ones(d, np.float32)
    _, alpha = oracle.gate(e, h, np.eye(d, dtype=np.float32), wv, ones, ones, 0.0, oracle.F32)
    for t in range(4):
        a, b = h[t].astype(np.float64), e[t].astype(np.float64)
        cos = a.dot(b) / (np.linalg.norm(a) * np.linalg.norm(b))
        assert abs(alpha[t] - 1 / (1 + math.exp(-math.sqrt(d) * cos))) < 1e-12


def test_gate_memory_scale_invariance():
    """RMSNorm makes alpha invariant to scaling e (eps = 0); out - h scales with e."""
    rng = np.random.default_rng(4)
    e, h, wk, wv, gq, gk = _rand_gate(rng, 6, 20, 12)
    o1, a1 = oracle.gate(e, h, wk, wv, gq, gk, 0.0, oracle.F32)
    o2, a2 = oracle.gate(e * np.float32(4.0), h, wk, wv, gq, gk, 0.0, oracle.F32)
    np.testing.assert_allclose(a1, a2, rtol=1e-13, atol=0)
    np.testing.assert_allclose(o2 - h, 4.0 * (o1 - h), rtol=1e-10, atol=1e-13)


def test_gate_tokens_independent():
    rng = np.random.default_rng(5)
    e, h, wk, wv, gq, gk = _rand_gate(rng, 7, 20, 12)
    o, a = oracle.gate(e, h, wk, wv, gq, gk, 1e-6, oracle.F32)
    o3, a3 = oracle.gate(e[3:4], h[3:4], wk, wv, gq, gk, 1e-6, oracle.F32)
    assert np.array_equal(o[3:4], o3) and a[3] == a3[0]


def test_gate_bf16_decoding_matches_float_path():
    """The bf16 entry decodes bits exactly: same values given as fp32 and as bf16 bits agree exactly."""
    import torch
    rng = np.random.default_rng(6)
    arrs = _rand_gate(rng, 3, 16, 8)
    rounded = [torch.as_tensor(a).to(torch.bfloat16).to(torch.float32).numpy() for a in arrs]
    bits = [bf16_bits(a) for a in arrs]
    o1, a1 = oracle.gate(*rounded, 1e-6, oracle.F32)
    o2, a2 = oracle.gate(*bits, 1e-6, oracle.BF16)
    assert np.array_equal(o1, o2) and np.array_equal(a1, a2)


# ---------------------------------------------------------------------------
# whole path on the tiny configuration
# ---------------------------------------------------------------------------
def test_tiny_pipeline_end_to_end():
    import torch
    cfg = synth.CONFIGS["tiny"]
    raw = synth.raw_ids(cfg)
    ids, bad = oracle.compress(raw, synth.comp_map(cfg))
    assert bad == 0
    idx = oracle.hash_ids(ids, cfg.orders, cfg.heads, synth.multipliers(cfg), synth.table_rows_u32(cfg),
                          cfg.vocab_c)
    assert idx.shape == (cfg.tokens, cfg.n_tables) and idx.min() >= 0 and idx.max() < cfg.rows
    tables = [synth.table_rows(cfg, b, torch.arange(cfg.rows)).numpy() for b in range(cfg.n_tables)]
    e = oracle.gather(idx, tables)
    h = synth.hidden_rows(cfg, 0, torch.arange(cfg.tokens)).numpy()
    wk, wv = (x.numpy() for x in synth.weights(cfg, 0))
    gq, gk = (x.numpy() for x in synth.gains(cfg, 0))
    out, alpha = oracle.gate(e, h, wk, wv, gq, gk, cfg.eps, oracle.F32)
    assert np.all((alpha > 0) & (alpha < 1)) and np.isfinite(out).all()
    # tables ~ N(0, 0.02): the update is small next to the residual
    assert np.abs(out - h).max() < 0.2


# ---------------------------------------------------------------------------
# Short depthwise causal convolution (section 2.3, Eq. (5))

def _silu_lib(x):
    from scipy.special import expit  # the logistic function, as a library routine
    return np.asarray(x, dtype=np.float64) * expit(x)


def test_conv_zero_weights_leave_the_base():
    """SiLU(0) = 0: with all kernel weights zero the output is the base, bit for bit."""
    rng = np.random.default_rng(31)
    b, s, d = 2, 11, 6
    v = rng.standard_normal((b * s, d))
    base = rng.standard_normal((b * s, d))
    w = np.zeros((d, 4), dtype=np.float32)
    g = rng.standard_normal(d).astype(np.float32)
    out = oracle.conv(v, b, s, w, g, 3, 1e-6, oracle.F32, base)
    assert np.array_equal(out, base)


def test_conv_delta_reaches_exactly_the_dilated_taps():
    """One non-zero token (a constant row, whose RMSNorm is gamma) in sequence 0: tap j
    of the kernel shows up j * dil positions later and nowhere else; sequence 1 and
    earlier positions stay zero.  Values are SiLU of the tap weights, SiLU computed
    from scipy's logistic function."""
    b, s, d, dil, t0 = 2, 16, 5, 3, 2
    v = np.zeros((b * s, d))
    v[t0, :] = 0.37
    taps = np.array([1.0, -1.0, 2.0, 0.5], dtype=np.float32)
    w = np.tile(taps, (d, 1))
    g = np.ones(d, dtype=np.float32)
    out = oracle.conv(v, b, s, w, g, dil, 1e-12, oracle.F32, np.zeros_like(v))
    expect = np.zeros_like(v)
    for j in range(4):
        expect[t0 + j * dil, :] = _silu_lib(np.float64(taps[j]))
    assert np.allclose(out, expect, rtol=1e-10, atol=1e-12)
    assert np.count_nonzero(out[s:]) == 0 and np.count_nonzero(out[:t0]) == 0


def test_conv_delta_with_gamma_hand_values():
    """tests/golden/conv_delta_gamma.txt: one constant token row, gains != 1 and a
    different kernel per channel; the output is SiLU(w[c][j] * gamma_c) exactly j * dil
    tokens later, which pins gamma after the normalisation (rms(gamma) != 1)."""
    g = {r[0]: r[1:] for r in read_golden("conv_delta_gamma.txt")}
    d, t0, dil, a = int(g["d_model"][0]), int(g["t0"][0]), int(g["dil"][0]), float(g["a"][0])
    gamma = np.array(g["gamma"], np.float32)
    w = np.array([g[f"w{c}"] for c in range(d)], np.float32)
    y = np.array([g[f"y{c}"] for c in range(d)], np.float64)
    s = t0 + 3 * dil + 4
    v = np.zeros((s, d))
    v[t0, :] = a
    out = oracle.conv(v, 1, s, w, gamma, dil, 1e-12, oracle.F32, np.zeros_like(v))
    expect = np.zeros_like(v)
    for j in range(4):
        expect[t0 + j * dil, :] = y[:, j]
    np.testing.assert_allclose(out, expect, rtol=1e-10, atol=1e-12)


def test_conv_is_causal_per_sequence_with_dilated_reach():
    """Changing the gated value of one token changes the outputs of exactly the
    tokens t, t + dil, t + 2 dil, t + 3 dil of the same sequence."""
    rng = np.random.default_rng(32)
    b, s, d, dil = 3, 20, 7, 3
    v = rng.standard_normal((b * s, d))
    w = rng.standard_normal((d, 4)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    base = np.zeros_like(v)
    o1 = oracle.conv(v, b, s, w, g, dil, 1e-6, oracle.F32, base)
    v2 = v.copy()
    tb, tt = 1, 5
    v2[tb * s + tt] += 1.0
    o2 = oracle.conv(v2, b, s, w, g, dil, 1e-6, oracle.F32, base)
    changed = np.nonzero(np.any(o1 != o2, axis=1))[0]
    assert list(changed) == [tb * s + tt + j * dil for j in range(4)]


def test_conv_rmsnorm_makes_it_scale_invariant():
    rng = np.random.default_rng(33)
    b, s, d = 1, 13, 8
    v = rng.standard_normal((b * s, d))
    w = rng.standard_normal((d, 4)).astype(np.float32)
    g = rng.standard_normal(d).astype(np.float32)
    base = rng.standard_normal((b * s, d))
    o1 = oracle.conv(v, b, s, w, g, 3, 0.0, oracle.F32, base)
    o2 = oracle.conv(v * 7.5, b, s, w, g, 3, 0.0, oracle.F32, base)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_gate_value_output_is_the_gated_value():
    """The gate's optional value output is alpha * v = out - h."""
    rng = np.random.default_rng(34)
    n, dm, d = 5, 16, 12
    e = rng.standard_normal((n, dm)).astype(np.float32)
    h = rng.standard_normal((n, d)).astype(np.float32)
    wk = rng.standard_normal((d, dm)).astype(np.float32)
    wv = rng.standard_normal((d, dm)).astype(np.float32)
    ones_q, ones_k = np.ones(d, dtype=np.float32), np.ones(dm, dtype=np.float32)
    out, alpha, value = oracle.gate(e, h, wk, wv, ones_q, ones_k, 1e-6, oracle.F32, with_value=True)
    assert np.allclose(value, out - h.astype(np.float64), rtol=1e-12, atol=1e-12)
    v = e.astype(np.float64) @ wv.astype(np.float64).T
    assert np.allclose(value, alpha[:, None] * v, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# The paper's key placement (Eq. (4) / Eq. (6)): RMSNorm after W_K

def test_gate_projected_key_equals_memory_key_for_orthogonal_wk():
    """For an orthogonal W_K (d_model = d_mem) and unit gains, RMSNorm(W_K e) = W_K RMSNorm(e),
    so the two placements of the key's norm give the same gate."""
    rng = np.random.default_rng(41)
    d = 24
    q_mat, _ = np.linalg.qr(rng.standard_normal((d, d)))
    e, h, _, wv, gq, _ = _rand_gate(rng, 6, d, d)
    wk = q_mat.astype(np.float32)
    ones = np.ones(d, np.float32)
    _, a_mem = oracle.gate(e, h, wk, wv, gq, ones, 0.0, oracle.F32, key_norm=oracle.KEY_NORM_MEMORY)
    _, a_proj = oracle.gate(e, h, wk, wv, gq, ones, 0.0, oracle.F32, key_norm=oracle.KEY_NORM_PROJECTED)
    # wk is orthogonal only to float32 rounding
    np.testing.assert_allclose(a_proj, a_mem, rtol=0, atol=1e-6)


def test_gate_projected_key_ignores_the_scale_of_wk():
    """Normalising after the projection removes W_K's scale (eps = 0; the factor 4 is exact);
    normalising the memory before it does not."""
    rng = np.random.default_rng(42)
    e, h, wk, wv, gq, _ = _rand_gate(rng, 7, 20, 12)
    gk = (1 + 0.2 * rng.standard_normal(12)).astype(np.float32)
    _, a1 = oracle.gate(e, h, wk, wv, gq, gk, 0.0, oracle.F32, key_norm=oracle.KEY_NORM_PROJECTED)
    _, a4 = oracle.gate(e, h, 4 * wk, wv, gq, gk, 0.0, oracle.F32, key_norm=oracle.KEY_NORM_PROJECTED)
    np.testing.assert_allclose(a4, a1, rtol=1e-12, atol=0)
    gk_m = np.ones(20, np.float32)
    _, m1 = oracle.gate(e, h, wk, wv, gq, gk_m, 0.0, oracle.F32)
    _, m4 = oracle.gate(e, h, 4 * wk, wv, gq, gk_m, 0.0, oracle.F32)
    assert np.abs(m4 - m1).max() > 1e-3


def test_gate_projected_key_limits():
    """W_K = 0 gives alpha = 1/2; out and the value projection do not depend on the key's form."""
    rng = np.random.default_rng(43)
    e, h, wk, wv, gq, gk = _rand_gate(rng, 5, 16, 8)
    gk_d = np.ones(8, np.float32)
    _, a0 = oracle.gate(e, h, np.zeros_like(wk), wv, gq, gk_d, 1e-6, oracle.F32, key_norm=1)
    assert np.all(a0 == 0.5)
    out_p, a_p, v_p = oracle.gate(e, h, wk, wv, gq, gk_d, 1e-6, oracle.F32, with_value=True, key_norm=1)
    np.testing.assert_allclose(v_p, out_p - h.astype(np.float64), rtol=1e-12, atol=1e-12)
    v = e.astype(np.float64) @ wv.astype(np.float64).T
    np.testing.assert_allclose(v_p, a_p[:, None] * v, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) codes and the FP8 gate

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_e4m3_known_codes():
    d = dict(zip(range(256), oracle.e4m3_decode(np.arange(256))))
    assert d[0x38] == 1.0 and d[0x40] == 2.0 and d[0x3C] == 1.5 and d[0x37] == 0.9375
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0 and d[0xB8] == -1.0
    assert d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9 and d[0x08] == 2.0 ** -6
    assert d[0x00] == 0.0 and np.signbit(d[0x80])
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    pos = oracle.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)                    # strictly increasing magnitudes


def test_e4m3_encode_round_trips_every_finite_code():
    vals = oracle.e4m3_decode(np.array(FINITE, np.uint8)).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), np.array(FINITE, np.uint8))


def test_e4m3_encode_ties_to_even_and_neighbours():
    lo = oracle.e4m3_decode(np.arange(0x7E))
    hi = oracle.e4m3_decode(np.arange(1, 0x7F))
    mid = ((lo + hi) / 2).astype(np.float32)            # exact: at most 5 significant bits
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    got = oracle.e4m3_encode(mid)
    even = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F)).astype(np.uint8)
    assert np.array_equal(got, even)
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mid, np.float32(np.inf))), np.arange(1, 0x7F, dtype=np.uint8))
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mid, np.float32(0))), np.arange(0x7E, dtype=np.uint8))
    assert np.array_equal(oracle.e4m3_encode(-mid), even | 0x80)


def test_e4m3_encode_saturates():
    assert list(oracle.e4m3_encode([448.0, 460.0, 464.0, 1e30, -1e30, -470.0])) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert oracle.e4m3_encode([2.0 ** -10])[0] == 0x00          # tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_encode([3 * 2.0 ** -10])[0] == 0x02      # tie between 2^-9 and 2^-8 -> even


def test_quant_rows_scale_and_error_bound():
    rng = np.random.default_rng(50)
    x = (rng.standard_normal((40, 300)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    x[3] = 0.0
    codes, scales = oracle.quant_rows(x)
    mx = np.abs(x).max(axis=1)
    assert np.array_equal(scales, np.where(mx > 0, mx / np.float32(448), np.float32(1)).astype(np.float32))
    assert np.all(codes[3] == 0) and scales[3] == 1.0
    deq = oracle.e4m3_decode(codes) * scales[:, None].astype(np.float64)
    err = np.abs(deq - x.astype(np.float64))
    # half a spacing: 2^-4 of the value for normals, 2^-10 of the scale for subnormals
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scales[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    amax = np.abs(x).argmax(axis=1)
    for r in range(40):
        if r != 3:
            assert codes[r, amax[r]] & 0x7F == 0x7E    # the largest element maps to 448


def _fp8_exact_gate_inputs(rng, n, dm, d):
    """Inputs that E4M3 with the per-row scales represents exactly: rows of grid values
    times a power of two, each row holding +-448 times that power."""
    grid = oracle.e4m3_decode(np.array([c for c in FINITE if c not in (0x80,)], np.uint8))
    def rows(r, c, p2):
        x = rng.choice(grid, size=(r, c)) * 2.0 ** p2
        x[:, 0] = 448.0 * 2.0 ** p2 * rng.choice([-1, 1], size=r)
        return x.astype(np.float32)
    return rows(n, dm, -8), rows(d, dm, -10), rows(d, dm, -10)


@pytest.mark.parametrize("key_norm", [0, 1])
def test_gate_fp8_equals_gate_on_exactly_representable_inputs(key_norm):
    rng = np.random.default_rng(51 + key_norm)
    n, dm, d = 6, 48, 20
    e, wk, wv = _fp8_exact_gate_inputs(rng, n, dm, d)
    h = rng.standard_normal((n, d)).astype(np.float32)
    gq = (1 + 0.2 * rng.standard_normal(d)).astype(np.float32) if key_norm else np.ones(d, np.float32)
    gk = (1 + 0.2 * rng.standard_normal(d if key_norm else dm)).astype(np.float32) if key_norm \
        else np.ones(dm, np.float32)
    out8, a8 = oracle.gate_fp8(e, h, wk, wv, gq, gk, 1e-6, oracle.F32, key_norm=key_norm)
    out, a = oracle.gate(e, h, wk, wv, gq, gk, 1e-6, oracle.F32, key_norm=key_norm)
    np.testing.assert_allclose(a8, a, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out8, out, rtol=1e-12, atol=1e-13)


def test_gate_fp8_close_to_gate_on_random_inputs():
    """Quantization moves each operand element by at most 2^-4 of itself, so alpha and the
    update stay within a few percent of the unquantized gate."""
    rng = np.random.default_rng(53)
    n, dm, d = 8, 64, 32
    e = rng.standard_normal((n, dm)).astype(np.float32)
    h = rng.standard_normal((n, d)).astype(np.float32)
    wk = (rng.standard_normal((d, dm)) / 8).astype(np.float32)
    wv = (rng.standard_normal((d, dm)) / 8).astype(np.float32)
    ones_d, ones_m = np.ones(d, np.float32), np.ones(dm, np.float32)
    out8, a8 = oracle.gate_fp8(e, h, wk, wv, ones_d, ones_m, 1e-6, oracle.F32)
    out, a = oracle.gate(e, h, wk, wv, ones_d, ones_m, 1e-6, oracle.F32)
    assert np.abs(a8 - a).max() < 0.05
    upd8, upd = out8 - h, out - h
    assert np.abs(upd8 - upd).max() < 0.08 * np.abs(upd).max()

"""Helpers of the GPU parity tests: error metric and oracle runs on sampled tokens.

The oracle side computes everything from the seeded inputs (synth) with the
CPU oracle; nothing here reads a result of the HIP path.
"""
import numpy as np
import torch

import oracle
import synth


def bf16_bits_np(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bits of a CPU bfloat16 tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def host_view(t: torch.Tensor) -> np.ndarray:
    """numpy view of a CPU tensor as the oracle expects it (float32, or bf16 bits)."""
    t = t.detach().cpu().contiguous()
    return bf16_bits_np(t) if t.dtype == torch.bfloat16 else t.numpy()


def sentinel_like(t: torch.Tensor) -> torch.Tensor:
    """Fill a result buffer, in place, with a value no correct result has: NaN for float
    dtypes (0xFFFF for bf16), -1 for integers, 0xFF bytes for uint8.  Returns t."""
    if t.dtype in (torch.float32, torch.float64, torch.float16, torch.bfloat16):
        if t.dtype == torch.bfloat16:
            t.view(torch.int16).fill_(-1)
        else:
            t.fill_(float("nan"))
    elif t.dtype == torch.uint8:
        t.fill_(0xFF)
    else:
        t.fill_(-1)
    return t


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """The parity metric: max relative error with the denominator floored at 1e-2 of the
    reference's RMS,
        max_i |gpu_i - ref_i| / max(|ref_i|, 1e-2 rms(ref)).
    The floor keeps elements that cancel to (near) zero from dominating; above it every
    element is judged relative to itself."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = 1e-2 * np.sqrt((ref ** 2).mean())
    if floor == 0.0:
        return float(np.abs(gpu - ref).max()) if ref.size else 0.0
    return float((np.abs(gpu - ref) / np.maximum(np.abs(ref), floor)).max())


def rel_err_rms(gpu: np.ndarray, ref: np.ndarray) -> float:
    """A looser companion metric, reported beside rel_err for the update out - h: the
    denominator floored at the reference's full RMS, max_i |g_i - r_i| / max(|r_i|, rms(r))."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = np.sqrt((ref ** 2).mean())
    return float((np.abs(gpu - ref) / np.maximum(np.abs(ref), floor)).max())


BF16_ONE = np.uint16(0x3F80)
# alpha against the oracle run on exactly the operands the kernel multiplies (the
# library's documented roundings applied): the two differ only by fp32 against fp64
# accumulation over d_mem and d_model terms (measured 1e-7 - 2e-5)
ALPHA_TOL_ARITH = 1e-4
# alpha against the unrounded definition with gains != 1 on the memory-side key: the
# bf16 path rounds gq W_K gk once to bf16 (relative 2^-8 per weight)
ALPHA_TOL_DEF = 2e-3
# update out - h (rel_err_rms) in cases where |alpha v| is comparable to |h|: the output's
# own bf16 rounding (2^-8 |out|) over |alpha v| ~ 0.5
UPDATE_TOL = 5e-2


def folded_key_weights(wk: np.ndarray, gq: np.ndarray, gk: np.ndarray) -> np.ndarray:
    """bf16 bits of W'[f][c] = bf16((gq[f] * W_K[f][c]) * gk[c]), products in fp32, one
    round-to-nearest-even: the key weights the bf16 gate multiplies with the memory-side
    key norm (engram.h documents this fold).  Inputs are bf16 bits."""
    f = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).float()
    w = (f(gq)[:, None] * f(wk)) * f(gk)[None, :]
    return w.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_is_one(x: np.ndarray) -> bool:
    return bool(np.all(x == BF16_ONE))


def check_gate(label, out, alpha, e, h, wk, wv, gq, gk, eps, key_norm=oracle.KEY_NORM_MEMORY, fp8=False,
               vals=None, dtype=oracle.BF16, update=False, out_bar=None, say=print):
    """Check one branch of a gate call against the oracle.

    out, alpha (and vals, the gated values): the GPU's results as numpy float arrays
    ([n, d_model], [n]); e, h, wk, wv, gq, gk: the inputs as the oracle takes them (bf16
    bits or float32).  Two oracle runs:
      arith: the oracle on exactly the operands the kernel multiplies.  That is the
             definition itself, except for the bf16 gate with the memory-side key norm
             and gains != 1, whose key weights are folded and rounded once
             (folded_key_weights).  FP8 runs take oracle.gate_fp8 (the same codes).
             Bars: rel_err(out) <= out_bar (1e-2 bf16, 1e-5 fp32), |alpha| <= 1e-4
             (fp32: 1e-5), rel_err(vals) <= out_bar.
      def:   the unrounded definition (differs from arith only in the folded case):
             |alpha| <= 2e-3; its rel_err on out is reported.
    update=True also bounds rel_err_rms(out - h) by UPDATE_TOL (cases whose |alpha v|
    is comparable to |h|)."""
    f32 = dtype == oracle.F32
    if out_bar is None:
        out_bar = 1e-5 if f32 else 1e-2
    a_tol = 1e-5 if f32 else ALPHA_TOL_ARITH
    if fp8:
        ref = lambda w_k, g_q, g_k: oracle.gate_fp8(e, h, w_k, wv, g_q, g_k, eps, dtype, key_norm=key_norm)
    else:
        ref = lambda w_k, g_q, g_k: oracle.gate(e, h, w_k, wv, g_q, g_k, eps, dtype, key_norm=key_norm)
    out_d, alpha_d = ref(wk, gq, gk)
    folded = (not fp8 and not f32 and key_norm == oracle.KEY_NORM_MEMORY
              and not (_bits_is_one(gq) and _bits_is_one(gk)))
    if folded:
        ones_q = np.full(gq.shape, BF16_ONE, np.uint16)
        ones_k = np.full(gk.shape, BF16_ONE, np.uint16)
        out_a, alpha_a = ref(folded_key_weights(wk, gq, gk), ones_q, ones_k)
    else:
        out_a, alpha_a = out_d, alpha_d
    h64 = h.astype(np.float64) if h.dtype != np.uint16 else \
        torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).double().numpy()
    out = np.asarray(out, np.float64)
    err = rel_err(out, out_a)
    err_def = rel_err(out, out_d)
    aerr = float(np.abs(np.asarray(alpha, np.float64) - alpha_a).max())
    aerr_def = float(np.abs(np.asarray(alpha, np.float64) - alpha_d).max())
    upd = rel_err_rms(out - h64, out_a - h64)
    msg = (f"  {label}: out rel err {err:.2e} (vs unrounded definition {err_def:.2e}), alpha abs err "
           f"{aerr:.2e} (definition {aerr_def:.2e}), update rel err (rms floor) {upd:.2e}")
    ok = err <= out_bar and aerr <= a_tol and aerr_def <= (ALPHA_TOL_DEF if folded else a_tol)
    if vals is not None:
        verr = rel_err(np.asarray(vals, np.float64), out_a - h64)
        msg += f", value rel err {verr:.2e}"
        ok = ok and verr <= out_bar
    if update:
        ok = ok and upd <= UPDATE_TOL
    say(msg)
    assert ok, msg
    return err, aerr


def oracle_ids_idx(cfg: synth.Config, raw: np.ndarray, t_begin=0, t_count=None):
    ids, bad = oracle.compress(raw, synth.comp_map(cfg))
    assert bad == 0
    idx = oracle.hash_ids(ids, cfg.orders, cfg.heads, synth.multipliers(cfg), synth.table_rows_u32(cfg),
                          cfg.vocab_c, t_begin=t_begin, t_count=t_count)
    return ids, idx


def oracle_memory(cfg: synth.Config, idx_rows: np.ndarray, nrows=None) -> np.ndarray:
    """Oracle memory vectors for the given index rows [n, n_tables]: the oracle gather over
    sub-tables holding just the referenced rows (regenerated from the seeded generator)."""
    subs, remap = [], np.empty_like(idx_rows)
    for b in range(cfg.n_tables):
        uniq, inv = np.unique(idx_rows[:, b], return_inverse=True)
        subs.append(host_view(synth.table_rows(cfg, b, torch.from_numpy(uniq.astype(np.int64)))))
        remap[:, b] = inv
    return oracle.gather(remap, subs)


def gate_inputs_tokens(cfg: synth.Config, m: int, tokens: np.ndarray, key_norm: int = oracle.KEY_NORM_MEMORY):
    """Host views (h, wk, wv, gq, gk) of branch m's gate inputs for global token numbers `tokens`."""
    h = host_view(synth.hidden_rows(cfg, m, torch.from_numpy(tokens.astype(np.int64))))
    wk, wv = (host_view(x) for x in synth.weights(cfg, m))
    proj = key_norm == oracle.KEY_NORM_PROJECTED
    gq, gk = (host_view(x) for x in synth.gains(cfg, m, projected_key=proj))
    return h, wk, wv, gq, gk


def oracle_gate_tokens(cfg: synth.Config, m: int, e: np.ndarray, tokens: np.ndarray,
                       key_norm: int = oracle.KEY_NORM_MEMORY):
    """Oracle (out [n, d_model] float64, alpha [n]) of branch m for global token numbers `tokens`."""
    h, wk, wv, gq, gk = gate_inputs_tokens(cfg, m, tokens, key_norm)
    dt = oracle.F32 if cfg.dtype == "f32" else oracle.BF16
    return oracle.gate(e, h, wk, wv, gq, gk, cfg.eps, dt, key_norm=key_norm)


def check_gate_tokens(label, cfg: synth.Config, m: int, out, alpha, e: np.ndarray, tokens: np.ndarray,
                      key_norm: int = oracle.KEY_NORM_MEMORY, update=False, say=print):
    """check_gate for branch m of a configuration on global token numbers `tokens`."""
    h, wk, wv, gq, gk = gate_inputs_tokens(cfg, m, tokens, key_norm)
    dt = oracle.F32 if cfg.dtype == "f32" else oracle.BF16
    return check_gate(label, out, alpha, e, h, wk, wv, gq, gk, cfg.eps, key_norm=key_norm, dtype=dt,
                      update=update, say=say)


def sample_tokens(cfg: synth.Config, n: int, seed: int = 0) -> np.ndarray:
    """Sorted global token numbers: every sequence's positions 0, 1, 2 and seq-1 plus random ones."""
    rng = np.random.default_rng([cfg.seed, seed, 7])
    fixed = []
    for b in range(cfg.batch):
        for p in (0, 1, 2, cfg.seq - 1):
            fixed.append(b * cfg.seq + p)
    fixed = np.unique(np.array(fixed))
    extra = rng.choice(cfg.tokens, size=max(0, n - len(fixed)), replace=False)
    return np.unique(np.concatenate([fixed, extra]))

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


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Max relative error with the denominator floored at the reference's RMS:
        max_i |gpu_i - ref_i| / max(|ref_i|, rms(ref)).
    Elements at least as large as the typical magnitude are judged relative to
    themselves; smaller ones (near-cancellations of h + alpha v) relative to
    the typical magnitude, the scale on which their rounding error lives."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = np.sqrt((ref ** 2).mean())
    return float((np.abs(gpu - ref) / np.maximum(np.abs(ref), floor)).max())


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


def oracle_gate_tokens(cfg: synth.Config, m: int, e: np.ndarray, tokens: np.ndarray,
                       key_norm: int = oracle.KEY_NORM_MEMORY):
    """Oracle (out [n, d_model] float64, alpha [n]) of branch m for global token numbers `tokens`."""
    h = host_view(synth.hidden_rows(cfg, m, torch.from_numpy(tokens.astype(np.int64))))
    wk, wv = (host_view(x) for x in synth.weights(cfg, m))
    proj = key_norm == oracle.KEY_NORM_PROJECTED
    gq, gk = (host_view(x) for x in synth.gains(cfg, m, projected_key=proj))
    dt = oracle.F32 if cfg.dtype == "f32" else oracle.BF16
    return oracle.gate(e, h, wk, wv, gq, gk, cfg.eps, dt, key_norm=key_norm)


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

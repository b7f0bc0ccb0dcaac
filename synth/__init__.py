"""Seeded synthetic inputs for the Engram forward pass.

Test and benchmark infrastructure shared by the CPU oracle's tests, the GPU
parity tests, ``bench.py`` and ``smoke()``.  It draws inputs only: token ids,
the compression surjection, hash multipliers, embedding-table contents, hidden
states, projection weights and RMSNorm gains.  It performs no step of the
method itself (no compression lookup, hashing, gathering or gating).

Workload shapes follow the paper "Conditional Memory via Scalable Lookup"
(section 2.2: n-gram orders {2,3}, K hash heads per order, prime-sized tables;
Appendix A, Table 5: memory dim 1280, 8 heads, 129,280-token vocabulary;
Appendix C, Table 6: the normalising surjection shrinks that vocabulary by
about 23 %) and the five synthetic configurations listed in ``CONFIGS``.

Generators
----------
* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014) draws the hash multipliers.
* A counter-based generator (SplitMix64's output finaliser applied to a
  (seed, stream, row, column) counter, four 16-bit limbs summed into an
  Irwin-Hall(4) variate) fills tables, hidden states and weights.  It is
  written once in torch integer ops, so the same function fills a 26 GB table
  on the GPU and regenerates any handful of rows on the CPU bit-identically.
  ``counter_normal_numpy`` is a uint64 numpy restatement used to pin that the
  torch version's wrapping int64 arithmetic is right.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

# exact standard deviation of the sum of four independent uniform 16-bit limbs
_IH4_MEAN = 2 * 65535
_IH4_STD = math.sqrt(4 * (65536.0 ** 2 - 1) / 12.0)


# --------------------------------------------------------------------------
# SplitMix64
# --------------------------------------------------------------------------
def splitmix64(seed: int, n: int) -> List[int]:
    """First ``n`` outputs of SplitMix64 started at state ``seed``."""
    s = seed & MASK64
    out = []
    for _ in range(n):
        s = (s + GOLDEN) & MASK64
        z = s
        z = ((z ^ (z >> 30)) * MIX1) & MASK64
        z = ((z ^ (z >> 27)) * MIX2) & MASK64
        out.append(z ^ (z >> 31))
    return out


def _fmix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def hash_multipliers(seed: int, orders: Sequence[int], heads: int) -> np.ndarray:
    """Odd 64-bit multipliers, array [n_orders][heads][max_order] (uint64).

    Drawn from SplitMix64(seed) in the order: order ascending, head ascending,
    position-in-gram ascending; each draw is forced odd.  Slots j >= n of an
    order-n gram are unused and left 0.
    """
    max_order = max(orders)
    out = np.zeros((len(orders), heads, max_order), dtype=np.uint64)
    draws = iter(splitmix64(seed, sum(n * heads for n in orders)))
    for oi, n in enumerate(orders):
        for k in range(heads):
            for j in range(n):
                out[oi, k, j] = next(draws) | 1
    return out


# --------------------------------------------------------------------------
# primes
# --------------------------------------------------------------------------
def is_prime(n: int) -> bool:
    if n < 2:
        return False
    small = (2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37)
    for p in small:
        if n % p == 0:
            return n == p
    d, s = n - 1, 0
    while d % 2 == 0:
        d //= 2
        s += 1
    for a in small:  # deterministic for n < 3.3e24
        x = pow(a, d, n)
        if x in (1, n - 1):
            continue
        for _ in range(s - 1):
            x = x * x % n
            if x == n - 1:
                break
        else:
            return False
    return True


def next_prime(n: int) -> int:
    while not is_prime(n):
        n += 1
    return n


# --------------------------------------------------------------------------
# token ids and the compression surjection
# --------------------------------------------------------------------------
def zipf_ids(rng: np.random.Generator, vocab: int, s: float, shape) -> np.ndarray:
    """i.i.d. finite Zipf ids on 0..vocab-1, P(i) proportional to (i+1)^-s (inverse CDF)."""
    p = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(int(np.prod(shape)))
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32).reshape(shape)


def compression_map(rng: np.random.Generator, vocab: int, vocab_c: int) -> np.ndarray:
    """Seeded surjection {0..vocab-1} -> {0..vocab_c-1} (int32[vocab]).

    A random permutation gives the first vocab_c raw ids one canonical id each
    (so the map is onto); the remaining raw ids fold onto uniform targets.
    """
    perm = rng.permutation(vocab)
    m = np.empty(vocab, dtype=np.int32)
    m[perm[:vocab_c]] = np.arange(vocab_c, dtype=np.int32)
    m[perm[vocab_c:]] = rng.integers(0, vocab_c, vocab - vocab_c, dtype=np.int32)
    return m


# --------------------------------------------------------------------------
# counter-based approximately-normal values
# --------------------------------------------------------------------------
def _i64(x: int) -> int:
    x &= MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def _stream_base(seed: int, stream: int) -> int:
    return _fmix64_int((seed * GOLDEN + stream) & MASK64)


def counter_normal(seed: int, stream: int, rows, ncols: int, std: float,
                   dtype=None, device=None):
    """Approximately N(0, std^2) values for the given rows of a counter-addressed matrix.

    Element (row r, col c) of stream ``stream`` is
        u = fmix64(base ^ (((r << 16) | c) * GOLDEN mod 2^64)),
        base = fmix64(seed * GOLDEN + stream mod 2^64),
        S = sum of the four 16-bit limbs of u,
        value = fp32(S - 131070) * fp32(std / 37837.23), then cast to ``dtype``.
    ``rows`` is an int64 tensor (or sequence) of row numbers < 2^47 and ncols <= 65536.
    Returns a torch tensor [len(rows), ncols] on ``device`` (default: rows' device).
    """
    import torch

    if dtype is None:
        dtype = torch.float32
    if not torch.is_tensor(rows):
        rows = torch.as_tensor(np.asarray(rows, dtype=np.int64))
    if device is None:
        device = rows.device
    rows = rows.to(device=device, dtype=torch.int64)
    assert ncols <= 65536
    base = _i64(_stream_base(seed, stream))
    cols = torch.arange(ncols, device=device, dtype=torch.int64)
    x = (rows[:, None] << 16) | cols[None, :]
    x = x * _i64(GOLDEN)
    x = x ^ base
    # fmix64 with logical right shifts on wrapping int64
    x = x ^ ((x >> 30) & ((1 << 34) - 1))
    x = x * _i64(MIX1)
    x = x ^ ((x >> 27) & ((1 << 37) - 1))
    x = x * _i64(MIX2)
    x = x ^ ((x >> 31) & ((1 << 33) - 1))
    s = (x & 0xFFFF) + ((x >> 16) & 0xFFFF) + ((x >> 32) & 0xFFFF) + ((x >> 48) & 0xFFFF)
    scale = torch.tensor(std / _IH4_STD, dtype=torch.float32, device=device)
    v = (s - _IH4_MEAN).to(torch.float32) * scale
    return v.to(dtype)


def counter_normal_numpy(seed: int, stream: int, rows, ncols: int, std: float) -> np.ndarray:
    """The same values as ``counter_normal`` in fp32, computed with numpy uint64 arithmetic."""
    rows = np.asarray(rows, dtype=np.uint64)
    cols = np.arange(ncols, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = (rows[:, None] << np.uint64(16)) | cols[None, :]
        x = x * np.uint64(GOLDEN)
        x = x ^ np.uint64(_stream_base(seed, stream))
        x = x ^ (x >> np.uint64(30))
        x = x * np.uint64(MIX1)
        x = x ^ (x >> np.uint64(27))
        x = x * np.uint64(MIX2)
        x = x ^ (x >> np.uint64(31))
    m = np.uint64(0xFFFF)
    s = (x & m) + ((x >> np.uint64(16)) & m) + ((x >> np.uint64(32)) & m) + ((x >> np.uint64(48)) & m)
    v = (s.astype(np.int64) - _IH4_MEAN).astype(np.float32) * np.float32(std / _IH4_STD)
    return v


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    vocab: int
    vocab_c: int
    batch: int
    seq: int
    orders: tuple
    heads: int
    rows: int            # rows of every table (prime)
    w: int               # columns per table
    dtype: str           # "f32" or "bf16": tables, hidden, weights, outputs
    d_model: int
    n_branch: int
    zipf_s: float
    seed: int
    table_std: float = 0.02
    gamma_jitter: float = 0.0   # gains are 1 + jitter * N(0,1); 0 means all ones
    eps: float = 1e-6
    decode_steps: int = 0       # > 0: decode workload, hashing position seq + step

    @property
    def n_tables(self) -> int:
        return len(self.orders) * self.heads

    @property
    def d_mem(self) -> int:
        return self.n_tables * self.w

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


V_FULL = 129_280
V_COMP = round(0.77 * V_FULL)          # 99,546: about 23 % fewer canonical ids
ROWS_SMALL = 1_000_003
ROWS_LARGE = next_prime(-(-13_000_000_000 // (16 * 80)))     # 13e9 params over 16 tables of 80 cols
ROWS_OFFLOAD = next_prime(-(-100_000_000_000 // 1280))       # 100e9 params over 16 x 80 cols

CONFIGS = {
    "tiny": Config("tiny", 1000, 770, 1, 64, (2, 3), 2, 4093, 32, "f32", 128, 1, 1.1, 1),
    "small": Config("small", V_FULL, V_COMP, 4, 4096, (2, 3), 8, ROWS_SMALL, 80, "bf16", 2560, 1, 1.1, 2),
    "multi": Config("multi", V_FULL, V_COMP, 8, 8192, (2, 3), 8, ROWS_SMALL, 80, "bf16", 4096, 4, 1.1, 3,
                    gamma_jitter=0.1),
    "large": Config("large", V_FULL, V_COMP, 8, 32768, (2, 3), 8, ROWS_LARGE, 80, "bf16", 4096, 2, 1.05, 4),
    # decode: 256 sequences with 4096-token histories, one new token per step
    "offload": Config("offload", V_FULL, V_COMP, 256, 4096, (2, 3), 8, ROWS_OFFLOAD, 80, "bf16", 4096, 1,
                      1.1, 5, decode_steps=128),
}

# streams of the counter-based generator
STREAM_TABLE = 0          # + table index
STREAM_HIDDEN = 1 << 20   # + branch
STREAM_WK = 2 << 20       # + branch
STREAM_WV = 3 << 20       # + branch
STREAM_GQ = 4 << 20       # + branch
STREAM_GK = 5 << 20       # + branch
STREAM_CONV_W = 6 << 20   # + branch
STREAM_CONV_G = 7 << 20   # + branch
STREAM_GKP = 8 << 20      # + branch: the key gain over d_model (key normalised after W_K)

# the short convolution of the pages' configuration: kernel size 4, dilation = the
# largest n-gram order
CONV_TAPS = 4


def rng_for(cfg: Config, what: str) -> np.random.Generator:
    keys = {"ids": 0, "map": 1, "decode": 2, "sample": 3}
    ss = np.random.SeedSequence([cfg.seed, keys[what]])
    return np.random.default_rng(ss)


def raw_ids(cfg: Config) -> np.ndarray:
    """int32 [batch, seq + decode_steps] raw token ids."""
    return zipf_ids(rng_for(cfg, "ids"), cfg.vocab, cfg.zipf_s, (cfg.batch, cfg.seq + cfg.decode_steps))


def comp_map(cfg: Config) -> np.ndarray:
    return compression_map(rng_for(cfg, "map"), cfg.vocab, cfg.vocab_c)


def multipliers(cfg: Config) -> np.ndarray:
    return hash_multipliers(cfg.seed, cfg.orders, cfg.heads)


def table_rows_u32(cfg: Config) -> np.ndarray:
    return np.full(cfg.n_tables, cfg.rows, dtype=np.uint32)


def torch_dtype(cfg: Config):
    import torch
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def table_rows(cfg: Config, b: int, rows, device="cpu"):
    """Rows ``rows`` of table ``b`` as a [len(rows), w] tensor of the config dtype."""
    return counter_normal(cfg.seed, STREAM_TABLE + b, rows, cfg.w, cfg.table_std,
                          torch_dtype(cfg), device)


def fill_table(cfg: Config, b: int, out, chunk_rows: int = 1 << 22):
    """Fill a preallocated [rows, w] tensor (any device) with table ``b``."""
    import torch
    n = out.shape[0]
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        rows = torch.arange(r0, r1, dtype=torch.int64, device=out.device)
        out[r0:r1].copy_(table_rows(cfg, b, rows, out.device))
    return out


def hidden_rows(cfg: Config, m: int, tokens, device="cpu"):
    """Hidden-state rows (global token numbers ``tokens``) of branch m, ~N(0,1)."""
    return counter_normal(cfg.seed, STREAM_HIDDEN + m, tokens, cfg.d_model, 1.0,
                          torch_dtype(cfg), device)


def fill_hidden(cfg: Config, m: int, out, chunk_rows: int = 1 << 16):
    import torch
    n = out.shape[0]
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        rows = torch.arange(r0, r1, dtype=torch.int64, device=out.device)
        out[r0:r1].copy_(hidden_rows(cfg, m, rows, out.device))
    return out


def weights(cfg: Config, m: int, device="cpu"):
    """(W_K, W_V) of branch m: [d_model, d_mem] each, ~N(0, 1/d_mem) (fan-in scaling)."""
    import torch
    rows = torch.arange(cfg.d_model, dtype=torch.int64, device=device)
    std = 1.0 / math.sqrt(cfg.d_mem)
    wk = counter_normal(cfg.seed, STREAM_WK + m, rows, cfg.d_mem, std, torch_dtype(cfg), device)
    wv = counter_normal(cfg.seed, STREAM_WV + m, rows, cfg.d_mem, std, torch_dtype(cfg), device)
    return wk, wv


def gains(cfg: Config, m: int, device="cpu", projected_key: bool = False):
    """(gamma_q [d_model], gamma_k) of branch m: 1 + jitter * N(0,1).  gamma_k has d_mem
    entries, or d_model with projected_key (the key normalised after W_K)."""
    import torch
    dt = torch_dtype(cfg)
    nk = cfg.d_model if projected_key else cfg.d_mem
    if cfg.gamma_jitter == 0.0:
        return (torch.ones(cfg.d_model, dtype=dt, device=device), torch.ones(nk, dtype=dt, device=device))
    zero = torch.zeros(1, dtype=torch.int64, device=device)
    gq = counter_normal(cfg.seed, STREAM_GQ + m, zero, cfg.d_model, cfg.gamma_jitter, torch.float32, device)[0]
    gk = counter_normal(cfg.seed, (STREAM_GKP if projected_key else STREAM_GK) + m, zero, nk, cfg.gamma_jitter,
                        torch.float32, device)[0]
    return (gq + 1.0).to(dt), (gk + 1.0).to(dt)


def conv_dilation(cfg: Config) -> int:
    return max(cfg.orders)


def conv_params(cfg: Config, m: int, taps: int = CONV_TAPS, std: float = 0.5, device="cpu"):
    """(w [d_model, taps], gamma [d_model]) of branch m's short convolution.

    The pages start the kernel at zero (the module then adds nothing); the
    synthetic kernel is ~N(0, std) so that every tap contributes, and gamma is
    1 + jitter * N(0,1) like the other gains."""
    import torch
    dt = torch_dtype(cfg)
    rows = torch.arange(cfg.d_model, dtype=torch.int64, device=device)
    w = counter_normal(cfg.seed, STREAM_CONV_W + m, rows, taps, std, dt, device)
    zero = torch.zeros(1, dtype=torch.int64, device=device)
    jitter = cfg.gamma_jitter if cfg.gamma_jitter > 0 else 0.1
    g = counter_normal(cfg.seed, STREAM_CONV_G + m, zero, cfg.d_model, jitter, torch.float32, device)[0]
    return w, (g + 1.0).to(dt)


def offload_rows(cfg: Config, mem_available_bytes: Optional[int]) -> int:
    """Table rows for the host-offloaded decode workload: the full 100B-parameter
    size, scaled down to fit 60 % of available host memory when that is smaller."""
    elem = 4 if cfg.dtype == "f32" else 2
    full = cfg.rows * cfg.n_tables * cfg.w * elem
    if mem_available_bytes is None or full <= 0.6 * mem_available_bytes:
        return cfg.rows
    f = 0.6 * mem_available_bytes / full
    return next_prime(int(cfg.rows * f))


OFFLOAD_HOST_GB = 48.0   # cap on pinned host table bytes (the GPU's system-memory aperture is shared)


def offload_table_rows(cfg: Config, mem_available_bytes: Optional[int], hbm_free_bytes: Optional[int],
                       host_gb: float = OFFLOAD_HOST_GB) -> int:
    """Rows per table of the offload workload as it is measured: the full size
    (offload_rows), capped at host_gb of pinned host memory and at 80 % of free HBM (the
    HBM-resident copy it is compared with must fit too); a prime each time it is cut."""
    rows = offload_rows(cfg, mem_available_bytes)
    row_bytes = cfg.w * (4 if cfg.dtype == "f32" else 2)
    cap_rows = int(host_gb * 1e9 / (cfg.n_tables * row_bytes))
    if rows > cap_rows:
        rows = next_prime(cap_rows)
    if hbm_free_bytes is not None and cfg.n_tables * rows * row_bytes > 0.8 * hbm_free_bytes:
        rows = next_prime(int(0.8 * hbm_free_bytes / (cfg.n_tables * row_bytes)))
    return rows


def mem_available_bytes() -> Optional[int]:
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return None


def device_inputs(cfg: Config, device, tables: bool = True, table_rows_override: Optional[int] = None):
    """All inputs of one configuration, generated directly on ``device``.

    Returns a dict: raw ids [batch, seq(+decode)] int32, map int32[vocab],
    mult (numpy uint64), rows (numpy uint32, per table), tables (list of
    [rows, w] tensors, omitted when tables=False), h / wk / wv / gq / gk (lists
    per branch).  Hidden states cover the batch * seq prefill tokens.
    """
    import torch
    dt = torch_dtype(cfg)
    nrows = table_rows_override or cfg.rows
    out = {
        "raw": torch.from_numpy(raw_ids(cfg)).to(device),
        "map": torch.from_numpy(comp_map(cfg)).to(device),
        "mult": multipliers(cfg),
        "rows": np.full(cfg.n_tables, nrows, dtype=np.uint32),
    }
    if tables:
        tabs = []
        for b in range(cfg.n_tables):
            t = torch.empty((nrows, cfg.w), dtype=dt, device=device)
            tabs.append(fill_table(cfg, b, t))
        out["tables"] = tabs
    out["h"], out["wk"], out["wv"], out["gq"], out["gk"] = [], [], [], [], []
    for m in range(cfg.n_branch):
        h = torch.empty((cfg.tokens, cfg.d_model), dtype=dt, device=device)
        out["h"].append(fill_hidden(cfg, m, h))
        wk, wv = weights(cfg, m, device)
        gq, gk = gains(cfg, m, device)
        out["wk"].append(wk)
        out["wv"].append(wv)
        out["gq"].append(gq)
        out["gk"].append(gk)
    return out

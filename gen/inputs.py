"""Seeded input recipes for the five PLE workloads.

Workload shapes follow the PLE n-gram table as the pages describe it:
width 2560 (hidden size, kipfel.ltd "Qwen3.8-Flash-Next-Uncensored in NVIDIA
Jetson AGX Thor", section 2 model spec), vocabulary 248,320 (same table),
an FP8 table of 51,200,245,760 bytes (bittide model-card copy, "what this
model is") = 20,000,096 rows of 2560 bytes.

Everything here is integer/bit plumbing or plain sampling; none of it is the
PLE method. bf16 rounding of sampled values is done by torch on the CPU.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

D = 2560                 # row width = hidden size
VOCAB = 248_320          # tokenizer vocabulary
R_FULL = 20_000_096      # rows of the full FP8 table (51,200,245,760 B / 2560)
R_TINY = 65_536          # rows of the tiny table
TABLE_SEED = 0x504C45    # seed of the FP8 table generator
WEIGHT_SEED = 0x57454947  # seed of W and conv_w (shared by every workload)
CONFIG_SEED_BASE = 1234  # workload k draws from PCG64(1234 + k)
ZIPF_S = 1.1

CONFIG_NAMES = ("tiny", "decode", "prefill", "ragged", "long")


# ----------------------------------------------------------------------------
# Samplers
# ----------------------------------------------------------------------------

_zipf_cdf_cache: dict = {}


def _zipf_cdf(vocab: int, s: float) -> np.ndarray:
    key = (vocab, s)
    if key not in _zipf_cdf_cache:
        ranks = np.arange(1, vocab + 1, dtype=np.float64)
        w = ranks ** (-s)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        _zipf_cdf_cache[key] = cdf
    return _zipf_cdf_cache[key]


def zipf_tokens(rng: np.random.Generator, n: int, vocab: int = VOCAB,
                s: float = ZIPF_S) -> np.ndarray:
    """Truncated Zipf: P(rank r) proportional to r**-s for r = 1..vocab,
    token id = r - 1, drawn by inverse CDF (numpy's zipf is unbounded)."""
    cdf = _zipf_cdf(vocab, s)
    u = rng.random(n)
    r = np.searchsorted(cdf, u, side="right")
    return np.minimum(r, vocab - 1).astype(np.int32)


def uniform_tokens(rng: np.random.Generator, n: int, vocab: int = VOCAB) -> np.ndarray:
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def long_context_tokens(rng: np.random.Generator, n: int, vocab: int = VOCAB,
                        pool_size: int = 10_000, lo: int = 16, hi: int = 64,
                        s: float = ZIPF_S) -> np.ndarray:
    """Half uniform runs, half repeated phrases from a fixed pool.

    A fair coin picks each span: either a run of uniform tokens or a phrase
    from a pool of `pool_size` phrases (each of uniform tokens); span lengths
    are uniform on [lo, hi]. Phrases are picked by Zipf(s) over pool rank so
    that the repeated spans actually recur (uniform picks from 10,000
    phrases would almost never repeat within a 16K-token chunk).
    """
    lens = rng.integers(lo, hi + 1, size=pool_size)
    offs = np.concatenate([[0], np.cumsum(lens)])
    pool_tokens = uniform_tokens(rng, int(offs[-1]), vocab)
    pool_cdf = _zipf_cdf(pool_size, s)
    out = np.empty(n, dtype=np.int32)
    pos = 0
    while pos < n:
        if rng.random() < 0.5:
            k = int(min(np.searchsorted(pool_cdf, rng.random(), side="right"), pool_size - 1))
            span = pool_tokens[offs[k]:offs[k + 1]]
        else:
            span = uniform_tokens(rng, int(rng.integers(lo, hi + 1)), vocab)
        m = min(len(span), n - pos)
        out[pos:pos + m] = span[:m]
        pos += m
    return out


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) samples rounded to bfloat16 by torch (CPU); returned as the
    raw uint16 bit patterns."""
    import torch
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: a bf16 is the top half of an f32)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# Model weights (shared by every workload)
# ----------------------------------------------------------------------------

def weights(seed: int = WEIGHT_SEED):
    """W ~ N(0, 1/2560) bf16 [2560][2560] (out, in); conv_w ~ N(0, 0.5) bf16 [2560][4].

    The second parameter of N(., .) is read as the variance."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W = normal_bf16(rng, (D, D), std=math.sqrt(1.0 / D))
    conv_w = normal_bf16(rng, (D, 4), std=math.sqrt(0.5))
    return W, conv_w


# ----------------------------------------------------------------------------
# FP8 table generator parameters
# ----------------------------------------------------------------------------

def e4m3_magnitude_thresholds() -> np.ndarray:
    """31-bit thresholds that map a uniform u in [0, 2^31) to the E4M3FN
    magnitude code of a half-normal sample, rounded to nearest.

    The E4M3FN value grid is read from torch's float8_e4m3fn type. Threshold
    k sits at the midpoint between magnitude codes k and k+1 (k = 0..125);
    the magnitude code of u is the number of thresholds <= u. P(|Z| <= x) =
    erf(x / sqrt 2) for a standard normal Z.
    """
    import torch
    grid = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = 0.5 * (grid[:-1] + grid[1:])
    thr = np.array([math.floor(math.erf(m / math.sqrt(2.0)) * 2.0 ** 31 + 0.5) for m in mids],
                   dtype=np.uint64)
    thr = np.minimum(thr, 2 ** 31).astype(np.uint32)
    assert thr.shape == (126,) and np.all(np.diff(thr.astype(np.int64)) >= 0)
    return thr


# NVFP4 table (E2M1 codes, one E4M3 scale per 16 elements, the fp32 row scale):
# the E2M1 magnitude grid of the OCP Microscaling formats (v1.0, FP4 E2M1),
# codes drawn for |Z| * 2, Z ~ N(0,1); block scales uniform over the E4M3
# codes 0x28 .. 0x47 (0.25 .. 3.75)
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
NVFP4_BLOCK_CODE_LO = 0x28
NVFP4_BLOCK_CODES = 32


def e2m1_magnitude_thresholds() -> np.ndarray:
    """7 31-bit thresholds mapping a uniform u in [0, 2^31) to the E2M1
    magnitude code of |Z| * 2 rounded to nearest (the number of thresholds
    <= u); threshold k sits at the midpoint of grid values k, k+1."""
    mids = [0.5 * (E2M1_GRID[k] + E2M1_GRID[k + 1]) / 2.0 for k in range(7)]   # in units of |Z|
    thr = np.array([math.floor(math.erf(m / math.sqrt(2.0)) * 2.0 ** 31 + 0.5) for m in mids], dtype=np.uint64)
    thr = np.minimum(thr, 2 ** 31).astype(np.uint32)
    assert np.all(np.diff(thr.astype(np.int64)) > 0)
    return thr


SCALE_M_LO = 83_887      # scale = m * 2^-23, m in [83887, 838861): [0.0100001, 0.0999999]
SCALE_M_SPAN = 838_861 - 83_887


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    seed: int
    R: int
    # Each chunk: (tokens int32[T], cu_seqlens int32[S+1]). Hidden states are
    # drawn per chunk by `hidden(i)` so that long runs never hold them all.
    chunks: list = field(default_factory=list)
    S: int = 1
    fresh_state: bool = True
    # decode: per-sequence history run through the path before the timed steps
    history: list = field(default_factory=list)

    def hidden(self, i: int, T: int | None = None) -> np.ndarray:
        """bf16 bits [T][2560] of chunk i, N(0,1), from PCG64([seed, 1 + i])."""
        if T is None:
            T = len(self.chunks[i][0])
        rng = np.random.Generator(np.random.PCG64([self.seed, 1 + i]))
        return normal_bf16(rng, (T, D))

    def history_hidden(self, T: int) -> np.ndarray:
        rng = np.random.Generator(np.random.PCG64([self.seed, 0x4849]))
        return normal_bf16(rng, (T, D))

    @property
    def total_tokens(self) -> int:
        return int(sum(len(c[0]) for c in self.chunks))


def _cu(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def make_workload(name: str, decode_steps: int = 64, long_chunks: int = 16) -> Workload:
    """The five synthetic workloads (seeded PCG64(1234 + k))."""
    k = CONFIG_NAMES.index(name)
    seed = CONFIG_SEED_BASE + k
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "tiny":
        toks = uniform_tokens(rng, 128)
        return Workload(name, seed, R_TINY, [(toks, _cu([128]))], S=1)
    if name == "decode":
        S, hist = 8, 4096
        history = zipf_tokens(rng, S * hist).reshape(S, hist)
        steps = []
        for _ in range(decode_steps):
            steps.append((zipf_tokens(rng, S), _cu([1] * S)))
        w = Workload(name, seed, R_FULL, steps, S=S, fresh_state=False)
        w.history = [history]
        return w
    if name == "prefill":
        toks = zipf_tokens(rng, 32_768)
        return Workload(name, seed, R_FULL, [(toks, _cu([32_768]))], S=1)
    if name == "ragged":
        toks = uniform_tokens(rng, 64 * 256)
        return Workload(name, seed, R_FULL, [(toks, _cu([256] * 64))], S=64)
    if name == "long":
        chunk = 16_384
        toks = long_context_tokens(rng, chunk * long_chunks)
        chunks = [(toks[i * chunk:(i + 1) * chunk].copy(), _cu([chunk]))
                  for i in range(long_chunks)]
        return Workload(name, seed, R_FULL, chunks, S=1)
    raise ValueError(name)

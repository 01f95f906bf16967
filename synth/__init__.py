"""Seeded synthetic KV-cache inputs (data only; no codec arithmetic).

The CacheGen page measures its codec on long-context Mistral-7B, Llama-34B and
Llama-70B fine-tunes over LongChat / TriviaQA / NarrativeQA / WikiText
(CacheGen wiki page, "实验与结果" setup paragraph), and motivates long contexts
with an ~80K-token document (same page, "问题与动机").  Neither the weights nor
the datasets are available here, so this module stands in for them with an
AR(1) process per (layer, K/V, channel), shaped like those models' KV caches.
The token-wise locality it has is the property the codec exploits (same page,
"关键观察", observation 1: neighbouring tokens' K/V values are close).

The configurations (shapes, chunking, level schedule) are defined here once
and used by the oracle's tests, the GPU tests and the benchmark alike.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvsynth.c")
_LIB = os.path.join(_HERE, "libkvsynth.so")

SEED_BASE = 0x4B5643  # data seed of configuration k is SEED_BASE + k
PROFILE_SEED_STRIDE = 1000  # profiling chunk p uses data seed + 1000 * (p + 1)
LEVEL_SEED_OFFSET = 100  # level schedule seed = SEED_BASE + 100 + k

CHUNK_TOKENS = 1500
GROUP_TOKENS = 10
ANCHOR_BITS = 8
CDF_PREC_BITS = 15
LEVEL_BITS = ((6, 5, 4), (5, 4, 3), (4, 3, 2))  # delta bits per layer third
N_PROFILE_CHUNKS = 3


@dataclasses.dataclass(frozen=True)
class Config:
    seed_index: int  # offset of this workload's seeds from SEED_BASE
    name: str
    n_layers: int
    n_channels: int  # per K and per V: kv_heads * head_dim
    n_tokens: int
    rho_mode: int  # 0: constant rho_lo, 1: U(rho_lo, rho_hi) per channel
    rho_lo: float
    rho_hi: float
    outlier_frac: float
    outlier_scale: float
    n_levels: int  # levels encoded into the tables/profile
    schedule: str  # "level0", "level1", "mixed"
    describe: str

    @property
    def seed(self) -> int:
        return SEED_BASE + self.seed_index

    @property
    def n_chunks(self) -> int:
        return (self.n_tokens + CHUNK_TOKENS - 1) // CHUNK_TOKENS

    @property
    def n_streams_per_chunk(self) -> int:
        return 2 * self.n_layers * self.n_channels

    @property
    def delta_bits(self):
        return LEVEL_BITS[: self.n_levels]

    def chunk_levels(self) -> List[int]:
        if self.schedule == "level0":
            return [0] * self.n_chunks
        if self.schedule == "level1":
            return [1] * self.n_chunks
        if self.schedule == "mixed":
            return levels_sequence(SEED_BASE + LEVEL_SEED_OFFSET + self.seed_index,
                                   self.n_chunks, self.n_levels)
        raise ValueError(self.schedule)

    def chunk_tokens(self, k: int) -> int:
        return min(CHUNK_TOKENS, self.n_tokens - k * CHUNK_TOKENS)

    def fp16_bytes(self) -> int:
        return 2 * self.n_layers * self.n_channels * self.n_tokens * 2


TINY = Config(0, "tiny-4L-512ch-1.5K", 4, 512, 1500, 0, 0.9, 0.9, 0.0, 8.0, 1,
              "level0", "4 layers, 8 heads x 64, one 1,500-token chunk, no outliers")
SHAPE_7B_9K = Config(1, "llama2-7b-shape-9K", 32, 4096, 9000, 0, 0.9, 0.9, 0.01, 8.0, 1,
                     "level0", "32 layers, 32 heads x 128, 6 chunks of 1,500 tokens")
SHAPE_13B_16K = Config(2, "llama2-13b-shape-16K", 40, 5120, 16000, 0, 0.9, 0.9, 0.01, 8.0, 3,
                       "level1",
                       "40 layers, 40 heads x 128, 16,000 tokens, 3 levels, decode the middle one")
SHAPE_34B_GQA_80K = Config(3, "34b-gqa-shape-80K", 48, 1024, 80000, 1, 0.8, 0.97, 0.01, 8.0, 1,
                           "level0", "48 layers, 8 KV heads x 128, 80,000 tokens, rho ~ U(0.8, 0.97)")
SHAPE_70B_GQA_16K = Config(4, "llama-70b-gqa-shape-16K", 80, 1024, 16000, 0, 0.9, 0.9, 0.01, 8.0, 3,
                           "mixed", "80 layers, 8 KV heads x 128, 16,000 tokens, seeded mixed levels")
# the workloads by name
WORKLOADS = {w.name: w for w in (TINY, SHAPE_7B_9K, SHAPE_13B_16K, SHAPE_34B_GQA_80K,
                                 SHAPE_70B_GQA_16K)}


def small_config(n_layers: int, n_channels: int, n_tokens: int, n_levels: int = 3,
                 schedule: str = "mixed", seed_index: int = 90, rho_mode: int = 0,
                 outlier_frac: float = 0.01, rho: Optional[float] = None) -> Config:
    """A reduced configuration with the same value model, for quick tests
    (`rho` overrides the constant AR(1) coefficient, e.g. 0 for white noise)."""
    lo = 0.8 if rho_mode else (0.9 if rho is None else rho)
    hi = 0.97 if rho_mode else lo
    return Config(seed_index, f"small-{n_layers}L-{n_channels}ch-{n_tokens}", n_layers,
                  n_channels, n_tokens, rho_mode, lo, hi, outlier_frac, 8.0, n_levels, schedule,
                  "reduced test configuration")


# --------------------------------------------------------------------------
# native generator


def _build() -> None:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", _SRC, "-o",
           _LIB + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)


def build() -> None:
    _build()


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        _build()
    lib = ctypes.CDLL(_LIB)
    u32, u64, dp, vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p
    lib.kvs_philox4x32_10.argtypes = [vp, vp, vp]
    lib.kvs_params.argtypes = [u64, u32, u32, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                               ctypes.c_double, ctypes.c_double, dp, dp, dp, vp]
    lib.kvs_generate.argtypes = [u64, u32, u32, u32, u32, dp, dp, dp, vp]
    lib.kvs_innovations.argtypes = [u64, u32, u32, u32, dp]
    lib.kvs_levels.argtypes = [u64, u32, u32, vp]
    lib.kvs_to_half.argtypes = [ctypes.c_double]
    lib.kvs_to_half.restype = ctypes.c_uint16
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def philox4x32_10(ctr: Sequence[int], key: Sequence[int]) -> List[int]:
    lib = _load()
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    lib.kvs_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return [int(x) for x in o]


def levels_sequence(seed: int, n_chunks: int, n_levels: int) -> List[int]:
    lib = _load()
    out = np.zeros(max(n_chunks, 1), dtype=np.uint8)
    lib.kvs_levels(seed, n_chunks, n_levels, _ptr(out))
    return [int(x) for x in out[:n_chunks]]


@dataclasses.dataclass
class Params:
    mu: np.ndarray
    s: np.ndarray
    rho: np.ndarray
    is_outlier: np.ndarray


def params(cfg: Config) -> Params:
    lib = _load()
    S = 2 * cfg.n_layers * cfg.n_channels
    mu = np.zeros(S, np.float64)
    s = np.zeros(S, np.float64)
    rho = np.zeros(S, np.float64)
    out = np.zeros(S, np.uint8)
    lib.kvs_params(cfg.seed, cfg.n_layers, cfg.n_channels, cfg.rho_mode, cfg.rho_lo, cfg.rho_hi,
                   cfg.outlier_frac, cfg.outlier_scale, _ptr(mu), _ptr(s), _ptr(rho), _ptr(out))
    return Params(mu, s, rho, out)


def _generate(cfg: Config, innov_seed: int, n_tokens: int, layers: Optional[range],
              p: Optional[Params]) -> np.ndarray:
    lib = _load()
    if p is None:
        p = params(cfg)
    if layers is None:
        layers = range(cfg.n_layers)
    row0, row1 = 2 * layers.start, 2 * layers.stop
    out = np.empty((len(layers), 2, n_tokens, cfg.n_channels), dtype=np.uint16)
    lib.kvs_generate(innov_seed, cfg.n_channels, n_tokens, row0, row1, _ptr(p.mu), _ptr(p.s),
                     _ptr(p.rho), _ptr(out))
    return out


def make_kv(cfg: Config, layers: Optional[range] = None, p: Optional[Params] = None,
            n_tokens: Optional[int] = None) -> np.ndarray:
    """The context's KV cache: binary16 bit patterns, shape [L][2][T][C]."""
    return _generate(cfg, cfg.seed, cfg.n_tokens if n_tokens is None else n_tokens, layers, p)


def make_profile_kv(cfg: Config, layers: Optional[range] = None,
                    p: Optional[Params] = None) -> np.ndarray:
    """Profiling data: N_PROFILE_CHUNKS chunks of CHUNK_TOKENS tokens from the same
    processes (same mu, s, rho, outliers) with fresh innovations, concatenated
    along tokens: shape [L][2][3*1500][C]."""
    if p is None:
        p = params(cfg)
    parts = [_generate(cfg, cfg.seed + PROFILE_SEED_STRIDE * (i + 1), CHUNK_TOKENS, layers, p)
             for i in range(N_PROFILE_CHUNKS)]
    return np.ascontiguousarray(np.concatenate(parts, axis=2))


def innovations(seed: int, m0: int, count: int, n_tokens: int) -> np.ndarray:
    lib = _load()
    e = np.zeros((count, n_tokens), np.float64)
    lib.kvs_innovations(seed, m0, count, n_tokens, _ptr(e))
    return e


def to_half_bits(v: float) -> int:
    return int(_load().kvs_to_half(float(v)))


def bandwidth_trace(seed: int, median_bytes_per_s: float, sigma: float = 0.7,
                    n_pieces: int = 128, min_s: float = 0.05,
                    max_s: float = 0.4) -> List[tuple]:
    """A seeded piecewise-constant link: pieces of U(min_s, max_s) seconds
    at median * exp(sigma * N(0, 1)) bytes per second, the first at time 0
    (the CacheGen page evaluates its streaming adaptation on random bandwidth
    traces without describing them; this is a log-normal stand-in).
    Returns [(start_s, bytes_per_s), ...]."""
    rng = np.random.default_rng(seed)
    durations = rng.uniform(min_s, max_s, n_pieces - 1)
    starts = np.concatenate([[0.0], np.cumsum(durations)])
    rates = median_bytes_per_s * np.exp(sigma * rng.standard_normal(n_pieces))
    return [(float(a), float(b)) for a, b in zip(starts, rates)]

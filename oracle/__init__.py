"""CPU oracle for the CacheGen-style KV-cache codec -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package entry's smoke check and the benchmark's CPU
baseline leg import this module.  The product (the HIP library and its
binding) never does, and this module never imports the product.

The arithmetic lives in ``kvc_oracle.c`` (plain scalar C, one stream at a
time, OpenMP only across independent streams).  This wrapper only marshals
numpy arrays.  Every function cites the part of the CacheGen wiki page's
"核心方法" (core method) section that it follows, or the reading taken where
the page is silent.

Parity status: every exported function has at least one pin in
``tests/test_oracle_*.py`` (closed forms, brute force, page-fixed invariants,
library routines).  Nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_kvc.so")

OK, ERR_ARG, ERR_SHAPE, ERR_PROFILE, ERR_CORRUPT, ERR_NONFINITE, ERR_CAPACITY = 0, -1, -2, -3, -4, -5, -6
PREC = 15
TOT = 1 << PREC
ANCHOR_ALPHA = 256
DELTA_STRIDE = 64
HDR_BYTES = 64
REC_BYTES = 16


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


@dataclasses.dataclass(frozen=True)
class Desc:
    """Codec parameters (the page's constants: ~1.5K-token chunks, groups of
    10 tokens, 8-bit anchors, three layer groups with coarser deltas deeper)."""
    n_layers: int
    n_channels: int
    group_tokens: int = 10
    chunk_tokens: int = 1500
    anchor_bits: int = 8
    delta_bits: Tuple[Tuple[int, int, int], ...] = ((6, 5, 4),)
    cdf_prec_bits: int = 15

    @property
    def n_levels(self) -> int:
        return len(self.delta_bits)

    @property
    def n_streams(self) -> int:
        return 2 * self.n_layers * self.n_channels

    def words(self) -> np.ndarray:
        w = [self.n_layers, self.n_channels, self.group_tokens, self.chunk_tokens,
             self.anchor_bits, self.n_levels, self.cdf_prec_bits]
        bits = [0] * 12
        for i, row in enumerate(self.delta_bits):
            for j in range(3):
                bits[3 * i + j] = row[j]
        return np.asarray(w + bits, dtype=np.uint32)

    def third(self, layer: int) -> int:
        return (3 * layer) // self.n_layers

    def bits(self, level: int, layer: int) -> int:
        return self.delta_bits[level][self.third(layer)]


def desc_for(cfg) -> Desc:
    """Oracle descriptor for a ``synth.Config``."""
    return Desc(cfg.n_layers, cfg.n_channels, 10, 1500, 8, tuple(tuple(r) for r in cfg.delta_bits), 15)


# --------------------------------------------------------------------------
def build() -> None:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    vp, u32, u64, i64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64
    lib.orc_h2f.argtypes = [ctypes.c_uint16]
    lib.orc_h2f.restype = ctypes.c_float
    lib.orc_f2h.argtypes = [ctypes.c_float]
    lib.orc_f2h.restype = ctypes.c_uint16
    lib.orc_fnv1a64.argtypes = [vp, u64, u64]
    lib.orc_fnv1a64.restype = u64
    lib.orc_quantize.argtypes = [vp, u32, u32, u32, vp, vp, vp, vp]
    lib.orc_dequantize.argtypes = [vp, u32, u32, u32, ctypes.c_float, ctypes.c_float,
                                   ctypes.c_float, vp]
    lib.orc_normalize.argtypes = [vp, u32, vp]
    lib.orc_rc_encode.argtypes = [vp, u32, u32, vp, u32, vp, u32, vp, u64]
    lib.orc_rc_encode.restype = i64
    lib.orc_rc_decode.argtypes = [vp, u64, u32, u32, vp, u32, vp, u32, vp]
    lib.orc_profile_id.argtypes = [vp, vp, vp]
    lib.orc_profile_id.restype = u64
    lib.orc_profile.argtypes = [vp, vp, u32, vp, vp, vp]
    lib.orc_container_bound.argtypes = [vp, u32]
    lib.orc_container_bound.restype = u64
    lib.orc_encode_chunk.argtypes = [vp, vp, vp, u64, vp, u32, u32, u32, vp, u64]
    lib.orc_encode_chunk.restype = i64
    lib.orc_stream_offsets.argtypes = [vp, vp, u64, vp]
    lib.orc_decode_chunk.argtypes = [vp, vp, vp, u64, vp, u64, u32, u32, u32, vp, u32]
    lib.orc_decode_streams.argtypes = [vp, vp, vp, u64, vp, u64, vp, u32, vp, vp]
    lib.orc_unit_order.argtypes = [vp, vp, vp, u64, vp, u64, u32, vp, u64, vp]
    lib.orc_block_order_trace.argtypes = [u32, u32, u32, vp, vp, vp, u64]
    lib.orc_block_order_trace.restype = i64
    lib.orc_rc_shifts.argtypes = [vp, u64, u32, u32, vp, u32, vp, u32, vp]
    lib.orc_f2h_array.argtypes = [vp, vp, u64]
    lib.orc_h2f_array.argtypes = [vp, vp, u64]
    lib.orc_f2h_patterns.argtypes = [u32, u64, vp]
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_get_threads.restype = ctypes.c_int
    lib.orc_refine_quantize.argtypes = [vp, u32, u32, u32, u32, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_refine_dequantize.argtypes = [vp, vp, u32, u32, u32, u32, ctypes.c_float,
                                          ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_float, vp]
    lib.orc_refine_profile_id.argtypes = [vp, u32, u64, vp, vp]
    lib.orc_refine_profile_id.restype = u64
    lib.orc_profile_refine.argtypes = [vp, vp, u32, u32, u64, vp, vp, vp]
    lib.orc_encode_refine_chunk.argtypes = [vp, vp, vp, u64, u64, u32, vp, u32, u32, u32, vp, u64]
    lib.orc_encode_refine_chunk.restype = i64
    lib.orc_decode_refined_chunk.argtypes = [vp, vp, vp, u64, vp, u64, vp, vp, u64, vp, u64,
                                             u32, u32, u32, vp, u32]
    lib.orc_decode_refine_symbols.argtypes = [vp, vp, vp, u64, u64, vp, u64, vp, u32, vp]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


# ------------------------------------------------------------- primitives
def h2f(bits: int) -> float:
    """Exact binary16 -> binary32 widening (the stream's input values)."""
    return float(_load().orc_h2f(int(bits)))


def f2h(x: float) -> int:
    """binary32 -> binary16, round to nearest even (the decoder's store)."""
    return int(_load().orc_f2h(ctypes.c_float(x)))


def f2h_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32).ravel()
    out = np.zeros(len(x), np.uint16)
    _load().orc_f2h_array(_p(x), _p(out), len(x))
    return out


def f2h_patterns(start: int, n: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    """f2h of the binary32 bit patterns start .. start+n-1."""
    if out is None:
        out = np.zeros(n, np.uint16)
    _load().orc_f2h_patterns(start, n, _p(out))
    return out


def h2f_array(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, np.uint16).ravel()
    out = np.zeros(len(h), np.float32)
    _load().orc_h2f_array(_p(h), _p(out), len(h))
    return out


def fnv1a64(data: bytes, h: int = 0xcbf29ce484222325) -> int:
    buf = np.frombuffer(data, np.uint8) if len(data) else np.zeros(1, np.uint8)
    return int(_load().orc_fnv1a64(_p(buf), len(data), h))


def quantize(x: np.ndarray, group: int, dbits: int):
    """Change-based encoding + layer-wise quantization of one stream (CacheGen
    page, "核心方法" steps 1-2): returns (lo, sa, dl, symbols)."""
    x = np.ascontiguousarray(x, np.float32)
    n = len(x)
    sym = np.zeros(max(n, 1), np.int32)
    lo, sa, dl = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    st = _load().orc_quantize(_p(x), n, group, dbits, ctypes.byref(lo), ctypes.byref(sa),
                              ctypes.byref(dl), _p(sym))
    if st:
        raise OracleError(st, "quantize")
    return np.float32(lo.value), np.float32(sa.value), np.float32(dl.value), sym[:n]


def dequantize(sym: np.ndarray, group: int, dbits: int, lo, sa, dl) -> np.ndarray:
    sym = np.ascontiguousarray(sym, np.int32)
    out = np.zeros(max(len(sym), 1), np.uint16)
    _load().orc_dequantize(_p(sym), len(sym), group, dbits, ctypes.c_float(lo),
                           ctypes.c_float(sa), ctypes.c_float(dl), _p(out))
    return out[: len(sym)]


def normalize(counts: Sequence[int]) -> np.ndarray:
    """Profiled counts -> frequencies summing to 2^15 (reading R5)."""
    c = np.ascontiguousarray(counts, np.uint64)
    f = np.zeros(len(c), np.uint32)
    _load().orc_normalize(_p(c), len(c), _p(f))
    return f


def rc_encode(sym: Sequence[int], fA: Sequence[int], fD: Optional[Sequence[int]] = None,
              group: int = 1) -> bytes:
    """Range-encode (reading R4).  With group=1 every symbol uses model fA."""
    s = np.ascontiguousarray(sym, np.int32)
    a = np.ascontiguousarray(fA, np.uint32)
    d = np.ascontiguousarray(fA if fD is None else fD, np.uint32)
    cap = 4 + 2 * len(s) + 16
    out = np.zeros(cap, np.uint8)
    n = _load().orc_rc_encode(_p(s) if len(s) else None, len(s), group, _p(a), len(a), _p(d),
                              len(d), _p(out), cap)
    if n < 0:
        raise OracleError(int(n), "rc_encode")
    return out[:n].tobytes()


def rc_decode(data: bytes, n: int, fA: Sequence[int], fD: Optional[Sequence[int]] = None,
              group: int = 1) -> np.ndarray:
    buf = np.frombuffer(data, np.uint8).copy() if len(data) else np.zeros(1, np.uint8)
    a = np.ascontiguousarray(fA, np.uint32)
    d = np.ascontiguousarray(fA if fD is None else fD, np.uint32)
    sym = np.zeros(max(n, 1), np.int32)
    st = _load().orc_rc_decode(_p(buf), len(data), n, group, _p(a), len(a), _p(d), len(d), _p(sym))
    if st:
        raise OracleError(st, "rc_decode")
    return sym[:n]


def rc_shifts(data: bytes, n: int, fA: Sequence[int], fD: Optional[Sequence[int]] = None,
              group: int = 1) -> np.ndarray:
    """Bytes shifted in by each decoded symbol (0..2): the decoder's
    consumption trace that the reference reader of reading R17 follows."""
    buf = np.frombuffer(data, np.uint8).copy() if len(data) else np.zeros(1, np.uint8)
    a = np.ascontiguousarray(fA, np.uint32)
    d = np.ascontiguousarray(fA if fD is None else fD, np.uint32)
    k = np.zeros(max(n, 1), np.uint8)
    st = _load().orc_rc_shifts(_p(buf), len(data), n, group, _p(a), len(a), _p(d), len(d), _p(k))
    if st:
        raise OracleError(st, "rc_shifts")
    return k[:n]


def block_order_trace(nblk: Sequence[int], shifts: np.ndarray, group: int) -> np.ndarray:
    """Reading R17 on an explicit trace: slot order (lane << 16 | block) of a
    unit whose lanes have nblk[l] blocks and shift counts shifts[l][j]."""
    nb = np.ascontiguousarray(nblk, np.uint32)
    k = np.ascontiguousarray(shifts, np.uint8)
    nv, n = k.shape
    cap = int(nb.sum()) + 1
    order = np.zeros(cap, np.uint32)
    r = _load().orc_block_order_trace(nv, n, group, _p(nb), _p(k), _p(order), cap)
    if r < 0:
        raise OracleError(int(r), "block_order_trace")
    return order[:r]


# -------------------------------------------------------------- the codec
@dataclasses.dataclass
class Tables:
    """Profiled models: fA[m][256], fD[level][m][64] (u16), and their id."""
    fA: np.ndarray
    fD: np.ndarray
    profile_id: int


def profile(desc: Desc, kv_prof: np.ndarray) -> Tables:
    """Offline profiling per channel-layer combination, anchors and deltas
    separately (CacheGen page, "核心方法" step 3; reading R5)."""
    kv = np.ascontiguousarray(kv_prof, np.uint16)
    L, two, T, C = kv.shape
    assert (L, two, C) == (desc.n_layers, 2, desc.n_channels)
    S = desc.n_streams
    fA = np.zeros((S, ANCHOR_ALPHA), np.uint16)
    fD = np.zeros((desc.n_levels, S, DELTA_STRIDE), np.uint16)
    pid = ctypes.c_uint64()
    w = desc.words()
    st = _load().orc_profile(_p(w), _p(kv), T, _p(fA), _p(fD), ctypes.byref(pid))
    if st:
        raise OracleError(st, "profile")
    return Tables(fA, fD, int(pid.value))


def profile_id(desc: Desc, fA: np.ndarray, fD: np.ndarray) -> int:
    w = desc.words()
    return int(_load().orc_profile_id(_p(w), _p(np.ascontiguousarray(fA, np.uint16)),
                                      _p(np.ascontiguousarray(fD, np.uint16))))


def encode_chunk(desc: Desc, tables: Tables, kv: np.ndarray, chunk: int, level: int) -> np.ndarray:
    """One container for tokens [chunk*chunk_tokens, ...) at `level`."""
    kv = np.ascontiguousarray(kv, np.uint16)
    T = kv.shape[2]
    w = desc.words()
    n = min(desc.chunk_tokens, T - chunk * desc.chunk_tokens)
    cap = int(_load().orc_container_bound(_p(w), n))
    out = np.zeros(cap, np.uint8)
    r = _load().orc_encode_chunk(_p(w), _p(tables.fA), _p(tables.fD), tables.profile_id, _p(kv),
                                 T, chunk, level, _p(out), cap)
    if r < 0:
        raise OracleError(int(r), "encode_chunk")
    return out[:r].copy()


def encode(desc: Desc, tables: Tables, kv: np.ndarray, levels: Sequence[int]) -> List[np.ndarray]:
    """Encode every chunk of kv [L][2][T][C] at its level (one container each)."""
    T = kv.shape[2]
    nch = (T + desc.chunk_tokens - 1) // desc.chunk_tokens
    assert len(levels) == nch
    return [encode_chunk(desc, tables, kv, k, int(levels[k])) for k in range(nch)]


def container_bound(desc: Desc, n_tokens: int) -> int:
    return int(_load().orc_container_bound(_p(desc.words()), n_tokens))


def stream_offsets(desc: Desc, container: np.ndarray) -> np.ndarray:
    offs = np.zeros(desc.n_streams, np.uint32)
    st = _load().orc_stream_offsets(_p(desc.words()), _p(container), len(container), _p(offs))
    if st:
        raise OracleError(st, "stream_offsets")
    return offs


def decode_chunk_into(desc: Desc, tables: Tables, container: np.ndarray, first_token: int,
                      n_tokens: int, level: int, out: np.ndarray) -> None:
    """Decode one container into out [L][2][T_total][C] (binary16 bits)."""
    assert out.dtype == np.uint16 and out.flags.c_contiguous
    st = _load().orc_decode_chunk(_p(desc.words()), _p(tables.fA), _p(tables.fD),
                                  tables.profile_id, _p(container), len(container), first_token,
                                  n_tokens, level, _p(out), out.shape[2])
    if st:
        raise OracleError(st, "decode_chunk")


def decode(desc: Desc, tables: Tables, containers: Sequence[np.ndarray], levels: Sequence[int],
           T_total: int) -> np.ndarray:
    out = np.zeros((desc.n_layers, 2, T_total, desc.n_channels), np.uint16)
    for k, c in enumerate(containers):
        n = min(desc.chunk_tokens, T_total - k * desc.chunk_tokens)
        decode_chunk_into(desc, tables, c, k * desc.chunk_tokens, n, int(levels[k]), out)
    return out


def decode_streams(desc: Desc, tables: Tables, container: np.ndarray, ids: Sequence[int],
                   n_tokens: int):
    """Decode selected streams of one container: (values [k][n] u16, symbols)."""
    ids = np.ascontiguousarray(ids, np.uint32)
    vals = np.zeros((len(ids), n_tokens), np.uint16)
    syms = np.zeros((len(ids), n_tokens), np.int32)
    st = _load().orc_decode_streams(_p(desc.words()), _p(tables.fA), _p(tables.fD),
                                    tables.profile_id, _p(container), len(container), _p(ids),
                                    len(ids), _p(vals), _p(syms))
    if st:
        raise OracleError(st, "decode_streams")
    return vals, syms


def unit_order(desc: Desc, tables: Tables, container: np.ndarray, unit: int):
    """Slot order of one unit's payload (lane << 16 | block per slot), as the
    reference reader of reading R17 reads it, and the unit's lane count."""
    cap = 64 * (4 + 2 * desc.chunk_tokens) // 8 + 64
    order = np.zeros(cap, np.uint32)
    nv = np.zeros(1, np.uint32)
    st = _load().orc_unit_order(_p(desc.words()), _p(tables.fA), _p(tables.fD),
                                tables.profile_id, _p(container), len(container), unit,
                                _p(order), cap, _p(nv))
    if st:
        raise OracleError(st, "unit_order")
    m0, n_lanes = unit_streams(desc, unit)
    nb = records(desc, container)["nbytes"][m0:m0 + n_lanes].astype(np.int64)
    return order[:int(((nb + 7) // 8).sum())], int(nv[0])


def n_units(desc: Desc) -> int:
    return 2 * desc.n_layers * ((desc.n_channels + 63) // 64)


def unit_streams(desc: Desc, unit: int) -> Tuple[int, int]:
    """First stream and stream count of a unit (reading R6)."""
    ncb = (desc.n_channels + 63) // 64
    row, cb = divmod(unit, ncb)
    return row * desc.n_channels + 64 * cb, min(64, desc.n_channels - 64 * cb)


# ------------------------------------------------------ container parsing
def parse_header(container: np.ndarray) -> dict:
    b = bytes(container[:HDR_BYTES])
    le = lambda o, n: int.from_bytes(b[o:o + n], "little")
    return {
        "magic": b[0:4], "version": le(4, 2), "level": b[6], "anchor_bits": b[7],
        "group_tokens": le(8, 2), "cdf_prec": b[10], "delta_bits": tuple(b[11:14]),
        "n_layers": le(16, 4), "n_channels": le(20, 4), "n_tokens": le(24, 4),
        "first_token": le(28, 4), "profile_id": le(32, 8), "payload_bytes": le(40, 8),
        "chunk_tokens": le(48, 4), "n_streams": le(52, 4),
    }


def records(desc: Desc, container: np.ndarray) -> np.ndarray:
    """Stream records as a structured array (lo, sa, dl, nbytes)."""
    dt = np.dtype([("lo", "<f4"), ("sa", "<f4"), ("dl", "<f4"), ("nbytes", "<u4")])
    S = desc.n_streams
    return np.frombuffer(container[HDR_BYTES:HDR_BYTES + REC_BYTES * S].tobytes(), dt)


# ------------------------------------------------------- refinement (R19)
def refine_quantize(x: np.ndarray, group: int, dbits: int, ebits: int):
    """Base quantization at dbits, then the refinement quantizer at ebits on
    the residual against the binary32 base reconstruction (reading R19):
    (lo, sa, dl, symbols, Da, Dd, refinement symbols)."""
    x = np.ascontiguousarray(x, np.float32)
    n = len(x)
    sym = np.zeros(max(n, 1), np.int32)
    esym = np.zeros(max(n, 1), np.int32)
    v = [ctypes.c_float() for _ in range(5)]
    st = _load().orc_refine_quantize(_p(x), n, group, dbits, ebits, *[ctypes.byref(t) for t in v[:3]],
                                     _p(sym), ctypes.byref(v[3]), ctypes.byref(v[4]), _p(esym))
    if st:
        raise OracleError(st, "refine_quantize")
    lo, sa, dl, Da, Dd = (np.float32(t.value) for t in v)
    return lo, sa, dl, sym[:n], Da, Dd, esym[:n]


def refine_dequantize(sym, esym, group: int, dbits: int, ebits: int, lo, sa, dl, Da, Dd):
    """Refined values binary16(fma(q, D, xh)) of one stream (binary16 bits)."""
    sym = np.ascontiguousarray(sym, np.int32)
    esym = np.ascontiguousarray(esym, np.int32)
    out = np.zeros(max(len(sym), 1), np.uint16)
    f = ctypes.c_float
    _load().orc_refine_dequantize(_p(sym), _p(esym), len(sym), group, dbits, ebits, f(lo), f(sa),
                                  f(dl), f(Da), f(Dd), _p(out))
    return out[: len(sym)]


@dataclasses.dataclass
class RefineTables:
    """Refinement models: fEA / fED [level][m][64] (u16; anchor tokens / the
    other tokens), their bits E, their id and the base tables' id."""
    fEA: np.ndarray
    fED: np.ndarray
    ebits: int
    refine_id: int
    base_id: int


def profile_refine(desc: Desc, kv_prof: np.ndarray, ebits: int, base_id: int) -> RefineTables:
    kv = np.ascontiguousarray(kv_prof, np.uint16)
    L, two, T, C = kv.shape
    assert (L, two, C) == (desc.n_layers, 2, desc.n_channels)
    S = desc.n_streams
    fEA = np.zeros((desc.n_levels, S, DELTA_STRIDE), np.uint16)
    fED = np.zeros((desc.n_levels, S, DELTA_STRIDE), np.uint16)
    rid = ctypes.c_uint64()
    st = _load().orc_profile_refine(_p(desc.words()), _p(kv), T, ebits, base_id, _p(fEA), _p(fED),
                                    ctypes.byref(rid))
    if st:
        raise OracleError(st, "profile_refine")
    return RefineTables(fEA, fED, ebits, int(rid.value), base_id)


def refine_profile_id(desc: Desc, rt: RefineTables) -> int:
    return int(_load().orc_refine_profile_id(_p(desc.words()), rt.ebits, rt.base_id,
                                             _p(np.ascontiguousarray(rt.fEA, np.uint16)),
                                             _p(np.ascontiguousarray(rt.fED, np.uint16))))


def encode_refine_chunk(desc: Desc, rt: RefineTables, kv: np.ndarray, chunk: int,
                        level: int) -> np.ndarray:
    """The refinement container of chunk `chunk` over its base layer at `level`."""
    kv = np.ascontiguousarray(kv, np.uint16)
    T = kv.shape[2]
    n = min(desc.chunk_tokens, T - chunk * desc.chunk_tokens)
    cap = int(_load().orc_container_bound(_p(desc.words()), n))
    out = np.zeros(cap, np.uint8)
    r = _load().orc_encode_refine_chunk(_p(desc.words()), _p(rt.fEA), _p(rt.fED), rt.refine_id,
                                        rt.base_id, rt.ebits, _p(kv), T, chunk, level, _p(out), cap)
    if r < 0:
        raise OracleError(int(r), "encode_refine_chunk")
    return out[:r].copy()


def encode_refine(desc: Desc, rt: RefineTables, kv: np.ndarray,
                  levels: Sequence[int]) -> List[np.ndarray]:
    T = kv.shape[2]
    nch = (T + desc.chunk_tokens - 1) // desc.chunk_tokens
    assert len(levels) == nch
    return [encode_refine_chunk(desc, rt, kv, k, int(levels[k])) for k in range(nch)]


def decode_refined_chunk_into(desc: Desc, tables: Tables, container: np.ndarray,
                              rt: RefineTables, rcontainer: np.ndarray, first_token: int,
                              n_tokens: int, level: int, out: np.ndarray) -> None:
    assert out.dtype == np.uint16 and out.flags.c_contiguous
    st = _load().orc_decode_refined_chunk(_p(desc.words()), _p(tables.fA), _p(tables.fD),
                                          tables.profile_id, _p(container), len(container),
                                          _p(rt.fEA), _p(rt.fED), rt.refine_id, _p(rcontainer),
                                          len(rcontainer), first_token, n_tokens, level, _p(out),
                                          out.shape[2])
    if st:
        raise OracleError(st, "decode_refined_chunk")


def decode_refined(desc: Desc, tables: Tables, containers: Sequence[np.ndarray],
                   rt: RefineTables, rcontainers: Sequence[np.ndarray], levels: Sequence[int],
                   T_total: int) -> np.ndarray:
    out = np.zeros((desc.n_layers, 2, T_total, desc.n_channels), np.uint16)
    for k, (c, rc) in enumerate(zip(containers, rcontainers)):
        n = min(desc.chunk_tokens, T_total - k * desc.chunk_tokens)
        decode_refined_chunk_into(desc, tables, c, rt, rc, k * desc.chunk_tokens, n,
                                  int(levels[k]), out)
    return out


def decode_refine_symbols(desc: Desc, rt: RefineTables, rcontainer: np.ndarray,
                          ids: Sequence[int], n_tokens: int) -> np.ndarray:
    ids = np.ascontiguousarray(ids, np.uint32)
    syms = np.zeros((len(ids), n_tokens), np.int32)
    st = _load().orc_decode_refine_symbols(_p(desc.words()), _p(rt.fEA), _p(rt.fED), rt.refine_id,
                                           rt.base_id, _p(rcontainer), len(rcontainer), _p(ids),
                                           len(ids), _p(syms))
    if st:
        raise OracleError(st, "decode_refine_symbols")
    return syms


def parse_refine_header(container: np.ndarray) -> dict:
    b = bytes(container[:HDR_BYTES])
    le = lambda o, n: int.from_bytes(b[o:o + n], "little")
    return {
        "magic": b[0:4], "version": le(4, 2), "level": b[6], "ebits": b[7],
        "group_tokens": le(8, 2), "cdf_prec": b[10], "delta_bits": tuple(b[11:14]),
        "n_layers": le(16, 4), "n_channels": le(20, 4), "n_tokens": le(24, 4),
        "first_token": le(28, 4), "refine_id": le(32, 8), "payload_bytes": le(40, 8),
        "chunk_tokens": le(48, 4), "n_streams": le(52, 4), "base_id": le(56, 8),
    }


def refine_records(desc: Desc, container: np.ndarray) -> np.ndarray:
    """Refinement stream records as a structured array (Da, Dd, nbytes)."""
    dt = np.dtype([("Da", "<f4"), ("Dd", "<f4"), ("zero", "<u4"), ("nbytes", "<u4")])
    S = desc.n_streams
    return np.frombuffer(container[HDR_BYTES:HDR_BYTES + REC_BYTES * S].tobytes(), dt)

"""MI355X-native CacheGen-style KV-cache codec: Python binding over libkvc.

The codec follows the CacheGen wiki page's method (section 核心方法): KV split
into ~1.5K-token chunks; 10-token groups with an 8-bit anchor and deltas to
it; coarser delta quantization for deeper layer thirds; arithmetic coding
against per channel-layer distributions profiled offline, anchors and deltas
separately; decode of fetched chunks back into the KV cache on the GPU.

This module only marshals arguments: torch tensors supply device memory
(``data_ptr()``) and the HIP stream (``torch.cuda.current_stream()``); every
step runs in the HIP kernels of ``libkvc.so`` behind ``include/kvc.h``.
There is no CPU fallback: if the library is missing, importing works but
every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import List, Optional, Sequence, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvc.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_SHAPE = -2
ERR_PROFILE_MISMATCH = -3
ERR_CORRUPT_STREAM = -4
ERR_NONFINITE = -5
ERR_CAPACITY = -6
ERR_HIP = -7

EXPORTED = (
    "kvc_version", "kvc_status_str", "kvc_validate_desc", "kvc_tables_bytes",
    "kvc_profile_ws_bytes", "kvc_profile", "kvc_container_bound", "kvc_encode_bound",
    "kvc_encode_ws_bytes", "kvc_encode", "kvc_decode_ws_bytes", "kvc_decode",
    "kvc_decode_index", "kvc_decode_symbols", "kvc_restore_staging_bytes", "kvc_restore",
    "kvc_plan_stream", "kvc_decode_multi", "kvc_decode_static", "kvc_refine_tables_bytes",
    "kvc_refine_profile_ws_bytes", "kvc_profile_refine", "kvc_encode_refine_ws_bytes",
    "kvc_encode_refine", "kvc_decode_refined_ws_bytes", "kvc_decode_refined",
)


class KvcError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_str(code)} ({code})")
        self.code = code


class CodecDesc(ctypes.Structure):
    """kvc_codec_desc: the page's constants (1,500-token chunks, groups of 10,
    8-bit anchors, delta bits per layer third and level, 15-bit models)."""
    _fields_ = [
        ("n_layers", ctypes.c_uint32),
        ("n_channels", ctypes.c_uint32),
        ("group_tokens", ctypes.c_uint32),
        ("chunk_tokens", ctypes.c_uint32),
        ("anchor_bits", ctypes.c_uint32),
        ("n_levels", ctypes.c_uint32),
        ("delta_bits", (ctypes.c_uint8 * 3) * 4),
        ("cdf_prec_bits", ctypes.c_uint32),
    ]

    @property
    def n_streams(self) -> int:
        return 2 * self.n_layers * self.n_channels


class ChunkRef(ctypes.Structure):
    """kvc_chunk_ref: one fetched chunk handed to the decoder."""
    _fields_ = [
        ("container", ctypes.c_void_p),
        ("container_bytes", ctypes.c_uint64),
        ("first_token", ctypes.c_uint32),
        ("n_tokens", ctypes.c_uint32),
        ("level", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class RequestChunk(ctypes.Structure):
    """kvc_request_chunk: a chunk of one of several requests, with that
    request's KV cache."""
    _fields_ = [
        ("container", ctypes.c_void_p),
        ("container_bytes", ctypes.c_uint64),
        ("first_token", ctypes.c_uint32),
        ("n_tokens", ctypes.c_uint32),
        ("level", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
        ("kv_out", ctypes.c_void_p),
        ("T_total", ctypes.c_uint32),
        ("reserved2", ctypes.c_uint32),
    ]


class RefinedChunkRef(ctypes.Structure):
    """kvc_refined_chunk_ref: a chunk's base and refinement containers."""
    _fields_ = [
        ("container", ctypes.c_void_p),
        ("container_bytes", ctypes.c_uint64),
        ("refinement", ctypes.c_void_p),
        ("refinement_bytes", ctypes.c_uint64),
        ("first_token", ctypes.c_uint32),
        ("n_tokens", ctypes.c_uint32),
        ("level", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class HostChunk(ctypes.Structure):
    """kvc_host_chunk: one encoded chunk still in (pinned) host memory."""
    _fields_ = [
        ("host_container", ctypes.c_void_p),
        ("container_bytes", ctypes.c_uint64),
        ("first_token", ctypes.c_uint32),
        ("n_tokens", ctypes.c_uint32),
        ("level", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


def make_desc(n_layers: int, n_channels: int,
              delta_bits: Sequence[Sequence[int]] = ((6, 5, 4),),
              group_tokens: int = 10, chunk_tokens: int = 1500) -> CodecDesc:
    d = CodecDesc()
    d.n_layers = n_layers
    d.n_channels = n_channels
    d.group_tokens = group_tokens
    d.chunk_tokens = chunk_tokens
    d.anchor_bits = 8
    d.n_levels = len(delta_bits)
    for i, row in enumerate(delta_bits):
        for j in range(3):
            d.delta_bits[i][j] = int(row[j])
    d.cdf_prec_bits = 15
    return d


_lib = None


def lib():
    """Load libkvc.so (built in-tree by ``python -m kv_cache_compression_decode_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m kv_cache_compression_decode_amd.build` (no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, u32, u64, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32
    dp = ctypes.POINTER(CodecDesc)
    L.kvc_version.restype = ctypes.c_int
    L.kvc_status_str.argtypes = [ctypes.c_int]
    L.kvc_status_str.restype = ctypes.c_char_p
    L.kvc_validate_desc.argtypes = [dp]
    L.kvc_validate_desc.restype = ctypes.c_int
    for name in ("kvc_tables_bytes", "kvc_profile_ws_bytes"):
        getattr(L, name).argtypes = [dp]
        getattr(L, name).restype = u64
    for name in ("kvc_container_bound", "kvc_encode_bound", "kvc_encode_ws_bytes",
                 "kvc_decode_ws_bytes"):
        getattr(L, name).argtypes = [dp, u32]
        getattr(L, name).restype = u64
    L.kvc_profile.argtypes = [dp, vp, u32, vp, vp, u64, vp, vp]
    L.kvc_profile.restype = ctypes.c_int
    L.kvc_encode.argtypes = [dp, vp, vp, u32, vp, vp, u64, vp, vp, u64, vp, vp]
    L.kvc_encode.restype = ctypes.c_int
    L.kvc_decode.argtypes = [dp, vp, vp, u32, vp, u32, vp, u64, vp, vp]
    L.kvc_decode.restype = ctypes.c_int
    L.kvc_decode_symbols.argtypes = [dp, vp, vp, u32, vp, u32, vp, u64, vp, vp]
    L.kvc_decode_symbols.restype = ctypes.c_int
    L.kvc_decode_index.argtypes = [dp, vp, vp, u32, vp, vp, u64, vp, vp]
    L.kvc_decode_index.restype = ctypes.c_int
    L.kvc_restore_staging_bytes.argtypes = [vp, u32, u32]
    L.kvc_restore_staging_bytes.restype = u64
    L.kvc_restore.argtypes = [dp, vp, vp, u32, u32, vp, u32, vp, u64, vp, u64, vp, vp, vp, vp]
    L.kvc_restore.restype = ctypes.c_int
    L.kvc_decode_multi.argtypes = [dp, vp, vp, u32, vp, u64, vp, vp]
    L.kvc_decode_multi.restype = ctypes.c_int
    L.kvc_decode_static.argtypes = [dp, vp, vp, u32, vp, u32, vp, vp]
    L.kvc_decode_static.restype = ctypes.c_int
    for name in ("kvc_refine_tables_bytes", "kvc_refine_profile_ws_bytes"):
        getattr(L, name).argtypes = [dp]
        getattr(L, name).restype = u64
    for name in ("kvc_encode_refine_ws_bytes", "kvc_decode_refined_ws_bytes"):
        getattr(L, name).argtypes = [dp, u32]
        getattr(L, name).restype = u64
    L.kvc_profile_refine.argtypes = [dp, vp, vp, u32, u32, vp, vp, u64, vp, vp]
    L.kvc_profile_refine.restype = ctypes.c_int
    L.kvc_encode_refine.argtypes = [dp, vp, u32, vp, u32, vp, vp, u64, vp, vp, u64, vp, vp]
    L.kvc_encode_refine.restype = ctypes.c_int
    L.kvc_decode_refined.argtypes = [dp, vp, vp, u32, vp, u32, vp, u32, vp, u64, vp, vp]
    L.kvc_decode_refined.restype = ctypes.c_int
    L.kvc_plan_stream.argtypes = [vp, u32, u32, vp, u32, ctypes.c_double, ctypes.c_double, vp, vp]
    L.kvc_plan_stream.restype = ctypes.c_int
    _lib = L
    return L


def status_str(code: int) -> str:
    try:
        return lib().kvc_status_str(int(code)).decode()
    except Exception:  # library missing: still format the code
        return f"status {code}"


def _stream(stream: Optional[torch.cuda.Stream]) -> ctypes.c_void_p:
    """The HIP stream to launch on: `stream`, else torch's current stream.  A
    stream other than the current one first waits for the work already
    queued on the current stream (among it the allocation and zero-fill of
    the tensors the launch uses)."""
    cur = torch.cuda.current_stream()
    if stream is None:
        return ctypes.c_void_p(cur.cuda_stream)
    if stream.cuda_stream != cur.cuda_stream:
        stream.wait_stream(cur)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(code: int, what: str) -> None:
    if code != OK:
        raise KvcError(code, what)


def _dev_status(device) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device)


def read_status(status: torch.Tensor, what: str, stream=None) -> None:
    """Wait for the launch (on `stream`, else the current stream) and raise on
    a device error."""
    if stream is not None:
        stream.synchronize()
    code = int(status.item())
    if code != OK:
        raise KvcError(code, what)


def _kv_ptr(t: torch.Tensor) -> int:
    if not t.is_cuda or t.element_size() != 2 or not t.is_contiguous():
        raise ValueError("KV tensors must be contiguous 2-byte CUDA tensors [L][2][T][C]")
    return t.data_ptr()


# --------------------------------------------------------------------- API
def tables_bytes(desc: CodecDesc) -> int:
    return int(lib().kvc_tables_bytes(ctypes.byref(desc)))


def profile(desc: CodecDesc, kv_prof: torch.Tensor, stream=None, check: bool = True) -> torch.Tensor:
    """Profile per channel-layer distributions on kv_prof [L][2][T][C]; returns
    the tables blob (uint8 tensor on the same device)."""
    L = lib()
    T = kv_prof.shape[2]
    nb = tables_bytes(desc)
    if nb == 0:
        raise KvcError(ERR_INVALID_ARG, "profile")
    tables = torch.empty(nb, dtype=torch.uint8, device=kv_prof.device)
    wsb = int(L.kvc_profile_ws_bytes(ctypes.byref(desc)))
    ws = torch.empty(wsb, dtype=torch.uint8, device=kv_prof.device)
    st = _dev_status(kv_prof.device)
    _check(L.kvc_profile(ctypes.byref(desc), _kv_ptr(kv_prof), T, tables.data_ptr(), ws.data_ptr(),
                         wsb, st.data_ptr(), _stream(stream)), "kvc_profile")
    if check:
        read_status(st, "kvc_profile", stream)
    return tables


def profile_id(tables: torch.Tensor) -> int:
    return int(tables[48:56].cpu().numpy().view("<u8")[0])


@dataclasses.dataclass
class Encoded:
    """Containers of one context, back to back in `blob`; chunk k is
    blob[offsets[k]:offsets[k+1]] at level levels[k], tokens
    [k*chunk_tokens, ...)."""
    blob: torch.Tensor
    offsets: List[int]
    levels: List[int]
    n_tokens: List[int]
    chunk_tokens: int

    @property
    def n_chunks(self) -> int:
        return len(self.levels)

    def container(self, k: int) -> torch.Tensor:
        return self.blob[self.offsets[k]:self.offsets[k + 1]]

    def total_bytes(self) -> int:
        return self.offsets[-1]


class EncodeWorkspace:
    """Reusable device buffers of kvc_encode for one (descriptor, T)."""

    def __init__(self, desc: CodecDesc, T: int, device):
        L = lib()
        self.T = T
        self.ws_bytes = int(L.kvc_encode_ws_bytes(ctypes.byref(desc), T))
        self.cap = int(L.kvc_encode_bound(ctypes.byref(desc), T))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.out = torch.empty(self.cap, dtype=torch.uint8, device=device)
        n_chunks = (T + desc.chunk_tokens - 1) // desc.chunk_tokens
        self.offsets = torch.empty(n_chunks + 1, dtype=torch.int64, device=device)
        self.status = _dev_status(device)


def encode_async(desc: CodecDesc, tables: torch.Tensor, kv: torch.Tensor, levels: Sequence[int],
                 wsp: EncodeWorkspace, stream=None) -> None:
    """Launch kvc_encode into wsp.out / wsp.offsets / wsp.status (no sync)."""
    L = lib()
    T = kv.shape[2]
    lv = (ctypes.c_uint8 * max(len(levels), 1))(*[int(x) for x in levels])
    _check(L.kvc_encode(ctypes.byref(desc), tables.data_ptr(), _kv_ptr(kv), T, lv,
                        wsp.out.data_ptr(), wsp.cap, wsp.offsets.data_ptr(), wsp.ws.data_ptr(),
                        wsp.ws_bytes, wsp.status.data_ptr(), _stream(stream)), "kvc_encode")


def encode(desc: CodecDesc, tables: torch.Tensor, kv: torch.Tensor, levels: Sequence[int],
           stream=None, wsp: Optional[EncodeWorkspace] = None) -> Encoded:
    """Encode kv [L][2][T][C] (chunk k at levels[k]); returns the containers."""
    T = kv.shape[2]
    n_chunks = (T + desc.chunk_tokens - 1) // desc.chunk_tokens
    if len(levels) != n_chunks:
        raise ValueError(f"{n_chunks} chunk levels expected")
    if wsp is None:
        wsp = EncodeWorkspace(desc, T, kv.device)
    encode_async(desc, tables, kv, levels, wsp, stream)
    read_status(wsp.status, "kvc_encode", stream)
    offs = [int(x) for x in wsp.offsets.cpu().tolist()]
    blob = wsp.out[: offs[-1]].clone()
    ntok = [min(desc.chunk_tokens, T - k * desc.chunk_tokens) for k in range(n_chunks)]
    return Encoded(blob, offs, [int(x) for x in levels], ntok, desc.chunk_tokens)


def chunk_refs(enc: Encoded, chunks: Optional[Sequence[int]] = None,
               first_tokens: Optional[Sequence[int]] = None) -> List[ChunkRef]:
    """ChunkRefs for (a subset of) an Encoded context; by default every chunk
    goes back to its own token range."""
    ks = list(range(enc.n_chunks)) if chunks is None else list(chunks)
    out = []
    base = enc.blob.data_ptr()
    for i, k in enumerate(ks):
        r = ChunkRef()
        r.container = base + enc.offsets[k]
        r.container_bytes = enc.offsets[k + 1] - enc.offsets[k]
        r.first_token = k * enc.chunk_tokens if first_tokens is None else int(first_tokens[i])
        r.n_tokens = enc.n_tokens[k]
        r.level = enc.levels[k]
        r.reserved = 0
        out.append(r)
    return out


class DecodeWorkspace:
    """Reusable workspace + status word of kvc_decode for up to n_chunks."""

    def __init__(self, desc: CodecDesc, n_chunks: int, device):
        self.ws_bytes = int(lib().kvc_decode_ws_bytes(ctypes.byref(desc), n_chunks))
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.status = _dev_status(device)
        self.n_chunks = n_chunks


def _refs_array(refs: Sequence[ChunkRef]):
    arr = (ChunkRef * max(len(refs), 1))()
    for i, r in enumerate(refs):
        arr[i] = r
    return arr


def decode_async(desc: CodecDesc, tables: torch.Tensor, refs: Sequence[ChunkRef],
                 out: torch.Tensor, wsp: DecodeWorkspace, stream=None) -> None:
    """Launch kvc_decode into out [L][2][T_total][C] (no sync)."""
    arr = _refs_array(refs)
    _check(lib().kvc_decode(ctypes.byref(desc), tables.data_ptr(), arr, len(refs), _kv_ptr(out),
                            out.shape[2], wsp.ws.data_ptr(), wsp.ws_bytes, wsp.status.data_ptr(),
                            _stream(stream)), "kvc_decode")


def decode(desc: CodecDesc, tables: torch.Tensor, refs: Sequence[ChunkRef], T_total: int,
           out: Optional[torch.Tensor] = None, stream=None,
           wsp: Optional[DecodeWorkspace] = None) -> torch.Tensor:
    """Decode chunks into the KV cache [L][2][T_total][C] (int16 bit patterns
    of binary16)."""
    dev = tables.device
    if out is None:
        out = torch.zeros((desc.n_layers, 2, T_total, desc.n_channels), dtype=torch.int16, device=dev)
    if wsp is None:
        wsp = DecodeWorkspace(desc, len(refs), dev)
    decode_async(desc, tables, refs, out, wsp, stream)
    read_status(wsp.status, "kvc_decode", stream)
    return out


def decode_static(desc: CodecDesc, tables: torch.Tensor, refs: Sequence[ChunkRef],
                  out: torch.Tensor, status: torch.Tensor, stream=None) -> None:
    """kvc_decode_static: decode into out [L][2][T_total][C] using the
    library's own fixed device scratch (no workspace, nothing allocated);
    `status` is a caller-owned int32 device word, read after synchronizing."""
    arr = _refs_array(refs)
    _check(lib().kvc_decode_static(ctypes.byref(desc), tables.data_ptr(), arr, len(refs),
                                   _kv_ptr(out), out.shape[2], status.data_ptr(),
                                   _stream(stream)), "kvc_decode_static")


def decode_symbols(desc: CodecDesc, tables: torch.Tensor, refs: Sequence[ChunkRef],
                   T_total: int, stream=None) -> torch.Tensor:
    dev = tables.device
    out = torch.zeros((desc.n_layers, 2, T_total, desc.n_channels), dtype=torch.uint8, device=dev)
    wsp = DecodeWorkspace(desc, len(refs), dev)
    arr = _refs_array(refs)
    _check(lib().kvc_decode_symbols(ctypes.byref(desc), tables.data_ptr(), arr, len(refs),
                                    out.data_ptr(), T_total, wsp.ws.data_ptr(), wsp.ws_bytes,
                                    wsp.status.data_ptr(), _stream(stream)), "kvc_decode_symbols")
    read_status(wsp.status, "kvc_decode_symbols", stream)
    return out


def decode_index(desc: CodecDesc, tables: torch.Tensor, refs: Sequence[ChunkRef],
                 stream=None) -> torch.Tensor:
    """Per-stream payload offsets [n_chunks][2LC] (int32 view of u32)."""
    dev = tables.device
    offs = torch.zeros((len(refs), desc.n_streams), dtype=torch.int32, device=dev)
    wsp = DecodeWorkspace(desc, len(refs), dev)
    arr = _refs_array(refs)
    _check(lib().kvc_decode_index(ctypes.byref(desc), tables.data_ptr(), arr, len(refs),
                                  offs.data_ptr(), wsp.ws.data_ptr(), wsp.ws_bytes,
                                  wsp.status.data_ptr(), _stream(stream)), "kvc_decode_index")
    read_status(wsp.status, "kvc_decode_index", stream)
    return offs


# ------------------------------------------------------------ streamed restore
def host_chunks(enc: Encoded, host_blob: torch.Tensor,
                chunks: Optional[Sequence[int]] = None) -> List[HostChunk]:
    """HostChunks for (a subset of) an Encoded context whose containers were
    copied to `host_blob` (a CPU uint8 tensor laid out like enc.blob; pinned
    memory lets the copies overlap the decode)."""
    if host_blob.is_cuda or host_blob.dtype != torch.uint8 or not host_blob.is_contiguous():
        raise ValueError("host_blob must be a contiguous CPU uint8 tensor")
    ks = list(range(enc.n_chunks)) if chunks is None else list(chunks)
    base = host_blob.data_ptr()
    out = []
    for k in ks:
        c = HostChunk()
        c.host_container = base + enc.offsets[k]
        c.container_bytes = enc.offsets[k + 1] - enc.offsets[k]
        c.first_token = k * enc.chunk_tokens
        c.n_tokens = enc.n_tokens[k]
        c.level = enc.levels[k]
        c.reserved = 0
        out.append(c)
    return out


def _host_array(chunks: Sequence[HostChunk]):
    arr = (HostChunk * max(len(chunks), 1))()
    for i, c in enumerate(chunks):
        arr[i] = c
    return arr


def restore_staging_bytes(chunks: Sequence[HostChunk], batch: int) -> int:
    return int(lib().kvc_restore_staging_bytes(_host_array(chunks), len(chunks), batch))


class RestoreWorkspace:
    """Device staging slots, decode workspace, status word and copy stream
    of kvc_restore for these chunks in batches of `batch`."""

    def __init__(self, desc: CodecDesc, chunks: Sequence[HostChunk], batch: int, device,
                 min_staging_bytes: int = 0):
        self.batch = batch
        self.staging_bytes = max(restore_staging_bytes(chunks, batch), min_staging_bytes, 256)
        self.staging = torch.empty(self.staging_bytes, dtype=torch.uint8, device=device)
        per = max(1, min(batch, len(chunks)))
        self.ws_bytes = int(lib().kvc_decode_ws_bytes(ctypes.byref(desc), per))
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.status = _dev_status(device)
        self.copy_stream = torch.cuda.Stream(device=device)


class HipEvents:
    """Raw HIP events (timing disabled) for kvc_restore's per-batch signal."""

    def __init__(self, n: int):
        try:
            self._hip = ctypes.CDLL("libamdhip64.so")
        except OSError:
            self._hip = ctypes.CDLL("/opt/rocm/lib/libamdhip64.so")
        self.handles = (ctypes.c_void_p * max(n, 1))()
        self.n = n
        for i in range(n):
            ev = ctypes.c_void_p()
            if self._hip.hipEventCreateWithFlags(ctypes.byref(ev), ctypes.c_uint(2)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.handles[i] = ev

    def query(self, i: int) -> bool:
        """True once event i has completed."""
        return self._hip.hipEventQuery(ctypes.c_void_p(self.handles[i])) == 0

    def synchronize(self, i: int) -> None:
        if self._hip.hipEventSynchronize(ctypes.c_void_p(self.handles[i])) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def close(self) -> None:
        """Destroy the events (also done when the object is collected)."""
        for i in range(self.n):
            if self.handles[i]:
                self._hip.hipEventDestroy(ctypes.c_void_p(self.handles[i]))
                self.handles[i] = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown: the runtime may be gone
            pass


def restore_async(desc: CodecDesc, tables: torch.Tensor, chunks: Sequence[HostChunk],
                  out: torch.Tensor, rws: RestoreWorkspace, stream=None,
                  events: Optional[HipEvents] = None) -> None:
    """Queue kvc_restore: batches of rws.batch chunks copied on rws.copy_stream
    and decoded on `stream` (default: the current stream) into out."""
    arr = _host_array(chunks)
    ev = events.handles if events is not None else None
    _check(lib().kvc_restore(ctypes.byref(desc), tables.data_ptr(), arr, len(chunks), rws.batch,
                             _kv_ptr(out), out.shape[2], rws.staging.data_ptr(),
                             rws.staging_bytes, rws.ws.data_ptr(), rws.ws_bytes,
                             rws.status.data_ptr(), _stream(stream),
                             ctypes.c_void_p(rws.copy_stream.cuda_stream), ev), "kvc_restore")


def restore(desc: CodecDesc, tables: torch.Tensor, chunks: Sequence[HostChunk], T_total: int,
            batch: int = 2, out: Optional[torch.Tensor] = None, stream=None,
            rws: Optional[RestoreWorkspace] = None) -> torch.Tensor:
    """Restore host-resident chunks into the KV cache [L][2][T_total][C]."""
    dev = tables.device
    if out is None:
        out = torch.zeros((desc.n_layers, 2, T_total, desc.n_channels), dtype=torch.int16, device=dev)
    if rws is None:
        rws = RestoreWorkspace(desc, chunks, batch, dev)
    restore_async(desc, tables, chunks, out, rws, stream)
    read_status(rws.status, "kvc_restore", stream)
    return out


# ------------------------------------------------------ per-chunk level choice
class BwPiece(ctypes.Structure):
    """kvc_bw_piece: from start_s on, the link moves bytes_per_s."""
    _fields_ = [("start_s", ctypes.c_double), ("bytes_per_s", ctypes.c_double)]


def plan_stream(chunk_bytes, trace: Sequence[Tuple[float, float]], slo_s: float,
                init_bytes_per_s: float) -> Tuple[List[int], List[float]]:
    """kvc_plan_stream: the level chosen for each chunk and its arrival time.
    chunk_bytes: [n_chunks][n_levels] container sizes (best quality first);
    trace: (start_s, bytes_per_s) pieces, the first at 0."""
    import numpy as np

    cb = np.ascontiguousarray(np.asarray(chunk_bytes, dtype=np.uint64))
    if cb.ndim != 2:
        raise ValueError("chunk_bytes must be [n_chunks][n_levels]")
    n, L = cb.shape
    tr = (BwPiece * max(len(trace), 1))()
    for i, (t0, r) in enumerate(trace):
        tr[i].start_s = float(t0)
        tr[i].bytes_per_s = float(r)
    levels = np.zeros(max(n, 1), dtype=np.uint8)
    finish = np.zeros(max(n, 1), dtype=np.float64)
    _check(lib().kvc_plan_stream(cb.ctypes.data, n, L, tr, len(trace), float(slo_s),
                                 float(init_bytes_per_s), levels.ctypes.data,
                                 finish.ctypes.data), "kvc_plan_stream")
    return [int(x) for x in levels[:n]], [float(x) for x in finish[:n]]


# ------------------------------------------------- several requests, one call
def request_chunks(enc: Encoded, out: torch.Tensor,
                   chunks: Optional[Sequence[int]] = None) -> List[RequestChunk]:
    """RequestChunks of (a subset of) one request's Encoded context, each
    going back to its own token range of that request's cache `out`."""
    _kv_ptr(out)
    ks = list(range(enc.n_chunks)) if chunks is None else list(chunks)
    base = enc.blob.data_ptr()
    res = []
    for k in ks:
        c = RequestChunk()
        c.container = base + enc.offsets[k]
        c.container_bytes = enc.offsets[k + 1] - enc.offsets[k]
        c.first_token = k * enc.chunk_tokens
        c.n_tokens = enc.n_tokens[k]
        c.level = enc.levels[k]
        c.reserved = 0
        c.kv_out = out.data_ptr()
        c.T_total = out.shape[2]
        c.reserved2 = 0
        res.append(c)
    return res


def decode_multi_async(desc: CodecDesc, tables: torch.Tensor, chunks: Sequence[RequestChunk],
                       wsp: DecodeWorkspace, stream=None) -> None:
    """Queue kvc_decode_multi: every chunk into its own request's cache."""
    arr = (RequestChunk * max(len(chunks), 1))()
    for i, c in enumerate(chunks):
        arr[i] = c
    _check(lib().kvc_decode_multi(ctypes.byref(desc), tables.data_ptr(), arr, len(chunks),
                                  wsp.ws.data_ptr(), wsp.ws_bytes, wsp.status.data_ptr(),
                                  _stream(stream)), "kvc_decode_multi")


def decode_multi(desc: CodecDesc, tables: torch.Tensor, chunks: Sequence[RequestChunk],
                 stream=None, wsp: Optional[DecodeWorkspace] = None) -> None:
    if wsp is None:
        wsp = DecodeWorkspace(desc, len(chunks), tables.device)
    decode_multi_async(desc, tables, chunks, wsp, stream)
    read_status(wsp.status, "kvc_decode_multi", stream)


# ------------------------------------------------------ incremental refinement
def refine_tables_bytes(desc: CodecDesc) -> int:
    return int(lib().kvc_refine_tables_bytes(ctypes.byref(desc)))


def profile_refine(desc: CodecDesc, tables: torch.Tensor, kv_prof: torch.Tensor, refine_bits: int,
                   stream=None, check: bool = True) -> torch.Tensor:
    """Profile the refinement models (refine_bits bits) on kv_prof
    [L][2][T][C] for the base `tables`; returns the refinement tables blob."""
    L = lib()
    nb = refine_tables_bytes(desc)
    if nb == 0:
        raise KvcError(ERR_INVALID_ARG, "profile_refine")
    rtables = torch.empty(nb, dtype=torch.uint8, device=kv_prof.device)
    wsb = int(L.kvc_refine_profile_ws_bytes(ctypes.byref(desc)))
    ws = torch.empty(wsb, dtype=torch.uint8, device=kv_prof.device)
    st = _dev_status(kv_prof.device)
    _check(L.kvc_profile_refine(ctypes.byref(desc), tables.data_ptr(), _kv_ptr(kv_prof),
                                kv_prof.shape[2], refine_bits, rtables.data_ptr(), ws.data_ptr(),
                                wsb, st.data_ptr(), _stream(stream)), "kvc_profile_refine")
    if check:
        read_status(st, "kvc_profile_refine", stream)
    return rtables


def refine_id(rtables: torch.Tensor) -> int:
    return int(rtables[48:56].cpu().numpy().view("<u8")[0])


def encode_refine(desc: CodecDesc, rtables: torch.Tensor, refine_bits: int, kv: torch.Tensor,
                  levels: Sequence[int], stream=None) -> Encoded:
    """The refinement containers of kv [L][2][T][C] over base layers at
    `levels` (one per chunk)."""
    L = lib()
    T = kv.shape[2]
    n_chunks = (T + desc.chunk_tokens - 1) // desc.chunk_tokens
    if len(levels) != n_chunks:
        raise ValueError(f"{n_chunks} chunk levels expected")
    wsb = int(L.kvc_encode_refine_ws_bytes(ctypes.byref(desc), T))
    cap = int(L.kvc_encode_bound(ctypes.byref(desc), T))
    ws = torch.empty(wsb, dtype=torch.uint8, device=kv.device)
    out = torch.empty(cap, dtype=torch.uint8, device=kv.device)
    offsets = torch.empty(n_chunks + 1, dtype=torch.int64, device=kv.device)
    st = _dev_status(kv.device)
    lv = (ctypes.c_uint8 * max(len(levels), 1))(*[int(x) for x in levels])
    _check(L.kvc_encode_refine(ctypes.byref(desc), rtables.data_ptr(), refine_bits, _kv_ptr(kv), T,
                               lv, out.data_ptr(), cap, offsets.data_ptr(), ws.data_ptr(), wsb,
                               st.data_ptr(), _stream(stream)), "kvc_encode_refine")
    read_status(st, "kvc_encode_refine", stream)
    offs = [int(x) for x in offsets.cpu().tolist()]
    ntok = [min(desc.chunk_tokens, T - k * desc.chunk_tokens) for k in range(n_chunks)]
    return Encoded(out[: offs[-1]].clone(), offs, [int(x) for x in levels], ntok,
                   desc.chunk_tokens)


def refined_chunk_refs(enc: Encoded, renc: Encoded, chunks: Optional[Sequence[int]] = None,
                       first_tokens: Optional[Sequence[int]] = None) -> List[RefinedChunkRef]:
    """RefinedChunkRefs pairing each chunk's base container (enc) with its
    refinement container (renc); by default each goes back to its own
    token range."""
    ks = list(range(enc.n_chunks)) if chunks is None else list(chunks)
    out = []
    for i, k in enumerate(ks):
        r = RefinedChunkRef()
        r.container = enc.blob.data_ptr() + enc.offsets[k]
        r.container_bytes = enc.offsets[k + 1] - enc.offsets[k]
        r.refinement = renc.blob.data_ptr() + renc.offsets[k]
        r.refinement_bytes = renc.offsets[k + 1] - renc.offsets[k]
        r.first_token = k * enc.chunk_tokens if first_tokens is None else int(first_tokens[i])
        r.n_tokens = enc.n_tokens[k]
        r.level = enc.levels[k]
        r.reserved = 0
        out.append(r)
    return out


class RefinedDecodeWorkspace:
    """Reusable workspace + status word of kvc_decode_refined for up to n_chunks."""

    def __init__(self, desc: CodecDesc, n_chunks: int, device):
        self.ws_bytes = int(lib().kvc_decode_refined_ws_bytes(ctypes.byref(desc), n_chunks))
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.status = _dev_status(device)
        self.n_chunks = n_chunks


def decode_refined_async(desc: CodecDesc, tables: torch.Tensor, rtables: torch.Tensor,
                         refine_bits: int, refs: Sequence[RefinedChunkRef], out: torch.Tensor,
                         wsp: RefinedDecodeWorkspace, stream=None) -> None:
    """Launch kvc_decode_refined into out [L][2][T_total][C] (no sync)."""
    arr = (RefinedChunkRef * max(len(refs), 1))()
    for i, r in enumerate(refs):
        arr[i] = r
    _check(lib().kvc_decode_refined(ctypes.byref(desc), tables.data_ptr(), rtables.data_ptr(),
                                    refine_bits, arr, len(refs), _kv_ptr(out), out.shape[2],
                                    wsp.ws.data_ptr(), wsp.ws_bytes, wsp.status.data_ptr(),
                                    _stream(stream)), "kvc_decode_refined")


def decode_refined(desc: CodecDesc, tables: torch.Tensor, rtables: torch.Tensor, refine_bits: int,
                   refs: Sequence[RefinedChunkRef], T_total: int,
                   out: Optional[torch.Tensor] = None, stream=None,
                   wsp: Optional[RefinedDecodeWorkspace] = None) -> torch.Tensor:
    """Decode base + refinement layers into the KV cache [L][2][T_total][C]
    (int16 bit patterns of binary16)."""
    dev = tables.device
    if out is None:
        out = torch.zeros((desc.n_layers, 2, T_total, desc.n_channels), dtype=torch.int16, device=dev)
    if wsp is None:
        wsp = RefinedDecodeWorkspace(desc, len(refs), dev)
    decode_refined_async(desc, tables, rtables, refine_bits, refs, out, wsp, stream)
    read_status(wsp.status, "kvc_decode_refined", stream)
    return out

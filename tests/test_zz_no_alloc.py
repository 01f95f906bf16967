"""kvc_decode_static (the decode entry point that allocates nothing and uses
the library's fixed per-GPU scratch) against kvc_decode (the same decode
with a caller workspace): identical binary16 output, element by element, on
two calls in a row, the second one smaller and into other token positions,
and an oversized request refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_compression_decode_amd as kvc
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def test_decode_static_equals_decode_two_calls():
    print("\n[gpu no-alloc] 8 layers x 320 channels, 6,100 tokens, mixed levels", flush=True)
    cfg = synth.small_config(8, 320, 6100, n_levels=3, schedule="mixed", seed_index=96)
    levels = [2, 0, 1, 1, 0]
    d = kvc.make_desc(cfg.n_layers, cfg.n_channels, cfg.delta_bits)
    tables = kvc.profile(d, _t(synth.make_profile_kv(cfg)))
    enc = kvc.encode(d, tables, _t(synth.make_kv(cfg)), levels)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    # call 1: every chunk
    refs = kvc.chunk_refs(enc)
    want = kvc.decode(d, tables, refs, cfg.n_tokens)
    got = torch.full_like(want, 0x3C00)
    kvc.decode_static(d, tables, refs, got, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(got, want)

    # call 2: two chunks into other positions of a shorter cache
    refs2 = kvc.chunk_refs(enc, chunks=[4, 1], first_tokens=[0, 100])
    want2 = kvc.decode(d, tables, refs2, 1600)
    got2 = torch.full_like(want2, 0x3C00)
    kvc.decode_static(d, tables, refs2, got2, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(got2, want2)


def test_decode_static_refuses_oversized_request():
    """A request whose decode scratch exceeds the fixed array is refused
    synchronously with KVC_ERR_CAPACITY, and nothing is written."""
    d = kvc.make_desc(80, 1024)
    n = 64  # 64 chunks x 163,840 streams x 4-byte offsets > 32 MiB
    assert kvc.lib().kvc_decode_ws_bytes(ctypes.byref(d), n) > 32 << 20
    refs = (kvc.ChunkRef * n)()
    out = torch.zeros(8, dtype=torch.int16, device=DEV)
    status = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    st = kvc.lib().kvc_decode_static(ctypes.byref(d), out.data_ptr(), refs, n, out.data_ptr(), 1,
                                     status.data_ptr(), None)
    assert st == kvc.ERR_CAPACITY
    torch.cuda.synchronize()
    assert int(status.item()) == 7

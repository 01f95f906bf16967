"""The Python binding on a side stream: every call that takes `stream=` must
order itself after the work already queued on torch's current stream (the
allocation and zero-fill of its own output and status word) and read its
status only after its own launches finished.  A long matrix product queued on
the current stream before each call makes a missing dependency show up as a
wiped or stale result.  Results must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import kv_cache_compression_decode_amd as kvc
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def _busy_current_stream():
    """About 20-40 ms of work on the current stream (fp32 products)."""
    a = torch.full((6144, 6144), 1e-3, device=DEV)
    for _ in range(6):
        a = a @ a
    return a


def test_side_stream_calls_bit_exact():
    print("\n[gpu streams] 4 layers x 192 channels, 3,100 tokens, mixed levels", flush=True)
    cfg = synth.small_config(4, 192, 3100, n_levels=3, schedule="mixed", seed_index=95)
    levels = [1, 2, 0]
    kv = synth.make_kv(cfg)
    kvp = synth.make_profile_kv(cfg)
    od = oracle.desc_for(cfg)
    otb = oracle.profile(od, kvp)
    ocont = oracle.encode(od, otb, kv, levels)
    want = oracle.decode(od, otb, ocont, levels, cfg.n_tokens)
    d = kvc.make_desc(cfg.n_layers, cfg.n_channels, cfg.delta_bits)
    side = torch.cuda.Stream(device=DEV)

    _busy_current_stream()
    tables = kvc.profile(d, _t(kvp), stream=side)
    assert kvc.profile_id(tables) == otb.profile_id
    _busy_current_stream()
    enc = kvc.encode(d, tables, _t(kv), levels, stream=side)
    for k, c in enumerate(ocont):
        np.testing.assert_array_equal(enc.container(k).cpu().numpy(), c)
    _busy_current_stream()
    out = kvc.decode(d, tables, kvc.chunk_refs(enc), cfg.n_tokens, stream=side)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), want)

    _busy_current_stream()
    out2 = torch.zeros_like(out)
    kvc.decode_multi(d, tables, kvc.request_chunks(enc, out2), stream=side)
    np.testing.assert_array_equal(out2.cpu().numpy().view(np.uint16), want)

    host = torch.empty(enc.total_bytes(), dtype=torch.uint8, pin_memory=True)
    host.copy_(enc.blob.cpu())
    _busy_current_stream()
    out3 = kvc.restore(d, tables, kvc.host_chunks(enc, host), cfg.n_tokens, batch=1, stream=side)
    np.testing.assert_array_equal(out3.cpu().numpy().view(np.uint16), want)

"""Streamed restore (kvc_restore) against the CPU oracle, through the C ABI.

Containers written by the oracle sit in pinned host memory; kvc_restore
copies them in batches on a copy stream and decodes each batch on the
compute stream.  The restored binary16 KV must equal the oracle's decode
bit for bit for every batch size (one chunk per batch up to all chunks in
one), for chunks sent to other token positions, for calls that reuse one
staging buffer back to back, and with copy and compute on one stream; a
corrupt container in a later batch must still be reported.
"""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_compression_decode_amd as kvc
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


class Ctx:
    """Nine chunks (13,000 tokens: the last one 1,000) at mixed levels."""

    def __init__(self):
        cfg = synth.small_config(2, 64, 13000, n_levels=3, seed_index=99)
        self.cfg = cfg
        self.levels = [0, 1, 2, 2, 1, 0, 0, 2, 1]
        kv = synth.make_kv(cfg)
        kvp = synth.make_profile_kv(cfg)
        od = oracle.desc_for(cfg)
        otb = oracle.profile(od, kvp)
        self.ocont = oracle.encode(od, otb, kv, self.levels)
        self.oout = oracle.decode(od, otb, self.ocont, self.levels, cfg.n_tokens)
        self.d = kvc.make_desc(cfg.n_layers, cfg.n_channels, cfg.delta_bits)
        self.tables = kvc.profile(self.d, torch.from_numpy(kvp.view(np.int16)).to(DEV))
        sizes = [len(c) for c in self.ocont]
        offs = np.concatenate([[0], np.cumsum(sizes)])
        blob = np.concatenate(self.ocont)
        # pinned memory allocated as such, then filled
        self.host = torch.empty(len(blob), dtype=torch.uint8, pin_memory=True)
        self.host.copy_(torch.from_numpy(blob))
        self.enc = kvc.Encoded(torch.empty(0, dtype=torch.uint8), [int(x) for x in offs],
                               list(self.levels),
                               [min(1500, cfg.n_tokens - 1500 * k) for k in range(len(sizes))],
                               1500)

    def new_out(self, T=None, fill=0):
        T = self.cfg.n_tokens if T is None else T
        return torch.full((self.cfg.n_layers, 2, T, self.cfg.n_channels), fill, dtype=torch.int16,
                          device=DEV)


@pytest.fixture(scope="module")
def ctx():
    print("\n[gpu restore] nine-chunk context", flush=True)
    return Ctx()


@pytest.mark.parametrize("batch", [1, 2, 4, 9, 20])
def test_restore_bit_exact(ctx, batch):
    print(f"[gpu restore] batch {batch}", flush=True)
    chunks = kvc.host_chunks(ctx.enc, ctx.host)
    out = kvc.restore(ctx.d, ctx.tables, chunks, ctx.cfg.n_tokens, batch=batch)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), ctx.oout)


def test_restore_subset_to_other_positions(ctx):
    """Chunks go to the token ranges given; tokens not covered are untouched."""
    chunks = kvc.host_chunks(ctx.enc, ctx.host, chunks=[8, 3, 0])
    firsts = [100, 1200, 2900]
    for c, t0 in zip(chunks, firsts):
        c.first_token = t0
    out = ctx.new_out(T=5000, fill=0x7BCD)
    kvc.restore(ctx.d, ctx.tables, chunks, 5000, batch=2, out=out)
    got = out.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got[:, :, 100:1100], ctx.oout[:, :, 12000:13000])
    np.testing.assert_array_equal(got[:, :, 1200:2700], ctx.oout[:, :, 4500:6000])
    np.testing.assert_array_equal(got[:, :, 2900:4400], ctx.oout[:, :, 0:1500])
    untouched = np.ones(5000, bool)
    for a, b in ((100, 1100), (1200, 2700), (2900, 4400)):
        untouched[a:b] = False
    assert np.all(got[:, :, untouched] == 0x7BCD)


def test_restore_back_to_back_reuses_staging(ctx):
    """Two restores queued without a synchronization between them share the
    staging slots: the second call's copies wait for the first call's
    decodes."""
    all_chunks = kvc.host_chunks(ctx.enc, ctx.host)
    # the reversed order pairs the chunks differently: room for both
    need = max(kvc.restore_staging_bytes(all_chunks, 2),
               kvc.restore_staging_bytes(all_chunks[::-1], 2))
    rws = kvc.RestoreWorkspace(ctx.d, all_chunks, 2, DEV, min_staging_bytes=need)
    a, b = ctx.new_out(), ctx.new_out()
    kvc.restore_async(ctx.d, ctx.tables, all_chunks, a, rws)
    kvc.restore_async(ctx.d, ctx.tables, all_chunks[::-1], b, rws)
    kvc.read_status(rws.status, "kvc_restore")
    np.testing.assert_array_equal(a.cpu().numpy().view(np.uint16), ctx.oout)
    np.testing.assert_array_equal(b.cpu().numpy().view(np.uint16), ctx.oout)


def test_restore_one_stream(ctx):
    """Copy and compute on the same stream: no overlap, same result."""
    chunks = kvc.host_chunks(ctx.enc, ctx.host)
    rws = kvc.RestoreWorkspace(ctx.d, chunks, 3, DEV)
    out = ctx.new_out()
    s = torch.cuda.current_stream()
    arr = kvc._host_array(chunks)
    code = kvc.lib().kvc_restore(ctypes.byref(ctx.d), ctx.tables.data_ptr(), arr, len(chunks), 3,
                                 out.data_ptr(), ctx.cfg.n_tokens, rws.staging.data_ptr(),
                                 rws.staging_bytes, rws.ws.data_ptr(), rws.ws_bytes,
                                 rws.status.data_ptr(), ctypes.c_void_p(s.cuda_stream),
                                 ctypes.c_void_p(s.cuda_stream), None)
    assert code == kvc.OK
    kvc.read_status(rws.status, "kvc_restore")
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), ctx.oout)


def test_restore_batch_events(ctx):
    """Each batch's event completes, in order, once the compute stream has
    passed it."""
    chunks = kvc.host_chunks(ctx.enc, ctx.host)
    rws = kvc.RestoreWorkspace(ctx.d, chunks, 4, DEV)
    ev = kvc.HipEvents(3)  # 9 chunks in batches of 4: 3 batches
    out = ctx.new_out()
    kvc.restore_async(ctx.d, ctx.tables, chunks, out, rws, events=ev)
    ev.synchronize(0)
    torch.cuda.current_stream().synchronize()
    assert all(ev.query(i) for i in range(3))
    kvc.read_status(rws.status, "kvc_restore")
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), ctx.oout)


def test_restore_reports_corrupt_later_batch(ctx):
    """A bad magic in chunk 5 (the third batch of 2) is reported even though
    the earlier batches decode cleanly; the host copy is restored after."""
    k = 5
    pos = ctx.enc.offsets[k]
    ctx.host[pos] ^= 0xFF
    try:
        with pytest.raises(kvc.KvcError) as e:
            kvc.restore(ctx.d, ctx.tables, kvc.host_chunks(ctx.enc, ctx.host), ctx.cfg.n_tokens,
                        batch=2)
        assert e.value.code == kvc.ERR_CORRUPT_STREAM
    finally:
        ctx.host[pos] ^= 0xFF

"""Several requests decoded in one call (kvc_decode_multi) against the CPU
oracle, through the C ABI.

Three contexts of one model (one profiled set of tables) with different
contents and lengths are encoded by the oracle; all their chunks, shuffled,
go to one kvc_decode_multi call, each into its own request's KV cache.  Every
cache must equal the oracle's decode of that request bit for bit, and equal
what kvc_decode gives for the request alone.
"""
import numpy as np
import pytest
import torch

import kv_cache_compression_decode_amd as kvc
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


class Requests:
    def __init__(self):
        base = synth.small_config(2, 96, 3700, n_levels=3, seed_index=91)
        self.d = kvc.make_desc(base.n_layers, base.n_channels, base.delta_bits)
        od = oracle.desc_for(base)
        kvp = synth.make_profile_kv(base)
        otb = oracle.profile(od, kvp)
        self.tables = kvc.profile(self.d, torch.from_numpy(kvp.view(np.int16)).to(DEV))
        self.req = []
        for idx, T, levels in ((91, 3700, [0, 2, 1]), (92, 1600, [1, 0]), (93, 900, [2])):
            cfg = synth.small_config(2, 96, T, n_levels=3, seed_index=idx)
            kv = synth.make_kv(cfg)
            cont = oracle.encode(od, otb, kv, levels)
            want = oracle.decode(od, otb, cont, levels, T)
            offs = np.concatenate([[0], np.cumsum([len(c) for c in cont])])
            enc = kvc.Encoded(torch.from_numpy(np.concatenate(cont)).to(DEV),
                              [int(x) for x in offs], levels,
                              [min(1500, T - 1500 * k) for k in range(len(cont))], 1500)
            self.req.append((T, enc, want))


@pytest.fixture(scope="module")
def reqs():
    print("\n[gpu multi] three requests", flush=True)
    return Requests()


def test_multi_bit_exact_per_request(reqs):
    outs = [torch.zeros((2, 2, T, 96), dtype=torch.int16, device=DEV) for T, _, _ in reqs.req]
    chunks = []
    for (T, enc, _), out in zip(reqs.req, outs):
        chunks += kvc.request_chunks(enc, out)
    order = np.random.default_rng(5).permutation(len(chunks))
    kvc.decode_multi(reqs.d, reqs.tables, [chunks[i] for i in order])
    for (T, enc, want), out in zip(reqs.req, outs):
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), want)


def test_multi_equals_single_request_decodes(reqs):
    outs = [torch.zeros((2, 2, T, 96), dtype=torch.int16, device=DEV) for T, _, _ in reqs.req]
    chunks = []
    for (T, enc, _), out in zip(reqs.req, outs):
        chunks += kvc.request_chunks(enc, out)
    kvc.decode_multi(reqs.d, reqs.tables, chunks)
    for (T, enc, _), out in zip(reqs.req, outs):
        single = kvc.decode(reqs.d, reqs.tables, kvc.chunk_refs(enc), T)
        assert torch.equal(single, out)


def test_multi_subsets_to_other_positions(reqs):
    """A request may receive only some chunks, at other positions; the rest
    of every cache is left untouched."""
    (T0, e0, w0), (T1, e1, w1), _ = reqs.req
    a = torch.full((2, 2, 2000, 96), 0x1234, dtype=torch.int16, device=DEV)
    b = torch.full((2, 2, 700, 96), 0x1234, dtype=torch.int16, device=DEV)
    ca = kvc.request_chunks(e0, a, chunks=[2])
    ca[0].first_token = 1000  # chunk 2 of request 0 (700 tokens) to 1000..1700
    cb = kvc.request_chunks(e1, b, chunks=[1])
    cb[0].first_token = 550   # chunk 1 of request 1 (100 tokens) to 550..650
    kvc.decode_multi(reqs.d, reqs.tables, ca + cb)
    ga, gb = a.cpu().numpy().view(np.uint16), b.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(ga[:, :, 1000:1700], w0[:, :, 3000:3700])
    np.testing.assert_array_equal(gb[:, :, 550:650], w1[:, :, 1500:1600])
    assert np.all(ga[:, :, :1000] == 0x1234) and np.all(ga[:, :, 1700:] == 0x1234)
    assert np.all(gb[:, :, :550] == 0x1234) and np.all(gb[:, :, 650:] == 0x1234)


def test_multi_reports_a_corrupt_request(reqs):
    (T0, e0, _), (T1, e1, _), _ = reqs.req
    blob = e1.blob.clone()
    blob[e1.offsets[1]] ^= 0xFF  # bad magic in request 1, chunk 1
    bad = kvc.Encoded(blob, e1.offsets, e1.levels, e1.n_tokens, 1500)
    a = torch.zeros((2, 2, T0, 96), dtype=torch.int16, device=DEV)
    b = torch.zeros((2, 2, T1, 96), dtype=torch.int16, device=DEV)
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_multi(reqs.d, reqs.tables, kvc.request_chunks(e0, a) + kvc.request_chunks(bad, b))
    assert e.value.code == kvc.ERR_CORRUPT_STREAM

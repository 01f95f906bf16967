"""GPU encode of streams whose range-coder carries run back through long
strings of 0xFF bytes (up to 100 of them; the inputs are built in
tests/carry_runs.py).  The containers must equal the oracle's byte for byte,
and decoding them must give back the input exactly (CacheGen page, 核心方法
step 3: every symbol is arithmetic coded, whatever the symbol sequence)."""
import numpy as np
import pytest
import torch

import carry_runs as cr
import kv_cache_compression_decode_amd as kvc
import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def test_carry_through_long_ff_runs_bit_exact():
    print("\n[gpu carry] 1 layer x 70 channels, group 1, chunks of 1024, runs up to 100",
          flush=True)
    od = oracle.Desc(cr.N_LAYERS, cr.N_CHANNELS, 1, cr.CHUNK, 8, ((4, 3, 2),), 15)
    d = kvc.make_desc(cr.N_LAYERS, cr.N_CHANNELS, ((4, 3, 2),), group_tokens=1,
                      chunk_tokens=cr.CHUNK)
    kvp = cr.make_profile_kv()
    kv, runs = cr.make_kv()
    assert runs.max() >= 100
    otb = oracle.profile(od, kvp)
    tables = kvc.profile(d, _t(kvp))
    assert kvc.profile_id(tables) == otb.profile_id
    levels = [0] * ((cr.N_TOKENS + cr.CHUNK - 1) // cr.CHUNK)
    ocont = oracle.encode(od, otb, kv, levels)
    for rep in range(2):  # a second call reuses nothing from the first
        enc = kvc.encode(d, tables, _t(kv), levels)
        for k, c in enumerate(ocont):
            np.testing.assert_array_equal(enc.container(k).cpu().numpy(), c)
    got = kvc.decode(d, tables, kvc.chunk_refs(enc), cr.N_TOKENS).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, kv)

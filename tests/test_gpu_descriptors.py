"""GPU parity away from the page's default constants: group and chunk sizes
and delta alphabets the descriptor allows (group_tokens in [1, chunk_tokens],
chunks up to 65,535 tokens, delta bits 2..6).  For each descriptor the GPU's
tables, containers and decoded KV must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import kv_cache_compression_decode_amd as kvc
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

# name: (layers, channels, tokens, group, chunk, delta bits per level, chunk levels, index)
CASES = {
    "every_token_an_anchor": (2, 64, 700, 1, 300, ((6, 5, 4), (4, 3, 2)), [0, 1, 0], 71),
    "groups_not_dividing_chunks": (3, 80, 2500, 7, 1000, ((5, 4, 3), (4, 3, 2)), [1, 0, 1], 72),
    "one_anchor_per_chunk": (2, 64, 600, 250, 250, ((6, 5, 4),), [0, 0, 0], 73),
    "long_chunks": (2, 64, 5000, 10, 4096, ((6, 5, 4), (5, 4, 3)), [1, 0], 74),
    "two_token_chunks": (2, 64, 9, 2, 2, ((6, 5, 4),), [0] * 5, 75),
    "smallest_alphabets": (3, 64, 1700, 10, 1500, ((2, 2, 2),), [0, 0], 76),
    "largest_alphabets": (3, 64, 1700, 5, 1500, ((6, 6, 6),), [0, 0], 77),
    # the largest chunk the descriptor allows, then a ragged one
    "longest_chunks": (2, 64, 65535 + 100, 10, 65535, ((6, 5, 4), (4, 3, 2)), [0, 1], 79),
    # one group over a whole 65,535-token chunk: one anchor, then 65,534 deltas
    "longest_group": (1, 64, 65535, 65535, 65535, ((5, 4, 3),), [0], 80),
    # the most levels a descriptor holds
    "four_levels": (3, 96, 5600, 10, 1500, ((6, 5, 4), (5, 4, 3), (4, 3, 2), (3, 2, 2)),
                    [3, 1, 2, 0], 86),
}


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


@pytest.mark.parametrize("name", sorted(CASES))
def test_descriptor_bit_exact(name):
    L, C, T, G, chunk, bits, levels, index = CASES[name]
    print(f"\n[gpu descriptor] {name}", flush=True)
    cfg = synth.small_config(L, C, T, n_levels=len(bits), seed_index=index)
    kv = synth.make_kv(cfg)
    kvp = synth.make_profile_kv(cfg)
    od = oracle.Desc(L, C, G, chunk, 8, tuple(tuple(b) for b in bits), 15)
    d = kvc.make_desc(L, C, bits, group_tokens=G, chunk_tokens=chunk)
    otb = oracle.profile(od, kvp)
    tables = kvc.profile(d, _t(kvp))
    assert kvc.profile_id(tables) == otb.profile_id
    ocont = oracle.encode(od, otb, kv, levels)
    enc = kvc.encode(d, tables, _t(kv), levels)
    for k, c in enumerate(ocont):
        np.testing.assert_array_equal(enc.container(k).cpu().numpy(), c)
    want = oracle.decode(od, otb, ocont, levels, T)
    got = kvc.decode(d, tables, kvc.chunk_refs(enc), T).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_many_chunks_in_one_call():
    """140 chunks of 10 tokens: the chunk table reaches the device in three
    batches of at most 64 and each channel block's chunks split into
    several groups (at most four pairs per wave); tables, containers and the
    decoded KV must still equal the oracle's, and so must a decode of the
    chunks in reverse order through kvc_decode_multi."""
    L, C, T, G, chunk = 2, 64, 1400, 5, 10
    print("\n[gpu descriptor] 140 chunks", flush=True)
    cfg = synth.small_config(L, C, T, n_levels=3, seed_index=78)
    kv = synth.make_kv(cfg)
    kvp = synth.make_profile_kv(cfg)
    bits = ((6, 5, 4), (5, 4, 3), (4, 3, 2))
    levels = [(k * 7) % 3 for k in range(T // chunk)]
    od = oracle.Desc(L, C, G, chunk, 8, bits, 15)
    d = kvc.make_desc(L, C, bits, group_tokens=G, chunk_tokens=chunk)
    otb = oracle.profile(od, kvp)
    tables = kvc.profile(d, _t(kvp))
    ocont = oracle.encode(od, otb, kv, levels)
    enc = kvc.encode(d, tables, _t(kv), levels)
    for k, c in enumerate(ocont):
        np.testing.assert_array_equal(enc.container(k).cpu().numpy(), c)
    want = oracle.decode(od, otb, ocont, levels, T)
    got = kvc.decode(d, tables, kvc.chunk_refs(enc), T).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    out = torch.zeros((L, 2, T, C), dtype=torch.int16, device=DEV)
    kvc.decode_multi(d, tables, kvc.request_chunks(enc, out)[::-1])
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), want)

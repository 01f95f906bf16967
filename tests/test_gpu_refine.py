"""GPU parity of the incremental refinement layer (CacheGen page, 局限与
Future Work: low-quality KV first, refinement bits after; reading R19):
the GPU's refinement tables, refinement containers and the refined KV
decoded from base + refinement containers in one launch must equal the
oracle's, bit for bit, on several descriptors (ragged channel blocks, a
partial last chunk, mixed levels, group sizes 1 / 7 / 10, refinement widths
2 to 6 bits); plus decode to other positions and the error paths."""
import ctypes

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


def _check_rtables(desc_o, rtables, ort):
    S = desc_o.n_streams
    A = (1 << ort.ebits) - 1
    blob = rtables.cpu().numpy()
    sec = blob[128:].view(np.uint16).reshape(2, desc_o.n_levels, S, 64)
    for kind, want in ((0, ort.fEA), (1, ort.fED)):
        got = np.diff(sec[kind][:, :, :A + 1].astype(np.int32), axis=2)
        np.testing.assert_array_equal(got, want[:, :, :A].astype(np.int32))
        assert np.all(sec[kind][:, :, A + 1:] == 0xFFFF)
    assert kvc.refine_id(rtables) == ort.refine_id


# name: (layers, channels, tokens, group, chunk, delta bits, chunk levels, E, index)
CASES = {
    "mixed_levels_E4": (6, 96, 3700, 10, 1500, ((6, 5, 4), (5, 4, 3), (4, 3, 2)), [2, 0, 1], 4, 81),
    "E2_one_level": (3, 64, 1600, 10, 1500, ((5, 4, 3),), [0, 0], 2, 82),
    "E6_every_token_anchor": (2, 70, 900, 1, 400, ((6, 5, 4), (4, 3, 2)), [1, 0, 1], 6, 83),
    "E5_groups_of_7": (3, 130, 2100, 7, 1000, ((4, 3, 2), (6, 6, 6)), [1, 0, 1], 5, 84),
    # 60 chunks of 50 tokens: several workgroup chunk groups, each over
    # three levels
    "E6_many_small_chunks": (2, 64, 3000, 10, 50, ((6, 5, 4), (5, 4, 3), (4, 3, 2)),
                             [(7 * i) % 3 for i in range(60)], 6, 85),
    # the largest chunk the descriptor allows, then a ragged one; four levels
    "E3_longest_chunks": (2, 64, 65535 + 77, 10, 65535,
                          ((6, 5, 4), (5, 4, 3), (4, 3, 2), (3, 2, 2)), [3, 0], 3, 87),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_refinement_bit_exact(name):
    L, C, T, G, chunk, bits, levels, E, index = CASES[name]
    print(f"\n[gpu refine] {name}", flush=True)
    cfg = synth.small_config(L, C, T, n_levels=len(bits), seed_index=index)
    kv = synth.make_kv(cfg)
    kvp = synth.make_profile_kv(cfg)
    od = oracle.Desc(L, C, G, chunk, 8, tuple(tuple(b) for b in bits), 15)
    d = kvc.make_desc(L, C, bits, group_tokens=G, chunk_tokens=chunk)
    otb = oracle.profile(od, kvp)
    ort = oracle.profile_refine(od, kvp, E, otb.profile_id)
    ocont = oracle.encode(od, otb, kv, levels)
    orc = oracle.encode_refine(od, ort, kv, levels)
    want = oracle.decode_refined(od, otb, ocont, ort, orc, levels, T)

    tables = kvc.profile(d, _t(kvp))
    rtables = kvc.profile_refine(d, tables, _t(kvp), E)
    _check_rtables(od, rtables, ort)
    kv_dev = _t(kv)
    enc = kvc.encode(d, tables, kv_dev, levels)
    renc = kvc.encode_refine(d, rtables, E, kv_dev, levels)
    for k, c in enumerate(orc):
        np.testing.assert_array_equal(renc.container(k).cpu().numpy(), c, err_msg=f"chunk {k}")
    got = kvc.decode_refined(d, tables, rtables, E, kvc.refined_chunk_refs(enc, renc), T)
    np.testing.assert_array_equal(got.cpu().numpy().view(np.uint16), want)


def test_refined_chunks_to_other_positions():
    L, C, T, G, chunk, bits, levels, E, index = CASES["mixed_levels_E4"]
    print("\n[gpu refine] chunks to other positions", flush=True)
    cfg = synth.small_config(L, C, T, n_levels=len(bits), seed_index=index)
    kv = synth.make_kv(cfg)
    kvp = synth.make_profile_kv(cfg)
    od = oracle.desc_for(cfg)
    d = kvc.make_desc(L, C, bits)
    otb = oracle.profile(od, kvp)
    ort = oracle.profile_refine(od, kvp, E, otb.profile_id)
    ocont = oracle.encode(od, otb, kv, levels)
    orc = oracle.encode_refine(od, ort, kv, levels)
    tables = kvc.profile(d, _t(kvp))
    rtables = kvc.profile_refine(d, tables, _t(kvp), E)
    enc = kvc.encode(d, tables, _t(kv), levels)
    renc = kvc.encode_refine(d, rtables, E, _t(kv), levels)
    # chunk 2 (700 tokens) to token 0, chunk 0 to token 800
    refs = kvc.refined_chunk_refs(enc, renc, chunks=[2, 0], first_tokens=[0, 800])
    got = kvc.decode_refined(d, tables, rtables, E, refs, 2400).cpu().numpy().view(np.uint16)
    want = np.zeros((L, 2, 2400, C), np.uint16)
    oracle.decode_refined_chunk_into(od, otb, ocont[2], ort, orc[2], 0, 700, levels[2], want)
    oracle.decode_refined_chunk_into(od, otb, ocont[0], ort, orc[0], 800, 1500, levels[0], want)
    np.testing.assert_array_equal(got, want)


def test_refinement_errors_reported():
    L, C, T, G, chunk, bits, levels, E, index = CASES["mixed_levels_E4"]
    print("\n[gpu refine] error paths", flush=True)
    cfg = synth.small_config(L, C, T, n_levels=len(bits), seed_index=index)
    kv = synth.make_kv(cfg)
    kvp = synth.make_profile_kv(cfg)
    d = kvc.make_desc(L, C, bits)
    tables = kvc.profile(d, _t(kvp))
    rtables = kvc.profile_refine(d, tables, _t(kvp), E)
    enc = kvc.encode(d, tables, _t(kv), levels)
    renc = kvc.encode_refine(d, rtables, E, _t(kv), levels)
    # refinement tables made for other base tables (the profile of another context)
    other_tables = kvc.profile(d, _t(synth.make_kv(cfg)))
    other_rt = kvc.profile_refine(d, other_tables, _t(kvp), E)
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_refined(d, tables, other_rt, E, kvc.refined_chunk_refs(enc, renc), T)
    assert e.value.code == kvc.ERR_PROFILE_MISMATCH
    # a refinement of another chunk (same level and length: chunks 0 and 1
    # hold 1,500 tokens; give chunk 1 level 0 too)
    enc2 = kvc.encode(d, tables, _t(kv), [0, 0, 1])
    renc2 = kvc.encode_refine(d, rtables, E, _t(kv), [0, 0, 1])
    refs = kvc.refined_chunk_refs(enc2, renc2, chunks=[0])
    swapped = kvc.refined_chunk_refs(enc2, renc2, chunks=[1])
    refs[0].refinement = swapped[0].refinement
    refs[0].refinement_bytes = swapped[0].refinement_bytes
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_refined(d, tables, rtables, E, refs, T)
    assert e.value.code == kvc.ERR_CORRUPT_STREAM
    # refine_bits other than the tables'
    with pytest.raises(kvc.KvcError) as e:
        kvc.encode_refine(d, rtables, 5, _t(kv), levels)
    assert e.value.code == kvc.ERR_PROFILE_MISMATCH
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_refined(d, tables, rtables, 5, kvc.refined_chunk_refs(enc, renc), T)
    assert e.value.code in (kvc.ERR_PROFILE_MISMATCH, kvc.ERR_CORRUPT_STREAM)
    # refinement records: two stream lengths changed by +-4 (the sum agrees,
    # both streams end wrongly)
    S = d.n_streams
    bad = renc.blob.clone()
    rec = bad[renc.offsets[1] + 64:renc.offsets[1] + 64 + 16 * S].view(torch.int32).view(S, 4)
    rec[10, 3] -= 4
    rec[11, 3] += 4
    renc_bad = kvc.Encoded(bad, renc.offsets, renc.levels, renc.n_tokens, renc.chunk_tokens)
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_refined(d, tables, rtables, E, kvc.refined_chunk_refs(enc, renc_bad), T)
    assert e.value.code == kvc.ERR_CORRUPT_STREAM
    # refinement tables and containers consistent with each other but made
    # over other base tables
    renc_o = kvc.encode_refine(d, other_rt, E, _t(kv), levels)
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_refined(d, tables, other_rt, E, kvc.refined_chunk_refs(enc, renc_o), T)
    assert e.value.code == kvc.ERR_PROFILE_MISMATCH
    # a base container where the refinement container belongs
    with pytest.raises(kvc.KvcError) as e:
        kvc.decode_refined(d, tables, rtables, E, kvc.refined_chunk_refs(enc, enc), T)
    assert e.value.code == kvc.ERR_CORRUPT_STREAM


def test_refined_decode_of_no_chunks_is_a_no_op():
    L, C, T, G, chunk, bits, levels, E, index = CASES["E2_one_level"]
    print("\n[gpu refine] no chunks", flush=True)
    cfg = synth.small_config(L, C, T, n_levels=len(bits), seed_index=index)
    kvp = synth.make_profile_kv(cfg)
    d = kvc.make_desc(L, C, bits, group_tokens=G, chunk_tokens=chunk)
    tables = kvc.profile(d, _t(kvp))
    rtables = kvc.profile_refine(d, tables, _t(kvp), E)
    out = torch.full((L, 2, T, C), 0x1234, dtype=torch.int16, device=DEV)
    kvc.decode_refined(d, tables, rtables, E, [], T, out=out)
    assert bool((out == 0x1234).all())

"""GPU parity at the full workload sizes (the 7B-, 13B-, 34B-GQA- and 70B-GQA-shaped
workloads), through the C ABI.

Against the oracle, chunk by chunk (one chunk's oracle container and
decoded KV in host memory at a time):
 * the profiled tables, completely (every frequency of every model, and the
   profile id);
 * every chunk of every workload: the GPU container is byte-identical to the
   oracle's, and the GPU-decoded binary16 KV equals the oracle's decode of its
   own container, element by element;
 * the 13B-shaped workload is also encoded with every chunk at level 0 and at
   level 2 (its tables hold three levels): the first, middle and last chunks
   of those containers equal the oracle's, and every chunk's container
   shrinks from level 0 to level 1 to level 2;
and, for every chunk, properties that hold at any size: container invariants
(header fields, stream lengths summing to the payload) and the half-step
reconstruction bound on every element, evaluated on the GPU.
"""
import time

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


def _check_tables(d, tables, otb, od):
    S = d.n_streams
    blob = tables.cpu().numpy()
    a = blob[128:128 + S * 528].view(np.uint16).reshape(S, 264)
    np.testing.assert_array_equal(np.diff(a[:, :257].astype(np.int32), axis=1), otb.fA.astype(np.int32))
    dl = blob[128 + S * 528:].view(np.uint16).reshape(d.n_levels, S, 64)
    for lv in range(d.n_levels):
        for third in range(3):
            b = od.delta_bits[lv][third]
            A = (1 << b) - 1
            layers = [l for l in range(d.n_layers) if od.third(l) == third]
            ms = np.concatenate([np.arange(2 * l * d.n_channels, 2 * (l + 1) * d.n_channels)
                                 for l in layers])
            got = np.diff(dl[lv, ms, :A + 1].astype(np.int32), axis=1)
            np.testing.assert_array_equal(got, otb.fD[lv, ms, :A].astype(np.int32))
    assert kvc.profile_id(tables) == otb.profile_id


def _half_step_on_gpu(d, enc, kv_dev, out, cfg):
    """|x - xhat| <= step/2 + step 2^-14 + ulp16(xhat)/2 + 4 ulp32(max(|x|, |a|+step))
    for every element, step = sa (anchor tokens) or dl (delta tokens).  The
    step 2^-14 term covers the binary32 quotient x/step rounding across a
    half-integer (at most qmax 2^-23 step with qmax <= 255)."""
    S = d.n_streams
    L, C = cfg.n_layers, cfg.n_channels
    for k in range(enc.n_chunks):
        c = enc.container(k)
        n = enc.n_tokens[k]
        t0 = 1500 * k
        rec = c[64:64 + 16 * S].view(torch.float32).view(S, 4)
        sa = rec[:, 1].reshape(L, 2, 1, C)
        dl = rec[:, 2].reshape(L, 2, 1, C)
        x = kv_dev[:, :, t0:t0 + n].view(torch.float16).float()
        y = out[:, :, t0:t0 + n].view(torch.float16).float()
        assert torch.isfinite(y).all()
        is_anchor = (torch.arange(n, device=DEV) % 10 == 0).view(1, 1, n, 1)
        step = torch.where(is_anchor, sa, dl)
        # unit in the last place: binary16 (normal spacing 2^(e-11), subnormal
        # 2^-24) and binary32 (2^(e-24)) with |v| = m 2^e, m in [0.5, 1)
        _, e16 = torch.frexp(y.abs())
        ulp16 = torch.clamp(torch.ldexp(torch.ones_like(y), e16 - 11), min=2.0 ** -24)
        big = torch.maximum(x.abs(), x[:, :, ::10].abs().repeat_interleave(10, dim=2)[:, :, :n] + step)
        _, e32 = torch.frexp(big)
        ulp32 = torch.clamp(torch.ldexp(torch.ones_like(big), e32 - 24), min=2.0 ** -149)
        bound = step / 2 + step * 2.0 ** -14 + ulp16 / 2 + 4 * ulp32
        err = (x - y).abs()
        bad = (err > bound)
        assert not bad.any(), (k, int(bad.sum()), float((err - bound).max()))


def _sample_chunks(cfg):
    ks = {0, cfg.n_chunks - 1, cfg.n_chunks // 2}
    return sorted(ks)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", [synth.SHAPE_7B_9K.name, synth.SHAPE_13B_16K.name,
                                  synth.SHAPE_34B_GQA_80K.name, synth.SHAPE_70B_GQA_16K.name])
def test_full_size_workload(name):
    cfg = synth.WORKLOADS[name]
    print(f"\n[fullsize] {cfg.name}: generating", flush=True)
    p = synth.params(cfg)
    kv = synth.make_kv(cfg, p=p)
    kvp = synth.make_profile_kv(cfg, p=p)
    levels = cfg.chunk_levels()
    d = kvc.make_desc(cfg.n_layers, cfg.n_channels, cfg.delta_bits)
    od = oracle.desc_for(cfg)

    print("[fullsize] gpu profile / encode / decode", flush=True)
    kv_dev = _t(kv)
    tables = kvc.profile(d, _t(kvp))
    enc = kvc.encode(d, tables, kv_dev, levels)
    out = kvc.decode(d, tables, kvc.chunk_refs(enc), cfg.n_tokens)
    torch.cuda.synchronize()

    print("[fullsize] oracle profile", flush=True)
    otb = oracle.profile(od, kvp)
    del kvp
    _check_tables(d, tables, otb, od)

    print("[fullsize] container invariants", flush=True)
    S = d.n_streams
    for k in range(enc.n_chunks):
        hdr = oracle.parse_header(enc.container(k)[:64].cpu().numpy())
        assert hdr["magic"] == b"KVC1" and hdr["level"] == levels[k]
        assert hdr["n_tokens"] == enc.n_tokens[k] and hdr["first_token"] == 1500 * k
        assert hdr["profile_id"] == otb.profile_id
        nb = enc.container(k)[64:64 + 16 * S].view(torch.int32).view(S, 4)[:, 3].long()
        assert int(((nb + 7) // 8 * 8).sum()) == hdr["payload_bytes"]
        assert enc.offsets[k + 1] - enc.offsets[k] == 64 + 16 * S + hdr["payload_bytes"]

    print("[fullsize] half-step bound on every element", flush=True)
    _half_step_on_gpu(d, enc, kv_dev, out, cfg)

    t_start = time.time()
    for k in range(enc.n_chunks):
        print(f"[fullsize] oracle chunk {k} of {enc.n_chunks} (level {levels[k]})", flush=True)
        oc = oracle.encode_chunk(od, otb, kv, k, levels[k])
        assert np.array_equal(enc.container(k).cpu().numpy(), oc), f"container {k}"
        n = enc.n_tokens[k]
        oo = np.zeros((cfg.n_layers, 2, n, cfg.n_channels), np.uint16)
        oracle.decode_chunk_into(od, otb, oc, 0, n, levels[k], oo)
        got = out[:, :, 1500 * k:1500 * k + n].cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, oo)
        del oc, oo, got
    t_all = time.time() - t_start

    if cfg.schedule == "level1":
        sizes = [[enc.offsets[k + 1] - enc.offsets[k] for k in range(enc.n_chunks)]]
        del out
        for lv in (0, 2):
            print(f"[fullsize] every chunk at level {lv}", flush=True)
            e2 = kvc.encode(d, tables, kv_dev, [lv] * enc.n_chunks)
            sizes.insert(lv, [e2.offsets[k + 1] - e2.offsets[k] for k in range(enc.n_chunks)])
            for k in _sample_chunks(cfg):
                oc = oracle.encode_chunk(od, otb, kv, k, lv)
                assert np.array_equal(e2.container(k).cpu().numpy(), oc), f"level {lv} container {k}"
            del e2
        for k in range(enc.n_chunks):
            assert sizes[0][k] > sizes[1][k] > sizes[2][k], (k, sizes[0][k], sizes[1][k], sizes[2][k])
    ratio = cfg.fp16_bytes() / enc.total_bytes()
    print(f"[fullsize] {cfg.name}: all {enc.n_chunks} chunks bit-exact "
          f"(oracle comparison {t_all:.1f} s), compression {ratio:.3f}", flush=True)


@pytest.mark.timeout(900)
def test_full_size_refinement():
    """The refinement layer (4 bits) over the 70B-shaped workload's mixed
    levels: the refinement tables completely, the refinement containers and
    the refined KV of the first, middle and last chunks against the oracle,
    and on every element the half-refinement-step bound, evaluated on the
    GPU; the refined mean error is far below the base layer's."""
    cfg = synth.SHAPE_70B_GQA_16K
    E = 4
    print(f"\n[fullsize refine] {cfg.name}: generating", flush=True)
    p = synth.params(cfg)
    kv = synth.make_kv(cfg, p=p)
    kvp = synth.make_profile_kv(cfg, p=p)
    levels = cfg.chunk_levels()
    d = kvc.make_desc(cfg.n_layers, cfg.n_channels, cfg.delta_bits)
    od = oracle.desc_for(cfg)

    print("[fullsize refine] gpu profile / encode / decode", flush=True)
    kv_dev = _t(kv)
    kvp_dev = _t(kvp)
    tables = kvc.profile(d, kvp_dev)
    rtables = kvc.profile_refine(d, tables, kvp_dev, E)
    del kvp_dev
    enc = kvc.encode(d, tables, kv_dev, levels)
    renc = kvc.encode_refine(d, rtables, E, kv_dev, levels)
    base = kvc.decode(d, tables, kvc.chunk_refs(enc), cfg.n_tokens)
    ref = kvc.decode_refined(d, tables, rtables, E, kvc.refined_chunk_refs(enc, renc), cfg.n_tokens)
    torch.cuda.synchronize()

    print("[fullsize refine] oracle profiles", flush=True)
    otb = oracle.profile(od, kvp)
    ort = oracle.profile_refine(od, kvp, E, otb.profile_id)
    del kvp
    S = d.n_streams
    A = (1 << E) - 1
    blob = rtables.cpu().numpy()
    sec = blob[128:].view(np.uint16).reshape(2, d.n_levels, S, 64)
    for kind, want in ((0, ort.fEA), (1, ort.fED)):
        got = np.diff(sec[kind][:, :, :A + 1].astype(np.int32), axis=2)
        np.testing.assert_array_equal(got, want[:, :, :A].astype(np.int32))
    assert kvc.refine_id(rtables) == ort.refine_id

    print("[fullsize refine] half-refinement-step bound on every element", flush=True)
    L, C = cfg.n_layers, cfg.n_channels
    err_b = err_r = 0.0
    for k in range(renc.n_chunks):
        n = renc.n_tokens[k]
        t0 = 1500 * k
        rec = renc.container(k)[64:64 + 16 * S].view(torch.float32).view(S, 4)
        Da = rec[:, 0].reshape(L, 2, 1, C).double()
        Dd = rec[:, 1].reshape(L, 2, 1, C).double()
        is_anchor = (torch.arange(n, device=DEV) % 10 == 0).view(1, 1, n, 1)
        D = torch.where(is_anchor, Da, Dd)
        x = kv_dev[:, :, t0:t0 + n].view(torch.float16).double()
        y = ref[:, :, t0:t0 + n].view(torch.float16).double()
        xb = base[:, :, t0:t0 + n].view(torch.float16).double()
        assert torch.isfinite(y).all()
        _, e16 = torch.frexp(y.abs())
        ulp16 = torch.clamp(torch.ldexp(torch.ones_like(y), e16 - 11), min=2.0 ** -24)
        big = x.abs() + 8 * D + xb.abs()
        _, e32 = torch.frexp(big)
        ulp32 = torch.clamp(torch.ldexp(torch.ones_like(big), e32 - 24), min=2.0 ** -149)
        bound = D / 2 + D * 2.0 ** -14 + ulp16 / 2 + 4 * ulp32
        bad = (x - y).abs() > bound
        assert not bad.any(), (k, int(bad.sum()))
        err_b += float((x - xb).abs().sum())
        err_r += float((x - y).abs().sum())
        del x, y, xb, big, bound, bad, D
    assert err_r < err_b / 5, (err_r, err_b)

    for k in _sample_chunks(cfg):
        print(f"[fullsize refine] oracle chunk {k} (level {levels[k]})", flush=True)
        oc = oracle.encode_chunk(od, otb, kv, k, levels[k])
        orc = oracle.encode_refine_chunk(od, ort, kv, k, levels[k])
        assert np.array_equal(renc.container(k).cpu().numpy(), orc), f"refinement container {k}"
        n = renc.n_tokens[k]
        oo = np.zeros((cfg.n_layers, 2, n, cfg.n_channels), np.uint16)
        oracle.decode_refined_chunk_into(od, otb, oc, ort, orc, 0, n, levels[k], oo)
        got = ref[:, :, 1500 * k:1500 * k + n].cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, oo)
        del oc, orc, oo, got
    print(f"[fullsize refine] refinement {renc.total_bytes() / 1e9:.3f} GB over base "
          f"{enc.total_bytes() / 1e9:.3f} GB; mean |error| {err_b / kv.size:.3e} -> "
          f"{err_r / kv.size:.3e}", flush=True)

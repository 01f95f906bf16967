"""Pins of the oracle's refinement layer (reading R19 of the CacheGen page's
future-work item in 局限与 Future Work: send a low-quality KV first, then
refinement bits).

The refinement layer re-quantizes, per stream, the residual between the input
and the base layer's binary32 reconstruction, with one scale for anchor
tokens and one for the others, and range-codes the symbols with their own
profiled models.  What fixes it, independently of the oracle's code:
 * the base layer is untouched: the binary16 rounding of the base
   reconstruction the refinement starts from is the base decode, bit for
   bit, and a refinement of all-zero symbols gives the base decode back;
 * every refinement symbol and scale equals an exact-rational restatement
   (each binary32 operation rounded once, rint half to even);
 * the refined output is within half a refinement step of the input (plus
   the binary16 and binary32 rounding terms), and the refinement step is
   about 1/(2 Me) of the base step;
 * the refinement streams meet the range coder's redundancy bound;
 * headers, records, the refinement id's definition and mismatch detection.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from fp_exact import round_f16_bits, round_f32

TOT = 1 << 15
RED = -math.log2(1 - 2.0 ** -9)


@pytest.fixture(scope="module")
def mixed():
    cfg = synth.small_config(6, 96, 3700, n_levels=3, schedule="mixed", seed_index=98)
    d = oracle.desc_for(cfg)
    kv = synth.make_kv(cfg)
    kvp = synth.make_profile_kv(cfg)
    tb = oracle.profile(d, kvp)
    rt = oracle.profile_refine(d, kvp, 4, tb.profile_id)
    levels = [2, 0, 1]
    cont = oracle.encode(d, tb, kv, levels)
    rcont = oracle.encode_refine(d, rt, kv, levels)
    base = oracle.decode(d, tb, cont, levels, cfg.n_tokens)
    ref = oracle.decode_refined(d, tb, cont, rt, rcont, levels, cfg.n_tokens)
    return cfg, d, kv, tb, rt, levels, cont, rcont, base, ref


def _exact_refine(x16, G, b, E):
    """Base quantizer then refinement quantizer in exact arithmetic."""
    x = [Fraction(float(v)) for v in x16]
    n = len(x)
    M, Me = (1 << (b - 1)) - 1, (1 << (E - 1)) - 1
    anchors = x[::G]
    lo, hi = min(anchors), max(anchors)
    sa = round_f32(round_f32(hi - lo) / 255)
    xh = [None] * n
    qa = {}
    for j in range(0, n, G):
        q = 0 if sa == 0 else min(max(round(round_f32(round_f32(x[j] - lo) / sa)), 0), 255)
        qa[j] = q
        xh[j] = round_f32(q * sa + lo)
    d = {j: round_f32(x[j] - xh[j - j % G]) for j in range(n) if j % G}
    dl = round_f32(max((abs(v) for v in d.values()), default=Fraction(0)) / M)
    for j, v in d.items():
        q = 0 if dl == 0 else min(max(round(round_f32(v / dl)), -M), M)
        xh[j] = round_f32(q * dl + xh[j - j % G])
    e = [round_f32(x[j] - xh[j]) for j in range(n)]
    Da = round_f32(max(abs(e[j]) for j in range(0, n, G)) / Me)
    Dd = round_f32(max((abs(e[j]) for j in range(n) if j % G), default=Fraction(0)) / Me)
    esym, y = [], []
    for j in range(n):
        D = Da if j % G == 0 else Dd
        q = 0 if D == 0 else min(max(round(round_f32(e[j] / D)), -Me), Me)
        esym.append(q + Me)
        y.append(round_f16_bits(round_f32(q * D + xh[j])))
    return Da, Dd, esym, y


def test_refinement_quantizer_exact():
    rng = np.random.default_rng(31)
    for trial in range(120):
        n = int(rng.integers(1, 40))
        G = int(rng.integers(1, 12))
        b = int(rng.integers(2, 7))
        E = int(rng.integers(2, 7))
        scale = float(np.exp(rng.uniform(-12, 5)))
        x16 = (rng.standard_normal(n).cumsum() * scale).astype(np.float16)
        if not np.all(np.isfinite(x16)):
            continue
        x32 = x16.astype(np.float32)
        lo, sa, dl, sym, Da, Dd, esym = oracle.refine_quantize(x32, G, b, E)
        eDa, eDd, eesym, ey = _exact_refine(x16, G, b, E)
        assert Fraction(float(Da)) == eDa and Fraction(float(Dd)) == eDd, trial
        assert esym.tolist() == eesym, trial
        y = oracle.refine_dequantize(sym, esym, G, b, E, lo, sa, dl, Da, Dd)
        assert y.tolist() == ey, trial


def test_refinement_quantizer_ties_to_even():
    """Residuals at exact half-integers of the refinement step.  Constant
    anchors (so xh = lo = 0 exactly) and 2-bit base deltas whose step is 4
    (one delta of 4), so that every other delta, |d| <= 0.4375 < 2, is
    quantized to 0 by the base layer and its residual is the value itself.
    One residual of 0.4375 = 7 x 2^-4 makes the refinement step (E = 4,
    Me = 7) exactly 2^-4, and the others sit at (k + 1/2) 2^-4."""
    vals = [4.0, 0.4375] + [(k + 0.5) * 0.0625 for k in range(-7, 7)]
    x = []
    for i in range(0, len(vals), 9):
        x.append(0.0)
        x.extend(vals[i:i + 9])
    x16 = np.array(x, np.float16)
    assert np.all(x16.astype(np.float64) == np.array(x))
    x32 = x16.astype(np.float32)
    lo, sa, dl, sym, Da, Dd, esym = oracle.refine_quantize(x32, 10, 2, 4)
    assert Dd == np.float32(0.0625) and Da == 0
    eDa, eDd, eesym, ey = _exact_refine(x16, 10, 2, 4)
    assert esym.tolist() == eesym
    got = [int(esym[j]) - 7 for j in range(len(x)) if j % 10]
    for v, q in zip(vals[2:], got[2:]):
        r = Fraction(v) / Fraction(1, 16)
        assert r.denominator == 2 and q == round(r) and q % 2 == 0


def test_base_reconstruction_rounds_to_the_base_decode(mixed):
    """A refinement of zeros (every symbol Me) gives the base decode back:
    the refinement starts from the base layer's own binary32 values."""
    cfg, d, kv, tb, rt, levels, cont, rcont, base, ref = mixed
    x = kv.view(np.float16).astype(np.float32)
    rng = np.random.default_rng(5)
    for _ in range(60):
        l = int(rng.integers(0, d.n_layers))
        kvi = int(rng.integers(0, 2))
        c = int(rng.integers(0, d.n_channels))
        k = int(rng.integers(0, len(levels)))
        t0 = 1500 * k
        n = min(1500, cfg.n_tokens - t0)
        b = d.bits(levels[k], l)
        lo, sa, dl, sym, Da, Dd, esym = oracle.refine_quantize(x[l, kvi, t0:t0 + n, c], 10, b, 4)
        zero = np.full(n, (1 << 3) - 1, np.int32)
        y0 = oracle.refine_dequantize(sym, zero, 10, b, 4, lo, sa, dl, Da, Dd)
        np.testing.assert_array_equal(y0, base[l, kvi, t0:t0 + n, c])
        np.testing.assert_array_equal(oracle.dequantize(sym, 10, b, lo, sa, dl), y0)


def _ulp16(bits):
    return np.spacing(np.abs(bits.view(np.float16))).astype(np.float64)


def _ulp32(v):
    return np.spacing(np.abs(np.asarray(v, np.float32))).astype(np.float64)


def test_refined_within_half_a_refinement_step(mixed):
    cfg, d, kv, tb, rt, levels, cont, rcont, base, ref = mixed
    x = kv.view(np.float16).astype(np.float64)
    y = ref.view(np.float16).astype(np.float64)
    for k, rc in enumerate(rcont):
        t0 = 1500 * k
        n = oracle.parse_refine_header(rc)["n_tokens"]
        rec = oracle.refine_records(d, rc)
        shp = (d.n_layers, 2, 1, d.n_channels)
        Da = rec["Da"].reshape(shp).astype(np.float64)
        Dd = rec["Dd"].reshape(shp).astype(np.float64)
        is_anchor = (np.arange(n) % 10 == 0)[None, None, :, None]
        D = np.where(is_anchor, Da, Dd)
        xs, ys = x[:, :, t0:t0 + n], y[:, :, t0:t0 + n]
        big = np.abs(xs) + 8 * D + np.abs(base[:, :, t0:t0 + n].view(np.float16).astype(np.float64))
        bound = D / 2 + D * 2.0 ** -14 + _ulp16(ref[:, :, t0:t0 + n]) / 2 + 4 * _ulp32(big)
        assert np.all(np.abs(xs - ys) <= bound), k


def test_refinement_step_is_a_fraction_of_the_base_step(mixed):
    """max |e| is the base layer's half step (plus rounding), so
    Me D <= step/2 (1 + 2^-12) + a few binary32 ulps."""
    cfg, d, kv, tb, rt, levels, cont, rcont, base, ref = mixed
    x = kv.view(np.float16).astype(np.float64)
    for k, (c, rc) in enumerate(zip(cont, rcont)):
        t0 = 1500 * k
        n = oracle.parse_header(c)["n_tokens"]
        r = oracle.records(d, c)
        rr = oracle.refine_records(d, rc)
        xmax = np.abs(x[:, :, t0:t0 + n]).max(axis=2).reshape(-1)
        slack = 8 * _ulp32(xmax + r["sa"].astype(np.float64) * 256 + r["dl"].astype(np.float64) * 64)
        assert np.all(7 * rr["Da"].astype(np.float64) <= r["sa"] / 2 * (1 + 2.0 ** -12) + slack)
        assert np.all(7 * rr["Dd"].astype(np.float64) <= r["dl"] / 2 * (1 + 2.0 ** -12) + slack)


def test_refinement_error_far_below_base_error(mixed):
    cfg, d, kv, tb, rt, levels, cont, rcont, base, ref = mixed
    x = kv.view(np.float16).astype(np.float64)
    eb = np.abs(base.view(np.float16).astype(np.float64) - x).mean()
    er = np.abs(ref.view(np.float16).astype(np.float64) - x).mean()
    assert er < eb / 5


def test_refinement_coder_bound(mixed):
    cfg, d, kv, tb, rt, levels, cont, rcont, base, ref = mixed
    A = (1 << rt.ebits) - 1
    for k, rc in enumerate(rcont):
        n = oracle.parse_refine_header(rc)["n_tokens"]
        rec = oracle.refine_records(d, rc)
        ids = np.arange(0, d.n_streams, 5)
        esyms = oracle.decode_refine_symbols(d, rt, rc, ids, n)
        for i, m in enumerate(ids):
            fa = rt.fEA[levels[k], m, :A].astype(np.float64)
            fd = rt.fED[levels[k], m, :A].astype(np.float64)
            ideal = sum(-math.log2((fa if j % 10 == 0 else fd)[esyms[i, j]] / TOT) for j in range(n))
            bits = 8 * int(rec["nbytes"][m])
            assert ideal + 24 - 1e-6 <= bits <= ideal + n * RED + 33 + 1e-6


def test_refinement_container_structure(mixed):
    cfg, d, kv, tb, rt, levels, cont, rcont, base, ref = mixed
    S = d.n_streams
    for k, rc in enumerate(rcont):
        h = oracle.parse_refine_header(rc)
        assert h["magic"] == b"KVCR" and h["version"] == 1 and h["ebits"] == 4
        assert h["level"] == levels[k] and h["delta_bits"] == d.delta_bits[levels[k]]
        assert h["first_token"] == 1500 * k and h["n_tokens"] == min(1500, cfg.n_tokens - 1500 * k)
        assert h["refine_id"] == rt.refine_id and h["base_id"] == tb.profile_id
        rec = oracle.refine_records(d, rc)
        assert np.all(rec["zero"] == 0) and np.all(rec["nbytes"] >= 4)
        assert len(rc) == 64 + 16 * S + h["payload_bytes"]
        assert int(((rec["nbytes"].astype(np.int64) + 7) // 8 * 8).sum()) == h["payload_bytes"]


def test_refinement_tables_and_id(mixed):
    cfg, d, kv, tb, rt, levels, cont, rcont, base, ref = mixed
    A = (1 << rt.ebits) - 1
    for f in (rt.fEA, rt.fED):
        assert np.all(f[:, :, :A].astype(np.int64).sum(axis=2) == TOT)
        assert f[:, :, :A].min() >= 1 and np.all(f[:, :, A:] == 0)
    # independent rendering of the id from its definition
    desc = b"".join(int(v).to_bytes(4, "little") for v in
                    (d.n_layers, d.n_channels, 10, 1500, 8, d.n_levels, 15))
    desc += bytes(b for row in d.delta_bits for b in row)
    h = oracle.fnv1a64(desc)
    h = oracle.fnv1a64(rt.ebits.to_bytes(4, "little") + tb.profile_id.to_bytes(8, "little"), h)
    for row in range(2 * d.n_layers):
        hr_in = b""
        for c in range(d.n_channels):
            m = row * d.n_channels + c
            blob = b"".join(rt.fEA[lv, m, :A].astype("<u2").tobytes() +
                            rt.fED[lv, m, :A].astype("<u2").tobytes() for lv in range(d.n_levels))
            hr_in += oracle.fnv1a64(blob).to_bytes(8, "little")
        h = oracle.fnv1a64(oracle.fnv1a64(hr_in).to_bytes(8, "little"), h)
    assert h == rt.refine_id == oracle.refine_profile_id(d, rt)


def test_refinement_mismatch_and_corruption_detected(mixed):
    cfg, d, kv, tb, rt, levels, cont, rcont, base, ref = mixed
    out = np.zeros((d.n_layers, 2, cfg.n_tokens, d.n_channels), np.uint16)
    other = oracle.RefineTables(rt.fEA, rt.fED, rt.ebits, rt.refine_id ^ 1, rt.base_id)
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode_refined_chunk_into(d, tb, cont[0], other, rcont[0], 0, 1500, levels[0], out)
    assert e.value.code == oracle.ERR_PROFILE
    with pytest.raises(oracle.OracleError) as e:  # refinement of another chunk
        oracle.decode_refined_chunk_into(d, tb, cont[0], rt, rcont[1], 0, 1500, levels[0], out)
    assert e.value.code in (oracle.ERR_CORRUPT, oracle.ERR_ARG)
    bad = rcont[0].copy()
    bad[0] ^= 0xFF
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode_refined_chunk_into(d, tb, cont[0], rt, bad, 0, 1500, levels[0], out)
    assert e.value.code == oracle.ERR_CORRUPT


def test_constant_channel_refines_to_itself():
    x = np.full(23, 0.8125, np.float32)
    lo, sa, dl, sym, Da, Dd, esym = oracle.refine_quantize(x, 10, 4, 5)
    assert Da == 0 and Dd == 0 and np.all(esym == 15)
    y = oracle.refine_dequantize(sym, esym, 10, 4, 5, lo, sa, dl, Da, Dd)
    np.testing.assert_array_equal(y, np.full(23, np.float16(0.8125).view(np.uint16)))


def test_refinement_thread_count_independent(mixed):
    cfg, d, kv, tb, rt, levels, cont, rcont, base, ref = mixed
    old = oracle.get_threads()
    try:
        oracle.set_threads(1)
        rt1 = oracle.profile_refine(d, synth.make_profile_kv(cfg), 4, tb.profile_id)
        rc1 = oracle.encode_refine(d, rt1, kv, levels)
    finally:
        oracle.set_threads(old)
    assert rt1.refine_id == rt.refine_id
    for a, b in zip(rc1, rcont):
        np.testing.assert_array_equal(a, b)

"""Pins of the oracle's floating-point primitives.

The decoder's output is defined as one binary32 fused multiply-add followed
by a round-to-nearest-even conversion to binary16 (so a 0-ulp comparison is
meaningful).  The oracle implements both conversions on bit patterns; here
they are checked against numpy's IEEE casts (exhaustively) and the fused
multiply-add against exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from fp_exact import round_f16_bits as _round_f16_bits, round_f32 as _round_f32


def test_h2f_exhaustive_against_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.h2f_array(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_f2h_sample_against_numpy():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    got = oracle.f2h_array(x)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    ok = ~np.isnan(x)
    np.testing.assert_array_equal(got[ok], want[ok])


@pytest.mark.slow
def test_f2h_exhaustive_against_library_cast():
    """All 2^32 binary32 patterns, in slices, against the library cast
    (torch's CPU float32 -> float16 conversion, IEEE round to nearest even;
    numpy's cast is used on a random sample above).  NaNs: only NaN-ness."""
    import torch

    step = 1 << 24
    base = torch.arange(step, dtype=torch.int32)
    xi = torch.empty(step, dtype=torch.int32)
    half = torch.empty(step, dtype=torch.float16)
    got = np.empty(step, np.uint16)
    for start in range(0, 1 << 32, step):
        signed = start - (1 << 32) if start >= (1 << 31) else start
        torch.add(base, signed, out=xi)  # the patterns start .. start+step-1
        x = xi.view(torch.float32)
        half.copy_(x)
        want = half.view(torch.int16).numpy().view(np.uint16)
        oracle.f2h_patterns(start, step, got)
        nan = torch.isnan(x).numpy()
        if nan.any():
            assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)
        bad = np.nonzero((got != want) & ~nan)[0]
        assert bad.size == 0, (hex(start), bad[:4], got[bad[:4]], want[bad[:4]])


def test_round_helpers_agree_with_numpy():
    rng = np.random.default_rng(3)
    for x in rng.standard_normal(300) * np.exp(rng.uniform(-20, 10, 300)):
        f = Fraction(float(x))
        assert float(_round_f32(f)) == float(np.float32(x))


def test_dequantize_is_one_fma_then_rne_to_half():
    """Decode arithmetic: anchor = fp16(fma(qa, sa, lo)); delta =
    fp16(fma(q, dl, ahat)) with the binary32 ahat, checked with exact
    rationals (one binary32 rounding of the exact a*b+c, then one binary16
    rounding)."""
    rng = np.random.default_rng(11)
    G, b = 10, 5
    M = (1 << (b - 1)) - 1
    for trial in range(200):
        n = int(rng.integers(1, 40))
        sym = np.empty(n, np.int32)
        for j in range(n):
            sym[j] = rng.integers(0, 256) if j % G == 0 else rng.integers(0, 2 * M + 1)
        scale = float(np.exp(rng.uniform(-12, 6)))
        lo = np.float32(rng.standard_normal() * scale)
        sa = np.float32(abs(rng.standard_normal()) * scale / 255)
        dl = np.float32(abs(rng.standard_normal()) * scale / M)
        got = oracle.dequantize(sym, G, b, lo, sa, dl)
        ahat = None
        for j in range(n):
            if j % G == 0:
                ahat = _round_f32(Fraction(int(sym[j])) * Fraction(float(sa)) + Fraction(float(lo)))
                want = _round_f16_bits(ahat)
            else:
                v = _round_f32(Fraction(int(sym[j]) - M) * Fraction(float(dl)) + ahat)
                want = _round_f16_bits(v)
            assert int(got[j]) == want, (trial, j)


def test_fnv1a64_published_vectors():
    # Test vectors from the FNV reference test suite (64-bit FNV-1a).
    assert oracle.fnv1a64(b"") == 0xCBF29CE484222325
    assert oracle.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert oracle.fnv1a64(b"foobar") == 0x85944171F73967E8

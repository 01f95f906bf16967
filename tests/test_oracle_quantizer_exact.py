"""Exact pins of the oracle's quantizer.

CacheGen page, 核心方法, layer-wise quantization paragraph: each group's
anchor is kept at 8 bits, the other tokens are quantized as deltas to the
anchor, more coarsely in deeper layer groups.  The quantizer the codec takes
from that paragraph (one affine 8-bit anchor scale and one symmetric delta
scale per stream, deltas against the reconstructed anchor) is restated here
with exact rational arithmetic, independently of the oracle's C code:

* every binary32 operation (subtraction, division, fused multiply-add) is the
  exact rational result rounded once to binary32 (``round_f32``);
* ``rint`` is round-half-to-even of that binary32 value (Python's ``round`` of
  a ``Fraction``).

Every output of the oracle's quantizer (``lo``, ``sa``, ``dl`` and each
symbol) must equal this restatement exactly.  Besides random streams the
inputs include quotients that are exact half-integers (where ties-to-even and
ties-away-from-zero differ) and quotients one binary32 step either side of a
half-integer (where dividing by multiplying with a rounded reciprocal can move
the result across the half).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from fp_exact import round_f32


def _exact_quantize(x16, G, b):
    """The quantizer in exact arithmetic: x16 are binary16 values (floats)."""
    x = [Fraction(float(v)) for v in x16]
    n = len(x)
    M = (1 << (b - 1)) - 1
    anchors = x[::G]
    lo, hi = min(anchors), max(anchors)
    sa = round_f32(round_f32(hi - lo) / 255)
    sym = [0] * n
    ahat = [None] * n
    for j in range(0, n, G):
        qa = 0
        if sa != 0:
            qa = min(max(round(round_f32(round_f32(x[j] - lo) / sa)), 0), 255)
        sym[j] = qa
        ahat[j] = round_f32(qa * sa + lo)
    d = {j: round_f32(x[j] - ahat[j - j % G]) for j in range(n) if j % G}
    maxabs = max((abs(v) for v in d.values()), default=Fraction(0))
    dl = round_f32(maxabs / M)
    for j, v in d.items():
        q = 0
        if dl != 0:
            q = min(max(round(round_f32(v / dl)), -M), M)
        sym[j] = q + M
    return lo, sa, dl, sym


def _check(x16, G, b):
    x32 = np.asarray(x16, np.float16).astype(np.float32)
    lo, sa, dl, sym = oracle.quantize(x32, G, b)
    elo, esa, edl, esym = _exact_quantize(x32, G, b)
    assert Fraction(float(lo)) == elo
    assert Fraction(float(sa)) == esa, (float(sa), float(esa))
    assert Fraction(float(dl)) == edl, (float(dl), float(edl))
    assert sym.tolist() == esym
    return esym


def test_random_streams_exact():
    """Random walks over many magnitudes (subnormal binary16 inputs included),
    every group size from 1 to 12 and every delta width 2..6."""
    rng = np.random.default_rng(2024)
    for trial in range(300):
        n = int(rng.integers(1, 61))
        G = int(rng.integers(1, 13))
        b = int(rng.integers(2, 7))
        scale = float(np.exp(rng.uniform(-17, 6)))
        x = (rng.standard_normal(n).cumsum() * scale + rng.normal() * scale * 3)
        x16 = x.astype(np.float16)
        if not np.all(np.isfinite(x16)):
            continue
        _check(x16, G, b)


def _ties_cover_even_and_odd(pairs):
    """pairs: (quotient, symbol).  Both parities of the lower integer occur,
    so ties-to-even differs from rounding half away from zero somewhere."""
    low = {int(q - Fraction(1, 2)) % 2 for q, _ in pairs}
    assert low == {0, 1}


@pytest.mark.parametrize("s, e", [(1, 4), (3, 6), (5, 7), (7, 8), (1, 10), (3, 1), (5, 12), (7, 14)])
def test_anchor_quotients_at_half_integers(s, e):
    """Anchors at lo + (k + 1/2) sa for sa = s 2^-e: the binary32 quotient is
    exactly k + 1/2 and the symbol is the even neighbour."""
    sa = Fraction(s, 2 ** e)
    hi = 255 * sa
    assert float(np.float16(float(hi))) == float(hi)
    ks = [k for k in range(0, 255) if float(np.float16(float((2 * k + 1) * sa / 2))) == float((2 * k + 1) * sa / 2)]
    assert len(ks) >= 20
    x = []
    for k in ks:
        x.append(float((2 * k + 1) * sa / 2))
    # anchors every 1 token: lo = 0 first, hi last
    x16 = np.array([0.0] + x + [float(hi)], np.float16)
    sym = _check(x16, 1, 4)
    pairs = [(Fraction(2 * k + 1, 2), sym[i + 1]) for i, k in enumerate(ks)]
    for q, v in pairs:
        assert v == round(q) and v % 2 == 0
    _ties_cover_even_and_odd(pairs)


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6])
@pytest.mark.parametrize("s, e", [(1, 6), (3, 8), (5, 9), (7, 10), (9, 11)])
def test_delta_quotients_at_half_integers(b, s, e):
    """Constant anchors (sa = 0, ahat = lo = 0) and deltas at (k + 1/2) dl for
    dl = s 2^-e, one delta at M dl so that maxabs / M is exactly dl."""
    M = (1 << (b - 1)) - 1
    dl = Fraction(s, 2 ** e)
    vals = [float(M * dl)] + [float((2 * k + 1) * dl / 2) for k in range(-M, M)]
    for v in vals:
        assert float(np.float16(v)) == v
    G = 10
    x = []
    for i in range(0, len(vals), G - 1):
        x.append(0.0)
        x.extend(vals[i:i + G - 1])
    sym = _check(np.array(x, np.float16), G, b)
    if M >= 1:
        got = [sym[j] - M for j in range(len(x)) if j % G]
        for v, q in zip(vals, got):
            r = Fraction(v) / dl
            if r.denominator == 2:
                assert q == round(r) and q % 2 == 0
    if M >= 2:
        _ties_cover_even_and_odd([(Fraction(2 * k + 1, 2), 0) for k in range(-M, M)])


def _near_half_anchors(lo, hi):
    """binary16 values x in [lo, hi] whose binary32 quotient (x - lo) / sa
    lies one binary32 step either side of a half-integer (found with numpy's
    IEEE binary32 operations, checked exactly below)."""
    sa = np.float32(np.float32(hi) - np.float32(lo)) / np.float32(255)
    xs = np.arange(0, 1 << 16, dtype=np.uint16).view(np.float16)
    xs = xs[np.isfinite(xs)]
    xs = xs[(xs >= np.float16(lo)) & (xs <= np.float16(hi))].astype(np.float32)
    q = (xs - np.float32(lo)) / sa
    half = np.floor(q) + np.float32(0.5)
    up = np.nextafter(half, np.float32(np.inf))
    down = np.nextafter(half, np.float32(-np.inf))
    return xs[(q == up) | (q == down)]


def test_anchor_quotients_one_step_from_half_integers():
    """Quotients one binary32 step above or below k + 1/2: the symbol is the
    integer on that side.  Some of these quotients differ from the product
    with the rounded reciprocal 1/sa in which integer they round to, so a
    quantizer dividing by multiplication would fail here."""
    rng = np.random.default_rng(77)
    found = 0
    recip_differs = 0
    for _ in range(400):
        lo = float(np.float16(rng.uniform(-4, 0)))
        hi = float(np.float16(lo + rng.uniform(0.5, 12)))
        xs = _near_half_anchors(lo, hi)
        if len(xs) == 0:
            continue
        x16 = np.concatenate([[lo], xs, [hi]]).astype(np.float16)
        sym = _check(x16, 1, 5)
        found += len(xs)
        sa = np.float32(np.float32(hi) - np.float32(lo)) / np.float32(255)
        inv = np.float32(1) / sa
        prod = (xs - np.float32(lo)) * inv
        recip_differs += int(np.sum(np.rint(prod) != np.array(sym[1:-1], np.float32)))
        if found >= 300 and recip_differs >= 3:
            break
    assert found >= 300
    assert recip_differs >= 3


def test_delta_quotients_one_step_from_half_integers():
    """Deltas whose binary32 quotient d / dl is one binary32 step from a
    half-integer, with constant anchors (ahat = lo exactly)."""
    rng = np.random.default_rng(78)
    found = 0
    for b in (3, 4, 5, 6):
        M = (1 << (b - 1)) - 1
        for _ in range(200):
            top = np.float16(rng.uniform(0.25, 8))
            dl = np.float32(top) / np.float32(M)
            xs = np.arange(0, 1 << 16, dtype=np.uint16).view(np.float16)
            xs = xs[np.isfinite(xs)]
            xs = xs[np.abs(xs) < top].astype(np.float32)
            q = xs / dl
            half = np.floor(q) + np.float32(0.5)
            hit = (q == np.nextafter(half, np.float32(np.inf))) | (q == np.nextafter(half, np.float32(-np.inf)))
            xs = xs[hit]
            if len(xs) == 0:
                continue
            G = 10
            vals = [float(top)] + xs.tolist()
            x = []
            for i in range(0, len(vals), G - 1):
                x.append(0.0)
                x.extend(vals[i:i + G - 1])
            _check(np.array(x, np.float16), G, b)
            found += len(xs)
    assert found >= 50

"""Pins of the oracle's arithmetic (range) coder and model normalisation.

The CacheGen page ("核心方法", step 3) compresses the quantized symbols with
arithmetic coding against profiled distributions; the page fixes no coder
variant, so the oracle uses a static multi-symbol range coder (32-bit range,
15-bit model precision, byte renormalisation below 2^24, carry propagation,
4-byte flush).  These tests pin it by brute force on tiny inputs, by closed
forms (degenerate and uniform models, Shannon entropy) and by the coder's
redundancy bound.
"""
import itertools
import math

import numpy as np
import pytest

import oracle

TOT = 1 << 15
# per-symbol redundancy of truncating range/2^15 with range >= 2^24
RED = -math.log2(1 - 2.0 ** -9)


def ideal_bits(sym, f):
    return sum(-math.log2(f[s] / TOT) for s in sym)


def _tables():
    return [
        [TOT // 2, TOT // 2],
        [1, TOT - 1],
        [TOT - 1, 1],
        [10000, 12768, 10000],
        [1, 1, TOT - 2],
        [8192] * 4,
        [1, 16000, 1, TOT - 16002],
        [TOT - 3, 1, 1, 1],
    ]


@pytest.mark.slow
def test_brute_force_roundtrip_distinct_and_bounded():
    """Every sequence over alphabets <= 4 up to length 8 (length 6 for the
    4-symbol tables): decode(encode(x)) == x, encodings of equal-length
    sequences are distinct, and 8*nbytes <= ideal + n*RED + 33."""
    for f in _tables():
        A = len(f)
        assert sum(f) == TOT
        max_len = 8 if A <= 3 else 6
        for n in range(0, max_len + 1):
            seen = set()
            for seq in itertools.product(range(A), repeat=n):
                code = oracle.rc_encode(seq, f)
                assert oracle.rc_decode(code, n, f).tolist() == list(seq)
                assert code not in seen
                seen.add(code)
                assert 8 * len(code) <= ideal_bits(seq, f) + n * RED + 33 + 1e-9


def test_single_symbol_model_costs_exactly_the_flush():
    f = [TOT]
    for n in (0, 1, 7, 1000, 20000):
        code = oracle.rc_encode([0] * n, f)
        assert len(code) == 4
        assert oracle.rc_decode(code, n, f).tolist() == [0] * n


@pytest.mark.parametrize("k", [1, 2, 4, 6, 8])
def test_uniform_power_of_two_alphabet(k):
    """A uniform 2^k-symbol model spends k bits per symbol: 8*nbytes lies in
    [n*k + 24, n*k + 33 + RED*n]."""
    A = 1 << k
    f = [TOT // A] * A
    rng = np.random.default_rng(k)
    for n in (1, 10, 333, 5000):
        seq = rng.integers(0, A, n)
        code = oracle.rc_encode(seq, f)
        assert n * k + 24 <= 8 * len(code) <= n * k + 33 + RED * n
        np.testing.assert_array_equal(oracle.rc_decode(code, n, f), seq)


@pytest.mark.parametrize("A", [3, 15, 63, 256])
def test_entropy_closed_form(A):
    """1e6 i.i.d. symbols drawn from a normalised model q code to within 0.5%
    of n*H(q) + 32 bits (Shannon's bound is met by arithmetic coding)."""
    rng = np.random.default_rng(A)
    w = rng.gamma(0.7, size=A)
    f = oracle.normalize(np.round(w / w.sum() * 1e6).astype(np.uint64))
    q = f / TOT
    H = -(q * np.log2(q)).sum()
    n = 1_000_000
    seq = rng.choice(A, size=n, p=q)
    code = oracle.rc_encode(seq, f)
    bits = 8 * len(code)
    assert abs(bits - n * H) <= 0.005 * n * H + 32
    np.testing.assert_array_equal(oracle.rc_decode(code, n, f), seq)


def test_two_models_alternate_by_group():
    fa = [100] * 256
    fa[0] += TOT - sum(fa)
    fd = [1000, 30000, 1768]
    rng = np.random.default_rng(5)
    n = 97
    seq = [int(rng.integers(0, 256)) if j % 10 == 0 else int(rng.integers(0, 3)) for j in range(n)]
    code = oracle.rc_encode(seq, fa, fd, group=10)
    assert oracle.rc_decode(code, n, fa, fd, group=10).tolist() == seq
    ideal = sum(-math.log2((fa if j % 10 == 0 else fd)[s] / TOT) for j, s in enumerate(seq))
    assert 8 * len(code) <= ideal + n * RED + 33


def test_truncated_or_extended_streams_are_rejected():
    rng = np.random.default_rng(9)
    f = oracle.normalize(rng.integers(0, 50, 31).astype(np.uint64))
    seq = rng.integers(0, 31, 400)
    code = oracle.rc_encode(seq, f)
    with pytest.raises(oracle.OracleError) as e:
        oracle.rc_decode(code[:-1], 400, f)
    assert e.value.code == oracle.ERR_CORRUPT
    with pytest.raises(oracle.OracleError) as e:
        oracle.rc_decode(code + b"\x00", 400, f)
    assert e.value.code == oracle.ERR_CORRUPT
    with pytest.raises(oracle.OracleError):
        oracle.rc_decode(code[:3], 400, f)


def test_t_out_of_range_is_corrupt():
    # code = 0xFFFFFFFF with range 0xFFFFFFFF gives t = 2^15 exactly
    with pytest.raises(oracle.OracleError) as e:
        oracle.rc_decode(b"\xff\xff\xff\xff", 1, [TOT])
    assert e.value.code == oracle.ERR_CORRUPT


# ---------------------------------------------------------------- normalise
def test_normalize_invariants_random():
    rng = np.random.default_rng(1)
    for _ in range(500):
        A = int(rng.integers(1, 257))
        counts = rng.integers(0, 1000, A) * (rng.random(A) < 0.6)
        f = oracle.normalize(counts.astype(np.uint64))
        assert f.sum() == TOT and f.min() >= 1
        N = counts.sum()
        if N == 0:
            continue
        arg = int(np.argmax(counts))  # numpy: first index of the maximum
        base = 1 + (counts.astype(np.int64) * (TOT - A)) // N
        others = np.arange(A) != arg
        np.testing.assert_array_equal(f[others], base[others])
        assert f[arg] >= base[arg]
        # the remainder handed to the argmax is below A (sum of floors)
        assert f[arg] - base[arg] < A
        # the most frequent symbol keeps the largest frequency
        assert f[arg] == f.max()


def test_normalize_closed_forms():
    # no data: as uniform as possible, low symbols take the remainder
    f = oracle.normalize([0] * 3)
    assert f.tolist() == [10923, 10923, 10922]
    assert oracle.normalize([0] * 256).tolist() == [128] * 256
    # equal counts: every symbol gets 1 + floor((TOT - A) / A), symbol 0 the rest
    f = oracle.normalize([7, 7, 7])
    assert f.tolist() == [10924, 10922, 10922]
    # a single observed symbol takes everything but the floors
    f = oracle.normalize([0, 5, 0, 0])
    assert f.tolist() == [1, TOT - 3, 1, 1]
    # ties: lowest index receives the remainder
    f = oracle.normalize([3, 9, 9])
    assert f[1] > f[2]

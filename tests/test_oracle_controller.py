"""Pins of the oracle's per-chunk level choice (CacheGen page, 核心方法,
online streaming paragraph; 关键观察, assumption 1; reading R18).

Hand-worked cases use sizes and rates that are powers of two, so every
comparison and time below is exact; the invariants hold on any trace.
"""
import math

import numpy as np

from oracle.controller import arrival_time, plan_stream

SIZES = [[128, 64, 32]]  # bytes at levels 0 (best), 1, 2


def test_arrival_time_across_pieces():
    trace = [(0.0, 10.0), (1.0, 20.0), (3.0, 5.0)]
    # from 0.5: 5 B until 1.0, 40 B until 3.0, the last 55 B at 5 B/s
    assert arrival_time(trace, 0.5, 100.0) == 14.0
    assert arrival_time(trace, 2.0, 10.0) == 2.5  # inside the second piece
    assert arrival_time(trace, 0.0, 10.0) == 1.0  # ends exactly at a boundary
    assert arrival_time(trace, 7.0, 5.0) == 8.0   # the last piece lasts forever


def test_best_level_when_it_fits_exactly():
    # 384 B at 128 B/s is exactly the 3 s SLO
    levels, finish = plan_stream(SIZES * 3, [(0.0, 128.0)], 3.0, 128.0)
    assert levels == [0, 0, 0] and finish == [1.0, 2.0, 3.0]


def test_quality_recovers_when_slack_appears():
    """SLO 2 s: level 0 needs 3 s, level 1 1.5 s; after two level-1 chunks
    (t = 1 s) the last chunk fits at level 0 (1 + 1 = 2 s)."""
    levels, finish = plan_stream(SIZES * 3, [(0.0, 128.0)], 2.0, 128.0)
    assert levels == [1, 1, 0] and finish == [0.5, 1.0, 2.0]


def test_estimate_trails_the_link_by_one_chunk():
    """The link drops from 128 to 32 B/s at t = 1 s.  Chunk 1 still goes at
    level 0 (its estimate is chunk 0's 128 B/s); chunk 1 takes 4 s, so the
    estimate falls to 32 B/s; then no level meets the 4 s SLO and the
    fewest-bytes level (2) is sent."""
    trace = [(0.0, 128.0), (1.0, 32.0)]
    levels, finish = plan_stream(SIZES * 4, trace, 4.0, 128.0)
    assert levels == [0, 0, 2, 2] and finish == [1.0, 5.0, 6.0, 7.0]


def test_no_level_fits_sends_fewest_bytes():
    # level 1 is the smallest here; an impossible SLO picks it every time
    sizes = [[100, 10, 20]] * 3
    levels, _ = plan_stream(sizes, [(0.0, 1.0)], -1.0, 1.0)
    assert levels == [1, 1, 1]
    # a tie in remaining bytes goes to the lower index
    levels, _ = plan_stream([[5, 5]], [(0.0, 1.0)], 0.0, 1.0)
    assert levels == [0]


def _trace(rng, n=40):
    starts = np.concatenate([[0.0], np.cumsum(rng.uniform(0.05, 0.4, n - 1))])
    rates = 1e9 * np.exp(rng.normal(0.0, 0.7, n))
    return [(float(s), float(r)) for s, r in zip(starts, rates)]


def _sizes(rng, n=11):
    base = rng.uniform(0.8e8, 1.6e8, n)
    return [[int(b), int(b * 0.78), int(b * 0.6)] for b in base]


def test_constant_link_never_misses_when_a_level_fits():
    """With an exact estimate on a constant link, if one fixed level meets
    the SLO the controller meets it too, starting at that level or better:
    the level it picks always still fits for the chunks after it."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        sizes = _sizes(rng)
        rate = float(rng.uniform(0.5e9, 2e9))
        slo = float(rng.uniform(0.6, 2.0))
        fixed = [sum(c[l] for c in sizes) / rate for l in range(3)]
        levels, finish = plan_stream(sizes, [(0.0, rate)], slo, rate)
        ok = [l for l in range(3) if fixed[l] <= slo]
        if ok:
            assert levels[0] <= ok[0]
            assert finish[-1] <= slo * (1 + 1e-12)


def test_decisions_depend_only_on_the_past():
    """Two links equal until time T: every chunk that starts before T gets
    the same level on both (the estimate only uses finished chunks)."""
    rng = np.random.default_rng(11)
    for _ in range(100):
        sizes = _sizes(rng)
        a = _trace(rng)
        T = float(rng.uniform(0.2, 1.0))
        b = [p for p in a if p[0] < T] + [(T, float(rng.uniform(0.2e9, 3e9)))]
        la, fa = plan_stream(sizes, a, 1.0, 1e9)
        lb, fb = plan_stream(sizes, b, 1.0, 1e9)
        t0 = [0.0] + fa[:-1]
        for i in range(len(sizes)):
            if t0[i] >= T or (i and fa[i - 1] != fb[i - 1]):
                break
            assert la[i] == lb[i]


def test_arrival_matches_integral_of_the_rate():
    """The bytes delivered between t and arrival_time equal the integral of
    the piecewise-constant rate over that interval."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        tr = _trace(rng)
        t = float(rng.uniform(0, 5))
        nb = float(rng.uniform(1e6, 5e9))
        end = arrival_time(tr, t, nb)
        starts = [p[0] for p in tr] + [math.inf]
        got = sum(max(0.0, min(end, starts[k + 1]) - max(t, starts[k])) * tr[k][1]
                  for k in range(len(tr)))
        assert abs(got - nb) <= 1e-9 * nb

"""Pins of the seeded input generator (not part of the codec).

The generator stands in for the CacheGen page's model KV caches; these tests
check it against its published PRNG definition and the closed-form
statistics of a stationary AR(1) process.
"""
import numpy as np
import pytest

import synth


def test_philox_known_answers():
    # Known-answer vectors distributed with the Random123 library for
    # philox4x32 with 10 rounds (Salmon et al., SC 2011).
    assert synth.philox4x32_10([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert synth.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [
        0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert synth.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344],
                               [0xA4093822, 0x299F31D0]) == [
        0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_half_rounding_matches_numpy():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-25, 11, 20000))
    got = np.array([synth.to_half_bits(x) for x in v], np.uint16)
    want = v.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_innovations_are_standard_normal():
    e = synth.innovations(1234, 0, 64, 4000).ravel()
    n = e.size
    assert abs(e.mean()) < 4 / np.sqrt(n)
    assert abs(e.var() - 1) < 4 * np.sqrt(2 / n)


def test_outlier_count_exact_per_row():
    for cfg in (synth.SHAPE_7B_9K, synth.SHAPE_34B_GQA_80K, synth.SHAPE_70B_GQA_16K):
        p = synth.params(cfg)
        per_row = p.is_outlier.reshape(2 * cfg.n_layers, cfg.n_channels).sum(axis=1)
        assert np.all(per_row == round(0.01 * cfg.n_channels))
    p0 = synth.params(synth.TINY)
    assert p0.is_outlier.sum() == 0


def test_rho_per_channel_range():
    cfg = synth.SHAPE_34B_GQA_80K
    p = synth.params(cfg)
    assert p.rho.min() >= 0.8 and p.rho.max() <= 0.97
    assert np.std(p.rho) > 0.04  # U(0.8, 0.97) has sd 0.049
    assert np.all(synth.params(synth.SHAPE_70B_GQA_16K).rho == 0.9)


def test_lag_difference_variance_closed_form():
    """Var(x[t+k] - x[t]) = 2 s^2 (1 - rho^k) / (1 - rho^2) for a stationary
    AR(1); pooled over channels after dividing by s^2, within 3 standard
    errors for k = 1..9."""
    cfg = synth.small_config(4, 512, 1500, outlier_frac=0.0)
    p = synth.params(cfg)
    x = synth.make_kv(cfg, p=p).view(np.float16).astype(np.float64)  # [L][2][T][C]
    s = p.s.reshape(cfg.n_layers, 2, 1, cfg.n_channels)
    rho = 0.9
    z = x / s
    starts = np.arange(0, 1500 - 10, 60)  # well-separated pairs: nearly independent
    for k in range(1, 10):
        d = (z[:, :, starts + k, :] - z[:, :, starts, :]).ravel()
        want = 2 * (1 - rho ** k) / (1 - rho ** 2)
        se = want * np.sqrt(2.0 / d.size)
        assert abs(d.var() - want) < 3 * se + 1e-3, (k, d.var(), want)


def test_stationary_start_variance():
    cfg = synth.small_config(8, 512, 2, outlier_frac=0.0)
    p = synth.params(cfg)
    x = synth.make_kv(cfg, p=p).view(np.float16).astype(np.float64)
    z0 = (x[:, :, 0, :] - p.mu.reshape(cfg.n_layers, 2, cfg.n_channels)) / p.s.reshape(
        cfg.n_layers, 2, cfg.n_channels)
    want = 1 / (1 - 0.81)
    se = want * np.sqrt(2.0 / z0.size)
    assert abs(z0.var() - want) < 3 * se


def test_layer_subsets_match_full_generation():
    cfg = synth.small_config(6, 128, 300)
    full = synth.make_kv(cfg)
    part = synth.make_kv(cfg, layers=range(2, 5))
    np.testing.assert_array_equal(full[2:5], part)


def test_profile_chunks_share_processes_not_innovations():
    cfg = synth.small_config(2, 64, 1500, outlier_frac=0.0)
    p = synth.params(cfg)
    kv = synth.make_kv(cfg, p=p).view(np.float16).astype(np.float64)
    pr = synth.make_profile_kv(cfg, p=p).view(np.float16).astype(np.float64)
    assert pr.shape == (2, 2, 4500, 64)
    assert not np.array_equal(kv[:, :, :1500], pr[:, :, :1500])
    # same channel means: per-channel averages agree far better than across channels
    m1 = kv.mean(axis=2).ravel()
    m2 = pr.mean(axis=2).ravel()
    assert np.corrcoef(m1, m2)[0, 1] > 0.9


def test_level_schedule_is_seeded_and_mixed():
    cfg = synth.SHAPE_70B_GQA_16K
    lv = cfg.chunk_levels()
    assert len(lv) == 11 and set(lv) == {0, 1, 2}
    assert lv == cfg.chunk_levels()
    assert synth.SHAPE_13B_16K.chunk_levels() == [1] * 11
    assert synth.SHAPE_34B_GQA_80K.n_chunks == 54

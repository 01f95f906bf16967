"""The oracle reproduces its stored regression fixture (tests/golden)."""
import json
import os

import pytest

from golden.make_golden import record  # noqa: E402
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _load():
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        return json.load(f)


def test_tiny_fixture():
    want = _load()["tiny"]
    got = record(synth.TINY, synth.TINY.chunk_levels())
    assert got == want


def test_mixed_small_fixture():
    want = _load()["mixed_small"]
    got = record(synth.small_config(6, 96, 3700, n_levels=3, schedule="mixed", seed_index=91), [0, 2, 1])
    assert got == want

"""The oracle's range coder on streams whose carries run through long strings
of 0xFF bytes (CacheGen page, 核心方法 step 3: every symbol is arithmetic
coded; a carry has to reach back into bytes already emitted).  The inputs are
built in tests/carry_runs.py; the checks are the coder's definition run in
Python, the round trip, and exact reconstruction."""
import numpy as np

import carry_runs as cr
import oracle


def _desc():
    return oracle.Desc(cr.N_LAYERS, cr.N_CHANNELS, 1, cr.CHUNK, 8, ((4, 3, 2),), 15)


def test_prefix_carries_through_k_bytes():
    cum = [128 * s for s in range(257)]
    freq = [128] * 256
    for k in cr.RUNS[1:]:
        sym = cr.carry_prefix(k) + [7, 0, 255]
        data, longest = cr.longest_carry_run(sym, cum, freq)
        assert longest >= k
        assert oracle.rc_encode(sym, freq) == data
        assert oracle.rc_decode(data, len(sym), freq).tolist() == sym


def test_uniform_profile():
    d = _desc()
    tb = oracle.profile(d, cr.make_profile_kv())
    assert np.all(tb.fA == 128)


def test_containers_round_trip_exactly():
    """Every stream of every chunk: the oracle's container holds the coder's
    bytes for the stream's symbols, and decoding gives back the input."""
    d = _desc()
    tb = oracle.profile(d, cr.make_profile_kv())
    kv, runs = cr.make_kv()
    levels = [0] * ((cr.N_TOKENS + cr.CHUNK - 1) // cr.CHUNK)
    cont = oracle.encode(d, tb, kv, levels)
    out = oracle.decode(d, tb, cont, levels, cr.N_TOKENS)
    np.testing.assert_array_equal(out, kv)
    cum = [128 * s for s in range(257)]
    x = kv.view(np.float16).astype(np.int64)
    seen = 0
    for k, c in enumerate(cont):
        rec = oracle.records(d, c)
        t0 = k * cr.CHUNK
        n = min(cr.CHUNK, cr.N_TOKENS - t0)
        for row in range(2):
            for ch in range(cr.N_CHANNELS):
                m = row * cr.N_CHANNELS + ch
                sym = x[0, row, t0:t0 + n, ch].tolist()
                data, longest = cr.longest_carry_run(sym, cum, [128] * 256)
                assert longest >= runs[k, row, ch]
                assert int(rec["nbytes"][m]) == len(data)
                seen += longest >= 8
    assert seen >= 100

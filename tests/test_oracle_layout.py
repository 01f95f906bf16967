"""Pins of the oracle's container payload layout (readings R6 and R17): each
unit's payload holds its streams' 8-byte blocks in the order the reference
reader asks for them.

The reader's rule (R17): every lane asks for blocks 0, 1, 2 first (block
outer, lane inner); then before token j a lane whose ring holds at most 8
bytes (anchor token, j % G == 0) or fewer than 2 bytes (any other token)
takes its next block and asks for the one after it.
"""
import numpy as np
import pytest

import oracle
import synth


def _pairs(order):
    return [(int(x) >> 16, int(x) & 0xFFFF) for x in order]


def test_block_order_worked_example():
    """A hand-worked trace of the rule: lane 0 shifts in 1 byte per token,
    lane 1 two bytes per token, G = 10, 11 tokens.
      start: (0,0) (1,0) (0,1) (1,1) (0,2) (1,2); W = 16, R = 4 for both.
      lane 1 reaches R = 16 after token 5 (W - R = 0 < 2 at token 6): asks
      for block 3.  At the anchor token 10 lane 0 has W - R = 16 - 14 <= 8
      but no block 3 (3 blocks), lane 1 has 24 - 24 <= 8 and asks for 4."""
    k = np.array([[1] * 11, [2] * 11], np.uint8)
    order = oracle.block_order_trace([3, 5], k, group=10)
    assert _pairs(order) == [(0, 0), (1, 0), (0, 1), (1, 1), (0, 2), (1, 2), (1, 3), (1, 4)]


def test_block_order_anchor_threshold():
    """At an anchor the threshold is 8 bytes inclusive, elsewhere 2 exclusive:
    a lane at W - R = 8 on an anchor asks, at W - R = 2 off an anchor does
    not."""
    # lane 0: R = 4 + 4 = 8 before token 1 (not an anchor, W - R = 8: no);
    # tokens 1..3 add 2 each -> R = 14 before token 4; G = 4 makes token 4
    # an anchor with W - R = 2 <= 8: asks for block 3.
    k = np.array([[4, 2, 2, 2, 0]], np.uint8)
    order = oracle.block_order_trace([6], k, group=4)
    assert _pairs(order) == [(0, 0), (0, 1), (0, 2), (0, 3)]
    # same consumption with G = 10: token 4 is not an anchor and W - R = 2
    # is not below 2, so nothing is asked for.
    order = oracle.block_order_trace([6], k, group=10)
    assert _pairs(order) == [(0, 0), (0, 1), (0, 2)]


def test_block_order_short_streams():
    """Streams of one or two blocks ask for only the blocks they have."""
    k = np.zeros((3, 4), np.uint8)
    order = oracle.block_order_trace([1, 2, 3], k, group=10)
    assert _pairs(order) == [(0, 0), (1, 0), (2, 0), (1, 1), (2, 1), (2, 2)]


@pytest.fixture(scope="module")
def mixed():
    cfg = synth.small_config(3, 150, 3100, seed_index=95)  # 3 channel blocks per row (64, 64, 22)
    d = oracle.desc_for(cfg)
    kv = synth.make_kv(cfg)
    tb = oracle.profile(d, synth.make_profile_kv(cfg))
    levels = [0, 2, 1]
    cont = oracle.encode(d, tb, kv, levels)
    return cfg, d, kv, tb, cont, levels


def _streams_of_unit(d, c, order, unit):
    """The contiguous bytes of each stream of a unit, gathered from the
    payload by the slot order."""
    S = d.n_streams
    m0, nv = oracle.unit_streams(d, unit)
    rec = oracle.records(d, c)
    offs = oracle.stream_offsets(d, c)
    pay = c[64 + 16 * S + offs[m0]:]
    nblk = (rec["nbytes"][m0:m0 + nv].astype(np.int64) + 7) // 8
    blocks = [[None] * int(nblk[l]) for l in range(nv)]
    for slot, (l, b) in enumerate(_pairs(order)):
        assert blocks[l][b] is None, "block placed twice"
        blocks[l][b] = pay[8 * slot:8 * slot + 8]
    out = []
    for l in range(nv):
        assert all(x is not None for x in blocks[l]), "block missing"
        out.append(np.concatenate(blocks[l]) if blocks[l] else np.zeros(0, np.uint8))
    return out, rec["nbytes"][m0:m0 + nv]


def test_units_hold_every_block_once_in_block_order(mixed):
    cfg, d, kv, tb, cont, levels = mixed
    for c in cont:
        for u in range(oracle.n_units(d)):
            order, nv = oracle.unit_order(d, tb, c, u)
            pairs = _pairs(order)
            m0, n_lanes = oracle.unit_streams(d, u)
            assert nv == n_lanes
            rec = oracle.records(d, c)
            nblk = (rec["nbytes"][m0:m0 + nv].astype(np.int64) + 7) // 8
            assert sorted(pairs) == sorted((l, b) for l in range(nv) for b in range(int(nblk[l])))
            for l in range(nv):
                mine = [b for (ll, b) in pairs if ll == l]
                assert mine == sorted(mine)


def test_gathered_streams_are_the_encoded_streams(mixed):
    """Each stream gathered from the payload decodes to the chunk's symbols,
    consumes exactly nbytes, and its block padding is zero; the reader's slot
    order is the rule applied to those streams' own consumption traces."""
    cfg, d, kv, tb, cont, levels = mixed
    S = d.n_streams
    for k, c in enumerate(cont):
        n = cfg.chunk_tokens(k)
        lv = levels[k]
        for u in range(oracle.n_units(d)):
            order, nv = oracle.unit_order(d, tb, c, u)
            streams, nbytes = _streams_of_unit(d, c, order, u)
            m0, _ = oracle.unit_streams(d, u)
            _, want = oracle.decode_streams(d, tb, c, list(range(m0, m0 + nv)), n)
            shifts = np.zeros((nv, n), np.uint8)
            for l in range(nv):
                m = m0 + l
                fA = tb.fA[m]
                A = (1 << d.bits(lv, m // (2 * d.n_channels))) - 1
                fD = tb.fD[lv, m, :A]
                data = streams[l][:nbytes[l]].tobytes()
                assert np.all(streams[l][nbytes[l]:] == 0)
                sym = oracle.rc_decode(data, n, fA, fD, group=10)
                np.testing.assert_array_equal(sym, want[l])
                shifts[l] = oracle.rc_shifts(data, n, fA, fD, group=10)
                assert 4 + int(shifts[l].sum()) == nbytes[l]
            nblk = (nbytes.astype(np.int64) + 7) // 8
            np.testing.assert_array_equal(oracle.block_order_trace(nblk, shifts, 10), order)


def test_layout_round_trip_small_units(mixed):
    """Decoding the oracle's own containers reproduces its quantized values
    (the layout is read back in the order it was written)."""
    cfg, d, kv, tb, cont, levels = mixed
    out = oracle.decode(d, tb, cont, levels, cfg.n_tokens)
    for k, c in enumerate(cont):
        n = cfg.chunk_tokens(k)
        vals, _ = oracle.decode_streams(d, tb, c, [0, 63, 64, 149, d.n_streams - 1], n)
        for i, m in enumerate([0, 63, 64, 149, d.n_streams - 1]):
            row, ch = divmod(m, d.n_channels)
            np.testing.assert_array_equal(out[row // 2, row % 2, 1500 * k:1500 * k + n, ch], vals[i])

"""Seeded inputs whose range-coder carries run through long strings of 0xFF
bytes (no codec arithmetic here: the expected containers come from the
oracle).

With every token an anchor (group size 1) and a uniform anchor model (all 256
frequencies 128), the coder's r = range >> 15 is 2^17 - 1 at every symbol:
range is 2^32 - 1 at the start, r * 128 = 2^24 - 128 then needs exactly one
byte shifted out, which leaves range = 2^32 - 2^15, whose r is again
2^17 - 1.  So symbol s adds c * s to low, c = 128 (2^17 - 1), and one byte
leaves per symbol: after symbols s_1..s_j the encoder's whole output (bytes
emitted, then the 4 bytes of low) is the integer P_j = 256 c Q_j, where Q_j
has the base-256 digits s_1..s_j.

256 c = 2^15 m with m = 2^17 - 1 odd.  Taking Q = -m^-1 mod 2^(8(k+4) - 15)
gives P = -2^15 mod 2^(8(k+4)): low = 2^32 - 2^15, and the k bytes emitted
last are all 0xFF.  The next symbol 1 adds c > 2^15 to low, so its carry runs
through all k of them.
"""
import numpy as np

_M = (1 << 17) - 1


def carry_prefix(k: int):
    """Anchor symbols after which the encoder holds k pending 0xFF bytes,
    followed by the symbol 1 whose carry passes all of them."""
    mod = 1 << (8 * (k + 4) - 15)
    q = (-pow(_M, -1, mod)) % mod
    return list(q.to_bytes(k + 3, "big")) + [1]


def longest_carry_run(symbols, cum, freq):
    """The range coder's definition (32-bit range, 15-bit models, carry into
    the bytes emitted, 4-byte flush) run on one stream: its bytes and the
    longest run of 0xFF bytes a carry turned into 0x00."""
    low, rng, out, longest = 0, 0xFFFFFFFF, [], 0
    for s in symbols:
        r = rng >> 15
        low += r * cum[s]
        rng = r * freq[s]
        if low >= 1 << 32:
            low -= 1 << 32
            i, run = len(out) - 1, 0
            while out[i] == 0xFF:
                out[i] = 0
                i -= 1
                run += 1
            out[i] += 1
            longest = max(longest, run)
        while rng < 1 << 24:
            out.append(low >> 24)
            low = (low << 8) & 0xFFFFFFFF
            rng <<= 8
    out += list(low.to_bytes(4, "big"))
    return bytes(out), longest


RUNS = (0, 6, 8, 12, 16, 24, 40, 64, 100)

# group size 1, chunks of 1,024 tokens (the profiling chunk below holds every
# anchor symbol exactly 4 times), 70 channels: a full and a ragged unit
N_LAYERS, N_CHANNELS, CHUNK, N_TOKENS = 1, 70, 1024, 1700


def stream_symbols(rng, n: int, k: int):
    """One stream of n anchor symbols: the k-run prefix (none for k = 0), then
    random symbols, with 0 and 255 present so that lo = 0 and hi = 255 (the
    anchor step is then exactly 1 and value s codes as symbol s)."""
    pre = carry_prefix(k) if k else []
    s = pre + rng.integers(0, 256, n - len(pre)).tolist()
    s[-2:] = [0, 255]
    return s


def make_kv(seed: int = 5):
    """KV [1][2][N_TOKENS][N_CHANNELS] binary16 bits: channel c of each row
    and chunk starts with the carry prefix for RUNS[(c + row) % len(RUNS)]."""
    rng = np.random.default_rng(seed)
    kv = np.zeros((N_LAYERS, 2, N_TOKENS, N_CHANNELS), np.float16)
    runs = np.zeros((2, 2, N_CHANNELS), np.int64)
    for row in range(2):
        for c in range(N_CHANNELS):
            for k0 in range(0, N_TOKENS, CHUNK):
                n = min(CHUNK, N_TOKENS - k0)
                k = RUNS[(c + row + k0 // CHUNK) % len(RUNS)]
                kv[0, row, k0:k0 + n, c] = stream_symbols(rng, n, k)
                runs[k0 // CHUNK, row, c] = k
    return kv.view(np.uint16), runs


def make_profile_kv():
    """One profiling chunk in which every channel holds each of 0..255 four
    times: uniform anchor counts, so every anchor frequency is 128."""
    x = (np.arange(CHUNK) % 256).astype(np.float16)
    kv = np.broadcast_to(x[None, None, :, None], (N_LAYERS, 2, CHUNK, N_CHANNELS))
    return np.ascontiguousarray(kv).view(np.uint16)

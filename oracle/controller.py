"""Oracle of the per-chunk level choice for streaming -- TEST INFRASTRUCTURE ONLY.

Only the tests and the benchmark import this module; the product never does.
Plain Python, one chunk at a time, IEEE binary64 arithmetic in the order
written out below.

What it computes (CacheGen wiki page, 核心方法, the online streaming
paragraph): every chunk is sent at one of the stored compression levels; the
sender estimates how long the remaining chunks will take from the throughput
the previous chunk achieved, and among the levels whose estimate still meets
the TTFT SLO sends the best-quality one.  关键观察, assumption 1: this estimate
trails the link by at most one chunk.  Readings where the page is silent
(reading R18): levels are ordered best quality first; a candidate level
applies to all remaining chunks; the first chunk uses a given initial
estimate; if no level meets the SLO, the level with the fewest remaining
bytes is sent (the page's text fallback needs a model and is not modelled);
the decode, overlapped with the transfer, adds nothing.

A link is a piecewise-constant bandwidth trace: a list of (start_s, bytes_per_s)
pieces, the first starting at 0, each lasting until the next one starts, the
last one forever.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


def arrival_time(trace: Sequence[Tuple[float, float]], t: float, nbytes: float) -> float:
    """Time at which `nbytes` sent from time `t` have arrived over `trace`."""
    k = 0
    while k + 1 < len(trace) and trace[k + 1][0] <= t:
        k += 1
    while True:
        rate = trace[k][1]
        if k + 1 == len(trace):
            return t + nbytes / rate
        can_send = (trace[k + 1][0] - t) * rate  # before the next piece starts
        if nbytes <= can_send:
            return t + nbytes / rate
        nbytes -= can_send
        t = trace[k + 1][0]
        k += 1


def plan_stream(chunk_bytes: Sequence[Sequence[int]], trace: Sequence[Tuple[float, float]],
                slo_s: float, init_bytes_per_s: float) -> Tuple[List[int], List[float]]:
    """Levels chosen for chunks 0..n-1 and each chunk's arrival time.

    chunk_bytes[i][l]: the size of chunk i's container at level l."""
    n = len(chunk_bytes)
    L = len(chunk_bytes[0]) if n else 0
    t = 0.0
    estimate = float(init_bytes_per_s)
    levels: List[int] = []
    finish: List[float] = []
    for i in range(n):
        remaining = [sum(int(chunk_bytes[j][l]) for j in range(i, n)) for l in range(L)]
        fits = [l for l in range(L) if t + float(remaining[l]) / estimate <= slo_s]
        if fits:
            level = fits[0]  # best quality among those meeting the SLO
        else:
            level = min(range(L), key=lambda l: (remaining[l], l))  # fewest bytes
        nbytes = float(chunk_bytes[i][level])
        end = arrival_time(trace, t, nbytes)
        levels.append(level)
        finish.append(end)
        if end > t and nbytes > 0.0:
            estimate = nbytes / (end - t)  # this chunk's throughput
        t = end
    return levels, finish

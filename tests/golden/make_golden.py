"""Write tests/golden/oracle_tiny.json from the oracle alone.

Regression fixture: the CacheGen page prints no worked example, so the stored
values are the oracle's own outputs on the seeded tiny workload (4 layers,
512 channels per K/V, one 1,500-token chunk) and on a reduced mixed-level
workload.  They guard against unintended changes to the oracle's arithmetic;
a deliberate change re-runs this script and names the page passage (or the
reading of it) that justifies it in its commit message.

Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def record(cfg, levels):
    d = oracle.desc_for(cfg)
    kv = synth.make_kv(cfg)
    tb = oracle.profile(d, synth.make_profile_kv(cfg))
    cont = oracle.encode(d, tb, kv, levels)
    out = oracle.decode(d, tb, cont, levels, cfg.n_tokens)
    return {
        "config": cfg.name,
        "levels": list(levels),
        "kv_sha256": hashlib.sha256(kv.tobytes()).hexdigest(),
        "profile_id": f"{tb.profile_id:016x}",
        "tables_sha256": hashlib.sha256(tb.fA.tobytes() + tb.fD.tobytes()).hexdigest(),
        "container_bytes": [int(len(c)) for c in cont],
        "container_sha256": [hashlib.sha256(c.tobytes()).hexdigest() for c in cont],
        "decoded_sha256": hashlib.sha256(out.tobytes()).hexdigest(),
        "decoded_head": [int(v) for v in out[0, 0, :12, 0]],
    }


def main():
    data = {
        "note": "oracle outputs on seeded synthetic KV; regression fixture written by make_golden.py",
        "tiny": record(synth.TINY, synth.TINY.chunk_levels()),
        "mixed_small": record(synth.small_config(6, 96, 3700, n_levels=3, schedule="mixed", seed_index=91),
                              [0, 2, 1]),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()

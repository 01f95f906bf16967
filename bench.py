#!/usr/bin/env python3
"""Benchmark of the KV-cache restore path on one MI355X.

Workload: the 70B-shaped GQA KV cache (80 layers, 8 KV heads x 128 = 1,024
channels per K and per V, 16,000 tokens = 11 chunks of <= 1,500 tokens, each
chunk at a seeded compression level), the configuration the codec's
throughput target is stated for.  A step is one kvc_decode call that restores
the whole context (bitstream index + fused range decode / dequantize / store)
from containers already resident in HBM into the preallocated binary16
[L][2][T][C] KV cache.

Printed: one JSON line with decoded-KV GB/s (binary16 bytes written per
second), the HBM roofline of the decode kernel (also against a device copy
measured in the same run, and beside its VALU issue rate), the compression
ratio, a bit-exactness check against the CPU oracle on a sample of chunks,
the oracle's own decode rate on the host cores, the encode rate, and SHA-256
digests of the binary16 tensors.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
# VALU issue ceiling: 256 CUs x 4 SIMDs, one wave64 vector instruction per
# SIMD every 4 cycles (16 lanes per cycle) at 2.4 GHz
VALU_PEAK_WAVE_INSTS = 256 * 4 * 2.4e9 / 4
COPY_CALIBRATION_BYTES = 1 << 30
# rocprofv3 HBM counter summary of the decode kernel on the 70B-shaped GQA
# workload; its figures are reported only for that workload, and only while the
# kernel sources still hash to the value recorded there.
COUNTERS_MD = os.path.join(ROOT, "profiles", "k_decode_70b-gqa-16K_hbm_counters.md")
# the workload the metric is quoted on, and the one the committed counters cover
DEFAULT_WORKLOAD = "llama-70b-gqa-shape-16K"
COUNTERS_WORKLOAD = DEFAULT_WORKLOAD
DECODE_SOURCES = [os.path.join(ROOT, "kv_cache_compression_decode_amd", "csrc", f)
                  for f in ("kvc_decode.hip", "kvc_internal.h")]
METRIC = "decoded KV GB/s on 1 MI355X (+% HBM roofline), bit-exact vs oracle; compression ratio"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def strip_comments(text: str) -> str:
    """C/HIP source without its comments and blank lines (the sources hold no
    string literal with comment markers), so that documentation edits keep
    the counters' provenance while any code change breaks it."""
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def decode_source_hash() -> str:
    """SHA-256 of the decode kernel's sources, comments stripped."""
    import hashlib

    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()


def counter_fields(workload: str):
    """(fields, note): the committed counter summary's `- key: value` lines,
    or None for another workload or while the decode kernel sources no longer
    hash to its value."""
    if workload != COUNTERS_WORKLOAD:
        return None, f"counters were taken on {COUNTERS_WORKLOAD} only"
    if not os.path.exists(COUNTERS_MD):
        return None, "no counter summary"
    fields = {}
    with open(COUNTERS_MD) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                fields[k.strip("`")] = v.strip().strip("`")
    if fields.get("decode_source_sha256") != decode_source_hash():
        return None, "decode kernel changed since the counters were taken"
    return fields, "rocprofv3 counters of this kernel source"


def measured_traffic(workload: str):
    """(bytes per decode launch, note) from the committed counter summary."""
    fields, note = counter_fields(workload)
    if fields is None:
        return None, note
    try:
        traffic = int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None, "counter summary unreadable"
    return traffic, f"rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a {COPY_CALIBRATION_BYTES}-byte copy"


def measured_valu_insts(workload: str):
    """VALU wave-instructions per decode launch (rocprofv3 SQ_INSTS_VALU)
    from the committed counter summary, or None."""
    fields, _ = counter_fields(workload)
    try:
        return int(fields["valu_insts_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def hip_clocks(compute_units: int) -> dict:
    """Peak engine and memory clocks (MHz) from hipDeviceGetAttribute, called
    through the HIP runtime this process has already loaded (found in
    /proc/self/maps, so no second copy is opened).  Attribute numbers of
    hipDeviceAttribute_t in hip_runtime_api.h: 5 clock rate, 60 memory clock
    rate, 63 multiprocessor count, which must read back the CU count torch
    reports; otherwise nothing is recorded."""
    import ctypes

    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64.so" in ln}
        if len(paths) != 1:
            return {}
        hip = ctypes.CDLL(paths.pop())
        value = ctypes.c_int()

        def attr(n: int):
            if hip.hipDeviceGetAttribute(ctypes.byref(value), ctypes.c_int(n), ctypes.c_int(0)) != 0:
                return None
            return value.value

        if attr(63) != compute_units:
            return {}
        out = {}
        for key, n in (("max_engine_clock_MHz", 5), ("max_memory_clock_MHz", 60)):
            v = attr(n)
            if v:
                out[key] = round(v / 1000)
        return out
    except OSError:
        return {}


def sha256_of(a) -> str:
    import hashlib

    return hashlib.sha256(memoryview(a).cast("B")).hexdigest()


def copy_rate(src, reps: int = 5) -> float:
    """GB/s (bytes read + written) of a plain device-to-device copy of
    `src`, measured with HIP events on the current stream."""
    import torch

    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ms.append(a.elapsed_time(b))
    del dst
    nbytes = 2 * src.numel() * src.element_size()
    return nbytes / (statistics.median(ms) * 1e-3) / 1e9


def copy_calibration() -> int:
    """A plain device-to-device copy of known size, run under the HBM counters
    to scale FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ok = bool(torch.equal(src[:4096], dst[:4096]))
    print(json.dumps({"calibration": "copy", "bytes": COPY_CALIBRATION_BYTES, "launches": 3,
                      "ok": ok}), flush=True)
    return 0 if ok else 1


def measure_restore(kvc, d, tables, enc, cfg, ref_out, reps: int = 3) -> dict:
    """The containers handed over in pinned host memory instead: the PCIe
    host-to-device rate, and kvc_restore (batched copies overlapping the
    decode) at several batch sizes; one batch of all chunks copies
    everything, then decodes.  Times: HIP events on the compute stream
    around the whole call (the copies wait for its start)."""
    import torch

    dev = tables.device
    host = torch.empty(enc.total_bytes(), dtype=torch.uint8, pin_memory=True)
    host.copy_(enc.blob)
    chunks = kvc.host_chunks(enc, host)
    staging = torch.empty(enc.total_bytes(), dtype=torch.uint8, device=dev)

    def timed(fn) -> float:
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ms.append(a.elapsed_time(b))
        return statistics.median(ms)

    h2d_ms = timed(lambda: staging.copy_(host, non_blocking=True))
    del staging
    out = torch.empty_like(ref_out)
    res = {"h2d_GBps": round(enc.total_bytes() / (h2d_ms * 1e-3) / 1e9, 2),
           "h2d_ms": round(h2d_ms, 3), "batches": {}}
    exact = True
    for batch in (cfg.n_chunks, 4, 2, 1):
        rws = kvc.RestoreWorkspace(d, chunks, batch, dev)
        ms = timed(lambda: kvc.restore_async(d, tables, chunks, out, rws))
        kvc.read_status(rws.status, "kvc_restore")
        exact = exact and bool(torch.equal(out, ref_out))
        res["batches"][str(batch)] = round(ms, 3)
        del rws
    best = min(res["batches"].values())
    res["sequential_ms"] = res["batches"][str(cfg.n_chunks)]
    res["best_ms"] = best
    res["decoded_GBps_pcie_inclusive"] = round(cfg.fp16_bytes() / (best * 1e-3) / 1e9, 2)
    res["same_as_decode"] = exact
    log(f"restore from pinned host memory: h2d {res['h2d_GBps']} GB/s, {res['batches']} ms")
    return res


def measure_controller(kvc, d, tables, kv_dev, cfg, n_traces: int = 500, slo_s: float = 1.0,
                       sigma: float = 0.3) -> dict:
    """The per-chunk level choice (kvc_plan_stream) on seeded bandwidth
    traces, with this workload's real container sizes at every level (the
    context encoded once per level).  Two links: median rate just enough for
    all chunks at level 0, and at level 1, within the SLO.  The baselines are
    the fixed levels, sent back to back (the same call with one level)."""
    import numpy as np

    import synth

    sizes = []
    for lv in range(d.n_levels):
        e = kvc.encode(d, tables, kv_dev, [lv] * cfg.n_chunks)
        sizes.append(np.diff(np.asarray(e.offsets, dtype=np.int64)))
        del e
    sizes = np.stack(sizes, axis=1)  # [chunk][level]
    res = {"slo_s": slo_s, "traces": n_traces,
           "link": f"log-normal pieces of 0.05-0.4 s, sigma {sigma} (seeded)",
           "level_bytes_GB": [round(float(x) / 1e9, 4) for x in sizes.sum(axis=0)],
           "scenarios": {}}
    plan_s, plans = 0.0, 0
    # the second link needs a second level to be just enough for
    for ref in range(min(2, d.n_levels)):
        median = float(sizes[:, ref].sum()) / slo_s
        viol = np.zeros(d.n_levels + 1)
        share = np.zeros(d.n_levels)
        for i in range(n_traces):
            trace = synth.bandwidth_trace(5000 + i, median, sigma=sigma)
            a = time.perf_counter()
            levels, finish = kvc.plan_stream(sizes, trace, slo_s, median)
            plan_s += time.perf_counter() - a
            plans += 1
            viol[d.n_levels] += finish[-1] > slo_s
            share += np.bincount(levels, minlength=d.n_levels)
            for lv in range(d.n_levels):
                _, f = kvc.plan_stream(sizes[:, lv:lv + 1], trace, slo_s, median)
                viol[lv] += f[-1] > slo_s
        share /= share.sum()
        res["scenarios"][f"link_fits_level{ref}"] = {
            "median_link_GBps": round(median / 1e9, 3),
            "adaptive": {"violation_rate": round(viol[d.n_levels] / n_traces, 4),
                         "level_share": [round(float(x), 4) for x in share],
                         "mean_level": round(float((share * np.arange(d.n_levels)).sum()), 4)},
            "fixed_violation_rate": {str(lv): round(viol[lv] / n_traces, 4)
                                     for lv in range(d.n_levels)},
        }
    res["plan_us"] = round(plan_s / plans * 1e6, 2)
    log(f"level controller: {res['scenarios']}")
    return res


def measure_multi(kvc, d, tables, kv_dev, cfg, n_req: int = 8, req_tokens: int = 2000,
                  reps: int = 3) -> dict:
    """Several requests at once: the context cut into n_req requests of
    req_tokens tokens (two chunks each: 1,500 + 500), each encoded on its own
    at levels (r mod 3, r+1 mod 3); decoded as one kvc_decode per request, and
    as one kvc_decode_multi call for all their chunks, into per-request KV
    caches.  Both must give the same bits."""
    import torch

    dev = tables.device
    n_req = min(n_req, cfg.n_tokens // req_tokens)  # whole requests of this context
    encs, outs_a, outs_b = [], [], []
    for r in range(n_req):
        kv_r = kv_dev[:, :, r * req_tokens:(r + 1) * req_tokens].contiguous()
        n_ch = (req_tokens + cfg.chunk_tokens(0) - 1) // cfg.chunk_tokens(0)
        encs.append(kvc.encode(d, tables, kv_r, [(r + i) % d.n_levels for i in range(n_ch)]))
        del kv_r
        outs_a.append(torch.zeros((cfg.n_layers, 2, req_tokens, cfg.n_channels),
                                  dtype=torch.int16, device=dev))
        outs_b.append(torch.zeros_like(outs_a[-1]))
    refs = [kvc.chunk_refs(e) for e in encs]
    wss = [kvc.DecodeWorkspace(d, len(rf), dev) for rf in refs]
    chunks = [c for e, o in zip(encs, outs_b) for c in kvc.request_chunks(e, o)]
    wsm = kvc.DecodeWorkspace(d, len(chunks), dev)

    def one_by_one():
        for rf, o, w in zip(refs, outs_a, wss):
            kvc.decode_async(d, tables, rf, o, w)

    def together():
        kvc.decode_multi_async(d, tables, chunks, wsm)

    res = {"requests": n_req, "tokens_per_request": req_tokens, "chunks": len(chunks)}
    total = sum(o.numel() * 2 for o in outs_a)
    for name, fn in (("per_request_calls", one_by_one), ("one_multi_call", together)):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ms.append(a.elapsed_time(b))
        res[name] = {"ms": round(statistics.median(ms), 3),
                     "decoded_GBps": round(total / (statistics.median(ms) * 1e-3) / 1e9, 2)}
    for w in wss:
        kvc.read_status(w.status, "kvc_decode")
    kvc.read_status(wsm.status, "kvc_decode_multi")
    res["same_bits"] = all(bool(torch.equal(x, y)) for x, y in zip(outs_a, outs_b))
    res["speedup"] = round(res["per_request_calls"]["ms"] / res["one_multi_call"]["ms"], 3)
    log(f"multi-request decode: {res}")
    return res


def measure_refine(kvc, d, tables, rtables, ebits, enc, kv_dev, base_out, cfg, levels,
                   reps: int = 5) -> dict:
    """The refinement layer (ebits bits) over the same chunks: its containers'
    size, the refined decode (base + refinement streams in one launch) timed
    like the base decode, and the mean |error| of both decodes against the
    input."""
    import torch

    dev = tables.device
    renc = kvc.encode_refine(d, rtables, ebits, kv_dev, levels)
    refs = kvc.refined_chunk_refs(enc, renc)
    out = torch.zeros_like(kv_dev)
    wsp = kvc.RefinedDecodeWorkspace(d, len(refs), dev)
    for _ in range(2):
        kvc.decode_refined_async(d, tables, rtables, ebits, refs, out, wsp)
    kvc.read_status(wsp.status, "kvc_decode_refined")
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        kvc.decode_refined_async(d, tables, rtables, ebits, refs, out, wsp)
        b.record()
        b.synchronize()
        ms.append(a.elapsed_time(b))
    kvc.read_status(wsp.status, "kvc_decode_refined")
    err_b = err_r = 0.0
    for t0 in range(0, cfg.n_tokens, 1500):
        x = kv_dev[:, :, t0:t0 + 1500].view(torch.float16).float()
        err_b += float((base_out[:, :, t0:t0 + 1500].view(torch.float16).float() - x).abs().sum())
        err_r += float((out[:, :, t0:t0 + 1500].view(torch.float16).float() - x).abs().sum())
        del x
    med = statistics.median(ms)
    fp16_bytes = cfg.fp16_bytes()
    res = {
        "refine_bits": ebits,
        "refinement_bytes": renc.total_bytes(),
        "base_bytes": enc.total_bytes(),
        "ms": round(med, 3),
        "decoded_GBps": round(fp16_bytes / (med * 1e-3) / 1e9, 2),
        "algorithmic_GBps": round((fp16_bytes + enc.total_bytes() + renc.total_bytes())
                                  / (med * 1e-3) / 1e9, 2),
        # binary16 written + both layers' containers read, against 8 TB/s
        "hbm_frac": round((fp16_bytes + enc.total_bytes() + renc.total_bytes())
                          / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "mean_abs_error_base": err_b / (fp16_bytes // 2),
        "mean_abs_error_refined": err_r / (fp16_bytes // 2),
    }
    log(f"refinement: {res}")
    return res, renc, out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="a workload of synth.WORKLOADS, by name")
    ap.add_argument("--oracle-chunks", type=int, default=11,
                    help="chunks decoded by the CPU oracle for the baseline and the bit-exact check")
    ap.add_argument("--no-oracle", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="skip the restore, level-choice and multi-request measurements "
                         "(profiler passes of the decode kernel)")
    ap.add_argument("--with-refinement", action="store_true",
                    help="with --decode-only: still measure the refinement layer")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer three times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: the codec shards with no exchange between GPUs "
              f"(each GPU decodes its own slice of streams), so --gpus {args.gpus} is not run.",
              flush=True)
        return 2
    if args.copy_calibration:
        return copy_calibration()

    import numpy as np
    import torch

    import kv_cache_compression_decode_amd as kvc
    import synth

    dev = torch.device("cuda:0")
    cfg = synth.WORKLOADS[args.workload]
    levels = cfg.chunk_levels()
    log(f"workload {cfg.name}: generating {cfg.fp16_bytes() / 1e9:.2f} GB of binary16 KV")
    t0 = time.time()
    params = synth.params(cfg)
    kv = synth.make_kv(cfg, p=params)
    kvp = synth.make_profile_kv(cfg, p=params)
    log(f"generated in {time.time() - t0:.1f} s")

    d = kvc.make_desc(cfg.n_layers, cfg.n_channels, cfg.delta_bits)
    kv_dev = torch.from_numpy(kv.view(np.int16)).to(dev)
    kvp_dev = torch.from_numpy(kvp.view(np.int16)).to(dev)
    tables = kvc.profile(d, kvp_dev)
    refine_bits = 4
    do_refine = args.with_refinement or not args.decode_only
    rtables = kvc.profile_refine(d, tables, kvp_dev, refine_bits) if do_refine else None
    del kvp_dev
    torch.cuda.synchronize()

    # ---- encode (second priority): timed, then the containers it made
    wsp = kvc.EncodeWorkspace(d, cfg.n_tokens, dev)
    for _ in range(2):
        kvc.encode_async(d, tables, kv_dev, levels, wsp)
    kvc.read_status(wsp.status, "kvc_encode")
    enc_ms = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        kvc.encode_async(d, tables, kv_dev, levels, wsp)
        b.record()
        b.synchronize()
        enc_ms.append(a.elapsed_time(b))
    kvc.read_status(wsp.status, "kvc_encode")
    enc = kvc.encode(d, tables, kv_dev, levels, wsp=wsp)
    del wsp
    container_bytes = enc.total_bytes()
    fp16_bytes = cfg.fp16_bytes()
    ratio = fp16_bytes / container_bytes
    log(f"encoded: {container_bytes / 1e9:.3f} GB of containers, ratio {ratio:.3f}")

    # ---- decode: the timed step
    refs = kvc.chunk_refs(enc)
    out = torch.zeros_like(kv_dev)
    dws = kvc.DecodeWorkspace(d, len(refs), dev)
    for _ in range(args.warmup):
        kvc.decode_async(d, tables, refs, out, dws)
    kvc.read_status(dws.status, "kvc_decode")
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for a, b in evs:
        a.record()
        kvc.decode_async(d, tables, refs, out, dws)
        b.record()
    t_end.record()
    torch.cuda.synchronize()
    kvc.read_status(dws.status, "kvc_decode")
    total_ms = t_start.elapsed_time(t_end)
    step_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = total_ms / args.steps

    # the index kernels alone (same workspace), to isolate the decode kernel
    idx_ev = []
    offs = torch.zeros((len(refs), d.n_streams), dtype=torch.int32, device=dev)
    import ctypes

    arr = kvc._refs_array(refs)
    for i in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        kvc.lib().kvc_decode_index(ctypes.byref(d), tables.data_ptr(), arr, len(refs),
                                   offs.data_ptr(), dws.ws.data_ptr(), dws.ws_bytes,
                                   dws.status.data_ptr(), kvc._stream(None))
        b.record()
        idx_ev.append((a, b))
    torch.cuda.synchronize()
    kvc.read_status(dws.status, "kvc_decode_index")
    index_ms = statistics.mean(a.elapsed_time(b) for a, b in idx_ev)
    kernel_ms = max(ms_per_step - index_ms, 1e-6)

    # correctness of the timed output: identical to the input within the
    # codec's own reconstruction (checked bit-exactly against the oracle below)
    decoded_ok = bool(torch.isfinite(out.view(torch.float16)).all().item())

    # a plain device copy of the decoded tensor in the same run: the HBM rate
    # this GPU actually sustains, as a second reference for the roofline
    copy_gbs = copy_rate(out)
    torch.cuda.synchronize()

    restore = controller = multi = refine = None
    renc = refined_out = None
    if do_refine:
        refine, renc, refined_out = measure_refine(kvc, d, tables, rtables, refine_bits, enc,
                                                   kv_dev, out, cfg, levels)
    if not args.decode_only:
        restore = measure_restore(kvc, d, tables, enc, cfg, out)
        controller = measure_controller(kvc, d, tables, kv_dev, cfg)
        multi = measure_multi(kvc, d, tables, kv_dev, cfg)

    traffic, traffic_note = measured_traffic(cfg.name)
    valu_insts = measured_valu_insts(cfg.name)
    value = fp16_bytes / (ms_per_step * 1e-3) / 1e9
    algo_bytes = fp16_bytes + container_bytes
    achieved = algo_bytes / (kernel_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32+f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.describe}",
            "layers": cfg.n_layers, "channels_per_kv": cfg.n_channels, "tokens": cfg.n_tokens,
            "chunks": cfg.n_chunks, "chunk_tokens": 1500, "group_tokens": 10,
            "levels": levels, "delta_bits": [list(r) for r in cfg.delta_bits],
            "fp16_bytes": fp16_bytes, "container_bytes": container_bytes,
        },
        "compression_ratio": round(ratio, 4),
        "step_ms_median": round(statistics.median(step_ms), 4),
        "step_ms_min": round(min(step_ms), 4),
        "hbm_frac_step": round(algo_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {
            "kernel": "k_decode (fused range decode + dequantize + store)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_note": traffic_note,
            "kernel_ms": round(kernel_ms, 4),
            "index_ms": round(index_ms, 4),
            "algorithmic_bytes": algo_bytes,
            "copy_GBps": round(copy_gbs, 1),
            "frac_of_copy": round(achieved / copy_gbs, 4),
        },
        # the co-bound: the decode kernel's VALU instruction issue against the
        # chip's ceiling (instruction count from rocprofv3 SQ_INSTS_VALU of
        # this kernel source, rate from this run's kernel time)
        "alu": {
            "bound": "alu",
            "unit": "wave64 VALU instructions/s",
            "insts_per_launch": valu_insts,
            "achieved": (round(valu_insts / (kernel_ms * 1e-3), -6) if valu_insts else None),
            "peak": VALU_PEAK_WAVE_INSTS,
            "frac": (round(valu_insts / (kernel_ms * 1e-3) / VALU_PEAK_WAVE_INSTS, 4)
                     if valu_insts else None),
        },
        "encode": {
            "ms": round(statistics.median(enc_ms), 3),
            "fp16_GBps": round(fp16_bytes / (statistics.median(enc_ms) * 1e-3) / 1e9, 2),
            # algorithmic bytes: the binary16 KV read once, the containers
            # written once (the statistics pass re-reads the KV; not counted)
            "roofline": {
                "bound": "hbm",
                "achieved": round((fp16_bytes + container_bytes)
                                  / (statistics.median(enc_ms) * 1e-3) / 1e9, 2),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round((fp16_bytes + container_bytes)
                              / (statistics.median(enc_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            },
        },
        "decoded_finite": decoded_ok,
        "restore": restore,
        "level_controller": controller,
        "multi_request": multi,
        "refinement": refine,
        "sha256": {"kv_fp16": sha256_of(kv), "profile_kv_fp16": sha256_of(kvp)},
    }
    props = torch.cuda.get_device_properties(dev)
    result["device"] = {
        "name": props.name, "arch": getattr(props, "gcnArchName", ""),
        "compute_units": props.multi_processor_count,
    }
    result["device"].update(hip_clocks(props.multi_processor_count))

    # ---- CPU oracle: bit-exact check on a sample of chunks + its own rate
    if not args.no_oracle:
        import oracle

        ks = list(range(min(args.oracle_chunks, cfg.n_chunks)))
        od = oracle.desc_for(cfg)
        t0 = time.time()
        otb = oracle.profile(od, kvp)
        conts = [oracle.encode_chunk(od, otb, kv, k, levels[k]) for k in ks]
        log(f"oracle profile + encode of {len(ks)} chunks in {time.time() - t0:.1f} s")
        exact = otb.profile_id == kvc.profile_id(tables)
        for i, k in enumerate(ks):
            exact = exact and np.array_equal(enc.container(k).cpu().numpy(), conts[i])
        oout = np.zeros((cfg.n_layers, 2, cfg.n_tokens, cfg.n_channels), np.uint16)
        t0 = time.perf_counter()
        for i, k in enumerate(ks):
            oracle.decode_chunk_into(od, otb, conts[i], 1500 * k, cfg.chunk_tokens(k), levels[k], oout)
        cpu_s = time.perf_counter() - t0
        hi = 1500 * ks[-1] + cfg.chunk_tokens(ks[-1])
        got = out[:, :, :hi].cpu().numpy().view(np.uint16)
        exact = exact and np.array_equal(got, oout[:, :, :hi])
        if hi == cfg.n_tokens:
            result["sha256"]["decoded_fp16"] = sha256_of(np.ascontiguousarray(got))
        sample_bytes = 2 * cfg.n_layers * cfg.n_channels * hi * 2
        result["bit_exact"] = bool(exact)
        result["cpu_baseline"] = {
            "value": round(sample_bytes / cpu_s / 1e9, 4),
            "unit": "GB/s",
            "cores": oracle.get_threads(),
            "kind": "oracle",
            "sample": f"oracle decode of chunks {ks} ({hi} tokens, all {cfg.n_layers} layers, "
                      f"{sample_bytes / 1e9:.2f} GB of binary16) in {cpu_s:.2f} s",
        }
        log(f"oracle decode {sample_bytes / 1e9:.2f} GB in {cpu_s:.1f} s; bit_exact={exact}")
        if renc is not None:
            # the refinement layer: tables id, first and last chunk's refinement
            # container and refined KV against the oracle's
            ort = oracle.profile_refine(od, kvp, refine_bits, otb.profile_id)
            rexact = ort.refine_id == kvc.refine_id(rtables)
            for k in sorted({0, cfg.n_chunks - 1}):
                oc = conts[k] if k < len(conts) else oracle.encode_chunk(od, otb, kv, k, levels[k])
                orc = oracle.encode_refine_chunk(od, ort, kv, k, levels[k])
                rexact = rexact and np.array_equal(renc.container(k).cpu().numpy(), orc)
                n = cfg.chunk_tokens(k)
                oo = np.zeros((cfg.n_layers, 2, n, cfg.n_channels), np.uint16)
                oracle.decode_refined_chunk_into(od, otb, oc, ort, orc, 0, n, levels[k], oo)
                got = refined_out[:, :, 1500 * k:1500 * k + n].cpu().numpy().view(np.uint16)
                rexact = rexact and np.array_equal(got, oo)
            result["refinement"]["bit_exact_first_last_chunk"] = bool(rexact)
            log(f"refinement bit_exact (chunks 0 and last) = {rexact}")
        # the same oracle on one core, on its first chunk
        threads = oracle.get_threads()
        oracle.set_threads(1)
        one = np.zeros((cfg.n_layers, 2, cfg.chunk_tokens(0), cfg.n_channels), np.uint16)
        t0 = time.perf_counter()
        oracle.decode_chunk_into(od, otb, conts[0], 0, cfg.chunk_tokens(0), levels[0], one)
        one_s = time.perf_counter() - t0
        oracle.set_threads(threads)
        one_bytes = one.size * 2
        result["cpu_baseline_one_core"] = {
            "value": round(one_bytes / one_s / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle decode of chunk 0 ({cfg.chunk_tokens(0)} tokens, "
                      f"{one_bytes / 1e9:.2f} GB of binary16) in {one_s:.2f} s on one thread",
        }
        log(f"oracle on one core: {one_bytes / 1e9:.2f} GB in {one_s:.1f} s")
        # and on the tiny workload (one 1,500-token chunk of 4 layers x 512
        # channels), also on one core
        tiny = synth.TINY
        tkv = synth.make_kv(tiny)
        tod = oracle.desc_for(tiny)
        ttb = oracle.profile(tod, synth.make_profile_kv(tiny))
        tlev = tiny.chunk_levels()
        tcont = oracle.encode(tod, ttb, tkv, tlev)
        oracle.set_threads(1)
        t0 = time.perf_counter()
        oracle.decode(tod, ttb, tcont, tlev, tiny.n_tokens)
        tiny_s = time.perf_counter() - t0
        oracle.set_threads(threads)
        result["cpu_baseline_tiny_one_core"] = {
            "value": round(tiny.fp16_bytes() / tiny_s / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle decode of the whole {tiny.name} workload ({tiny.fp16_bytes() / 1e6:.1f} MB "
                      f"of binary16) in {tiny_s:.2f} s on one thread",
        }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Benchmark of the Muse Glimmer attention core on one MI355X.

Default workload: the 52-layer attention schedule (layers l % 4 == 3 full
NoPE, the others sliding RoPE with a 2,048-key window) for 4 sequences with
32,768 cached rows per layer: a chunked prefill of 4,096 new tokens through
all 52 layers, then decode steps.  One "step" is one decode step of all 52
layers -- QK-norm, RoPE, KV append, split-K attention, merge and gate in
every layer, then the device-side position increment -- replayed from a
HIP graph.  `value` is the decode phase's attention KV bytes per second
(the visible K/V rows, 1,024 B per row per sequence, summed over the timed
steps and layers).  The chunked prefill is timed in the same run and
reported under "prefill" in TFLOP/s (16,384 flop per visible (query, key)
pair over 32 heads), so the line carries both halves of the metric.  The
other workloads (the 1 x 512 f32 prefill, the 64 x 8,192 decode, the 8 x
8,192 prefill, the 16 x 131,072 decode) are extra legs under "configs".

Inputs are seeded synthetic tensors already resident in HBM.  `roofline`
uses the attention kernel's own launch time from HIP events the library
records around it.  `cpu_baseline` times the CPU oracle on a bounded sample
of the same workload (rank 0, N=1); each leg carries its own.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attn KV GB/s (% HBM peak) + prefill attn TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 / fp16 MFMA
FP32_PEAK_TFLOPS = 157.3         # MI355X fp32 (the 1 x 512 f32 workload)
FLOP_PER_PAIR = 32 * 4 * 128     # 32 heads x (2*128 for Q.K + 2*128 for P.V)
MALL_BYTES = 256 << 20
HEADLINE = "schedule_52x4_32768p4096_256d"


def kv_row_bytes(dtype: int) -> int:
    return 2 * 2 * 128 * (2 if dtype == 1 else 4)   # K and V, 2 kv heads x 128


def visible_rows(spec, p: int) -> int:
    return p + 1 if spec.window == 0 else min(spec.window, p + 1)


def prefill_pairs(spec, L: int, N: int) -> int:
    return sum(visible_rows(spec, L + t) for t in range(N))


PROFILES = os.path.join(ROOT, "profiles")
COUNTERS_FILE = os.path.join(PROFILES, "decode_schedule_52x4_hbm_counters.md")
DECODE_SOURCES = ["full_gqa_attention_amd/csrc/decode.hip", "full_gqa_attention_amd/csrc/device_common.h",
                  "full_gqa_attention_amd/csrc/kernels.h", "full_gqa_attention_amd/csrc/muse_attn.cpp"]
MFMA_FILE = os.path.join(PROFILES, "prefill_8x8192_bf16_mfma_counters.md")
PREFILL_SOURCES = ["full_gqa_attention_amd/csrc/prefill.hip", "full_gqa_attention_amd/csrc/device_common.h",
                   "full_gqa_attention_amd/csrc/kernels.h", "full_gqa_attention_amd/csrc/muse_attn.cpp"]
SIMDS = 256 * 4                  # 256 CUs x 4 SIMDs
XCDS = 8
# A plain 1 GiB device copy read back 524,315 KiB on FETCH_SIZE and 1,048,576 KiB
# on WRITE_SIZE: the factors that turn the counters into bytes.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0


def sources_hash(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_summary_values(path: str) -> dict:
    """The indented `key: value` lines of a committed counter summary."""
    kv = {}
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("    ") and ":" in line:
                    k, v = line.strip().split(":", 1)
                    kv[k.strip()] = v.strip()
    except OSError:
        pass
    return kv


def counter_traffic():
    """HBM bytes per decode-kernel launch of the headline schedule (full and
    sliding layers) from the committed counter summary, or None when the
    decode kernel's sources changed since it was taken."""
    kv = read_summary_values(COUNTERS_FILE)
    if kv.get("decode_sources_sha256_16") != sources_hash(DECODE_SOURCES):
        return None
    try:
        return {"all": float(kv["hbm_bytes_per_launch"]), "full": float(kv["hbm_bytes_per_launch_full"]),
                "sliding": float(kv["hbm_bytes_per_launch_sliding"])}
    except (KeyError, ValueError):
        return None


def prefill_counters():
    """MFMA utilisation of the prefill kernel per layer from the committed
    counter summary, or None when the prefill sources changed since."""
    kv = read_summary_values(MFMA_FILE)
    if kv.get("prefill_sources_sha256_16") != sources_hash(PREFILL_SOURCES):
        return None
    try:
        return {"mfma_busy": {"sliding": float(kv["mfma_busy_sliding"]), "full": float(kv["mfma_busy_full"])},
                "clock_GHz": {"sliding": float(kv["clock_ghz_sliding"]), "full": float(kv["clock_ghz_full"])},
                "source": os.path.relpath(MFMA_FILE, ROOT)}
    except (KeyError, ValueError):
        return None


def summarize_counters(fetch_csv: str, write_csv: str, out: str, command: str):
    """Write the decode kernels' HBM-traffic summary from two --pmc runs of
    `bench.py --counters-run` (eager decode steps of the 52-layer schedule:
    dispatches in layer order, layer l full NoPE iff l % 4 == 3)."""
    import csv

    def per_kernel(path):
        copy, dec, merge = [], [], []
        for r in csv.DictReader(open(path)):
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            if "decode_merge_kernel" in name:
                merge.append(v)
            elif "decode_kernel" in name:
                dec.append(v)
            elif "copyBuffer" in name:
                copy.append(v)
        return copy, dec, merge

    fc, fd, fm = per_kernel(fetch_csv)
    wc, wd, wm = per_kernel(write_csv)
    kinds = ["full" if i % 52 % 4 == 3 else "sliding" for i in range(len(fd))]

    def avg(xs, kind):
        v = [x for x, k in zip(xs, kinds) if kind in (k, "all")]
        return sum(v) / len(v)

    mk = ["full" if i % 52 % 4 == 3 else "sliding" for i in range(len(fm))]

    def mavg(xs, kind):
        v = [x for x, k in zip(xs, mk) if kind in (k, "all")]
        return sum(v) / len(v)

    rows, vals = [], {}
    for kind in ("sliding", "full", "all"):
        fb = avg(fd, kind) * 1024 * FETCH_SCALE
        wb = avg(wd, kind) * 1024 * WRITE_SCALE
        rows.append(f"| decode_kernel, {kind} | {avg(fd, kind):.1f} | {avg(wd, kind):.1f} | {fb / 1e6:.2f} | "
                    f"{wb / 1e6:.3f} |")
        mf = mavg(fm, kind) * 1024 * FETCH_SCALE
        mw = mavg(wm, kind) * 1024 * WRITE_SCALE
        rows.append(f"| decode_merge_kernel, {kind} | {mavg(fm, kind):.1f} | {mavg(wm, kind):.1f} | "
                    f"{mf / 1e6:.2f} | {mw / 1e6:.3f} |")
        vals[kind] = fb + wb + mf + mw                 # one decode call: the split kernel and the merge kernel
    lines = ["# HBM traffic of the decode kernels: 52-layer schedule, 4 sequences at 36,864 + step cached rows", "",
             "Two counter runs (from /tmp, repository at $ROOT):", "", "```", command, "```", "",
             f"Calibration: the first copy in each run is a 1 GiB device copy (`--calibrate-copy`); it read "
             f"{fc[0]:.1f} KiB on FETCH_SIZE and {wc[0]:.1f} KiB on WRITE_SIZE, so FETCH_SIZE is scaled by "
             f"{FETCH_SCALE} and WRITE_SIZE by {WRITE_SCALE}.  Algorithmic KV bytes per launch: sliding "
             f"4 x 2,048 x 1,024 B = 8.39 MB; full 4 x (p + 1) x 1,024 B = 151.0 MB at p = 36,864.", "",
             "| kernel, layers | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |",
             "|---|---|---|---|---|", *rows, "",
             "Values read by bench.py: HBM bytes per decode call, split and merge kernels together (traffic is "
             "reported only while these sources are unchanged):", "",
             f"    decode_sources_sha256_16: {sources_hash(DECODE_SOURCES)}",
             f"    hbm_bytes_per_launch: {vals['all']:.0f}",
             f"    hbm_bytes_per_launch_full: {vals['full']:.0f}",
             f"    hbm_bytes_per_launch_sliding: {vals['sliding']:.0f}", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed decode steps of the schedule (at most 256)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prefill-steps", type=int, default=3, help="timed chunked-prefill passes")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' legs")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timings")
    ap.add_argument("--ring", action="store_true",
                    help="sliding layers keep their window in a ring cache (kv_ring) in the schedule")
    ap.add_argument("--verify", action="store_true",
                    help="also time the 16-token verify call (64 x 8,192 cached rows, both layers)")
    ap.add_argument("--out-proj", action="store_true",
                    help="also time the block's tail (o_proj + post-attention norm) at 65,536 and 64 tokens")
    ap.add_argument("--summarize-legs", nargs=5, metavar=("TRACE_CSV", "FETCH_CSV", "WRITE_CSV", "OUT", "COMMAND"),
                    help="write the per-kernel summary of the verify / o_proj / relocate legs")
    ap.add_argument("--only-next", action="store_true",
                    help="run only the legs asked for with --verify / --out-proj / --relocate (no schedule, no configs)")
    ap.add_argument("--relocate", action="store_true",
                    help="also time NoPE tile relocation (muse_kv_relocate) of a 64 x 8,192 full-layer cache")
    ap.add_argument("--counters-run", action="store_true",
                    help="only the schedule's chunk and 2 eager decode steps (for --pmc counter runs)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the 8 x 8,192 prefill and print its JSON object (for counter runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy first (scale for HBM byte counters)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_CSV", "OUT", "COMMAND"),
                    help="write a kernel-trace summary from rocprofv3 kernel_trace.csv and exit")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "OUT", "COMMAND"),
                    help="write the decode kernels' HBM-traffic summary from two --pmc runs and exit")
    ap.add_argument("--decode-timeline", nargs="?", const="", metavar="OUT_MD",
                    help="per-phase decode timelines from the profiling build (build it with "
                         "`python full_gqa_attention_amd/build.py --timeline`); optional markdown summary path")
    ap.add_argument("--decode-leg", nargs=2, metavar=("WORKLOAD", "KIND"),
                    help="replay one layer kind of a decode workload from a HIP graph (for a kernel trace)")
    ap.add_argument("--summarize-leg-traces", nargs="+", metavar="ARG",
                    help="OUT COMMAND LABEL CSV [LABEL CSV ...]: per-layer decode summary from --decode-leg traces")
    ap.add_argument("--summarize-mfma", nargs=4, metavar=("PMC1_CSV", "PMC2_CSV", "OUT", "COMMAND"),
                    help="write the prefill kernel's MFMA-utilisation summary from two --pmc runs and exit")
    return ap.parse_args()


def percentiles(xs):
    """p10, p50, p90 (nearest rank) of a list of launch times."""
    v = sorted(xs)
    return [v[min(len(v) - 1, int(q * len(v)))] for q in (0.1, 0.5, 0.9)]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _kind(spec, synth) -> str:
    return "full" if spec.kind == synth.FULL_NOPE else "sliding"


def kernel_roofline(kind_ms, kind_bytes, peak, unit, scale, kernel):
    """Roofline of a kernel from per-launch times (ms) and algorithmic work per
    launch, overall and per layer kind: achieved = average work per launch /
    average launch time."""
    per = {}
    all_ms, all_w = [], []
    for kind in kind_ms:
        ms, wk = kind_ms[kind], kind_bytes[kind]
        all_ms += ms
        all_w += wk
        a = (sum(wk) / len(wk)) / (sum(ms) / len(ms) * 1e-3) / scale
        per[kind] = {"launches": len(ms), "avg_launch_us": round(1e3 * sum(ms) / len(ms), 2),
                     "p10_p50_p90_us": [round(1e3 * x, 2) for x in percentiles(ms)],
                     "algorithmic_per_launch": round(sum(wk) / len(wk)), "achieved": round(a, 1),
                     "frac": round(a / peak, 4)}
    a = (sum(all_w) / len(all_w)) / (sum(all_ms) / len(all_ms) * 1e-3) / scale
    return {"achieved": round(a, 1), "peak": peak, "unit": unit, "frac": round(a / peak, 4), "kernel": kernel,
            "launches": len(all_ms), "avg_launch_us": round(1e3 * sum(all_ms) / len(all_ms), 2),
            "algorithmic_per_launch": round(sum(all_w) / len(all_w)), "per_kind": per}


# ---------------------------------------------------------------- headline

def bench_schedule(args, fa, synth, torch):
    """The 52-layer schedule: the chunked prefill (eager calls, timed as a
    phase and per attention kernel), then the decode phase: a few eager steps
    with the library's kernel timer on every call (the roofline), and the
    timed steps replayed from a captured HIP graph (`value`)."""
    from full_gqa_attention_amd.schedule import Schedule
    from full_gqa_attention_amd.timing import KernelTimers
    w = synth.WORKLOADS[HEADLINE]
    S, L0, N = w.n_seq, w.prefix, w.n_new
    K = max(1, min(args.steps, w.decode_steps))
    sch = Schedule(w, ring=args.ring)
    kinds = [_kind(s, synth) for s in sch.specs]
    log(f"schedule {w.name}: {len(sch.specs)} layers, cache {sch.cache_bytes() / 1e9:.2f} GB, ring={args.ring}")
    torch.cuda.synchronize()
    # ---- chunked prefill: one warm-up pass, then timed passes (each rewrites the same rows)
    sch.prefill()
    torch.cuda.synchronize()
    P = max(1, args.prefill_steps)
    timers = KernelTimers(P * len(sch.specs))
    t0 = time.perf_counter()
    for i in range(P):
        sch.prefill(timers=[timers[i * len(sch.specs) + l] for l in range(len(sch.specs))])
    torch.cuda.synchronize()
    t_prefill = (time.perf_counter() - t0) / P
    pms = {"sliding": [], "full": []}
    pfl = {"sliding": [], "full": []}
    for i in range(P):
        for l, spec in enumerate(sch.specs):
            pms[kinds[l]].append(timers.elapsed_ms(i * len(sch.specs) + l))
            pfl[kinds[l]].append(FLOP_PER_PAIR * S * prefill_pairs(spec, L0, N))
    timers.close()
    flops = sum(FLOP_PER_PAIR * S * prefill_pairs(spec, L0, N) for spec in sch.specs)
    prefill = {"workload": f"{w.name} (chunk of {N} tokens onto {L0} cached rows, 52 layers)",
               "ms": round(t_prefill * 1e3, 3), "tflop": round(flops / 1e12, 3),
               "tflops": round(flops / t_prefill / 1e12, 1),
               "frac_mfma_peak": round(flops / t_prefill / 1e12 / MFMA_PEAK_TFLOPS, 4),
               "launch": "eager calls, prep (K-hat, V append) and attention per layer",
               "roofline": dict(bound="mfma", traffic=None, **kernel_roofline(
                   pms, pfl, MFMA_PEAK_TFLOPS, "TFLOP/s", 1e12,
                   "muse::prefill_group_kernel<1, 8, 1> (bf16)"))}
    # ---- decode roofline: per layer kind, a HIP graph of that kind's decode
    # calls at the first decode position (split kernel + merge kernel each),
    # replayed between HIP events on the stream it runs on
    R = 8
    dms = {"sliding": [], "full": []}
    dby = {"sliding": [], "full": []}
    sch.start_decode()
    for kind in ("sliding", "full"):
        idx = [l for l in range(len(sch.specs)) if kinds[l] == kind]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in idx:
                sch.decode_layer(l)
        g.replay()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R)]
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        for a, b in ev:
            dms[kind] += [a.elapsed_time(b) / len(idx)] * len(idx)
            dby[kind] += [kv_row_bytes(w.dtype) * S * visible_rows(sch.specs[l], L0 + N) for l in idx]
        del g
    roof = dict(bound="hbm", **kernel_roofline(
        dms, dby, HBM_PEAK_GBS, "GB/s", 1e9,
        "one decode call: muse::decode_kernel<bf16> (split) + muse::decode_merge_kernel<bf16> (merge)"))
    roof["measured"] = ("per layer kind, a graph of that kind's decode calls replayed between HIP events; "
                        "the trace's per-call time is the two kernels' averages added")
    tr = counter_traffic() if not args.ring else None
    roof["traffic"] = tr["all"] if tr else None
    if tr:
        for kind in ("full", "sliding"):
            roof["per_kind"][kind]["traffic"] = tr[kind]
    # the split kernel alone, from the library's timer on eager calls (the
    # events' own cost is a few microseconds of these times)
    E = min(4, K)
    sch.start_decode()
    timers = KernelTimers(E * len(sch.specs))
    for i in range(E):
        sch.decode_step(timers=[timers[i * len(sch.specs) + l] for l in range(len(sch.specs))])
    torch.cuda.synchronize()
    split = {"sliding": [], "full": []}
    for i in range(E):
        for l in range(len(sch.specs)):
            split[kinds[l]].append(1e3 * timers.elapsed_ms(i * len(sch.specs) + l))
    timers.close()
    roof["split_kernel_eager_event_us"] = {k: round(sum(v) / len(v), 2) for k, v in split.items()}
    # ---- decode: the timed steps, replayed from one captured step
    sch.start_decode()
    graph = sch.capture_step()
    for _ in range(args.warmup):
        graph.replay()
    sch.start_decode()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del graph
    kv = sum(kv_row_bytes(w.dtype) * S * visible_rows(spec, L0 + N + i) for i in range(K) for spec in sch.specs)
    res = {"value": kv / wall / 1e9, "ms_per_step": wall * 1e3 / K, "kv_bytes": kv, "steps": K,
           "roofline": roof, "prefill": prefill,
           "config": {"workload": w.name, "layers": len(sch.specs), "full_layers": kinds.count("full"),
                      "n_seq": S, "cached_tokens": L0, "chunk_tokens": N,
                      "decode_positions": [L0 + N, L0 + N + K - 1], "q_heads": 32, "kv_heads": 2,
                      "head_dim": 128, "window": 2048, "rope_theta": 500000.0, "kv_ring_sliding": bool(args.ring),
                      "kv_cache_GB": round(sch.cache_bytes() / 1e9, 3),
                      "decode_kv_bytes_per_step": round(kv / K)}}
    return res, sch


def oracle_layer_of(spec, dtype):
    import oracle
    return oracle.Layer(kind=spec.kind, window=spec.window, rope_theta=spec.rope_theta, rms_eps=spec.rms_eps,
                        q_gain=spec.q_gain, k_gain=spec.k_gain, scale=spec.scale, dtype=dtype)


def cpu_schedule_sample(sch, fa, synth, torch, n_steps: int = 4):
    """The oracle on a bounded sample of the schedule, on the cache the GPU
    holds: every layer's decode rows (all 4 sequences, all 32 heads) at the
    first n_steps decode positions (the GPU's outputs there come from eager
    decode steps run again here), and two rows of every layer's chunk
    (sequence 0, tokens 0 and n_new - 1; linear caches only).  Returns the
    oracle's times and work and the parity of the sampled GPU outputs."""
    import numpy as np
    import oracle
    w = sch.w
    S, L0, N = w.n_seq, w.prefix, w.n_new
    sch.start_decode()
    outs = []
    for i in range(n_steps):
        sch.decode_step()
        torch.cuda.synchronize()
        outs.append([d[4][:, 0].double().cpu().numpy() for d in sch.dec])
    t_dec = t_pre = 0.0
    kv = pairs = 0
    worst, ok = 0.0, True
    prows = np.array([(0, 0), (0, N - 1)], np.int32)

    def check(got, ref):
        nonlocal worst, ok
        err = np.abs(got - ref)
        worst = max(worst, float(err.max()))
        ok = ok and bool(np.all(err <= 2e-2 + 1e-2 * np.abs(ref)))

    for l, spec in enumerate(sch.specs):
        inp = sch.inputs[l]
        q, k, v, g, _ = sch.dec[l]
        top = L0 + N + n_steps
        ring = sch.is_ring(spec)
        lo = 0 if spec.window == 0 else max(0, (L0 + N if ring else L0) - spec.window + 1)
        ck = np.zeros((S, top, 2, 128), np.uint16)
        cv = np.zeros_like(ck)
        pos = torch.arange(lo, top, device=inp.cache_k.device)
        rows = pos % spec.window if ring else pos
        ck[:, lo:top] = synth.to_storage_numpy(inp.cache_k[:, rows])
        cv[:, lo:top] = synth.to_storage_numpy(inp.cache_v[:, rows])
        lay = oracle_layer_of(spec, w.dtype)
        u16 = synth.to_storage_numpy
        for i in range(n_steps):
            p = L0 + N + i
            args = (lay, np.full(S, p, np.int32), u16(k), u16(v), ck, cv, oracle.all_rows(S, 1),
                    u16(q).reshape(S, 32, 128), u16(g).reshape(S, 4096))
            t0 = time.perf_counter()
            ref = oracle.attn_rows(*args)
            t_dec += time.perf_counter() - t0
            kv += kv_row_bytes(w.dtype) * S * visible_rows(spec, p)
            check(outs[i][l], ref)
        if not ring:                                   # a ring no longer holds the chunk's prefix
            sel = (prows[:, 0], prows[:, 1])
            args = (lay, np.full(S, L0, np.int32), u16(inp.k), u16(inp.v), ck, cv, prows,
                    u16(inp.q)[sel], u16(inp.gate)[sel])
            t0 = time.perf_counter()
            ref = oracle.attn_rows(*args)
            t_pre += time.perf_counter() - t0
            pairs += sum(visible_rows(spec, L0 + int(t)) for t in prows[:, 1])
            check(sch.outs[l][sel].double().cpu().numpy().reshape(len(prows), -1), ref)
    return {"decode_s": t_dec, "decode_kv": kv, "prefill_s": t_pre, "prefill_pairs": pairs,
            "parity": {"max_abs_err": worst, "within_tolerance": ok,
                       "rows": f"{n_steps} decode steps x 52 layers x {S} sequences and 2 chunk rows per layer, "
                               "all 32 heads, against the oracle"}}


# ----------------------------------------------------------- other workloads

class LayerRun:
    """One layer of a decode or prefill workload with its inputs and caches
    (decode: rotated over `copies` cache copies, so the 256 MB Infinity Cache
    cannot serve a step from the previous one)."""

    def __init__(self, w, spec, copies, decode, fa, synth):
        import torch
        self.spec = spec
        self.inp = synth.layer_inputs(w, spec, device="cuda", backend="torch")
        self.caches = [(self.inp.cache_k, self.inp.cache_v)]
        for _ in range(1, copies):
            self.caches.append((self.inp.cache_k.clone(), self.inp.cache_v.clone()))
        self.layer = fa.make_layer(spec.kind, window=spec.window, rope_theta=spec.rope_theta,
                                   rms_eps=spec.rms_eps, q_norm_gain=spec.q_gain,
                                   k_norm_gain=spec.k_gain, attn_scale=spec.scale, dtype=w.dtype)
        self.decode = decode
        self.ws = fa.workspace(self.layer, w.n_seq, w.n_new, w.prefix, decode)
        self.out = torch.empty_like(self.inp.gate)
        self.max_seq_len = w.prefix

    def call(self, fa, copy, timer=None):
        ck, cv = self.caches[copy]
        fn = fa.decode if self.decode else fa.prefill
        fn(self.layer, self.inp.q, self.inp.k, self.inp.v, self.inp.gate, ck, cv, self.inp.seq_len,
           self.out, max_seq_len=self.max_seq_len, workspace=self.ws, timer=timer)


def run_timed(runs, steps, warmup, copies, fa, torch):
    """W untimed steps, then K timed steps between synchronisations, with the
    kernel timer on every call."""
    from full_gqa_attention_amd.timing import KernelTimers
    timers = KernelTimers(steps * len(runs))
    for i in range(warmup):
        for r in runs:
            r.call(fa, i % copies)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for j, r in enumerate(runs):
            r.call(fa, (warmup + i) % copies, timers[i * len(runs) + j])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = [timers.elapsed_ms(i) for i in range(len(timers))]
    timers.close()
    return wall, per_launch


def run_graphs(runs, steps, warmup, copies, fa, torch):
    """The same steps replayed from HIP graphs (one captured step per cache copy)."""
    graphs = []
    for c in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in runs:
                r.call(fa, c)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[(warmup + i) % copies].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del graphs
    return wall


def leg_decode(w, fa, synth, torch, steps=20, warmup=3, cpu=True):
    """A decode workload (both layer kinds), graph-replayed; the kernel
    timer on every call of an eager pass gives the per-kind roofline.  The CPU
    oracle runs on the whole step and checks the GPU output."""
    per_step = sum(kv_row_bytes(w.dtype) * w.n_seq * visible_rows(s, w.prefix) for s in w.layers)
    copies = min(8, max(1, -(-(2 * MALL_BYTES) // max(per_step, 1)) + 1))
    log(f"decode {w.name}: {copies} cache copies, {per_step / 1e6:.1f} MB KV per step")
    runs = [LayerRun(w, spec, copies, True, fa, synth) for spec in w.layers]
    torch.cuda.synchronize()
    _, per_launch = run_timed(runs, steps, warmup, copies, fa, torch)
    wall = run_graphs(runs, steps, warmup, copies, fa, torch)
    ms = {"sliding": [], "full": []}
    by = {"sliding": [], "full": []}
    for j, r in enumerate(runs):
        ms[_kind(r.spec, synth)] += per_launch[j::len(runs)]
        by[_kind(r.spec, synth)] += [kv_row_bytes(w.dtype) * w.n_seq * visible_rows(r.spec, w.prefix)] * steps
    res = {"metric": "decode attn KV GB/s", "value": round(per_step * steps / wall / 1e9, 1), "unit": "GB/s",
           "ms_per_step": round(wall * 1e3 / steps, 5), "frac_hbm_peak": round(per_step * steps / wall / 1e9 / HBM_PEAK_GBS, 4),
           "launch": "each step replayed from a HIP graph", "cache_copies": copies,
           "roofline": dict(bound="hbm", traffic=None, **kernel_roofline(ms, by, HBM_PEAK_GBS, "GB/s", 1e9,
                                                                         "muse::decode_kernel<bf16>"))}
    if cpu:
        res["cpu_baseline"], res["parity"] = cpu_decode_full(w, runs, synth, torch)
    del runs
    torch.cuda.empty_cache()
    return res


def cpu_decode_full(w, runs, synth, torch):
    """The oracle on every row of the decode step (all sequences, both layers)."""
    import numpy as np
    import oracle
    rows = oracle.all_rows(w.n_seq, 1)
    t_oracle, worst, ok = 0.0, 0.0, True
    for r in runs:
        ck, cv = r.caches[0]
        args = (oracle_layer_of(r.spec, w.dtype), r.inp.seq_len.cpu().numpy(), synth.to_storage_numpy(r.inp.k),
                synth.to_storage_numpy(r.inp.v), synth.to_storage_numpy(ck), synth.to_storage_numpy(cv), rows,
                synth.to_storage_numpy(r.inp.q).reshape(-1, 32, 128),
                synth.to_storage_numpy(r.inp.gate).reshape(-1, 4096))
        t0 = time.perf_counter()
        ref = oracle.attn_rows(*args)
        t_oracle += time.perf_counter() - t0
        err = np.abs(r.out.double().cpu().numpy().reshape(-1, 4096) - ref)
        worst = max(worst, float(err.max()))
        ok = ok and bool(np.all(err <= 2e-2 + 1e-2 * np.abs(ref)))
    kv = sum(kv_row_bytes(w.dtype) * w.n_seq * visible_rows(r.spec, w.prefix) for r in runs)
    return ({"value": round(kv / t_oracle / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
             "sample": f"the whole step: {w.n_seq} sequences x {len(runs)} layers, all 32 heads",
             "seconds": round(t_oracle, 3)},
            {"max_abs_err": worst, "within_tolerance": ok})


def leg_prefill(w, fa, synth, torch, steps=5, warmup=2, cpu=True, cpu_rows=None, single_core=False):
    """A prefill workload (both layer kinds), eager calls with the kernel
    timer on each; the CPU oracle on every row (cpu_rows None) or a sample."""
    log(f"prefill {w.name}")
    runs = [LayerRun(w, spec, 1, False, fa, synth) for spec in w.layers]
    torch.cuda.synchronize()
    wall, per_launch = run_timed(runs, steps, warmup, 1, fa, torch)
    flops = sum(FLOP_PER_PAIR * w.n_seq * prefill_pairs(s, w.prefix, w.n_new) for s in w.layers)
    ms = {"sliding": [], "full": []}
    fl = {"sliding": [], "full": []}
    for j, r in enumerate(runs):
        ms[_kind(r.spec, synth)] += per_launch[j::len(runs)]
        fl[_kind(r.spec, synth)] += [FLOP_PER_PAIR * w.n_seq * prefill_pairs(r.spec, w.prefix, w.n_new)] * steps
    bf16 = w.dtype == synth.BF16
    peak = MFMA_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS
    kern = "muse::prefill_group_kernel<1, 8, 1> (bf16)" if bf16 else "muse::prefill_kernel<float> (f32)"
    res = {"metric": "prefill attn TFLOP/s", "value": round(flops * steps / wall / 1e12, 2), "unit": "TFLOP/s",
           "ms_per_step": round(wall * 1e3 / steps, 4), "frac_peak": round(flops * steps / wall / 1e12 / peak, 4),
           "launch": "eager calls (prep and attention kernels per layer)",
           "roofline": dict(bound="mfma", traffic=None, **kernel_roofline(ms, fl, peak, "TFLOP/s", 1e12, kern))}
    if w.name == "prefill_8x8192_bf16":
        res["roofline"]["counters"] = prefill_counters()
    if cpu:
        res["cpu_baseline"], res["parity"] = cpu_prefill(w, runs, synth, cpu_rows, single_core)
    del runs
    torch.cuda.empty_cache()
    return res


def cpu_prefill(w, runs, synth, rows, single_core):
    """The oracle on every row (rows None) or on the given (s, t) sample, in
    pairs/s and rows/s; a sample reports the extrapolated full-run time."""
    import numpy as np
    import oracle
    full = rows is None
    rows = oracle.all_rows(w.n_seq, w.n_new) if full else np.asarray(rows, np.int32)
    res, worst, ok = {}, 0.0, True
    default_threads = oracle.num_threads()
    for threads in ([1] if single_core else []) + [0]:
        if threads:
            oracle.set_num_threads(threads)
        t_oracle, pairs = 0.0, 0
        for r in runs:
            sel = (rows[:, 0], rows[:, 1])
            q = synth.to_storage_numpy(r.inp.q)[sel]
            g = synth.to_storage_numpy(r.inp.gate)[sel]
            args = (oracle_layer_of(r.spec, w.dtype), r.inp.seq_len.cpu().numpy(), synth.to_storage_numpy(r.inp.k),
                    synth.to_storage_numpy(r.inp.v), None, None, rows, q, g)
            t0 = time.perf_counter()
            ref = oracle.attn_rows(*args)
            t_oracle += time.perf_counter() - t0
            pairs += sum(visible_rows(r.spec, w.prefix + int(t)) for t in rows[:, 1])
            got = r.out.double().cpu().numpy()[sel].reshape(len(rows), -1)
            err = np.abs(got - ref)
            worst = max(worst, float(err.max()))
            tol = 1e-4 if w.dtype == synth.F32 else 2e-2 + 1e-2 * np.abs(ref)
            ok = ok and bool(np.all(err <= tol))
        total_pairs = sum(w.n_seq * prefill_pairs(r.spec, w.prefix, w.n_new) for r in runs)
        entry = {"value": round(pairs * FLOP_PER_PAIR / t_oracle / 1e12, 6), "unit": "TFLOP/s",
                 "pairs_per_s": round(pairs / t_oracle), "rows_per_s": round(len(rows) * len(runs) / t_oracle, 1),
                 "cores": oracle.num_threads(), "kind": "oracle", "seconds": round(t_oracle, 3),
                 "sample": ("every row" if full else f"{len(rows)} (sequence, token) rows per layer (window and "
                            f"tile edges), all 32 heads, both layers")}
        if not full:
            entry["extrapolated_full_run_s"] = round(t_oracle * total_pairs / pairs, 1)
            entry["extrapolation"] = "full-run time = sample time x all visible pairs / sampled pairs"
        res["single_core" if threads == 1 else "all_cores"] = entry
        if threads:
            oracle.set_num_threads(default_threads)
    out = res["all_cores"]
    if single_core:
        out = dict(out, single_core=res["single_core"])
    return out, {"max_abs_err": worst, "within_tolerance": ok}


def summarize_mfma(pmc1_csv: str, pmc2_csv: str, out: str, command: str):
    """Write the prefill kernel's MFMA-utilisation summary from two --pmc runs
    of `bench.py --prefill-only` (launches alternate sliding, full)."""
    import csv
    per = {}
    for path in (pmc1_csv, pmc2_csv):
        for r in csv.DictReader(open(path)):
            if "prefill_group_kernel" not in r["Kernel_Name"]:
                continue
            key = (path, int(r["Dispatch_Id"]))
            d = per.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    layers = {"sliding": [], "full": []}
    for path in (pmc1_csv, pmc2_csv):
        ds = [per[k] for k in sorted(k for k in per if k[0] == path)]
        layers["sliding"] += ds[0::2]
        layers["full"] += ds[1::2]

    def avg(ds, c):
        vals = [d[c] for d in ds if c in d]
        return sum(vals) / len(vals) if vals else float("nan")

    flops = {"sliding": 1.9243e12, "full": 4.3986e12}     # algorithmic, 8 x 8,192 tokens
    rows, vals = [], {}
    for name, ds in layers.items():
        ns = avg(ds, "ns")
        cyc = avg(ds, "GRBM_GUI_ACTIVE") / XCDS                  # per-XCD busy cycles
        clock = cyc / ns
        busy = avg(ds, "SQ_VALU_MFMA_BUSY_CYCLES") / (SIMDS * cyc)
        coexec = avg(ds, "SQ_VALU_MFMA_COEXEC_CYCLES") / (SIMDS * cyc)
        mfma = avg(ds, "SQ_INSTS_MFMA")
        executed = mfma * 32 * 32 * 16 * 2                        # v_mfma_f32_32x32x16 flops
        rows.append(f"| {name} | {ns / 1e6:.3f} | {clock:.2f} | {busy * 100:.1f} | {coexec * 100:.1f} | "
                    f"{flops[name] / (ns * 1e-9) / 1e12:.0f} | {executed / flops[name]:.3f} | "
                    f"{avg(ds, 'SQ_INSTS_VALU') / mfma:.2f} | {avg(ds, 'SQ_INSTS_LDS') / mfma:.2f} |")
        vals[name] = (busy, clock)
    lines = ["# MFMA utilisation of the prefill kernel: 8 x 8,192 bf16 prefill (sliding W 2048, full NoPE)", "",
             "Two counter runs (from /tmp, repository at $ROOT):", "", "```", command, "```", "",
             "GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the clock is GRBM_GUI_ACTIVE / 8 over the "
             "dispatch time; SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES are summed over the "
             "1,024 SIMDs and divided by 1,024 times the per-XCD cycles.  Executed flops count every "
             "`v_mfma_f32_32x32x16` (32,768 flop), masked tiles included.", "",
             "| layer | ms per launch | clock GHz | MFMA busy % | VALU+MFMA co-issue % | algorithmic TFLOP/s "
             "| executed / algorithmic flop | VALU instr per MFMA | LDS instr per MFMA |",
             "|---|---|---|---|---|---|---|---|---|", *rows, "",
             "Values read by bench.py (reported only while these sources are unchanged):", "",
             f"    prefill_sources_sha256_16: {sources_hash(PREFILL_SOURCES)}",
             f"    mfma_busy_sliding: {vals['sliding'][0]:.4f}",
             f"    mfma_busy_full: {vals['full'][0]:.4f}",
             f"    clock_ghz_sliding: {vals['sliding'][1]:.3f}",
             f"    clock_ghz_full: {vals['full'][1]:.3f}", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")



def summarize_legs(trace_csv: str, fetch_csv: str, write_csv: str, out: str, command: str):
    """Per-kernel summary of `bench.py --only-next ...` (verify, o_proj,
    relocate legs): average duration from the kernel trace, and FETCH_SIZE /
    WRITE_SIZE (medians over the dispatches, scaled by the 1 GiB copy of
    `--calibrate-copy`) from two counter runs.  Verify launches of the sliding
    and the full layer share a grid; they are told apart by duration (the
    full layer's calls take about three times longer)."""
    import csv
    import statistics

    def rows_of(path, value):
        out = []
        for r in csv.DictReader(open(path)):
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            out.append((int(r["Start_Timestamp"]), r["Kernel_Name"], int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0),
                        dur, value(r)))
        return [x[1:] for x in sorted(out)]                # dispatch order

    def keys(lst, cut):
        # a verify merge belongs to the layer of the verify launch before it
        out, last = [], ""
        for n, g, d, v in lst:
            short = n.split("(")[0].replace("void ", "")
            if "verify_kernel" in short and cut is not None:
                last = ", full layer" if d > cut else ", sliding layer"
                out.append(short + last)
            elif "verify_merge" in short:
                out.append(short + last)
            elif short.startswith("Cijk"):                  # hipBLASLt's GEMM kernels
                out.append("hipBLASLt GEMM (o_proj): " + short[:48])
            else:
                out.append(short)
        return out

    trace = rows_of(trace_csv, lambda r: 0.0)
    fetch = rows_of(fetch_csv, lambda r: float(r["Counter_Value"]))
    write = rows_of(write_csv, lambda r: float(r["Counter_Value"]))
    vd = sorted(d for n, g, d, v in trace if "verify_kernel" in n)
    cut = (vd[0] + vd[-1]) / 2 if vd else None
    copy_f = [v for n, g, d, v in fetch if "copyBuffer" in n]
    copy_w = [v for n, g, d, v in write if "copyBuffer" in n]
    fs = FETCH_SCALE if not copy_f else round((1 << 30) / (copy_f[0] * 1024), 2)
    ws = WRITE_SCALE if not copy_w else round((1 << 30) / (copy_w[0] * 1024), 2)
    groups = {}
    ours = lambda n: "muse::" in n or n.startswith("Cijk")
    for (n, g, d, v), k in zip(trace, keys(trace, cut)):
        if ours(n):
            groups.setdefault(k, {"dur": [], "f": [], "w": []})["dur"].append(d)
    for lst, tag in ((fetch, "f"), (write, "w")):
        fd = sorted(d for n, g, d, v in lst if "verify_kernel" in n)
        fcut = (fd[0] + fd[-1]) / 2 if fd else None
        for (n, g, d, v), k in zip(lst, keys(lst, fcut)):
            if ours(n) and k in groups:
                groups[k][tag].append(v)
    lines = ["# Kernel trace and HBM traffic of the verify, o_proj and relocate legs", "",
             "Commands (from /tmp, repository at $ROOT): the trace, then the two counter runs:", "", "```",
             command, "```", "",
             f"FETCH_SIZE is scaled by {fs} and WRITE_SIZE by {ws} (a 1 GiB device copy, `--calibrate-copy`, "
             f"read {copy_f[0] if copy_f else 0:.1f} KiB and wrote {copy_w[0] if copy_w else 0:.1f} KiB on them). "
             "FETCH_SIZE counts what the L2s fetch from memory, Infinity Cache hits included.  Counter values "
             "are medians over the dispatches.", "",
             "Algorithmic bytes per launch: verify reads every visible cache row once (64 x 8,208 x 1,024 B = "
             "537.9 MB full; 64 x 2,063 x 1,024 B = 135.2 MB sliding) and writes 35.7 MB of f32 partials (2 splits); "
             "relocate moves up to 120 tiles of 512 rows per launch (62.9 MB of K and V read, the same written); "
             "o_proj: W (54.5 MB) and the attention rows once, f32 projection written.", "",
             "| kernel | dispatches | avg us | min us | read MB | write MB |", "|---|---|---|---|---|---|"]
    for k in sorted(groups):
        gd = groups[k]
        fmb = statistics.median(gd["f"]) * 1024 * fs / 1e6 if gd["f"] else float("nan")
        wmb = statistics.median(gd["w"]) * 1024 * ws / 1e6 if gd["w"] else float("nan")
        lines.append(f"| `{k}` | {len(gd['dur'])} | {sum(gd['dur']) / len(gd['dur']):.2f} | {min(gd['dur']):.2f} | "
                     f"{fmb:.2f} | {wmb:.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_trace(trace_csv: str, out: str, command: str):
    """Write a kernel-trace summary (text) from rocprofv3's kernel_trace.csv of
    a default run: the schedule phase (every dispatch before the first f32
    kernel, which starts the other workloads' legs), its decode and
    prefill kernels by layer kind (the calls run in layer order, layer l full
    iff l % 4 == 3), then the legs by kernel."""
    import csv
    import re
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))

    def short(name):
        m = re.match(r"_ZN4muse(\d+)", name)
        if m:
            n = int(m.group(1))
            kname = name[m.end():m.end() + n]
            return f"muse::{kname}<{'bf16' if 'DF16b' in name[m.end() + n:] else 'f32'}>"
        return name.split("(")[0].replace("void ", "")

    import collections
    legs_at = next((i for i, r in enumerate(rows) if "muse" in r["Kernel_Name"] and short(r["Kernel_Name"]).endswith(
        ("<f32>", "<float>(muse::AttnArgs)", "<float>(muse::PrepArgs)")) or "<float>" in r["Kernel_Name"]), len(rows))
    # in the schedule phase the split kernel's grid tells the layer kind (the
    # 39 sliding layers' grid is the more frequent one), a merge kernel takes
    # the kind of the split before it, and prefill calls run in layer order
    grids = collections.Counter(r["Grid_Size_X"] if "Grid_Size_X" in r else r["Grid_Size"]
                                for r in rows[:legs_at] if "decode_kernel" in r["Kernel_Name"])
    sliding_grid = grids.most_common(1)[0][0] if grids else None
    groups = {}
    counters = {}
    last_kind = "sliding"
    for i, r in enumerate(rows):
        name = r["Kernel_Name"]
        if "muse" not in name:
            continue
        k = short(name)
        phase = "schedule" if i < legs_at else "legs"
        if phase == "schedule":
            kind = None
            if "decode_merge_kernel" in k:
                kind = last_kind
            elif "decode_kernel" in k:
                kind = "sliding" if (r.get("Grid_Size_X") or r.get("Grid_Size")) == sliding_grid else "full"
                last_kind = kind
            elif "prefill_group_kernel" in k or "prep_kernel" in k:
                c = counters.get(k, 0)
                counters[k] = c + 1
                kind = "full" if c % 52 % 4 == 3 else "sliding"
            if kind:
                k = f"{k}, {kind} layers"
        groups.setdefault((phase, k), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel trace summary", "", "Command (from /tmp, repository at $ROOT):", "", "```", command, "```", "",
             "Per kernel: the 52-layer schedule phase of the run (chunked prefill, eager and graph-replayed decode "
             "steps), with layer kinds, then the other workloads' legs.", "",
             "| phase | kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for (phase, k), v in sorted(groups.items(), key=lambda x: (x[0][0] != "schedule", -sum(x[1]))):
        lines.append(f"| {phase} | {k} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    lines += ["", "One decode call of the schedule (split kernel + merge kernel, the unit of the bench line's "
              "roofline), from the averages above:", ""]
    for kind in ("sliding", "full"):
        a = groups.get(("schedule", f"muse::decode_kernel<bf16>, {kind} layers"))
        b = groups.get(("schedule", f"muse::decode_merge_kernel<bf16>, {kind} layers"))
        if a and b:
            lines.append(f"    decode_call_us_{kind}: {sum(a) / len(a) + sum(b) / len(b):.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


TL_PHASES = ["seq_len read", "raw Q rows arrived", "Q-hat shared (barrier)", "sub-tiles done",
             "partials merged in LDS", "stores complete"]


def timeline_summary(split, merge):
    """Phase times of one decode call from the profiling build's records
    (10 ns units): per split workgroup, the medians (p10, p90) of each phase's
    duration after the previous one; the call's critical path from the first
    split workgroup's start to the last merge workgroup's end."""
    import numpy as np
    d = split[split[:, 6] > 0]
    m = merge[merge[:, 2] > 0]
    k0 = int(d[:, 0].min())
    ph = np.diff(d[:, :7], axis=1) / 100.0
    res = {"split_workgroups": int(len(d)), "sub_tiles_per_wave_p50": float(np.median(d[:, 7])),
           "start_spread_us": round(float(d[:, 0].max() - k0) / 100.0, 2),
           "phases_us": {n: [round(float(np.percentile(ph[:, i], q)), 2) for q in (50, 10, 90)]
                         for i, n in enumerate(TL_PHASES)},
           "workgroup_total_us_p50": round(float(np.median(d[:, 6] - d[:, 0])) / 100.0, 2),
           "last_split_end_us": round(float(d[:, 6].max() - k0) / 100.0, 2)}
    if len(m):
        res["merge"] = {"workgroups": int(len(m)),
                        "first_start_after_last_split_us": round(float(m[:, 0].min() - d[:, 6].max()) / 100.0, 2),
                        "loads_arrived_us_p50": round(float(np.median(m[:, 1] - m[:, 0])) / 100.0, 2),
                        "stores_complete_us_p50": round(float(np.median(m[:, 2] - m[:, 1])) / 100.0, 2),
                        "last_end_us": round(float(m[:, 2].max() - k0) / 100.0, 2)}
    return res


def decode_timeline(fa, synth, torch, out_path=None, command=""):
    """Per-phase decode timelines from the profiling build
    (libmuse_attn_timeline.so): the 52-layer schedule's sliding and full
    layers (a graph of that kind's calls, as the roofline times them) and the
    64 x 8,192 and 16 x 131,072 decode layers (a graph of one call per cache
    copy, as their legs time them); the records are those of the graph's last
    call.  Prints one JSON object; writes a markdown summary to out_path."""
    from full_gqa_attention_amd.schedule import Schedule
    fa.use_timeline_library()

    def capture(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        return g

    def run(g, n_calls):
        g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) for a, b in ev)[2] * 1e3 / n_calls
        fa.decode_timeline_read(clear=True)
        g.replay()
        split, merge = fa.decode_timeline_read(clear=True)
        return round(us, 2), timeline_summary(split, merge)

    cases = {}
    w = synth.WORKLOADS[HEADLINE]
    sch = Schedule(w)
    sch.prefill()
    sch.start_decode()
    kinds = [_kind(s, synth) for s in sch.specs]
    for kind in ("sliding", "full"):
        idx = [l for l in range(len(sch.specs)) if kinds[l] == kind]
        g = capture([(lambda l=l: sch.decode_layer(l)) for l in idx])
        us, tl = run(g, len(idx))
        cases[f"{w.name} {kind}"] = dict(graph=f"{len(idx)} calls ({kind} layers), records of the last",
                                         us_per_call=us, **tl)
        del g
    del sch
    torch.cuda.empty_cache()
    for name in ("decode_64x8192_bf16", "decode_16x131072_bf16"):
        wl = synth.WORKLOADS[name]
        for spec in wl.layers:
            per = kv_row_bytes(wl.dtype) * wl.n_seq * visible_rows(spec, wl.prefix)
            copies = min(8, max(1, -(-(2 * MALL_BYTES) // max(per, 1)) + 1))
            r = LayerRun(wl, spec, copies, True, fa, synth)
            g = capture([(lambda c=c: r.call(fa, c)) for c in range(copies)])
            us, tl = run(g, copies)
            cases[f"{name} {_kind(spec, synth)}"] = dict(graph=f"{copies} calls (one per cache copy), records of the last",
                                                          us_per_call=us, **tl)
            del g, r
            torch.cuda.empty_cache()
    print(json.dumps({"decode_timeline": cases}), flush=True)
    if out_path:
        lines = ["# Decode phase timeline (profiling build): 52-layer schedule, 64 x 8,192 and 16 x 131,072 decode", "",
                 "Command (repository root, one MI355X):", "", "```", command, "```", "",
                 "The profiling build (`libmuse_attn_timeline.so`, `include/muse_attn_timeline.h`) is the regular "
                 "library with per-workgroup stamps (`s_memrealtime`, 10 ns) in the decode split and merge kernels. "
                 "Each phase is the median time (p10, p90) a split workgroup spends after the previous one; "
                 "the stores phase waits for the workgroup's stores to complete. "
                 "`us per call` is the graph-replayed call of the profiling build (split + merge).", ""]
        for cname, c in cases.items():
            lines += [f"## {cname}", "", f"{c['graph']}; {c['us_per_call']} us per call; {c['split_workgroups']} split "
                      f"workgroups, {c['sub_tiles_per_wave_p50']:.0f} sub-tiles per wave (median), starts spread over "
                      f"{c['start_spread_us']} us", "", "| split phase | us p50 | p10 | p90 |", "|---|---|---|---|"]
            for n, (a, lo, hi) in c["phases_us"].items():
                lines.append(f"| {n} | {a} | {lo} | {hi} |")
            lines += ["", f"Split workgroup total (p50) {c['workgroup_total_us_p50']} us; last split workgroup done at "
                      f"{c['last_split_end_us']} us after the first started."]
            if "merge" in c:
                mg = c["merge"]
                lines.append(f"Merge: {mg['workgroups']} workgroups, the first starting {mg['first_start_after_last_split_us']} us "
                             f"after the last split ended; loads in after {mg['loads_arrived_us_p50']} us, output stores "
                             f"complete {mg['stores_complete_us_p50']} us later (p50); last merge workgroup done at "
                             f"{mg['last_end_us']} us.")
            lines.append("")
        with open(out_path, "w") as f:
            f.write("\n".join(lines))
    return cases


def decode_leg_only(fa, synth, torch, name, kind, reps=20):
    """One layer kind of a decode workload, replayed from a HIP graph of one
    call per cache copy (as its leg times it), for a kernel trace of that
    layer alone.  Prints one JSON object with the per-call time between events."""
    wl = synth.WORKLOADS[name]
    spec = next(s for s in wl.layers if _kind(s, synth) == kind)
    per = kv_row_bytes(wl.dtype) * wl.n_seq * visible_rows(spec, wl.prefix)
    copies = min(8, max(1, -(-(2 * MALL_BYTES) // max(per, 1)) + 1))
    r = LayerRun(wl, spec, copies, True, fa, synth)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in range(copies):
            r.call(fa, c)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * copies)
    print(json.dumps({"decode_leg": name, "kind": kind, "calls": (reps + 3) * copies, "cache_copies": copies,
                      "us_per_call": round(us, 2), "kv_bytes_per_call": per,
                      "GBps": round(per / us / 1e3, 1)}), flush=True)


def summarize_leg_traces(out: str, command: str, *pairs):
    """Write per-layer decode summaries from kernel traces of `--decode-leg`
    runs: pairs of (label, kernel_trace.csv)."""
    import csv
    lines = ["# Decode legs, one layer kind per run: kernel trace", "", "Commands (from /tmp, repository at $ROOT), one per row:",
             "", "```", command, "```", "",
             "Each run replays one layer kind of the workload from a HIP graph (one call per cache copy, enough "
             "copies that the 256 MB Infinity Cache cannot serve a call from the previous one), 3 warm-up "
             "and 20 timed replays; every traced call is averaged.", "",
             "| workload, layer | split kernel avg us (min, max) | merge kernel avg us | call (sum) us | KV GB/s per call |",
             "|---|---|---|---|---|"]
    for i in range(0, len(pairs), 2):
        label, path = pairs[i], pairs[i + 1]
        rows = list(csv.DictReader(open(path)))
        sp = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
              if "decode_kernel" in r["Kernel_Name"] and "merge" not in r["Kernel_Name"]]
        mg = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
              if "decode_merge_kernel" in r["Kernel_Name"]]
        name, kind = label.split(":")
        wl_bytes = {"decode_64x8192_bf16": {"full": 64 * 8193 * 1024, "sliding": 64 * 2048 * 1024},
                    "decode_16x131072_bf16": {"full": 16 * 131073 * 1024, "sliding": 16 * 2048 * 1024}}[name][kind]
        a = sum(sp) / len(sp)
        m = sum(mg) / len(mg) if mg else 0.0
        lines.append(f"| {name}, {kind} | {a:.2f} ({min(sp):.2f}, {max(sp):.2f}) | {m:.2f} | {a + m:.2f} | "
                     f"{wl_bytes / (a + m) / 1e3:.0f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def bench_verify(fa, synth, torch, steps=20, warmup=3, n_new=16):
    """Multi-token verify: 16 drafted tokens per sequence scored against the
    64 x 8,192 cached rows (the drafting-and-verifying section of "How Muse
    Glimmer Fits an Agent on Your Device"), one sliding and one full layer,
    through muse_attn_prefill (which takes the verify kernels for such short
    bf16 chunks).  The roofline is HBM: the call reads every visible cache row
    once (1,024 B per row per sequence) and does 16,384 flop per visible
    (query, key) pair, 256 flop per byte at 16 tokens, under the 312 flop/B
    ridge of 2.5 PFLOP/s over 8 TB/s.  Kernel time = the split kernel and the
    merge kernel, between the library's events; call = prep (append) too."""
    import dataclasses
    base = synth.WORKLOADS["decode_64x8192_bf16"]
    w = dataclasses.replace(base, name="verify_64x8192p16_bf16", n_new=n_new)
    runs = [LayerRun(w, spec, 2, False, fa, synth) for spec in w.layers]
    torch.cuda.synchronize()
    wall, per_launch = run_timed(runs, steps, warmup, 2, fa, torch)
    per_layer, total_bytes, total_kern = {}, 0, 0.0
    for j, r in enumerate(runs):
        lt = per_launch[j::len(runs)]
        avg = sum(lt) / len(lt)
        rows = sum(visible_rows(r.spec, w.prefix + t) for t in range(n_new)) // n_new   # per token, ~window or L
        kv = w.n_seq * (min(w.prefix + n_new, r.spec.window + n_new - 1) if r.spec.window else w.prefix + n_new) * 1024
        flop = FLOP_PER_PAIR * w.n_seq * prefill_pairs(r.spec, w.prefix, n_new)
        per_layer[r.spec.name] = {"kernel_us": round(avg * 1e3, 2), "kv_MB": round(kv / 1e6, 3),
                                  "kernel_GBps": round(kv / (avg * 1e-3) / 1e9, 1),
                                  "kernel_TFLOPs": round(flop / (avg * 1e-3) / 1e12, 1),
                                  "visible_rows_per_token": rows,
                                  "p10_p50_p90_us": [round(x * 1e3, 2) for x in percentiles(lt)]}
        total_bytes += kv
        total_kern += avg
    achieved = total_bytes / (total_kern * 1e-3) / 1e9
    return {"workload": w.name, "n_seq": w.n_seq, "cached_tokens": w.prefix, "new_tokens": n_new,
            "call_us_per_layer": round(wall / steps / len(runs) * 1e6, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "muse::verify_kernel + muse::verify_merge_kernel (bf16)",
                         "per_layer": per_layer},
            "steps": steps, "warmup": warmup}



def bench_out_proj(fa, synth, torch, steps=10, warmup=3):
    """The block's tail after attention (muse_out_proj: o_proj 4096 -> 6656,
    post-attention RMSNorm eps 1e-8, residual add; "Chapter 9 - The Muse
    Glimmer architecture" 9.8, 9.9) on seeded synthetic weights, at the token
    counts of the two headline workloads: 65,536 (the 8 x 8,192 prefill
    batch; the GEMM is MFMA-bound, 2 * 4096 * 6656 flop per token) and 64
    (one decode step of 64 sequences; reading W's 54.5 MB bounds it).  The
    kernel timer brackets the GEMM; the call adds the norm pass."""
    from full_gqa_attention_amd.timing import KernelTimers
    res = {}
    for M in (65536, 64):
        inp = synth.out_proj_inputs(M, config=80, device="cuda", backend="torch")
        ws = torch.empty(max(fa.out_proj_workspace_size(M), 16), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(inp.residual)
        for _ in range(warmup):
            fa.out_proj(inp.attn, inp.w, inp.gamma, inp.residual, out=out, workspace=ws)
        torch.cuda.synchronize()
        timers = KernelTimers(steps)
        t0 = time.perf_counter()
        for i in range(steps):
            fa.out_proj(inp.attn, inp.w, inp.gamma, inp.residual, out=out, workspace=ws, timer=timers[i])
        torch.cuda.synchronize()
        call = (time.perf_counter() - t0) / steps
        g = [timers.elapsed_ms(i) for i in range(steps)]
        timers.close()
        gemm = sorted(g)[len(g) // 2] * 1e-3
        flop = 2.0 * M * 4096 * 6656
        wbytes = 6656 * 4096 * 2 + M * 4096 * 2              # W and attn, read once
        r = {"tokens": M, "call_us": round(call * 1e6, 1), "gemm_us": round(gemm * 1e6, 1),
             "gemm_TFLOPs": round(flop / gemm / 1e12, 1), "gemm_GBps_W_and_attn": round(wbytes / gemm / 1e9, 1)}
        if M >= 4096:
            r["roofline"] = {"bound": "mfma", "achieved": r["gemm_TFLOPs"], "peak": MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(r["gemm_TFLOPs"] / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                             "kernel": "hipBLASLt GEMM (bf16 x bf16 -> f32, the heuristic's pick among "
                                       "algorithms that need no workspace)"}
        else:
            r["roofline"] = {"bound": "hbm", "achieved": r["gemm_GBps_W_and_attn"], "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(r["gemm_GBps_W_and_attn"] / HBM_PEAK_GBS, 4),
                             "traffic": None,
                             "kernel": f"muse::out_proj_skinny_kernel<{(M + 15) // 16}> (bf16)"}
        res[f"tokens_{M}"] = r
        del inp, ws, out
        torch.cuda.empty_cache()
    return res



def bench_relocate(fa, synth, torch, steps=10):
    """NoPE tile relocation ("Chapter 14 - QK-norm and RoPE" 14.6): the whole
    cache of a full layer of the 64 x 8,192 decode workload, moved as 512-row
    tiles from one cache to another (K and V; 1,024 tiles per pass)."""
    S, L, T = 64, 8192, 512
    spec = synth.full()
    lay = fa.make_layer(spec.kind, dtype=synth.BF16)
    g = torch.Generator(device="cuda").manual_seed(5)
    a_k = torch.randn((S, L, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    a_v = torch.randn((S, L, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    b_k, b_v = torch.empty_like(a_k), torch.empty_like(a_v)
    # each sequence's tiles land reversed in another sequence, so no tile is a plain block copy of the whole cache
    tiles = fa.kv_tiles([(s, i * T, (s + 1) % S, (L // T - 1 - i) * T, T) for s in range(S) for i in range(L // T)])
    fa.kv_relocate(lay, a_k, a_v, b_k, b_v, tiles)
    torch.cuda.synchronize()
    # The host checks the tile list and splits it into launches on every call
    # (timed here on its own).  The GPU time of a pass comes from a HIP graph
    # of one call: the tile descriptors travel as kernel arguments, so the
    # replays run the copy kernels only.
    host = 0.0
    for _ in range(steps):
        t0 = time.perf_counter()
        fa.kv_relocate(lay, a_k, a_v, b_k, b_v, tiles)
        host += time.perf_counter() - t0
        torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.kv_relocate(lay, a_k, a_v, b_k, b_v, tiles)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_ms = []
    for _ in range(steps):
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        gpu_ms.append(e0.elapsed_time(e1))
    dt = sorted(gpu_ms)[len(gpu_ms) // 2] * 1e-3
    moved = 2 * a_k.numel() * a_k.element_size()           # K and V bytes per pass
    ok = bool(torch.equal(b_k[1, (L // T - 1) * T:], a_k[0, :T]))
    del graph
    return {"tiles": tiles[1], "tile_rows": T, "MB_moved": round(moved / 1e6, 1),
            "gpu_ms": round(dt * 1e3, 3), "gpu_ms_measured": "one pass replayed from a HIP graph, between events",
            "host_ms_per_call": round(host / steps * 1e3, 3),
            "GBps_read_plus_write": round(2 * moved / dt / 1e9, 1),
            "frac_hbm_peak": round(2 * moved / dt / 1e9 / HBM_PEAK_GBS, 4), "bytes_checked": ok}


def main():
    args = parse()
    if args.summarize_legs:
        summarize_legs(*args.summarize_legs)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_leg_traces:
        summarize_leg_traces(*args.summarize_leg_traces)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path to measure.", file=sys.stderr)
        sys.exit(2)
    import torch
    import full_gqa_attention_amd as fa
    from full_gqa_attention_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.decode_leg:
        fa.lib()
        decode_leg_only(fa, synth, torch, *args.decode_leg)
        return
    if args.decode_timeline is not None:
        decode_timeline(fa, synth, torch, out_path=args.decode_timeline or None,
                        command="python bench.py --decode-timeline " + (args.decode_timeline or ""))
        return
    fa.lib()                                  # fails loudly when the HIP library is missing
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.prefill_only:
        pw = synth.WORKLOADS["prefill_8x8192_bf16"]
        print(json.dumps({"prefill": leg_prefill(pw, fa, synth, torch, steps=5, cpu=False)}), flush=True)
        return
    if args.only_next:
        extra = {}
        if args.verify:
            extra["verify"] = bench_verify(fa, synth, torch)
            torch.cuda.empty_cache()
        if args.out_proj:
            extra["out_proj"] = bench_out_proj(fa, synth, torch)
            torch.cuda.empty_cache()
        if args.relocate:
            extra["relocate"] = bench_relocate(fa, synth, torch)
        print(json.dumps(extra), flush=True)
        return
    if args.counters_run:
        from full_gqa_attention_amd.schedule import Schedule
        sch = Schedule(synth.WORKLOADS[HEADLINE], ring=args.ring)
        sch.prefill()
        sch.start_decode()
        for _ in range(2):
            sch.decode_step()
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": HEADLINE, "decode_steps": 2}), flush=True)
        return

    res, sch = bench_schedule(args, fa, synth, torch)
    K = res["steps"]
    line = {
        "metric": METRIC, "value": round(res["value"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) inputs and cache prefixes, resident in HBM",
        "config": res["config"], "roofline": res["roofline"],
        "frac_hbm_peak": round(res["value"] / HBM_PEAK_GBS, 4),
        "launch": "each decode step (52 layers' decode calls, then the seq_len increment) replayed from a HIP graph",
        "prefill": res["prefill"],
    }
    if not args.no_cpu_baseline and not args.ring:
        import oracle
        log("timing the CPU oracle on a sample of the schedule")
        cs = cpu_schedule_sample(sch, fa, synth, torch)
        w = sch.w
        total_pairs = sum(w.n_seq * prefill_pairs(s, w.prefix, w.n_new) for s in sch.specs)
        total_kv = sum(kv_row_bytes(w.dtype) * w.n_seq * visible_rows(s, w.prefix + w.n_new + i)
                       for i in range(w.decode_steps) for s in sch.specs)
        line["cpu_baseline"] = {
            "value": round(cs["decode_kv"] / cs["decode_s"] / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "decode: the first 4 decode steps of all 52 layers, 4 sequences, all 32 heads "
                      f"({cs['decode_kv'] / 1e9:.2f} GB of KV rows, {cs['decode_s']:.2f} s); prefill: 2 chunk rows "
                      f"per layer ({cs['prefill_pairs']} visible pairs, {cs['prefill_s']:.2f} s)",
            "seconds": round(cs["decode_s"] + cs["prefill_s"], 3),
            "prefill_tflops": round(cs["prefill_pairs"] * FLOP_PER_PAIR / max(cs["prefill_s"], 1e-9) / 1e12, 6),
            "extrapolated_full_run_s": {
                "chunked_prefill": round(cs["prefill_s"] * total_pairs / max(cs["prefill_pairs"], 1), 1),
                "decode_256_steps": round(cs["decode_s"] * total_kv / cs["decode_kv"], 1),
                "note": "extrapolation: sample time x the workload's visible pairs (or KV bytes) / the sample's"}}
        line["parity"] = cs["parity"]
    del sch
    torch.cuda.empty_cache()
    if not args.no_configs:
        cpu = not args.no_cpu_baseline
        legs = {}
        import numpy as np
        w1 = synth.WORKLOADS["prefill_1x512_f32"]
        legs[w1.name] = leg_prefill(w1, fa, synth, torch, steps=20, cpu=cpu, single_core=True)
        legs["decode_64x8192_bf16"] = leg_decode(synth.WORKLOADS["decode_64x8192_bf16"], fa, synth, torch, cpu=cpu)
        w3 = synth.WORKLOADS["prefill_8x8192_bf16"]
        edges = sorted({0, 1, 63, 64, 127, 128, 2046, 2047, 2048, 2049, 4095, 8191})
        rows3 = np.array([(s, t) for s in (0, 7) for t in edges], np.int32)
        legs[w3.name] = leg_prefill(w3, fa, synth, torch, steps=5, cpu=cpu, cpu_rows=rows3)
        legs["decode_16x131072_bf16"] = leg_decode(synth.WORKLOADS["decode_16x131072_bf16"], fa, synth, torch,
                                                   steps=10, cpu=cpu)
        line["configs"] = legs
    if args.verify:
        torch.cuda.empty_cache()
        line["verify"] = bench_verify(fa, synth, torch)
    if args.out_proj:
        torch.cuda.empty_cache()
        line["out_proj"] = bench_out_proj(fa, synth, torch)
    if args.relocate:
        torch.cuda.empty_cache()
        line["relocate"] = bench_relocate(fa, synth, torch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

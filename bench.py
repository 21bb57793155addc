#!/usr/bin/env python3
"""Benchmark of the Muse Glimmer attention core on one MI355X.

Default workload (one "step"): a decode step of 64 sequences x 8,192 cached
tokens, bf16, on one sliding layer (RoPE, window 2,048) and one full NoPE
layer -- QK-norm, RoPE, KV append, split-K attention and the gate, for both
layers.  `value` is decode attention KV bytes per second over the whole step
(the visible K/V rows, 1,024 B per row per sequence).  The 8 x 8,192 bf16
prefill (both layer kinds) is timed in the same run and reported under
"prefill" in TFLOP/s (16,384 flop per visible (query, key) pair over 32
heads), so the line carries both halves of the metric.

Inputs are seeded synthetic tensors already resident in HBM.  Decode caches
are rotated over enough copies that every step reads bytes the 256 MB
Infinity Cache cannot still hold.  `roofline` uses the attention kernel's own
launch time from HIP events recorded by the library around that kernel.
`cpu_baseline` times the CPU oracle on the same step's inputs (rank 0, N=1).
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
FLOP_PER_PAIR = 32 * 4 * 128     # 32 heads x (2*128 for Q.K + 2*128 for P.V)
MALL_BYTES = 256 << 20


def kv_row_bytes(dtype: int) -> int:
    return 2 * 2 * 128 * (2 if dtype == 1 else 4)   # K and V, 2 kv heads x 128


def visible_rows(spec, p: int) -> int:
    return p + 1 if spec.window == 0 else min(spec.window, p + 1)


def prefill_pairs(spec, L: int, N: int) -> int:
    return sum(visible_rows(spec, L + t) for t in range(N))


PROFILES = os.path.join(ROOT, "profiles")
COUNTERS_FILE = os.path.join(PROFILES, "decode_64x8192_bf16_hbm_counters.md")
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


def counter_traffic():
    """HBM bytes per decode-kernel launch from the committed counter summary,
    or None when the decode kernel's sources changed since it was taken."""
    try:
        kv = {}
        with open(COUNTERS_FILE) as f:
            for line in f:
                if line.startswith("    ") and ":" in line:
                    k, v = line.strip().split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("decode_sources_sha256_16") != sources_hash(DECODE_SOURCES):
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


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


def summarize_trace(stats_csv: str, out: str, command: str):
    """Write a kernel-trace summary (text) from rocprofv3's kernel_stats.csv."""
    import csv
    rows = [r for r in csv.DictReader(open(stats_csv)) if "muse" in r["Name"]]
    lines = ["# Kernel trace summary", "", "Command (from /tmp, repository at $ROOT):", "", "```",
             command, "```", "", "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    import re
    for r in rows:
        name = r["Name"]
        m = re.match(r"_ZN4muse(\d+)", name)
        if m:
            n = int(m.group(1))
            kname = name[m.end():m.end() + n]
            dt = "bf16" if "DF16b" in name[m.end() + n:] else "f32"
            name = f"muse::{kname}<{dt}>"
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_counters(fetch_csv: str, write_csv: str, out: str, command: str):
    """Write the decode kernel's HBM-traffic summary from two --pmc runs."""
    import csv

    def per_kernel(path):
        copy, dec = [], []
        for r in csv.DictReader(open(path)):
            v = float(r["Counter_Value"])
            if "decode_kernel" in r["Kernel_Name"]:
                dec.append(v)
            elif "copyBuffer" in r["Kernel_Name"]:
                copy.append(v)
        return copy, dec

    fc, fd = per_kernel(fetch_csv)
    wc, wd = per_kernel(write_csv)
    # launches alternate sliding, full (the benchmark's layer order)
    f_sl, f_fu = sum(fd[0::2]) / len(fd[0::2]), sum(fd[1::2]) / len(fd[1::2])
    w_sl, w_fu = sum(wd[0::2]) / len(wd[0::2]), sum(wd[1::2]) / len(wd[1::2])
    fetch_b = [x * 1024 * FETCH_SCALE for x in (f_sl, f_fu)]
    write_b = [x * 1024 * WRITE_SCALE for x in (w_sl, w_fu)]
    per_launch = (sum(fetch_b) + sum(write_b)) / 2
    lines = ["# HBM traffic of the decode kernel: 64 x 8,192 bf16 decode step", "",
             "Two counter runs (from /tmp, repository at $ROOT):", "", "```", command, "```", "",
             f"Calibration: the first copy in each run is a 1 GiB device copy (`--calibrate-copy`); it read "
             f"{fc[0]:.1f} KiB on FETCH_SIZE and {wc[0]:.1f} KiB on WRITE_SIZE, so FETCH_SIZE is scaled by "
             f"{FETCH_SCALE} and WRITE_SIZE by {WRITE_SCALE}.", "",
             "| launch | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB | algorithmic KV MB |",
             "|---|---|---|---|---|---|",
             f"| sliding (W 2048) | {f_sl:.1f} | {w_sl:.1f} | {fetch_b[0] / 1e6:.1f} | {write_b[0] / 1e6:.2f} | 134.2 |",
             f"| full | {f_fu:.1f} | {w_fu:.1f} | {fetch_b[1] / 1e6:.1f} | {write_b[1] / 1e6:.2f} | 536.9 |",
             "", "Values read by bench.py (traffic is reported only while these sources are unchanged):", "",
             f"    decode_sources_sha256_16: {sources_hash(DECODE_SOURCES)}",
             f"    hbm_bytes_per_launch: {per_launch:.0f}", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_64x8192_bf16")
    ap.add_argument("--prefill-workload", default="prefill_8x8192_bf16")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--schedule", action="store_true",
                    help="also time the 52-layer schedule workload (chunked prefill phase + 256 decode steps)")
    ap.add_argument("--ring", action="store_true",
                    help="sliding layers keep their window in a ring cache (kv_ring) in the decode and schedule runs")
    ap.add_argument("--verify", action="store_true",
                    help="also time the 16-token verify call (64 x 8,192 cached rows, both layers)")
    ap.add_argument("--out-proj", action="store_true",
                    help="also time the block's tail (o_proj + post-attention norm) at 65,536 and 64 tokens")
    ap.add_argument("--relocate", action="store_true",
                    help="also time NoPE tile relocation (muse_kv_relocate) of a 64 x 8,192 full-layer cache")
    ap.add_argument("--eager", action="store_true",
                    help="time decode steps as eager calls only (no HIP graph), e.g. under counter collection")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy first (scale for HBM byte counters)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "OUT", "COMMAND"),
                    help="write a kernel-trace summary from rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "OUT", "COMMAND"),
                    help="write the decode kernel's HBM-traffic summary from two --pmc runs and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill workload and print its JSON object (for counter runs)")
    ap.add_argument("--summarize-mfma", nargs=4, metavar=("PMC1_CSV", "PMC2_CSV", "OUT", "COMMAND"),
                    help="write the prefill kernel's MFMA-utilisation summary from two --pmc runs and exit")
    return ap.parse_args()


def percentiles(xs):
    """p10, p50, p90 (nearest rank) of a list of launch times."""
    v = sorted(xs)
    return [v[min(len(v) - 1, int(q * len(v)))] for q in (0.1, 0.5, 0.9)]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ring_of(cache, L: int, cap: int):
    """A ring of `cap` rows holding positions [L - cap, L) of every sequence
    at row p % cap (the same stored rows as the linear cache)."""
    import torch
    ring = torch.empty((cache.shape[0], cap) + tuple(cache.shape[2:]), dtype=cache.dtype, device=cache.device)
    pos = torch.arange(max(0, L - cap), L, device=cache.device)
    ring[:, pos % cap] = cache[:, pos]
    if L < cap:
        ring[:, L:] = 0
    return ring


def uses_ring(spec, ring: bool, synth) -> bool:
    return ring and spec.kind == synth.SLIDING_ROPE


class LayerRun:
    def __init__(self, w, spec, copies, decode, fa, synth, ring=False):
        import torch
        self.spec = spec
        self.inp = synth.layer_inputs(w, spec, device="cuda", backend="torch")
        self.ring = uses_ring(spec, ring, synth) and decode
        if self.ring:                                 # the window's rows only, as a ring
            self.inp.cache_k = ring_of(self.inp.cache_k, w.prefix, spec.window)
            self.inp.cache_v = ring_of(self.inp.cache_v, w.prefix, spec.window)
        self.caches = [(self.inp.cache_k, self.inp.cache_v)]
        for _ in range(1, copies):
            self.caches.append((self.inp.cache_k.clone(), self.inp.cache_v.clone()))
        self.layer = fa.make_layer(spec.kind, window=spec.window, rope_theta=spec.rope_theta,
                                   rms_eps=spec.rms_eps, q_norm_gain=spec.q_gain,
                                   k_norm_gain=spec.k_gain, attn_scale=spec.scale, dtype=w.dtype,
                                   kv_ring=1 if self.ring else 0)
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
    """W untimed steps, then K timed steps between synchronisations."""
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
    """The same steps replayed from HIP graphs (one captured step per cache
    copy): W untimed replays, then K timed ones between synchronisations.
    Every kernel of every step still runs; the graph only removes the host's
    per-call Python/ctypes cost from between the launches."""
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


def bench_decode(w, args, fa, synth, torch):
    per_step_unique = sum(kv_row_bytes(w.dtype) * w.n_seq * visible_rows(s, w.prefix) for s in w.layers)
    copies = max(1, -(-(2 * MALL_BYTES) // max(per_step_unique, 1)) + 1)
    copies = min(copies, 8)
    log(f"decode {w.name}: {len(w.layers)} layers, {copies} cache copies, "
        f"{per_step_unique / 1e6:.1f} MB KV per step")
    runs = [LayerRun(w, spec, copies, True, fa, synth, ring=args.ring) for spec in w.layers]
    torch.cuda.synchronize()
    wall_eager, per_launch = run_timed(runs, args.steps, args.warmup, copies, fa, torch)
    wall = wall_eager if args.eager else run_graphs(runs, args.steps, args.warmup, copies, fa, torch)
    kv_per_step = per_step_unique
    ms_per_step = wall * 1e3 / args.steps
    launches = len(per_launch)
    avg_launch_ms = sum(per_launch) / launches
    bytes_per_launch = kv_per_step / len(runs)
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    per_layer = {}
    for j, r in enumerate(runs):
        lt = per_launch[j::len(runs)]
        b = kv_row_bytes(w.dtype) * w.n_seq * visible_rows(r.spec, w.prefix)
        per_layer[r.spec.name] = {"kernel_us": round(1e3 * sum(lt) / len(lt), 2),
                                  "kv_MB": round(b / 1e6, 3),
                                  "kernel_GBps": round(b / (sum(lt) / len(lt) * 1e-3) / 1e9, 1),
                                  "p10_p50_p90_us": [round(1e3 * x, 2) for x in percentiles(lt)]}
    res = {
        "value": kv_per_step / (ms_per_step * 1e-3) / 1e9,
        "ms_per_step": ms_per_step,
        "eager": {"value": round(kv_per_step * args.steps / wall_eager / 1e9, 1),
                  "ms_per_step": round(wall_eager * 1e3 / args.steps, 5),
                  "note": "same steps launched one call at a time from Python, with per-kernel events"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic() if w.name == "decode_64x8192_bf16" else None,
                     "kernel": "muse::decode_kernel<bf16>" if w.dtype == 1 else "muse::decode_kernel<f32>",
                     "launches": launches, "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": int(bytes_per_launch),
                     "per_layer": per_layer},
        "config": {"workload": w.name, "n_seq": w.n_seq, "cached_tokens": w.prefix, "new_tokens": 1,
                   "layers": [f"{s.name}" + (f"_w{s.window}_theta{int(s.rope_theta)}" if s.window else "_nope")
                              for s in w.layers],
                   "q_heads": 32, "kv_heads": 2, "head_dim": 128, "cache_copies": copies,
                   "kv_bytes_per_step": kv_per_step, "kv_ring_sliding": bool(args.ring)},
    }
    return res, runs


def bench_prefill(w, steps, warmup, fa, synth, torch):
    log(f"prefill {w.name}: {len(w.layers)} layers")
    runs = [LayerRun(w, spec, 1, False, fa, synth) for spec in w.layers]
    torch.cuda.synchronize()
    wall, per_launch = run_timed(runs, steps, warmup, 1, fa, torch)
    flops_step = sum(FLOP_PER_PAIR * w.n_seq * prefill_pairs(s, w.prefix, w.n_new) for s in w.layers)
    ms_per_step = wall * 1e3 / steps
    per_layer = {}
    for j, r in enumerate(runs):
        lt = per_launch[j::len(runs)]
        f = FLOP_PER_PAIR * w.n_seq * prefill_pairs(r.spec, w.prefix, w.n_new)
        avg = sum(lt) / len(lt)
        per_layer[r.spec.name] = {"kernel_ms": round(avg, 4), "tflop": round(f / 1e12, 4),
                                  "kernel_TFLOPs": round(f / (avg * 1e-3) / 1e12, 1),
                                  "p10_p50_p90_ms": [round(x, 4) for x in percentiles(lt)]}
    kern = sum(per_launch) / len(per_launch)
    achieved = flops_step / len(runs) / (kern * 1e-3) / 1e12
    return {
        "workload": w.name,
        "tflops": round(flops_step / (ms_per_step * 1e-3) / 1e12, 2),
        "ms_per_step": round(ms_per_step, 4),
        "frac_mfma_peak": round(flops_step / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "muse::prefill_group_kernel<1, 8, 1, false> (bf16)", "avg_launch_ms": round(kern, 4),
                     "per_layer": per_layer,
                     "counters": prefill_counters() if w.name == "prefill_8x8192_bf16" else None},
        "flop_per_step": flops_step, "steps": steps, "warmup": warmup,
    }


def bench_schedule(w, fa, synth, torch, ring=False):
    """The 52-layer schedule workload: 4 sequences with 32,768 cached rows per
    layer, a 4,096-token chunked prefill through all 52 layers (timed as one
    phase, eager calls), then 256 decode steps of all 52 layers (one step =
    52 decode calls and the seq_len increment, replayed from a HIP graph).
    ring: the sliding layers keep their window in a ring of `window` rows."""
    S, L0, N, steps = w.n_seq, w.prefix, w.n_new, w.decode_steps
    extra = 4                                          # warm-up decode steps, rows overwritten later
    cap = L0 + N + steps + extra
    max_dec = L0 + N + steps + extra - 1
    log(f"schedule {w.name}: {len(w.layers)} layers, capacity {cap}")
    layers, inputs, outs, dec_in = [], [], [], []
    for spec in w.layers:
        r = uses_ring(spec, ring, synth)
        inp = synth.layer_inputs(w, spec, device="cuda", backend="torch",
                                 capacity=L0 if r else cap)
        if r:
            inp.cache_k = ring_of(inp.cache_k, L0, spec.window)
            inp.cache_v = ring_of(inp.cache_v, L0, spec.window)
        layers.append(fa.make_layer(spec.kind, window=spec.window, rope_theta=spec.rope_theta,
                                    rms_eps=spec.rms_eps, q_norm_gain=spec.q_gain,
                                    k_norm_gain=spec.k_gain, attn_scale=spec.scale, dtype=w.dtype,
                                    kv_ring=1 if r else 0))
        inputs.append(inp)
        outs.append(torch.empty_like(inp.gate))
        d = synth.layer_inputs(w, spec, device="cuda", backend="torch", n_new=1, prefix=0,
                               step=1, with_cache=False)
        dec_in.append((d.q, d.k, d.v, d.gate, torch.empty_like(d.gate)))
    seq_len = torch.full((S,), L0, dtype=torch.int32, device="cuda")
    ws_p = torch.empty(max(fa.workspace_size(lay, S, N, L0, False) for lay in layers),
                       dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(max(fa.workspace_size(lay, S, 1, max_dec, True) for lay in layers),
                       dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for lay, inp, out in zip(layers, inputs, outs):
        fa.prefill(lay, inp.q, inp.k, inp.v, inp.gate, inp.cache_k, inp.cache_v, seq_len, out,
                   max_seq_len=L0, workspace=ws_p)
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    flops = sum(FLOP_PER_PAIR * S * prefill_pairs(spec, L0, N) for spec in w.layers)
    seq_len.fill_(L0 + N)

    def one_step():
        for lay, inp, (q, k, v, g, o) in zip(layers, inputs, dec_in):
            fa.decode(lay, q, k, v, g, inp.cache_k, inp.cache_v, seq_len, o, max_seq_len=max_dec,
                      workspace=ws_d)
        seq_len.add_(1)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_step()
    for _ in range(extra):
        graph.replay()
    torch.cuda.synchronize()
    seq_len.fill_(L0 + N)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    t_decode = time.perf_counter() - t0
    kv = sum(kv_row_bytes(w.dtype) * S * visible_rows(spec, L0 + N + i)
             for i in range(steps) for spec in w.layers)
    del graph
    cache_bytes = sum(2 * inp.cache_k.numel() * inp.cache_k.element_size() for inp in inputs)
    return {"workload": w.name, "layers": len(w.layers), "n_seq": S,
            "kv_ring_sliding": bool(ring), "kv_cache_GB": round(cache_bytes / 1e9, 3),
            "prefill": {"tokens_per_seq": N, "at_position": L0, "ms": round(t_prefill * 1e3, 2),
                        "tflop": round(flops / 1e12, 3), "TFLOPs": round(flops / t_prefill / 1e12, 1),
                        "frac_mfma_peak": round(flops / t_prefill / 1e12 / MFMA_PEAK_TFLOPS, 4),
                        "launch": "eager"},
            "decode": {"steps": steps, "ms": round(t_decode * 1e3, 2), "kv_GB": round(kv / 1e9, 2),
                       "GBps": round(kv / t_decode / 1e9, 1),
                       "frac_hbm_peak": round(kv / t_decode / 1e9 / HBM_PEAK_GBS, 4),
                       "launch": "each step (52 decode calls + seq_len increment) replayed from a HIP graph"}}


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
                             "kernel": "muse::out_proj_gemm_kernel (bf16)"}
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
    # GPU time of one pass between events (the host builds and checks the
    # tile list before enqueueing; that is timed separately)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_ms = []
    host = 0.0
    for _ in range(steps):
        t0 = time.perf_counter()
        e0.record()
        fa.kv_relocate(lay, a_k, a_v, b_k, b_v, tiles)
        e1.record()
        host += time.perf_counter() - t0
        torch.cuda.synchronize()
        gpu_ms.append(e0.elapsed_time(e1))
    dt = sorted(gpu_ms)[len(gpu_ms) // 2] * 1e-3
    moved = 2 * a_k.numel() * a_k.element_size()           # K and V bytes per pass
    ok = bool(torch.equal(b_k[1, (L // T - 1) * T:], a_k[0, :T]))
    return {"tiles": tiles[1], "tile_rows": T, "MB_moved": round(moved / 1e6, 1), "gpu_ms": round(dt * 1e3, 3),
            "host_ms_per_call": round(host / steps * 1e3, 3),
            "GBps_read_plus_write": round(2 * moved / dt / 1e9, 1),
            "frac_hbm_peak": round(2 * moved / dt / 1e9 / HBM_PEAK_GBS, 4), "bytes_checked": ok}


def cpu_baseline_decode(w, runs, synth, torch):
    """Time the CPU oracle on this step's inputs (all rows of both layers) and
    check the benchmarked GPU output against it."""
    import numpy as np
    import oracle
    rows = oracle.all_rows(w.n_seq, 1)
    t_oracle = 0.0
    worst = 0.0
    ok = True
    for r in runs:
        ck, cv = r.caches[0]
        pk, pv = synth.to_storage_numpy(ck), synth.to_storage_numpy(cv)   # rows < seq_len untouched
        lay = oracle.Layer(kind=r.spec.kind, window=r.spec.window, rope_theta=r.spec.rope_theta,
                           rms_eps=r.spec.rms_eps, q_gain=r.spec.q_gain, k_gain=r.spec.k_gain,
                           scale=r.spec.scale, dtype=w.dtype)
        args = (lay, r.inp.seq_len.cpu().numpy(), synth.to_storage_numpy(r.inp.k),
                synth.to_storage_numpy(r.inp.v), pk, pv, rows,
                synth.to_storage_numpy(r.inp.q).reshape(-1, 32, 128),
                synth.to_storage_numpy(r.inp.gate).reshape(-1, 4096))
        t0 = time.perf_counter()
        ref = oracle.attn_rows(*args)
        t_oracle += time.perf_counter() - t0
        got = r.out.double().cpu().numpy().reshape(-1, 4096)
        err = np.abs(got - ref)
        worst = max(worst, float(err.max()))
        ok = ok and bool(np.all(err <= 2e-2 + 1e-2 * np.abs(ref)))
    kv = sum(kv_row_bytes(w.dtype) * w.n_seq * visible_rows(r.spec, w.prefix) for r in runs)
    return {"value": round(kv / t_oracle / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole step: {w.n_seq} sequences x {len(runs)} layers, all 32 heads "
                      f"({t_oracle:.2f} s)",
            "seconds": round(t_oracle, 3)}, {"max_abs_err": worst, "within_tolerance": ok}


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
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
    fa.lib()                                  # fails loudly when the HIP library is missing
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.prefill_only:
        pw = synth.WORKLOADS[args.prefill_workload]
        print(json.dumps({"prefill": bench_prefill(pw, args.prefill_steps, 2, fa, synth, torch)}), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    if not w.is_decode:
        print(f"--workload must be a decode workload, got {w.name}", file=sys.stderr)
        sys.exit(2)
    res, runs = bench_decode(w, args, fa, synth, torch)
    line = {
        "metric": METRIC, "value": round(res["value"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == 1 else "f32",
        "data": "synthetic: seeded N(0,1) inputs and cache prefixes, resident in HBM",
        "config": res["config"], "roofline": res["roofline"],
        "frac_hbm_peak": round(res["value"] / HBM_PEAK_GBS, 4),
        "launch": "eager calls" if args.eager else "each step replayed from a HIP graph of its kernel launches",
        "eager": res["eager"],
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same step")
        cb, parity = cpu_baseline_decode(w, runs, synth, torch)
        line["cpu_baseline"] = cb
        line["parity"] = parity
    del runs
    torch.cuda.empty_cache()
    if not args.no_prefill:
        pw = synth.WORKLOADS[args.prefill_workload]
        line["prefill"] = bench_prefill(pw, args.prefill_steps, 2, fa, synth, torch)
    if args.verify:
        torch.cuda.empty_cache()
        line["verify"] = bench_verify(fa, synth, torch)
    if args.out_proj:
        torch.cuda.empty_cache()
        line["out_proj"] = bench_out_proj(fa, synth, torch)
    if args.relocate:
        torch.cuda.empty_cache()
        line["relocate"] = bench_relocate(fa, synth, torch)
    if args.schedule:
        torch.cuda.empty_cache()
        line["schedule"] = bench_schedule(synth.WORKLOADS["schedule_52x4_32768p4096_256d"], fa, synth, torch,
                                          ring=args.ring)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

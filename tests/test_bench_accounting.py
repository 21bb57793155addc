"""The benchmark's algorithmic work, checked on the CPU against closed forms:
1,024 bytes of K and V per visible row per sequence for bf16 decode
("Chapter 9 - The Muse Glimmer architecture" 9.5, 9.6), 16,384 flop per
visible (query, key) pair over 32 heads for prefill, and the visibility rule
(key j visible to the query at p iff j <= p and, on sliding layers,
p - j < window; Ch 9, 9.7).  The rooflines and `value` divide these by
measured times, so a slip here would skew every reported fraction.  Also the
phase-timeline summary on synthetic records."""
import numpy as np

import bench
from full_gqa_attention_amd import synth


def _wl(name):
    return synth.WORKLOADS[name]


def test_row_bytes_and_visibility():
    assert bench.kv_row_bytes(synth.BF16) == 2 * 2 * 128 * 2
    assert bench.kv_row_bytes(synth.F32) == 2 * 2 * 128 * 4
    sl, fu = synth.sliding(2048, 500000.0), synth.full()
    for p in (0, 1, 2046, 2047, 2048, 10_000):
        assert bench.visible_rows(fu, p) == p + 1
        assert bench.visible_rows(sl, p) == min(2048, p + 1)
    # brute force on a tiny window
    w = synth.sliding(5, 10000.0)
    for p in range(12):
        assert bench.visible_rows(w, p) == sum(1 for j in range(p + 1) if p - j < 5)


def test_prefill_pairs_closed_forms():
    sl, fu = synth.sliding(2048, 500000.0), synth.full()
    N = 8192
    assert bench.prefill_pairs(fu, 0, N) == N * (N + 1) // 2
    W = 2048
    assert bench.prefill_pairs(sl, 0, N) == W * (W + 1) // 2 + (N - W) * W
    # a chunk onto a prefix: every query sees the whole prefix (full) or a full window (sliding)
    L, M = 32768, 4096
    assert bench.prefill_pairs(fu, L, M) == sum(L + t + 1 for t in range(M))
    assert bench.prefill_pairs(sl, L, M) == M * W


def test_decode_bytes_of_the_workloads():
    c2, c4 = _wl("decode_64x8192_bf16"), _wl("decode_16x131072_bf16")
    by = {w.name: {s.name: bench.kv_row_bytes(w.dtype) * w.n_seq * bench.visible_rows(s, w.prefix)
                   for s in w.layers} for w in (c2, c4)}
    assert by[c2.name]["full"] == 64 * 8193 * 1024          # 536.94 MB
    assert by[c2.name]["sliding"] == 64 * 2048 * 1024       # 134.22 MB
    assert by[c4.name]["full"] == 16 * 131073 * 1024        # 2.1475 GB
    assert by[c4.name]["sliding"] == 16 * 2048 * 1024       # 33.55 MB


def test_prefill_flops_of_the_workloads():
    c3 = _wl("prefill_8x8192_bf16")
    fl = {s.name: bench.FLOP_PER_PAIR * c3.n_seq * bench.prefill_pairs(s, c3.prefix, c3.n_new) for s in c3.layers}
    assert abs(fl["full"] / 1e12 - 4.3986) < 5e-4
    assert abs(fl["sliding"] / 1e12 - 1.9243) < 5e-4


def test_schedule_totals():
    """52 layers (13 full at l % 4 == 3), 4 sequences, a 4,096 chunk onto 32,768 cached
    rows, then 256 decode steps: 142.94 TFLOP of chunked prefill and 588.0 GB of KV reads."""
    w = _wl("schedule_52x4_32768p4096_256d")
    assert len(w.layers) == 52 and sum(1 for s in w.layers if s.window == 0) == 13
    assert all((s.window == 0) == (i % 4 == 3) for i, s in enumerate(w.layers))
    flop = sum(bench.FLOP_PER_PAIR * w.n_seq * bench.prefill_pairs(s, w.prefix, w.n_new) for s in w.layers)
    assert abs(flop / 1e12 - 142.94) < 0.01
    kv = sum(bench.kv_row_bytes(w.dtype) * w.n_seq * bench.visible_rows(s, w.prefix + w.n_new + i)
             for i in range(w.decode_steps) for s in w.layers)
    assert w.decode_steps == 256
    assert abs(kv / 1e9 - 588.0) < 0.1


def test_timeline_summary_on_synthetic_records():
    split = np.zeros((8, 8), np.int64)
    merge = np.zeros((4, 4), np.int64)
    # two split workgroups (10 ns units): start, seq_len, Q, Q-hat, sub-tiles, LDS merge, stores, sub-tiles
    split[0] = [1000, 1030, 1200, 1260, 1340, 1400, 1450, 1]
    split[1] = [1010, 1040, 1220, 1280, 1380, 1450, 1500, 1]
    merge[0] = [1620, 1780, 1900, 32]
    merge[1] = [1630, 1790, 1910, 32]
    t = bench.timeline_summary(split, merge)
    assert t["split_workgroups"] == 2
    assert t["start_spread_us"] == 0.1
    assert t["phases_us"]["seq_len read"][0] == 0.3
    assert t["last_split_end_us"] == 5.0
    assert t["merge"]["first_start_after_last_split_us"] == 1.2
    assert t["merge"]["loads_arrived_us_p50"] == 1.6
    assert t["merge"]["last_end_us"] == 9.1


def test_leg_trace_summary(tmp_path):
    """The per-leg trace summary averages the split and merge kernels of a
    trace and prices the call at the leg's algorithmic bytes."""
    import csv
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        t = 0
        for i in range(4):                              # split 20/22 us, merge 4 us (ns stamps)
            wr.writerow({"Kernel_Name": "void muse::decode_kernel<__bf16, 3, 4>(muse::DecodeArgs)",
                         "Start_Timestamp": t, "End_Timestamp": t + (20000 if i % 2 == 0 else 22000)})
            t += 30000
            wr.writerow({"Kernel_Name": "void muse::decode_merge_kernel<__bf16>(muse::DecodeArgs)",
                         "Start_Timestamp": t, "End_Timestamp": t + 4000})
            t += 10000
        wr.writerow({"Kernel_Name": "other_kernel", "Start_Timestamp": t, "End_Timestamp": t + 999000})
    out = tmp_path / "out.md"
    bench.summarize_leg_traces(str(out), "cmd", "decode_64x8192_bf16:sliding", str(path))
    row = [l for l in open(out).read().splitlines() if l.startswith("| decode_64x8192_bf16, sliding")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "21.00 (20.00, 22.00)" and cells[2] == "4.00" and cells[3] == "25.00"
    assert cells[4] == str(round(64 * 2048 * 1024 / 25.0 / 1e3))

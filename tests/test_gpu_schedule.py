"""End-to-end parity of the 52-layer schedule as the benchmark runs it
("Chapter 9 - The Muse Glimmer architecture" 9.4 and Figure 9.4: layers
l % 4 == 3 full NoPE, the others sliding RoPE with a 2,048-key window; 9.7
for the ring): 4 sequences with 32,768 cached rows per layer, a 4,096-token
chunk through all 52 layers, then decode steps replayed from one captured
HIP graph in which every layer's decode call is followed by the device-side
seq_len increment -- the Schedule object the benchmark times.

Every layer is checked: sampled chunk rows of two sequences (window and tile
edges, all 32 heads), every decode output of every replayed step (all 4
sequences), and every cache row the chunk and the steps appended (on a ring
layer, the rows the ring holds).  The oracle keeps its own cache: the
synthetic prefix plus the rows it appended itself.
"""
import numpy as np
import pytest
import torch

import oracle
from full_gqa_attention_amd import synth
from full_gqa_attention_amd.schedule import Schedule
from parity import assert_close, check_rows, edge_rows, oracle_layer, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
STEPS = 4


def _u16(t: torch.Tensor) -> np.ndarray:
    return synth.to_storage_numpy(t)


def _bits(x64: np.ndarray) -> np.ndarray:
    """bf16-representable doubles -> their bf16 bit patterns (exact)."""
    return torch.from_numpy(np.ascontiguousarray(x64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rows_of(sch: Schedule, l: int, positions) -> torch.Tensor:
    """Cache rows holding `positions` in layer l's cache (ring or linear)."""
    spec = sch.specs[l]
    pos = torch.as_tensor(np.asarray(positions), device=DEV)
    return pos % spec.window if sch.is_ring(spec) else pos


@pytest.mark.parametrize("ring", [False, True], ids=["linear", "ring"])
def test_schedule_end_to_end(ring):
    w = synth.WORKLOADS["schedule_52x4_32768p4096_256d"]
    S, L0, N, K = w.n_seq, w.prefix, w.n_new, STEPS
    sch = Schedule(w, ring=ring, steps=K)
    print(f"schedule: 52 layers, ring={ring}, cache {sch.cache_bytes() / 1e9:.2f} GB", flush=True)
    # the prefix rows a sliding layer's chunk can see, read before the chunk
    # overwrites a ring
    pre = {}
    for l, spec in enumerate(sch.specs):
        if spec.kind == synth.SLIDING_ROPE:
            lo = L0 - spec.window + 1
            r = _rows_of(sch, l, np.arange(lo, L0))
            pre[l] = (lo, _u16(sch.inputs[l].cache_k[:, r]), _u16(sch.inputs[l].cache_v[:, r]))
    sch.prefill()
    torch.cuda.synchronize()
    samples, got_chunk = {}, {}
    for l, spec in enumerate(sch.specs):
        rows = edge_rows(N, spec.window, (1000, 3000), seqs=(l % S, (l + 2) % S))
        samples[l] = rows
        sel = (torch.as_tensor(rows[:, 0], device=DEV).long(), torch.as_tensor(rows[:, 1], device=DEV).long())
        got_chunk[l] = to_f64(sch.outs[l][sel])
    sch.start_decode()
    graph = sch.capture_step()
    got_steps = []
    for k in range(K):
        graph.replay()
        torch.cuda.synchronize()
        got_steps.append([to_f64(d[4][:, 0]) for d in sch.dec])
    assert sch.seq_len.tolist() == [L0 + N + K] * S       # advanced on the device, once per replay
    print("gpu done; checking against the oracle", flush=True)

    for l, spec in enumerate(sch.specs):
        lay = oracle_layer(spec, w.dtype)
        inp = sch.inputs[l]
        ck = np.zeros((S, sch.capacity, 2, 128), np.uint16)
        cv = np.zeros_like(ck)
        if spec.kind == synth.FULL_NOPE:                   # rows below the prefix are never written
            ck[:, :L0] = _u16(inp.cache_k[:, :L0])
            cv[:, :L0] = _u16(inp.cache_v[:, :L0])
        else:
            lo, pk, pv = pre[l]
            ck[:, lo:L0], cv[:, lo:L0] = pk, pv
        rows = samples[l]
        ref, kst, vst = oracle.attn_rows(
            lay, np.full(S, L0, np.int32), _u16(inp.k), _u16(inp.v), ck, cv, rows,
            _u16(inp.q)[rows[:, 0], rows[:, 1]], _u16(inp.gate)[rows[:, 0], rows[:, 1]], want_store=True)
        assert_close(got_chunk[l], ref, w.dtype, f"layer {l} chunk")
        # the chunk's stored rows: on a ring the last `window` positions, less
        # the slots the decode steps have since reused (checked with the steps)
        first = L0 + N - spec.window + K if sch.is_ring(spec) else L0
        r = _rows_of(sch, l, np.arange(first, L0 + N))
        check_rows(to_f64(inp.cache_k[:, r]), to_f64(inp.cache_v[:, r]), kst[:, first - L0:],
                   vst[:, first - L0:], w.dtype, f"layer {l} chunk rows")
        ck[:, L0:L0 + N], cv[:, L0:L0 + N] = _bits(kst), _bits(vst)
        q, kk, vv, g, _ = sch.dec[l]
        for k in range(K):
            p = L0 + N + k
            dref, dk, dv = oracle.attn_rows(
                lay, np.full(S, p, np.int32), _u16(kk), _u16(vv), ck, cv, oracle.all_rows(S, 1),
                _u16(q).reshape(S, 32, 128), _u16(g).reshape(S, 4096), want_store=True)
            assert_close(got_steps[k][l], dref, w.dtype, f"layer {l} decode step {k}")
            r = _rows_of(sch, l, [p])
            check_rows(to_f64(inp.cache_k[:, r]), to_f64(inp.cache_v[:, r]), dk, dv, w.dtype,
                       f"layer {l} step {k} row")
            ck[:, p], cv[:, p] = _bits(dk[:, 0]), _bits(dv[:, 0])
        if l % 13 == 12:
            print(f"layers 0..{l} match", flush=True)

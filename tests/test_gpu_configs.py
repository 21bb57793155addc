"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: every row where the oracle finishes in seconds (the 64 x
8,192 and 16 x 131,072 decode steps), sampled rows of every sequence elsewhere.  A sample always includes the
window and tile edges; each attention row depends only on its own query and
the cache, so checking a row checks it exactly.  Every appended cache row is
checked in all cases.
"""
import numpy as np
import pytest
import torch

import oracle
from full_gqa_attention_amd import synth
from parity import (assert_close, check_appended, check_layer, edge_rows, host_cache, run_gpu,
                    run_oracle, to_f64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _name(spec):
    return spec.name


@pytest.mark.parametrize("li", [0, 1], ids=["sliding", "full"])
def test_decode_64x8192_all_rows(li):
    w = synth.WORKLOADS["decode_64x8192_bf16"]
    spec = w.layers[li]
    inp = synth.layer_inputs(w, spec, device=DEV, backend="torch")
    check_layer(w, spec, inp, decode=True, max_seq_len=w.prefix)


@pytest.mark.parametrize("li", [0, 1], ids=["sliding", "full"])
def test_prefill_8x8192_sampled(li):
    w = synth.WORKLOADS["prefill_8x8192_bf16"]
    spec = w.layers[li]
    inp = synth.layer_inputs(w, spec, device=DEV, backend="torch")
    # every sequence: the window and tile edges and 16 rows of its own
    rng = np.random.default_rng(7)
    rows = np.concatenate([edge_rows(w.n_new, spec.window, tuple(int(x) for x in rng.integers(0, w.n_new, 16)),
                                     seqs=(s,)) for s in range(w.n_seq)])
    check_layer(w, spec, inp, decode=False, rows=rows, untouched=False)


@pytest.mark.parametrize("li", [0, 1], ids=["full", "sliding"])
def test_decode_16x131072_sampled(li):
    """Long-context decode: 16 sequences x 131,072 cached rows; every
    sequence's row checked against the oracle (all 32 heads), every appended
    row checked."""
    w = synth.WORKLOADS["decode_16x131072_bf16"]
    spec = w.layers[li]
    inp = synth.layer_inputs(w, spec, device=DEV, backend="torch")
    check_layer(w, spec, inp, decode=True, max_seq_len=w.prefix, untouched=False)


def _bf16_from_f64(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


@pytest.mark.parametrize("layer_index", [3, 4], ids=["full_l3", "sliding_l4"])
def test_schedule_chunk_then_decode(layer_index):
    """One layer of the 52-layer schedule at its real shape: a 4,096-token
    chunk onto 32,768 cached rows for 4 sequences (sampled rows), then 3
    decode steps (every row).  The oracle's cache for the decode steps is the
    synthetic prefix plus the rows the oracle itself appended."""
    w = synth.WORKLOADS["schedule_52x4_32768p4096_256d"]
    spec = synth.model_layer(layer_index)
    steps = 3
    cap = w.prefix + w.n_new + steps
    inp = synth.layer_inputs(w, spec, device=DEV, backend="torch", capacity=cap)
    seq = inp.seq_len.cpu().numpy()
    pk, pv = host_cache(inp)                           # the oracle's own cache copy
    out = run_gpu(spec, w.dtype, inp, decode=False, max_seq_len=w.prefix)
    rows = np.concatenate([edge_rows(w.n_new, spec.window, (1000, 3000), seqs=(s,)) for s in range(w.n_seq)])
    ref, kst, vst = run_oracle(spec, w.dtype, inp, rows, pk, pv, seq)
    got = to_f64(out[torch.as_tensor(rows[:, 0], device=DEV).long(), torch.as_tensor(rows[:, 1], device=DEV).long()])
    assert_close(got, ref, w.dtype, f"chunk l{layer_index}")
    check_appended(inp, kst, vst, seq, w.dtype, w.n_new)
    # the oracle's cache: prefix + its own appended rows
    ok_k = torch.from_numpy(pk.view(np.int16)).view(torch.bfloat16)
    ok_v = torch.from_numpy(pv.view(np.int16)).view(torch.bfloat16)
    ok_k[:, w.prefix:w.prefix + w.n_new] = _bf16_from_f64(kst)
    ok_v[:, w.prefix:w.prefix + w.n_new] = _bf16_from_f64(vst)
    L = w.prefix + w.n_new
    for step in range(1, steps + 1):
        d = synth.layer_inputs(w, spec, device=DEV, backend="torch", n_new=1, prefix=0,
                               step=step, with_cache=False)
        d.cache_k, d.cache_v = inp.cache_k, inp.cache_v
        d.seq_len = torch.full((w.n_seq,), L, dtype=torch.int32, device=DEV)
        dout = run_gpu(spec, w.dtype, d, decode=True, max_seq_len=cap - 1)
        drows = oracle.all_rows(w.n_seq, 1)
        dref, dk, dv = run_oracle(spec, w.dtype, d, drows,
                                  ok_k.view(torch.int16).numpy().view(np.uint16),
                                  ok_v.view(torch.int16).numpy().view(np.uint16),
                                  np.full(w.n_seq, L, np.int32))
        assert_close(to_f64(dout[:, 0]), dref, w.dtype, f"decode step {step} l{layer_index}")
        check_appended(d, dk, dv, np.full(w.n_seq, L, np.int32), w.dtype, 1)
        ok_k[:, L] = _bf16_from_f64(dk[:, 0])
        ok_v[:, L] = _bf16_from_f64(dv[:, 0])
        L += 1

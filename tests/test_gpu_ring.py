"""Ring KV cache for sliding layers ("Chapter 9 - The Muse Glimmer
architecture" 9.7: each sliding layer keeps a fixed 2,048-row ring, token-
major): position p lives in cache row p % capacity.

The oracle is unchanged (the visible set is the same), so each test runs the
same inputs twice through the C ABI -- once with a linear cache, checked
against the oracle, once with a ring built from the same rows -- and requires
the ring run to reproduce the linear run bit for bit, and the ring to hold
exactly the rows of the last `capacity` positions afterwards.  Ring slots
that hold no visible position are filled with other finite values, so a read
of a wrong slot changes the result.
"""
import numpy as np
import pytest
import torch

import full_gqa_attention_amd as fa
from full_gqa_attention_amd import synth
from parity import check_layer, lib_layer, edge_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(spec, lens, N, step=0):
    w = synth.Workload("ring", 91, synth.BF16, len(lens), max(lens), N, (spec,))
    inp = synth.layer_inputs(w, spec, device=DEV, prefix=max(lens), n_new=N,
                             capacity=max(lens) + N, step=step)
    inp.seq_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return w, inp


def _ring_from(cache: torch.Tensor, lens, cap: int, seed: int) -> torch.Tensor:
    """Ring of `cap` rows holding positions [max(0, L - cap), L) of each
    sequence at row p % cap; the other rows get unrelated finite values."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    ring = (torch.randn((cache.shape[0], cap) + tuple(cache.shape[2:]), generator=g) * 3.0)
    ring = ring.to(device=cache.device, dtype=cache.dtype)
    for s, L in enumerate(lens):
        pos = torch.arange(max(0, L - cap), L, device=cache.device)
        ring[s, pos % cap] = cache[s, pos]
    return ring


def _ring_layer(spec):
    l = lib_layer(spec, synth.BF16)
    l.kv_ring = 1
    return l


def _check_ring_rows(ring: torch.Tensor, cache: torch.Tensor, lens_after, cap: int):
    for s, L in enumerate(lens_after):
        pos = torch.arange(max(0, L - cap), L, device=cache.device)
        assert torch.equal(ring[s, pos % cap], cache[s, pos]), f"sequence {s}"


@pytest.mark.parametrize("cap", [2048, 2500], ids=["cap_eq_window", "cap_gt_window"])
def test_ring_decode_matches_linear(cap):
    spec = synth.sliding(2048, 500000.0)
    lens = [0, 1, 1500, 2047, 2048, 5000, 6143]
    w, inp = _inputs(spec, lens, 1)
    ck0, cv0 = inp.cache_k.clone(), inp.cache_v.clone()
    lin, _ = check_layer(w, spec, inp, decode=True)                  # linear run vs the oracle
    rk, rv = _ring_from(ck0, lens, cap, 1), _ring_from(cv0, lens, cap, 2)
    out = fa.decode(_ring_layer(spec), inp.q, inp.k, inp.v, inp.gate, rk, rv, inp.seq_len,
                    max_seq_len=max(lens))
    torch.cuda.synchronize()
    assert torch.equal(out, lin)
    _check_ring_rows(rk, inp.cache_k, [L + 1 for L in lens], cap)
    _check_ring_rows(rv, inp.cache_v, [L + 1 for L in lens], cap)


@pytest.mark.parametrize("lens,N", [([0, 0], 3000), ([5000, 100], 200), ([1000, 2047], 1500)],
                         ids=["chunk_longer_than_ring", "wrapped_prefix", "partial"])
def test_ring_prefill_matches_linear(lens, N):
    spec = synth.sliding(2048, 500000.0)
    cap = 2048
    w, inp = _inputs(spec, lens, N)
    ck0, cv0 = inp.cache_k.clone(), inp.cache_v.clone()
    rows = edge_rows(N, spec.window, extra=(N // 2, N - 2), seqs=range(len(lens)))
    lin, _ = check_layer(w, spec, inp, decode=False, rows=rows)
    rk, rv = _ring_from(ck0, lens, cap, 3), _ring_from(cv0, lens, cap, 4)
    out = fa.prefill(_ring_layer(spec), inp.q, inp.k, inp.v, inp.gate, rk, rv, inp.seq_len,
                     max_seq_len=max(lens))
    torch.cuda.synchronize()
    assert torch.equal(out, lin)
    _check_ring_rows(rk, inp.cache_k, [L + N for L in lens], cap)
    _check_ring_rows(rv, inp.cache_v, [L + N for L in lens], cap)


def test_ring_prefill_then_decode_steps():
    """A chunked prefill and then decode steps that wrap the ring several
    times, linear and ring side by side, bit for bit."""
    spec = synth.sliding(128, 10000.0)
    cap, lens, N, steps = 128, [40, 300], 200, 300
    w, inp = _inputs(spec, lens, N)
    total = max(lens) + N + steps
    lin_k = torch.zeros((2, total, 2, 128), dtype=torch.bfloat16, device=DEV)
    lin_v = torch.zeros_like(lin_k)
    lin_k[:, :inp.cache_k.shape[1]] = inp.cache_k
    lin_v[:, :inp.cache_v.shape[1]] = inp.cache_v
    rk, rv = _ring_from(lin_k, lens, cap, 5), _ring_from(lin_v, lens, cap, 6)
    lay_lin, lay_ring = lib_layer(spec, synth.BF16), _ring_layer(spec)
    seq = inp.seq_len.clone()
    a = fa.prefill(lay_lin, inp.q, inp.k, inp.v, inp.gate, lin_k, lin_v, seq, max_seq_len=max(lens))
    b = fa.prefill(lay_ring, inp.q, inp.k, inp.v, inp.gate, rk, rv, seq, max_seq_len=max(lens))
    assert torch.equal(a, b)
    seq += N
    for i in range(steps):
        d = synth.layer_inputs(w, spec, device=DEV, n_new=1, prefix=0, step=i + 1, with_cache=False)
        mx = max(lens) + N + i
        a = fa.decode(lay_lin, d.q, d.k, d.v, d.gate, lin_k, lin_v, seq, max_seq_len=mx)
        b = fa.decode(lay_ring, d.q, d.k, d.v, d.gate, rk, rv, seq, max_seq_len=mx)
        assert torch.equal(a, b), f"decode step {i}"
        seq += 1
    torch.cuda.synchronize()
    _check_ring_rows(rk, lin_k, seq.tolist(), cap)
    _check_ring_rows(rv, lin_v, seq.tolist(), cap)

"""Short bf16 chunks (1 to 16 new tokens per sequence: the verify step of
speculative decoding, "How Muse Glimmer Fits an Agent on Your Device",
section on drafting and verifying) against the oracle.

These calls take the verify kernels (split-K over the key range, all 16
heads of a KV head per workgroup, splits merged in a second kernel); the
attention they compute is the prefill's ("Chapter 9 - The Muse Glimmer
architecture" 9.5-9.8): causal within the chunk, over the cached prefix,
inside the window on sliding layers.  Cases span one to many splits, empty
and ragged prefixes, prefixes shorter than the window, windows of 1 and 64
keys, padding rows (N < 16), and the rejected-draft pattern where the next
call starts inside rows the last one wrote.
"""
import numpy as np
import pytest
import torch

import full_gqa_attention_amd as fa
from full_gqa_attention_amd import synth
from parity import check_layer, run_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"

SPECS = [synth.full(), synth.sliding(2048, 500000.0), synth.sliding(64, 10000.0), synth.sliding(1, 500000.0)]


def _inputs(spec, lens, N, capacity=None, step=0, config=94):
    w = synth.Workload("verify", config, synth.BF16, len(lens), max(lens), N, (spec,))
    inp = synth.layer_inputs(w, spec, device=DEV, prefix=max(lens), n_new=N,
                             capacity=capacity or max(lens) + N, step=step)
    inp.seq_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return w, inp


@pytest.mark.parametrize("N", [1, 2, 7, 16])
@pytest.mark.parametrize("spec", SPECS, ids=["full", "w2048", "w64", "w1"])
def test_verify_ragged(spec, N):
    lens = [0, 1, 100, 3000, 2047]
    w, inp = _inputs(spec, lens, N)
    check_layer(w, spec, inp, decode=False)


@pytest.mark.parametrize("spec", [synth.full(), synth.sliding(2048, 500000.0)], ids=["full", "w2048"])
def test_verify_long_prefix_many_splits(spec):
    """One sequence with a long prefix: the most splits (64) on the full
    layer; tiles cut at odd places by the window on the sliding one."""
    w, inp = _inputs(spec, [40000], 16)
    check_layer(w, spec, inp, decode=False)
    w, inp = _inputs(spec, [9001, 31], 13, step=1)
    check_layer(w, spec, inp, decode=False)


def test_verify_rejected_drafts_overwritten():
    """Verify 16 drafts, accept 5 (seq_len += 5), verify the next 16: the
    second call overwrites rows the first wrote past the accepted ones and
    reads only the accepted prefix."""
    spec = synth.sliding(64, 10000.0)
    lens = [200, 37]
    w, inp = _inputs(spec, lens, 16, capacity=300)
    check_layer(w, spec, inp, decode=False)
    w2, inp2 = _inputs(spec, lens, 16, capacity=300, step=1)
    inp2.cache_k.copy_(inp.cache_k)
    inp2.cache_v.copy_(inp.cache_v)
    inp2.seq_len = inp.seq_len + 5
    check_layer(w2, spec, inp2, decode=False, max_seq_len=max(lens) + 5)


def test_verify_deterministic_and_bad_seq_len():
    spec = synth.full()
    w, inp = _inputs(spec, [500, 700, 20], 9, capacity=800)
    a = run_gpu(spec, w.dtype, inp, False, max_seq_len=700).clone()
    b = run_gpu(spec, w.dtype, inp, False, max_seq_len=700).clone()
    assert torch.equal(a, b)
    inp.seq_len[1] = 701                       # above max_seq_len: refused on the device
    before = inp.cache_k.clone()
    out = run_gpu(spec, w.dtype, inp, False, max_seq_len=700)
    assert torch.isnan(out[1].float()).all()
    assert torch.equal(inp.cache_k[1], before[1])
    assert torch.equal(out[0], a[0]) and torch.equal(out[2], a[2])


def test_verify_split_count_invariance():
    """The same rows with a smaller batch (more splits per sequence) agree
    within the bf16 tolerance: the split count changes only the summation
    order."""
    spec = synth.full()
    w, inp = _inputs(spec, [3000] * 64, 16)      # 2 splits per (sequence, KV head)
    many = run_gpu(spec, w.dtype, inp, False).float()
    w1, inp1 = _inputs(spec, [3000], 16)          # 6 splits
    one = run_gpu(spec, w1.dtype, inp1, False).float()
    assert torch.allclose(many[0], one[0], atol=2e-2, rtol=1e-2)


def test_verify_reference_far_below_row_max():
    """Scores that climb by far more than 2^128 after a split's first keys.

    Full (NoPE) layer with Q gain 16 and every query along one direction u;
    cached keys 0..31 point along -u (score -B) and key 100 along +u (score
    +B), with B = |q-hat| |k-hat| * scale * log2(e) ~ 261 in log2 units.  One
    split covers the 216 keys, so a reference taken from its first tile sits
    2B below the row maximum and exp2(s - ref) overflows f32: the kernel must
    notice and recompute the split with exact row maxima.  Every row then
    reduces to V[100] * sigmoid(gate) up to the weight of the random keys.
    """
    spec = synth.full(q_gain=16.0)
    B = spec.q_gain * spec.k_gain * 128 * spec.scale * np.log2(np.e)
    assert 2 * B > 300
    w, inp = _inputs(spec, [200], 16, config=95)
    gen = torch.Generator(device="cpu").manual_seed(2025)
    u = torch.randn(128, generator=gen, dtype=torch.float64)
    u = u / u.pow(2).mean().sqrt()                     # unit RMS, as a normed key row
    q = u.view(1, 1, 1, 128) + 0.05 * torch.randn(1, 16, 32, 128, generator=gen, dtype=torch.float64)
    inp.q.copy_(q.to(inp.q.dtype))
    ck = inp.cache_k.double().cpu()
    ck[0, :32] = -u
    ck[0, 100] = u
    inp.cache_k.copy_(ck.to(inp.cache_k.dtype))
    check_layer(w, spec, inp, decode=False)


@pytest.mark.parametrize("lens", [[40000], [3000, 2047, 100, 0]], ids=["one_seq_many_splits", "ragged"])
def test_verify_graph_replays_match_eager(lens):
    """A captured verify call (split kernel, then merge kernel) replays with new
    inputs copied in and eager work in between; every replay must equal the
    eager result on the same inputs, bit for bit."""
    spec = synth.full()
    N, L = 16, max(lens)
    w, inp = _inputs(spec, lens, N, config=96)
    lay = fa.make_layer(spec.kind, window=spec.window, rope_theta=spec.rope_theta, dtype=w.dtype)
    ws = fa.workspace(lay, len(lens), N, L, False)
    q, k, v, g = inp.q.clone(), inp.k.clone(), inp.v.clone(), inp.gate.clone()
    out = torch.empty_like(g)
    ck, cv = inp.cache_k.clone(), inp.cache_v.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                         # warm-up outside the capture
        fa.prefill(lay, q, k, v, g, ck, cv, inp.seq_len, out, max_seq_len=L, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.prefill(lay, q, k, v, g, ck, cv, inp.seq_len, out, max_seq_len=L, workspace=ws)
    for rep in range(3):
        new = synth.layer_inputs(w, spec, device=DEV, n_new=N, prefix=0, step=20 + rep, with_cache=False)
        q.copy_(new.q); k.copy_(new.k); v.copy_(new.v); g.copy_(new.gate)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = fa.prefill(lay, q, k, v, g, ck.clone(), cv.clone(), inp.seq_len, max_seq_len=L)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep}"

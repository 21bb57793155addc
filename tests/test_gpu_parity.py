"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, at sizes the oracle finishes in seconds that still span
several tiles and a ragged tail, plus the degenerate cases.

Tolerances are in tests/parity.py: 1e-4 absolute on the f32 path, 2e-2 +
1e-2 * |ref| on the bf16 path; appended V rows bit-exact, K rows within one
bf16 ulp of the oracle's rounded value.
"""
import numpy as np
import pytest
import torch

import full_gqa_attention_amd as fa
import oracle
from full_gqa_attention_amd import synth
from parity import check_layer as _check_layer, run_gpu, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _custom(name, dtype, S, Lmax, N, layers, config=90):
    return synth.Workload(name, config, dtype, S, Lmax, N, tuple(layers))


def _ragged_inputs(w, spec, seq_lens, N, capacity=None, step=0):
    Lmax = max(seq_lens)
    inp = synth.layer_inputs(w, spec, device=DEV, prefix=Lmax, n_new=N,
                             capacity=capacity or Lmax + N, step=step)
    inp.seq_len = torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    return inp


# ------------------------------------------------------------------ prefill

@pytest.mark.parametrize("li", [0, 1], ids=["sliding_w128", "full"])
def test_prefill_1x512_f32(li):
    """The 1 x 512 f32 workload at full size, every row (both layer kinds)."""
    w = synth.WORKLOADS["prefill_1x512_f32"]
    spec = w.layers[li]
    inp = synth.layer_inputs(w, spec, device=DEV)
    _check_layer(w, spec, inp, decode=False)


PREFILL_SPECS = [synth.sliding(64, 500000.0), synth.sliding(1, 500000.0), synth.sliding(300, 10000.0),
                 synth.full()]


@pytest.mark.parametrize("spec", PREFILL_SPECS, ids=["w64", "w1", "w300", "full"])
@pytest.mark.parametrize("seq_lens", [(0, 0, 0), (77, 0, 130)], ids=["fresh", "chunked"])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32], ids=["bf16", "f32"])
def test_prefill_ragged(spec, seq_lens, dtype):
    """3 sequences x 200 new tokens: two full 128-row query blocks and a
    ragged tail, several 64-key tiles, per-sequence prefixes."""
    w = _custom("ragged_prefill", dtype, 3, max(seq_lens), 200, [spec])
    inp = _ragged_inputs(w, spec, list(seq_lens), 200)
    _check_layer(w, spec, inp, decode=False)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32], ids=["bf16", "f32"])
def test_prefill_reference_far_below_row_max(dtype):
    """Scores that climb by far more than 2^128 after a row's first keys.

    Full (NoPE) layer with Q gain 16, every query along one direction u: keys
    0..31 point along -u (score -B), key 100 along +u (score +B), the rest are
    random; B = |q-hat| |k-hat| * scale * log2(e) = 16 * 128 * scale * log2(e)
    ~ 261 in log2 units.  A reference taken from a row's first keys sits 2B
    below its maximum, so exp2(s - ref) overflows f32: the kernel has to
    notice and redo those rows with the exact maxima.  Rows >= 100 reduce to
    V[100] * sigmoid(gate); rows 32..99 to a softmax over the random keys.
    """
    spec = synth.full(q_gain=16.0)
    B = spec.q_gain * spec.k_gain * 128 * spec.scale * np.log2(np.e)
    assert 2 * B > 300                                  # far beyond the f32 range of exp2
    N = 200
    w = _custom("overflow_prefill", dtype, 1, 0, N, [spec])
    inp = synth.layer_inputs(w, spec, device=DEV)
    gen = torch.Generator(device="cpu").manual_seed(2024)
    u = torch.randn(128, generator=gen, dtype=torch.float64)
    tdt = inp.q.dtype
    q = u.view(1, 1, 1, 128) + 0.05 * torch.randn(1, N, 32, 128, generator=gen, dtype=torch.float64)
    inp.q.copy_(q.to(tdt))
    k = inp.k.double().cpu()
    k[0, :32] = -u
    k[0, 100] = u
    inp.k.copy_(k.to(tdt))
    _check_layer(w, spec, inp, decode=False)


@pytest.mark.parametrize("N", [1, 2, 31, 129])
def test_prefill_tiny_chunks(N):
    spec = synth.sliding(16, 500000.0)
    w = _custom("tiny", synth.BF16, 2, 40, N, [spec])
    inp = _ragged_inputs(w, spec, [40, 3], N)
    _check_layer(w, spec, inp, decode=False)


# ------------------------------------------------------------------- decode

DECODE_SPECS = [synth.sliding(128, 500000.0), synth.sliding(1, 500000.0), synth.sliding(2048, 500000.0),
                synth.full()]


@pytest.mark.parametrize("spec", DECODE_SPECS, ids=["w128", "w1", "w2048", "full"])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32], ids=["bf16", "f32"])
def test_decode_ragged(spec, dtype):
    """Sequences of very different lengths (0 .. 3000 cached rows) in one call."""
    lens = [0, 1, 63, 64, 65, 1000, 2047, 3000]
    w = _custom("ragged_decode", dtype, len(lens), max(lens), 1, [spec])
    inp = _ragged_inputs(w, spec, lens, 1)
    _check_layer(w, spec, inp, decode=True)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("lens", [[40000, 9000, 7680], [60000]], ids=["3seq", "1seq"])
def test_decode_long_context_many_splits(dtype, lens):
    """Long contexts make many splits per (sequence, KV head), merged by the
    merge kernel 32 splits per round trip: three sequences of 40,000, 9,000
    and 7,680 cached rows (42 splits in two batches, fewer live in the
    shorter ones, whose last live split may be an even or an odd one), and
    one of 60,000 (126 splits in four batches: the (m, l) slots past 64 sit
    in a second register per lane)."""
    spec = synth.full()
    w = _custom("long_decode", dtype, len(lens), max(lens), 1, [spec])
    inp = _ragged_inputs(w, spec, lens, 1)
    _check_layer(w, spec, inp, decode=True)


@pytest.mark.parametrize("spec", [synth.sliding(100, 500000.0), synth.full()], ids=["w100", "full"])
def test_decode_equals_last_prefill_row(spec):
    """Cross-entry: decode at p reproduces row p of a (p+1)-token prefill."""
    T = 300
    w = _custom("cross", synth.BF16, 2, 0, T, [spec])
    full_inp = synth.layer_inputs(w, spec, device=DEV, prefix=0, n_new=T)
    mono = run_gpu(spec, w.dtype, full_inp, decode=False)
    # same tokens: prefill T-1, then decode the last one
    part = synth.LayerInputs(full_inp.q[:, :T - 1].contiguous(), full_inp.k[:, :T - 1].contiguous(),
                             full_inp.v[:, :T - 1].contiguous(), full_inp.gate[:, :T - 1].contiguous(),
                             torch.zeros_like(full_inp.cache_k), torch.zeros_like(full_inp.cache_v),
                             torch.zeros(2, dtype=torch.int32, device=DEV))
    run_gpu(spec, w.dtype, part, decode=False, max_seq_len=1)
    last = synth.LayerInputs(full_inp.q[:, T - 1:].contiguous(), full_inp.k[:, T - 1:].contiguous(),
                             full_inp.v[:, T - 1:].contiguous(), full_inp.gate[:, T - 1:].contiguous(),
                             part.cache_k, part.cache_v,
                             torch.full((2,), T - 1, dtype=torch.int32, device=DEV))
    dec = run_gpu(spec, w.dtype, last, decode=True)
    assert torch.equal(last.cache_k, full_inp.cache_k) and torch.equal(last.cache_v, full_inp.cache_v)
    a, b = to_f64(dec[:, 0]), to_f64(mono[:, T - 1])
    assert np.all(np.abs(a - b) <= 2e-2 + 1e-2 * np.abs(b))


def test_decode_split_count_invariance():
    """The split-K result does not depend on how many splits there are."""
    spec = synth.full()
    w = _custom("splits", synth.BF16, 3, 5000, 1, [spec])
    inp = _ragged_inputs(w, spec, [5000, 4000, 10], 1)
    outs = []
    for max_len in (5000, 6000, 20000):       # changes the split size
        inp2 = synth.LayerInputs(inp.q, inp.k, inp.v, inp.gate, inp.cache_k.clone(),
                                 inp.cache_v.clone(), inp.seq_len)
        lay = fa.make_layer(spec.kind, dtype=w.dtype)
        cap = max_len + 1
        ck = torch.zeros((3, cap, 2, 128), dtype=torch.bfloat16, device=DEV)
        cv = torch.zeros_like(ck)
        ck[:, :inp.cache_k.shape[1]] = inp2.cache_k
        cv[:, :inp.cache_v.shape[1]] = inp2.cache_v
        out = fa.decode(lay, inp.q, inp.k, inp.v, inp.gate, ck, cv, inp.seq_len, max_seq_len=max_len)
        outs.append(to_f64(out))
    for o in outs[1:]:
        assert np.all(np.abs(o - outs[0]) <= 1e-2 + 5e-3 * np.abs(outs[0]))


# ------------------------------------------------------ edge and error cases

def test_deterministic_repeat():
    spec = synth.sliding(64, 500000.0)
    w = _custom("det", synth.BF16, 2, 500, 1, [spec])
    inp = _ragged_inputs(w, spec, [500, 320], 1)
    a = run_gpu(spec, w.dtype, inp, True).clone()
    b = run_gpu(spec, w.dtype, inp, True).clone()
    assert torch.equal(a, b)
    wp = _custom("detp", synth.BF16, 2, 0, 150, [spec])
    inp = _ragged_inputs(wp, spec, [0, 0], 150)
    a = run_gpu(spec, wp.dtype, inp, False).clone()
    b = run_gpu(spec, wp.dtype, inp, False).clone()
    assert torch.equal(a, b)


@pytest.mark.parametrize("decode", [False, True])
def test_device_side_bad_seq_len_is_refused(decode):
    """seq_len above max_seq_len (the host cannot see it): that sequence's
    output is NaN and its cache untouched; the others are computed."""
    spec = synth.sliding(64, 500000.0)
    N = 1 if decode else 50
    w = _custom("bad_len", synth.BF16, 3, 100, N, [spec])
    inp = _ragged_inputs(w, spec, [100, 100, 40], N, capacity=100 + N + 10)
    inp.seq_len[1] = 100 + 7                        # > max_seq_len = 100
    before_k = inp.cache_k.clone()
    out = run_gpu(spec, w.dtype, inp, decode, max_seq_len=100)
    assert torch.isnan(out[1].float()).all()
    assert torch.equal(inp.cache_k[1], before_k[1])
    assert torch.isfinite(out[0].float()).all() and torch.isfinite(out[2].float()).all()
    inp.seq_len[1] = -3                             # negative
    out = run_gpu(spec, w.dtype, inp, decode, max_seq_len=100)
    assert torch.isnan(out[1].float()).all()


def test_empty_inputs():
    lay = fa.make_layer(fa.FULL_NOPE, dtype=fa.BF16)
    S = 2
    q = torch.empty((S, 0, 32, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((S, 0, 2, 128), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((S, 0, 4096), dtype=torch.bfloat16, device=DEV)
    ck = torch.zeros((S, 8, 2, 128), dtype=torch.bfloat16, device=DEV)
    cv = torch.zeros_like(ck)
    out = fa.prefill(lay, q, k, k, g, ck, cv, torch.zeros(S, dtype=torch.int32, device=DEV),
                     workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert out.shape == (S, 0, 4096)
    assert torch.count_nonzero(ck) == 0


def test_decode_workspace_reuse_and_garbage():
    """A workspace full of random bytes, reused across calls of different
    batch sizes, gives the same results as a fresh one: the merge reads every
    partial slot of a call but uses only the live splits' (the slots of a
    shorter sequence's missing splits hold whatever was there)."""
    spec = synth.full()
    w = _custom("ws", synth.BF16, 6, 3000, 1, [spec])
    inp = _ragged_inputs(w, spec, [3000, 2500, 100, 3000, 1, 2048], 1)
    lay = fa.make_layer(spec.kind, dtype=w.dtype)

    def call(n_seq, ws=None):
        return fa.decode(lay, inp.q[:n_seq], inp.k[:n_seq], inp.v[:n_seq], inp.gate[:n_seq],
                         inp.cache_k[:n_seq].clone(), inp.cache_v[:n_seq].clone(), inp.seq_len[:n_seq],
                         max_seq_len=3000, workspace=ws).clone()

    fresh = {n: call(n) for n in (6, 3, 1)}          # the split count depends on the batch
    n = max(fa.workspace_size(lay, k, 1, 3000, True) for k in (6, 3, 1))
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
    for n_seq in (6, 3, 6, 1, 6, 3):
        out = call(n_seq, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, fresh[n_seq])


@pytest.mark.parametrize("spec", [synth.sliding(2048, 500000.0), synth.full()], ids=["w2048", "full"])
def test_decode_graph_replays_match_eager(spec):
    """A captured decode call (split kernel, then merge kernel) replays with
    new inputs copied in and eager work in between; every replay must equal
    the eager result on the same inputs."""
    S, L = 4, 5000
    w = _custom("graph", synth.BF16, S, L, 1, [spec])
    inp = _ragged_inputs(w, spec, [L, 4000, 2999, 17], 1)
    lay = fa.make_layer(spec.kind, window=spec.window, rope_theta=spec.rope_theta, dtype=w.dtype)
    ws = fa.workspace(lay, S, 1, L, True)
    q, k, v, g = inp.q.clone(), inp.k.clone(), inp.v.clone(), inp.gate.clone()
    out = torch.empty_like(g)
    ck, cv = inp.cache_k.clone(), inp.cache_v.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm-up outside the capture
        fa.decode(lay, q, k, v, g, ck, cv, inp.seq_len, out, max_seq_len=L, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.decode(lay, q, k, v, g, ck, cv, inp.seq_len, out, max_seq_len=L, workspace=ws)
    for rep in range(4):
        new = synth.layer_inputs(w, spec, device=DEV, n_new=1, prefix=0, step=10 + rep, with_cache=False)
        q.copy_(new.q); k.copy_(new.k); v.copy_(new.v); g.copy_(new.gate)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = fa.decode(lay, q, k, v, g, ck.clone(), cv.clone(), inp.seq_len, max_seq_len=L)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep}"

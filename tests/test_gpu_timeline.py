"""The profiling build (libmuse_attn_timeline.so): its decode kernels give the
same bits as the regular library's, and the per-workgroup phase records it
keeps are consistent (every phase after the previous one, the merge kernel
starting after the last split workgroup's stores completed, on one clock).

The records are only read here; the phase times themselves are reported by
`bench.py --decode-timeline`."""
import numpy as np
import pytest
import torch

import full_gqa_attention_amd as fa
from full_gqa_attention_amd import synth

pytestmark = pytest.mark.gpu


def _decode_case(spec, n_seq, prefix, dtype=synth.BF16, dev="cuda:0"):
    w = synth.Workload("timeline", 41, dtype, n_seq, prefix, 1, (spec,))
    inp = synth.layer_inputs(w, spec, device=dev, backend="torch", n_new=1, capacity=prefix + 1)
    lay = fa.make_layer(spec.kind, window=spec.window, rope_theta=spec.rope_theta, dtype=w.dtype)
    return lay, inp


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_timeline_build_matches_regular_build(kind, dtype):
    spec = synth.sliding(2048, 500000.0) if kind == "sliding" else synth.full()
    n_seq, prefix = 4, 6000
    lay, inp = _decode_case(spec, n_seq, prefix, dtype)
    print(f"timeline: {kind} decode S={n_seq} at position {prefix} (dtype {dtype}), regular then profiling build",
          flush=True)
    ck0, cv0 = inp.cache_k.clone(), inp.cache_v.clone()
    out_a = fa.decode(lay, inp.q, inp.k, inp.v, inp.gate, inp.cache_k, inp.cache_v, inp.seq_len)
    torch.cuda.synchronize()
    ck_a, cv_a = inp.cache_k.clone(), inp.cache_v.clone()
    saved = (fa._lib, fa.LIB_PATH)
    try:
        fa.use_timeline_library()
        fa.decode_timeline_read(clear=True)
        inp.cache_k.copy_(ck0)
        inp.cache_v.copy_(cv0)
        out_b = fa.decode(lay, inp.q, inp.k, inp.v, inp.gate, inp.cache_k, inp.cache_v, inp.seq_len)
        torch.cuda.synchronize()
        split, merge = fa.decode_timeline_read(clear=True)
    finally:
        fa._lib, fa.LIB_PATH = saved
    bits = torch.int16 if dtype == synth.BF16 else torch.int32
    assert torch.equal(out_a.view(bits), out_b.view(bits))
    assert torch.equal(ck_a.view(bits), inp.cache_k.view(bits))
    assert torch.equal(cv_a.view(bits), inp.cache_v.view(bits))
    d = split[split[:, 6] > 0]
    assert len(d) >= 2 * n_seq, len(d)                 # at least one split per (sequence, KV head)
    assert np.all(np.diff(d[:, :7], axis=1) >= 0)
    assert np.all(d[:, 7] >= 1)
    m = merge[merge[:, 2] > 0]
    assert len(m) == n_seq * 32                        # one merge workgroup per (sequence, head)
    assert np.all(m[:, 1] >= m[:, 0]) and np.all(m[:, 2] >= m[:, 1])
    assert m[:, 0].min() >= d[:, 6].max()              # the merge launch follows every split's stores
    assert np.all(m[:, 3] > 1)

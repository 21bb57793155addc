"""The allocation-free decode entry point (muse_attn_decode_noalloc) against
the existing one (muse_attn_decode with a caller workspace), through the C
ABI: two calls in a row, the second with a smaller batch, so the second
finds the first call's partials in the library's static scratch.  The same
kernels run in both, so outputs and appended cache rows must be identical
(which meets the parity bar of the existing entry point a fortiori)."""
import numpy as np
import pytest
import torch

import full_gqa_attention_amd as fa
from full_gqa_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(S, L, spec, step):
    w = synth.Workload("noalloc", 77, synth.BF16, S, L, 1, (spec,))
    inp = synth.layer_inputs(w, spec, device=DEV, backend="torch", step=step)
    lens = torch.tensor([L - 37 * i for i in range(S)], dtype=torch.int32, device=DEV)   # ragged
    inp.seq_len = lens.clamp(min=1)
    lay = fa.make_layer(spec.kind, window=spec.window, rope_theta=spec.rope_theta, dtype=synth.BF16)
    return inp, lay


@pytest.mark.parametrize("spec", [synth.sliding(2048, 500000.0), synth.full()], ids=["sliding", "full"])
def test_noalloc_matches_decode_twice(spec):
    for S, L, step in ((8, 20000, 1), (2, 900, 2)):           # the second call is smaller
        print(f"noalloc decode: {spec.name} S={S} L={L}", flush=True)
        inp, lay = _case(S, L, spec, step)
        ck1, cv1 = inp.cache_k.clone(), inp.cache_v.clone()
        ck2, cv2 = inp.cache_k.clone(), inp.cache_v.clone()
        assert fa.workspace_size(lay, S, 1, L, True) > 0      # the calls split, so the scratch is used
        ref = fa.decode(lay, inp.q, inp.k, inp.v, inp.gate, ck1, cv1, inp.seq_len, max_seq_len=L)
        got = fa.decode_noalloc(lay, inp.q, inp.k, inp.v, inp.gate, ck2, cv2, inp.seq_len, max_seq_len=L)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert torch.equal(ck2, ck1) and torch.equal(cv2, cv1)
        assert torch.isfinite(got.float()).all()

"""NoPE rows are position-free, so they relocate by a byte copy ("Chapter 14 -
QK-norm and RoPE" 14.6; "How Muse Glimmer Fits an Agent on Your Device",
section "Global attention without RoPE").

A 512-token chunk prefilled at position 0 leaves the same K and V bytes as
the same chunk prefilled after a 1,024-row prefix (on a full layer; on a
sliding layer the K rows differ, rotated by their positions).  Copying the
first tile into the second cache's place with muse_kv_relocate therefore
gives a cache -- and a decode over it -- identical to recomputing it.
"""
import pytest
import torch

import full_gqa_attention_amd as fa
from full_gqa_attention_amd import synth
from parity import lib_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = 512          # the engine's NoPE tile


def _chunk(spec, L):
    """One sequence: a T-token chunk (the same tokens for every L) after L
    cached rows, prefilled; returns the caches (capacity L + T + 1)."""
    w = synth.Workload("relocate", 92, synth.BF16, 1, L, T, (spec,))
    inp = synth.layer_inputs(w, spec, device=DEV, prefix=L, n_new=T, capacity=L + T + 1)
    chunk = synth.layer_inputs(synth.Workload("relocate", 92, synth.BF16, 1, 0, T, (spec,)), spec,
                               device=DEV, prefix=0, n_new=T, capacity=T)
    seq = torch.tensor([L], dtype=torch.int32, device=DEV)
    fa.prefill(lib_layer(spec, synth.BF16), chunk.q, chunk.k, chunk.v, chunk.gate,
               inp.cache_k, inp.cache_v, seq, max_seq_len=L)
    torch.cuda.synchronize()
    return inp.cache_k, inp.cache_v


def test_nope_rows_are_position_free_and_sliding_rows_are_not():
    a_k, a_v = _chunk(synth.full(), 0)
    b_k, b_v = _chunk(synth.full(), 1024)
    assert torch.equal(a_k[0, :T], b_k[0, 1024:1024 + T]) and torch.equal(a_v[0, :T], b_v[0, 1024:1024 + T])
    s_spec = synth.sliding(2048, 500000.0)
    c_k, c_v = _chunk(s_spec, 0)
    d_k, d_v = _chunk(s_spec, 1024)
    assert torch.equal(c_v[0, :T], d_v[0, 1024:1024 + T])       # V never rotates
    assert not torch.equal(c_k[0, :T], d_k[0, 1024:1024 + T])   # K rotated by its position


def test_relocated_tile_equals_recomputed_cache_and_decode():
    spec = synth.full()
    lay = lib_layer(spec, synth.BF16)
    a_k, a_v = _chunk(spec, 0)                    # the chunk computed at positions 0..511
    b_k, b_v = _chunk(spec, 1024)                 # ... and at 1024..1535 after a prefix
    c_k, c_v = b_k.clone(), b_v.clone()
    c_k[0, 1024:1024 + T] = 0                     # forget the recomputed tile
    c_v[0, 1024:1024 + T] = 0
    fa.kv_relocate(lay, a_k, a_v, c_k, c_v, [(0, 0, 0, 1024, T)])
    torch.cuda.synchronize()
    assert torch.equal(c_k, b_k) and torch.equal(c_v, b_v)
    # a decode step over either cache is bit-identical
    w = synth.Workload("relocate_dec", 93, synth.BF16, 1, 1024 + T, 1, (spec,))
    d = synth.layer_inputs(w, spec, device=DEV, n_new=1, prefix=0, with_cache=False)
    seq = torch.tensor([1024 + T], dtype=torch.int32, device=DEV)
    o1 = fa.decode(lay, d.q, d.k, d.v, d.gate, b_k, b_v, seq, max_seq_len=1024 + T)
    o2 = fa.decode(lay, d.q, d.k, d.v, d.gate, c_k, c_v, seq, max_seq_len=1024 + T)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_relocate_tiles_in_order_within_one_cache():
    spec = synth.full()
    lay = lib_layer(spec, synth.BF16)
    g = torch.Generator(device="cpu").manual_seed(7)
    k = torch.randn((3, 2048, 2, 128), generator=g).to(DEV, torch.bfloat16)
    v = torch.randn((3, 2048, 2, 128), generator=g).to(DEV, torch.bfloat16)
    k0, v0 = k.clone(), v.clone()
    # tile 1 moves rows of sequence 0 to sequence 2; tile 2 then moves the
    # moved rows on again; the empty tile is skipped
    fa.kv_relocate(lay, k, v, k, v, [(0, 100, 2, 700, 300), (2, 700, 1, 0, 300), (1, 5, 2, 5, 0)])
    torch.cuda.synchronize()
    want_k, want_v = k0.clone(), v0.clone()
    want_k[2, 700:1000] = k0[0, 100:400]
    want_v[2, 700:1000] = v0[0, 100:400]
    want_k[1, 0:300] = k0[0, 100:400]
    want_v[1, 0:300] = v0[0, 100:400]
    assert torch.equal(k, want_k) and torch.equal(v, want_v)


def test_relocate_refuses_sliding_layers():
    spec = synth.sliding(2048, 500000.0)
    k = torch.zeros((1, 1024, 2, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa.MuseError):
        fa.kv_relocate(lib_layer(spec, synth.BF16), k, k.clone(), k.clone(), k.clone(), [(0, 0, 0, 512, 512)])


def test_relocate_many_tiles_applies_in_order():
    """More tiles than one launch holds, some reading rows earlier tiles wrote."""
    spec = synth.full()
    lay = lib_layer(spec, synth.BF16)
    g = torch.Generator(device="cpu").manual_seed(11)
    S, cap = 6, 3000
    k = torch.randn((S, cap, 2, 128), generator=g).to(DEV, torch.bfloat16)
    v = torch.randn((S, cap, 2, 128), generator=g).to(DEV, torch.bfloat16)
    rng = torch.Generator(device="cpu").manual_seed(12)
    tiles = []
    for _ in range(130):
        n = int(torch.randint(0, 300, (1,), generator=rng))
        ss, ds = (int(x) for x in torch.randint(0, S, (2,), generator=rng))
        sp, dp = (int(x) for x in torch.randint(0, cap - n + 1, (2,), generator=rng))
        if ss == ds and sp < dp + n and dp < sp + n:
            continue                      # a tile may not overlap itself
        tiles.append((ss, sp, ds, dp, n))
    want_k, want_v = k.clone(), v.clone()
    for ss, sp, ds, dp, n in tiles:       # the same tiles, one after another
        want_k[ds, dp:dp + n] = want_k[ss, sp:sp + n].clone()
        want_v[ds, dp:dp + n] = want_v[ss, sp:sp + n].clone()
    fa.kv_relocate(lay, k, v, k, v, tiles)
    torch.cuda.synchronize()
    assert torch.equal(k, want_k) and torch.equal(v, want_v)

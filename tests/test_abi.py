"""C-ABI tests that need no GPU: the library loads, exports every function the
header declares, refuses bad arguments with the documented status codes
before enqueueing anything, and its host helpers agree with the oracle.

Every call below carries at least one violation, so none reaches a kernel
launch; the pointers are fake addresses that are never dereferenced.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import full_gqa_attention_amd as fa
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muse_attn.h")

OK, NULL, SHAPE, LAYER, CAPACITY, WORKSPACE, DTYPE, HIP, ALIGN, ALIAS = range(10)


@pytest.fixture(scope="module")
def lib():
    return fa.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muse_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = header_functions()
    assert set(names) == set(fa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_timeline_build_exports():
    """The profiling build exports muse_attn.h's functions and its own
    (include/muse_attn_timeline.h); the regular build does not export the
    latter."""
    tl_header = os.path.join(ROOT, "include", "muse_attn_timeline.h")
    text = re.sub(r"/\*.*?\*/", "", open(tl_header).read(), flags=re.S)
    tl_names = sorted(set(re.findall(r"\b(muse_[a-z_0-9]+)\s*\(", text)))
    assert tl_names == sorted(fa.TIMELINE_EXPORTS)
    tl = ctypes.CDLL(fa.TIMELINE_LIB_PATH)
    for n in header_functions() + tl_names:
        assert hasattr(tl, n), n
    regular = ctypes.CDLL(fa.LIB_PATH)
    for n in tl_names:
        assert not hasattr(regular, n), n


def test_status_strings(lib):
    for code in range(10):
        assert fa.status_str(code).startswith(fa.STATUS[code])
    assert fa.status_str(99) == "unknown muse_status"


def test_layer_kind_rule_and_init():
    full = [l for l in range(52) if fa.layer_kind_for(l) == fa.FULL_NOPE]
    assert full == list(range(3, 52, 4))
    assert fa.layer_kind_for(52) == -1 and fa.layer_kind_for(-1) == -1
    assert fa.layer_kind_for(3, 0) == -1
    for l in range(52):
        assert fa.layer_kind_for(l) == oracle.layer_kind(l)
        lay = fa.layer_init(l, fa.BF16)
        assert (lay.n_heads, lay.n_kv_heads, lay.head_dim) == (32, 2, 128)
        assert lay.kind == fa.layer_kind_for(l)
        if lay.kind == fa.FULL_NOPE:
            assert lay.window == 0 and lay.rope_theta == 0.0
        else:
            assert lay.window == 2048 and lay.rope_theta == 500000.0
        assert lay.attn_scale == np.float32(1 / math.sqrt(128))
        assert round(lay.attn_scale, 7) == 0.0883883
        assert lay.q_norm_gain == np.float32(3.87) and lay.k_norm_gain == 1.0
        assert lay.rms_eps == np.float32(1e-5)
    with pytest.raises(fa.MuseError):
        fa.layer_init(52)
    with pytest.raises(fa.MuseError):
        fa.layer_init(0, 7)


@pytest.mark.parametrize("theta", [10000.0, 500000.0, 1e6, 2.5])
def test_rope_table_matches_oracle_bitwise(theta):
    got = np.array(fa.rope_theta_table(theta), dtype=np.float32)
    want = oracle.rope_theta_table(theta)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_rope_table_rejects_bad_theta():
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(fa.MuseError) as e:
            fa.rope_theta_table(bad)
        assert e.value.code == LAYER


# --------------------------------------------------------- validation

BASE = 0x7F0000000000   # fake, 256-aligned addresses, never dereferenced
MB = 1 << 20


class Fake:
    """A full set of argument values for one call, each buffer in its own range."""

    def __init__(self, decode=False, dtype=fa.BF16, kind=fa.SLIDING_ROPE):
        self.layer = fa.make_layer(kind, window=2048 if kind == fa.SLIDING_ROPE else 0,
                                   rope_theta=500000.0 if kind == fa.SLIDING_ROPE else 0.0,
                                   dtype=dtype)
        self.decode = decode
        self.n_seq, self.n_new, self.max_seq_len = 4, 1 if decode else 64, 100
        self.cap = 256
        addrs = iter(range(BASE, BASE + 64 * 512 * MB, 512 * MB))
        self.seq_len, self.q, self.k, self.v, self.gate, self.out, self.ws = (next(addrs) for _ in range(7))
        self.cache = fa.KvCache(next(addrs), next(addrs), self.cap)
        self.ws_bytes = 1 << 28
        self.timer = None

    def call(self, lib):
        vp = ctypes.c_void_p
        c = ctypes.byref(self.cache) if self.cache is not None else None
        lay = ctypes.byref(self.layer) if self.layer is not None else None
        t = ctypes.byref(self.timer) if self.timer is not None else None
        if self.decode:
            return lib.muse_attn_decode(lay, self.n_seq, vp(self.seq_len), self.max_seq_len,
                                        vp(self.q), vp(self.k), vp(self.v), vp(self.gate), c,
                                        vp(self.out), vp(self.ws), self.ws_bytes, None, t)
        return lib.muse_attn_prefill(lay, self.n_seq, self.n_new, vp(self.seq_len), self.max_seq_len,
                                     vp(self.q), vp(self.k), vp(self.v), vp(self.gate), c,
                                     vp(self.out), vp(self.ws), self.ws_bytes, None, t)


def _mut(attr, value):
    def f(x):
        setattr(x, attr, value)
    return f


def _long_prefix(x):
    """A prefix long enough that the call needs a workspace (several decode splits)."""
    x.max_seq_len = 600
    x.cache.capacity = 1024


def _lay(attr, value):
    def f(x):
        setattr(x.layer, attr, value)
    return f


CASES = [
    ("layer NULL", _mut("layer", None), NULL),
    ("n_heads 16", _lay("n_heads", 16), SHAPE),
    ("n_kv_heads 4", _lay("n_kv_heads", 4), SHAPE),
    ("head_dim 64", _lay("head_dim", 64), SHAPE),
    ("dtype 5", _lay("dtype", 5), DTYPE),
    ("kind 7", _lay("kind", 7), LAYER),
    ("sliding window 0", _lay("window", 0), LAYER),
    ("sliding theta 0", _lay("rope_theta", 0.0), LAYER),
    ("sliding theta nan", _lay("rope_theta", float("nan")), LAYER),
    ("sliding theta inf", _lay("rope_theta", float("inf")), LAYER),
    ("eps 0", _lay("rms_eps", 0.0), LAYER),
    ("scale negative", _lay("attn_scale", -0.1), LAYER),
    ("q gain inf", _lay("q_norm_gain", float("inf")), LAYER),
    ("k gain nan", _lay("k_norm_gain", float("nan")), LAYER),
    ("q gain above fp16-safe bound", _lay("q_norm_gain", 4097.0), LAYER),
    ("k gain below -4096", _lay("k_norm_gain", -5000.0), LAYER),
    ("n_seq negative", _mut("n_seq", -1), SHAPE),
    ("max_seq_len negative", _mut("max_seq_len", -1), SHAPE),
    ("max_seq_len beyond f32-exact positions", _mut("max_seq_len", 1 << 24), SHAPE),
    ("capacity too small", _mut("max_seq_len", 256), CAPACITY),
    ("cache NULL", _mut("cache", None), NULL),
    ("q NULL", _mut("q", 0), NULL),
    ("gate NULL", _mut("gate", 0), NULL),
    ("seq_len NULL", _mut("seq_len", 0), NULL),
    ("workspace NULL", lambda x: (_long_prefix(x), setattr(x, "ws", 0)), NULL),
    ("workspace too small", lambda x: (_long_prefix(x), setattr(x, "ws_bytes", 1024)), WORKSPACE),
    ("q misaligned", _mut("q", BASE + 512 * MB * 1 + 8), ALIGN),
    ("out overlaps q", _mut("out", BASE + 512 * MB * 1 + 4096), ALIAS),
    ("workspace overlaps cache k", _mut("ws", BASE + 512 * MB * 7 + 4096), ALIAS),
]


@pytest.mark.parametrize("decode", [False, True])
@pytest.mark.parametrize("name,mutate,code", CASES, ids=[c[0] for c in CASES])
def test_validation_fails_closed(lib, name, mutate, code, decode):
    assert code != 0                 # fake pointers: every case must stop before a launch
    f = Fake(decode=decode)
    mutate(f)
    assert f.call(lib) == code


@pytest.mark.parametrize("decode", [False, True])
def test_validation_layer_kinds(lib, decode):
    f = Fake(decode=decode, kind=fa.FULL_NOPE)
    f.layer.window = 2048            # a full layer must not carry a window
    assert f.call(lib) == LAYER
    f = Fake(decode=decode, kind=fa.FULL_NOPE)
    f.layer.rope_theta = 500000.0    # nor a RoPE base
    assert f.call(lib) == LAYER
    f = Fake(decode=decode)
    f.cache = fa.KvCache(f.cache.k, f.cache.k, f.cap)   # K and V caches alias
    assert f.call(lib) == ALIAS
    f = Fake(decode=decode)
    f.cache.v = 0
    assert f.call(lib) == NULL
    f = Fake(decode=decode)
    f.timer = fa.KernelTimer(None, None)
    assert f.call(lib) == NULL


@pytest.mark.parametrize("decode", [False, True])
def test_validation_ring(lib, decode):
    """kv_ring: sliding bf16 layers only; the ring needs min(window,
    max_seq_len + n_new) rows, a linear cache every position."""
    for kind, dtype, ring in ((fa.FULL_NOPE, fa.BF16, 1), (fa.SLIDING_ROPE, fa.F32, 1),
                              (fa.SLIDING_ROPE, fa.BF16, 2), (fa.SLIDING_ROPE, fa.BF16, -1)):
        f = Fake(decode=decode, kind=kind, dtype=dtype)
        f.layer.kv_ring = ring
        assert f.call(lib) == LAYER, (kind, dtype, ring)
    # a ring of window - 1 rows cannot hold the window once positions pass it
    f = Fake(decode=decode)
    f.layer.kv_ring = 1
    f.cache.capacity = 2047
    f.max_seq_len = 10000
    f.ws = 0                         # would be NULL -- but the capacity check comes first
    assert f.call(lib) == CAPACITY
    # ... and the same cache without the ring cannot hold the positions either
    f = Fake(decode=decode)
    f.cache.capacity = 2048
    f.max_seq_len = 10000
    assert f.call(lib) == CAPACITY
    # short sequences need only their positions, even on a ring layer
    f = Fake(decode=decode)
    f.layer.kv_ring = 1
    f.cache.capacity = 700           # under the window, over the 600 + 64 positions
    f.max_seq_len = 600
    f.ws = 0
    assert f.call(lib) == NULL       # passes the capacity check, stops at the NULL workspace


def _relocate(lib, layer, tiles, n_src=2, n_dst=2, cap=1024, same=False, null_tiles=False):
    src = fa.KvCache(BASE, BASE + 512 * MB, cap)
    dst = src if same else fa.KvCache(BASE + 1024 * MB, BASE + 1536 * MB, cap)
    arr = (fa.KvTile * max(1, len(tiles)))(*[fa.KvTile(ss, ds, sp, dp, n) for ss, sp, ds, dp, n in tiles])
    return lib.muse_kv_relocate(ctypes.byref(layer), ctypes.byref(src), n_src, ctypes.byref(dst), n_dst,
                                None if null_tiles else arr, len(tiles), None)


def test_relocate_validation(lib):
    """NoPE rows only ("Chapter 14 - QK-norm and RoPE" 14.6), every tile checked
    before anything is copied.  The addresses are fake: none of these copies."""
    full = fa.make_layer(fa.FULL_NOPE, window=0, rope_theta=0.0, dtype=fa.BF16)
    sliding = fa.make_layer(fa.SLIDING_ROPE, window=2048, rope_theta=5e5, dtype=fa.BF16)
    good = (0, 0, 1, 512, 512)
    assert _relocate(lib, sliding, [good]) == LAYER
    assert _relocate(lib, full, []) == OK                       # nothing to copy
    assert _relocate(lib, full, [good], n_src=0) == SHAPE
    assert _relocate(lib, full, [good, (2, 0, 0, 0, 1)]) == SHAPE   # sequence 2 of 2
    assert _relocate(lib, full, [(0, -1, 0, 0, 1)]) == SHAPE
    assert _relocate(lib, full, [(0, 0, 0, 0, -5)]) == SHAPE
    assert _relocate(lib, full, [good, (0, 600, 1, 0, 512)]) == CAPACITY   # rows 600..1111 of 1024
    assert _relocate(lib, full, [(0, 0, 0, 256, 512)], same=True) == ALIAS    # overlapping rows
    assert _relocate(lib, full, [good], null_tiles=True) == NULL
    bad_theta = fa.make_layer(fa.FULL_NOPE, window=0, rope_theta=0.0, dtype=fa.BF16)
    bad_theta.rope_theta = 10000.0                              # a NoPE layer cannot carry a RoPE base
    assert _relocate(lib, bad_theta, [good]) == LAYER


def test_empty_batches_are_valid_noops(lib):
    f = Fake()
    f.n_seq = 0
    assert f.call(lib) == OK
    f = Fake()
    f.n_new = 0
    assert f.call(lib) == OK
    f = Fake(decode=True)
    f.n_seq = 0
    assert f.call(lib) == OK


def test_workspace_sizes():
    lay = fa.make_layer(fa.FULL_NOPE, dtype=fa.BF16)
    # bf16 prefill: an fp16 copy of the keys the chunk can see (Q-hat is made in
    # the attention kernel); f32 prefill: Q-hat
    assert fa.workspace_size(lay, 8, 8192, 0, False) == 8 * 8192 * 256 * 2
    assert fa.workspace_size(lay, 4, 4096, 32768, False) == 4 * 36864 * 256 * 2
    # sliding bf16 layers copy only the window's keys (the window - 1 prefix rows, from a
    # start rounded down to 64 rows, + the chunk); ring layers copy the same rows of V too
    sl16 = fa.make_layer(fa.SLIDING_ROPE, window=2048, rope_theta=5e5, dtype=fa.BF16)
    assert fa.workspace_size(sl16, 4, 4096, 32768, False) == 4 * (2047 + 63 + 4096) * 256 * 2
    assert fa.workspace_size(sl16, 4, 4096, 100, False) == 4 * (100 + 4096) * 256 * 2
    ring = fa.make_layer(fa.SLIDING_ROPE, window=2048, rope_theta=5e5, dtype=fa.BF16, kv_ring=1)
    assert fa.workspace_size(ring, 4, 4096, 32768, False) == 2 * 4 * (2047 + 63 + 4096) * 256 * 2
    f32 = fa.make_layer(fa.FULL_NOPE, dtype=fa.F32)
    assert fa.workspace_size(f32, 1, 512, 0, False) == 512 * 4096 * 4
    d1 = fa.workspace_size(lay, 64, 1, 8192, True)
    d2 = fa.workspace_size(lay, 64, 1, 131072, True)
    assert 64 * 4096 * 2 < d1 <= d2
    sl = fa.make_layer(fa.SLIDING_ROPE, window=2048, rope_theta=5e5, dtype=fa.BF16)
    # a sliding layer's split depends on the window, not the context
    assert fa.workspace_size(sl, 16, 1, 131072, True) == fa.workspace_size(sl, 16, 1, 4096, True)
    with pytest.raises(fa.MuseError):
        fa.workspace_size(lay, -1, 1, 10, True)


# ---------------------------------------------- the block's tail: muse_out_proj

def _op_call(lib, n=4, attn=0x10000, w=0x20000000, gamma=0x40000000, res=0x50000000, out=0x60000000,
             eps=1e-8, ws=0x70000000, ws_bytes=None):
    """Fake 16-byte-aligned device addresses, far apart: every check runs on
    the host before anything is enqueued, so no pointer is dereferenced."""
    vp = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = fa.out_proj_workspace_size(n) if 0 <= n <= (1 << 24) else 0
    return lib.muse_out_proj(n, vp(attn) if attn else None, vp(w) if w else None, vp(gamma) if gamma else None,
                             vp(res) if res else None, vp(out) if out else None, ctypes.c_float(eps),
                             vp(ws) if ws else None, ws_bytes, None, None)


def test_out_proj_workspace_size():
    assert fa.out_proj_workspace_size(0) == 0
    assert fa.out_proj_workspace_size(64) == 8 * 64 * 6656 * 4
    assert fa.out_proj_workspace_size(65) == 65 * 6656 * 4
    assert fa.out_proj_workspace_size(65536) == 65536 * 6656 * 4
    with pytest.raises(fa.MuseError):
        fa.out_proj_workspace_size(-1)
    with pytest.raises(fa.MuseError):
        fa.out_proj_workspace_size((1 << 24) + 1)


@pytest.mark.parametrize("kw, code", [
    ({"attn": 0}, 1), ({"w": 0}, 1), ({"gamma": 0}, 1), ({"res": 0}, 1), ({"out": 0}, 1), ({"ws": 0}, 1),
    ({"n": -1}, 2), ({"n": (1 << 24) + 1}, 2),
    ({"eps": 0.0}, 3), ({"eps": -1e-8}, 3), ({"eps": float("inf")}, 3), ({"eps": float("nan")}, 3),
    ({"attn": 0x10008}, 8), ({"w": 0x20000004}, 8), ({"gamma": 0x40000002}, 8), ({"out": 0x60000008}, 8),
    ({"ws": 0x70000001}, 8),
    ({"ws_bytes": 4 * 6656 * 4 - 1}, 5),
    ({"out": 0x50000000 + 16}, 9),                  # partly over the residual
    ({"out": 0x10000}, 9),                          # over attn
    ({"ws": 0x20000000 + 4096}, 9),                 # workspace over w
    ({"ws": 0x60000000}, 9),                        # workspace over out
])
def test_out_proj_fails_closed(lib, kw, code):
    assert _op_call(lib, **kw) == code


def test_out_proj_in_place_residual_and_empty(lib):
    assert _op_call(lib, n=0) == OK                 # nothing enqueued
    # out == residual is the in-place stream update (validated, then nothing
    # enqueued for n == 0; with n > 0 the launch needs a GPU)
    assert _op_call(lib, n=0, out=0x50000000) == OK


def test_decode_workspace_zero_for_one_split(lib):
    """A decode whose keys fit one split per (sequence, KV head) needs no
    workspace (the header allows a NULL workspace then); a longer one does."""
    lay = fa.make_layer(fa.FULL_NOPE, dtype=fa.BF16)
    n = ctypes.c_size_t()
    assert lib.muse_attn_workspace_size(ctypes.byref(lay), 4, 1, 100, 1, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.muse_attn_workspace_size(ctypes.byref(lay), 4, 1, 8192, 1, ctypes.byref(n)) == 0
    assert n.value > 0


def test_decode_noalloc_refuses_beyond_its_scratch(lib):
    """The allocation-free decode keeps its split partials in a 4 MiB static
    array: a call needing more (127 sequences, 2 splits each: 4.23 MB) is
    refused before anything is enqueued; 126 sequences would fit."""
    lay = fa.make_layer(fa.FULL_NOPE, dtype=fa.BF16)
    n = ctypes.c_size_t()
    assert lib.muse_attn_workspace_size(ctypes.byref(lay), 127, 1, 200, 1, ctypes.byref(n)) == 0
    assert n.value > 4 << 20
    assert lib.muse_attn_workspace_size(ctypes.byref(lay), 126, 1, 200, 1, ctypes.byref(n)) == 0
    assert n.value <= 4 << 20
    f = Fake(decode=True, kind=fa.FULL_NOPE)
    f.n_seq, f.max_seq_len = 127, 200
    vp = ctypes.c_void_p
    rc = lib.muse_attn_decode_noalloc(ctypes.byref(f.layer), f.n_seq, vp(f.seq_len), f.max_seq_len, vp(f.q),
                                      vp(f.k), vp(f.v), vp(f.gate), ctypes.byref(f.cache), vp(f.out), None, None)
    assert rc == WORKSPACE
    f.layer.n_heads = 16                               # and the layer checks come first
    rc = lib.muse_attn_decode_noalloc(ctypes.byref(f.layer), f.n_seq, vp(f.seq_len), f.max_seq_len, vp(f.q),
                                      vp(f.k), vp(f.v), vp(f.gate), ctypes.byref(f.cache), vp(f.out), None, None)
    assert rc == SHAPE

"""MI355X (gfx950) attention core of one Muse Glimmer text layer.

A thin ctypes binding over ``libmuse_attn.so`` (see ``include/muse_attn.h``
for the contract).  The functions here only marshal arguments: they take
torch tensors that already live on the GPU, check device/dtype/shape/
contiguity, and pass raw pointers and the current HIP stream to the C ABI.
Every step of the computation runs in the library's HIP kernels.  There is no
CPU fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

from . import build as _build

LIB_PATH = _build.LIB_PATH

F32, BF16 = 0, 1
SLIDING_ROPE, FULL_NOPE = 0, 1
N_HEADS, N_KV_HEADS, HEAD_DIM = 32, 2, 128
ATTN_DIM = N_HEADS * HEAD_DIM

STATUS = {0: "MUSE_OK", 1: "MUSE_ERR_NULL", 2: "MUSE_ERR_SHAPE", 3: "MUSE_ERR_LAYER",
          4: "MUSE_ERR_CAPACITY", 5: "MUSE_ERR_WORKSPACE", 6: "MUSE_ERR_DTYPE",
          7: "MUSE_ERR_HIP", 8: "MUSE_ERR_ALIGN", 9: "MUSE_ERR_ALIAS"}

EXPORTS = ("muse_attn_prefill", "muse_attn_decode", "muse_attn_decode_noalloc", "muse_attn_workspace_size",
           "muse_attn_layer_init", "muse_layer_kind_for", "muse_rope_theta_table",
           "muse_status_str", "muse_kv_relocate", "muse_out_proj", "muse_out_proj_workspace_size")


class MuseError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)}")


class Layer(ctypes.Structure):
    """muse_attn_layer."""
    _fields_ = [("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("window", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("q_norm_gain", ctypes.c_float),
                ("k_norm_gain", ctypes.c_float), ("attn_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("kv_ring", ctypes.c_int32)]


class KvCache(ctypes.Structure):
    """muse_kv_cache."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int64)]


class KvTile(ctypes.Structure):
    """muse_kv_tile."""
    _fields_ = [("src_seq", ctypes.c_int32), ("dst_seq", ctypes.c_int32), ("src_pos", ctypes.c_int64),
                ("dst_pos", ctypes.c_int64), ("n_rows", ctypes.c_int64)]


class KernelTimer(ctypes.Structure):
    """muse_kernel_timer (two hipEvent_t)."""
    _fields_ = [("start", ctypes.c_void_p), ("stop", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lp = ctypes.POINTER(Layer)
        L.muse_attn_prefill.argtypes = [lp, i32, i32, vp, i32, vp, vp, vp, vp,
                                        ctypes.POINTER(KvCache), vp, vp, sz, vp,
                                        ctypes.POINTER(KernelTimer)]
        L.muse_attn_prefill.restype = ctypes.c_int
        L.muse_attn_decode.argtypes = [lp, i32, vp, i32, vp, vp, vp, vp,
                                       ctypes.POINTER(KvCache), vp, vp, sz, vp,
                                       ctypes.POINTER(KernelTimer)]
        L.muse_attn_decode.restype = ctypes.c_int
        L.muse_attn_decode_noalloc.argtypes = [lp, i32, vp, i32, vp, vp, vp, vp,
                                               ctypes.POINTER(KvCache), vp, vp, ctypes.POINTER(KernelTimer)]
        L.muse_attn_decode_noalloc.restype = ctypes.c_int
        L.muse_attn_workspace_size.argtypes = [lp, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.muse_attn_workspace_size.restype = ctypes.c_int
        L.muse_attn_layer_init.argtypes = [lp, i32, i32]
        L.muse_attn_layer_init.restype = ctypes.c_int
        L.muse_layer_kind_for.argtypes = [i32, i32]
        L.muse_layer_kind_for.restype = i32
        L.muse_rope_theta_table.argtypes = [ctypes.c_float, ctypes.POINTER(ctypes.c_float)]
        L.muse_rope_theta_table.restype = ctypes.c_int
        L.muse_status_str.argtypes = [ctypes.c_int]
        L.muse_status_str.restype = ctypes.c_char_p
        cp = ctypes.POINTER(KvCache)
        L.muse_kv_relocate.argtypes = [lp, cp, i32, cp, i32, ctypes.POINTER(KvTile), i32, vp]
        L.muse_kv_relocate.restype = ctypes.c_int
        L.muse_out_proj.argtypes = [i32, vp, vp, vp, vp, vp, ctypes.c_float, vp, sz, vp,
                                    ctypes.POINTER(KernelTimer)]
        L.muse_out_proj.restype = ctypes.c_int
        L.muse_out_proj_workspace_size.argtypes = [i32, ctypes.POINTER(sz)]
        L.muse_out_proj_workspace_size.restype = ctypes.c_int
        _lib = L
    return _lib


TIMELINE_LIB_PATH = _build.TIMELINE_LIB_PATH
TIMELINE_EXPORTS = ("muse_decode_timeline_read",)
TL_SPLIT_WORKGROUPS, TL_SPLIT_SLOTS, TL_MERGE_WORKGROUPS, TL_MERGE_SLOTS = 4096, 8, 4096, 4


def use_timeline_library() -> ctypes.CDLL:
    """Send this process's later calls to the profiling build
    (libmuse_attn_timeline.so, include/muse_attn_timeline.h): the same C ABI,
    whose decode kernels also record per-workgroup phase times.  Raises if
    the profiling build is missing."""
    global _lib, LIB_PATH
    if not os.path.exists(TIMELINE_LIB_PATH):
        raise RuntimeError(f"{TIMELINE_LIB_PATH} is missing: build it with "
                           "`python full_gqa_attention_amd/build.py --timeline`")
    _lib = None
    LIB_PATH = TIMELINE_LIB_PATH
    L = lib()
    L.muse_decode_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_int32]
    L.muse_decode_timeline_read.restype = ctypes.c_int
    return L


def decode_timeline_read(clear: bool = True):
    """The profiling build's per-workgroup decode records (numpy int64
    arrays [4096][8] for the split kernel and [4096][4] for the merge kernel,
    10 ns units, zero rows for workgroups that did not record); clears them
    afterwards unless clear is False."""
    import numpy as np
    split = np.zeros(TL_SPLIT_WORKGROUPS * TL_SPLIT_SLOTS, dtype=np.uint64)
    merge = np.zeros(TL_MERGE_WORKGROUPS * TL_MERGE_SLOTS, dtype=np.uint64)
    _check(lib().muse_decode_timeline_read(split.ctypes.data, split.size, merge.ctypes.data, merge.size,
                                           1 if clear else 0), "muse_decode_timeline_read")
    return (split.reshape(TL_SPLIT_WORKGROUPS, TL_SPLIT_SLOTS).astype(np.int64),
            merge.reshape(TL_MERGE_WORKGROUPS, TL_MERGE_SLOTS).astype(np.int64))


def _check(code: int, where: str):
    if code != 0:
        raise MuseError(code, where)


# ------------------------------------------------------------ host helpers

def make_layer(kind: int, *, window: int = 0, rope_theta: float = 0.0, rms_eps: float = 1e-5,
               q_norm_gain: float = 3.87, k_norm_gain: float = 1.0,
               attn_scale: float = 1.0 / math.sqrt(128.0), dtype: int = BF16,
               kv_ring: int = 0) -> Layer:
    """kv_ring=1 (sliding bf16 layers): the cache is a ring, position p in row p % capacity."""
    return Layer(N_HEADS, N_KV_HEADS, HEAD_DIM, kind, window, rope_theta, rms_eps,
                 q_norm_gain, k_norm_gain, attn_scale, dtype, kv_ring)


def layer_init(layer_index: int, dtype: int = BF16) -> Layer:
    """The model's parameters for layer `layer_index` (muse_attn_layer_init)."""
    l = Layer()
    _check(lib().muse_attn_layer_init(ctypes.byref(l), layer_index, dtype), "muse_attn_layer_init")
    return l


def layer_kind_for(layer_index: int, n_layers: int = 52) -> int:
    return lib().muse_layer_kind_for(layer_index, n_layers)


def rope_theta_table(theta: float):
    out = (ctypes.c_float * 64)()
    _check(lib().muse_rope_theta_table(theta, out), "muse_rope_theta_table")
    return list(out)


def status_str(code: int) -> str:
    return lib().muse_status_str(code).decode()


def workspace_size(layer: Layer, n_seq: int, n_new: int, max_seq_len: int, decode: bool) -> int:
    n = ctypes.c_size_t()
    _check(lib().muse_attn_workspace_size(ctypes.byref(layer), n_seq, n_new, max_seq_len,
                                          1 if decode else 0, ctypes.byref(n)),
           "muse_attn_workspace_size")
    return n.value


def workspace_buffer(nbytes: int, device="cuda") -> torch.Tensor:
    """A byte tensor of at least `nbytes` (never empty, so it has an address)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def workspace(layer: Layer, n_seq: int, n_new: int, max_seq_len: int, decode: bool,
              device="cuda") -> torch.Tensor:
    """A byte tensor large enough for one call."""
    return workspace_buffer(workspace_size(layer, n_seq, n_new, max_seq_len, decode), device)


# ------------------------------------------------------------------ calls

_TORCH = {F32: torch.float32, BF16: torch.bfloat16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t: torch.Tensor, name: str, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _call(decode: bool, layer: Layer, q, k, v, gate, cache_k, cache_v, seq_len, out,
          max_seq_len: int, ws: Optional[torch.Tensor], stream, timer):
    dt = _TORCH.get(layer.dtype)
    if dt is None:
        raise MuseError(6, "layer.dtype")
    S, N = q.shape[0], q.shape[1]
    _expect(q, "q", (S, N, N_HEADS, HEAD_DIM), dt)
    _expect(k, "k", (S, N, N_KV_HEADS, HEAD_DIM), dt)
    _expect(v, "v", (S, N, N_KV_HEADS, HEAD_DIM), dt)
    _expect(gate, "gate", (S, N, ATTN_DIM), dt)
    _expect(out, "out", (S, N, ATTN_DIM), dt)
    _expect(cache_k, "cache_k", None, dt)
    _expect(cache_v, "cache_v", tuple(cache_k.shape), dt)
    if cache_k.dim() != 4 or cache_k.shape[0] != S or tuple(cache_k.shape[2:]) != (N_KV_HEADS, HEAD_DIM):
        raise ValueError("cache_k/cache_v must be [n_seq, capacity, 2, 128]")
    _expect(seq_len, "seq_len", (S,), torch.int32)
    if decode and N != 1:
        raise ValueError("decode takes exactly one new token per sequence")
    if ws is None:
        ws = workspace(layer, S, N, max_seq_len, decode, device=q.device)
    _expect(ws, "workspace", None, torch.uint8)
    cache = KvCache(cache_k.data_ptr(), cache_v.data_ptr(), cache_k.shape[1])
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    tptr = ctypes.byref(timer) if timer is not None else None
    L = lib()
    if decode:
        rc = L.muse_attn_decode(ctypes.byref(layer), S, _ptr(seq_len), max_seq_len,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(gate), ctypes.byref(cache),
                                _ptr(out), _ptr(ws), ws.numel(), ctypes.c_void_p(stream), tptr)
        _check(rc, "muse_attn_decode")
    else:
        rc = L.muse_attn_prefill(ctypes.byref(layer), S, N, _ptr(seq_len), max_seq_len,
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(gate), ctypes.byref(cache),
                                 _ptr(out), _ptr(ws), ws.numel(), ctypes.c_void_p(stream), tptr)
        _check(rc, "muse_attn_prefill")
    return out


def prefill(layer: Layer, q, k, v, gate, cache_k, cache_v, seq_len, out=None, *,
            max_seq_len: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
            stream=None, timer: Optional[KernelTimer] = None) -> torch.Tensor:
    """muse_attn_prefill on torch tensors (see include/muse_attn.h).

    max_seq_len defaults to capacity - n_new (an upper bound of seq_len that
    needs no device read); a kv_ring layer must pass it."""
    if out is None:
        out = torch.empty(gate.shape, dtype=gate.dtype, device=gate.device)
    if max_seq_len is None:
        if layer.kv_ring:
            raise ValueError("a kv_ring layer needs max_seq_len (positions outgrow the ring)")
        max_seq_len = cache_k.shape[1] - q.shape[1]
    return _call(False, layer, q, k, v, gate, cache_k, cache_v, seq_len, out, max_seq_len,
                 workspace, stream, timer)


def decode(layer: Layer, q, k, v, gate, cache_k, cache_v, seq_len, out=None, *,
           max_seq_len: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
           stream=None, timer: Optional[KernelTimer] = None) -> torch.Tensor:
    """muse_attn_decode on torch tensors: q [S, 1, 32, 128] etc."""
    if out is None:
        out = torch.empty(gate.shape, dtype=gate.dtype, device=gate.device)
    if max_seq_len is None:
        if layer.kv_ring:
            raise ValueError("a kv_ring layer needs max_seq_len (positions outgrow the ring)")
        max_seq_len = cache_k.shape[1] - 1
    return _call(True, layer, q, k, v, gate, cache_k, cache_v, seq_len, out, max_seq_len,
                 workspace, stream, timer)


def decode_noalloc(layer: Layer, q, k, v, gate, cache_k, cache_v, seq_len, out=None, *,
                   max_seq_len: Optional[int] = None, stream=None,
                   timer: Optional[KernelTimer] = None) -> torch.Tensor:
    """muse_attn_decode_noalloc on torch tensors: muse_attn_decode with the
    library's static scratch instead of a workspace argument."""
    dt = _TORCH.get(layer.dtype)
    if dt is None:
        raise MuseError(6, "layer.dtype")
    S = q.shape[0]
    if out is None:
        out = torch.empty(gate.shape, dtype=gate.dtype, device=gate.device)
    if max_seq_len is None:
        if layer.kv_ring:
            raise ValueError("a kv_ring layer needs max_seq_len (positions outgrow the ring)")
        max_seq_len = cache_k.shape[1] - 1
    _expect(q, "q", (S, 1, N_HEADS, HEAD_DIM), dt)
    _expect(k, "k", (S, 1, N_KV_HEADS, HEAD_DIM), dt)
    _expect(v, "v", (S, 1, N_KV_HEADS, HEAD_DIM), dt)
    _expect(gate, "gate", (S, 1, ATTN_DIM), dt)
    _expect(out, "out", (S, 1, ATTN_DIM), dt)
    _expect(cache_k, "cache_k", None, dt)
    _expect(cache_v, "cache_v", tuple(cache_k.shape), dt)
    if cache_k.dim() != 4 or cache_k.shape[0] != S or tuple(cache_k.shape[2:]) != (N_KV_HEADS, HEAD_DIM):
        raise ValueError("cache_k/cache_v must be [n_seq, capacity, 2, 128]")
    _expect(seq_len, "seq_len", (S,), torch.int32)
    cache = KvCache(cache_k.data_ptr(), cache_v.data_ptr(), cache_k.shape[1])
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    tptr = ctypes.byref(timer) if timer is not None else None
    rc = lib().muse_attn_decode_noalloc(ctypes.byref(layer), S, _ptr(seq_len), max_seq_len, _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(gate), ctypes.byref(cache), _ptr(out), ctypes.c_void_p(stream), tptr)
    _check(rc, "muse_attn_decode_noalloc")
    return out


def kv_tiles(tiles):
    """A muse_kv_tile array from (src_seq, src_pos, dst_seq, dst_pos, n_rows) tuples."""
    arr = (KvTile * max(1, len(tiles)))()
    for i, (ss, sp, ds, dp, n) in enumerate(tiles):
        arr[i] = KvTile(ss, ds, sp, dp, n)
    return arr, len(tiles)


def kv_relocate(layer: Layer, src_k, src_v, dst_k, dst_v, tiles, stream=None) -> None:
    """muse_kv_relocate on torch caches [n_seq, capacity, 2, 128]; tiles is a
    sequence of (src_seq, src_pos, dst_seq, dst_pos, n_rows), or the result of
    kv_tiles()."""
    dt = _TORCH.get(layer.dtype)
    if dt is None:
        raise MuseError(6, "layer.dtype")
    for name, t in (("src_k", src_k), ("src_v", src_v), ("dst_k", dst_k), ("dst_v", dst_v)):
        _expect(t, name, None, dt)
        if t.dim() != 4 or tuple(t.shape[2:]) != (N_KV_HEADS, HEAD_DIM):
            raise ValueError(f"{name} must be [n_seq, capacity, 2, 128]")
    if src_v.shape != src_k.shape or dst_v.shape != dst_k.shape:
        raise ValueError("K and V caches must have the same shape")
    arr, n_tiles = tiles if isinstance(tiles, tuple) and len(tiles) == 2 and isinstance(tiles[1], int) \
        else kv_tiles(tiles)
    src = KvCache(src_k.data_ptr(), src_v.data_ptr(), src_k.shape[1])
    dst = KvCache(dst_k.data_ptr(), dst_v.data_ptr(), dst_k.shape[1])
    if stream is None:
        stream = torch.cuda.current_stream(src_k.device).cuda_stream
    rc = lib().muse_kv_relocate(ctypes.byref(layer), ctypes.byref(src), src_k.shape[0], ctypes.byref(dst),
                                dst_k.shape[0], arr, n_tiles, ctypes.c_void_p(stream))
    _check(rc, "muse_kv_relocate")


# ------------------------------------------ the block's tail: o_proj + post-norm

MODEL_DIM = 6656
POST_NORM_EPS = 1e-8


def out_proj_workspace_size(n_tokens: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().muse_out_proj_workspace_size(n_tokens, ctypes.byref(n)), "muse_out_proj_workspace_size")
    return n.value


def out_proj(attn, w, gamma, residual, out=None, *, eps: float = POST_NORM_EPS,
             workspace: Optional[torch.Tensor] = None, stream=None,
             timer: Optional[KernelTimer] = None) -> torch.Tensor:
    """muse_out_proj on torch tensors (see include/muse_attn.h): attn [..., 4096]
    bf16 (the attention output), w [6656, 4096] bf16, gamma [6656] f32,
    residual [..., 6656] bf16; returns hidden [..., 6656] bf16 (out may be
    residual itself)."""
    lead = tuple(attn.shape[:-1])
    M = 1
    for d in lead:
        M *= d
    _expect(attn, "attn", lead + (ATTN_DIM,), torch.bfloat16)
    _expect(w, "w", (MODEL_DIM, ATTN_DIM), torch.bfloat16)
    _expect(gamma, "gamma", (MODEL_DIM,), torch.float32)
    _expect(residual, "residual", lead + (MODEL_DIM,), torch.bfloat16)
    if out is None:
        out = torch.empty(residual.shape, dtype=torch.bfloat16, device=residual.device)
    _expect(out, "out", lead + (MODEL_DIM,), torch.bfloat16)
    if workspace is None:
        workspace = torch.empty(max(out_proj_workspace_size(M), 16), dtype=torch.uint8, device=attn.device)
    _expect(workspace, "workspace", None, torch.uint8)
    if stream is None:
        stream = torch.cuda.current_stream(attn.device).cuda_stream
    tptr = ctypes.byref(timer) if timer is not None else None
    _check(lib().muse_out_proj(M, _ptr(attn), _ptr(w), _ptr(gamma), _ptr(residual), _ptr(out), float(eps),
                               _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream), tptr),
           "muse_out_proj")
    return out


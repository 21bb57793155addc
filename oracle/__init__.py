"""CPU oracle for the Muse Glimmer attention core.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and ``bench.py``'s CPU-baseline leg may import this package.  The product
path (``full_gqa_attention_amd``) never imports it, and it never imports the
product: the two share no code.  The arithmetic lives in ``oracle.c`` (plain
C, fp64, OpenMP); this module only marshals numpy arrays into it.

Every function cites the page passage it follows (see ``oracle.c``).
Inputs in bf16 are passed as their raw ``uint16`` bit patterns; inputs in f32
as ``float32`` arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
SLIDING_ROPE, FULL_NOPE = 0, 1
ANGLE_F32, ANGLE_EXACT = 0, 1

HEAD_DIM, N_HEADS, N_KV_HEADS = 128, 32, 2


_SAN_LIB_PATH = os.path.join(_HERE, "liboracle_san.so")


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(clang: str = "/opt/rocm/llvm/bin/clang") -> str:
    """liboracle_san.so: oracle.c with AddressSanitizer and
    UndefinedBehaviorSanitizer, built with clang so that it shares one ASan
    runtime with the sanitized HIP library in a test process."""
    tmp = _SAN_LIB_PATH + ".tmp"
    cmd = [clang, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-shared-libasan", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SAN_LIB_PATH)
    return _SAN_LIB_PATH


def use_sanitized_build() -> None:
    """Load liboracle_san.so instead of liboracle.so (before the first call)."""
    global _LIB_PATH
    if _lib is not None:
        raise RuntimeError("the oracle library is already loaded")
    _LIB_PATH = _SAN_LIB_PATH


class _Layer(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("rms_eps", ctypes.c_double),
        ("q_gain", ctypes.c_double),
        ("k_gain", ctypes.c_double),
        ("scale", ctypes.c_double),
        ("store_dtype", ctypes.c_int32),
        ("angle_mode", ctypes.c_int32),
    ]


@dataclass
class Layer:
    """Parameters of one attention layer (exact values of the f32 parameters)."""
    kind: int
    window: int = 0
    rope_theta: float = 0.0
    rms_eps: float = 1e-5
    q_gain: float = 1.0
    k_gain: float = 1.0
    scale: float = 1.0 / np.sqrt(128.0)
    dtype: int = BF16
    angle_mode: int = ANGLE_F32

    def _c(self) -> _Layer:
        f32 = lambda x: float(np.float32(x))  # the library receives f32 parameters
        return _Layer(self.kind, self.window, f32(self.rope_theta), f32(self.rms_eps),
                      f32(self.q_gain), f32(self.k_gain), f32(self.scale),
                      self.dtype, self.angle_mode)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        vp = ctypes.c_void_p
        lib.oracle_layer_kind.argtypes = [ctypes.c_int]
        lib.oracle_layer_kind.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_double
        lib.oracle_round_store.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.oracle_round_store.restype = ctypes.c_double
        lib.oracle_rms_norm.argtypes = [dp, ctypes.c_int, ctypes.c_double, ctypes.c_double, dp]
        lib.oracle_rope_theta_table.argtypes = [ctypes.c_double, ctypes.c_int,
                                                ctypes.POINTER(ctypes.c_float)]
        lib.oracle_rope.argtypes = [dp, ctypes.c_int, ctypes.c_int64, ctypes.c_double,
                                    ctypes.c_int, dp]
        lib.oracle_sigmoid.argtypes = [ctypes.c_double]
        lib.oracle_sigmoid.restype = ctypes.c_double
        lib.oracle_attn_rows.argtypes = [
            ctypes.POINTER(_Layer), ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int32),
            vp, vp, vp, vp, ctypes.c_int64,
            ctypes.c_int, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
            vp, vp, dp, dp, dp]
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_out_proj.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp,
                                        ctypes.c_double, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64),
                                        dp, dp]
        lib.oracle_out_proj.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _storage(a: np.ndarray, dtype: int) -> np.ndarray:
    """Check an input array is in the storage dtype and C-contiguous."""
    want = np.uint16 if dtype == BF16 else np.float32
    if a.dtype != want:
        raise TypeError(f"oracle input must be {want.__name__} for dtype {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


# ----------------------------------------------------------------- scalars

def layer_kind(layer: int) -> int:
    return _load().oracle_layer_kind(int(layer))


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Threads the oracle's later calls use (OpenMP)."""
    _load().oracle_set_num_threads(int(n))


def round_bf16(x: float) -> float:
    return _load().oracle_round_bf16(float(x))


def round_store(x: float, dtype: int) -> float:
    return _load().oracle_round_store(float(x), int(dtype))


def sigmoid(g: float) -> float:
    return _load().oracle_sigmoid(float(g))


def rms_norm(x, eps: float, gain: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().oracle_rms_norm(_dp(x), x.size, float(eps), float(gain), _dp(y))
    return y


def rope_theta_table(base: float, n: int = HEAD_DIM) -> np.ndarray:
    out = np.empty(n // 2, dtype=np.float32)
    _load().oracle_rope_theta_table(float(base), int(n),
                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return out


def rope(x, pos: int, base: float, angle_mode: int = ANGLE_F32) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().oracle_rope(_dp(x), x.size, int(pos), float(base), int(angle_mode), _dp(y))
    return y


# ------------------------------------------------------------------- layer

def attn_rows(layer: Layer, seq_len, k_new, v_new, cache_k, cache_v, rows, q_rows, gate_rows,
              want_store: bool = False):
    """One attention layer evaluated on a list of (sequence, new-token) rows.

    seq_len   int array [S]: prefix length of each sequence
    k_new, v_new [S, N, 2, 128] storage dtype
    cache_k, cache_v [S, capacity, 2, 128] storage dtype (rows < seq_len read);
              may be None when every seq_len is 0
    rows      int array [R, 2] of (s, t)
    q_rows    [R, 32, 128], gate_rows [R, 4096] storage dtype
    Returns out [R, 4096] float64 (and k_store, v_store [S, N, 2, 128] float64
    when want_store).
    """
    dt = layer.dtype
    seq_len = np.ascontiguousarray(seq_len, dtype=np.int32)
    k_new = _storage(k_new, dt)
    v_new = _storage(v_new, dt)
    S, N = k_new.shape[0], k_new.shape[1]
    if k_new.shape != (S, N, N_KV_HEADS, HEAD_DIM) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [S, N, 2, 128]")
    if cache_k is None:
        if np.any(seq_len != 0):
            raise ValueError("a prefix cache is required when seq_len > 0")
        cap = N
        cache_k = np.zeros((S, max(cap, 1), N_KV_HEADS, HEAD_DIM), dtype=k_new.dtype)
        cache_v = cache_k
    cache_k = _storage(cache_k, dt)
    cache_v = _storage(cache_v, dt)
    cap = cache_k.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
    R = rows.shape[0]
    row_s = np.ascontiguousarray(rows[:, 0])
    row_t = np.ascontiguousarray(rows[:, 1])
    q_rows = _storage(q_rows, dt).reshape(R, N_HEADS, HEAD_DIM)
    gate_rows = _storage(gate_rows, dt).reshape(R, N_HEADS * HEAD_DIM)
    out = np.empty((R, N_HEADS * HEAD_DIM), dtype=np.float64)
    kst = np.empty((S, N, N_KV_HEADS, HEAD_DIM), dtype=np.float64) if want_store else None
    vst = np.empty_like(kst) if want_store else None
    i32p = ctypes.POINTER(ctypes.c_int32)
    c_layer = layer._c()
    rc = _load().oracle_attn_rows(
        ctypes.byref(c_layer), S, N, seq_len.ctypes.data_as(i32p),
        k_new.ctypes.data, v_new.ctypes.data, cache_k.ctypes.data, cache_v.ctypes.data, cap,
        R, row_s.ctypes.data_as(i32p), row_t.ctypes.data_as(i32p),
        q_rows.ctypes.data, gate_rows.ctypes.data, _dp(out),
        _dp(kst) if want_store else None, _dp(vst) if want_store else None)
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return (out, kst, vst) if want_store else out


def all_rows(n_seq: int, n_new: int) -> np.ndarray:
    """Every (s, t) row of an [S, N] batch, in row-major order."""
    s, t = np.meshgrid(np.arange(n_seq), np.arange(n_new), indexing="ij")
    return np.stack([s.ravel(), t.ravel()], axis=1).astype(np.int32)


# ------------------------------------------------- next step: o_proj + post-norm

POST_NORM_EPS = 1e-8      # [Ch9] 9.9: the post-sublayer norms' own epsilon
HIDDEN = 6656             # model width ([Ch9] 9.8: o_proj [4096 -> 6656])


def out_proj_rows(attn, w, gamma, residual, rows=None, eps: float = POST_NORM_EPS, want_proj: bool = False):
    """The attention block's tail on chosen token rows ([Ch9] 9.8, 9.9 and
    Figure 9.1): y = RMSNorm_eps(attn . W^T) * gamma + residual.

    attn      [M, K] bf16 bit patterns (uint16): the gated attention output
    w         [N, K] bf16 bit patterns: o_proj, one row per output channel
    gamma     [N] float32: the post-attention norm's effective gain
    residual  [M, N] bf16 bit patterns
    rows      int array of token indices (default: all M)
    Returns y [R, N] float64 (and proj [R, N] float64 when want_proj).
    """
    attn = _storage(attn, BF16)
    w = _storage(w, BF16)
    residual = _storage(residual, BF16)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    M, K = attn.shape
    N = w.shape[0]
    if w.shape != (N, K) or gamma.shape != (N,) or residual.shape != (M, N):
        raise ValueError("shapes must be attn [M, K], w [N, K], gamma [N], residual [M, N]")
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.size
    y = np.empty((R, N), dtype=np.float64)
    proj = np.empty((R, N), dtype=np.float64) if want_proj else None
    rc = _load().oracle_out_proj(M, K, N, attn.ctypes.data, w.ctypes.data, gamma.ctypes.data,
                                 residual.ctypes.data, float(eps), R,
                                 rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dp(y),
                                 _dp(proj) if want_proj else None)
    if rc != 0:
        raise ValueError("oracle_out_proj rejected its arguments")
    return (y, proj) if want_proj else y


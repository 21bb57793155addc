"""Seeded synthetic workloads for the Muse Glimmer attention core.

This module holds none of the method's arithmetic: only random draws, storage
rounding and the shapes/parameters of the workloads.  It is the one piece the
HIP path's tests/benchmark and the CPU oracle's callers both use, so that the
two sides see the same bytes.

Recipe (every tensor): standard normal in f32 from
``numpy.random.default_rng([seed, config, layer, tensor, step])``, then
rounded to nearest-even into the storage dtype.  Large tensors that live on
the GPU can instead be drawn on the device with a ``torch.Generator`` seeded
from the same tuple (``backend="torch"``); the oracle then reads back the
exact stored bytes of the rows it checks.  Outliers (the 8x8192 prefill): an
independent Bernoulli(p) mask per element, drawn from the stream with tensor
id + 16, multiplies the selected entries by 8.

Cache prefixes are synthetic stored rows: N(0,1) values written directly in
the storage dtype (K rows stand for normed-and-rotated keys, whose entries
have unit RMS; V rows for raw values).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

SEED = 1234
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "gate": 3, "cache_k": 4, "cache_v": 5,
              "attn": 6, "o_proj_w": 7, "post_gain": 8, "residual": 9}

N_HEADS, N_KV_HEADS, HEAD_DIM = 32, 2, 128
ATTN_DIM = N_HEADS * HEAD_DIM
SLIDING_ROPE, FULL_NOPE = 0, 1
F32, BF16 = 0, 1
TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


def seed_tuple(config: int, layer: int, tensor: str, step: int = 0, seed: int = SEED):
    return [seed, config, layer, TENSOR_IDS[tensor], step]


def _torch_seed(entropy) -> int:
    st = np.random.SeedSequence(entropy).generate_state(2, dtype=np.uint32)
    return (int(st[0]) << 31) ^ int(st[1])


def normal(shape, *, config: int, layer: int, tensor: str, step: int = 0, dtype: int = BF16,
           device="cpu", seed: int = SEED, outliers: float = 0.0, outlier_scale: float = 8.0,
           backend: str = "numpy") -> torch.Tensor:
    """Seeded N(0,1) tensor of `shape`, stored in `dtype` on `device`."""
    shape = tuple(int(s) for s in shape)
    ent = seed_tuple(config, layer, tensor, step, seed)
    if backend == "numpy":
        x = np.random.default_rng(ent).standard_normal(size=shape, dtype=np.float32)
        if outliers:
            ment = list(ent)
            ment[3] += 16
            mask = np.random.default_rng(ment).random(size=shape, dtype=np.float32) < outliers
            x[mask] *= np.float32(outlier_scale)
        t = torch.from_numpy(x)
        return t.to(TORCH_DTYPE[dtype]).to(device)
    if backend == "torch":
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(ent))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if outliers:
            ment = list(ent)
            ment[3] += 16
            gm = torch.Generator(device=device)
            gm.manual_seed(_torch_seed(ment))
            mask = torch.rand(shape, generator=gm, device=device) < outliers
            x = torch.where(mask, x * outlier_scale, x)
        return x.to(TORCH_DTYPE[dtype])
    raise ValueError(f"unknown backend {backend!r}")


# ------------------------------------------------------------- workloads

@dataclass(frozen=True)
class LayerSpec:
    """Parameters of one attention layer of a workload."""
    kind: int
    window: int = 0
    rope_theta: float = 0.0
    q_gain: float = 3.87
    k_gain: float = 1.0
    rms_eps: float = 1e-5
    scale: float = 1.0 / math.sqrt(128.0)
    seed_layer: int = 0      # layer id used in the seed tuple

    @property
    def name(self) -> str:
        return "sliding" if self.kind == SLIDING_ROPE else "full"


def sliding(window=2048, theta=500000.0, q_gain=3.87, k_gain=1.0, seed_layer=0) -> LayerSpec:
    return LayerSpec(SLIDING_ROPE, window, theta, q_gain, k_gain, seed_layer=seed_layer)


def full(q_gain=3.87, k_gain=1.0, seed_layer=1) -> LayerSpec:
    return LayerSpec(FULL_NOPE, 0, 0.0, q_gain, k_gain, seed_layer=seed_layer)


def model_layer(index: int) -> LayerSpec:
    """Layer `index` of the 52-layer schedule: full NoPE iff index % 4 == 3."""
    if index % 4 == 3:
        return full(seed_layer=index)
    return sliding(seed_layer=index)


@dataclass(frozen=True)
class Workload:
    name: str
    config: int                 # seed-tuple config id
    dtype: int
    n_seq: int
    prefix: int                 # rows already cached per sequence
    n_new: int                  # new tokens per sequence (1 = decode)
    layers: Tuple[LayerSpec, ...]
    outliers: float = 0.0
    decode_steps: int = 0       # extra decode steps after a chunked prefill

    @property
    def is_decode(self) -> bool:
        return self.n_new == 1 and self.decode_steps == 0 and self.prefix > 0

    @property
    def capacity(self) -> int:
        return self.prefix + self.n_new + self.decode_steps


WORKLOADS = {
    "prefill_1x512_f32": Workload(
        "prefill_1x512_f32", 1, F32, 1, 0, 512,
        (sliding(128, 10000.0, 1.0, 1.0, 0), full(1.0, 1.0, 1))),
    "decode_64x8192_bf16": Workload(
        "decode_64x8192_bf16", 2, BF16, 64, 8192, 1, (sliding(), full())),
    "prefill_8x8192_bf16": Workload(
        "prefill_8x8192_bf16", 3, BF16, 8, 0, 8192, (sliding(), full()), outliers=0.01),
    "decode_16x131072_bf16": Workload(
        "decode_16x131072_bf16", 4, BF16, 16, 131072, 1, (full(seed_layer=1), sliding(seed_layer=0))),
    "schedule_52x4_32768p4096_256d": Workload(
        "schedule_52x4_32768p4096_256d", 5, BF16, 4, 32768, 4096,
        tuple(model_layer(i) for i in range(52)), decode_steps=256),
}


@dataclass
class LayerInputs:
    """Device (or host) tensors for one layer call."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    gate: torch.Tensor
    cache_k: torch.Tensor
    cache_v: torch.Tensor
    seq_len: torch.Tensor


def layer_inputs(w: Workload, layer: LayerSpec, *, device="cpu", backend="numpy",
                 n_seq: Optional[int] = None, prefix: Optional[int] = None,
                 n_new: Optional[int] = None, capacity: Optional[int] = None,
                 step: int = 0, with_cache: bool = True) -> LayerInputs:
    """Inputs of one layer of workload `w` (sizes overridable for small cases)."""
    S = w.n_seq if n_seq is None else n_seq
    L = w.prefix if prefix is None else prefix
    N = w.n_new if n_new is None else n_new
    cap = (L + N if capacity is None else capacity)
    kw = dict(config=w.config, layer=layer.seed_layer, step=step, dtype=w.dtype,
              device=device, backend=backend, outliers=w.outliers)
    q = normal((S, N, N_HEADS, HEAD_DIM), tensor="q", **kw)
    k = normal((S, N, N_KV_HEADS, HEAD_DIM), tensor="k", **kw)
    v = normal((S, N, N_KV_HEADS, HEAD_DIM), tensor="v", **kw)
    gate = normal((S, N, ATTN_DIM), tensor="gate", **kw)
    tdt = TORCH_DTYPE[w.dtype]
    if with_cache:
        ck = torch.zeros((S, cap, N_KV_HEADS, HEAD_DIM), dtype=tdt, device=device)
        cv = torch.zeros_like(ck)
        if L > 0:
            ckw = dict(kw)
            ckw.pop("outliers")
            ck[:, :L] = normal((S, L, N_KV_HEADS, HEAD_DIM), tensor="cache_k", **ckw)
            cv[:, :L] = normal((S, L, N_KV_HEADS, HEAD_DIM), tensor="cache_v", **ckw)
    else:
        ck = cv = torch.empty(0, dtype=tdt, device=device)
    seq_len = torch.full((S,), L, dtype=torch.int32, device=device)
    return LayerInputs(q, k, v, gate, ck, cv, seq_len)


def to_storage_numpy(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a tensor as numpy: bf16 -> uint16 bit patterns, f32 -> float32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported storage dtype {t.dtype}")


# ------------------------------------------------ the block's tail (o_proj + post-norm)

MODEL_DIM = 6656


@dataclass
class OutProjInputs:
    attn: torch.Tensor       # bf16 [M, 4096]: stands for the gated attention output
    w: torch.Tensor          # bf16 [6656, 4096]: o_proj, N(0, 1/4096) so proj keeps attn's scale
    gamma: torch.Tensor      # f32 [6656]: 1 + 0.1 N(0, 1) (the norm's gain, an offset from one)
    residual: torch.Tensor   # bf16 [M, 6656]


def out_proj_inputs(n_tokens: int, *, config: int, layer: int = 0, step: int = 0, device="cpu",
                    backend: str = "numpy") -> OutProjInputs:
    """Seeded synthetic weights and activations for the block's tail (no
    trained weights exist here)."""
    kw = dict(config=config, layer=layer, step=step, device=device, backend=backend)
    attn = normal((n_tokens, ATTN_DIM), tensor="attn", **kw)
    w = (normal((MODEL_DIM, ATTN_DIM), tensor="o_proj_w", dtype=F32, **kw) * (1.0 / 64.0)).to(torch.bfloat16)
    gamma = 1.0 + 0.1 * normal((MODEL_DIM,), tensor="post_gain", dtype=F32, **kw)
    residual = normal((n_tokens, MODEL_DIM), tensor="residual", **kw)
    return OutProjInputs(attn, w, gamma.to(torch.float32), residual)


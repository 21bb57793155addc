"""The model's layer schedule on one batch: every layer's attention core, in
layer order, over per-layer KV caches ("Chapter 9 - The Muse Glimmer
architecture" 9.4 and Figure 9.4: layer l is full NoPE iff l % 4 == 3, else
sliding RoPE with a 2,048-key window).  A chunked prefill onto a cached prefix
runs every layer once; a decode step runs every layer once and then advances
the device-side seq_len, so a captured step replays as the next step.

Marshalling only: the layers' seeded synthetic inputs and caches come from
``synth``, and every call goes through the C ABI.  The benchmark times this
path and the end-to-end parity test checks it.
"""
from __future__ import annotations

from typing import List, Optional

import torch

import full_gqa_attention_amd as fa
from full_gqa_attention_amd import synth


def ring_of(cache: torch.Tensor, L: int, cap: int) -> torch.Tensor:
    """A ring of `cap` rows holding positions [L - cap, L) of every sequence
    at row p % cap (the same stored rows as the linear cache `cache`); rows
    of positions below 0 are zero ("Chapter 9" 9.7: a sliding layer keeps
    its window in a ring)."""
    ring = torch.empty((cache.shape[0], cap) + tuple(cache.shape[2:]), dtype=cache.dtype, device=cache.device)
    pos = torch.arange(max(0, L - cap), L, device=cache.device)
    ring[:, pos % cap] = cache[:, pos]
    if L < cap:
        ring[:, L:] = 0
    return ring


class Schedule:
    """The layers of workload `w` (a chunked prefill of w.n_new tokens onto
    w.prefix cached rows for w.n_seq sequences, then decode steps), each with
    its own seeded inputs and cache.

    ring: sliding layers keep their window as a ring of `window` rows.
    steps: decode steps the caches hold (default w.decode_steps).
    Decode steps feed each layer the same seeded one-token inputs (seeded by
    (seed, layer, step 1)); only the position advances from step to step.
    """

    def __init__(self, w: synth.Workload, *, ring: bool = False, steps: Optional[int] = None,
                 device: str = "cuda"):
        self.w = w
        self.ring = ring
        self.steps = w.decode_steps if steps is None else steps
        S, L0, N = w.n_seq, w.prefix, w.n_new
        self.capacity = L0 + N + self.steps
        self.max_decode_pos = L0 + N + max(self.steps, 1) - 1    # the last decode step's position
        self.specs = list(w.layers)
        self.layers: List[fa.Layer] = []
        self.inputs: List[synth.LayerInputs] = []               # prefill inputs and the layer's cache
        self.outs: List[torch.Tensor] = []                      # prefill outputs
        self.dec: List[tuple] = []                              # decode (q, k, v, gate, out)
        for spec in self.specs:
            r = self.is_ring(spec)
            inp = synth.layer_inputs(w, spec, device=device, backend="torch",
                                     capacity=L0 if r else self.capacity)
            if r:
                inp.cache_k = ring_of(inp.cache_k, L0, spec.window)
                inp.cache_v = ring_of(inp.cache_v, L0, spec.window)
            self.layers.append(fa.make_layer(spec.kind, window=spec.window, rope_theta=spec.rope_theta,
                                             rms_eps=spec.rms_eps, q_norm_gain=spec.q_gain,
                                             k_norm_gain=spec.k_gain, attn_scale=spec.scale, dtype=w.dtype,
                                             kv_ring=1 if r else 0))
            self.inputs.append(inp)
            self.outs.append(torch.empty_like(inp.gate))
            d = synth.layer_inputs(w, spec, device=device, backend="torch", n_new=1, prefix=0, step=1,
                                   with_cache=False)
            self.dec.append((d.q, d.k, d.v, d.gate, torch.empty_like(d.gate)))
        self.seq_len = torch.full((S,), L0, dtype=torch.int32, device=device)
        self.ws_prefill = fa.workspace_buffer(max(fa.workspace_size(l, S, N, L0, False) for l in self.layers), device)
        self.ws_decode = fa.workspace_buffer(
            max(fa.workspace_size(l, S, 1, self.max_decode_pos, True) for l in self.layers), device)

    def is_ring(self, spec: synth.LayerSpec) -> bool:
        return self.ring and spec.kind == synth.SLIDING_ROPE

    def prefill(self, timers=None):
        """The chunk through every layer (seq_len stays at the prefix; the
        caller moves it on, as `start_decode` does).  timers: optional
        per-layer muse_kernel_timer values."""
        L0 = self.w.prefix
        for l, (lay, inp, out) in enumerate(zip(self.layers, self.inputs, self.outs)):
            fa.prefill(lay, inp.q, inp.k, inp.v, inp.gate, inp.cache_k, inp.cache_v, self.seq_len, out,
                       max_seq_len=L0, workspace=self.ws_prefill, timer=timers[l] if timers else None)

    def start_decode(self):
        """Position the sequences after the chunk: the first decode step is at prefix + n_new."""
        self.seq_len.fill_(self.w.prefix + self.w.n_new)

    def decode_layer(self, l: int, timer=None):
        """Layer l's decode call at the current position (seq_len unchanged)."""
        q, k, v, g, o = self.dec[l]
        inp = self.inputs[l]
        fa.decode(self.layers[l], q, k, v, g, inp.cache_k, inp.cache_v, self.seq_len, o,
                  max_seq_len=self.max_decode_pos, workspace=self.ws_decode, timer=timer)

    def decode_step(self, timers=None):
        """Every layer's decode call at the current position, then seq_len += 1
        on the device.  timers: optional per-layer muse_kernel_timer values."""
        for l in range(len(self.layers)):
            self.decode_layer(l, timers[l] if timers else None)
        self.seq_len.add_(1)

    def capture_step(self) -> "torch.cuda.CUDAGraph":
        """A HIP graph of one decode step (every kernel of the step, and the
        seq_len increment); each replay is the next step."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.decode_step()
        return graph

    def cache_bytes(self) -> int:
        return sum(2 * inp.cache_k.numel() * inp.cache_k.element_size() for inp in self.inputs)

"""Helpers shared by the GPU parity tests: run one layer through the C ABI,
run the oracle on the same stored bytes, compare with the stated tolerances.

Tolerances (elementwise):
  f32 path:  |gpu - ref| <= 1e-4
  bf16 path: |gpu - ref| <= 2e-2 + 1e-2 * |ref|
Appended cache rows: V bit-exact.  K: for bf16, the oracle's rounded value
or one unit in the last place away (the GPU rounds an f32 value, the oracle a
double), or within 2e-6 of the head vector's largest entry; for f32, within
1e-6 of that largest entry.  The absolute allowance covers entries that the
rotation cancels towards zero, where a relative or ulp bound is meaningless.
"""
from __future__ import annotations

import numpy as np
import torch

import full_gqa_attention_amd as fa
import oracle
from full_gqa_attention_amd import synth

F32_ATOL = 1e-4
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def lib_layer(spec: synth.LayerSpec, dtype: int) -> fa.Layer:
    return fa.make_layer(spec.kind, window=spec.window, rope_theta=spec.rope_theta,
                         rms_eps=spec.rms_eps, q_norm_gain=spec.q_gain, k_norm_gain=spec.k_gain,
                         attn_scale=spec.scale, dtype=dtype)


def oracle_layer(spec: synth.LayerSpec, dtype: int) -> oracle.Layer:
    return oracle.Layer(kind=spec.kind, window=spec.window, rope_theta=spec.rope_theta,
                        rms_eps=spec.rms_eps, q_gain=spec.q_gain, k_gain=spec.k_gain,
                        scale=spec.scale, dtype=dtype)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def run_gpu(spec, dtype, inp: synth.LayerInputs, decode: bool, max_seq_len=None, timer=None):
    """One call through the C ABI; returns out (the cache tensors are updated in place)."""
    lay = lib_layer(spec, dtype)
    fn = fa.decode if decode else fa.prefill
    out = fn(lay, inp.q, inp.k, inp.v, inp.gate, inp.cache_k, inp.cache_v, inp.seq_len,
             max_seq_len=max_seq_len, timer=timer)
    torch.cuda.synchronize()
    return out


def run_oracle(spec, dtype, inp: synth.LayerInputs, rows, prefix_k, prefix_v, seq_len):
    """Oracle on (s, t) rows.  prefix_k/v are host copies of the cache taken
    before the GPU call (only rows < seq_len[s] are read)."""
    S = inp.k.shape[0]
    rows = np.asarray(rows, dtype=np.int32).reshape(-1, 2)
    sel_s = torch.as_tensor(rows[:, 0], dtype=torch.long, device=inp.q.device)
    sel_t = torch.as_tensor(rows[:, 1], dtype=torch.long, device=inp.q.device)
    q_rows = synth.to_storage_numpy(inp.q[sel_s, sel_t])
    g_rows = synth.to_storage_numpy(inp.gate[sel_s, sel_t])
    out, kst, vst = oracle.attn_rows(
        oracle_layer(spec, dtype), np.asarray(seq_len, dtype=np.int32),
        synth.to_storage_numpy(inp.k), synth.to_storage_numpy(inp.v),
        prefix_k, prefix_v, rows, q_rows, g_rows, want_store=True)
    return out, kst, vst


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: int, what: str = ""):
    err = np.abs(got - ref)
    if dtype == synth.F32:
        bad = ~(err <= F32_ATOL)
    else:
        bad = ~(err <= BF16_ATOL + BF16_RTOL * np.abs(ref))
    stats = dict(max_abs=float(np.nanmax(err)) if err.size else 0.0,
                 max_rel=float(np.nanmax(err / np.maximum(np.abs(ref), 1e-30))) if err.size else 0.0,
                 n=int(err.size))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; "
                             f"first at {idx.tolist()}: got {got[tuple(idx[0])]}, "
                             f"ref {ref[tuple(idx[0])]}; stats {stats}")
    return stats


def bf16_neighbours_ok(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """got == ref, or the adjacent bf16 value (ref holds bf16-representable doubles)."""
    g = torch.from_numpy(got.astype(np.float32)).view(torch.int32).numpy().astype(np.int64)
    r = torch.from_numpy(ref.astype(np.float32)).view(torch.int32).numpy().astype(np.int64)
    return np.abs((g >> 16) - (r >> 16)) <= 1


def check_rows(gk: np.ndarray, gv: np.ndarray, kst: np.ndarray, vst: np.ndarray, dtype: int, what: str):
    """Stored cache rows (gk, gv: the GPU's, as float64) against the oracle's
    K-hat and V rows (kst, vst): V bit-exact, K as the module docstring says."""
    assert np.array_equal(gv, vst), f"{what}: V rows differ"
    scale = np.max(np.abs(kst), axis=-1, keepdims=True)
    if dtype == synth.F32:
        # a few f32 roundings of values bounded by the head's largest entry
        assert np.all(np.abs(gk - kst) <= 1e-6 * scale), f"{what}: K rows differ"
        return
    # one bf16 ulp apart, or (entries that rotation cancels towards zero,
    # where an ulp is tiny) within the f32 pipeline's absolute error of 2e-6
    # of the head vector's largest entry
    ok = bf16_neighbours_ok(gk, kst) | (np.abs(gk - kst) <= 2e-6 * scale)
    if not np.all(ok):
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} K entries off, first at {i}: gpu {gk[i]!r} "
                             f"oracle {kst[i]!r} row max {scale[i[:-1]]}")


def check_appended(inp: synth.LayerInputs, kst, vst, seq_len, dtype: int, n_new: int):
    """The cache rows [L_s, L_s + n_new) hold the oracle's stored K-hat and V."""
    for s in range(kst.shape[0]):
        L = int(seq_len[s])
        check_rows(to_f64(inp.cache_k[s, L:L + n_new]), to_f64(inp.cache_v[s, L:L + n_new]),
                   kst[s], vst[s], dtype, f"appended rows of sequence {s}")


def host_cache(inp: synth.LayerInputs, seqs=None):
    """Host copies of the cache (storage bytes) before a call."""
    ck, cv = inp.cache_k, inp.cache_v
    if seqs is not None:
        idx = torch.as_tensor(seqs, dtype=torch.long, device=ck.device)
        ck, cv = ck[idx], cv[idx]
    return synth.to_storage_numpy(ck), synth.to_storage_numpy(cv)


def edge_rows(n_new: int, window: int, extra=(), seqs=(0,)):
    """(s, t) sample that always includes window and tile edges."""
    ts = {0, 1, 63, 64, 127, 128, n_new - 1, *extra}
    if window:
        ts |= {window - 2, window - 1, window, window + 1}
    ts = sorted(t for t in ts if 0 <= t < n_new)
    return np.array([(s, t) for s in seqs for t in ts], dtype=np.int32)


def check_layer(w, spec, inp, decode, rows=None, max_seq_len=None, untouched=True):
    """Run GPU and oracle on the same inputs; compare outputs (all rows, or
    the sampled `rows`), the appended cache rows, and (if `untouched`) that no
    other cache row changed.  Returns (out, error stats)."""
    S, N = inp.k.shape[0], inp.k.shape[1]
    seq = inp.seq_len.cpu().numpy()
    pk, pv = host_cache(inp)
    if untouched:
        before_k, before_v = inp.cache_k.clone(), inp.cache_v.clone()
    out = run_gpu(spec, w.dtype, inp, decode, max_seq_len=max_seq_len)
    rows = oracle.all_rows(S, N) if rows is None else rows
    ref, kst, vst = run_oracle(spec, w.dtype, inp, rows, pk, pv, seq)
    got = to_f64(out[torch.as_tensor(rows[:, 0], device=inp.q.device).long(),
                     torch.as_tensor(rows[:, 1], device=inp.q.device).long()])
    stats = assert_close(got, ref, w.dtype, f"{w.name}/{spec.name}")
    check_appended(inp, kst, vst, seq, w.dtype, N)
    # every other cache row is untouched
    for s in range(S if untouched else 0):
        L = int(seq[s])
        keep = torch.ones(inp.cache_k.shape[1], dtype=torch.bool, device=inp.q.device)
        keep[L:L + N] = False
        assert torch.equal(inp.cache_k[s][keep], before_k[s][keep])
        assert torch.equal(inp.cache_v[s][keep], before_v[s][keep])
    return out, stats

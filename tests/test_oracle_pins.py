"""Pins of the CPU oracle against what the pages and the mathematics fix.

The oracle (oracle/oracle.c) is the reference the HIP path is checked
against, so it is itself checked here against things other than itself:
values the pages print (tests/golden/), closed forms, invariants, brute force
on tiny inputs, and special cases that reduce to library routines (torch SDPA
and rms_norm in fp64).  Each test names the mistake it is meant to catch.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ANGLE_EXACT, ANGLE_F32, BF16, F32, FULL_NOPE, SLIDING_ROPE, Layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D, H, G = 128, 32, 2


def golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ------------------------------------------------------------------ RoPE

def test_rope_worked_example():
    """Page's worked example (Ch 14, 14.4.2): catches a wrong pairing, sign or frequency."""
    g = golden("rope_worked_example.txt")
    n, base, pos = int(g["head_dim"][0]), float(g["base"][0]), int(g["pos"][0])
    th = oracle.rope_theta_table(base, n)
    assert list(th) == [np.float32(float(v)) for v in g["theta"]]
    x = [float(v) for v in g["input"]]
    want = np.array([float(v) for v in g["output"]])
    dec = int(g["decimals"][0])
    for mode in (ANGLE_F32, ANGLE_EXACT):
        y = oracle.rope(x, pos, base, mode)
        assert np.max(np.abs(y - want)) <= 0.5 * 10.0 ** (-dec) + 1e-12


def test_rope_pairs_are_adjacent():
    """GPT-J / NORM pairing (Ch 14, Figure 14.2): index 1 rotates with 0, never with 65."""
    for pos in (1, 7, 1000):
        e1 = np.zeros(D)
        e1[1] = 1.0
        y = oracle.rope(e1, pos, 500000.0, ANGLE_EXACT)
        a = pos * 1.0  # theta_0 = 1
        assert y[0] == pytest.approx(-math.sin(a), abs=1e-15)
        assert y[1] == pytest.approx(math.cos(a), abs=1e-15)
        assert np.all(y[2:] == 0.0)
        e0 = np.zeros(D)
        e0[0] = 1.0
        y = oracle.rope(e0, pos, 500000.0, ANGLE_EXACT)
        assert (y[0], y[1]) == pytest.approx((math.cos(a), math.sin(a)), abs=1e-15)


def test_rope_position_zero_is_identity_and_length_preserved():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(D)
    assert np.array_equal(oracle.rope(x, 0, 500000.0, ANGLE_F32), x)
    y = oracle.rope(x, 12345, 500000.0, ANGLE_F32)
    pair_len = lambda v: v[0::2] ** 2 + v[1::2] ** 2
    assert np.allclose(pair_len(y), pair_len(x), rtol=1e-14, atol=1e-15)


def _theta_exact(base):
    return base ** (-np.arange(D // 2) * 2.0 / D)


@pytest.mark.parametrize("base", [10000.0, 500000.0])
def test_rope_dot_depends_only_on_offset(base):
    """q(m).k(n) = q(m+d).k(n+d) and equals the page's closed form (Ch 14, 14.4.3)."""
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((2, D))
    th = _theta_exact(base)
    for m, n, d in [(5, 3, 100), (1000, 0, 70000), (131072, 100, -5000), (0, 9, 17)]:
        a = oracle.rope(q, m, base, ANGLE_EXACT) @ oracle.rope(k, n, base, ANGLE_EXACT)
        b = oracle.rope(q, m + d, base, ANGLE_EXACT) @ oracle.rope(k, n + d, base, ANGLE_EXACT)
        q0, q1, k0, k1 = q[0::2], q[1::2], k[0::2], k[1::2]
        closed = np.sum((q0 * k0 + q1 * k1) * np.cos((m - n) * th)
                        + (q0 * k1 - q1 * k0) * np.sin((m - n) * th))
        assert abs(a - b) < 1e-8
        assert abs(a - closed) < 1e-8


def test_rope_f32_angle_within_rounding_bound():
    """With f32 angles the identity holds to the angle-rounding bound."""
    base = 500000.0
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((2, D))
    th32 = oracle.rope_theta_table(base).astype(np.float64)
    pair = np.hypot(q[0::2], q[1::2]) * np.hypot(k[0::2], k[1::2])
    for m, n, d in [(40, 3, 9), (8192, 6000, 100), (131072, 129000, -3)]:
        a = oracle.rope(q, m, base, ANGLE_F32) @ oracle.rope(k, n, base, ANGLE_F32)
        b = oracle.rope(q, m + d, base, ANGLE_F32) @ oracle.rope(k, n + d, base, ANGLE_F32)
        # each f32 angle is within half an f32 ulp of pos*theta32
        err = sum(np.spacing(np.float32(p * th32)).astype(np.float64) / 2
                  for p in (m, n, m + d, n + d))
        assert abs(a - b) <= np.sum(pair * err) + 1e-12


def test_rope_angle_is_f32_product():
    """The angle is the f32 product pos * theta_i (Ch 14, 14.5 kernel listing), not
    the exact one: at large positions the two differ by up to ~4e-3 rad."""
    base = 500000.0
    th32 = oracle.rope_theta_table(base)
    for pos in (131071, 100003, 8191):
        for i in (1, 5, 17):
            x = np.zeros(D)
            x[2 * i] = 1.0
            y = oracle.rope(x, pos, base, ANGLE_F32)
            a = float(np.float32(pos) * th32[i])          # numpy's f32 multiply
            assert (y[2 * i], y[2 * i + 1]) == pytest.approx((math.cos(a), math.sin(a)), abs=1e-15)
    # and the two readings really are distinguishable there
    x = np.zeros(D)
    x[2] = 1.0
    ya = oracle.rope(x, 131071, base, ANGLE_F32)
    yb = oracle.rope(x, 131071, base, ANGLE_EXACT)
    assert abs(ya[3] - yb[3]) > 1e-6


def test_rope_theta_table_closed_forms():
    for base in (10000.0, 500000.0):
        th = oracle.rope_theta_table(base)
        assert th.dtype == np.float32 and th.shape == (64,)
        assert th[0] == np.float32(1.0)
        assert th[32] == np.float32(1.0 / math.sqrt(base))  # base^(-64/128)
        assert np.all(np.diff(th) < 0)
        ratio = th[1:].astype(np.float64) / th[:-1]
        assert np.allclose(ratio, base ** (-1.0 / 64), rtol=3e-7)


# -------------------------------------------------------------- QK-norm

def test_rms_norm_closed_form_and_library():
    rng = np.random.default_rng(6)
    for scale in (1e-3, 1.0, 40.0):
        x = rng.standard_normal(D) * scale
        eps, gain = 1e-5, 3.87
        y = oracle.rms_norm(x, eps, gain)
        ms = np.mean(x * x)
        # RMS of the output, closed form: catches eps placement and mean vs sum
        assert math.sqrt(np.mean(y * y)) == pytest.approx(gain * math.sqrt(ms / (ms + eps)), rel=1e-13)
        # direction kept
        assert np.allclose(y / np.linalg.norm(y), x / np.linalg.norm(x), atol=1e-14)
        ref = torch.nn.functional.rms_norm(torch.tensor(x), (D,),
                                           weight=torch.full((D,), gain, dtype=torch.float64), eps=eps)
        assert np.allclose(y, ref.numpy(), rtol=1e-13, atol=1e-15)


def test_rms_norm_scale_invariant_and_bounded():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(D)
    y1 = oracle.rms_norm(x, 1e-5, 1.0)
    y2 = oracle.rms_norm(1000.0 * x, 1e-5, 1.0)
    assert np.allclose(y1, y2, rtol=2e-5)
    # Cauchy-Schwarz logit bound of the News article: |q^.k^| <= gq*gk*128
    for _ in range(50):
        a, b = rng.standard_normal((2, D)) * rng.uniform(0.01, 100, 2)[:, None]
        qa, kb = oracle.rms_norm(a, 1e-5, 3.87), oracle.rms_norm(b, 1e-5, 1.0)
        assert abs(qa @ kb) <= 3.87 * 1.0 * D
        assert np.linalg.norm(qa) <= 3.87 * math.sqrt(D) * (1 + 1e-15)
    # equality case: q = k gives the bound up to the eps factor
    qa, ka = oracle.rms_norm(x, 1e-5, 3.87), oracle.rms_norm(x, 1e-5, 1.0)
    ms = np.mean(x * x)
    assert qa @ ka == pytest.approx(3.87 * D * ms / (ms + 1e-5), rel=1e-13)


def test_norm_commutes_with_rotation():
    """spec pin: norm(R_p x) = R_p norm(x), since each pair rotation keeps length."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal(D)
    for p in (1, 77, 8192, 131072):
        a = oracle.rms_norm(oracle.rope(x, p, 500000.0, ANGLE_EXACT), 1e-5, 3.87)
        b = oracle.rope(oracle.rms_norm(x, 1e-5, 3.87), p, 500000.0, ANGLE_EXACT)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------- rounding, gate

def _bf16_brute(x):
    """Nearest bf16 to x by enumerating neighbours of x's f32 pattern; ties to even."""
    base = int(np.array(x, dtype=np.float32).view(np.uint32)) >> 16
    best = None
    for b in range(base - 3, base + 4):
        if not (0 <= b < 1 << 16):
            continue
        c = float(np.array(b << 16, dtype=np.uint32).view(np.float32))
        if not math.isfinite(c) or (c != 0 and math.copysign(1, c) != math.copysign(1, x)):
            continue
        d = abs(c - x)
        key = (d, b & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_round_bf16_brute_force():
    rng = np.random.default_rng(9)
    xs = list(rng.standard_normal(2000) * np.exp(rng.uniform(-30, 30, 2000)))
    one = 1.0
    xs += [one + 2 ** -8, one + 3 * 2 ** -8, -(one + 2 ** -8), one + 2 ** -8 + 2 ** -30,
           3.0e-39, 1.5e-40, -7.0e-41, 2.0 ** -130 * 1.5]
    for x in xs:
        assert oracle.round_bf16(x) == _bf16_brute(x), x
    # exact ties go to even; a value just above a tie is rounded once (no double rounding)
    assert oracle.round_bf16(1 + 2 ** -8) == 1.0
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert oracle.round_bf16(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7
    assert math.isinf(oracle.round_bf16(3.5e38))
    # library routine: torch's f32 -> bf16 is round-to-nearest-even
    f = rng.standard_normal(5000).astype(np.float32) * np.float32(100)
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_bf16(float(v)) for v in f])
    assert np.array_equal(got, ref)
    assert oracle.round_store(1 + 2 ** -30, F32) == 1.0


def test_sigmoid_gate_half_at_zero():
    assert oracle.sigmoid(0.0) == 0.5
    for g in np.linspace(-30, 30, 61):
        assert oracle.sigmoid(g) + oracle.sigmoid(-g) == pytest.approx(1.0, abs=1e-15)
    assert oracle.sigmoid(50.0) == 1.0


def test_layer_schedule_matches_pages():
    g = golden("model_constants.txt")
    n = int(g["n_layers"][0])
    full = [l for l in range(n) if oracle.layer_kind(l) == FULL_NOPE]
    assert full == [int(v) for v in g["full_layers"]]
    assert sum(oracle.layer_kind(l) == SLIDING_ROPE for l in range(n)) == 39


# ------------------------------------------------------ attention layer

def _as_storage(x, dtype):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_f64(a, dtype):
    if dtype == F32:
        return a.astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _case(S, T, L, dtype=F32, seed=0, cap=None):
    rng = np.random.default_rng(seed)
    cap = L + T if cap is None else cap
    q = _as_storage(rng.standard_normal((S, T, H, D)), dtype)
    k = _as_storage(rng.standard_normal((S, T, G, D)), dtype)
    v = _as_storage(rng.standard_normal((S, T, G, D)), dtype)
    gate = _as_storage(rng.standard_normal((S, T, H * D)), dtype)
    ck = _as_storage(rng.standard_normal((S, cap, G, D)), dtype)
    cv = _as_storage(rng.standard_normal((S, cap, G, D)), dtype)
    return q, k, v, gate, ck, cv


def _run(layer, L, q, k, v, gate, ck, cv, rows=None, want_store=False):
    S, T = k.shape[:2]
    rows = oracle.all_rows(S, T) if rows is None else np.asarray(rows, dtype=np.int32)
    qr = q[rows[:, 0], rows[:, 1]]
    gr = gate[rows[:, 0], rows[:, 1]]
    seq_len = np.full(S, L, dtype=np.int32)
    return oracle.attn_rows(layer, seq_len, k, v, ck, cv, rows, qr, gr, want_store=want_store)


def _layer(kind, W=0, theta=0.0, dtype=F32, gq=3.87, gk=1.0, angle=ANGLE_F32):
    if kind == FULL_NOPE:
        W, theta = 0, 0.0
    return Layer(kind=kind, window=W, rope_theta=theta, q_gain=gq, k_gain=gk, dtype=dtype,
                 angle_mode=angle)


def _visible(p, j, kind, W):
    return j <= p and (kind == FULL_NOPE or p - j < W)


def _nearest_storage(x64, dtype):
    """The storage value nearest to each float64 (ties to the even pattern),
    found by comparing neighbours rather than by the oracle's frexp rounding.
    numpy's float64 -> float32 cast is correctly rounded; torch's float64 ->
    bfloat16 cast goes through float32 (a double rounding), so its result is
    only a starting point: the nearest of it and its two bf16 neighbours wins."""
    x64 = np.asarray(x64, dtype=np.float64)
    if dtype == F32:
        return np.float32(x64).astype(np.float64)
    start = torch.from_numpy(x64.ravel()).float().to(torch.bfloat16).view(torch.int16).numpy()
    bits = start.astype(np.int64) & 0xFFFF
    cand = np.stack([(bits + d) & 0xFFFF for d in (-1, 0, 1)])            # [3, n]
    vals = (cand.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dist = np.abs(vals - x64.ravel()[None])
    dist[~np.isfinite(vals)] = np.inf
    dist[(cand & 0x7FFF) == 0x7F80] = np.inf                               # +-inf patterns
    best = dist.min(axis=0)
    tie_even = np.where(dist == best[None], (cand & 1), 2)                 # prefer an even pattern
    pick = np.argmin(tie_even, axis=0)
    return vals[pick, np.arange(vals.shape[1])].reshape(x64.shape)


def _khat_independent(k_raw64, positions, kind, theta, k_gain, eps=1e-5):
    """K-hat of raw key rows, written apart from the oracle: torch's fp64
    rms_norm with the K gain ("Chapter 14 - QK-norm and RoPE" 14.3: K is a plain
    normalize, gain 1 in the model, Q alone takes the 3.87 factor), then on
    sliding layers the adjacent-pair rotation as a complex product
    (x0 + i x1) * e^(i a) with a the f32 product f32(p) * f32(theta_i)
    (14.4.1, 14.5 listing); keys rotate before they are stored (14.7).
    k_raw64 [..., 128] float64, positions broadcastable to k_raw64.shape[:-1]."""
    x = torch.tensor(k_raw64, dtype=torch.float64)
    y = torch.nn.functional.rms_norm(x, (D,), weight=torch.full((D,), float(np.float32(k_gain)),
                                                                dtype=torch.float64),
                                     eps=float(np.float32(eps))).numpy()
    if kind == FULL_NOPE:
        return y
    th32 = np.float32(float(np.float32(theta)) ** (-np.arange(D // 2) * 2.0 / D))
    pos32 = np.float32(np.broadcast_to(positions, y.shape[:-1]))[..., None]
    ang = (pos32 * th32).astype(np.float64)                                 # numpy f32 multiply
    z = (y[..., 0::2] + 1j * y[..., 1::2]) * np.exp(1j * ang)
    out = np.empty_like(y)
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("kind,W", [(SLIDING_ROPE, 1), (SLIDING_ROPE, 2), (SLIDING_ROPE, 3),
                                    (SLIDING_ROPE, 5), (SLIDING_ROPE, 12), (SLIDING_ROPE, 15),
                                    (FULL_NOPE, 0)])
@pytest.mark.parametrize("L", [0, 5])
def test_layer_matches_sdpa_fp64(kind, W, L, dtype):
    """Library routine: fp64 SDPA with K/V repeated x16 and a brute-force mask.

    Catches a wrong GQA map (h % 2 instead of h / 16), a window off-by-one,
    the wrong scale, a gate applied before the softmax, a missing append."""
    S, T = 2, 12
    theta = 10000.0
    layer = _layer(kind, W, theta, dtype)
    q, k, v, gate, ck, cv = _case(S, T, L, dtype, seed=11 + W + L)
    out, kst, vst = _run(layer, L, q, k, v, gate, ck, cv, want_store=True)
    out = out.reshape(S, T, H * D)
    assert np.array_equal(vst, _to_f64(v, dtype))
    # the appended keys, recomputed apart from the oracle and rounded to the
    # nearest storage value: the stored rows must be exactly these
    pos = L + np.arange(T)[None, :, None]
    kexact = _khat_independent(_to_f64(k, dtype), pos, kind, theta, 1.0)
    knew = _nearest_storage(kexact, dtype)
    assert np.array_equal(kst, knew)
    q64 = _to_f64(q, dtype)
    for s in range(S):
        keys = np.concatenate([_to_f64(ck[s, :L], dtype), knew[s]], axis=0)   # [L+T, G, D]
        vals = np.concatenate([_to_f64(cv[s, :L], dtype), vst[s]], axis=0)
        qh = np.empty((H, T, D))
        for t in range(T):
            for h in range(H):
                y = oracle.rms_norm(q64[s, t, h], 1e-5, float(np.float32(3.87)))
                if kind == SLIDING_ROPE:
                    y = oracle.rope(y, L + t, theta, ANGLE_F32)
                qh[h, t] = y
        mask = np.array([[_visible(L + t, j, kind, W) for j in range(L + T)] for t in range(T)])
        Kr = torch.tensor(keys).permute(1, 0, 2).repeat_interleave(16, dim=0)
        Vr = torch.tensor(vals).permute(1, 0, 2).repeat_interleave(16, dim=0)
        att = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(qh), Kr, Vr, attn_mask=torch.tensor(mask),
            scale=float(np.float32(1 / math.sqrt(128))))
        ref = att.permute(1, 0, 2).reshape(T, H * D).numpy()
        ref = ref * (1.0 / (1.0 + np.exp(-_to_f64(gate[s], dtype))))
        assert np.allclose(out[s], ref, rtol=1e-11, atol=1e-12)
    if dtype == BF16:
        assert all(oracle.round_bf16(x) == x for x in kst.ravel()[:4096])


@pytest.mark.parametrize("kind,W", [(SLIDING_ROPE, 5), (SLIDING_ROPE, 1), (FULL_NOPE, 0)])
@pytest.mark.parametrize("L", [0, 30])
def test_visible_set_brute_force(kind, W, L):
    """One-hot V with K = 0 makes each output row show its visible set exactly.

    K = 0 normalises to 0, so all scores tie and the weights are uniform over
    the visible keys; V row j is the unit vector e_j."""
    S, T = 1, 40
    ck = np.zeros((S, L + T, G, D), np.float32)
    cv = np.zeros_like(ck)
    for j in range(L):
        cv[0, j, :, j] = 1.0
    k = np.zeros((S, T, G, D), np.float32)
    v = np.zeros((S, T, G, D), np.float32)
    for t in range(T):
        v[0, t, :, L + t] = 1.0
    q = np.random.default_rng(1).standard_normal((S, T, H, D)).astype(np.float32)
    gate = np.full((S, T, H * D), 50.0, np.float32)   # sigma(50) == 1.0 in double
    out = _run(_layer(kind, W, 500000.0), L, q, k, v, gate, ck, cv).reshape(T, H, D)
    for t in range(T):
        p = L + t
        vis = {j for j in range(L + T) if _visible(p, j, kind, W)}
        for h in (0, 15, 16, 31):
            got = {d for d in range(D) if out[t, h, d] != 0.0}
            assert got == vis
            assert np.allclose(out[t, h, sorted(vis)], 1.0 / len(vis), rtol=1e-15)


def test_three_windows_reach_receptive_field():
    """Composing the window rule three times reaches 1 + 3(W-1) positions (News article)."""
    g = golden("model_constants.txt")
    W_page, field_page = (int(x) for x in g["receptive_field_3_windows"])
    assert 1 + 3 * (W_page - 1) == field_page
    # reveal the oracle's rule at small W as above, then compose it
    W, T = 4, 40
    S = 1
    k = np.zeros((S, T, G, D), np.float32)
    v = np.zeros((S, T, G, D), np.float32)
    for t in range(T):
        v[0, t, :, t] = 1.0
    q = np.ones((S, T, H, D), np.float32)
    gate = np.full((S, T, H * D), 50.0, np.float32)
    out = _run(_layer(SLIDING_ROPE, W, 1e4), 0, q, k, v, gate, None, None).reshape(T, H, D)
    vis = [{d for d in range(D) if out[t, 0, d] != 0} for t in range(T)]
    reach = {T - 1}
    for _ in range(3):
        reach = set().union(*(vis[p] for p in reach))
    assert len(reach) == 1 + 3 * (W - 1)


def test_closed_forms_and_hull():
    S, T, L = 1, 16, 0
    q, k, v, gate, ck, cv = _case(S, T, L, F32, seed=21)
    v64, g64 = _to_f64(v, F32), _to_f64(gate, F32)
    sig = 1.0 / (1.0 + np.exp(-g64))
    # W = 1: each token sees only itself -> out = v_self * sigma(gate)
    out = _run(_layer(SLIDING_ROPE, 1, 1e4), L, q, k, v, gate, ck, cv).reshape(T, H, D)
    for h in range(H):
        # numpy's exp and the C library's may differ in the last ulp
        assert np.allclose(out[:, h], v64[0, :, h // 16] * sig[0].reshape(T, H, D)[:, h],
                           rtol=1e-15, atol=0)
    # identical keys on a NoPE layer: all scores tie -> mean of visible V
    k_same = np.repeat(k[:, :1], T, axis=1)
    out = _run(_layer(FULL_NOPE), L, q, k_same, v, gate, ck, cv).reshape(T, H, D)
    sigr = sig[0].reshape(T, H, D)
    for t in range(T):
        for h in (0, 20):
            mean = v64[0, : t + 1, h // 16].mean(axis=0)
            assert np.allclose(out[t, h], mean * sigr[t, h], rtol=1e-13, atol=1e-15)
    # hull: attention output (before the gate) lies between the visible V per channel
    out = _run(_layer(FULL_NOPE), L, q, k, v, gate, ck, cv).reshape(T, H, D) / sigr
    for t in range(T):
        for h in range(0, H, 5):
            vv = v64[0, : t + 1, h // 16]
            assert np.all(out[t, h] <= vv.max(axis=0) + 1e-12)
            assert np.all(out[t, h] >= vv.min(axis=0) - 1e-12)


def test_gate_zero_halves_output():
    S, T, L = 2, 9, 4
    q, k, v, gate, ck, cv = _case(S, T, L, F32, seed=31)
    lay = _layer(SLIDING_ROPE, 6, 500000.0)
    half = _run(lay, L, q, k, v, np.zeros_like(gate), ck, cv)
    whole = _run(lay, L, q, k, v, np.full_like(gate, 50.0), ck, cv)
    assert np.array_equal(2.0 * half, whole)


def test_gqa_heads_isolated():
    S, T, L = 1, 10, 3
    q, k, v, gate, ck, cv = _case(S, T, L, F32, seed=41)
    lay = _layer(SLIDING_ROPE, 7, 500000.0)
    base = _run(lay, L, q, k, v, gate, ck, cv).reshape(S * T, H, D)
    k2, v2, ck2, cv2 = k.copy(), v.copy(), ck.copy(), cv.copy()
    k2[:, :, 1] += 1.0
    v2[:, :, 1] *= -2.0
    cv2[:, :, 1] += 0.5
    pert = _run(lay, L, q, k2, v2, gate, ck2, cv2).reshape(S * T, H, D)
    assert np.array_equal(pert[:, :16], base[:, :16])
    assert not np.allclose(pert[:, 16:], base[:, 16:])


@pytest.mark.parametrize("kind,W", [(SLIDING_ROPE, 6), (FULL_NOPE, 0)])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_chunked_and_decode_equal_monolithic(kind, W, dtype):
    """Cross-entry pin: chunked prefill and decode reproduce rows of one prefill.

    Catches positions taken as t instead of seq_len + t for Q or K."""
    S, T, T1 = 2, 20, 13
    q, k, v, gate, _, _ = _case(S, T, 0, dtype, seed=51)
    lay = _layer(kind, W, 500000.0, dtype)
    mono, kst, vst = _run(lay, 0, q, k, v, gate, None, None, want_store=True)
    mono = mono.reshape(S, T, H * D)
    # chunk 1, then chunk 2 on top of the cache chunk 1 stored
    _, k1, v1 = _run(lay, 0, q[:, :T1], k[:, :T1], v[:, :T1], gate[:, :T1], None, None,
                     want_store=True)
    ck = _as_storage(np.concatenate([k1, np.zeros((S, T - T1, G, D))], axis=1), dtype)
    cv = _as_storage(np.concatenate([v1, np.zeros((S, T - T1, G, D))], axis=1), dtype)
    out2 = _run(lay, T1, q[:, T1:], k[:, T1:], v[:, T1:], gate[:, T1:], ck, cv).reshape(S, T - T1, H * D)
    assert np.array_equal(out2, mono[:, T1:])
    # decode of the last token on a cache holding the first T-1 stored rows
    ck = _as_storage(np.concatenate([kst[:, :T - 1], np.zeros((S, 1, G, D))], axis=1), dtype)
    cv = _as_storage(np.concatenate([vst[:, :T - 1], np.zeros((S, 1, G, D))], axis=1), dtype)
    dec = _run(lay, T - 1, q[:, T - 1:], k[:, T - 1:], v[:, T - 1:], gate[:, T - 1:], ck, cv)
    assert np.array_equal(dec.reshape(S, H * D), mono[:, T - 1])


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("kind", [SLIDING_ROPE, FULL_NOPE])
@pytest.mark.parametrize("gk", [1.0, 0.5])
def test_appended_keys_match_independent_khat(kind, dtype, gk):
    """Every appended K row is the nearest storage value to K-hat recomputed
    outside the oracle (torch rms_norm with the K gain, then the rotation at
    the row's position on sliding layers): catches the Q gain used for K, an
    unnormalised K, a position offset on K, or a missing or wrong rounding.
    A K gain apart from the Q gain (3.87) and from 1 separates the gains."""
    S, T, L = 2, 24, 37
    theta = 500000.0
    layer = _layer(kind, 8, theta, dtype, gq=3.87, gk=gk)
    rng = np.random.default_rng(81)
    q, k, v, gate, ck, cv = _case(S, T, L, dtype, seed=81)
    # a spread of magnitudes per row, so that a missing normalisation shows
    k = _as_storage(_to_f64(k, dtype) * rng.uniform(0.05, 20.0, (S, T, G, 1)), dtype)
    _, kst, _ = _run(layer, L, q, k, v, gate, ck, cv, rows=[(0, 0)], want_store=True)
    pos = L + np.arange(T)[None, :, None]
    kexact = _khat_independent(_to_f64(k, dtype), pos, kind, theta, gk)
    assert np.array_equal(kst, _nearest_storage(kexact, dtype))
    # and the stored value is within half a storage ulp of the exact K-hat
    ulp = np.spacing(np.abs(kexact).astype(np.float32)).astype(np.float64) * (65536.0 if dtype == BF16 else 1.0)
    assert np.all(np.abs(kst - kexact) <= 0.5 * ulp * (1 + 1e-12))
    # closed form of the stored rows' RMS: gk * sqrt(ms / (ms + eps)) of the raw row
    ms = np.mean(_to_f64(k, dtype) ** 2, axis=-1)
    rms = np.sqrt(np.mean(kst * kst, axis=-1))
    assert np.allclose(rms, gk * np.sqrt(ms / (ms + float(np.float32(1e-5)))),
                       rtol=4e-3 if dtype == BF16 else 1e-6)


def test_nope_rows_are_position_free():
    """NoPE K rows do not depend on position (Ch 9, 9.7; Ch 14, 14.6); RoPE rows do."""
    S, T = 1, 8
    q, k, v, gate, ck, cv = _case(S, T, 1000, F32, seed=61)
    _, k0, _ = _run(_layer(FULL_NOPE), 0, q, k, v, gate, None, None, want_store=True)
    _, k1, _ = _run(_layer(FULL_NOPE), 1000, q, k, v, gate, ck, cv, want_store=True)
    assert np.array_equal(k0, k1)
    _, r0, _ = _run(_layer(SLIDING_ROPE, 16, 1e4), 0, q, k, v, gate, None, None, want_store=True)
    _, r1, _ = _run(_layer(SLIDING_ROPE, 16, 1e4), 1000, q, k, v, gate, ck, cv, want_store=True)
    assert not np.allclose(r0, r1)


def test_sliding_output_shift_invariant():
    """Rows that only see new tokens do not change when every position shifts
    (exact angles; f32 storage rounds the rotated keys, hence the tolerance)."""
    S, T, W, delta = 1, 12, 4, 1000
    q, k, v, gate, ck, cv = _case(S, T, delta, F32, seed=71)
    lay = _layer(SLIDING_ROPE, W, 1e4, angle=ANGLE_EXACT)
    a = _run(lay, 0, q, k, v, gate, None, None).reshape(T, H * D)
    b = _run(lay, delta, q, k, v, gate, ck, cv).reshape(T, H * D)
    assert np.allclose(a[W - 1:], b[W - 1:], rtol=1e-5, atol=1e-6)
    assert not np.allclose(a[: W - 1], b[: W - 1], atol=1e-3)   # those rows see the prefix

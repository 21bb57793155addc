"""Pins for the oracle of the attention block's tail ([Ch9] "Chapter 9 - The
Muse Glimmer architecture" 9.8 and 9.9, Figure 9.1): o_proj [4096 -> 6656],
the post-attention RMSNorm with its own epsilon 1e-8, then the residual add.

Each pin is fixed by something other than the oracle's own formula: a closed
form, a one-hot special case, library routines (numpy matmul, torch rms_norm
in float64), or a brute-force loop on tiny inputs.  A transposed W, a wrong
epsilon, sum instead of mean, a dropped gain or residual each fail one.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (RNE), through torch."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_vals(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def rand_case(M, K, N, seed=0, wscale=None):
    rng = np.random.default_rng(seed)
    attn = bf16_bits(rng.standard_normal((M, K)))
    w = bf16_bits(rng.standard_normal((N, K)) * (wscale if wscale else 1.0 / np.sqrt(K)))
    gamma = (1.0 + 0.1 * rng.standard_normal(N)).astype(np.float32)
    res = bf16_bits(rng.standard_normal((M, N)))
    return attn, w, gamma, res


def test_library_routines_small():
    """numpy matmul and torch's rms_norm (float64) on the exact bf16 values."""
    attn, w, gamma, res = rand_case(7, 64, 48, seed=1)
    y = oracle.out_proj_rows(attn, w, gamma, res)
    proj = bf16_vals(attn) @ bf16_vals(w).T
    ref = torch.nn.functional.rms_norm(torch.from_numpy(proj), (48,), weight=torch.from_numpy(gamma.astype(np.float64)),
                                       eps=1e-8).numpy() + bf16_vals(res)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_brute_force_tiny():
    attn, w, gamma, res = rand_case(2, 5, 3, seed=2, wscale=1.0)
    a, W, r = bf16_vals(attn), bf16_vals(w), bf16_vals(res)
    y = oracle.out_proj_rows(attn, w, gamma, res)
    for t in range(2):
        p = [sum(a[t, k] * W[n, k] for k in range(5)) for n in range(3)]
        ms = sum(v * v for v in p) / 3
        for n in range(3):
            assert abs(y[t, n] - (p[n] / (ms + 1e-8) ** 0.5 * float(gamma[n]) + r[t, n])) < 1e-12


def test_one_hot_input_selects_a_column_of_w():
    """attn = e_k makes proj column k of W (a transposed W fails here)."""
    K, N = 16, 24
    _, w, _, _ = rand_case(1, K, N, seed=3, wscale=1.0)
    gamma = np.ones(N, dtype=np.float32)
    zero_res = np.zeros((K, N), dtype=np.uint16)
    attn = bf16_bits(np.eye(K))
    y, proj = oracle.out_proj_rows(attn, w, gamma, zero_res, want_proj=True)
    assert np.array_equal(proj, bf16_vals(w).T)
    ms = np.mean(proj ** 2, axis=1, keepdims=True)
    assert np.allclose(np.sqrt(np.mean(y ** 2, axis=1, keepdims=True)), np.sqrt(ms / (ms + 1e-8)), rtol=1e-12)


def test_epsilon_is_1e8():
    """A constant projection c = 2^-13 (c^2 = 1.49e-8, comparable to 1e-8):
    y = c / sqrt(c^2 + 1e-8) exactly; an epsilon of 1e-5 would give 0.039."""
    K, N = 8, 10
    c = 2.0 ** -13
    attn = bf16_bits(np.full((1, K), c))
    w = np.zeros((N, K), dtype=np.uint16)
    w[:, 0] = bf16_bits(np.array([1.0]))[0]           # every output takes attn[0]
    y = oracle.out_proj_rows(attn, w, np.ones(N, dtype=np.float32), np.zeros((1, N), dtype=np.uint16))
    assert np.allclose(y, c / np.sqrt(c * c + 1e-8), rtol=1e-14)
    assert abs(y[0, 0] - 0.7735) < 1e-3


def test_zero_projection_passes_the_residual():
    attn, _, gamma, res = rand_case(3, 32, 40, seed=4)
    y = oracle.out_proj_rows(attn, np.zeros((40, 32), dtype=np.uint16), gamma, res)
    assert np.array_equal(y, bf16_vals(res))


def test_gain_scale_and_sign():
    """gamma multiplies channel by channel; scaling attn by 2^j leaves the
    normalised projection unchanged (up to the epsilon); negating attn
    negates it."""
    attn, w, gamma, res = rand_case(4, 64, 32, seed=5)
    zero = np.zeros_like(res)
    base = oracle.out_proj_rows(attn, w, np.ones(32, dtype=np.float32), zero)
    g = oracle.out_proj_rows(attn, w, gamma, zero)
    assert np.allclose(g, base * gamma.astype(np.float64), rtol=1e-12, atol=1e-14)
    x4 = oracle.out_proj_rows(bf16_bits(bf16_vals(attn) * 4.0), w, np.ones(32, dtype=np.float32), zero)
    assert np.allclose(x4, base, rtol=1e-7)
    neg = oracle.out_proj_rows(bf16_bits(-bf16_vals(attn)), w, np.ones(32, dtype=np.float32), zero)
    assert np.array_equal(neg, -base)


def test_rows_are_independent():
    attn, w, gamma, res = rand_case(9, 32, 16, seed=6)
    full = oracle.out_proj_rows(attn, w, gamma, res)
    some = oracle.out_proj_rows(attn, w, gamma, res, rows=np.array([8, 0, 3]))
    assert np.array_equal(some, full[[8, 0, 3]])


def test_model_width_constants():
    """The oracle's width and epsilon are the pages' (golden fixture)."""
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "model_constants.txt")
    g = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            g[k] = v
    assert int(g["o_proj_in_out"][0]) == 4096 and int(g["o_proj_in_out"][1]) == oracle.HIDDEN
    assert float(g["post_norm_eps"][0]) == oracle.POST_NORM_EPS

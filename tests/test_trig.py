"""The library's RoPE sine and cosine (full_gqa_attention_amd/csrc/trig.h:
Cody-Waite reduction by pi/2 in double, Taylor series, one rounding to f32),
built for the host and checked against numpy's double-precision sin and cos
of the same f32 angles ("Chapter 14 - QK-norm and RoPE" 14.5 takes the
angle in f32 and its sin and cos accurately).

Angles: every RoPE frequency of bases 1e4 and 5e5 (f32 table, f32 product)
at positions 0 .. 140,000 (sampled) and at the edges the workloads use, plus
random f32 angles up to 2^29 and angles next to multiples of pi/2.  The
results must be the correctly rounded f32 values, with at most a few one-ulp
differences where the exact value lies within the double evaluation's error
of a rounding boundary.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "full_gqa_attention_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("trig") / "trig_driver")
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-I", CSRC,
                    os.path.join(ROOT, "tests", "trig_driver.cpp"), "-o", exe], check=True)
    return exe


def run(driver, tmp_path, angles):
    a = np.ascontiguousarray(angles, dtype=np.float32)
    inp, out = tmp_path / "a.bin", tmp_path / "sc.bin"
    a.tofile(inp)
    subprocess.run([driver, str(inp), str(out)], check=True)
    sc = np.fromfile(out, dtype=np.float32)
    return sc[:a.size], sc[a.size:]


def ulps(got, ref):
    g = got.view(np.int32).astype(np.int64)
    r = ref.view(np.int32).astype(np.int64)
    # map the sign-magnitude bit patterns to a monotonic integer line
    g = np.where(g < 0, -(g & 0x7fffffff), g)
    r = np.where(r < 0, -(r & 0x7fffffff), r)
    return np.abs(g - r)


def rope_angles():
    i = np.arange(64, dtype=np.float64)
    pos = np.unique(np.concatenate([np.arange(0, 140001, 7), [1, 2, 8191, 8192, 36864, 37119, 131071, 131072,
                                                               131073, 1 << 20]])).astype(np.float32)
    out = []
    for base in (1e4, 5e5):
        theta = (base ** (-2.0 * i / 128.0)).astype(np.float32)          # one rounding to f32
        out.append((pos[:, None] * theta[None, :]).ravel())             # f32 product
    return np.concatenate(out)


def check(driver, tmp_path, a, max_mismatch_frac):
    s, c = run(driver, tmp_path, a)
    ref_s = np.sin(a.astype(np.float64)).astype(np.float32)
    ref_c = np.cos(a.astype(np.float64)).astype(np.float32)
    for got, ref, name in ((s, ref_s, "sin"), (c, ref_c, "cos")):
        d = ulps(got, ref)
        assert d.max() <= 1, f"{name}: {d.max()} ulp at angle {a[np.argmax(d)]!r}"
        assert (d > 0).mean() <= max_mismatch_frac, f"{name}: {(d > 0).sum()} of {d.size} off by one ulp"


def test_rope_angles_correctly_rounded(driver, tmp_path):
    check(driver, tmp_path, rope_angles(), 1e-6)


def test_random_and_near_quadrant_angles(driver, tmp_path):
    rng = np.random.default_rng(7)
    wide = (rng.uniform(-1, 1, 400000) * 2.0 ** rng.uniform(-20, 29, 400000)).astype(np.float32)
    k = rng.integers(-(1 << 20), 1 << 20, 100000).astype(np.float64)
    near = (k * (np.pi / 2)).astype(np.float32)                        # f32 values next to k pi/2
    near = np.concatenate([near, np.nextafter(near, np.float32(np.inf)), np.nextafter(near, np.float32(-np.inf))])
    special = np.array([0.0, -0.0, 1e-30, -1e-30, 0.5, np.pi / 4, np.pi / 2, np.pi, 3 * np.pi / 2],
                       dtype=np.float32)
    check(driver, tmp_path, np.concatenate([wide, near, special]), 1e-6)


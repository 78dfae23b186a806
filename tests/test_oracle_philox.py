"""Pins for oracle.philox: Weyl increments re-derived with exact integer
arithmetic, rocRAND's open-source Philox4x32-10 engine (compiled here from
its header for the host) as an independent implementation, and statistics of
the keep mask."""

import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


def _isqrt_frac32(n):
    """floor(2^32 * frac(sqrt(n))) with exact integers."""
    s = math.isqrt(n << 64)          # floor(sqrt(n) * 2^32)
    return s - (math.isqrt(n) << 32)


def test_weyl_increments_from_golden_ratio_and_sqrt3():
    # golden ratio phi = (1 + sqrt 5) / 2; frac(phi) * 2^32 = (sqrt(5) - 1) * 2^31
    s5 = math.isqrt(5 << 64)         # floor(sqrt 5 * 2^32)
    w0 = (s5 - (1 << 32)) >> 1
    assert w0 == int(philox.PHILOX_W0)
    assert _isqrt_frac32(3) == int(philox.PHILOX_W1)


@pytest.fixture(scope="module")
def rocrand_kat(tmp_path_factory):
    inc = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(inc):
        pytest.skip("rocRAND header or g++ not available")
    exe = str(tmp_path_factory.mktemp("kat") / "kat")
    subprocess.check_call([gxx, "-O1", "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include",
                           os.path.join(HERE, "philox_rocrand_kat.cpp"),
                           "-o", exe])

    def run(rows):
        txt = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
        out = subprocess.run([exe], input=txt, capture_output=True, text=True,
                             check=True).stdout
        return np.array([[int(v) for v in l.split()] for l in out.strip().splitlines()],
                        dtype=np.uint64)
    return run


def test_philox_matches_rocrand(rocrand_kat):
    rng = np.random.default_rng(2024)
    rows = [(0, 0, 0, 0, 0, 0), (1, 2, 3, 4, 5, 6),
            (0xFFFFFFFF, 0, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF)]
    for _ in range(400):
        c = rng.integers(0, 2**32, 4, dtype=np.uint64)
        c[1] &= (1 << 30) - 1          # the helper advances counters by offset
        k = rng.integers(0, 2**32, 2, dtype=np.uint64)
        rows.append(tuple(int(v) for v in (*c, *k)))
    ref = rocrand_kat(rows)
    arr = np.array(rows, dtype=np.uint64)
    got = np.stack(philox.philox4x32_10(*arr.T), axis=1)
    assert np.array_equal(got, ref)


def test_mask_stream_is_rocrand_stream(rocrand_kat):
    """With this counter layout, element e's word is the e-th number of the
    rocRAND stream seeded with `seed`, in subsequence `offset`."""
    seed, offset = 0x1234_5678_9ABC_DEF0, 77
    e = np.arange(0, 64, dtype=np.uint64)
    words = philox.element_words(e, seed, offset)
    rows = [(b, 0, offset & 0xFFFFFFFF, offset >> 32, seed & 0xFFFFFFFF, seed >> 32)
            for b in range(16)]
    ref = rocrand_kat(rows).reshape(-1)
    assert np.array_equal(words, ref)


def test_threshold():
    assert philox.keep_threshold(0.1) == 429496729
    assert philox.keep_threshold(0.0) == 0
    assert philox.keep_threshold(1.0) == 1 << 32
    assert philox.keep_threshold(0.5) == 1 << 31


def test_keep_rate_within_6_sigma():
    rows, cols, p = 512, 1024, 0.1
    keep = philox.keep_mask(rows, cols, p, seed=0, offset=0)
    n = rows * cols
    mean = n * (1 - p)
    sigma = math.sqrt(n * p * (1 - p))
    assert abs(keep.sum() - mean) < 6 * sigma


def test_lanes_independent_chi_square():
    """Joint keep pattern of the 4 words of one block: 16 cells, chi-square
    with 15 degrees of freedom, far below the 1e-6 tail (about 48)."""
    keep = philox.keep_mask(1, 4 * 40000, 0.5, seed=9, offset=3)[0]
    codes = keep.reshape(-1, 4).astype(int) @ np.array([1, 2, 4, 8])
    obs = np.bincount(codes, minlength=16)
    exp = len(codes) / 16
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert chi2 < 48


def test_mask_depends_on_global_index_only():
    full = philox.keep_mask(8, 64, 0.3, seed=5, offset=1)
    part = philox.keep_mask(3, 16, 0.3, seed=5, offset=1, row0=2, col0=32, ld=64)
    assert np.array_equal(full[2:5, 32:48], part)


def test_p0_keeps_all_and_p1_drops_all():
    assert philox.keep_mask(4, 8, 0.0, 1, 2).all()
    assert not philox.keep_mask(4, 8, 1.0, 1, 2).any()


def test_seed_and_offset_change_the_mask():
    a = philox.keep_mask(16, 64, 0.5, seed=1, offset=0)
    b = philox.keep_mask(16, 64, 0.5, seed=2, offset=0)
    c = philox.keep_mask(16, 64, 0.5, seed=1, offset=1)
    assert (a != b).mean() > 0.3 and (a != c).mean() > 0.3

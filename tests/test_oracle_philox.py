"""Pins for the oracle's random streams (CPU only).

The projection P and the noise Z are the two random draws of the method
([GRAPE] Methodology, design choice 1: P is regenerated from a seed). The
oracle's Philox4x32-10 is pinned to (a) the published known-answer vectors of
the generator (tests/golden/philox4x32_10_kat.txt) and (b) two independent
open-source implementations compiled on the host. Its normals are pinned by
the Box-Muller identities, moments, a Kolmogorov-Smirnov test and the range
bound that follows from the uniform's resolution.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle.philox import (gaussian_stream, philox4x32_10, philox_words,
                           uniform_open01)

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((w[:4], w[4:6], w[6:10]))
    return rows


def test_known_answer_vectors():
    rows = _kat_rows()
    assert len(rows) == 3
    for ctr, key, want in rows:
        got = philox4x32_10(*[np.uint64(c) for c in ctr],
                            np.uint64(key[0]), np.uint64(key[1]))
        assert [int(g) for g in got] == want


@pytest.fixture(scope="module")
def host_reference(tmp_path_factory):
    """Build the host driver over the ATen and rocRAND Philox headers."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    try:
        import torch
        tinc = os.path.join(os.path.dirname(torch.__file__), "include")
    except Exception:  # pragma: no cover
        pytest.skip("torch headers not available")
    if not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("kat") / "philox_ref")
    subprocess.run([gxx, "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                    "-I" + tinc, "-I/opt/rocm/include",
                    os.path.join(HERE, "kat", "philox_ref.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def test_against_open_source_headers(host_reference):
    rng = np.random.default_rng(1234)
    ctr = rng.integers(0, 2 ** 32, size=(300, 6), dtype=np.uint64)
    # stream-layout shaped counters: (e >> 2, layer, step, tag)
    ctr[:100, 1] = rng.integers(0, 200, 100)
    ctr[:100, 2] = rng.integers(0, 10, 100)
    ctr[:100, 3] = rng.integers(0, 3, 100)
    ctr[100:150, 4:6] = 0                      # seed 0
    text = "\n".join(" ".join(str(int(v)) for v in row) for row in ctr) + "\n"
    out = subprocess.run([host_reference], input=text, capture_output=True,
                         text=True, check=True).stdout.split("\n")
    got = philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3],
                        ctr[:, 4], ctr[:, 5])
    got = np.stack(got, axis=1).astype(np.uint64)
    n_rocrand = 0
    for i in range(len(ctr)):
        aten = out[2 * i].split()
        assert aten[0] == "aten"
        assert [int(x) for x in aten[1:]] == [int(x) for x in got[i]], i
        roc = out[2 * i + 1].split()
        if roc[1] != "skip":
            n_rocrand += 1
            assert [int(x) for x in roc[1:]] == [int(x) for x in got[i]], i
    assert n_rocrand >= 100


def test_uniform_is_open_and_exact():
    x = np.array([0, 1, 511, 512, 2 ** 32 - 1], dtype=np.uint64)
    u = uniform_open01(x)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24
    assert u[3] == 3 * 2.0 ** -24
    assert u[4] == 1.0 - 2.0 ** -24
    # exactly representable in fp32
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_box_muller_pairing():
    """z0^2+z1^2 = -2 ln u(x0) and atan2(z1, z0) = 2 pi u(x1) (mod 2 pi), and
    likewise for (z2, z3) with (x2, x3): pins the pairing, the sin/cos order
    and the element-to-component mapping e & 3."""
    seed, lid, stp, tag = 77, 5, 3, 0
    n_ctr = 257
    z = gaussian_stream(seed, lid, stp, tag, 4 * n_ctr).reshape(n_ctr, 4)
    x0, x1, x2, x3 = philox_words(seed, lid, stp, tag,
                                  np.arange(n_ctr, dtype=np.uint64))
    for (za, zb, xa, xb) in ((z[:, 0], z[:, 1], x0, x1),
                             (z[:, 2], z[:, 3], x2, x3)):
        np.testing.assert_allclose(za * za + zb * zb,
                                   -2.0 * np.log(uniform_open01(xa)),
                                   rtol=1e-12, atol=1e-300)
        ang = np.mod(np.arctan2(zb, za), 2 * np.pi)
        want = 2 * np.pi * uniform_open01(xb)
        d = np.abs(np.mod(ang - want + np.pi, 2 * np.pi) - np.pi)
        assert d.max() < 1e-9


def test_offset_start_matches_full_stream():
    full = gaussian_stream(3, 1, 2, 1, 1000)
    for start in (0, 1, 2, 3, 5, 998):
        part = gaussian_stream(3, 1, 2, 1, 1000 - start, start=start)
        np.testing.assert_array_equal(part, full[start:])


def test_normal_moments_and_ks():
    z = gaussian_stream(0, 7, 1, 0, 400_000)
    assert abs(z.mean()) < 5 * (1 / math.sqrt(z.size))
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2 / z.size)
    assert abs(stats.skew(z)) < 0.02
    assert abs(stats.kurtosis(z)) < 0.04
    assert stats.kstest(z, "norm").pvalue > 1e-4
    assert np.abs(z).max() <= math.sqrt(48 * math.log(2)) + 1e-12


def test_streams_are_distinct():
    a = gaussian_stream(0, 1, 1, 0, 4096)
    for args in ((1, 1, 1, 0), (0, 2, 1, 0), (0, 1, 2, 0), (0, 1, 1, 1),
                 (2 ** 32, 1, 1, 0)):
        b = gaussian_stream(*args, 4096)
        assert not np.array_equal(a, b)
        assert abs(np.corrcoef(a, b)[0, 1]) < 0.08

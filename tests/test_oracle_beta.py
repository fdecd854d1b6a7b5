"""Pins of the exact-Beta codebook (the coordinate law of a random unit
vector, which the pages name before its Gaussian limit [ai.spot.hk,
隨機旋轉與Beta分佈; ICLR 2026 digest, Step 1]) and of the Haar-rotation
cross-check.

* d = 3: the law is uniform on [-1, 1], whose Lloyd-Max quantizer is the
  uniform one (closed form);
* Lloyd's conditions by independent numerical quadrature of the density;
* sqrt(d) times the levels tends to the N(0, 1) Lloyd-Max levels as d grows;
* under a Haar rotation (QR of a Gaussian matrix) the distortion of random
  unit vectors equals the Beta quantizer's own MSE, which is below the
  Gaussian quantizer's at small d;
* the host library's tables agree with the oracle's.
"""

import math

import numpy as np
import pytest
from scipy import integrate, special

import oracle as O

K = pytest.importorskip("kv_cache_vector_rotate_amd")


def _density(d):
    c = math.exp(special.gammaln(d / 2) - special.gammaln((d - 1) / 2) - 0.5 * math.log(math.pi))
    return lambda y: c * (1.0 - y * y) ** ((d - 3) / 2)


@pytest.mark.parametrize("B", [1, 2, 3])
def test_beta_d3_is_the_uniform_quantizer(B):
    lv, th = O.lloyd_max_beta(3, B)
    L = 1 << B
    assert np.allclose(lv, -1 + (2 * np.arange(L) + 1) / L, atol=1e-12)
    assert np.allclose(th, -1 + 2 * np.arange(1, L) / L, atol=1e-12)


@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("B", [1, 2, 3])
def test_beta_lloyd_conditions_by_quadrature(d, B):
    f = _density(d)
    assert abs(integrate.quad(f, -1, 1, limit=400)[0] - 1) < 1e-10
    lv, th = O.lloyd_max_beta(d, B)
    assert np.array_equal(th, (lv[:-1] + lv[1:]) / 2)
    assert th[len(th) // 2] == 0.0 and np.array_equal(lv, -lv[::-1])
    edges = [-1.0] + list(th) + [1.0]
    for c, a, b in zip(lv, edges[:-1], edges[1:]):
        num = integrate.quad(lambda y: y * f(y), a, b, limit=400, epsabs=1e-14)[0]
        den = integrate.quad(f, a, b, limit=400, epsabs=1e-14)[0]
        assert abs(c - num / den) < 1e-9 / math.sqrt(d)


def test_beta_tends_to_the_gaussian_codebook():
    gaps = []
    for d in (32, 256, 4096):
        lv, _ = O.lloyd_max_beta(d, 3)
        g, _ = O.lloyd_max_std_normal(3)
        gaps.append(np.max(np.abs(lv * math.sqrt(d) - g)))
    assert gaps[0] > gaps[1] > gaps[2] and gaps[2] < 2e-3


def _mse_quad(d, lv, th):
    f = _density(d)
    edges = [-1.0] + list(th) + [1.0]
    return sum(integrate.quad(lambda y: (y - c) ** 2 * f(y), a, b, limit=400)[0]
               for c, a, b in zip(lv, edges[:-1], edges[1:]))


def test_haar_rotation_distortion_matches_the_beta_quantizer():
    d, B = 32, 2
    R = O.haar_rotation(7, d)
    assert np.allclose(R @ R.T, np.eye(d), atol=1e-12)
    x = np.random.default_rng(3).standard_normal((40000, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    y = x @ R.T
    lb, tb = O.lloyd_max_beta(d, B)
    lg, tg = O.lloyd_max_std_normal(B)
    lg, tg = lg / math.sqrt(d), tg / math.sqrt(d)
    mse_b = np.mean((y - lb[np.searchsorted(tb, y, side="right")]) ** 2) * d
    mse_g = np.mean((y - lg[np.searchsorted(tg, y, side="right")]) ** 2) * d
    ref_b = _mse_quad(d, lb, tb) * d
    assert abs(mse_b - ref_b) / ref_b < 0.02
    assert ref_b < _mse_quad(d, lg, tg) * d
    assert mse_b < mse_g


@pytest.mark.parametrize("d,bits", [(32, 3), (128, 2), (128, 4), (1024, 4)])
def test_host_beta_tables_match_oracle(d, bits):
    t = K.codebook_tables(d, bits, d, 42, kind="beta")
    cb = O.make_codebook(d, bits, d, 42, kind="beta")
    assert np.max(np.abs(t["levels"] - cb.levels)) < 2e-11 / math.sqrt(d)
    assert np.max(np.abs(t["thresholds"] - cb.thresholds)) < 2e-11 / math.sqrt(d)
    assert np.array_equal(t["delta"], cb.delta)
    assert np.array_equal(t["S_rot"], cb.S_rot)

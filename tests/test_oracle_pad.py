"""Pins of the zero-padded variant: a dimension d that is not a power of two
is padded with zeros up to the next power of two D and the method runs in D
dimensions [ICLR 2026 digest, 実装のポイント: zero padding to the nearest power
of two for the Hadamard transform, e.g. 3072 -> 4096].

* rotation_dim follows that rule (the page's 3072 -> 4096 example included);
* the padded codebook is the D-dimensional one (same seed: same delta, S and
  levels) and takes rows of d elements;
* distortion: a unit vector in d dimensions loses about (d / D) of the
  D-dimensional Lloyd-Max MSE (Max's table) on its d coordinates, and the
  whole rotated-domain error matches the table;
* the QJL estimator stays unbiased for <q, k> over fresh Gaussian sketches
  of D columns (3 standard errors);
* the score without its QJL term is <q, decode_mse(k)> on the d coordinates;
* decoded values and attention outputs keep d coordinates; equal logits give
  the mean of the decoded values.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def test_rotation_dim_is_the_next_power_of_two():
    assert [O.rotation_dim(d) for d in (1, 2, 3, 96, 128, 129, 768, 1000, 1536, 3072)] == \
        [1, 2, 4, 128, 128, 256, 1024, 1024, 2048, 4096]


def test_padded_codebook_is_the_power_of_two_codebook():
    a = O.make_codebook(96, 3, 128, 42)
    b = O.make_codebook(128, 3, 128, 42)
    assert (a.d, a.din, b.din) == (128, 96, 128)
    for f in ("levels", "thresholds", "delta", "S", "R", "S_rot"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    # rows of 96 elements encode as the same rows padded to 128
    k = np.random.default_rng(1).standard_normal((50, 96))
    ea, eb = O.encode(a, k), O.encode(b, np.pad(k, ((0, 0), (0, 32))))
    assert np.array_equal(ea.codes, eb.codes) and np.array_equal(ea.signs, eb.signs)
    assert np.array_equal(ea.nu16, eb.nu16) and np.array_equal(ea.rho16, eb.rho16)
    with pytest.raises(AssertionError):
        O.encode(a, np.pad(k, ((0, 0), (0, 32))))   # padded rows are not accepted as input


@pytest.mark.parametrize("din,bits", [(96, 3), (80, 3), (112, 4), (768, 4)])
def test_padded_distortion(din, bits):
    mse = json.load(open(os.path.join(GOLDEN, "lloyd_max_gaussian.json")))[f"B{bits - 1}"]["mse"]
    cb = O.make_codebook(din, bits, O.rotation_dim(din), 42)
    D = cb.d
    n = 3000 if D == 128 else 400
    x = _unit(np.random.default_rng(din + bits), n, din)
    e = O.encode(cb, x)
    buf = O.pack(cb, e.codes[None], e.signs[None], e.nu16[None], e.rho16[None])
    xh = O.decode_mse(cb, buf, 1, n)[0]
    assert xh.shape == (n, din)
    dist = np.mean(np.sum((x - xh) ** 2, axis=1))
    # the rotated image of a padded unit vector spans a din-dimensional
    # subspace, so its coordinates are slightly correlated; the share of the
    # error that lands on the input coordinates is din / D up to that
    assert 0.9 < dist / (mse * din / D) < 1.12
    full = np.mean(np.sum((e.y - cb.levels[e.codes]) ** 2, axis=1))
    assert abs(full / mse - 1) < 0.04
    assert dist <= full


def test_padded_qjl_estimator_unbiased():
    din, D = 96, 128
    cb = O.make_codebook(din, 3, D, 42)
    rng = np.random.default_rng(91)
    k = rng.standard_normal(din) * np.exp(rng.normal(0, 0.7, din))
    e0 = O.encode(cb, k[None])
    kmse = e0.nu[0] * (cb.levels[e0.codes[0]] @ cb.R)          # D coordinates
    r = np.pad(k, (0, D - din)) - kmse
    q = rng.standard_normal(din) + 3.0 * r[:din] / np.linalg.norm(r[:din])
    qp = np.pad(q, (0, D - din))
    T = 10000
    est = np.empty(T)
    for t in range(T):
        S = rng.standard_normal((D, D))
        e = O.encode(cb, k[None], S=S)
        assert np.array_equal(e.codes, e0.codes)
        est[t] = O.estimate_inner_product(qp, kmse, e.rho[0], S, e.signs[0])
    truth = float(q @ k)
    se = est.std(ddof=1) / math.sqrt(T)
    assert abs(est.mean() - truth) < 3 * se
    assert abs(q @ r[:din]) > 20 * se   # the QJL term matters


def test_padded_score_without_qjl_is_decode_inner_product():
    din = 112
    cb = O.make_codebook(din, 4, 128, 7)
    rng = np.random.default_rng(3)
    G, N, Qg = 2, 40, 3
    k = rng.standard_normal((G * N, din)) * 2
    e = O.encode(cb, k)
    buf = O.pack(cb, e.codes.reshape(G, N, -1), e.signs.reshape(G, N, -1),
                 e.nu16.reshape(G, N), np.zeros((G, N), np.float16))   # rho = 0: no QJL term
    q = rng.standard_normal((G, Qg, din))
    got = O.score(cb, buf, G, N, q)
    ref = np.einsum("gqd,gnd->gqn", q, O.decode_mse(cb, buf, G, N))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_padded_values_and_attention():
    din = 80
    cb = O.make_codebook(din, 3, 128, 5)
    rng = np.random.default_rng(8)
    G, N, Qg = 2, 11, 4
    v = rng.standard_normal((G * N, din))
    ev = O.encode_values(cb, v)
    vb = O.pack_values(cb, ev.codes.reshape(G, N, -1), ev.nu16.reshape(G, N))
    vh = O.decode_values(cb, vb, G, N)
    assert vh.shape == (G, N, din)
    cos = np.sum(vh.reshape(-1, din) * v, axis=1) / np.linalg.norm(v, axis=1) / np.linalg.norm(
        vh.reshape(-1, din), axis=1)
    assert cos.min() > 0.9
    out = O.attention_from_logits(cb, np.zeros((G, Qg, N)), vb, G, N)
    assert out.shape == (G, Qg, din)
    assert np.allclose(out, np.broadcast_to(vh.mean(axis=1)[:, None, :], out.shape), atol=1e-12)

"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than the oracle
itself: closed forms, textbook constants, brute force on tiny inputs,
Monte-Carlo statistics, or numbers the pages print.  A plausible mistake in
the oracle (dropped term, wrong sign or index, transposed operand, wrong
constant) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- rotation

@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 128, 1024])
def test_sylvester_hadamard_is_orthogonal_and_closed_form(d):
    """H H^T = d I exactly; H_ij = (-1)^popcount(i & j) for the Sylvester
    construction [ICLR 2026 digest, Step 1: H_2d = [[H, H], [H, -H]]]."""
    H = O.sylvester_hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d, dtype=np.int64))
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(H, np.where(pc % 2 == 0, 1, -1))


@pytest.mark.parametrize("d", [4, 8, 32, 128, 1024])
def test_rotation_is_isometry(d):
    """||R x|| = ||x|| and R^T R = I to 1e-12 (R = H D / sqrt(d) is orthogonal)."""
    delta = O.rademacher_signs(7, d)
    R = O.rotation_matrix(delta)
    assert np.max(np.abs(R.T @ R - np.eye(d))) < 1e-12
    x = np.random.default_rng(d).standard_normal((16, d))
    nx = np.linalg.norm(x, axis=1)
    assert np.max(np.abs(np.linalg.norm(x @ R.T, axis=1) - nx) / nx) < 1e-12


def test_rotation_columns_and_first_row():
    """R e_j = delta_j H[:, j] / sqrt(d); row 0 of H is all ones, so
    (R x)_0 = sum_i delta_i x_i / sqrt(d)."""
    d = 64
    delta = O.rademacher_signs(3, d)
    R = O.rotation_matrix(delta)
    H = O.sylvester_hadamard(d)
    for j in (0, 1, 17, 63):
        e = np.zeros(d)
        e[j] = 1.0
        assert np.allclose(R @ e, delta[j] * H[:, j] / math.sqrt(d), atol=0, rtol=1e-15)
    x = np.random.default_rng(0).standard_normal(d)
    assert abs((R @ x)[0] - np.sum(delta * x) / math.sqrt(d)) < 1e-13


def _fwht_recursive(v):
    """Independent recursive Walsh-Hadamard transform (natural order)."""
    n = v.shape[0]
    if n == 1:
        return v.copy()
    a = _fwht_recursive(v[: n // 2])
    b = _fwht_recursive(v[n // 2:])
    return np.concatenate([a + b, a - b])


@pytest.mark.parametrize("d", [4, 8, 128])
def test_dense_rotation_equals_butterfly(d):
    """The dense matrix equals an independently written butterfly
    transform of delta * x, scaled by 1/sqrt(d) (the O(d log d) form the
    pages describe) to 1e-13."""
    delta = O.rademacher_signs(11, d)
    R = O.rotation_matrix(delta)
    x = np.random.default_rng(5).standard_normal(d)
    y_fast = _fwht_recursive(delta * x) / math.sqrt(d)
    assert np.max(np.abs(R @ x - y_fast)) < 1e-13


# ---------------------------------------------------------------- randomness

def test_splitmix64_known_answer():
    """The first output of SplitMix64 seeded with 0 is 0xE220A8397B1DCDAF
    (published reference value); our stream base of (seed 0, stream 1) is
    exactly that output, and draws are that sequence continued."""
    assert O.turboquant._mix64_int(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF
    # draw(seed, stream, i) = mix64(base + (i + 1) * gamma)
    base = O.turboquant._mix64_int(0 + 1 * 0x9E3779B97F4A7C15)
    d0 = O.splitmix64_draw(0, 1, [0, 1])
    g = 0x9E3779B97F4A7C15
    assert int(d0[0]) == O.turboquant._mix64_int(base + g)
    assert int(d0[1]) == O.turboquant._mix64_int(base + 2 * g)


def test_rademacher_balanced_and_seeded():
    s = O.rademacher_signs(42, 1 << 16)
    assert set(np.unique(s)) == {-1, 1}
    assert abs(s.mean()) < 4.0 / math.sqrt(s.size)
    assert np.array_equal(O.rademacher_signs(42, 128), s[:128])
    assert not np.array_equal(O.rademacher_signs(43, 128), s[:128])


def test_sketch_is_standard_normal():
    """The draws are exactly float16 and pass a Kolmogorov-Smirnov test
    against N(0,1); so do the entries of S = S_rot R (R orthogonal keeps the
    law); rows of both are uncorrelated, and S R^T gives the draws back."""
    G = O.gaussian_sketch(42, 128, 128)
    assert G.dtype == np.float16
    assert stats.kstest(G.ravel().astype(np.float64), "norm").pvalue > 1e-3
    cb = O.make_codebook(128, 3, 128, 42)
    assert np.array_equal(cb.S_rot, G.astype(np.float64))
    assert stats.kstest(cb.S.ravel(), "norm").pvalue > 1e-3
    for M in (cb.S, cb.S_rot):
        c = np.corrcoef(M[:8])
        assert np.max(np.abs(c - np.eye(8))) < 0.35
    assert np.max(np.abs(cb.S @ cb.R.T - cb.S_rot)) < 1e-12


# ---------------------------------------------------------------- Lloyd-Max

def _cond_mean_quad(a, b):
    num = integrate.quad(lambda x: x * math.exp(-x * x / 2), a, b, limit=200)[0]
    den = integrate.quad(lambda x: math.exp(-x * x / 2), a, b, limit=200)[0]
    return num / den


def _mse_quad(levels, thresholds):
    edges = [-np.inf] + list(thresholds) + [np.inf]
    tot = 0.0
    for c, a, b in zip(levels, edges[:-1], edges[1:]):
        tot += integrate.quad(lambda x: (x - c) ** 2 * math.exp(-x * x / 2) / math.sqrt(2 * math.pi),
                              a, b, limit=200)[0]
    return tot


def test_lloyd_max_one_bit_closed_form():
    lv, th = O.lloyd_max_std_normal(1)
    assert np.allclose(lv, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-15)
    assert th.tolist() == [0.0]
    assert abs(_mse_quad(lv, th) - (1 - 2 / math.pi)) < 1e-10


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_lloyd_max_fixed_point(B):
    """Boundaries are the midpoints, levels are conditional means (by
    numerical quadrature, independent of the oracle's erfc formula) to 1e-10;
    the code is odd-symmetric with middle threshold exactly 0."""
    lv, th = O.lloyd_max_std_normal(B)
    L = 1 << B
    assert lv.shape == (L,) and th.shape == (L - 1,)
    assert np.all(np.diff(lv) > 0)
    assert np.array_equal(th, (lv[:-1] + lv[1:]) / 2)
    assert th[L // 2 - 1] == 0.0
    assert np.array_equal(lv, -lv[::-1])
    edges = [-np.inf] + list(th) + [np.inf]
    for c, a, b in zip(lv, edges[:-1], edges[1:]):
        assert abs(c - _cond_mean_quad(a, b)) < 1e-10


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_lloyd_max_textbook_values(B):
    """Agreement with Max (1960) to the table's 4 significant digits."""
    ref = json.load(open(os.path.join(GOLDEN, "lloyd_max_gaussian.json")))[f"B{B}"]
    lv, th = O.lloyd_max_std_normal(B)
    K = len(lv) // 2
    assert np.allclose(lv[K:], ref["levels_pos"], rtol=6e-4, atol=0)
    assert np.allclose(th[K:], ref["thresholds_pos"], rtol=6e-4, atol=0)
    assert abs(_mse_quad(lv, th) - ref["mse"]) / ref["mse"] < 6e-4


def test_codebook_scaling_to_one_over_d():
    """Levels for N(0, 1/d) are the N(0,1) levels divided by sqrt(d)."""
    cb = O.make_codebook(128, 3, 128, 42)
    lv, th = O.lloyd_max_std_normal(2)
    assert np.allclose(cb.levels * math.sqrt(128), lv, rtol=1e-15, atol=0)
    assert np.allclose(cb.thresholds * math.sqrt(128), th, rtol=1e-15, atol=0)


# ---------------------------------------------------------------- encode

@pytest.mark.parametrize("d,bits", [(4, 2), (4, 3), (4, 4), (8, 2), (8, 3)])
def test_codes_equal_bruteforce_product_codebook(d, bits):
    """Per-coordinate threshold codes are the exhaustive nearest codeword of
    the product codebook {c}^d (separability), for random keys."""
    cb = O.make_codebook(d, bits, d, 9)
    keys = np.random.default_rng(d * 10 + bits).standard_normal((40, d))
    e = O.encode(cb, keys)
    L = cb.L
    grid = np.array(np.meshgrid(*[np.arange(L)] * d, indexing="ij")).reshape(d, -1).T
    cand = cb.levels[grid]                                    # [L^d, d]
    for n in range(keys.shape[0]):
        dist = np.sum((e.y[n][None, :] - cand) ** 2, axis=1)
        best = grid[np.argmin(dist)]
        assert np.array_equal(best, e.codes[n])


def test_encode_residual_and_norms_by_definition():
    """rho = ||k - nu R^T c[code]|| and the stored norms are float16 (RNE)."""
    cb = O.make_codebook(32, 3, 32, 1)
    k = np.random.default_rng(2).standard_normal((10, 32)) * 3.0
    e = O.encode(cb, k)
    nu = np.linalg.norm(k, axis=1)
    assert np.allclose(e.nu, nu, rtol=1e-15)
    kmse = np.stack([nu[i] * cb.R.T @ cb.levels[e.codes[i]] for i in range(10)])
    assert np.allclose(e.rho, np.linalg.norm(k - kmse, axis=1), rtol=1e-13)
    assert np.array_equal(e.nu16, nu.astype(np.float16))
    assert np.array_equal(e.signs, ((k - kmse) @ cb.S.T < 0).astype(np.uint8))


def test_zero_vector_rule():
    """||k|| < 1e-10 -> all-zero record and a zero logit
    [ICLR 2026 digest, 実装の擬似コード]."""
    cb = O.make_codebook(32, 3, 32, 1)
    k = np.zeros((3, 32))
    k[1, 5] = 5e-11
    k[2, 0] = 1.0
    e = O.encode(cb, k)
    assert e.zero.tolist() == [True, True, False]
    assert not e.codes[:2].any() and not e.signs[:2].any()
    assert float(e.nu16[0]) == 0.0 and float(e.rho16[1]) == 0.0
    buf = O.pack(cb, e.codes[None], e.signs[None], e.nu16[None], e.rho16[None])
    q = np.random.default_rng(0).standard_normal((1, 2, 32))
    lg = O.score(cb, buf, 1, 3, q)
    assert np.all(lg[0, :, :2] == 0.0)


def test_distortion_and_shannon_ratio():
    """E||x - R^T c[code]||^2 over random unit vectors matches the Lloyd-Max
    MSE (0.3634 / 0.1175 / 0.03455 per unit vector for B = 1/2/3) and stays
    under e * 2^(-2B) [ICLR 2026 digest, 理論的保証, Theorem 2]."""
    d = 128
    rng = np.random.default_rng(123)
    x = rng.standard_normal((10000, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    for B, mse in ((1, 0.3634), (2, 0.1175), (3, 0.03455)):
        cb = O.make_codebook(d, B + 1, d, 5)
        e = O.encode(cb, x)
        dist = np.mean(e.rho ** 2)            # rho = ||x - x_mse|| for unit x
        assert abs(dist - mse) / mse < 0.03
        assert dist <= math.e * 2.0 ** (-2 * B)
        assert 1.0 < dist / 2.0 ** (-2 * B) < math.e


# ---------------------------------------------------------------- estimator

def test_qjl_estimator_unbiased_and_variance():
    """Fixed q, k, delta; 10^4 independent Gaussian S.  The mean of the
    estimate (with exact norms) is within 3 standard errors of <q, k>, and the
    sample variance matches ((pi/2) ||q||^2 rho^2 - <q, r>^2) / m within a
    chi-square interval [Qiita explainer, Stage 2 estimator; ai.spot.hk,
    無偏內積估計]."""
    d = m = 128
    cb = O.make_codebook(d, 3, m, 42)
    rng = np.random.default_rng(77)
    k = rng.standard_normal(d) * np.exp(rng.normal(0, 0.7, d))
    e0 = O.encode(cb, k[None])
    kmse = e0.nu[0] * (cb.levels[e0.codes[0]] @ cb.R)
    r = k - kmse
    q = rng.standard_normal(d) + 3.0 * r / np.linalg.norm(r)   # <q, r> clearly non-zero
    T = 10000
    est = np.empty(T)
    for t in range(T):
        S = rng.standard_normal((m, d))
        e = O.encode(cb, k[None], S=S)
        assert np.array_equal(e.codes, e0.codes)
        est[t] = O.estimate_inner_product(q, kmse, e.rho[0], S, e.signs[0])
    truth = float(q @ k)
    se = est.std(ddof=1) / math.sqrt(T)
    assert abs(est.mean() - truth) < 3 * se
    rho = np.linalg.norm(r)
    var = ((math.pi / 2) * (q @ q) * rho ** 2 - (q @ r) ** 2) / m
    lo, hi = stats.chi2.ppf([0.0005, 0.9995], T - 1) / (T - 1)
    assert lo < est.var(ddof=1) / var < hi
    # the QJL term carries a sizeable share of <q, k>: a wrong constant or sign shows
    assert abs(q @ r) > 20 * se


def test_score_equals_estimator_on_packed_records():
    """score() reads records from the packed buffer; for every (query, key) it
    equals the Monte-Carlo-pinned estimator above, evaluated on the same
    record's pieces: the MSE reconstruction, the stored half norm of the
    residual, the codebook's S and the stored sign bits [Qiita explainer,
    Stage 2: QJL, estimator equation].  This ties the function every GPU
    logit test compares against to the unbiasedness pin."""
    cb = O.make_codebook(128, 3, 128, 42)
    rng = np.random.default_rng(91)
    G, N, Qg = 2, 37, 3
    k = rng.standard_normal((G, N, 128)) * np.exp(rng.normal(0, 0.7, 128))
    k[1, 5] = 0.0                                  # a zero record among them
    e = O.encode(cb, k.reshape(-1, 128))
    buf = O.pack(cb, e.codes.reshape(G, N, 128), e.signs.reshape(G, N, 128),
                 e.nu16.reshape(G, N), e.rho16.reshape(G, N))
    q = rng.standard_normal((G, Qg, 128))
    lg = O.score(cb, buf, G, N, q)
    codes, signs, nu16, rho16 = O.unpack(cb, buf, G, N)
    kmse = O.decode_mse(cb, buf, G, N)
    for g in range(G):
        for h in range(Qg):
            ref = O.estimate_inner_product(q[g, h][None, :], kmse[g], rho16[g].astype(np.float64),
                                           cb.S, signs[g])
            assert np.allclose(lg[g, h], ref, rtol=0, atol=1e-12)
    assert lg[1, :, 5].tolist() == [0.0] * Qg


def test_qjl_unbiased_with_half_precision_sketch_draws():
    """The sketch the library draws: S = S_rot R with S_rot's entries N(0,1)
    draws rounded to float16.  Over 10^4 independent such sketches, scoring
    a packed record with score() is unbiased for <q, k> (mean within 3
    standard errors, plus the bias the half-precision residual norm can
    carry, bounded below and far smaller) and its variance is the QJL
    variance ((pi/2) ||q||^2 rho^2 - <q, r>^2) / m of a Gaussian sketch
    within a chi-square interval [Qiita explainer, Stage 2: QJL; ai.spot.hk,
    無偏內積估計].  The key's norm is 16 exactly so that the stored half norm
    is exact."""
    import dataclasses
    d = m = 128
    cb0 = O.make_codebook(d, 3, m, 42)
    rng = np.random.default_rng(2024)
    k = rng.standard_normal(d) * np.exp(rng.normal(0, 0.7, d))
    k *= 16.0 / np.linalg.norm(k)
    e0 = O.encode(cb0, k[None])
    assert e0.nu16[0] == np.float16(16.0) and abs(e0.nu[0] - 16.0) < 1e-12
    kmse = e0.nu[0] * (cb0.levels[e0.codes[0]] @ cb0.R)
    r = k - kmse
    rho = float(np.linalg.norm(r))
    q = rng.standard_normal(d) + 3.0 * r / rho
    T = 10000
    est = np.empty(T)
    for t in range(T):
        S_rot = rng.standard_normal((m, d)).astype(np.float16).astype(np.float64)
        cb = dataclasses.replace(cb0, S_rot=S_rot, S=S_rot @ cb0.R)
        e = O.encode(cb, k[None])
        assert np.array_equal(e.codes, e0.codes)
        buf = O.pack(cb, e.codes[None], e.signs[None], e.nu16[None], e.rho16[None])
        est[t] = O.score(cb, buf, 1, 1, q[None, None])[0, 0, 0]
    truth = float(q @ k)
    se = est.std(ddof=1) / math.sqrt(T)
    # the stored residual norm rho~ = half(rho) scales the QJL term, whose
    # mean is <q, r>, by rho~ / rho: a fixed bias of at most 2^-11 |<q, r>|
    bias = abs(float(e0.rho16[0]) / rho - 1.0) * abs(float(q @ r))
    assert bias < 0.2 * se
    assert abs(est.mean() - truth) < 3 * se + bias
    var = ((math.pi / 2) * (q @ q) * rho ** 2 - (q @ r) ** 2) / m
    lo, hi = stats.chi2.ppf([0.0005, 0.9995], T - 1) / (T - 1)
    assert lo < est.var(ddof=1) / var < hi
    assert abs(q @ r) > 20 * se


def test_large_m_estimate_converges():
    """With m = 65536 sketch rows the estimate is within 5 standard
    deviations (~1/sqrt(m)) of the exact inner product."""
    d, m = 64, 65536
    cb = O.make_codebook(d, 3, 32, 1)
    rng = np.random.default_rng(8)
    S = rng.standard_normal((m, d))
    k = rng.standard_normal(d)
    q = rng.standard_normal(d)
    e = O.encode(cb, k[None], S=S)
    kmse = e.nu[0] * (cb.levels[e.codes[0]] @ cb.R)
    est = O.estimate_inner_product(q, kmse, e.rho[0], S, e.signs[0])
    r = k - kmse
    sd = math.sqrt(((math.pi / 2) * (q @ q) * (r @ r) - (q @ r) ** 2) / m)
    assert abs(est - q @ k) < 5 * sd


def test_score_without_qjl_term_is_decode_inner_product():
    """Setting the stored residual norm to 0 leaves exactly <q, decode_mse(k)>."""
    cb = O.make_codebook(128, 4, 128, 42)
    rng = np.random.default_rng(3)
    k = rng.standard_normal((2, 50, 128))
    e = O.encode(cb, k.reshape(-1, 128))
    codes = e.codes.reshape(2, 50, 128)
    signs = e.signs.reshape(2, 50, 128)
    nu16 = e.nu16.reshape(2, 50)
    buf0 = O.pack(cb, codes, signs, nu16, np.zeros((2, 50), np.float16))
    q = rng.standard_normal((2, 3, 128))
    lg = O.score(cb, buf0, 2, 50, q)
    dec = O.decode_mse(cb, buf0, 2, 50)
    assert np.allclose(lg, np.einsum("gqd,gnd->gqn", q, dec), rtol=0, atol=1e-12)


def test_score_unit_query_reads_one_coordinate():
    """q = e_i returns coordinate i of the estimate:
    k_mse_i + rho~ sqrt(pi/2)/m * sum_j S_ji sign_j."""
    cb = O.make_codebook(32, 3, 32, 4)
    k = np.random.default_rng(4).standard_normal((1, 7, 32))
    e = O.encode(cb, k[0])
    buf = O.pack(cb, e.codes[None], e.signs[None], e.nu16[None], e.rho16[None])
    dec = O.decode_mse(cb, buf, 1, 7)[0]
    for i in (0, 13, 31):
        q = np.zeros((1, 1, 32))
        q[0, 0, i] = 1.0
        lg = O.score(cb, buf, 1, 7, q)[0, 0]
        sgn = 1.0 - 2.0 * e.signs
        ref = dec[:, i] + e.rho16.astype(np.float64) * math.sqrt(math.pi / 2) / 32 * (sgn @ cb.S[:, i])
        assert np.allclose(lg, ref, rtol=0, atol=1e-12)


def test_estimate_tracks_exact_logits_on_synthetic_keys():
    """On the outlier-channel keys the 3-bit estimate correlates with the
    exact logits (cosine > 0.95), and 4 bits beat 2 bits."""
    from kv_cache_vector_rotate_amd import workloads as W
    wl = W.workload(0)
    k = W.group_keys(wl, 0)[:1024]
    q = W.group_queries(wl, 0)
    exact = O.exact_logits(k[None], q[None]).ravel()
    cos = {}
    for bits in (2, 3, 4):
        cb = O.make_codebook(128, bits, 128, 42)
        e = O.encode(cb, k)
        buf = O.pack(cb, e.codes[None], e.signs[None], e.nu16[None], e.rho16[None])
        est = O.score(cb, buf, 1, 1024, q[None]).ravel()
        cos[bits] = est @ exact / np.linalg.norm(est) / np.linalg.norm(exact)
    assert cos[3] > 0.95
    assert cos[2] < cos[3] < cos[4]


# ---------------------------------------------------------------- layout

def test_pack_layout_by_hand():
    """Bit positions of the packed record, checked against offsets computed
    by hand from the layout: planes uint32 [G][P][N][d/32], then half2 norms."""
    cb = O.make_codebook(64, 3, 64, 1)
    G, N, d = 2, 3, 64
    codes = np.zeros((G, N, d), np.uint8)
    signs = np.zeros((G, N, d), np.uint8)
    codes[1, 2, 37] = 3          # plane 0 and plane 1, word 1, bit 5
    signs[0, 1, 0] = 1           # plane 2, word 0, bit 0
    signs[1, 0, 63] = 1          # plane 2, word 1, bit 31
    nu16 = np.zeros((G, N), np.float16)
    rho16 = np.zeros((G, N), np.float16)
    nu16[0, 2] = 1.5
    rho16[1, 1] = -2.0
    buf = O.pack(cb, codes, signs, nu16, rho16)
    words = buf[: G * 3 * N * 2 * 4].view(np.uint32)
    expect = np.zeros(G * 3 * N * 2, np.uint32)

    def w(g, p, n, i):
        return ((g * 3 + p) * N + n) * 2 + i
    expect[w(1, 0, 2, 1)] = 1 << 5
    expect[w(1, 1, 2, 1)] = 1 << 5
    expect[w(0, 2, 1, 0)] = 1
    expect[w(1, 2, 0, 1)] = 1 << 31
    assert np.array_equal(words, expect)
    norms = buf[G * 3 * N * 2 * 4:].view(np.uint32)
    assert norms[2] == 0x3E00                 # half(1.5)
    assert norms[N + 1] == 0xC000 << 16       # half(-2.0) in the high half
    c2, s2, n2, r2 = O.unpack(cb, buf, G, N)
    assert np.array_equal(c2, codes) and np.array_equal(s2, signs)
    assert np.array_equal(n2, nu16) and np.array_equal(r2, rho16)


def test_pack_roundtrip_random():
    cb = O.make_codebook(128, 4, 128, 2)
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 8, (3, 5, 128)).astype(np.uint8)
    signs = rng.integers(0, 2, (3, 5, 128)).astype(np.uint8)
    nu16 = rng.standard_normal((3, 5)).astype(np.float16)
    rho16 = rng.standard_normal((3, 5)).astype(np.float16)
    buf = O.pack(cb, codes, signs, nu16, rho16)
    assert buf.size == O.packed_nbytes(cb, 3, 5) == 3 * 5 * (3 * 16 + 16 + 4)
    c, s, n, r = O.unpack(cb, buf, 3, 5)
    assert np.array_equal(c, codes) and np.array_equal(s, signs)
    assert np.array_equal(n.view(np.uint16), nu16.view(np.uint16))


def test_byte_table_matches_community_compression_table():
    """Keys: (b-1)-bit codes + d sign bits + two half norms; values: b-bit
    codes + one half norm.  The Qwen2.5-3B 8K cache then reproduces the
    printed sizes and ratios; float32 norms would not."""
    ref = json.load(open(os.path.join(GOLDEN, "qiita_compression_table.json")))
    s = ref["model_shape"]
    vecs = s["layers"] * s["kv_heads"] * s["context"]
    fp16 = vecs * s["head_dim"] * 2 * 2
    assert fp16 == 301989888                                  # 288.0 MiB
    for row in ref["rows"]:
        kb, vb = O.kv_bytes_per_vector(s["head_dim"], row["bits"])
        tot = vecs * (kb + vb)
        assert round(fp16 / tot, 1) == row["ratio"]
        assert math.ceil(tot / 2 ** 20) == row["MB"]
        tot32 = vecs * (kb + 4 + vb + 2)                      # fp32 norms instead
        assert math.ceil(tot32 / 2 ** 20) != row["MB"]


# ---------------------------------------------------------------- helpers

def test_top_k_orders_ties_by_index():
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, -1.0]])
    idx, val = O.top_k(s, 4)
    assert idx.tolist() == [[1, 2, 4, 3]]
    assert val.tolist() == [[3.0, 3.0, 3.0, 2.0]]


def test_fp16_midpoint_flag():
    a = np.float16(1.0)
    b = np.nextafter(a, np.float16(2))
    mid = (float(a) + float(b)) / 2
    f = O.fp16_midpoint_flag(np.array([mid, mid * (1 + 2e-6), float(a), 1.0003]))
    assert f.tolist() == [True, False, False, False]


def test_exact_zero_coordinates_take_the_upper_middle_level():
    """k = e_0 + e_1 rotates to coordinates (+-delta_0 +- delta_1)/(sqrt(2d)),
    exactly zero on half of them (Sylvester rows i and the sign pattern of
    delta); a value on the middle threshold 0 goes up, to level L/2."""
    d = 128
    for bits in (2, 3, 4):
        cb = O.make_codebook(d, bits, d, 42)
        k = np.zeros((1, d))
        k[0, :2] = 1.0
        e = O.encode(cb, k)
        H = O.sylvester_hadamard(d)
        zero = (cb.delta[0] * H[:, 0] + cb.delta[1] * H[:, 1]) == 0
        assert zero.sum() == d // 2
        assert np.all(e.y[0][zero] == 0.0)
        assert np.all(e.codes[0][zero] == cb.L // 2)
        assert np.allclose(np.abs(e.y[0][~zero]), 1.0 / math.sqrt(d // 2), rtol=1e-15)

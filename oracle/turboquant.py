"""Plain fp64 reference of the TurboQuant key path.  TEST INFRASTRUCTURE ONLY.

Sources (cited by page title and section; see oracle/__init__.py):

* [Qiita explainer]   "TurboQuant" explainer on qiita.com (kai_kou): sections
  "Stage 1: PolarQuant", "Stage 2: QJL" (estimator equation), the community
  compression table ("圧縮率（8Kコンテキスト、FP16ベースライン289MB）").
* [ai.spot.hk]        "Google TurboQuant：LLM KV Cache 壓縮 6 倍…": sections
  "隨機旋轉與Beta分佈" (per-coordinate quantisation after a random rotation) and
  "無偏內積估計" (TURBOQUANT_prod: (b-1)-bit MSE stage + 1-bit QJL, total b
  bits, unbiased inner products).
* [ICLR 2026 digest]  "ICLR 2026論文解説: TurboQuant — Shannon限界に迫る…":
  "Step 1: PolarQuant" (normalise, rotate, R = H_d D / sqrt(d), Sylvester
  recursion, coordinates ~ N(0, 1/d)), "理論的保証" (Theorem 2),
  "実装の擬似コード" (zero-vector rule, sign convention 0 = positive),
  "実装のポイント" (norm stored on the side, 8 sign bits per byte).

Readings where the pages are silent or disagree:

* b counts all bits: (b-1) Lloyd-Max bits + 1 QJL bit per coordinate.
* the codebook is Lloyd-Max for N(0, 1/d); the middle threshold is exactly 0.
* code_i = number of thresholds t_j with y_i >= t_j (a tie goes up).
* QJL sign bit = [ (S r)_j < 0 ]  (0 = positive, -0.0 counts as positive).
* S has i.i.d. N(0, 1) entries, m rows; r is formed in the original domain.
  S is drawn as S = S_rot R with S_rot's entries N(0, 1) draws rounded to
  float16: the same law (R is orthogonal) up to that rounding.
* both norms are stored as IEEE half (round to nearest even) and the
  estimator uses the stored values.
* delta and S come from a counter-based SplitMix64 stream (below), not from
  numpy's RandomState: only their distribution matters to the method.
* a dimension d that is not a power of two is zero-padded to the next power
  of two D and the method runs in D dimensions (delta of length D, S with
  m = D rows over D columns, the N(0, 1/D) codebook); decoded vectors keep
  their first d coordinates [ICLR 2026 digest, 実装のポイント: zero padding
  to the nearest power of two for the Hadamard transform].
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "splitmix64_draw", "rademacher_signs", "gaussian_sketch",
    "sylvester_hadamard", "rotation_matrix", "lloyd_max_std_normal",
    "Codebook", "make_codebook", "EncodeResult", "encode", "pack", "unpack",
    "packed_nbytes", "decode_mse", "score", "estimate_inner_product",
    "exact_logits", "top_k", "fp16_midpoint_flag", "ZERO_NORM",
    "FLAG_BAND", "kv_bytes_per_vector",
    "lloyd_max_beta", "haar_rotation", "rotation_dim", "value_quantizer", "ValueEncodeResult", "encode_values", "value_packed_nbytes",
    "value_group_size", "value_slot_coordinate",
    "pack_values", "unpack_values", "decode_values", "attention_from_logits", "attention",
]

ZERO_NORM = 1e-10      # zero-vector rule [ICLR 2026 digest, 実装の擬似コード]
FLAG_BAND = 1e-6       # decision-boundary band used to flag parity cases

_U64 = np.uint64
_GAMMA = 0x9E3779B97F4A7C15          # SplitMix64 increment (Steele, Lea & Flood 2014)
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1


# --------------------------------------------------------------------------
# Seeded randomness: counter-based SplitMix64 (published generator).
# --------------------------------------------------------------------------

def _mix64_int(z: int) -> int:
    """SplitMix64 output finaliser on one Python integer (mod 2**64)."""
    z &= _MASK
    z = ((z ^ (z >> 30)) * _M1) & _MASK
    z = ((z ^ (z >> 27)) * _M2) & _MASK
    return z ^ (z >> 31)


def _mix64_arr(z: np.ndarray) -> np.ndarray:
    z = z.astype(_U64, copy=True)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> _U64(30))) * _U64(_M1)
        z = (z ^ (z >> _U64(27))) * _U64(_M2)
    return z ^ (z >> _U64(31))


def splitmix64_draw(seed: int, stream: int, index) -> np.ndarray:
    """Draw number ``index`` of stream ``stream`` for ``seed`` (uint64).

    base  = mix64(seed + stream * GAMMA)
    draw  = mix64(base + (index + 1) * GAMMA)       (all mod 2**64)

    i.e. the index-th output of a SplitMix64 sequence whose seed is itself
    the stream-th SplitMix64 output of ``seed``.  Parity unpinned beyond the
    two independent implementations of this definition agreeing bit for bit.
    """
    base = _mix64_int(seed + stream * _GAMMA)
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = _U64(base) + (idx + _U64(1)) * _U64(_GAMMA)
    return _mix64_arr(state)


def rademacher_signs(seed: int, d: int) -> np.ndarray:
    """delta_i in {+1, -1}: +1 when bit 63 of draw (stream 1, index i) is 0.

    The Rademacher diagonal D of the rotation [ICLR 2026 digest, Step 1:
    D has independent +-1 entries with equal probability].
    """
    x = splitmix64_draw(seed, 1, np.arange(d, dtype=np.uint64))
    return np.where((x >> _U64(63)) == 0, 1, -1).astype(np.int8)


def gaussian_sketch(seed: int, m: int, d: int) -> np.ndarray:
    """G[j, i] ~ N(0, 1) by Box-Muller from stream-2 draws 2(jd+i), 2(jd+i)+1.

    u1 = ((x >> 11) + 1) * 2**-53 in (0, 1], u2 = (y >> 11) * 2**-53 in [0, 1),
    z = sqrt(-2 ln u1) cos(2 pi u2), rounded to float16 (nearest even).  The
    QJL projection is a Gaussian random matrix [Qiita explainer, Stage 2];
    make_codebook uses G as the sketch seen from the rotated domain,
    S R^T = G.  libm's log/cos (math module) are used so that the host
    library, which also calls libm, draws the same fp64 values.
    """
    n = m * d
    draws = splitmix64_draw(seed, 2, np.arange(2 * n, dtype=np.uint64))
    xs = (draws[0::2] >> _U64(11)).tolist()
    ys = (draws[1::2] >> _U64(11)).tolist()
    two53 = 2.0 ** -53
    out = np.empty(n, dtype=np.float64)
    log, cos, sqrt, tau = math.log, math.cos, math.sqrt, 2.0 * math.pi
    for t in range(n):
        u1 = (xs[t] + 1) * two53
        u2 = ys[t] * two53
        out[t] = sqrt(-2.0 * log(u1)) * cos(tau * u2)
    return out.astype(np.float16).reshape(m, d)


# --------------------------------------------------------------------------
# Rotation: R = H_d D / sqrt(d)  [ICLR 2026 digest, Step 1, eq. for R].
# --------------------------------------------------------------------------

def sylvester_hadamard(d: int) -> np.ndarray:
    """H_1 = [1];  H_2n = [[H_n, H_n], [H_n, -H_n]]  (integer matrix)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(delta: np.ndarray) -> np.ndarray:
    """Dense R = H_d diag(delta) / sqrt(d) in float64."""
    d = delta.shape[0]
    return sylvester_hadamard(d).astype(np.float64) * delta.astype(np.float64)[None, :] / math.sqrt(d)


# --------------------------------------------------------------------------
# Lloyd-Max quantizer for N(0, 1), then scaled to N(0, 1/d).
# --------------------------------------------------------------------------

def _phi(x: float) -> float:
    return 0.0 if math.isinf(x) else math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _upper_tail(x: float) -> float:
    """P(X >= x) for X ~ N(0,1), via erfc to keep tail accuracy."""
    return 0.0 if math.isinf(x) else 0.5 * math.erfc(x / math.sqrt(2.0))


def lloyd_max_std_normal(B: int, tol: float = 1e-15, max_iter: int = 100000):
    """(levels[2**B], thresholds[2**B - 1]) of the MSE-optimal quantizer of N(0,1).

    Lloyd's two conditions, iterated to a fixed point: every threshold is the
    midpoint of its two neighbouring levels, every level is the conditional
    mean of its cell, E[X | a <= X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
    The law is symmetric and L is even, so the iteration runs on the positive
    half with the middle threshold fixed at exactly 0 and the negative half
    mirrored.  Shared by all coordinates, "zero memory overhead"
    [Qiita explainer, Stage 1 step 3; ICLR 2026 digest, Step 1].
    """
    if B < 1:
        raise ValueError("B >= 1")
    K = (1 << B) // 2                      # levels on the positive half
    c = [0.5 + 2.0 * (k + 0.5) / K for k in range(K)]   # any increasing start
    for _ in range(max_iter):
        t = [0.0] + [(c[k - 1] + c[k]) / 2.0 for k in range(1, K)] + [math.inf]
        new = []
        for k in range(K):
            a, b = t[k], t[k + 1]
            mass = _upper_tail(a) - _upper_tail(b)
            new.append((_phi(a) - _phi(b)) / mass)
        delta = max(abs(x - y) for x, y in zip(new, c))
        c = new
        if delta < tol:
            break
    pos_levels = np.array(c, dtype=np.float64)
    pos_thr = np.array([(c[k - 1] + c[k]) / 2.0 for k in range(1, K)], dtype=np.float64)
    levels = np.concatenate([-pos_levels[::-1], pos_levels])
    thresholds = np.concatenate([-pos_thr[::-1], [0.0], pos_thr])
    return levels, thresholds


def lloyd_max_beta(d: int, B: int, tol: float = 1e-15, max_iter: int = 200000):
    """(levels, thresholds) of the MSE-optimal 2**B-level quantizer for one
    coordinate of a uniformly random unit vector in R^d, the law the pages
    give for a rotated coordinate before its Gaussian limit [ai.spot.hk,
    隨機旋轉與Beta分佈; ICLR 2026 digest, Step 1]: density proportional to
    (1 - y^2)^((d-3)/2) on [-1, 1] (y^2 ~ Beta(1/2, (d-1)/2)).

    The same two Lloyd conditions as :func:`lloyd_max_std_normal`, on the
    positive half with the middle threshold fixed at 0: a cell's mass is
    P(|Y| <= y) = I_{y^2}(1/2, (d-1)/2) (the regularised incomplete beta
    function), and its first moment has the closed form
    int_a^b y (1 - y^2)^((d-3)/2) dy = ((1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)) / (d-1).
    Scale: unit-vector coordinates (no 1/sqrt(d) factor to apply)."""
    from scipy import special
    if d < 2 or B < 1:
        raise ValueError("d >= 2, B >= 1")
    K = (1 << B) // 2
    h = (d - 1) / 2.0
    # normalising constant of the density on [-1, 1]
    cnorm = math.exp(special.gammaln(d / 2.0) - special.gammaln(h) - 0.5 * math.log(math.pi))

    def upper(y):          # P(Y >= y) for y >= 0, via the complementary incomplete beta
        return 0.0 if y >= 1.0 else 0.5 * special.betainc(h, 0.5, 1.0 - y * y)

    def moment(a, b):      # int_a^b y f(y) dy, 0 <= a <= b <= 1
        fa = (1.0 - a * a) ** h if a < 1.0 else 0.0
        fb = (1.0 - b * b) ** h if b < 1.0 else 0.0
        return cnorm * (fa - fb) / (d - 1)

    sd = 1.0 / math.sqrt(d)
    c = [sd * (0.5 + 2.0 * (k + 0.5) / K) / 2.0 for k in range(K)]
    for _ in range(max_iter):
        t = [0.0] + [(c[k - 1] + c[k]) / 2.0 for k in range(1, K)] + [1.0]
        new = [moment(t[k], t[k + 1]) / (upper(t[k]) - upper(t[k + 1])) for k in range(K)]
        delta = max(abs(x - y) for x, y in zip(new, c))
        c = new
        if delta < tol * sd:
            break
    pos_levels = np.array(c, dtype=np.float64)
    pos_thr = np.array([(c[k - 1] + c[k]) / 2.0 for k in range(1, K)], dtype=np.float64)
    return (np.concatenate([-pos_levels[::-1], pos_levels]),
            np.concatenate([-pos_thr[::-1], [0.0], pos_thr]))


def haar_rotation(seed: int, d: int) -> np.ndarray:
    """A Haar-distributed orthogonal matrix (QR of a Gaussian matrix with the
    signs of R's diagonal moved into Q).  Cross-check only: the library uses
    the randomized Hadamard rotation of the pages; under a Haar rotation each
    rotated coordinate has exactly the Beta law of :func:`lloyd_max_beta`."""
    g = np.random.default_rng(seed).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


# --------------------------------------------------------------------------
# Codebook = every piece of quantizer state derived from (d, b, m, seed).
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Codebook:
    d: int
    bits: int            # total bits per coordinate: (bits-1) Lloyd-Max + 1 QJL
    m: int               # QJL sketch rows
    seed: int
    levels: np.ndarray   # [L] ascending, for N(0, 1/d)
    thresholds: np.ndarray  # [L-1] ascending
    delta: np.ndarray    # [d] int8 Rademacher signs
    S: np.ndarray        # [m, d] float64 sketch, S = S_rot R
    R: np.ndarray        # [d, d] float64 dense rotation
    S_rot: np.ndarray    # [m, d] float64 = S R^T: float16-rounded N(0,1) draws
    kind: str = "gaussian"   # coordinate law of the Lloyd-Max tables: "gaussian" or "beta"
    d_in: int = 0        # length of input rows when they are zero-padded to d (0: d)

    @property
    def din(self) -> int:
        """Length of the vectors the caller passes (and gets back)."""
        return self.d_in or self.d

    @property
    def B(self) -> int:
        return self.bits - 1

    @property
    def L(self) -> int:
        return 1 << (self.bits - 1)


def _lloyd_tables(d: int, B: int, kind: str):
    """Lloyd-Max levels/thresholds on the unit-vector coordinate scale."""
    if kind == "gaussian":
        lv, th = lloyd_max_std_normal(B)
        return lv / math.sqrt(d), th / math.sqrt(d)
    if kind == "beta":
        return lloyd_max_beta(d, B)
    raise ValueError(kind)


def rotation_dim(d: int) -> int:
    """The power of two the method runs in for d-dimensional vectors: d
    itself, or the next power of two (zero padding) [ICLR 2026 digest,
    実装のポイント]."""
    if d < 1:
        raise ValueError("d >= 1")
    return 1 << (d - 1).bit_length()


def _pad_rows(cb: Codebook, x) -> np.ndarray:
    """Rows of length cb.din as float64, zero-padded to cb.d."""
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == cb.din, (x.shape, cb.din)
    if cb.din == cb.d:
        return x
    out = np.zeros(x.shape[:-1] + (cb.d,))
    out[..., :cb.din] = x
    return out


def make_codebook(d: int, bits: int, m: int, seed: int, kind: str = "gaussian") -> Codebook:
    """Quantizer state: Lloyd-Max for N(0,1/d) with L = 2**(bits-1) levels
    (scale equivariance: N(0,1) levels times 1/sqrt(d)), delta and S from the
    seed, and the dense rotation.  [ai.spot.hk, 無偏內積估計: (b-1)-bit MSE
    stage; ICLR 2026 digest, Step 1: coordinates ~ N(0, 1/d)].

    The sketch is drawn in the rotated basis: S_rot has i.i.d. N(0,1)
    entries (rounded to float16) and S = S_rot R.  R is orthogonal, so S has
    the same i.i.d. N(0,1) law [Qiita explainer, Stage 2: Gaussian random
    projection], and S r = S_rot (R r).

    A d that is not a power of two gives the codebook of D = rotation_dim(d)
    (same seed, so the same delta, S and levels) that takes rows of length d
    and zero-pads them."""
    if bits < 2:
        raise ValueError("bits >= 2 (one bit is the QJL sign)")
    d_in, d = d, rotation_dim(d)
    lv, th = _lloyd_tables(d, bits - 1, kind)
    delta = rademacher_signs(seed, d)
    R = rotation_matrix(delta)
    S_rot = gaussian_sketch(seed, m, d).astype(np.float64)
    return Codebook(d=d, bits=bits, m=m, seed=seed, levels=lv, thresholds=th, delta=delta,
                    S=S_rot @ R, R=R, S_rot=S_rot, kind=kind, d_in=d_in if d_in != d else 0)


# --------------------------------------------------------------------------
# Encode  [ICLR 2026 digest, Step 1 + 実装の擬似コード; Qiita explainer,
# Stage 2; ai.spot.hk, 無偏內積估計].
# --------------------------------------------------------------------------

@dataclasses.dataclass
class EncodeResult:
    codes: np.ndarray      # [n, d] uint8 level index
    signs: np.ndarray      # [n, m] uint8, 1 = (S r)_j < 0
    nu: np.ndarray         # [n] fp64 ||k||
    rho: np.ndarray        # [n] fp64 ||k - k_mse||
    nu16: np.ndarray       # [n] float16 stored norm
    rho16: np.ndarray      # [n] float16 stored residual norm
    y: np.ndarray          # [n, d] rotated unit key
    p: np.ndarray          # [n, m] S r
    zero: np.ndarray       # [n] bool: zero-vector rule applied
    code_flag: np.ndarray  # [n, d] y within FLAG_BAND of a threshold
    sign_flag: np.ndarray  # [n, m] |p|/nu within FLAG_BAND of 0
    nu16_flag: np.ndarray  # [n] nu within FLAG_BAND (relative) of an fp16 midpoint
    rho16_flag: np.ndarray
    zero_flag: np.ndarray  # [n] nu within FLAG_BAND (relative) of ZERO_NORM


def fp16_midpoint_flag(v: np.ndarray, band: float = FLAG_BAND) -> np.ndarray:
    """True where v lies within ``band`` (relative) of a point halfway
    between two adjacent float16 values, i.e. where float32 and float64
    rounding to half may legitimately disagree by one ulp."""
    v = np.asarray(v, dtype=np.float64)
    lo = v.astype(np.float16)
    lo = np.where(lo.astype(np.float64) > v, np.nextafter(lo, np.float16(-np.inf)), lo)
    hi = np.nextafter(lo, np.float16(np.inf))
    mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2.0
    return np.abs(v - mid) <= band * np.abs(v)


def quantize_rotated(cb: Codebook, y: np.ndarray) -> np.ndarray:
    """code = #{j : y >= t_j}  (levels ascending, ties go up)."""
    return np.searchsorted(cb.thresholds, y, side="right").astype(np.uint8)


def encode(cb: Codebook, keys: np.ndarray, S: Optional[np.ndarray] = None,
           codes: Optional[np.ndarray] = None) -> EncodeResult:
    """Encode rows of ``keys`` ([n, din], any float dtype, used as exact fp64;
    zero-padded to d when din < d).

    Per key k: nu = ||k||; if nu < 1e-10 the record is all zero.  Otherwise
    x = k / nu, y = R x, code_i = #{t_j <= y_i}, k_mse = nu R^T c[code],
    r = k - k_mse, rho = ||r||, p = S r, sign bit_j = [p_j < 0];
    nu and rho are stored as float16.  ``S`` overrides the codebook's sketch
    (Monte-Carlo tests); ``codes`` ([n, d]) replaces the threshold decision
    so that the residual stage can be recomputed for codes another encoder
    chose at a flagged boundary coordinate.
    """
    S = cb.S if S is None else np.asarray(S, dtype=np.float64)
    k = _pad_rows(cb, keys)
    n, d = k.shape
    assert d == cb.d
    nu = np.sqrt(np.sum(k * k, axis=1))
    zero = nu < ZERO_NORM
    safe = np.where(zero, 1.0, nu)
    # y = R x = H_d (D k) / (nu sqrt(d)): the integer matrix H_d is applied to
    # D k first, so a coordinate that is exactly zero stays exactly zero (fp64
    # sums of float32/bf16 inputs are exact) and the tie rule sees it as such.
    H = sylvester_hadamard(d).astype(np.float64)
    u = (k * cb.delta.astype(np.float64)[None, :]) @ H.T
    y = u / (safe[:, None] * math.sqrt(d))
    codes = quantize_rotated(cb, y) if codes is None else np.array(codes, dtype=np.uint8)
    yhat = cb.levels[codes]
    k_mse = safe[:, None] * (yhat @ cb.R)            # nu R^T yhat
    r = k - k_mse
    rho = np.sqrt(np.sum(r * r, axis=1))
    p = r @ S.T                                      # S r
    signs = (p < 0).astype(np.uint8)
    codes[zero] = 0
    signs[zero] = 0
    rho = np.where(zero, 0.0, rho)
    nu_st = np.where(zero, 0.0, nu)
    dist = np.min(np.abs(y[:, :, None] - cb.thresholds[None, None, :]), axis=2)
    code_flag = (dist <= FLAG_BAND) & ~zero[:, None]
    sign_flag = (np.abs(p) / safe[:, None] <= FLAG_BAND) & ~zero[:, None]
    return EncodeResult(
        codes=codes, signs=signs, nu=nu_st, rho=rho,
        nu16=nu_st.astype(np.float16), rho16=rho.astype(np.float16),
        y=y, p=p, zero=zero, code_flag=code_flag, sign_flag=sign_flag,
        nu16_flag=fp16_midpoint_flag(nu_st) & ~zero,
        rho16_flag=fp16_midpoint_flag(rho) & ~zero,
        zero_flag=np.abs(nu - ZERO_NORM) <= FLAG_BAND * ZERO_NORM)


# --------------------------------------------------------------------------
# Packed layout (the library's record format, implemented here on its own).
#   planes: uint32 [G][P][N][d/32], P = bits; planes 0..bits-2 hold code bit
#           p (LSB first), plane bits-1 holds the QJL sign bits (m = d);
#           bit j of word w is coordinate (or sketch row) 32 w + j;
#   then norms: uint32 [G][N] = half(nu) | half(rho) << 16.
# Eight sign bits per byte [ICLR 2026 digest, 実装のポイント].
# --------------------------------------------------------------------------

def packed_nbytes(cb: Codebook, G: int, N: int) -> int:
    return G * N * (cb.B * cb.d // 8 + cb.m // 8 + 4)


def _bits_to_words(bits: np.ndarray) -> np.ndarray:
    """[..., 32 W] of 0/1 -> [..., W] uint32 with bit j of word w = element 32w+j."""
    sh = bits.shape
    b = bits.reshape(sh[:-1] + (sh[-1] // 32, 32)).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (b * weights).sum(axis=-1).astype(np.uint32)


def _words_to_bits(words: np.ndarray) -> np.ndarray:
    w = words.astype(np.uint64)[..., None]
    bits = (w >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(words.shape[:-1] + (words.shape[-1] * 32,)).astype(np.uint8)


def pack(cb: Codebook, codes, signs, nu16, rho16) -> np.ndarray:
    """codes [G,N,d], signs [G,N,m], nu16/rho16 [G,N] -> uint8 buffer."""
    assert cb.m == cb.d, "the packed layout stores m = d sign bits"
    codes = np.asarray(codes, dtype=np.uint8)
    G, N, d = codes.shape
    planes = np.empty((G, cb.bits, N, d // 32), dtype=np.uint32)
    for p in range(cb.B):
        planes[:, p] = _bits_to_words((codes >> p) & 1)
    planes[:, cb.B] = _bits_to_words(np.asarray(signs, dtype=np.uint8))
    nb = np.asarray(nu16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    rb = np.asarray(rho16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    norms = (nb | (rb << np.uint32(16))).astype(np.uint32)
    out = np.concatenate([planes.reshape(-1).view(np.uint8), norms.reshape(-1).view(np.uint8)])
    assert out.size == packed_nbytes(cb, G, N)
    return out


def unpack(cb: Codebook, buf: np.ndarray, G: int, N: int):
    """Inverse of :func:`pack`: (codes [G,N,d], signs [G,N,m], nu16, rho16)."""
    buf = np.ascontiguousarray(np.asarray(buf).reshape(-1).view(np.uint8))
    assert buf.size == packed_nbytes(cb, G, N)
    d = cb.d
    nplane = G * cb.bits * N * (d // 32)
    planes = buf[: nplane * 4].view(np.uint32).reshape(G, cb.bits, N, d // 32)
    norms = buf[nplane * 4:].view(np.uint32).reshape(G, N)
    codes = np.zeros((G, N, d), dtype=np.uint8)
    for p in range(cb.B):
        codes |= (_words_to_bits(planes[:, p]) << p).astype(np.uint8)
    signs = _words_to_bits(planes[:, cb.B])
    nu16 = (norms & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    rho16 = (norms >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return codes, signs, nu16, rho16


# --------------------------------------------------------------------------
# Decode and score.
# --------------------------------------------------------------------------

def decode_mse(cb: Codebook, buf: np.ndarray, G: int, N: int) -> np.ndarray:
    """k_mse = nu~ R^T c[code] for every record: [G, N, din] fp64 (the first
    din coordinates).  The MSE-only reconstruction (what the community API
    calls the MSE compressor [Qiita explainer, API table])."""
    codes, _, nu16, _ = unpack(cb, buf, G, N)
    return (nu16.astype(np.float64)[..., None] * (cb.levels[codes] @ cb.R))[..., :cb.din]


def estimate_inner_product(q, k_mse, rho, S, sign_bits) -> np.ndarray:
    """<q, k_mse> + rho * sqrt(pi/2) / m * <S q, sign(S r)>
    [Qiita explainer, Stage 2: QJL, estimator equation].

    q [..., d]; k_mse [..., d]; rho [...]; S [m, d]; sign_bits [..., m] with
    1 meaning a negative projection.  Broadcasting over leading axes."""
    m = S.shape[0]
    q = np.asarray(q, dtype=np.float64)
    sgn = 1.0 - 2.0 * np.asarray(sign_bits, dtype=np.float64)
    return (np.sum(q * k_mse, axis=-1)
            + np.asarray(rho, dtype=np.float64) * math.sqrt(math.pi / 2.0) / m
            * np.sum((q @ S.T) * sgn, axis=-1))


def score(cb: Codebook, buf: np.ndarray, G: int, N: int, q: np.ndarray) -> np.ndarray:
    """Logits [G, Qg, N] of queries q [G, Qg, din] against the packed keys of
    their group, from the stored record only (so it can score any producer's
    buffer).  Queries stay full precision; keys are never dequantised by the
    estimator's definition beyond k_mse."""
    q = _pad_rows(cb, q)
    codes, signs, nu16, rho16 = unpack(cb, buf, G, N)
    k_mse = nu16.astype(np.float64)[..., None] * (cb.levels[codes] @ cb.R)   # [G,N,d]
    sgn = 1.0 - 2.0 * signs.astype(np.float64)                                # [G,N,m]
    sq = q @ cb.S.T                                                           # [G,Qg,m]
    mse = np.einsum("gqd,gnd->gqn", q, k_mse)
    qjl = np.einsum("gqm,gnm->gqn", sq, sgn)
    return mse + rho16.astype(np.float64)[:, None, :] * math.sqrt(math.pi / 2.0) / cb.m * qjl


def exact_logits(keys: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unquantised q . k in fp64: keys [G, N, d], q [G, Qg, d] -> [G, Qg, N]."""
    return np.einsum("gqd,gnd->gqn", np.asarray(q, np.float64), np.asarray(keys, np.float64))


def top_k(scores: np.ndarray, k: int):
    """Per row: the k largest scores, ordered by score descending and then by
    index ascending.  Returns (indices int64, values)."""
    s = np.asarray(scores)
    n = s.shape[-1]
    idx = np.lexsort((np.broadcast_to(np.arange(n), s.shape), -s), axis=-1)[..., :k]
    return idx, np.take_along_axis(s, idx, axis=-1)


# --------------------------------------------------------------------------
# Byte accounting of the packed cache (keys) and an MSE-only value cache.
# --------------------------------------------------------------------------

def kv_bytes_per_vector(d: int, bits: int):
    """(key bytes, value bytes) per cached vector: keys hold (bits-1)-bit codes,
    d sign bits and two half norms; values hold bits-bit MSE codes and one
    half norm.  Reproduces the community compression table on the Qiita
    explainer only with half-precision norms."""
    key = (bits - 1) * d // 8 + d // 8 + 4
    val = bits * d // 8 + 2
    return key, val


# --------------------------------------------------------------------------
# Value path: MSE-only compression of value vectors and decode attention
# over packed keys and values.  The community implementation on the Qiita
# explainer (API table) compresses values with the Stage-1 quantizer alone
# (rotation + Lloyd-Max, "TurboQuantCompressorMSE"); its byte table counts
# b-bit value codes plus one half-precision norm per value (reproduced by
# kv_bytes_per_vector).  Readings: values use the same rotation R as keys
# and a b-bit Lloyd-Max quantizer for N(0, 1/d) (all b bits, no QJL bit);
# attention is softmax(scale * logits) V with scale = 1/sqrt(d) by default
# (scaled dot-product attention; the pages do not restate it).
# --------------------------------------------------------------------------

_VQ_CACHE = {}


def value_quantizer(cb: Codebook):
    """(levels [2**bits], thresholds [2**bits - 1]) of the b-bit value
    quantizer: Lloyd-Max for N(0,1) times 1/sqrt(d)."""
    key = (cb.bits, cb.d, cb.kind)
    if key not in _VQ_CACHE:
        _VQ_CACHE[key] = _lloyd_tables(cb.d, cb.bits, cb.kind)
    return _VQ_CACHE[key]


@dataclasses.dataclass
class ValueEncodeResult:
    codes: np.ndarray      # [n, d] uint8 level index (bits bits)
    nu: np.ndarray         # [n] fp64 ||v||
    nu16: np.ndarray       # [n] float16 stored norm
    y: np.ndarray          # [n, d] rotated unit value
    zero: np.ndarray       # [n] bool
    code_flag: np.ndarray  # [n, d] y within FLAG_BAND of a threshold
    nu16_flag: np.ndarray  # [n]


def encode_values(cb: Codebook, values: np.ndarray) -> ValueEncodeResult:
    """Per value v: nu = ||v|| (zero record below ZERO_NORM), y = R v / nu,
    code_i = #{t_j <= y_i} over the b-bit thresholds, nu stored as float16
    [Qiita explainer, API table (value compression = Stage 1); ICLR 2026
    digest, Step 1 and the zero-vector rule]."""
    lv, th = value_quantizer(cb)
    v = _pad_rows(cb, values)
    n, d = v.shape
    assert d == cb.d
    nu = np.sqrt(np.sum(v * v, axis=1))
    zero = nu < ZERO_NORM
    safe = np.where(zero, 1.0, nu)
    H = sylvester_hadamard(d).astype(np.float64)
    u = (v * cb.delta.astype(np.float64)[None, :]) @ H.T      # exact zeros stay exact
    y = u / (safe[:, None] * math.sqrt(d))
    codes = np.searchsorted(th, y, side="right").astype(np.uint8)
    codes[zero] = 0
    nu_st = np.where(zero, 0.0, nu)
    dist = np.min(np.abs(y[:, :, None] - th[None, None, :]), axis=2)
    return ValueEncodeResult(codes=codes, nu=nu_st, nu16=nu_st.astype(np.float16), y=y, zero=zero,
                             code_flag=(dist <= FLAG_BAND) & ~zero[:, None],
                             nu16_flag=fp16_midpoint_flag(nu_st) & ~zero)


# Packed value layout (a storage format of this library; the pages fix only
# its size, b-bit codes and one half norm per value).  Values are grouped in
# tiles of 16 consecutive values of a group, T = ceil(N / 16) tiles per group:
#   codes: uint32 [G][T][bits * d / 2]: tile t holds values 16 t .. 16 t + 15
#          (values past N have code 0); its 16 * bits * d bits (bit k is bit
#          k % 32 of word k // 32) are d slots of 16 * bits bits, slot s holding
#          coordinate value_slot_coordinate(s).  A slot is a row of 8 groups
#          of K = value_group_size(bits) = 2 values: group q holds values 2 q
#          and 2 q + 1 in 2 * bits bits, bit 2 p + i of the group being bit p
#          of the code of value 2 q + i.
#   norms: uint16 [G][N] = half(nu).
# So one slot group is the index of a table of value pairs.

def value_group_size(bits: int) -> int:
    """Values per slot group (2: a group is a 2 * bits-bit table index)."""
    return 2


def value_slot_coordinate(s: np.ndarray) -> np.ndarray:
    """Coordinate held by slot s of a value tile: 32 (s // 32) + 16 (s % 2) +
    (s % 32) // 2."""
    s = np.asarray(s)
    return 32 * (s // 32) + 16 * (s % 2) + (s % 32) // 2


def value_packed_nbytes(cb: Codebook, G: int, N: int) -> int:
    T = (N + 15) // 16
    return G * (T * 16 * cb.bits * cb.d // 8 + 2 * N)


def _value_tile_bits(cb: Codebook, codes: np.ndarray) -> np.ndarray:
    """codes [G, T*16, d] -> bits [G, T, 16 * bits * d] in stream order."""
    G, NP, d = codes.shape
    b, K = cb.bits, value_group_size(cb.bits)
    T = NP // 16
    planes = (codes[..., None] >> np.arange(b, dtype=np.uint8)) & 1          # [G, NP, d, b]
    planes = planes[:, :, value_slot_coordinate(np.arange(d)), :]           # coordinate -> slot
    t = planes.reshape(G, T, 16 // K, K, d, b)                             # [G, T, q, i, slot, p]
    return t.transpose(0, 1, 4, 2, 5, 3).reshape(G, T, 16 * b * d)        # [slot][q][p][i]


def pack_values(cb: Codebook, codes, nu16) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    G, N, d = codes.shape
    T = (N + 15) // 16
    padded = np.zeros((G, T * 16, d), np.uint8)
    padded[:, :N] = codes
    words = _bits_to_words(_value_tile_bits(cb, padded))
    norms = np.asarray(nu16, dtype=np.float16).reshape(G, N).view(np.uint16)
    return np.concatenate([words.reshape(-1).view(np.uint8), norms.reshape(-1).view(np.uint8)])


def unpack_values(cb: Codebook, buf: np.ndarray, G: int, N: int):
    """Inverse of :func:`pack_values`: (codes [G, N, d], nu16 [G, N])."""
    buf = np.ascontiguousarray(np.asarray(buf).reshape(-1).view(np.uint8))
    assert buf.size == value_packed_nbytes(cb, G, N)
    d, b, K = cb.d, cb.bits, value_group_size(cb.bits)
    T = (N + 15) // 16
    nword = G * T * 16 * b * d // 32
    bits = _words_to_bits(buf[: nword * 4].view(np.uint32).reshape(G, T, 16 * b * d // 32))
    t = bits.reshape(G, T, d, 16 // K, b, K).transpose(0, 1, 3, 5, 2, 4)    # [G, T, q, i, slot, p]
    planes = t.reshape(G, T * 16, d, b)
    codes_slot = (planes.astype(np.uint8) << np.arange(b, dtype=np.uint8)).sum(axis=-1).astype(np.uint8)
    codes = np.empty_like(codes_slot)
    codes[:, :, value_slot_coordinate(np.arange(d))] = codes_slot
    nu16 = buf[nword * 4:].view(np.float16).reshape(G, N)
    return codes[:, :N], nu16


def decode_values(cb: Codebook, buf: np.ndarray, G: int, N: int) -> np.ndarray:
    """v_mse = nu~ R^T c_v[code]: [G, N, din] fp64 (the first din coordinates)."""
    lv, _ = value_quantizer(cb)
    codes, nu16 = unpack_values(cb, buf, G, N)
    return (nu16.astype(np.float64)[..., None] * (lv[codes] @ cb.R))[..., :cb.din]


def attention_from_logits(cb: Codebook, logits: np.ndarray, vbuf: np.ndarray, G: int, N: int,
                          scale: Optional[float] = None) -> np.ndarray:
    """out[g, h] = sum_n softmax_n(scale * logits[g, h, :]) v_mse[g, n]:
    [G, Qg, din] fp64, from the given logits and the packed values (scale
    1/sqrt(din) by default)."""
    scale = 1.0 / math.sqrt(cb.din) if scale is None else float(scale)
    z = scale * np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    w = np.exp(z)
    p = w / w.sum(axis=-1, keepdims=True)
    return np.einsum("gqn,gnd->gqd", p, decode_values(cb, vbuf, G, N))


def attention(cb: Codebook, kbuf: np.ndarray, vbuf: np.ndarray, G: int, N: int, q: np.ndarray,
              scale: Optional[float] = None) -> np.ndarray:
    """Decode attention of queries q [G, Qg, d] over packed keys and values:
    the estimated logits of :func:`score`, then :func:`attention_from_logits`."""
    return attention_from_logits(cb, score(cb, kbuf, G, N, q), vbuf, G, N, scale)

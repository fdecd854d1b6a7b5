// Host core of the TurboQuant key-path library: quantizer tables, the C ABI,
// argument validation and device set-up.  The kernels live in tq_kernels.hip.
//
// Method sources (by page title and section):
//  * rotation R = H_d D / sqrt(d), Sylvester H_d, Rademacher D:
//    ICLR 2026 paper digest (0h-n0.github.io), "Step 1: PolarQuant";
//  * shared Lloyd-Max scalar quantizer for the N(0, 1/d) coordinate law:
//    Qiita explainer (kai_kou), "Stage 1" step 3; ICLR 2026 digest, Theorem 1;
//  * (b-1)-bit MSE stage + 1-bit QJL of the residual, total b bits:
//    ai.spot.hk TurboQuant article, "無偏內積估計";
//  * Gaussian projection S and the sqrt(pi/2)/m estimator constant:
//    Qiita explainer, "Stage 2: QJL", estimator equation.

#include "tq_internal.h"

#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>
#include <new>

#include "../../include/tq.h"

struct tq_codebook : public tq::Codebook {};

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return TQ_ERR_HIP;
}

// ---------------------------------------------------------------- SplitMix64
// Counter-based use of the SplitMix64 generator (Steele, Lea & Flood 2014):
//   draw(seed, stream, i) = mix(mix(seed + stream*G) + (i + 1)*G),  G = golden gamma.
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

inline uint64_t splitmix_finalize(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct Stream {
  uint64_t base;
  Stream(uint64_t seed, uint64_t stream) : base(splitmix_finalize(seed + stream * kGamma)) {}
  uint64_t operator()(uint64_t i) const { return splitmix_finalize(base + (i + 1) * kGamma); }
};

void make_delta(uint64_t seed, int d, int8_t* out) {
  Stream s(seed, 1);
  for (int i = 0; i < d; ++i) out[i] = (s(static_cast<uint64_t>(i)) >> 63) ? int8_t(-1) : int8_t(1);
}

// The sketch seen from the rotated domain, S R^T: Box-Muller N(0,1) draws
// rounded to float16 (nearest even), held exactly in float64.
void make_sketch_rot(uint64_t seed, int m, int d, double* out) {
  Stream s(seed, 2);
  const double two_pi = 2.0 * M_PI;
  const double ulp53 = std::ldexp(1.0, -53);
  for (int64_t t = 0, n = int64_t(m) * d; t < n; ++t) {
    const uint64_t x = s(2 * uint64_t(t)), y = s(2 * uint64_t(t) + 1);
    const double u1 = double((x >> 11) + 1) * ulp53;   // (0, 1]
    const double u2 = double(y >> 11) * ulp53;         // [0, 1)
    const double z = std::sqrt(-2.0 * std::log(u1)) * std::cos(two_pi * u2);  // Box-Muller
    out[t] = double(static_cast<_Float16>(z));
  }
}

// ------------------------------------------------------------------ Lloyd-Max
// MSE-optimal L-level quantizer of the standard normal law.  The law is
// symmetric and L even, so only the positive half is iterated, with the
// centre boundary pinned at 0: alternate "boundary = midpoint of its two
// levels" and "level = centroid of its cell" until the levels stop moving.
void lloyd_max_normal(int L, double* levels, double* thresholds) {
  const int K = L / 2;
  std::vector<double> c(K), b(K + 1);
  for (int k = 0; k < K; ++k) c[k] = (k + 0.5) * 3.0 / K;
  const double inv_sqrt2 = 1.0 / std::sqrt(2.0), inv_sqrt2pi = 1.0 / std::sqrt(2.0 * M_PI);
  auto pdf = [&](double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) * inv_sqrt2pi; };
  auto tail = [&](double x) { return std::isinf(x) ? 0.0 : 0.5 * std::erfc(x * inv_sqrt2); };
  for (int it = 0; it < 200000; ++it) {
    b[0] = 0.0;
    b[K] = INFINITY;
    for (int k = 1; k < K; ++k) b[k] = 0.5 * (c[k - 1] + c[k]);
    double moved = 0.0;
    for (int k = 0; k < K; ++k) {
      const double nc = (pdf(b[k]) - pdf(b[k + 1])) / (tail(b[k]) - tail(b[k + 1]));
      moved = std::fmax(moved, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (moved < 1e-15) break;
  }
  for (int k = 0; k < K; ++k) {
    levels[K + k] = c[k];
    levels[K - 1 - k] = -c[k];
  }
  thresholds[K - 1] = 0.0;
  for (int k = 1; k < K; ++k) {
    const double t = 0.5 * (c[k - 1] + c[k]);
    thresholds[K - 1 + k] = t;
    thresholds[K - 1 - k] = -t;
  }
}

// ------------------------------------------------------- Lloyd-Max, Beta law
// One coordinate of a uniformly random unit vector in R^d has density
// proportional to (1 - y^2)^((d-3)/2) on [-1, 1] (y^2 ~ Beta(1/2, (d-1)/2)).
// Tail mass P(Y >= y) = I_{1-y^2}((d-1)/2, 1/2) / 2 with the regularised
// incomplete beta function I evaluated by its continued fraction (modified
// Lentz), switching to I_x(a, b) = 1 - I_{1-x}(b, a) where the fraction
// converges slowly; the first moment of a cell has a closed form.
double incbeta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  double c = 1.0, dd = 1.0 - (a + b) * x / (a + 1.0);
  if (std::fabs(dd) < tiny) dd = tiny;
  dd = 1.0 / dd;
  double f = dd;
  for (int m = 1; m < 100000; ++m) {
    // even step
    double num = m * (b - m) * x / ((a + 2 * m - 1) * (a + 2 * m));
    dd = 1.0 + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    f *= dd * c;
    // odd step
    num = -(a + m) * (a + b + m) * x / ((a + 2 * m) * (a + 2 * m + 1));
    dd = 1.0 + num * dd;
    if (std::fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    const double del = dd * c;
    f *= del;
    if (std::fabs(del - 1.0) < 1e-16) break;
  }
  return f;
}

double incbeta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double lfront = std::lgamma(a + b) - std::lgamma(a) - std::lgamma(b) + a * std::log(x) +
                        b * std::log1p(-x);
  if (x < (a + 1.0) / (a + b + 2.0)) return std::exp(lfront) * incbeta_cf(a, b, x) / a;
  return 1.0 - std::exp(lfront) * incbeta_cf(b, a, 1.0 - x) / b;
}

void lloyd_max_beta(int d, int L, double* levels, double* thresholds) {
  const int K = L / 2;
  const double h = 0.5 * (d - 1);
  const double cnorm = std::exp(std::lgamma(0.5 * d) - std::lgamma(h) - 0.5 * std::log(M_PI));
  auto upper = [&](double y) { return y >= 1.0 ? 0.0 : 0.5 * incbeta(h, 0.5, 1.0 - y * y); };
  auto moment = [&](double a, double b) {
    const double fa = a < 1.0 ? std::pow(1.0 - a * a, h) : 0.0;
    const double fb = b < 1.0 ? std::pow(1.0 - b * b, h) : 0.0;
    return cnorm * (fa - fb) / (d - 1);
  };
  const double sd = 1.0 / std::sqrt(double(d));
  std::vector<double> c(K), t(K + 1);
  for (int k = 0; k < K; ++k) c[k] = sd * (k + 0.5) * 1.5 / K;
  // stops once the levels move less than 1e-14 of the coordinate scale (the
  // continued fraction's own rounding keeps them moving at the ulp level)
  for (int it = 0; it < 100000; ++it) {
    t[0] = 0.0;
    t[K] = 1.0;
    for (int k = 1; k < K; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    double moved = 0.0;
    for (int k = 0; k < K; ++k) {
      const double nc = moment(t[k], t[k + 1]) / (upper(t[k]) - upper(t[k + 1]));
      moved = std::fmax(moved, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (moved < 1e-14 * sd) break;
  }
  for (int k = 0; k < K; ++k) {
    levels[K + k] = c[k];
    levels[K - 1 - k] = -c[k];
  }
  thresholds[K - 1] = 0.0;
  for (int k = 1; k < K; ++k) {
    const double tt = 0.5 * (c[k - 1] + c[k]);
    thresholds[K - 1 + k] = tt;
    thresholds[K - 1 - k] = -tt;
  }
}

// S = (S R^T) R = S_rot H D / sqrt(d) (R orthogonal, H symmetric): a
// Hadamard transform of each row of S_rot, then D, in float64.
void sketch_from_rotated(const double* S_rot, const int8_t* delta, int m, int d, double* out) {
  const double scale = 1.0 / std::sqrt(double(d));
  for (int j = 0; j < m; ++j) {
    double* row = out + int64_t(j) * d;
    for (int i = 0; i < d; ++i) row[i] = S_rot[int64_t(j) * d + i];
    for (int h = 1; h < d; h <<= 1)
      for (int i0 = 0; i0 < d; i0 += 2 * h)
        for (int i = i0; i < i0 + h; ++i) {
          const double a = row[i], c = row[i + h];
          row[i] = a + c;
          row[i + h] = a - c;
        }
    for (int i = 0; i < d; ++i) row[i] *= scale * delta[i];
  }
}

// The power of two D the method runs in for d-dimensional vectors: d itself,
// or the next power of two when d is a multiple of 16 (rows are zero-padded
// to D [ICLR 2026 paper digest, "実装のポイント": zero padding up to the
// nearest power of two for the Hadamard transform]); 0 when unsupported.
int rotation_dim(int d) {
  if (d < 1 || d > 4096) return 0;
  int D = 32;
  while (D < d) D <<= 1;
  return (D == d || d % 16 == 0) ? D : 0;
}

bool valid_params(int d, int bits, int m) {
  const int D = rotation_dim(d);
  if (D == 0) return false;
  if (bits < 2 || bits > 4) return false;
  return m == D;
}

bool device_params(int d) {
  const int D = rotation_dim(d);
  return D == 128 || D == 1024 || D == 2048 || D == 4096;
}

uint16_t half_bits(double v) {
  const _Float16 h = static_cast<_Float16>(v);   // round to nearest even
  uint16_t u;
  std::memcpy(&u, &h, 2);
  return u;
}

// Lane layout of the d = 128 float32-key encoder (two lanes per key): after its butterfly,
// register r of the lane in wave half h holds rotated coordinate
//   coord(h, r) = (r % 32) + 32 * (h + 2 * (r / 32)).
// The matrix-core B operand takes K-slice [8h, 8h+8) of each 16-wide chunk kc
// from registers r = 8*kc + t, so the A operand (S R^T rows) must present the
// same coordinates: fragment (kc, jb, lane L) holds row 32*jb + L%32 at
// coordinates coord(L/32, 8*kc + t), t = 0..7.  Stored negated (see the encoder).
void build_fragments_128(const std::vector<double>& S_rot, std::vector<uint16_t>& frag) {
  const int d = 128;
  frag.assign(8 * 4 * 64 * 8, 0);
  for (int kc = 0; kc < 8; ++kc)
    for (int jb = 0; jb < 4; ++jb)
      for (int L = 0; L < 64; ++L) {
        const int j = 32 * jb + (L & 31), h = L >> 5;
        for (int t = 0; t < 8; ++t) {
          const int r = 8 * kc + t;
          const int coord = (r & 31) + 32 * (h + 2 * (r >> 5));
          // negated (the encoder forms the negated residual c[code] - y);
          // S_rot holds float16 values, so the half is exact
          frag[((size_t(kc) * 4 + jb) * 64 + L) * 8 + t] = half_bits(-S_rot[size_t(j) * d + coord]);
        }
      }
}

// Lane layout of the 16-key bf16 encoder: lane L = 16 w + n serves key n and
// owns the 32 coordinates [32 w, 32 w + 32) (word w of every bit plane).
// Rotation block b leaves value i of that lane at coordinate 32 w + 4 b + i,
// and sketch k-step t takes the lane's blocks 2t and 2t + 1, so the matrix
// core's K index 8 w + j of step t is coordinate 32 w + 8 t + j.  The A
// operand of step t, row block b (16 x 16 x 32 products) puts row
// 32 (m / 4) + 4 b + m % 4 of S R^T on matrix row m = L % 16, so the lane
// holding rows 4 w .. 4 w + 3 of block b gets sketch rows 32 w + 4 b + i:
// fragment (t, b, lane L) holds that row at coordinates 32 (L / 16) + 8 t + j,
// j = 0..7, negated like the two-lane table.
void build_fragments_128_t16(const std::vector<double>& S_rot, std::vector<uint16_t>& frag) {
  const int d = 128;
  frag.assign(4 * 8 * 64 * 8, 0);
  for (int t = 0; t < 4; ++t)
    for (int b = 0; b < 8; ++b)
      for (int L = 0; L < 64; ++L) {
        const int m = L & 15, row = 32 * (m >> 2) + 4 * b + (m & 3);
        for (int j = 0; j < 8; ++j) {
          const int coord = 32 * (L >> 4) + 8 * t + j;
          frag[((size_t(t) * 8 + b) * 64 + L) * 8 + j] = half_bits(-S_rot[size_t(row) * d + coord]);
        }
      }
}

// d = 1024: fragment (rb, ks, lane L) holds row 32 rb + L % 32 of S R^T at
// coordinates 16 ks + 8 (L / 32) + t, t = 0..7 (matrix-core A order for
// 32x32x16); the values are exact in float16.
void build_fragments_wide(const std::vector<double>& S_rot, int d, std::vector<uint16_t>& frag) {
  const int nrb = d / 32, nks = d / 16;
  frag.assign(size_t(nrb) * nks * 64 * 8, 0);
  for (int rb = 0; rb < nrb; ++rb)
    for (int ks = 0; ks < nks; ++ks)
      for (int L = 0; L < 64; ++L) {
        const int j = 32 * rb + (L & 31);
        for (int t = 0; t < 8; ++t) {
          const int k = 16 * ks + 8 * (L >> 5) + t;
          frag[((size_t(rb) * nks + ks) * 64 + L) * 8 + t] = half_bits(S_rot[size_t(j) * d + k]);
        }
      }
}

void fill_consts(tq::Codebook& cb) {
  tq::DevConsts& k = cb.consts;
  std::memset(&k, 0, sizeof(k));
  const int L = 1 << (cb.bits - 1), K = L / 2;
  for (int i = 0; i < K - 1; ++i) k.tpos[i] = float(cb.thresholds[K + i]);
  for (int i = 0; i < K; ++i) k.cpos_s[i] = float(cb.levels[K + i] * double(tq::kResidualScale));
  for (int i = 0; i < L; ++i) k.levels[i] = float(cb.levels[i]);
  // Walsh expansion of the level table over s_p = 2*bit_p - 1:
  //   c(code) = sum_S alpha_S prod_{p in S} s_p ; only odd |S| survive (odd symmetry).
  const int B = cb.bits - 1;
  const int subsets[4] = {1, 2, 4, 7};
  double asum = 0.0;
  for (int a = 0; a < 4; ++a) {
    const int S = subsets[a];
    if (S >= (1 << B)) { k.alpha[a] = 0.f; continue; }
    double acc = 0.0;
    for (int code = 0; code < L; ++code) {
      double prod = 1.0;
      for (int p = 0; p < B; ++p)
        if (S >> p & 1) prod *= ((code >> p) & 1) ? 1.0 : -1.0;
      acc += cb.levels[code] * prod;
    }
    k.alpha[a] = float(acc / L);
    asum += acc / L;
  }
  k.alpha_sum = float(asum);
  const int LV = 1 << cb.bits, KV = LV / 2;
  for (int i = 0; i < KV - 1; ++i) k.vtpos[i] = float(cb.vthresholds[KV + i]);
  for (int i = 0; i < LV; ++i) k.vlevels[i] = float(cb.vlevels[i]);
  k.sqrt_d = float(std::sqrt(double(cb.d)));
  k.inv_sqrt_d = float(1.0 / std::sqrt(double(cb.d)));
  k.qjl_scale = float(std::sqrt(M_PI / 2.0) / cb.m);
  k.din = uint32_t(cb.d_in);
  for (int i = 0; i < cb.d; ++i)
    if (cb.delta[i] < 0) k.dneg[i >> 5] |= 1u << (i & 31);
}

int build_tables(tq::Codebook& cb) {
  const int d = cb.d, m = cb.m, L = 1 << (cb.bits - 1);
  try {
    cb.levels.resize(L);
    cb.thresholds.resize(L - 1);
    cb.delta.resize(d);
    cb.S.resize(size_t(m) * d);
    cb.S_rot.resize(size_t(m) * d);
  } catch (const std::bad_alloc&) {
    return TQ_ERR_ALLOC;
  }
  // Lloyd-Max tables on the unit-vector coordinate scale: the N(0, 1/d) law
  // (kind 0) or the exact coordinate law of a random unit vector (kind 1)
  const double sigma = 1.0 / std::sqrt(double(d));   // N(0,1) -> N(0, 1/d)
  auto tables = [&](int LL, double* lv, double* th) {
    if (cb.kind == TQ_CODEBOOK_BETA) {
      lloyd_max_beta(d, LL, lv, th);
    } else {
      lloyd_max_normal(LL, lv, th);
      for (int i = 0; i < LL; ++i) lv[i] *= sigma;
      for (int i = 0; i + 1 < LL; ++i) th[i] *= sigma;
    }
  };
  tables(L, cb.levels.data(), cb.thresholds.data());
  // value records: all `bits` bits go to the Lloyd-Max code (no sketch bit)
  const int LV = 1 << cb.bits;
  try {
    cb.vlevels.resize(LV);
    cb.vthresholds.resize(LV - 1);
  } catch (const std::bad_alloc&) {
    return TQ_ERR_ALLOC;
  }
  tables(LV, cb.vlevels.data(), cb.vthresholds.data());
  make_delta(cb.seed, d, cb.delta.data());
  make_sketch_rot(cb.seed, m, d, cb.S_rot.data());
  sketch_from_rotated(cb.S_rot.data(), cb.delta.data(), m, d, cb.S.data());
  fill_consts(cb);
  return TQ_OK;
}

void release_device(tq::Codebook& cb) {
  if (cb.d_consts) (void)hipFree(cb.d_consts);
  if (cb.d_frag) (void)hipFree(cb.d_frag);
  if (cb.d_St) (void)hipFree(cb.d_St);
  if (cb.d_Sh) (void)hipFree(cb.d_Sh);
  if (cb.d_flip_f32) (void)hipFree(cb.d_flip_f32);
  if (cb.d_fragW) (void)hipFree(cb.d_fragW);
  if (cb.d_Scol) (void)hipFree(cb.d_Scol);
  cb.d_Scol = nullptr;
  if (cb.d_frag16) (void)hipFree(cb.d_frag16);
  if (cb.d_dm16) (void)hipFree(cb.d_dm16);
  cb.d_fragW = nullptr;
  cb.d_frag16 = nullptr;
  cb.d_dm16 = nullptr;
  cb.d_consts = nullptr;
  cb.d_frag = nullptr;
  cb.d_St = nullptr;
  cb.d_Sh = nullptr;
  cb.d_flip_f32 = nullptr;
}

template <typename T>
hipError_t upload(T** dst, const void* src, size_t bytes) {
  hipError_t e = hipMalloc(reinterpret_cast<void**>(dst), bytes);
  if (e != hipSuccess) { *dst = nullptr; return e; }
  return hipMemcpy(*dst, src, bytes, hipMemcpyHostToDevice);
}

int upload_device(tq::Codebook& cb) {
  hipError_t e = hipGetDevice(&cb.device);
  if (e != hipSuccess) return hip_fail(e);
  if (hipDeviceGetAttribute(&cb.num_cus, hipDeviceAttributeMultiprocessorCount, cb.device) != hipSuccess ||
      cb.num_cus <= 0)
    cb.num_cus = 256;
  e = upload(&cb.d_consts, &cb.consts, sizeof(tq::DevConsts));
  if (e == hipSuccess && cb.d >= 1024) {
    std::vector<uint16_t> frag;
    build_fragments_wide(cb.S_rot, cb.d, frag);
    e = upload(&cb.d_fragW, frag.data(), frag.size() * sizeof(uint16_t));
  }
  if (e == hipSuccess && cb.d >= 1024) {   // the wide query preparation reads S column by column
    std::vector<float> st(cb.S.size());
    for (int j = 0; j < cb.m; ++j)
      for (int c = 0; c < cb.d; ++c) st[size_t(c) * cb.m + j] = float(cb.S[size_t(j) * cb.d + c]);
    e = upload(&cb.d_St, st.data(), st.size() * sizeof(float));
  }
  if (e == hipSuccess && cb.d > 1024) {    // sum_j (S q)_j = (column sums of S) . q
    std::vector<float> col(cb.d);
    for (int c = 0; c < cb.d; ++c) {
      double t = 0.0;
      for (int j = 0; j < cb.m; ++j) t += cb.S[size_t(j) * cb.d + c];
      col[c] = float(t);
    }
    e = upload(&cb.d_Scol, col.data(), col.size() * sizeof(float));
  }
  if (e == hipSuccess && cb.d == 128) {
    std::vector<uint16_t> frag;
    build_fragments_128(cb.S_rot, frag);
    e = upload(&cb.d_frag, frag.data(), frag.size() * sizeof(uint16_t));
    // float32 keys: sign-flip words for the lane holding [64h, 64h + 64)
    std::vector<uint32_t> ff(128, 0);
    for (int i = 0; i < 128; ++i)
      if (cb.delta[i] < 0) ff[(i >> 6) * 64 + (i & 63)] = 0x80000000u;
    if (e == hipSuccess) e = upload(&cb.d_flip_f32, ff.data(), ff.size() * 4);
    // 16-key encoder: [word w][k-step t][register j] covers coordinates
    // 32 w + 8 t + 2 j, +1 (low, high half)
    std::vector<uint16_t> f16;
    build_fragments_128_t16(cb.S_rot, f16);
    std::vector<uint32_t> dm(64, 0);
    for (int w = 0; w < 4; ++w)
      for (int t = 0; t < 4; ++t)
        for (int j = 0; j < 4; ++j) {
          const int i0 = 32 * w + 8 * t + 2 * j;
          dm[(w * 4 + t) * 4 + j] = (cb.delta[i0] < 0 ? 0x8000u : 0u) |
                                    (cb.delta[i0 + 1] < 0 ? 0x80000000u : 0u);
        }
    if (e == hipSuccess) e = upload(&cb.d_frag16, f16.data(), f16.size() * sizeof(uint16_t));
    // paged append (latency path): S R^T columns 16 s .. 16 s + 15 of row j, contiguous per (s, j)
    std::vector<uint16_t> sh(8 * 128 * 16);
    for (int sg = 0; sg < 8; ++sg)
      for (int j = 0; j < 128; ++j)
        for (int m = 0; m < 16; ++m)
          sh[(size_t(sg) * 128 + j) * 16 + m] = half_bits(cb.S_rot[size_t(j) * 128 + 16 * sg + m]);
    if (e == hipSuccess) e = upload(&cb.d_Sh, sh.data(), sh.size() * sizeof(uint16_t));
    if (e == hipSuccess) e = upload(&cb.d_dm16, dm.data(), dm.size() * 4);
  }
  if (e != hipSuccess) {
    release_device(cb);
    return hip_fail(e);
  }
  return TQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_device(const tq::Codebook& cb) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  return dev == cb.device ? TQ_OK : TQ_ERR_ARG;
}

}  // namespace

extern "C" {

int32_t tq_rotation_dim(int32_t d) { return rotation_dim(d); }

int tq_codebook_tables(int32_t d, int32_t bits, int32_t m, uint64_t seed, double* levels,
                       double* thresholds, int8_t* delta, double* S, double* S_rot) {
  return tq_codebook_tables_ex(d, bits, m, seed, TQ_CODEBOOK_GAUSSIAN, levels, thresholds, delta, S,
                               S_rot);
}

int tq_codebook_tables_ex(int32_t d, int32_t bits, int32_t m, uint64_t seed, int32_t kind,
                          double* levels, double* thresholds, int8_t* delta, double* S,
                          double* S_rot) {
  if (!valid_params(d, bits, m)) return TQ_ERR_UNSUPPORTED;
  if (kind != TQ_CODEBOOK_GAUSSIAN && kind != TQ_CODEBOOK_BETA) return TQ_ERR_ARG;
  tq::Codebook cb;
  cb.kind = kind;
  cb.d = rotation_dim(d);
  cb.d_in = d;
  cb.bits = bits;
  cb.m = m;
  cb.seed = seed;
  const int rc = build_tables(cb);
  if (rc != TQ_OK) return rc;
  const int L = 1 << (bits - 1);
  if (levels) std::memcpy(levels, cb.levels.data(), L * sizeof(double));
  if (thresholds) std::memcpy(thresholds, cb.thresholds.data(), (L - 1) * sizeof(double));
  if (delta) std::memcpy(delta, cb.delta.data(), cb.d);
  if (S) std::memcpy(S, cb.S.data(), cb.S.size() * sizeof(double));
  if (S_rot) std::memcpy(S_rot, cb.S_rot.data(), cb.S_rot.size() * sizeof(double));
  return TQ_OK;
}

int tq_make_codebook(int32_t d, int32_t bits, int32_t m, uint64_t seed, tq_codebook** out) {
  return tq_make_codebook_ex(d, bits, m, seed, TQ_CODEBOOK_GAUSSIAN, out);
}

int tq_make_codebook_ex(int32_t d, int32_t bits, int32_t m, uint64_t seed, int32_t kind,
                        tq_codebook** out) {
  if (!out) return TQ_ERR_ARG;
  *out = nullptr;
  if (kind != TQ_CODEBOOK_GAUSSIAN && kind != TQ_CODEBOOK_BETA) return TQ_ERR_ARG;
  if (!valid_params(d, bits, m) || !device_params(d)) return TQ_ERR_UNSUPPORTED;
  std::unique_ptr<tq_codebook> cb(new (std::nothrow) tq_codebook());
  if (!cb) return TQ_ERR_ALLOC;
  cb->kind = kind;
  cb->d = rotation_dim(d);
  cb->d_in = d;
  cb->bits = bits;
  cb->m = m;
  cb->seed = seed;
  int rc = build_tables(*cb);
  if (rc != TQ_OK) return rc;
  rc = upload_device(*cb);
  if (rc != TQ_OK) return rc;
  *out = cb.release();
  return TQ_OK;
}

void tq_free_codebook(tq_codebook* cb) {
  if (!cb) return;
  release_device(*cb);
  delete cb;
}

int tq_codebook_export(const tq_codebook* cb, double* levels, double* thresholds, int8_t* delta,
                       double* S, double* S_rot) {
  if (!cb) return TQ_ERR_ARG;
  const int L = 1 << (cb->bits - 1);
  if (levels) std::memcpy(levels, cb->levels.data(), L * sizeof(double));
  if (thresholds) std::memcpy(thresholds, cb->thresholds.data(), (L - 1) * sizeof(double));
  if (delta) std::memcpy(delta, cb->delta.data(), cb->d);
  if (S) std::memcpy(S, cb->S.data(), cb->S.size() * sizeof(double));
  if (S_rot) std::memcpy(S_rot, cb->S_rot.data(), cb->S_rot.size() * sizeof(double));
  return TQ_OK;
}

int tq_codebook_info(const tq_codebook* cb, int32_t* d, int32_t* bits, int32_t* m,
                     uint64_t* seed) {
  if (!cb) return TQ_ERR_ARG;
  if (d) *d = cb->d_in;
  if (bits) *bits = cb->bits;
  if (m) *m = cb->m;
  if (seed) *seed = cb->seed;
  return TQ_OK;
}

size_t tq_packed_bytes(const tq_codebook* cb, int64_t G, int64_t N) {
  if (!cb || G < 0 || N < 0) return 0;
  const int64_t per = int64_t(cb->bits - 1) * cb->d / 8 + cb->m / 8 + 4;
  return size_t(G) * size_t(N) * size_t(per);
}

int tq_encode_keys(const tq_codebook* cb, const void* keys, int32_t key_dtype, int64_t G,
                   int64_t N, void* packed, void* stream) {
  if (!cb || G < 0 || N < 0 || (key_dtype != TQ_F32 && key_dtype != TQ_BF16)) return TQ_ERR_ARG;
  if (G == 0 || N == 0) return TQ_OK;
  if (!keys || !packed || !aligned16(keys) || !aligned16(packed)) return TQ_ERR_ARG;
  if (!tq::encode_supported(*cb)) return TQ_ERR_UNSUPPORTED;
  // tile counts fit the kernels' 32-bit indices: 32-key tiles < 2^31, 16-key tiles < 2^32
  if (G * ((N + 31) / 32) >= (int64_t(1) << 31)) return TQ_ERR_UNSUPPORTED;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_encode(*cb, keys, key_dtype, G, N, N, 0, packed,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_append_keys(const tq_codebook* cb, const void* keys, int32_t key_dtype, int64_t G, int64_t T,
                   void* packed, int64_t Ncap, int64_t pos, void* stream) {
  if (!cb || G < 0 || T < 0 || Ncap < 0 || pos < 0 || (key_dtype != TQ_F32 && key_dtype != TQ_BF16))
    return TQ_ERR_ARG;
  if (pos > Ncap || T > Ncap - pos) return TQ_ERR_ARG;
  if (G == 0 || T == 0) return TQ_OK;
  if (!keys || !packed || !aligned16(keys) || !aligned16(packed)) return TQ_ERR_ARG;
  if (cb->d != 128) return TQ_ERR_UNSUPPORTED;
  if (G * ((T + 31) / 32) >= (int64_t(1) << 31)) return TQ_ERR_UNSUPPORTED;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_append_keys(*cb, keys, key_dtype, G, T, Ncap, pos, packed,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

namespace {
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shape of a paged pool the d = 128 kernels take: pages of a multiple of 64
// records (each 64-key score tile lies in one page).
int check_pool(const tq_codebook* cb, int64_t num_pages, int32_t page_size, int32_t ppg) {
  if (num_pages <= 0 || page_size <= 0 || ppg <= 0) return TQ_ERR_ARG;
  if (cb->d != 128 || page_size % 64 != 0 || page_size > (1 << 20) || num_pages > INT32_MAX)
    return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}
}  // namespace

int tq_paged_append_keys(const tq_codebook* cb, const void* keys, int32_t key_dtype, int64_t G,
                         int64_t T, void* pool, int64_t num_pages, int32_t page_size,
                         const int32_t* page_table, int32_t pages_per_group, const int32_t* pos,
                         void* stream) {
  if (!cb || G < 0 || T < 0 || (key_dtype != TQ_F32 && key_dtype != TQ_BF16)) return TQ_ERR_ARG;
  int rc = check_pool(cb, num_pages, page_size, pages_per_group);
  if (rc != TQ_OK) return rc;
  if (G == 0 || T == 0) return TQ_OK;
  if (G * T >= (int64_t(1) << 31) || G * int64_t(pages_per_group) >= (int64_t(1) << 31))
    return TQ_ERR_UNSUPPORTED;
  if (!keys || !pool || !page_table || !pos || !aligned16(keys) || !aligned16(pool) ||
      !aligned4(page_table) || !aligned4(pos))
    return TQ_ERR_ARG;
  rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_encode_paged(*cb, keys, key_dtype, G, T, pool, num_pages, page_size,
                                         page_table, pages_per_group, pos,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_paged_score(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                   const void* pool, int64_t num_pages, int32_t page_size, const int32_t* page_table,
                   int32_t pages_per_group, const int32_t* lens, int64_t Lmax, float* logits,
                   void* stream) {
  if (!cb || G < 0 || Qg < 0 || Lmax < 0 || (q_dtype != TQ_F32 && q_dtype != TQ_BF16)) return TQ_ERR_ARG;
  int rc = check_pool(cb, num_pages, page_size, pages_per_group);
  if (rc != TQ_OK) return rc;
  if (Qg > 256 || G > INT32_MAX || Lmax >= (int64_t(1) << 28) ||
      G * int64_t(pages_per_group) >= (int64_t(1) << 31))
    return TQ_ERR_UNSUPPORTED;
  if (G == 0 || Qg == 0 || Lmax == 0) return TQ_OK;
  if (!q || !pool || !page_table || !lens || !logits || !aligned16(q) || !aligned16(pool) ||
      !aligned4(page_table) || !aligned4(lens) || !aligned16(logits))
    return TQ_ERR_ARG;
  rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_score_paged(*cb, q, q_dtype, G, Qg, pool, num_pages, page_size, page_table,
                                        pages_per_group, lens, Lmax, logits,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_paged_append_values(const tq_codebook* cb, const void* values, int32_t dtype, int64_t G, int64_t T,
                           void* pool, int64_t num_pages, int32_t page_size, const int32_t* page_table,
                           int32_t pages_per_group, const int32_t* pos, void* stream) {
  if (!cb || G < 0 || T < 0 || (dtype != TQ_F32 && dtype != TQ_BF16)) return TQ_ERR_ARG;
  int rc = check_pool(cb, num_pages, page_size, pages_per_group);
  if (rc != TQ_OK) return rc;
  if (G == 0 || T == 0) return TQ_OK;
  if (G * T >= (int64_t(1) << 31) || G * int64_t(pages_per_group) >= (int64_t(1) << 31))
    return TQ_ERR_UNSUPPORTED;
  if (!values || !pool || !page_table || !pos || !aligned16(values) || !aligned16(pool) ||
      !aligned4(page_table) || !aligned4(pos))
    return TQ_ERR_ARG;
  rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_append_values_paged(*cb, values, dtype, G, T, pool, num_pages, page_size,
                                                page_table, pages_per_group, pos,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_paged_attention(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                       const void* kpool, const void* vpool, int64_t num_pages, int32_t page_size,
                       const int32_t* page_table, int32_t pages_per_group, const int32_t* lens, int64_t Lmax,
                       float scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!cb || G < 0 || Qg < 0 || Lmax < 0 || (q_dtype != TQ_F32 && q_dtype != TQ_BF16)) return TQ_ERR_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return TQ_ERR_ARG;
  int rc = check_pool(cb, num_pages, page_size, pages_per_group);
  if (rc != TQ_OK) return rc;
  if (Qg > 256 || G > INT32_MAX || G * Qg > INT32_MAX || Lmax >= (int64_t(1) << 28) ||
      G * int64_t(pages_per_group) >= (int64_t(1) << 31))
    return TQ_ERR_UNSUPPORTED;
  if (G == 0 || Qg == 0) return TQ_OK;
  if (Lmax == 0) return TQ_ERR_ARG;
  if (!q || !kpool || !vpool || !page_table || !lens || !out || !aligned16(q) || !aligned16(kpool) ||
      !aligned16(vpool) || !aligned4(page_table) || !aligned4(lens) || !aligned16(out))
    return TQ_ERR_ARG;
  const size_t need = tq::attention_workspace_bytes(*cb, G, Qg, Lmax);
  if (!ws || !aligned16(ws) || ws_bytes < need) return TQ_ERR_WORKSPACE;
  rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_attention_paged(*cb, q, q_dtype, G, Qg, kpool, vpool, num_pages, page_size,
                                            page_table, pages_per_group, lens, Lmax, scale, out, ws,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

size_t tq_value_packed_bytes(const tq_codebook* cb, int64_t G, int64_t N) {
  if (!cb || G < 0 || N < 0) return 0;
  // codes in tiles of 16 values (bits * d / 8 bytes per value), then one half norm per value
  return size_t(G) * (size_t((N + 15) / 16) * 16 * size_t(cb->bits * cb->d / 8) + 2 * size_t(N));
}

int tq_encode_values(const tq_codebook* cb, const void* values, int32_t dtype, int64_t G, int64_t N,
                     void* vpacked, void* stream) {
  if (!cb || G < 0 || N < 0 || (dtype != TQ_F32 && dtype != TQ_BF16)) return TQ_ERR_ARG;
  if (G == 0 || N == 0) return TQ_OK;
  if (!values || !vpacked || !aligned16(values) || !aligned16(vpacked)) return TQ_ERR_ARG;
  if (cb->d != 128) return TQ_ERR_UNSUPPORTED;
  if (G * ((N + 31) / 32) >= (int64_t(1) << 31)) return TQ_ERR_UNSUPPORTED;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_encode_values(*cb, values, dtype, G, N, vpacked,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_append_values(const tq_codebook* cb, const void* values, int32_t dtype, int64_t G, int64_t T,
                     void* vpacked, int64_t Ncap, int64_t pos, void* stream) {
  if (!cb || G < 0 || T < 0 || Ncap < 0 || pos < 0 || (dtype != TQ_F32 && dtype != TQ_BF16))
    return TQ_ERR_ARG;
  if (pos > Ncap || T > Ncap - pos) return TQ_ERR_ARG;
  if (G == 0 || T == 0) return TQ_OK;
  if (!values || !vpacked || !aligned16(values) || !aligned16(vpacked)) return TQ_ERR_ARG;
  if (cb->d != 128) return TQ_ERR_UNSUPPORTED;
  if (G * ((T + 31) / 32) >= (int64_t(1) << 31) || G * T >= (int64_t(1) << 33)) return TQ_ERR_UNSUPPORTED;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_append_values(*cb, values, dtype, G, T, vpacked, Ncap, pos,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

size_t tq_attention_workspace_bytes(const tq_codebook* cb, int64_t G, int32_t Qg, int64_t N) {
  if (!cb || G <= 0 || Qg <= 0 || N <= 0 || cb->d != 128) return 0;
  return tq::attention_workspace_bytes(*cb, G, Qg, N);
}

int tq_attention_decode(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                        const void* kpacked, const void* vpacked, int64_t N, float scale, float* out,
                        void* ws, size_t ws_bytes, void* stream) {
  if (!cb || G < 0 || N < 0 || Qg < 0 || (q_dtype != TQ_F32 && q_dtype != TQ_BF16)) return TQ_ERR_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return TQ_ERR_ARG;
  if (cb->d != 128 || Qg > 256 || G > INT32_MAX || G * Qg > INT32_MAX ||
      N >= (int64_t(1) << 28))
    return TQ_ERR_UNSUPPORTED;
  if (G == 0 || Qg == 0) return TQ_OK;
  if (N == 0) return TQ_ERR_ARG;   // softmax over no keys
  if (!q || !kpacked || !vpacked || !out || !aligned16(q) || !aligned16(kpacked) ||
      !aligned16(vpacked) || !aligned16(out))
    return TQ_ERR_ARG;
  const size_t need = tq::attention_workspace_bytes(*cb, G, Qg, N);
  if (!ws || !aligned16(ws) || ws_bytes < need) return TQ_ERR_WORKSPACE;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_attention(*cb, q, q_dtype, G, Qg, kpacked, vpacked, N, N, scale, out, ws,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_attention_cache(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                       const void* kpacked, const void* vpacked, int64_t Ncap, int64_t len, float scale,
                       float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!cb || G < 0 || Qg < 0 || Ncap < 0 || len < 0 || len > Ncap ||
      (q_dtype != TQ_F32 && q_dtype != TQ_BF16))
    return TQ_ERR_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return TQ_ERR_ARG;
  if (cb->d != 128 || Qg > 256 || G > INT32_MAX || G * Qg > INT32_MAX ||
      Ncap >= (int64_t(1) << 28))
    return TQ_ERR_UNSUPPORTED;
  if (G == 0 || Qg == 0) return TQ_OK;
  if (len == 0) return TQ_ERR_ARG;   // softmax over no keys
  if (!q || !kpacked || !vpacked || !out || !aligned16(q) || !aligned16(kpacked) ||
      !aligned16(vpacked) || !aligned16(out))
    return TQ_ERR_ARG;
  const size_t need = tq::attention_workspace_bytes(*cb, G, Qg, len);
  if (!ws || !aligned16(ws) || ws_bytes < need) return TQ_ERR_WORKSPACE;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_attention(*cb, q, q_dtype, G, Qg, kpacked, vpacked, len, Ncap, scale, out,
                                      ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_attention_decode_noalloc(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G,
                                int32_t Qg, const void* kpacked, const void* vpacked, int64_t N,
                                float scale, float* out, void* stream) {
  if (!cb || G < 0 || N < 0 || Qg < 0 || (q_dtype != TQ_F32 && q_dtype != TQ_BF16)) return TQ_ERR_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return TQ_ERR_ARG;
  if (cb->d != 128 || Qg > 256 || G > INT32_MAX || G * Qg > INT32_MAX ||
      N >= (int64_t(1) << 28))
    return TQ_ERR_UNSUPPORTED;
  if (G == 0 || Qg == 0) return TQ_OK;
  if (N == 0) return TQ_ERR_ARG;
  if (!q || !kpacked || !vpacked || !out || !aligned16(q) || !aligned16(kpacked) ||
      !aligned16(vpacked) || !aligned16(out))
    return TQ_ERR_ARG;
  if (tq::attention_workspace_bytes(*cb, G, Qg, N) > tq::kScratchBytes) return TQ_ERR_WORKSPACE;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  void* ws = nullptr;
  hipError_t e = tq::scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e);
  e = tq::launch_attention(*cb, q, q_dtype, G, Qg, kpacked, vpacked, N, N, scale, out, ws,
                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

size_t tq_attention_noalloc_max_bytes(void) { return tq::kScratchBytes; }

size_t tq_score_workspace_bytes(const tq_codebook* cb, int64_t G, int32_t Qg) {
  if (!cb || G < 0 || Qg < 0) return 0;
  return tq::score_workspace_bytes(*cb, G, Qg);
}

int tq_score_logits(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                    const void* packed, int64_t N, float* logits, void* ws, size_t ws_bytes,
                    void* stream) {
  if (!cb || G < 0 || N < 0 || Qg < 0 || (q_dtype != TQ_F32 && q_dtype != TQ_BF16))
    return TQ_ERR_ARG;
  if (Qg > 256 || G > INT32_MAX) return TQ_ERR_UNSUPPORTED;
  // d = 128 addresses records and logits of a group with 32-bit byte offsets
  if (cb->d == 128 && N >= (int64_t(1) << 28)) return TQ_ERR_UNSUPPORTED;
  if (G == 0 || N == 0 || Qg == 0) return TQ_OK;
  if (!q || !packed || !logits || !aligned16(q) || !aligned16(packed) || !aligned16(logits))
    return TQ_ERR_ARG;
  const size_t need = tq::score_workspace_bytes(*cb, G, Qg);
  if (need > 0 && (!ws || !aligned16(ws) || ws_bytes < need)) return TQ_ERR_WORKSPACE;
  if (!tq::score_supported(*cb)) return TQ_ERR_UNSUPPORTED;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_score(*cb, q, q_dtype, G, Qg, packed, N, N, logits, ws,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_score_cache(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                   const void* packed, int64_t Ncap, int64_t len, float* logits, void* stream) {
  if (!cb || G < 0 || Qg < 0 || Ncap < 0 || len < 0 || len > Ncap ||
      (q_dtype != TQ_F32 && q_dtype != TQ_BF16))
    return TQ_ERR_ARG;
  if (cb->d != 128 || Qg > 256 || G > INT32_MAX || Ncap >= (int64_t(1) << 28))
    return TQ_ERR_UNSUPPORTED;
  if (G == 0 || len == 0 || Qg == 0) return TQ_OK;
  if (!q || !packed || !logits || !aligned16(q) || !aligned16(packed) || !aligned16(logits))
    return TQ_ERR_ARG;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_score(*cb, q, q_dtype, G, Qg, packed, len, Ncap, logits, nullptr,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

size_t tq_score_topk_workspace_bytes(const tq_codebook* cb, int64_t G, int32_t Qg, int64_t N,
                                     int32_t k) {
  if (!cb || G <= 0 || Qg <= 0 || N <= 0 || k < 1 || k > tq::kMaxTopKAbi || cb->d != 1024) return 0;
  return tq::topk_wide_bytes(*cb, G, Qg, N, k);
}

int tq_score_topk(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                  const void* packed, int64_t N, int32_t k, int32_t* idx, float* scores, void* ws,
                  size_t ws_bytes, void* stream) {
  if (!cb || G < 0 || N < 0 || Qg < 0 || (q_dtype != TQ_F32 && q_dtype != TQ_BF16)) return TQ_ERR_ARG;
  if (k < 1 || k > tq::kMaxTopKAbi) return TQ_ERR_UNSUPPORTED;
  if (cb->d != 1024 || Qg > 256 || G > INT32_MAX || N > INT32_MAX) return TQ_ERR_UNSUPPORTED;
  if (G == 0 || Qg == 0) return TQ_OK;
  if (N == 0) return TQ_ERR_ARG;
  if (!q || !packed || !idx || !scores || !aligned16(q) || !aligned16(packed)) return TQ_ERR_ARG;
  const size_t need = tq::topk_wide_bytes(*cb, G, Qg, N, k);
  if (!ws || !aligned16(ws) || ws_bytes < need) return TQ_ERR_WORKSPACE;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_topk_wide(*cb, q, q_dtype, G, Qg, packed, N, k, idx, scores, ws,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_decode_mse(const tq_codebook* cb, const void* packed, int64_t G, int64_t N, void* out,
                  int32_t out_dtype, void* stream) {
  if (!cb || G < 0 || N < 0 || (out_dtype != TQ_F32 && out_dtype != TQ_BF16)) return TQ_ERR_ARG;
  if (G == 0 || N == 0) return TQ_OK;
  if (!packed || !out || !aligned16(packed) || !aligned16(out)) return TQ_ERR_ARG;
  if (!tq::encode_supported(*cb)) return TQ_ERR_UNSUPPORTED;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_decode(*cb, packed, G, N, out, out_dtype,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_dense_logits_bf16(const void* q, const void* keys, int64_t G, int32_t Qg, int64_t N,
                         int32_t d, float* logits, void* stream) {
  if (G < 0 || N < 0 || Qg < 0) return TQ_ERR_ARG;
  if (d != 128 || Qg > 8) return TQ_ERR_UNSUPPORTED;
  if (G == 0 || N == 0 || Qg == 0) return TQ_OK;
  if (!q || !keys || !logits || !aligned16(q) || !aligned16(keys) || !aligned16(logits))
    return TQ_ERR_ARG;
  hipError_t e = tq::launch_dense_bf16(q, keys, G, Qg, N, d, logits,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_clock_probe(uint64_t* out, int32_t ticks, void* stream) {
  if (!out || ticks <= 0 || (reinterpret_cast<uintptr_t>(out) & 7u)) return TQ_ERR_ARG;
  hipError_t e = tq::launch_clock_probe(out, uint32_t(ticks), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_stream_probe(const void* src, size_t src_bytes, void* dst, size_t dst_bytes, int32_t grid,
                    void* stream) {
  if ((src_bytes | dst_bytes) & 15u) return TQ_ERR_ARG;
  if ((src_bytes && (!src || !aligned16(src))) || (dst_bytes && (!dst || !aligned16(dst))))
    return TQ_ERR_ARG;
  if (grid > (1 << 20)) return TQ_ERR_UNSUPPORTED;
  if (src_bytes == 0 && dst_bytes == 0) return TQ_OK;
  hipError_t e = tq::launch_stream_probe(src, src_bytes, dst, dst_bytes, grid,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

int tq_score_stream_probe(const tq_codebook* cb, int64_t G, int32_t Qg, const void* packed, int64_t N,
                          float* logits, void* stream) {
  if (!cb || G < 0 || N < 0 || Qg < 0) return TQ_ERR_ARG;
  if (cb->d != 128 || Qg > 256 || G > INT32_MAX || N >= (int64_t(1) << 28)) return TQ_ERR_UNSUPPORTED;
  if (G == 0 || N == 0 || Qg == 0) return TQ_OK;
  if (!packed || !logits || !aligned16(packed) || !aligned16(logits)) return TQ_ERR_ARG;
  int rc = check_device(*cb);
  if (rc != TQ_OK) return rc;
  hipError_t e = tq::launch_score_stream_probe(*cb, G, Qg, packed, N, logits,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TQ_OK : hip_fail(e);
}

const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_ARG: return "invalid argument (null or misaligned pointer, negative size, bad dtype, wrong device)";
    case TQ_ERR_UNSUPPORTED: return "unsupported parameter";
    case TQ_ERR_ALLOC: return "allocation failed";
    case TQ_ERR_HIP: return "HIP runtime error";
    case TQ_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int tq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

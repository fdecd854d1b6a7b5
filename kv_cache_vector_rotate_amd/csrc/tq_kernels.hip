// HIP kernels (gfx950 / MI355X) of the TurboQuant key path, d = 128.
//
//  encode:  rotation y = H D k / (||k|| sqrt(d)) as a register-resident
//           Hadamard butterfly, Lloyd-Max codes by threshold comparison,
//           bit-plane packing, residual, and the QJL projection S r on the
//           matrix cores [ICLR 2026 paper digest (0h-n0), "Step 1:
//           PolarQuant"; Qiita explainer (kai_kou), "Stage 2: QJL"].
//  score:   streams packed records and evaluates
//             nu~ <R q, c[code]> + rho~ sqrt(pi/2)/m <S q, 1 - 2 sbit>
//           [Qiita explainer, "Stage 2: QJL", estimator equation] with
//           per-byte subset-sum tables of R q and S q held in LDS.
//  decode:  nu~ R^T c[code] (MSE-only reconstruction).
//  dense:   unquantised bf16 q.K logits (comparator, not part of the method).

#include "tq_internal.h"

#include <algorithm>
#include <mutex>

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));   // native: 16-byte LDS accesses

__device__ __forceinline__ uint32_t push_sign(uint32_t acc, float v) {
  // (acc << 1) | signbit(v)
  return __builtin_amdgcn_alignbit(acc, __float_as_uint(v), 31);
}

// Both lanes L and L^32 receive own + partner (a sum across wave halves).
__device__ __forceinline__ float xor32_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t xor32_or(uint32_t v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return r[0] | r[1];
}

__device__ __forceinline__ uint16_t f2h_bits(float v) {
  _Float16 h = static_cast<_Float16>(v);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float h2f_bits(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

int num_cus() {
  static int cus = 0;
  static std::once_flag once;
  std::call_once(once, [] {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
  });
  return cus;
}

// ============================================================== encode, d = 128
//
// Lane layout: a wave encodes 32 keys at a time, two lanes per key.  Lane
// L = 32h + kl loads coordinates [64h, 64h + 64) of key kl into x[0..63].
// Six butterfly stages run inside the register file; the stage across the
// two halves uses v_permlane32_swap on register pairs (r, r + 32), which
// leaves register r of half h holding coordinate
//   (r % 32) + 32 * (h + 2 * (r / 32)),
// i.e. bit-plane word h in x[0..31] and word 2 + h in x[32..63], bit r % 32.
// The residual registers feed the matrix-core B operand directly (K order
// = register order); the host lays S R^T out in the matching A order.

constexpr int kEncThreads = 256;
constexpr int kEncWaves = kEncThreads / 64;

template <int B, bool BF16>
__global__ __launch_bounds__(kEncThreads, 2) void encode128_kernel(
    const void* __restrict__ keys, int64_t G, int64_t N, uint32_t* __restrict__ planes,
    uint32_t* __restrict__ norms, const DevConsts* __restrict__ cst,
    const uint4* __restrict__ frag, const uint32_t* __restrict__ flip) {
  constexpr int K = 1 << (B - 1);      // levels on the positive half
  constexpr int P = B + 1;             // planes per key
  constexpr int NFLIP = BF16 ? 64 : 128;
  __shared__ uint4 s_frag[4096];       // [hi | lo][kc 8][jb 4][lane 64]
  __shared__ uint32_t s_flip[NFLIP];

  const int tid = threadIdx.x;
  for (int i = tid; i < 4096; i += kEncThreads) s_frag[i] = frag[i];
  for (int i = tid; i < NFLIP; i += kEncThreads) s_flip[i] = flip[i];
  float tpos[K > 1 ? K - 1 : 1], cpos[K];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) tpos[k] = cst->tpos[k];
#pragma unroll
  for (int k = 0; k < K; ++k) cpos[k] = cst->cpos_s[k];
  const float sqrt_d = cst->sqrt_d;
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6, h = lane >> 5, kl = lane & 31;
  const int64_t tpg = (N + 31) / 32;
  const int64_t ntiles = G * tpg;

  for (int64_t tile = int64_t(blockIdx.x) * kEncWaves + wave; tile < ntiles;
       tile += int64_t(gridDim.x) * kEncWaves) {
    const int64_t g = tile / tpg;
    const int64_t n = (tile - g * tpg) * 32 + kl;
    const bool valid = n < N;
    // Lanes past the end of a ragged group load the group's last key; their
    // results are never stored and each key occupies its own matrix column.
    const int64_t nl = valid ? n : N - 1;
    float x[64];
    float nu2 = 0.f;

    // ---- load, apply D (sign flips), accumulate ||k||^2
    if constexpr (BF16) {
      const uint4* src = reinterpret_cast<const uint4*>(
          static_cast<const uint16_t*>(keys) + ((g * N + nl) * 128 + 64 * h));
      const uint4* fl = reinterpret_cast<const uint4*>(s_flip) + h * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 v = src[c];
        const uint4 f = fl[c];
        const uint32_t w[4] = {v.x ^ f.x, v.y ^ f.y, v.z ^ f.z, v.w ^ f.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          x[8 * c + 2 * t] = __uint_as_float(w[t] << 16);
          x[8 * c + 2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
        }
      }
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(
          static_cast<const float*>(keys) + ((g * N + nl) * 128 + 64 * h));
      const uint4* fl = reinterpret_cast<const uint4*>(s_flip) + h * 16;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint4 v = src[c];
        const uint4 f = fl[c];
        x[4 * c + 0] = __uint_as_float(v.x ^ f.x);
        x[4 * c + 1] = __uint_as_float(v.y ^ f.y);
        x[4 * c + 2] = __uint_as_float(v.z ^ f.z);
        x[4 * c + 3] = __uint_as_float(v.w ^ f.w);
      }
    }
#pragma unroll
    for (int r = 0; r < 64; ++r) nu2 = fmaf(x[r], x[r], nu2);

    // ---- Hadamard butterfly: strides 1..32 in registers, stride 64 across halves
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
#pragma unroll
      for (int r = 0; r < 64; ++r) {
        if (r & s) continue;
        const float a = x[r], b = x[r + s];
        x[r] = a + b;
        x[r + s] = a - b;
      }
    }
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[r]), __float_as_uint(x[r + 32]),
                                                 false, false);
      const float a = __uint_as_float(pr[0]), b = __uint_as_float(pr[1]);
      x[r] = a + b;
      x[r + 32] = a - b;
    }

    nu2 = xor32_sum(nu2);
    const float nu = sqrtf(nu2);
    const bool zero = !(nu >= 1e-10f);
    const float nsd = nu * sqrt_d;                       // u = y * nu * sqrt(d)
    const float gsc = zero ? 0.f : kResidualScale / nsd;  // u -> 2^12 y
    float tu[K > 1 ? K - 1 : 1];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) tu[k] = tpos[k] * nsd;

    // ---- Lloyd-Max codes (sign bit + magnitude thresholds), residual, hi/lo split
    uint32_t wu[2] = {0u, 0u};
    uint32_t wd[K > 1 ? K - 1 : 1][2];
#pragma unroll
    for (int k = 0; k < (K > 1 ? K - 1 : 1); ++k) wd[k][0] = wd[k][1] = 0u;
    half8 bhi[8], blo[8];
    float rho2 = 0.f;
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      const int ws = r >> 5;
      // sign-flipped zero inputs can leave -0 after the butterfly; + 0 makes an
      // exact zero count as non-negative (a value on the middle threshold goes up)
      const float u = x[r] + 0.0f;
      const float a = fabsf(u);
      wu[ws] = push_sign(wu[ws], u);
      float mag = cpos[0];
#pragma unroll
      for (int k = 0; k < K - 1; ++k) {
        const float dk = a - tu[k];
        wd[k][ws] = push_sign(wd[k][ws], dk);
        mag = (dk >= 0.f) ? cpos[k + 1] : mag;
      }
      const float yh = copysignf(mag, u);
      const float ep = fmaf(u, gsc, -yh);
      rho2 = fmaf(ep, ep, rho2);
      const _Float16 hi = static_cast<_Float16>(ep);
      bhi[r >> 3][r & 7] = hi;
      blo[r >> 3][r & 7] = static_cast<_Float16>(ep - static_cast<float>(hi));
    }
    rho2 = xor32_sum(rho2);
    const float rho = zero ? 0.f : sqrtf(rho2) * (nu * (1.0f / kResidualScale));

    // words were filled oldest-bit-first: bit (r % 32) sits at 31 - r % 32
    uint32_t pw[P - 1][2];
#pragma unroll
    for (int ws = 0; ws < 2; ++ws) {
      const uint32_t u_ = __builtin_bitreverse32(wu[ws]);
      if constexpr (B == 1) {
        pw[0][ws] = ~u_;
      } else if constexpr (B == 2) {
        pw[1][ws] = ~u_;
        pw[0][ws] = ~(u_ ^ __builtin_bitreverse32(wd[0][ws]));
      } else {
        const uint32_t d0 = __builtin_bitreverse32(wd[0][ws]);
        const uint32_t d1 = __builtin_bitreverse32(wd[1][ws]);
        const uint32_t d2 = __builtin_bitreverse32(wd[2][ws]);
        pw[2][ws] = ~u_;
        pw[1][ws] = ~(u_ ^ d1);
        pw[0][ws] = ~(u_ ^ d0 ^ d1 ^ d2);
      }
    }
    const bool keep = valid && !zero;
    uint32_t* pl = planes + (g * P) * N * 4;
#pragma unroll
    for (int p = 0; p < P - 1; ++p) {
      // (word h, word 2+h) of each lane -> (words 2h, 2h+1): swap across halves
      auto pr = __builtin_amdgcn_permlane32_swap(pw[p][0], pw[p][1], false, false);
      if (valid)
        *reinterpret_cast<uint2*>(pl + (p * N + n) * 4 + 2 * h) =
            make_uint2(keep ? uint32_t(pr[0]) : 0u, keep ? uint32_t(pr[1]) : 0u);
    }

    // ---- QJL projection p = (S R^T) r_rot on the matrix cores (fp32 accumulate,
    //      three-term fp16 split: hi*hi + hi*lo + lo*hi), then sign words.
    // The fragment table never changes inside the tile loop; an opaque lane
    // offset keeps the compiler from hoisting all 64 reads (256 VGPRs) out of it.
    int fl_off = lane;
    asm volatile("" : "+v"(fl_off));
    const half8* fh = reinterpret_cast<const half8*>(s_frag) + fl_off;
    const half8* fo = reinterpret_cast<const half8*>(s_frag + 2048) + fl_off;
    uint32_t sw[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      f32x16 acc = {};
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const half8 ahi = fh[(kc * 4 + jb) * 64];
        const half8 alo = fo[(kc * 4 + jb) * 64];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bhi[kc], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, blo[kc], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bhi[kc], acc, 0, 0, 0);
      }
      // lane (kl, h) holds rows j = 32 jb + 8 (v / 4) + 4 h + (v % 4) of key kl
      uint32_t b16 = 0u;
#pragma unroll
      for (int v = 15; v >= 0; --v) b16 = push_sign(b16, acc[v]);
      uint32_t t = (b16 | (b16 << 8)) & 0x00FF00FFu;
      t = (t | (t << 4)) & 0x0F0F0F0Fu;
      sw[jb] = xor32_or(t << (4 * h));
    }

    if (valid) {
      const bool keep_s = keep && rho2 > 0.f;
      uint2 so = make_uint2(keep_s ? (h ? sw[2] : sw[0]) : 0u, keep_s ? (h ? sw[3] : sw[1]) : 0u);
      *reinterpret_cast<uint2*>(pl + ((P - 1) * N + n) * 4 + 2 * h) = so;
      if (h == 0) {
        const uint32_t nb = keep ? f2h_bits(nu) : 0u;
        const uint32_t rb = keep ? f2h_bits(rho) : 0u;
        norms[g * N + n] = nb | (rb << 16);
      }
    }
  }
}

// ============================================================== query prep
// One wave per query: Rq = R q (butterfly; lane L holds coordinates L, L+64),
// Sq = S q (lane L computes rows L and L + 64), and the sums of both.
// Workspace: float [G*Qg][2][128] then float [G*Qg][4] (sum Rq, sum Sq, 0, 0).

constexpr int kPrepThreads = 256;

template <bool BF16>
__global__ __launch_bounds__(kPrepThreads) void prep128_kernel(
    const void* __restrict__ q, int64_t nq, const DevConsts* __restrict__ cst,
    const float* __restrict__ S, float* __restrict__ ws) {
  __shared__ float s_q[kPrepThreads / 64][128];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t qv_ = int64_t(blockIdx.x) * (kPrepThreads / 64) + wave;
  const bool valid = qv_ < nq;           // every wave reaches the barrier below
  const int64_t qi = valid ? qv_ : nq - 1;
  float v0, v1;
  if constexpr (BF16) {
    const uint16_t* qb = static_cast<const uint16_t*>(q) + qi * 128;
    v0 = __uint_as_float(uint32_t(qb[lane]) << 16);
    v1 = __uint_as_float(uint32_t(qb[lane + 64]) << 16);
  } else {
    const float* qf = static_cast<const float*>(q) + qi * 128;
    v0 = qf[lane];
    v1 = qf[lane + 64];
  }
  s_q[wave][lane] = v0;
  s_q[wave][lane + 64] = v1;
  const uint32_t n0 = (cst->dneg[lane >> 5] >> (lane & 31)) & 1u;
  const uint32_t n1 = (cst->dneg[2 + (lane >> 5)] >> (lane & 31)) & 1u;
  float a = n0 ? -v0 : v0, b = n1 ? -v1 : v1;
  float y0 = a + b, y1 = a - b;       // stride 64 in registers
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const float p0 = __shfl_xor(y0, s), p1 = __shfl_xor(y1, s);
    const bool up = lane & s;
    y0 = up ? p0 - y0 : y0 + p0;
    y1 = up ? p1 - y1 : y1 + p1;
  }
  y0 *= cst->inv_sqrt_d;
  y1 *= cst->inv_sqrt_d;
  __syncthreads();   // s_q rows written by other lanes of the wave
  float s0 = 0.f, s1 = 0.f;
  const float4* r0 = reinterpret_cast<const float4*>(S + int64_t(lane) * 128);
  const float4* r1 = reinterpret_cast<const float4*>(S + int64_t(lane + 64) * 128);
  const float4* qv = reinterpret_cast<const float4*>(s_q[wave]);
#pragma unroll 8
  for (int i = 0; i < 32; ++i) {
    const float4 qq = qv[i], a0 = r0[i], a1 = r1[i];
    s0 = fmaf(a0.x, qq.x, fmaf(a0.y, qq.y, fmaf(a0.z, qq.z, fmaf(a0.w, qq.w, s0))));
    s1 = fmaf(a1.x, qq.x, fmaf(a1.y, qq.y, fmaf(a1.z, qq.z, fmaf(a1.w, qq.w, s1))));
  }
  float* out = ws + qi * 256;
  if (valid) {
    out[lane] = y0;
    out[lane + 64] = y1;
    out[128 + lane] = s0;
    out[128 + lane + 64] = s1;
  }
  float sr = y0 + y1, ss = s0 + s1;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    sr += __shfl_xor(sr, s);
    ss += __shfl_xor(ss, s);
  }
  if (valid && lane == 0) {
    float* sums = ws + nq * 256 + qi * 4;
    sums[0] = sr;
    sums[1] = ss;
    sums[2] = 0.f;
    sums[3] = 0.f;
  }
}

// ============================================================== score, d = 128
// One workgroup per (group, 4-query chunk, key range).  LDS holds, for the
// chunk's 4 queries, T[tab][pos][byte] = sum over set bits t of byte of
// 2 * X[8 pos + t] with X = R q (tab 0, indexed by code-plane bytes) or S q
// (tab 1, indexed by sign-plane bytes).  Each lane then scores one key per
// step with 16 table reads per plane.

constexpr int kScoreThreads = 512;

template <int B>
__global__ __launch_bounds__(kScoreThreads, 1) void score128_kernel(
    const uint4* __restrict__ planes, const uint32_t* __restrict__ norms, int64_t G, int64_t N,
    int Qg, int nqc, int splits, const float* __restrict__ ws, float* __restrict__ logits,
    const DevConsts* __restrict__ cst) {
  constexpr int P = B + 1;
  __shared__ f32x4 s_lut[2][16][256];      // 128 KB
  __shared__ f32x4 s_nib[2][16][2][16];    // 16 KB
  __shared__ f32x4 s_x[2][128];            // 4 KB

  const int tid = threadIdx.x;
  int64_t b = blockIdx.x;
  const int split = int(b % splits);
  b /= splits;
  const int qc = int(b % nqc);
  const int64_t g = b / nqc;
  const int64_t nq = G * Qg;

  for (int i = tid; i < 2 * 128 * 4; i += kScoreThreads) {
    const int qq = i & 3, c = (i >> 2) & 127, tab = i >> 9;
    const int qh = qc * 4 + qq;
    s_x[tab][c][qq] = (qh < Qg) ? 2.0f * ws[(g * Qg + qh) * 256 + tab * 128 + c] : 0.0f;  // element write
  }
  __syncthreads();
  for (int i = tid; i < 2 * 16 * 2 * 16; i += kScoreThreads) {
    const int nib = i & 15, hf = (i >> 4) & 1, pos = (i >> 5) & 15, tab = i >> 9;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (nib >> t & 1) acc += s_x[tab][8 * pos + 4 * hf + t];
    s_nib[tab][pos][hf][nib] = acc;
  }
  __syncthreads();
  for (int i = tid; i < 2 * 16 * 256; i += kScoreThreads) {
    const int byte = i & 255, pos = (i >> 8) & 15, tab = i >> 12;
    s_lut[tab][pos][byte] = s_nib[tab][pos][0][byte & 15] + s_nib[tab][pos][1][byte >> 4];
  }
  float sr[4], ss[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int qh = qc * 4 + qq;
    const float* sums = ws + nq * 256 + (g * Qg + (qh < Qg ? qh : 0)) * 4;
    sr[qq] = sums[0];
    ss[qq] = sums[1];
  }
  const float a0 = cst->alpha[0], a1 = cst->alpha[1], a2 = cst->alpha[2], a3 = cst->alpha[3];
  const float asum = cst->alpha_sum, qs = cst->qjl_scale;
  __syncthreads();

  const int64_t chunk = ((N + splits - 1) / splits + 63) / 64 * 64;
  const int64_t n0 = int64_t(split) * chunk;
  const int64_t n1 = std::min<int64_t>(N, n0 + chunk);
  const uint4* pg = planes + g * P * N;

  for (int64_t n = n0 + tid; n < n1; n += kScoreThreads) {
    uint4 w[P];
#pragma unroll
    for (int p = 0; p < P; ++p) w[p] = pg[p * N + n];
    const uint32_t nrm = norms[g * N + n];
    float acc[4][4];     // [term][query]: planes 0..B-1 (and parity), sign plane last
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) acc[t][qq] = 0.f;

    auto add_plane = [&](const uint4 wv, int tab, float* a) {
      const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int wi = 0; wi < 4; ++wi)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4 tv = s_lut[tab][wi * 4 + k][(ww[wi] >> (8 * k)) & 255u];
          a[0] += tv[0]; a[1] += tv[1]; a[2] += tv[2]; a[3] += tv[3];
        }
    };
    float mse[4], qjl[4];
    if constexpr (B == 1) {
      add_plane(w[0], 0, acc[0]);
      add_plane(w[1], 1, acc[3]);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) mse[qq] = a0 * acc[0][qq] - asum * sr[qq];
    } else if constexpr (B == 2) {
      add_plane(w[0], 0, acc[0]);
      add_plane(w[1], 0, acc[1]);
      add_plane(w[2], 1, acc[3]);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        mse[qq] = fmaf(a0, acc[0][qq], a1 * acc[1][qq]) - asum * sr[qq];
    } else {
      add_plane(w[0], 0, acc[0]);
      add_plane(w[1], 0, acc[1]);
      add_plane(w[2], 0, acc[2]);
      const uint4 px = make_uint4(w[0].x ^ w[1].x ^ w[2].x, w[0].y ^ w[1].y ^ w[2].y,
                                  w[0].z ^ w[1].z ^ w[2].z, w[0].w ^ w[1].w ^ w[2].w);
      float accx[4] = {0.f, 0.f, 0.f, 0.f};
      add_plane(px, 0, accx);
      add_plane(w[3], 1, acc[3]);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        mse[qq] = fmaf(a0, acc[0][qq], fmaf(a1, acc[1][qq], fmaf(a2, acc[2][qq], a3 * accx[qq]))) -
                  asum * sr[qq];
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) qjl[qq] = ss[qq] - acc[3][qq];
    const float nu = h2f_bits(nrm & 0xffffu), rho = h2f_bits(nrm >> 16);
    const float rs = rho * qs;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int qh = qc * 4 + qq;
      if (qh < Qg) logits[(g * Qg + qh) * N + n] = fmaf(nu, mse[qq], rs * qjl[qq]);
    }
  }
}

// ============================================================== decode, d = 128
// One wave per key: lane L reconstructs coordinates L and L + 64 of
// nu~ D H c[code] / sqrt(d)  (= nu~ R^T c[code]).

template <int B, bool BF16OUT>
__global__ __launch_bounds__(256) void decode128_kernel(const uint32_t* __restrict__ planes,
                                                         const uint32_t* __restrict__ norms,
                                                         int64_t G, int64_t N, void* __restrict__ out,
                                                         const DevConsts* __restrict__ cst) {
  constexpr int P = B + 1;
  const int lane = threadIdx.x & 63;
  const int64_t key = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (key >= G * N) return;
  const int64_t g = key / N, n = key - g * N;
  const uint32_t* pk = planes + (g * P * N + n) * 4;
  int c0 = 0, c1 = 0;
#pragma unroll
  for (int p = 0; p < B; ++p) {
    c0 |= int((pk[p * N * 4 + (lane >> 5)] >> (lane & 31)) & 1u) << p;
    c1 |= int((pk[p * N * 4 + 2 + (lane >> 5)] >> (lane & 31)) & 1u) << p;
  }
  float a = cst->levels[c0], b = cst->levels[c1];
  float y0 = a + b, y1 = a - b;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const float p0 = __shfl_xor(y0, s), p1 = __shfl_xor(y1, s);
    const bool up = lane & s;
    y0 = up ? p0 - y0 : y0 + p0;
    y1 = up ? p1 - y1 : y1 + p1;
  }
  const float nu = h2f_bits(norms[g * N + n] & 0xffffu);
  const float sc = nu * cst->inv_sqrt_d;
  const uint32_t n0 = (cst->dneg[lane >> 5] >> (lane & 31)) & 1u;
  const uint32_t n1 = (cst->dneg[2 + (lane >> 5)] >> (lane & 31)) & 1u;
  y0 = (n0 ? -y0 : y0) * sc;
  y1 = (n1 ? -y1 : y1) * sc;
  if constexpr (BF16OUT) {
    __bf16* o = static_cast<__bf16*>(out) + key * 128;
    o[lane] = static_cast<__bf16>(y0);
    o[lane + 64] = static_cast<__bf16>(y1);
  } else {
    float* o = static_cast<float*>(out) + key * 128;
    o[lane] = y0;
    o[lane + 64] = y1;
  }
}

// ============================================================== dense bf16 q.K
// Comparator: 16 lanes per key (8 bf16 each), the group's queries in
// registers, float32 accumulation, reduction over the 16 lanes.

template <int QG>
__global__ __launch_bounds__(256) void dense128_kernel(const uint16_t* __restrict__ q,
                                                        const uint4* __restrict__ keys, int64_t G,
                                                        int64_t N, int splits,
                                                        float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int64_t g = blockIdx.x / splits;
  const int split = blockIdx.x % splits;
  float qv[QG][8];
#pragma unroll
  for (int j = 0; j < QG; ++j)
#pragma unroll
    for (int t = 0; t < 8; ++t)
      qv[j][t] = __uint_as_float(uint32_t(q[(g * QG + j) * 128 + sub * 8 + t]) << 16);
  const int64_t chunk = (N + splits - 1) / splits;
  const int64_t n0 = split * chunk, n1 = std::min<int64_t>(N, n0 + chunk);
  const int slot = threadIdx.x >> 4;   // 16 keys per block step
  for (int64_t nb = n0; nb < n1; nb += 16) {
    const int64_t n = nb + slot;
    const bool valid = n < n1;
    uint4 kv = valid ? keys[(g * N + n) * 16 + sub] : make_uint4(0, 0, 0, 0);
    const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
    float kf[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kf[2 * t] = __uint_as_float(kw[t] << 16);
      kf[2 * t + 1] = __uint_as_float(kw[t] & 0xffff0000u);
    }
    float acc[QG];
#pragma unroll
    for (int j = 0; j < QG; ++j) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) s = fmaf(qv[j][t], kf[t], s);
      acc[j] = s;
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int j = 0; j < QG; ++j) acc[j] += __shfl_xor(acc[j], m);
    if (valid && sub < QG) {
      float v = acc[0];
#pragma unroll
      for (int j = 1; j < QG; ++j) v = (sub == j) ? acc[j] : v;
      logits[(g * QG + sub) * N + n] = v;
    }
  }
}

}  // namespace

bool encode_supported(const Codebook& cb) { return cb.d == 128; }
bool score_supported(const Codebook& cb) { return cb.d == 128; }

size_t score_workspace_bytes(const Codebook& cb, int64_t G, int Qg) {
  return size_t(G) * size_t(Qg) * (size_t(cb.d) + size_t(cb.m) + 4) * sizeof(float);
}

hipError_t launch_encode(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t N,
                         void* packed, hipStream_t s) {
  const int64_t ntiles = G * ((N + 31) / 32);
  const int64_t want = (ntiles + kEncWaves - 1) / kEncWaves;
  const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * 2));
  uint32_t* planes = static_cast<uint32_t*>(packed);
  uint32_t* norms = planes + G * N * int64_t(cb.bits) * (cb.d / 32);
  const bool bf = dtype == 1;
  const uint32_t* flip = bf ? cb.d_flip_bf16 : cb.d_flip_f32;
#define TQ_ENC(BB, BF)                                                                     \
  hipLaunchKernelGGL((encode128_kernel<BB, BF>), dim3(grid), dim3(kEncThreads), 0, s, keys, G, N, \
                     planes, norms, cb.d_consts, cb.d_frag, flip)
  switch (cb.bits - 1) {
    case 1: if (bf) TQ_ENC(1, true); else TQ_ENC(1, false); break;
    case 2: if (bf) TQ_ENC(2, true); else TQ_ENC(2, false); break;
    default: if (bf) TQ_ENC(3, true); else TQ_ENC(3, false); break;
  }
#undef TQ_ENC
  return hipGetLastError();
}

hipError_t launch_score(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                        const void* packed, int64_t N, float* logits, void* ws, hipStream_t s) {
  const int64_t nq = G * Qg;
  float* wsf = static_cast<float*>(ws);
  const int pgrid = int((nq + kPrepThreads / 64 - 1) / (kPrepThreads / 64));
  if (qdtype == 1)
    hipLaunchKernelGGL((prep128_kernel<true>), dim3(pgrid), dim3(kPrepThreads), 0, s, q, nq,
                       cb.d_consts, cb.d_S, wsf);
  else
    hipLaunchKernelGGL((prep128_kernel<false>), dim3(pgrid), dim3(kPrepThreads), 0, s, q, nq,
                       cb.d_consts, cb.d_S, wsf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqc = (Qg + 3) / 4;
  const int64_t units = G * nqc;
  const int64_t cus = num_cus();
  int splits = int(std::max<int64_t>(1, (cus + units - 1) / units));
  splits = int(std::min<int64_t>(splits, std::max<int64_t>(1, (N + 511) / 512)));
  const int64_t grid = units * splits;
  const uint4* planes = static_cast<const uint4*>(packed);
  const uint32_t* norms =
      static_cast<const uint32_t*>(packed) + G * N * int64_t(cb.bits) * (cb.d / 32);
#define TQ_SC(BB)                                                                        \
  hipLaunchKernelGGL((score128_kernel<BB>), dim3(grid), dim3(kScoreThreads), 0, s, planes, norms, \
                     G, N, Qg, nqc, splits, wsf, logits, cb.d_consts)
  switch (cb.bits - 1) {
    case 1: TQ_SC(1); break;
    case 2: TQ_SC(2); break;
    default: TQ_SC(3); break;
  }
#undef TQ_SC
  return hipGetLastError();
}

hipError_t launch_decode(const Codebook& cb, const void* packed, int64_t G, int64_t N, void* out,
                         int odtype, hipStream_t s) {
  const int64_t keys = G * N;
  const int grid = int((keys + 3) / 4);
  const uint32_t* planes = static_cast<const uint32_t*>(packed);
  const uint32_t* norms = planes + keys * int64_t(cb.bits) * (cb.d / 32);
#define TQ_DE(BB, BF)                                                                      \
  hipLaunchKernelGGL((decode128_kernel<BB, BF>), dim3(grid), dim3(256), 0, s, planes, norms, G, N, \
                     out, cb.d_consts)
  const bool bf = odtype == 1;
  switch (cb.bits - 1) {
    case 1: if (bf) TQ_DE(1, true); else TQ_DE(1, false); break;
    case 2: if (bf) TQ_DE(2, true); else TQ_DE(2, false); break;
    default: if (bf) TQ_DE(3, true); else TQ_DE(3, false); break;
  }
#undef TQ_DE
  return hipGetLastError();
}

hipError_t launch_dense_bf16(const void* q, const void* keys, int64_t G, int Qg, int64_t N, int d,
                             float* logits, hipStream_t s) {
  (void)d;
  const int64_t cus = num_cus();
  int splits = int(std::max<int64_t>(1, (cus * 8 + G - 1) / G));
  splits = int(std::min<int64_t>(splits, std::max<int64_t>(1, (N + 255) / 256)));
  const int64_t grid = G * splits;
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const uint4* kb = static_cast<const uint4*>(keys);
#define TQ_DN(QQ)                                                                             \
  hipLaunchKernelGGL((dense128_kernel<QQ>), dim3(grid), dim3(256), 0, s, qb, kb, G, N, splits, \
                     logits)
  switch (Qg) {
    case 1: TQ_DN(1); break;
    case 2: TQ_DN(2); break;
    case 3: TQ_DN(3); break;
    case 4: TQ_DN(4); break;
    case 5: TQ_DN(5); break;
    case 6: TQ_DN(6); break;
    case 7: TQ_DN(7); break;
    default: TQ_DN(8); break;
  }
#undef TQ_DN
  return hipGetLastError();
}

}  // namespace tq

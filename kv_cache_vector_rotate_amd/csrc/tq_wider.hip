// TurboQuant key path for rotation dimensions D = 2048 and 4096 on gfx950:
// vectors of more than 1024 coordinates, zero-padded to the next power of two
// (e.g. 3072-dimensional embeddings in D = 4096) [ICLR 2026 paper digest,
// "実装のポイント": zero padding to the nearest power of two].  Same method as
// the d = 1024 kernels, generalised:
//   rotate_wide_kernel   one key per wave, C = D / 64 coordinates per lane
//                        (log2 C butterfly stages inside the lane, six across
//                        lanes), Lloyd-Max codes, norms, residual to a
//                        workspace [ICLR 2026 digest, "Step 1: PolarQuant"];
//   qjl_wide_kernel      the QJL projection (S R^T) r_rot for 64 keys per
//                        workgroup on the matrix cores in passes of 1024
//                        sketch rows [Qiita explainer, "Stage 2: QJL"];
//   qprep_wide_kernel    2 R q, 2 S q and their sums per query;
//   score_wide_kernel    the estimator in slices of 1024 coordinates (nibble
//                        subset-sum tables of one slice in LDS at a time; the
//                        partial logits of earlier slices are read back);
//   decode_wide_kernel   nu~ R^T c[code].

#include "tq_internal.h"

#include <algorithm>
#include <cstdint>

namespace tq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t push_sign(uint32_t acc, float v) {
  return __builtin_amdgcn_alignbit(acc, __float_as_uint(v), 31);   // (acc << 1) | signbit(v)
}

__device__ __forceinline__ uint16_t f2h_bits(float v) {
  const _Float16 h = static_cast<_Float16>(v);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float h2f(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// value of lane L ^ S (S < 32)
template <int S>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __float_as_int(v);
  if constexpr (S == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
  if constexpr (S == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
  if constexpr (S == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x101F));
  if constexpr (S == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));
  if constexpr (S == 16) return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x401F));
}

// butterfly stage across lanes L, L ^ S on every register: (a, b) -> (a + b, a - b)
template <int S, int C>
__device__ __forceinline__ void stage_lanes(float (&x)[C], int lane) {
  const float sg = (lane & S) ? -1.0f : 1.0f;
#pragma unroll
  for (int t = 0; t < C; ++t) x[t] = fmaf(sg, x[t], lane_xor<S>(x[t]));
}

template <int C>
__device__ __forceinline__ void stage_lanes32(float (&x)[C], int lane) {
  const bool up = lane & 32;
#pragma unroll
  for (int t = 0; t < C; ++t) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[t]), __float_as_uint(x[t]), false, false);
    const float r0 = __uint_as_float(r[0]), r1 = __uint_as_float(r[1]);
    x[t] = up ? r0 - r1 : r0 + r1;   // lanes < 32: (own, partner); lanes >= 32: (partner, own)
  }
}

__device__ __forceinline__ float wave_sum(float v) {
  v += lane_xor<1>(v);
  v += lane_xor<2>(v);
  v += lane_xor<4>(v);
  v += lane_xor<8>(v);
  v += lane_xor<16>(v);
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The Hadamard transform of a D = 64 C point vector held as C coordinates
// per lane (lane L: coordinates C L + t): strides 1 .. C/2 inside the lane,
// C .. 32 C across lanes.  With `plus_zero` the first stage adds +0 so that
// no -0 survives (an exact zero counts as non-negative).
template <int C>
__device__ __forceinline__ void hadamard(float (&x)[C], int lane, bool plus_zero) {
#pragma unroll
  for (int t = 0; t < C; t += 2) {
    const float a = x[t], b = x[t + 1];
    x[t] = plus_zero ? (a + b) + 0.0f : a + b;
    x[t + 1] = plus_zero ? (a - b) + 0.0f : a - b;
  }
#pragma unroll
  for (int st = 2; st < C; st <<= 1)
#pragma unroll
    for (int t = 0; t < C; ++t) {
      if (t & st) continue;
      const float a = x[t], b = x[t + st];
      x[t] = a + b;
      x[t + st] = a - b;
    }
  stage_lanes<1>(x, lane);
  stage_lanes<2>(x, lane);
  stage_lanes<4>(x, lane);
  stage_lanes<8>(x, lane);
  stage_lanes<16>(x, lane);
  stage_lanes32(x, lane);
}

// C coordinates of a row of din elements (TQ_F32 or TQ_BF16) into registers;
// chunks at or past din (a multiple of 16) read the row start and give zeros.
template <bool BF16, int C>
__device__ __forceinline__ void load_row(const void* __restrict__ rows, int64_t row, int din, int lane,
                                         float (&x)[C]) {
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < C / 8; ++j) {
      const int c0 = C * lane + 8 * j;
      const bool in = c0 < din;
      uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(rows) + row * din + (in ? c0 : 0));
      if (!in) a = make_uint4(0u, 0u, 0u, 0u);
      const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * j + 2 * i] = __uint_as_float(u[i] << 16);
        x[8 * j + 2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < C / 4; ++j) {
      const int c0 = C * lane + 4 * j;
      const bool in = c0 < din;
      float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(rows) + row * din + (in ? c0 : 0));
      if (!in) v = make_float4(0.f, 0.f, 0.f, 0.f);
      x[4 * j] = v.x; x[4 * j + 1] = v.y; x[4 * j + 2] = v.z; x[4 * j + 3] = v.w;
    }
  }
}

// ---------------------------------------------------------------- rotate
// Lane L holds coordinates C L + t, i.e. words C L / 32 + w (w < C / 32) of
// every bit plane.  The residual is written as 2^12 (y - c[code]) (unit-vector
// units), zero for zero keys, in natural coordinate order: ws[key][D] float32.
template <int B, bool BF16, int C>
__global__ __launch_bounds__(256) void rotate_wide_kernel(const void* __restrict__ keys, int64_t k0,
                                                          int64_t nk, int64_t N,
                                                          uint32_t* __restrict__ planes,
                                                          uint32_t* __restrict__ norms,
                                                          float* __restrict__ ws,
                                                          const DevConsts* __restrict__ cst) {
  constexpr int DD = 64 * C, Wd = C / 32;
  constexpr int K = 1 << (B - 1);   // levels on the positive half
  constexpr int P = B + 1;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t wstride = int64_t(gridDim.x) * 4;
  float tpos[K > 1 ? K - 1 : 1], cpos[K];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) tpos[k] = cst->tpos[k];
#pragma unroll
  for (int k = 0; k < K; ++k) cpos[k] = cst->cpos_s[k];
  const float sqrt_d = cst->sqrt_d;
  uint32_t dn[Wd];
#pragma unroll
  for (int w = 0; w < Wd; ++w) dn[w] = cst->dneg[Wd * lane + w];
  const int din = int(cst->din);

  for (int64_t wv = wave0; wv < nk; wv += wstride) {
    const int64_t kk = k0 + wv;   // key index over [G][N]
    float x[C];
    load_row<BF16, C>(keys, kk, din, lane, x);
    float nu2 = 0.f;
#pragma unroll
    for (int t = 0; t < C; ++t) nu2 = fmaf(x[t], x[t], nu2);
#pragma unroll
    for (int t = 0; t < C; ++t)
      x[t] = __uint_as_float(__float_as_uint(x[t]) ^ (((dn[t >> 5] >> (t & 31)) & 1u) << 31));
    hadamard(x, lane, true);

    nu2 = wave_sum(nu2);
    const float nu = sqrtf(nu2);
    const bool zero = !(nu >= 1e-10f);
    const float nsd = nu * sqrt_d;                          // u = y nu sqrt(d)
    const float gsc = zero ? 0.f : kResidualScale / nsd;    // u -> 2^12 y
    float tu[K > 1 ? K - 1 : 1];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) tu[k] = tpos[k] * nsd;

    uint32_t wu[Wd], wd[K > 1 ? K - 1 : 1][Wd];
    float rho2 = 0.f;
#pragma unroll
    for (int w = 0; w < Wd; ++w) {
      wu[w] = 0u;
#pragma unroll
      for (int k = 0; k < (K > 1 ? K - 1 : 1); ++k) wd[k][w] = 0u;
#pragma unroll
      for (int j = 31; j >= 0; --j) {   // pushed last = bit 0: bit j holds coordinate C L + 32 w + j
        const int t = 32 * w + j;
        const float u = x[t], a = fabsf(u);
        wu[w] = push_sign(wu[w], u);
        float mag = cpos[0];
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
          const float dk = a - tu[k];
          wd[k][w] = push_sign(wd[k][w], dk);
          mag = (dk >= 0.f) ? cpos[k + 1] : mag;
        }
        const float e = fmaf(u, gsc, -copysignf(mag, u));   // 2^12 (y - c[code])
        x[t] = zero ? 0.f : e;
        rho2 = fmaf(x[t], x[t], rho2);
      }
    }
    rho2 = wave_sum(rho2);
    const float rho = zero ? 0.f : sqrtf(rho2) * (nu * (1.0f / kResidualScale));
    const int64_t g = kk / N, n = kk - g * N;
#pragma unroll
    for (int w = 0; w < Wd; ++w) {
      const uint32_t fu = wu[w];
      uint32_t pw[P - 1];
      if constexpr (B == 1) {
        pw[0] = ~fu;
      } else if constexpr (B == 2) {
        pw[1] = ~fu;
        pw[0] = ~(fu ^ wd[0][w]);
      } else {
        pw[2] = ~fu;
        pw[1] = ~(fu ^ wd[1][w]);
        pw[0] = ~(fu ^ wd[0][w] ^ wd[1][w] ^ wd[2][w]);
      }
#pragma unroll
      for (int p = 0; p < P - 1; ++p)
        planes[((g * P + p) * N + n) * (DD / 32) + Wd * lane + w] = zero ? 0u : pw[p];
    }
    if (lane == 0) norms[g * N + n] = zero ? 0u : (uint32_t(f2h_bits(nu)) | (uint32_t(f2h_bits(rho)) << 16));
    float4* dst = reinterpret_cast<float4*>(ws + wv * DD + C * lane);
#pragma unroll
    for (int i = 0; i < C / 4; ++i) dst[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  }
}

// ---------------------------------------------------------------- QJL projection
// Workgroup tile: 64 keys; the D sketch rows run in passes of 1024 (wave w of
// eight owns rows 1024 pass + [128 w, 128 w + 128)), each pass streaming the
// tile's residuals through LDS in 64-coordinate chunks as fp16 hi/lo
// fragments; (S R^T) fragments, exact in float16, come from global memory in
// matrix-core A order [row block][k-step][lane].
constexpr int kQjlThreads = 512;
constexpr int kQjlKeys = 64;

__device__ __forceinline__ void split_f16x8(const float (&v)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v hv = {static_cast<_Float16>(v[2 * i]), static_cast<_Float16>(v[2 * i + 1])};
    const half2v lv = {static_cast<_Float16>(v[2 * i] - static_cast<float>(hv[0])),
                       static_cast<_Float16>(v[2 * i + 1] - static_cast<float>(hv[1]))};
    h[i] = __builtin_bit_cast(uint32_t, hv);
    l[i] = __builtin_bit_cast(uint32_t, lv);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

template <int DD>
__global__ __launch_bounds__(kQjlThreads, 1) void qjl_wide_kernel(const float* __restrict__ ws, int64_t k0,
                                                                  int64_t nk, int64_t N, int P,
                                                                  uint32_t* __restrict__ planes,
                                                                  const uint4* __restrict__ fragA) {
  constexpr int NKS = DD / 16;          // k-steps of 16 coordinates
  constexpr int NCH = DD / 64;          // staged chunks of 64 coordinates
  constexpr int NSTEP = NCH * 16;       // (k-step, row block) steps per pass
  constexpr int NW = DD / 32;           // sign words per key
  __shared__ uint4 sb[2][4][2][2][64];  // [buf][k-step][key block][hi/lo][lane]: 32 KB
  __shared__ uint32_t s_sign[kQjlKeys][NW + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int64_t ntiles = (nk + kQjlKeys - 1) / kQjlKeys;
  const int skey = tid >> 3, spart = tid & 7;

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t kb = tile * kQjlKeys;
    const int64_t src_key = std::min<int64_t>(kb + skey, nk - 1);
    const float* srow = ws + src_key * DD + 8 * spart;
    auto load_chunk = [&](int c, float (&v)[8]) {
      const float4* p = reinterpret_cast<const float4*>(srow + 64 * c);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    };
    auto store_chunk = [&](int buf, const float (&v)[8]) {
      uint4 hi, lo;
      split_f16x8(v, hi, lo);
      const int ks = spart >> 1, slot = (skey & 31) + 32 * (spart & 1), cb = skey >> 5;
      sb[buf][ks][cb][0][slot] = hi;
      sb[buf][ks][cb][1][slot] = lo;
    };
#pragma unroll 1
    for (int pass = 0; pass < DD / 1024; ++pass) {
      float v[8];
      load_chunk(0, v);
      store_chunk(0, v);
      __syncthreads();
      f32x16 acc[4][2] = {};
      const uint4* fa = fragA + (size_t(32 * pass + 4 * wave) * NKS) * 64 + lane;
      auto load_a = [&](int step, half8& ah) {   // step = 4 ks + rb
        const int ks = step >> 2, rb = step & 3;
        ah = __builtin_bit_cast(half8, fa[(size_t(rb) * NKS + ks) * 64]);
      };
      half8 ah[8];
#pragma unroll
      for (int i = 0; i < 7; ++i) load_a(i, ah[i]);
#pragma unroll 1
      for (int c = 0; c < NCH; ++c) {
        const int buf = c & 1;
        if (c + 1 < NCH) load_chunk(c + 1, v);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          half8 bh[2], bl[2];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            bh[cb] = __builtin_bit_cast(half8, sb[buf][ks][cb][0][lane]);
            bl[cb] = __builtin_bit_cast(half8, sb[buf][ks][cb][1][lane]);
          }
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const int step = 16 * c + 4 * ks + rb;
            const int slot = (4 * ks + rb) & 7;
            if (step + 7 < NSTEP) load_a(step + 7, ah[(slot + 7) & 7]);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[slot], bh[cb], acc[rb][cb], 0, 0, 0);
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[slot], bl[cb], acc[rb][cb], 0, 0, 0);
            }
          }
        }
        if (c + 1 < NCH) store_chunk(buf ^ 1, v);
        __syncthreads();
      }
      // sign words of this pass: lane (key kl, half h) holds rows
      // 8 (v / 4) + 4 h + (v % 4) of each 32-row block
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          uint32_t b16 = 0u;
#pragma unroll
          for (int vv = 15; vv >= 0; --vv) b16 = push_sign(b16, acc[rb][cb][vv]);
          uint32_t t = (b16 | (b16 << 8)) & 0x00FF00FFu;
          t = (t | (t << 4)) & 0x0F0F0F0Fu;
          t <<= 4 * h;
          auto pr = __builtin_amdgcn_permlane32_swap(t, t, false, false);
          const uint32_t word = pr[0] | pr[1];
          if (h == 0) s_sign[32 * cb + (lane & 31)][32 * pass + 4 * wave + rb] = word;
        }
    }
    __syncthreads();
    // 64 keys x NW words: thread -> (key, 4 words) per round
    for (int e = tid; e < kQjlKeys * (NW / 4); e += kQjlThreads) {
      const int key = e / (NW / 4), q4 = e % (NW / 4);
      const int64_t kk = kb + key;
      if (kk < nk) {
        const int64_t gk = k0 + kk;
        const int64_t g = gk / N, n = gk - g * N;
        uint4* dst = reinterpret_cast<uint4*>(planes + ((g * P + (P - 1)) * N + n) * NW) + q4;
        *dst = make_uint4(s_sign[key][4 * q4], s_sign[key][4 * q4 + 1], s_sign[key][4 * q4 + 2],
                          s_sign[key][4 * q4 + 3]);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- query preparation
// Grid (query, D / 1024 row blocks), 1024 threads.  Every workgroup stages the
// query in LDS; thread j of block r forms row 1024 r + j of 2 S q from S^T
// columns.  Block 0 also forms 2 R q (one wave: the butterfly above), its sum,
// and sum_j (S q)_j as (column sums of S) . q.
// ws layout: float X[G*Qg][2][D], then float sums[G*Qg][4] (sum R q, sum S q).
template <bool QBF16, int DD>
__global__ __launch_bounds__(1024) void qprep_wide_kernel(const void* __restrict__ q, float* __restrict__ X,
                                                          float* __restrict__ sums,
                                                          const DevConsts* __restrict__ cst,
                                                          const float* __restrict__ St,
                                                          const float* __restrict__ Scol) {
  constexpr int C = DD / 64;
  __shared__ float s_q[DD];
  __shared__ float s_part[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gq = blockIdx.x;
  const int rblk = blockIdx.y;
  const int din = int(cst->din);
  for (int i = tid; i < DD; i += 1024) {
    if (i >= din)
      s_q[i] = 0.f;
    else if constexpr (QBF16)
      s_q[i] = __uint_as_float(uint32_t(static_cast<const uint16_t*>(q)[gq * din + i]) << 16);
    else
      s_q[i] = static_cast<const float*>(q)[gq * din + i];
  }
  __syncthreads();
  float* xr = X + gq * 2 * DD;
  if (rblk == 0 && wave == 0) {
    float x[C];
#pragma unroll
    for (int t = 0; t < C; ++t) {
      const int i = C * lane + t;
      const uint32_t neg = (cst->dneg[i >> 5] >> (i & 31)) & 1u;
      x[t] = __uint_as_float(__float_as_uint(s_q[i]) ^ (neg << 31));
    }
    hadamard(x, lane, false);
    float sr = 0.f;
#pragma unroll
    for (int t = 0; t < C; ++t) {
      x[t] *= cst->inv_sqrt_d;
      sr += x[t];
    }
    float4* dst = reinterpret_cast<float4*>(xr + C * lane);
#pragma unroll
    for (int i = 0; i < C / 4; ++i)
      dst[i] = make_float4(2.f * x[4 * i], 2.f * x[4 * i + 1], 2.f * x[4 * i + 2], 2.f * x[4 * i + 3]);
    sr = wave_sum(sr);
    if (lane == 0) sums[gq * 4 + 0] = sr;
  }
  // S q, row j: sum over c of S^T[c][j] q[c]
  const int j = 1024 * rblk + tid;
  float acc = 0.f;
#pragma unroll 16
  for (int c = 0; c < DD; ++c) acc = fmaf(St[int64_t(c) * DD + j], s_q[c], acc);
  xr[DD + j] = 2.f * acc;
  if (rblk == 0) {
    float t = 0.f;
    for (int c = tid; c < DD; c += 1024) t = fmaf(Scol[c], s_q[c], t);
    t = wave_sum(t);
    if (lane == 0) s_part[wave] = t;
    __syncthreads();
    if (tid == 0) {
      float u = 0.f;
#pragma unroll
      for (int w = 0; w < 16; ++w) u += s_part[w];
      sums[gq * 4 + 1] = u;
    }
  }
}

// ---------------------------------------------------------------- score
// Grid (g, chunk of 4 query heads, key range); 1024 threads.  For each slice
// of 1024 coordinates: nibble subset-sum tables of that slice in LDS
//   T[ty][pos][nib] = sum over set bits t of nib of X_ty[1024 s + 4 pos + t]
// (entry (ty, pos = 16 blk + pl, nib) at byte ty 64K + blk 4K + nib 256 + pl 16,
// conflict-free as in the d = 1024 scorer), then every key of the range adds
// the slice's share of its logit,
//   nu~ sum_t alpha_t A_t - rho~ sqrt(pi/2)/m A_sign
// (A = the table sums over the slice's plane words), to the logit the
// earlier slices left in the output; the first slice adds the constant part
// -nu~ alpha_sum sum(R q) + rho~ sqrt(pi/2)/m sum(S q).
constexpr int kWideThreads = 1024;

template <int B, int DD>
__global__ __launch_bounds__(kWideThreads, 1) void score_wide_kernel(
    const uint4* __restrict__ planes, const uint32_t* __restrict__ norms, int64_t N, int Qg,
    int64_t chunk, const float* __restrict__ X, const float* __restrict__ sums,
    float* __restrict__ logits, const DevConsts* __restrict__ cst) {
  constexpr int P = B + 1;
  constexpr int NW = B == 3 ? P + 1 : P;
  constexpr int REC = DD / 128;            // 16-byte pieces of one key's plane
  __shared__ f32x4 tab[2 * 16 * 16 * 16];  // 128 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.x;
  const int qc = blockIdx.y;
  const int64_t n0 = int64_t(blockIdx.z) * chunk;
  const int64_t n1 = std::min<int64_t>(N, n0 + chunk);

  float sr[4], ss[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int qh = std::min(qc * 4 + qq, Qg - 1);
    sr[qq] = sums[(g * Qg + qh) * 4 + 0];
    ss[qq] = sums[(g * Qg + qh) * 4 + 1];
  }
  const float a0 = cst->alpha[0], a1 = cst->alpha[1], a2 = cst->alpha[2], a3 = cst->alpha[3];
  const float asum = cst->alpha_sum, qs = cst->qjl_scale;
  const uint32_t r = lane & 15;
  uint32_t pk[16], nb[8];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    pk[k] = (uint32_t(k) ^ r) << 4;
    asm volatile("" : "+v"(pk[k]));
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    nb[k] = 4u * (uint32_t(k) ^ (r & 7));
    asm volatile("" : "+v"(nb[k]));
  }
  const bool swp = r & 8;
  const char* tabp = reinterpret_cast<const char*>(tab);
  const uint4* pg = planes + g * P * N * REC;
  const uint32_t* ng = norms + g * N;

  auto add_block = [&](uint32_t w0, uint32_t w1, int ty, int blk, float* acc) {
    const uint32_t u0 = swp ? w1 : w0, u1 = swp ? w0 : w1;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t nib = __builtin_amdgcn_ubfe(k < 8 ? u0 : u1, nb[k & 7], 4);
      uint32_t ad = (nib << 8) | pk[k];
      if (ty) ad |= 0x10000u;
      const f32x4 tv = *reinterpret_cast<const f32x4*>(tabp + ad + blk * 4096);
      acc[0] += tv[0]; acc[1] += tv[1]; acc[2] += tv[2]; acc[3] += tv[3];
      if ((k & 3) == 3)
        asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]) : : "memory");
    }
  };

#pragma unroll 1
  for (int sl = 0; sl < DD / 1024; ++sl) {
    if (sl > 0) __syncthreads();   // every wave is done with the previous slice's tables
    {
      const int pl = tid & 15, hf = (tid >> 4) & 1, blk = (tid >> 5) & 15, ty = tid >> 9;
      const int pos = 16 * blk + pl;
      f32x4 xv[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int qh = qc * 4 + qq;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (qh < Qg)
          v = *reinterpret_cast<const float4*>(X + ((g * Qg + qh) * 2 + ty) * DD + 1024 * sl + 4 * pos);
        xv[0][qq] = v.x; xv[1][qq] = v.y; xv[2][qq] = v.z; xv[3][qq] = v.w;
      }
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 b = hf ? xv[3] : z;
      f32x4 e[8];
      e[0] = b;
      e[1] = b + xv[0];
      e[2] = b + xv[1];
      e[3] = e[2] + xv[0];
      e[4] = b + xv[2];
      e[5] = e[4] + xv[0];
      e[6] = e[4] + xv[1];
      e[7] = e[6] + xv[0];
#pragma unroll
      for (int j = 0; j < 8; ++j) tab[((ty * 16 + blk) * 16 + 8 * hf + j) * 16 + pl] = e[j];
    }
    __syncthreads();
    for (int64_t base = n0 + int64_t(wave) * 64; base < n1; base += kWideThreads) {
      const int64_t n = std::min<int64_t>(base + lane, n1 - 1);
      float acc[NW][4];
#pragma unroll
      for (int t = 0; t < NW; ++t)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) acc[t][qq] = 0.f;
#pragma unroll 1
      for (int step = 0; step < 8; ++step) {   // 128 coordinates (four words) per step
        uint4 w[P];
#pragma unroll
        for (int p = 0; p < P; ++p) w[p] = pg[(p * N + n) * REC + 8 * sl + step];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int blk = 2 * step + hb;
          uint32_t wa[P], wb[P];
#pragma unroll
          for (int p = 0; p < P; ++p) {
            wa[p] = hb ? w[p].z : w[p].x;
            wb[p] = hb ? w[p].w : w[p].y;
          }
#pragma unroll
          for (int t = 0; t < B; ++t) add_block(wa[t], wb[t], 0, blk, acc[t]);
          if constexpr (B == 3) add_block(wa[0] ^ wa[1] ^ wa[2], wb[0] ^ wb[1] ^ wb[2], 0, blk, acc[P]);
          add_block(wa[B], wb[B], 1, blk, acc[B]);
        }
      }
      const uint32_t nrm = ng[n];
      const float nu = h2f(nrm & 0xffffu);
      const float rs = h2f(nrm >> 16) * qs;
      const bool valid = base + lane < n1;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        float mse;
        if constexpr (B == 1) {
          mse = a0 * acc[0][qq];
        } else if constexpr (B == 2) {
          mse = fmaf(a0, acc[0][qq], a1 * acc[1][qq]);
        } else {
          mse = fmaf(a0, acc[0][qq], fmaf(a1, acc[1][qq], fmaf(a2, acc[2][qq], a3 * acc[P][qq])));
        }
        float v = fmaf(nu, mse, -rs * acc[B][qq]);
        const int qh = qc * 4 + qq;
        if (valid && qh < Qg) {
          float* dst = &logits[(g * Qg + qh) * N + n];
          v += sl == 0 ? fmaf(nu, -asum * sr[qq], rs * ss[qq]) : *dst;
          *dst = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- decode
// nu~ R^T c[code] = nu~ D H c[code] / sqrt(d), one key per wave (lane L:
// coordinates C L + t, bits of plane words C L / 32 + w); rows of din elements.
template <int B, bool BF16OUT, int C>
__global__ __launch_bounds__(256) void decode_wide_kernel(const uint32_t* __restrict__ planes,
                                                          const uint32_t* __restrict__ norms,
                                                          int64_t total, int64_t N,
                                                          void* __restrict__ out,
                                                          const DevConsts* __restrict__ cst) {
  constexpr int DD = 64 * C, Wd = C / 32;
  constexpr int P = B + 1;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t wstride = int64_t(gridDim.x) * 4;
  uint32_t dn[Wd];
#pragma unroll
  for (int w = 0; w < Wd; ++w) dn[w] = cst->dneg[Wd * lane + w];
  const int din = int(cst->din);
  const float inv_sqrt_d = cst->inv_sqrt_d;
  for (int64_t kk = wave0; kk < total; kk += wstride) {
    const int64_t g = kk / N, n = kk - g * N;
    float x[C];
#pragma unroll
    for (int w = 0; w < Wd; ++w) {
      uint32_t bits[B];
#pragma unroll
      for (int p = 0; p < B; ++p) bits[p] = planes[((g * P + p) * N + n) * (DD / 32) + Wd * lane + w];
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        int c = 0;
#pragma unroll
        for (int p = 0; p < B; ++p) c |= int((bits[p] >> j) & 1u) << p;
        x[32 * w + j] = cst->levels[c];
      }
    }
    hadamard(x, lane, false);
    const float sc = h2f(norms[g * N + n] & 0xffffu) * inv_sqrt_d;
#pragma unroll
    for (int t = 0; t < C; ++t) x[t] = ((dn[t >> 5] >> (t & 31)) & 1u) ? -(x[t] * sc) : x[t] * sc;
    if constexpr (BF16OUT) {
#pragma unroll
      for (int j = 0; j < C / 8; ++j) {
        const int c0 = C * lane + 8 * j;
        if (c0 >= din) continue;
        uint32_t w4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 lo = static_cast<__bf16>(x[8 * j + 2 * i]), hi = static_cast<__bf16>(x[8 * j + 2 * i + 1]);
          w4[i] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + kk * din + c0) =
            make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < C / 4; ++j) {
        const int c0 = C * lane + 4 * j;
        if (c0 >= din) continue;
        *reinterpret_cast<float4*>(static_cast<float*>(out) + kk * din + c0) =
            make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
      }
    }
  }
}

}  // namespace

// Keys per workspace chunk of the D > 1024 encoder: 256 MiB of residuals.
static int64_t wider_chunk_keys(int D) { return (int64_t(1) << 26) / D; }

template <int DD>
static hipError_t encode_wider(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t N,
                               void* packed, hipStream_t s) {
  constexpr int C = DD / 64;
  const int64_t total = G * N;
  const int P = cb.bits;
  uint32_t* planes = static_cast<uint32_t*>(packed);
  uint32_t* norms = planes + total * int64_t(P) * (DD / 32);
  const int64_t chunk = std::min<int64_t>(total, wider_chunk_keys(DD));
  float* ws = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&ws), size_t(chunk) * DD * sizeof(float), s);
  if (e != hipSuccess) return e;
  const int cus = std::max(1, cb.num_cus);
  for (int64_t k0 = 0; k0 < total && e == hipSuccess; k0 += chunk) {
    const int64_t nk = std::min<int64_t>(chunk, total - k0);
    const int rgrid = int(std::min<int64_t>((nk + 3) / 4, int64_t(cus) * 8));
#define TQ_ROTW(BB, BF)                                                                              \
    hipLaunchKernelGGL((rotate_wide_kernel<BB, BF, C>), dim3(rgrid), dim3(256), 0, s, keys, k0, nk, N, \
                       planes, norms, ws, cb.d_consts)
    const bool bf = dtype == 1;
    switch (cb.bits - 1) {
      case 1: if (bf) TQ_ROTW(1, true); else TQ_ROTW(1, false); break;
      case 2: if (bf) TQ_ROTW(2, true); else TQ_ROTW(2, false); break;
      default: if (bf) TQ_ROTW(3, true); else TQ_ROTW(3, false); break;
    }
#undef TQ_ROTW
    const int qgrid = int(std::min<int64_t>((nk + kQjlKeys - 1) / kQjlKeys, int64_t(cus)));
    hipLaunchKernelGGL(qjl_wide_kernel<DD>, dim3(qgrid), dim3(kQjlThreads), 0, s, ws, k0, nk, N, P, planes,
                       cb.d_fragW);
    e = hipGetLastError();
  }
  const hipError_t ef = hipFreeAsync(ws, s);
  return e != hipSuccess ? e : ef;
}

hipError_t launch_encode_wider(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t N,
                               void* packed, hipStream_t s) {
  return cb.d == 2048 ? encode_wider<2048>(cb, keys, dtype, G, N, packed, s)
                      : encode_wider<4096>(cb, keys, dtype, G, N, packed, s);
}

size_t score_wider_prep_bytes(const Codebook& cb, int64_t G, int Qg) {
  return size_t(G) * Qg * (2 * size_t(cb.d) + 4) * sizeof(float);
}

template <int DD>
static hipError_t score_wider(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                              const void* packed, int64_t N, float* logits, void* ws, hipStream_t s) {
  float* X = static_cast<float*>(ws);
  float* sums = X + G * Qg * 2 * DD;
  const dim3 pgrid{unsigned(G * Qg), unsigned(DD / 1024)};
  if (qdtype == 1)
    hipLaunchKernelGGL((qprep_wide_kernel<true, DD>), pgrid, dim3(1024), 0, s, q, X, sums, cb.d_consts, cb.d_St,
                       cb.d_Scol);
  else
    hipLaunchKernelGGL((qprep_wide_kernel<false, DD>), pgrid, dim3(1024), 0, s, q, X, sums, cb.d_consts,
                       cb.d_St, cb.d_Scol);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqc = (Qg + 3) / 4;
  const int64_t units = G * nqc;
  const int64_t cus = std::max(1, cb.num_cus);
  int64_t want = std::max<int64_t>(1, (cus + units - 1) / units);
  want = std::min<int64_t>(want, std::max<int64_t>(1, (N + 1023) / 1024));
  const int64_t chunk = ((N + want - 1) / want + 63) / 64 * 64;
  const int64_t ranges = (N + chunk - 1) / chunk;
  const dim3 grid{unsigned(G), unsigned(nqc), unsigned(ranges)};
  const uint4* planes = static_cast<const uint4*>(packed);
  const uint32_t* norms = static_cast<const uint32_t*>(packed) + G * N * int64_t(cb.bits) * (DD / 32);
#define TQ_SWW(BB)                                                                                       \
  hipLaunchKernelGGL((score_wide_kernel<BB, DD>), grid, dim3(kWideThreads), 0, s, planes, norms, N, Qg, chunk, \
                     X, sums, logits, cb.d_consts)
  switch (cb.bits - 1) {
    case 1: TQ_SWW(1); break;
    case 2: TQ_SWW(2); break;
    default: TQ_SWW(3); break;
  }
#undef TQ_SWW
  return hipGetLastError();
}

hipError_t launch_score_wider(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                              const void* packed, int64_t N, float* logits, void* ws, hipStream_t s) {
  return cb.d == 2048 ? score_wider<2048>(cb, q, qdtype, G, Qg, packed, N, logits, ws, s)
                      : score_wider<4096>(cb, q, qdtype, G, Qg, packed, N, logits, ws, s);
}

template <int DD>
static hipError_t decode_wider(const Codebook& cb, const void* packed, int64_t G, int64_t N, void* out,
                               int odtype, hipStream_t s) {
  constexpr int C = DD / 64;
  const int64_t total = G * N;
  const uint32_t* planes = static_cast<const uint32_t*>(packed);
  const uint32_t* norms = planes + total * int64_t(cb.bits) * (DD / 32);
  const int grid = int(std::min<int64_t>((total + 3) / 4, int64_t(std::max(1, cb.num_cus)) * 16));
  const bool bf = odtype == 1;
#define TQ_DWW(BB, BF)                                                                                 \
  hipLaunchKernelGGL((decode_wide_kernel<BB, BF, C>), dim3(grid), dim3(256), 0, s, planes, norms, total, N, \
                     out, cb.d_consts)
  switch (cb.bits - 1) {
    case 1: if (bf) TQ_DWW(1, true); else TQ_DWW(1, false); break;
    case 2: if (bf) TQ_DWW(2, true); else TQ_DWW(2, false); break;
    default: if (bf) TQ_DWW(3, true); else TQ_DWW(3, false); break;
  }
#undef TQ_DWW
  return hipGetLastError();
}

hipError_t launch_decode_wider(const Codebook& cb, const void* packed, int64_t G, int64_t N, void* out,
                               int odtype, hipStream_t s) {
  return cb.d == 2048 ? decode_wider<2048>(cb, packed, G, N, out, odtype, s)
                      : decode_wider<4096>(cb, packed, G, N, out, odtype, s);
}

}  // namespace tq

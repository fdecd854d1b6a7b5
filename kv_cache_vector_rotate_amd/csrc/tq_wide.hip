// TurboQuant key path for d = m = 1024 (the vector-search shape) on gfx950.
//
// Encode is one kernel (encode1024_kernel), tiles of 32 keys per workgroup:
// each wave rotates keys (y = H D k / (nu sqrt(d)), a 1024-point butterfly:
// four stages inside the lane, six across lanes), writes their Lloyd-Max
// code planes, nu and rho, and leaves the residual 2^12 (y - c[code]) in LDS
// as float16 hi + lo; then the QJL projection p = (S R^T) r_rot of the tile
// runs on the matrix cores (S R^T exact in fp16, fp32 accumulation) and the
// sign words [p < 0] are stored.
// [ICLR 2026 paper digest, "Step 1: PolarQuant" (R = H_d D / sqrt(d)) and the
//  implementation pseudocode (zero vectors, sign convention); Qiita
//  explainer, "Stage 2: QJL" (sign sketch of the residual).]

#include "tq_internal.h"

#include <algorithm>
#include <cstdint>

namespace tq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 1024;

__device__ __forceinline__ uint32_t push_sign(uint32_t acc, float v) {
  return __builtin_amdgcn_alignbit(acc, __float_as_uint(v), 31);   // (acc << 1) | signbit(v)
}

__device__ __forceinline__ uint16_t f2h_bits(float v) {
  const _Float16 h = static_cast<_Float16>(v);
  return __builtin_bit_cast(uint16_t, h);
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

__device__ __forceinline__ uint32_t lane_xor1_u(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xF, 0xF, false));
}

// butterfly stage across lanes L, L ^ S on every register: (a, b) -> (a + b, a - b)
template <int S>
__device__ __forceinline__ void stage_lanes(float (&x)[16], int lane) {
  const float sg = (lane & S) ? -1.0f : 1.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t) x[t] = fmaf(sg, x[t], lane_xor<S>(x[t]));
}

__device__ __forceinline__ void stage_lanes32(float (&x)[16], int lane) {
  const bool up = lane & 32;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
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

// ---------------------------------------------------------------- rotate
// One key per wave.  Lane L holds coordinates 16 L + t, t = 0..15: strides
// 1..8 inside the lane, 16..512 across lanes.  Each lane fills 16 bits of a
// plane word (word L / 2, bits 16 (L & 1) + t); even lanes then hold whole
// words after one DPP swap.  The residual comes back as 2^12 (y - c[code])
// (unit-vector units), zero for zero keys.
template <int B>
struct Rot1024 {
  static constexpr int K = 1 << (B - 1);   // levels on the positive half
  float tpos[K > 1 ? K - 1 : 1], cpos[K];
  float sqrt_d;
  uint32_t dn;     // the lane's 16 sign bits of D
  int din, col;    // row length; the lane's first input column (0 for padding lanes)
  bool lane_in;    // lanes at or past din / 16 hold zero padding

  __device__ __forceinline__ void load(const DevConsts* __restrict__ cst, int lane) {
#pragma unroll
    for (int k = 0; k < K - 1; ++k) tpos[k] = cst->tpos[k];
#pragma unroll
    for (int k = 0; k < K; ++k) cpos[k] = cst->cpos_s[k];
    sqrt_d = cst->sqrt_d;
    dn = (cst->dneg[lane >> 1] >> (16 * (lane & 1))) & 0xffffu;
    // rows of din <= 1024 elements (a multiple of 16): padding lanes re-read
    // the row's first chunk and zero it
    din = int(cst->din);
    lane_in = 16 * lane < din;
    col = lane_in ? 16 * lane : 0;
  }
};

// the lane's 16 input coordinates of a key, as loaded (bf16: two 16-byte
// loads; float32: four)
template <bool BF16> struct KeyRegs1024;
template <> struct KeyRegs1024<true> {
  uint4 v[2];
  static constexpr int kParts = 2;
};
template <> struct KeyRegs1024<false> {
  float4 v[4];
  static constexpr int kParts = 4;
};

template <bool BF16>
__device__ __forceinline__ void load_key_part(KeyRegs1024<BF16>& r, int part, const void* __restrict__ keys,
                                              int64_t kk, int din, int col) {
  // streamed once: non-temporal, so the keys do not push the L2-resident
  // sketch fragments out
  if constexpr (BF16) {
    const u32x4 v = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(keys) + kk * din + col) + part);
    r.v[part] = make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    const f32x4 v = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(static_cast<const float*>(keys) + kk * din + col) + part);
    r.v[part] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack_key(const KeyRegs1024<BF16>& r, bool lane_in, float (&x)[16]) {
  if constexpr (BF16) {
    const uint32_t u[8] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w, r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = lane_in ? __uint_as_float(u[i] << 16) : 0.f;
      x[2 * i + 1] = lane_in ? __uint_as_float(u[i] & 0xffff0000u) : 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = r.v[i];
      x[4 * i] = lane_in ? v.x : 0.f;
      x[4 * i + 1] = lane_in ? v.y : 0.f;
      x[4 * i + 2] = lane_in ? v.z : 0.f;
      x[4 * i + 3] = lane_in ? v.w : 0.f;
    }
  }
}

// y = H D k / (nu sqrt(d)), Lloyd-Max codes -> code planes, nu and rho ->
// norms (both written when `store`), residual 2^12 (y - c[code]) -> ep.
template <int B>
__device__ __forceinline__ void rotate_quantize1024(float (&x)[16], const Rot1024<B>& rc, int lane, int64_t kk,
                                                    int64_t N, bool store, uint32_t* __restrict__ planes,
                                                    uint32_t* __restrict__ norms, float (&ep)[16]) {
  constexpr int K = Rot1024<B>::K;
  constexpr int P = B + 1;
  float nu2 = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t) nu2 = fmaf(x[t], x[t], nu2);
#pragma unroll
  for (int t = 0; t < 16; ++t) x[t] = __uint_as_float(__float_as_uint(x[t]) ^ (((rc.dn >> t) & 1u) << 31));
  // first stage adds +0: sign-flipped zeros would otherwise leave -0, and an
  // exact zero must count as non-negative
#pragma unroll
  for (int t = 0; t < 16; t += 2) {
    const float a = x[t], b = x[t + 1];
    x[t] = (a + b) + 0.0f;
    x[t + 1] = (a - b) + 0.0f;
  }
#pragma unroll
  for (int st = 2; st < 16; st <<= 1)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
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

  nu2 = wave_sum(nu2);
  const float nu = sqrtf(nu2);
  const bool zero = !(nu >= 1e-10f);
  const float nsd = nu * rc.sqrt_d;                       // u = y nu sqrt(d)
  const float gsc = zero ? 0.f : kResidualScale / nsd;    // u -> 2^12 y
  float tu[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) tu[k] = rc.tpos[k] * nsd;

  uint32_t wu = 0u, wd[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int k = 0; k < (K > 1 ? K - 1 : 1); ++k) wd[k] = 0u;
  float rho2 = 0.f;
#pragma unroll
  for (int t = 15; t >= 0; --t) {   // pushed last = bit 0: bit t holds coordinate 16 L + t
    const float u = x[t], a = fabsf(u);
    wu = push_sign(wu, u);
    float mag = rc.cpos[0];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
      const float dk = a - tu[k];
      wd[k] = push_sign(wd[k], dk);
      mag = (dk >= 0.f) ? rc.cpos[k + 1] : mag;
    }
    const float e = fmaf(u, gsc, -copysignf(mag, u));     // 2^12 (y - c[code])
    ep[t] = zero ? 0.f : e;
    rho2 = fmaf(ep[t], ep[t], rho2);
  }
  rho2 = wave_sum(rho2);
  const float rho = zero ? 0.f : sqrtf(rho2) * (nu * (1.0f / kResidualScale));

  // the low halves (even lanes) take the odd lane's 16 bits as their high half
  const uint32_t fu = (wu & 0xffffu) | (lane_xor1_u(wu) << 16);
  uint32_t fd[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) fd[k] = (wd[k] & 0xffffu) | (lane_xor1_u(wd[k]) << 16);
  uint32_t pw[P - 1];
  if constexpr (B == 1) {
    pw[0] = ~fu;
  } else if constexpr (B == 2) {
    pw[1] = ~fu;
    pw[0] = ~(fu ^ fd[0]);
  } else {
    pw[2] = ~fu;
    pw[1] = ~(fu ^ fd[1]);
    pw[0] = ~(fu ^ fd[0] ^ fd[1] ^ fd[2]);
  }
  if (store) {
    const int64_t g = kk / N, n = kk - g * N;
    if (!(lane & 1)) {
#pragma unroll
      for (int p = 0; p < P - 1; ++p)
        planes[((g * P + p) * N + n) * 32 + (lane >> 1)] = zero ? 0u : pw[p];
    }
    if (lane == 0) norms[g * N + n] = zero ? 0u : (uint32_t(f2h_bits(nu)) | (uint32_t(f2h_bits(rho)) << 16));
  }
}

// ---------------------------------------------------------------- decode
// MSE-only reconstruction nu~ R^T c[code] = nu~ D H c[code] / sqrt(d), one key
// per wave: lane L unpacks coordinates 16 L + t (bits 16 (L & 1) + t of plane
// word L / 2), applies the same 1024-point butterfly as the rotation (H is
// symmetric), then D and the scale; rows of din elements are written.
template <int B, bool BF16OUT>
__global__ __launch_bounds__(256) void decode1024_kernel(const uint32_t* __restrict__ planes,
                                                         const uint32_t* __restrict__ norms,
                                                         int64_t total, int64_t N,
                                                         void* __restrict__ out,
                                                         const DevConsts* __restrict__ cst) {
  constexpr int P = B + 1;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t wstride = int64_t(gridDim.x) * 4;
  const uint32_t dn = (cst->dneg[lane >> 1] >> (16 * (lane & 1))) & 0xffffu;
  const int din = int(cst->din);
  const bool lane_in = 16 * lane < din;
  const float inv_sqrt_d = cst->inv_sqrt_d;
  for (int64_t kk = wave0; kk < total; kk += wstride) {
    const int64_t g = kk / N, n = kk - g * N;
    uint32_t bits16[B];
#pragma unroll
    for (int p = 0; p < B; ++p)
      bits16[p] = (planes[((g * P + p) * N + n) * 32 + (lane >> 1)] >> (16 * (lane & 1))) & 0xffffu;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      int c = 0;
#pragma unroll
      for (int p = 0; p < B; ++p) c |= int((bits16[p] >> t) & 1u) << p;
      x[t] = cst->levels[c];
    }
#pragma unroll
    for (int st = 1; st < 16; st <<= 1)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
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
    const uint32_t nb = norms[g * N + n] & 0xffffu;
    const float sc = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(nb))) * inv_sqrt_d;
#pragma unroll
    for (int t = 0; t < 16; ++t) x[t] = ((dn >> t) & 1u) ? -(x[t] * sc) : x[t] * sc;
    if (!lane_in) continue;
    if constexpr (BF16OUT) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const __bf16 lo = static_cast<__bf16>(x[2 * i]), hi = static_cast<__bf16>(x[2 * i + 1]);
        w[i] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
      }
      uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + kk * din + 16 * lane);
      o[0] = make_uint4(w[0], w[1], w[2], w[3]);
      o[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + kk * din + 16 * lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
    }
  }
}

// ---------------------------------------------------------------- encoder
// One kernel per launch, one workgroup per CU walking tiles of 32 keys; the
// residuals never leave the chip.  Per tile:
//  * rotation: wave w rotates and quantises keys 4w .. 4w + 3 of the tile
//    (one key at a time, the whole wave per key), stores their code planes
//    and norms, and writes the residual into LDS as float16 hi + lo in the
//    matrix core's B order: rotating lane L holds coordinates 16 L + t, which
//    is exactly k-step L (its halves 8h .. 8h + 7 for the B lanes of half h);
//  * sketch: wave w owns sketch rows [128 w, 128 w + 128) (four 32-row
//    blocks) for all 32 keys and runs the 64 k-steps, each product two terms
//    S_rot r_hi + S_rot r_lo with (S R^T) exact in float16 (fragments read
//    from L2, 15 (row block, k-step) steps ahead in a ring of 16, the ring
//    running on into the next tile's first steps);
//  * signs: sign words [p < 0] through LDS, one 16-byte store per 4 words.
// The next tile's first keys are loaded into registers as the sketch loop
// starts, the rest as its rotation phase starts.
// LDS: 128 KB of residual fragments + 4 KB of sign words.
constexpr int kEncThreads = 512;
constexpr int kEncKeys = 32;
constexpr int kRing = 16;

__device__ __forceinline__ void split_f16x8(const float* v, uint4& hi, uint4& lo) {
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

template <int B, bool BF16>
__global__ __launch_bounds__(kEncThreads, 1) void encode1024_kernel(const void* __restrict__ keys, int64_t nk,
                                                                    int64_t N, uint32_t* __restrict__ planes,
                                                                    uint32_t* __restrict__ norms,
                                                                    const uint4* __restrict__ fragA,
                                                                    const DevConsts* __restrict__ cst) {
  constexpr int P = B + 1;
  constexpr int kParts = KeyRegs1024<BF16>::kParts;
  constexpr int kKeysPerWave = kEncKeys / (kEncThreads / 64);   // 4
  // [k-step][hi, lo][B lane ^ k-step]: the rotating lane L = k-step writes
  // the slots (32 h + key) ^ L, so the 8 lanes of one write cycle hit 8
  // different bank groups; a B read of one k-step is a permutation of one
  // contiguous 1 KB row
  __shared__ uint4 sb[64][2][64];
  __shared__ uint32_t s_sign[kEncKeys][33];   // [key][word], padded
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  Rot1024<B> rc;
  rc.load(cst, lane);
  const int64_t ntiles = (nk + kEncKeys - 1) / kEncKeys;

  // A fragments: row block 4 w + rb, k-step ks; step = 4 ks + rb.  Buffer
  // loads: the wave's 256 KB of fragments as the resource (its size as the
  // range, so a load past it returns zeros; the last word 0x00020000 gives
  // the 32-bit data format that raw buffer loads need on this family), the
  // lane's 16-byte slot as the vector offset, the step's 1 KB row as the
  // scalar offset.
  const __amdgpu_buffer_rsrc_t frs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(fragA + size_t(4 * wave) * 64 * 64), short(0), 4 * 64 * 64 * 16, 0x00020000);
  const int voff = 16 * lane;
  auto load_a = [&](int step, half8& ah) {
    const int ks = step >> 2, rb = step & 3;
    ah = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(frs, voff, (rb * 64 + ks) * 1024, 0));
  };
  half8 ah[kRing];
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i) load_a(i, ah[i]);

  // the wave's first two keys of a tile are loaded during the previous
  // tile's sketch loop, the other two as its rotation starts (they land while
  // the first two are rotated): registers for all four would not fit beside
  // the accumulators and the fragment ring
  constexpr int kEarly = 2;
  KeyRegs1024<BF16> pf[kKeysPerWave];
  auto key_of = [&](int64_t tile, int i) {   // clamped: tail keys re-read the last key
    return std::min<int64_t>(tile * kEncKeys + kKeysPerWave * wave + i, nk - 1);
  };
  int64_t tile = blockIdx.x;
  if (tile < ntiles) {
#pragma unroll
    for (int i = 0; i < kEarly; ++i)
#pragma unroll
      for (int part = 0; part < kParts; ++part) load_key_part<BF16>(pf[i], part, keys, key_of(tile, i), rc.din, rc.col);
  }

  for (; tile < ntiles; tile += gridDim.x) {
#pragma unroll
    for (int i = kEarly; i < kKeysPerWave; ++i)
#pragma unroll
      for (int part = 0; part < kParts; ++part) load_key_part<BF16>(pf[i], part, keys, key_of(tile, i), rc.din, rc.col);
#pragma unroll
    for (int i = 0; i < kKeysPerWave; ++i) {
      const int n = kKeysPerWave * wave + i;
      const int64_t kk = tile * kEncKeys + n;
      float x[16], ep[16];
      unpack_key<BF16>(pf[i], rc.lane_in, x);
      rotate_quantize1024<B>(x, rc, lane, kk, N, kk < nk, planes, norms, ep);
      uint4 hi, lo;
      split_f16x8(ep, hi, lo);
      sb[lane][0][n ^ lane] = hi;
      sb[lane][1][n ^ lane] = lo;
      split_f16x8(ep + 8, hi, lo);
      sb[lane][0][(32 + n) ^ lane] = hi;
      sb[lane][1][(32 + n) ^ lane] = lo;
    }
    __syncthreads();

    // the next tile's first keys: in flight while the first ring steps run
    const int64_t next = tile + gridDim.x;
    if (next < ntiles) {
#pragma unroll
      for (int i = 0; i < kEarly; ++i)
#pragma unroll
        for (int part = 0; part < kParts; ++part) load_key_part<BF16>(pf[i], part, keys, key_of(next, i), rc.din, rc.col);
    }
    f32x16 acc[4] = {};
    constexpr int kKsIter = kRing / 4;
    // B fragments one k-step ahead; the schedule is pinned step by step so
    // that each fragment load goes out kRing - 1 steps before its products
    half8 bh = __builtin_bit_cast(half8, sb[0][0][lane]);
    half8 bl = __builtin_bit_cast(half8, sb[0][1][lane]);
#pragma unroll 1
    for (int c = 0; c < 64 / kKsIter; ++c) {
#pragma unroll
      for (int k4 = 0; k4 < kKsIter; ++k4) {
        const int ks = kKsIter * c + k4;
        const int kn = (ks + 1) & 63;
        const half8 nh = __builtin_bit_cast(half8, sb[kn][0][lane ^ kn]);
        const half8 nl = __builtin_bit_cast(half8, sb[kn][1][lane ^ kn]);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int st = 4 * k4 + rb;              // step kRing c + st; ring slot st
          load_a((kRing * c + st + kRing - 1) & 255, ah[(st + kRing - 1) % kRing]);
          acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[st], bh, acc[rb], 0, 0, 0);
          acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[st], bl, acc[rb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        bh = nh;
        bl = nl;
      }
    }

    // sign words: lane (key kl, half h) holds rows 8 (v / 4) + 4 h + (v % 4) of
    // each 32-row block; spread the 16 bits into nibbles and OR the halves
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      uint32_t b16 = 0u;
#pragma unroll
      for (int vv = 15; vv >= 0; --vv) b16 = push_sign(b16, acc[rb][vv]);
      uint32_t t = (b16 | (b16 << 8)) & 0x00FF00FFu;
      t = (t | (t << 4)) & 0x0F0F0F0Fu;
      t <<= 4 * h;
      auto pr = __builtin_amdgcn_permlane32_swap(t, t, false, false);
      const uint32_t word = pr[0] | pr[1];
      if (h == 0) s_sign[lane & 31][4 * wave + rb] = word;
    }
    __syncthreads();
    // 32 keys x 32 words: thread -> (key, 4 words)
    if (tid < kEncKeys * 8) {
      const int key = tid >> 3, q4 = tid & 7;
      const int64_t kk = tile * kEncKeys + key;
      if (kk < nk) {
        const int64_t g = kk / N, n = kk - g * N;
        uint4* dst = reinterpret_cast<uint4*>(planes + ((g * P + (P - 1)) * N + n) * 32) + q4;
        *dst = make_uint4(s_sign[key][4 * q4], s_sign[key][4 * q4 + 1], s_sign[key][4 * q4 + 2],
                          s_sign[key][4 * q4 + 3]);
      }
    }
  }
}

// ---------------------------------------------------------------- query preparation
// One workgroup per query: X_0 = 2 R q (butterfly in wave 0), X_1 = 2 S q
// (thread j forms row j from S^T columns, the query in LDS), and their sums.
// ws layout: float X[G*Qg][2][1024], then float sums[G*Qg][4] (sum R q, sum S q).
template <bool QBF16>
__global__ __launch_bounds__(1024) void qprep1024_kernel(const void* __restrict__ q, int64_t nq,
                                                        float* __restrict__ X, float* __restrict__ sums,
                                                        const DevConsts* __restrict__ cst,
                                                        const float* __restrict__ St) {
  __shared__ float s_q[kD];
  __shared__ float s_part[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gq = blockIdx.x;
  const int din = int(cst->din);   // query rows of din elements; the rest is zero padding
  if (tid >= din)
    s_q[tid] = 0.f;
  else if constexpr (QBF16)
    s_q[tid] = __uint_as_float(uint32_t(static_cast<const uint16_t*>(q)[gq * din + tid]) << 16);
  else
    s_q[tid] = static_cast<const float*>(q)[gq * din + tid];
  __syncthreads();
  float* xr = X + gq * 2 * kD;
  if (wave == 0) {
    const uint32_t dn = (cst->dneg[lane >> 1] >> (16 * (lane & 1))) & 0xffffu;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) x[t] = __uint_as_float(__float_as_uint(s_q[16 * lane + t]) ^ (((dn >> t) & 1u) << 31));
#pragma unroll
    for (int st = 1; st < 16; st <<= 1)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
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
    float sr = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      x[t] *= cst->inv_sqrt_d;
      sr += x[t];
    }
    float4* dst = reinterpret_cast<float4*>(xr + 16 * lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[i] = make_float4(2.f * x[4 * i], 2.f * x[4 * i + 1], 2.f * x[4 * i + 2], 2.f * x[4 * i + 3]);
    sr = wave_sum(sr);
    if (lane == 0) sums[gq * 4 + 0] = sr;
  }
  // S q, row j = tid: sum over c of S^T[c][j] q[c]
  float acc = 0.f;
#pragma unroll 16
  for (int c = 0; c < kD; ++c) acc = fmaf(St[int64_t(c) * kD + tid], s_q[c], acc);
  xr[kD + tid] = 2.f * acc;
  const float ws_ = wave_sum(acc);
  if (lane == 0) s_part[wave] = ws_;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) t += s_part[w];
    sums[gq * 4 + 1] = t;
  }
}

// ---------------------------------------------------------------- score
// Grid (g, chunk of 4 query heads, key range); 1024 threads.  Nibble
// subset-sum tables cover all 1024 coordinates at once (no table rebuilds,
// each packed record is read once):
//   T[ty][pos][nib] = sum over set bits t of nib of X_ty[4 pos + t]
// (four queries per 16-byte entry), entry (ty, pos = 16 blk + pl, nib) at
// byte ty * 64K + blk * 4K + nib * 256 + pl * 16: position pl of a 16-position
// block always lies in LDS bank group pl, and lane L visits the positions of
// a block in the order k ^ (L & 15), so the sixteen lanes served together
// never share a bank group.  Per key and plane: 256 lookups, 4 adds each.
// TOPK: instead of storing logits, each wave keeps the best K (score desc,
// index asc) per query in lanes 0..K-1; the workgroup merges its waves' lists
// into ws_topk[g][qh][range][K].
constexpr int kWideThreads = 1024;
constexpr int kMaxTopK = 16;

struct WideLds {
  f32x4 tab[2 * 16 * 16 * 16];            // 128 KB
  float lst_s[16][4][kMaxTopK];           // per-wave lists for the merge
  int32_t lst_i[16][4][kMaxTopK];
};

__device__ __forceinline__ bool better(float s, int32_t i, float t_s, int32_t t_i) {
  return s > t_s || (s == t_s && i < t_i);
}

// insert (cs, ci) into the list held in lanes 0..K-1 (ls, li), if it belongs there
__device__ __forceinline__ void list_insert(float& ls, int32_t& li, float cs, int32_t ci, int lane, int K) {
  const bool ahead = lane < K && better(ls, li, cs, ci);
  const int pos = __builtin_popcountll(__builtin_amdgcn_ballot_w64(ahead));
  if (pos >= K) return;
  const float ps = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ls), 0x111, 0xF, 0xF, false));   // row_shr:1
  const int32_t pi = __builtin_amdgcn_mov_dpp(li, 0x111, 0xF, 0xF, false);
  if (lane < K) {
    if (lane == pos) { ls = cs; li = ci; }
    else if (lane > pos) { ls = ps; li = pi; }
  }
}

template <int B, bool TOPK>
__global__ __launch_bounds__(kWideThreads, 1) void score1024_kernel(
    const uint4* __restrict__ planes, const uint32_t* __restrict__ norms, int64_t N, int Qg,
    int64_t chunk, const float* __restrict__ X, const float* __restrict__ sums,
    float* __restrict__ logits, int K, float* __restrict__ tk_s, int32_t* __restrict__ tk_i,
    const DevConsts* __restrict__ cst) {
  constexpr int P = B + 1;
  constexpr int NW = B == 3 ? P + 1 : P;
  __shared__ WideLds sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.x;
  const int qc = blockIdx.y;
  const int64_t n0 = int64_t(blockIdx.z) * chunk;
  const int64_t n1 = std::min<int64_t>(N, n0 + chunk);

  // ---- tables: thread (pl, half, blk, ty) writes nibbles 8 half .. 8 half + 7
  {
    const int pl = tid & 15, hf = (tid >> 4) & 1, blk = (tid >> 5) & 15, ty = tid >> 9;
    const int pos = 16 * blk + pl;
    f32x4 xv[4];   // coordinate 4 pos + t, four queries
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int qh = qc * 4 + qq;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (qh < Qg) v = *reinterpret_cast<const float4*>(X + ((g * Qg + qh) * 2 + ty) * kD + 4 * pos);
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
    for (int j = 0; j < 8; ++j) sm.tab[((ty * 16 + blk) * 16 + 8 * hf + j) * 16 + pl] = e[j];
  }
  __syncthreads();

  float sr[4], ss[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int qh = std::min(qc * 4 + qq, Qg - 1);
    sr[qq] = sums[(g * Qg + qh) * 4 + 0];
    ss[qq] = sums[(g * Qg + qh) * 4 + 1];
  }
  const float a0 = cst->alpha[0], a1 = cst->alpha[1], a2 = cst->alpha[2], a3 = cst->alpha[3];
  const float asum = cst->alpha_sum, qs = cst->qjl_scale;

  // per-lane pieces of the lookup order: lookup k of a block reads position
  // pl = k ^ r: word (k >> 3) of the block after swapping the pair when
  // r >= 8, nibble (k & 7) ^ (r & 7)
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
  const char* tabp = reinterpret_cast<const char*>(sm.tab);
  const uint4* pg = planes + g * P * N * 8;   // 128-byte plane records: 8 x 16 B
  const uint32_t* ng = norms + g * N;

  float ls[4], tsc[4];
  int32_t li[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) { ls[qq] = -__builtin_huge_valf(); li[qq] = 0x7fffffff; tsc[qq] = 0.f; }

  // one block of 64 coordinates (two words) of one plane against table ty
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
      for (int p = 0; p < P; ++p) w[p] = pg[(p * N + n) * 8 + step];
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
    const float nu = __builtin_bit_cast(_Float16, uint16_t(nrm & 0xffffu));
    const float rs = float(__builtin_bit_cast(_Float16, uint16_t(nrm >> 16))) * qs;
    const bool valid = base + lane < n1;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      float mse;
      if constexpr (B == 1) {
        mse = a0 * acc[0][qq] - asum * sr[qq];
      } else if constexpr (B == 2) {
        mse = fmaf(a0, acc[0][qq], a1 * acc[1][qq]) - asum * sr[qq];
      } else {
        mse = fmaf(a0, acc[0][qq], fmaf(a1, acc[1][qq], fmaf(a2, acc[2][qq], a3 * acc[P][qq]))) -
              asum * sr[qq];
      }
      const float v = fmaf(nu, mse, rs * (ss[qq] - acc[B][qq]));
      const int qh = qc * 4 + qq;
      if constexpr (!TOPK) {
        if (valid && qh < Qg) __builtin_nontemporal_store(v, &logits[(g * Qg + qh) * N + n]);
      } else {
        // candidates against the list's current last entry, inserted one by one
        const float t_s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[qq]), K - 1));
        const int32_t t_i = __builtin_amdgcn_readlane(li[qq], K - 1);
        uint64_t m = __builtin_amdgcn_ballot_w64(valid && better(v, int32_t(n), t_s, t_i));
        while (m) {
          const int b = __builtin_ctzll(m);
          m &= m - 1;
          const float cs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), b));
          const int32_t ci = __builtin_amdgcn_readlane(int32_t(n), b);
          list_insert(ls[qq], li[qq], cs, ci, lane, K);
        }
      }
    }
  }
  if constexpr (TOPK) {
    if (lane < K) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) { sm.lst_s[wave][qq][lane] = ls[qq]; sm.lst_i[wave][qq][lane] = li[qq]; }
    }
    __syncthreads();
    if (wave < 4) {   // wave qq merges query qq's sixteen lists
      const int qq = wave;
      float ms = lane < K ? sm.lst_s[0][qq][lane] : -__builtin_huge_valf();
      int32_t mi = lane < K ? sm.lst_i[0][qq][lane] : 0x7fffffff;
      for (int w = 1; w < 16; ++w)
        for (int j = 0; j < K; ++j) {
          const float cs = sm.lst_s[w][qq][j];
          const int32_t ci = sm.lst_i[w][qq][j];
          list_insert(ms, mi, cs, ci, lane, K);
        }
      const int qh = qc * 4 + qq;
      if (qh < Qg && lane < K) {
        const int64_t at = ((g * Qg + qh) * int64_t(gridDim.z) + blockIdx.z) * K + lane;
        tk_s[at] = ms;
        tk_i[at] = mi;
      }
    }
  }
}

// merge the per-range lists of one query: one wave per (g, qh)
__global__ __launch_bounds__(64) void topk_merge_kernel(const float* __restrict__ tk_s,
                                                        const int32_t* __restrict__ tk_i, int ranges,
                                                        int K, int32_t* __restrict__ out_i,
                                                        float* __restrict__ out_s) {
  const int lane = threadIdx.x;
  const int64_t gq = blockIdx.x;
  float ms = -__builtin_huge_valf();
  int32_t mi = 0x7fffffff;
  // the query's ranges x K candidates, 64 per wave step and eight steps'
  // loads in flight; only candidates better than the current K-th are
  // inserted (the order of equal scores is by index, so the result does not
  // depend on the order of insertion)
  constexpr int U = 8;
  const int64_t total = int64_t(ranges) * K;
  const float* cs_q = tk_s + gq * total;
  const int32_t* ci_q = tk_i + gq * total;
  for (int64_t base = 0; base < total; base += 64 * U) {
    float cs[U];
    int32_t ci[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t at = base + u * 64 + lane;
      cs[u] = at < total ? cs_q[at] : -__builtin_huge_valf();
      ci[u] = at < total ? ci_q[at] : 0x7fffffff;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float t_s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ms), K - 1));
      const int32_t t_i = __builtin_amdgcn_readlane(mi, K - 1);
      uint64_t m = __builtin_amdgcn_ballot_w64(better(cs[u], ci[u], t_s, t_i));
      while (m) {
        const int b = __builtin_ctzll(m);
        m &= m - 1;
        list_insert(ms, mi, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs[u]), b)),
                    __builtin_amdgcn_readlane(ci[u], b), lane, K);
      }
    }
  }
  if (lane < K) {
    const bool some = mi != 0x7fffffff;
    out_i[gq * K + lane] = some ? mi : -1;
    out_s[gq * K + lane] = ms;
  }
}

// ---------------------------------------------------------------- many-query top-k, matrix cores
// With many queries per group the estimator is a dense contraction over the
// 1024 coordinates:
//   score(q, v) = nu~ sum_i (R q)_i c[code_v,i] + rho~ sqrt(pi/2)/m sum_j (S q)_j (1 - 2 s_v,j)
// and both sums run on v_mfma_f32_32x32x16_f16 into one accumulator.  Query
// side (A, per query a power of two sigma_q): R q / (sqrt(d) sigma_q) and
// sqrt(pi/2)/m S q / sigma_q, each split into fp16 hi + lo.  Vector side (B,
// per vector a power of two 2^-e_v that brings nu~ into [0.5, 1)):
// nu~ 2^-e_v sqrt(d) c[code] as fp16 hi + lo, and rho~ 2^-e_v (1 - 2 s) exactly
// in fp16.  Products hi*hi + hi*lo + lo*hi (levels) and hi*s + lo*s (signs),
// fp32 accumulation: score = sigma_q 2^e_v C.  One LDS table maps the code
// and sign bits of two adjacent coordinates to their two levels and sign
// pattern.  Each wave owns 32 queries and keeps each query's best K (of
// C 2^e_v: sigma_q > 0 does not change the order) in one 16-lane row of a
// register pair; a workgroup walks a contiguous run of 128-vector tiles and
// writes its lists (times sigma_q) as one range for topk_merge_kernel.
constexpr int kMqThreads = 512;   // 8 waves, wave w = query rows 32 w .. 32 w + 31
constexpr int kMqMaxRb = 8;       // up to 256 queries per group

// A fragments: frag[g][rb][tile][ks][lane] (half8) for tiles R hi, R lo, S hi,
// S lo: query 32 rb + lane % 32 (zero past Qg) at coordinates
// 16 ks + 8 (lane / 32) .. + 7; sigma[g][32 rb + r].
__global__ __launch_bounds__(256) void mqprep1024_kernel(const float* __restrict__ X, int Qg, int rbs,
                                                         uint4* __restrict__ frag,
                                                         float* __restrict__ sigma,
                                                         const DevConsts* __restrict__ cst) {
  __shared__ float s_max[8][32];
  __shared__ float s_mul[2][32];
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x / rbs;
  const int rb = int(blockIdx.x - g * rbs);
  // X holds 2 R q and 2 S q: the A values are X times these factors over sigma
  const float fR = 0.5f * cst->inv_sqrt_d, fS = 0.5f * cst->qjl_scale;
  {
    const int r = tid & 31, part = tid >> 5, qh = 32 * rb + r;
    float m = 0.f;
    if (qh < Qg) {
      const float* x = X + (g * Qg + qh) * 2 * kD + 128 * part;
      for (int c = 0; c < 128; ++c) m = fmaxf(m, fmaxf(fabsf(x[c]) * fR, fabsf(x[kD + c]) * fS));
    }
    s_max[part][r] = m;
  }
  __syncthreads();
  if (tid < 32) {
    float m = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) m = fmaxf(m, s_max[p][tid]);
    int e = 0;
    if (m > 0.f) (void)frexpf(m, &e);            // m = f 2^e, f in [0.5, 1)
    const float sig = m > 0.f ? ldexpf(1.f, e) : 1.f;
    s_mul[0][tid] = fR / sig;                    // exact: powers of two
    s_mul[1][tid] = fS / sig;
    sigma[(g * rbs + rb) * 32 + tid] = sig;
  }
  __syncthreads();
  for (int e = tid; e < 64 * 64; e += 256) {
    const int ks = e >> 6, ln = e & 63, r = ln & 31, qh = 32 * rb + r;
    const int c0 = 16 * ks + 8 * (ln >> 5);
#pragma unroll
    for (int ty = 0; ty < 2; ++ty) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v0 = 0.f, v1 = 0.f;
        if (qh < Qg) {
          const float* x = X + (g * Qg + qh) * 2 * kD + ty * kD + c0 + 2 * j;
          v0 = x[0] * s_mul[ty][r];
          v1 = x[1] * s_mul[ty][r];
        }
        const half2v hv = {static_cast<_Float16>(v0), static_cast<_Float16>(v1)};
        const half2v lv = {static_cast<_Float16>(v0 - static_cast<float>(hv[0])),
                           static_cast<_Float16>(v1 - static_cast<float>(hv[1]))};
        hw[j] = __builtin_bit_cast(uint32_t, hv);
        lw[j] = __builtin_bit_cast(uint32_t, lv);
      }
      const size_t at = (((size_t(g) * rbs + rb) * 4 + 2 * ty) * 64 + ks) * 64 + ln;
      frag[at] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      frag[at + 64 * 64] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  }
}

// insert (cs, ci) into row `row` (lanes 16 row .. 16 row + K - 1) of (ls, li)
__device__ __forceinline__ void row_insert(float& ls, int32_t& li, float cs, int32_t ci, int lane,
                                           int row, int K) {
  const int rl = lane & 15;
  const bool mine = (lane >> 4) == row && rl < K;
  const int pos = __builtin_popcountll(__builtin_amdgcn_ballot_w64(mine && better(ls, li, cs, ci)));
  if (pos >= K) return;
  const float ps = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ls), 0x111, 0xF, 0xF, false));
  const int32_t pi = __builtin_amdgcn_mov_dpp(li, 0x111, 0xF, 0xF, false);   // row_shr:1
  if (mine) {
    if (rl == pos) { ls = cs; li = ci; }
    else if (rl > pos) { ls = ps; li = pi; }
  }
}

template <int B>
__global__ __launch_bounds__(kMqThreads, 1) void mqtopk1024_kernel(
    const uint32_t* __restrict__ planes, const uint32_t* __restrict__ norms, int64_t N, int Qg,
    int rbs, int64_t tiles_per_wg, const uint4* __restrict__ frag, const float* __restrict__ sigma,
    int K, float* __restrict__ tk_s, int32_t* __restrict__ tk_i, const DevConsts* __restrict__ cst) {
  constexpr int P = B + 1;
  constexpr int NLUT = 1 << (2 * P);
  __shared__ uint4 s_lut[NLUT];                 // (level a, level b (times sqrt d), sign mask, 0)
  __shared__ uint4 s_b[2][4][4][3][64];         // [buffer][k-step][vector block][tile][lane]: 96 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.y;
  const int64_t ntiles = (N + 127) / 128;
  const int64_t t0 = int64_t(blockIdx.x) * tiles_per_wg;
  const int64_t t1 = std::min<int64_t>(ntiles, t0 + tiles_per_wg);

  for (int j = tid; j < NLUT; j += kMqThreads) {
    int ca = 0, cb = 0;
#pragma unroll
    for (int p = 0; p < B; ++p) {
      ca |= ((j >> (2 * p)) & 1) << p;
      cb |= ((j >> (2 * p + 1)) & 1) << p;
    }
    const float la = cst->levels[ca] * cst->sqrt_d, lb = cst->levels[cb] * cst->sqrt_d;
    const uint32_t sm = (((j >> (2 * B)) & 1u) << 15) | (((j >> (2 * B + 1)) & 1u) << 31);
    s_lut[j] = make_uint4(__float_as_uint(la), __float_as_uint(lb), sm, 0u);
  }

  float ls[8];      // query r: register r / 4, lanes 16 (r % 4) .. + K - 1
  int32_t li[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) { ls[k] = -__builtin_huge_valf(); li[k] = 0x7fffffff; }
  // each query's current k-th score (wave-uniform), read again only after an
  // insertion into its list
  float thr_s[8][4];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 4; ++r) thr_s[k][r] = -__builtin_huge_valf();
  float mone = -1.0f;
  asm volatile("" : "+v"(mone));

  const uint4* fa = frag + ((size_t(g) * rbs + (wave < rbs ? wave : 0)) * 4) * 64 * 64 + lane;
  // B operand of chunk c of tile t (k-steps 4c .. 4c+3), item i = (k-step,
  // vector block, lane), in two halves: the record loads (into registers, one
  // chunk ahead of their use, so that their latency is covered by a chunk of
  // products) and the expansion into LDS
  struct ChunkRegs {
    uint32_t by[2][P];
    uint32_t nr[2];
  };
  auto load_chunk = [&](int64_t tile, int c, ChunkRegs& r) {
    const int64_t nb = tile * 128;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + it * kMqThreads;
      const int ksl = i >> 8, vb = (i >> 6) & 3, ln = i & 63;
      const int ks = 4 * c + ksl;
      const int64_t v = std::min<int64_t>(nb + 32 * vb + (ln & 31), N - 1);
      const int w = ks >> 1;
#pragma unroll
      for (int p = 0; p < P; ++p) r.by[it][p] = planes[((g * P + p) * N + v) * 32 + w];
      r.nr[it] = norms[g * N + v];
    }
  };
  auto expand = [&](int c, int buf, const ChunkRegs& r) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + it * kMqThreads;
      const int ksl = i >> 8, vb = (i >> 6) & 3, ln = i & 63;
      const int ks = 4 * c + ksl;
      const int bo = 16 * (ks & 1) + 8 * (ln >> 5);
      uint32_t by[P];
#pragma unroll
      for (int p = 0; p < P; ++p) by[p] = (r.by[it][p] >> bo) & 0xffu;
      const uint32_t nr = r.nr[it];
      const float nu = __builtin_bit_cast(_Float16, uint16_t(nr & 0xffffu));
      const float rho = __builtin_bit_cast(_Float16, uint16_t(nr >> 16));
      int e = 0;
      if (nu > 0.f) (void)frexpf(nu, &e);
      const float nus = ldexpf(nu, -e), rhos = ldexpf(rho, -e);   // exact
      const uint32_t rb16 = f2h_bits(rhos);                        // exact: rho~ is a half
      const uint32_t rr = rb16 | (rb16 << 16);
      uint32_t ch[4], cl[4], sg[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t idx = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) idx |= ((by[p] >> (2 * j)) & 3u) << (2 * p);
        const uint4 en = s_lut[idx];
        const float ma = nus * __uint_as_float(en.x), mb = nus * __uint_as_float(en.y);
        const half2v hv = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(ma, mb));
        const half2v lv = {static_cast<_Float16>(__builtin_fmaf(static_cast<float>(hv[0]), mone, ma)),
                           static_cast<_Float16>(__builtin_fmaf(static_cast<float>(hv[1]), mone, mb))};
        ch[j] = __builtin_bit_cast(uint32_t, hv);
        cl[j] = __builtin_bit_cast(uint32_t, lv);
        sg[j] = rr ^ en.z;
      }
      s_b[buf][ksl][vb][0][ln] = make_uint4(ch[0], ch[1], ch[2], ch[3]);
      s_b[buf][ksl][vb][1][ln] = make_uint4(cl[0], cl[1], cl[2], cl[3]);
      s_b[buf][ksl][vb][2][ln] = make_uint4(sg[0], sg[1], sg[2], sg[3]);
    }
  };
  // A fragments of k-step ks (query R q hi, lo; S q hi, lo) in register set
  // ks % kAr, requested kAr - 1 k-steps before their products
  constexpr int kAr = 4;   // two ahead: 3.99 ms for workload 4; three ahead: 3.88
  half8 ar[kAr][4];
  auto load_a = [&](int ks, half8 (&a)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = __builtin_bit_cast(half8, fa[(t * 64 + ks) * 64]);
  };
  auto products = [&](int c, int buf, f32x16 (&acc)[4]) {
    if (wave < rbs) {
#pragma unroll
      for (int ksl = 0; ksl < 4; ++ksl) {
        const int ks = 4 * c + ksl;
        load_a((ks + kAr - 1) & 63, ar[(ksl + kAr - 1) % kAr]);   // on into the next tile's first k-steps
        const half8(&a)[4] = ar[ksl % kAr];
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) {
          const half8 bh = __builtin_bit_cast(half8, s_b[buf][ksl][vb][0][lane]);
          const half8 bl = __builtin_bit_cast(half8, s_b[buf][ksl][vb][1][lane]);
          const half8 bs = __builtin_bit_cast(half8, s_b[buf][ksl][vb][2][lane]);
          acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], bh, acc[vb], 0, 0, 0);
          acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0], bl, acc[vb], 0, 0, 0);
          acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[1], bh, acc[vb], 0, 0, 0);
          acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[2], bs, acc[vb], 0, 0, 0);
          acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[3], bs, acc[vb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if (wave < rbs) {
#pragma unroll
    for (int i = 0; i < kAr - 1; ++i) load_a(i, ar[i]);
  }
  // chunk k of the walk (tile t0 + k / 16, chunk k % 16): its records are
  // loaded while chunk k - 2 is multiplied, expanded into buffer k % 2 while
  // chunk k - 1 is; register set k % 2
  ChunkRegs rg[2];
  const int64_t nchunks = (t1 - t0) * 16;
  if (nchunks > 0) load_chunk(t0, 0, rg[0]);
  if (nchunks > 1) load_chunk(t0, 1, rg[1]);
  __syncthreads();             // the table
  if (nchunks > 0) expand(0, 0, rg[0]);
  __syncthreads();
  for (int64_t tile = t0; tile < t1; ++tile) {
    const int64_t nb = tile * 128;
    const int64_t kb = (tile - t0) * 16;
    f32x16 acc[4] = {};
#pragma unroll 1
    for (int c = 0; c < 16; c += 2) {
      // even chunk (buffer 0) multiplied; the odd one (set 1) expanded into
      // buffer 1; the next even one's records into set 0
      if (kb + c + 1 < nchunks) expand(c + 1, 1, rg[1]);
      if (kb + c + 2 < nchunks) load_chunk(t0 + (kb + c + 2) / 16, (c + 2) % 16, rg[0]);
      products(c, 0, acc);
      __syncthreads();
      if (kb + c + 2 < nchunks) expand((c + 2) % 16, 0, rg[0]);
      if (kb + c + 3 < nchunks) load_chunk(t0 + (kb + c + 3) / 16, (c + 3) % 16, rg[1]);
      products(c + 1, 1, acc);
      __syncthreads();
    }
    if (wave < rbs) {
      const int h = lane >> 5;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        const int64_t v = nb + 32 * vb + (lane & 31);
        const bool valid = v < N;
        const uint32_t nr = norms[g * N + std::min<int64_t>(v, N - 1)];
        const float nu = __builtin_bit_cast(_Float16, uint16_t(nr & 0xffffu));
        int e = 0;
        if (nu > 0.f) (void)frexpf(nu, &e);
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const float sc = ldexpf(acc[vb][a], e);      // score / sigma_q
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            const int r = 8 * (a >> 2) + 4 * hs + (a & 3);
            const int reg = r >> 2, row = r & 3;
            // (a superset of the candidates that beat the k-th; row_insert
            // places each exactly and drops the rest)
            uint64_t m = __builtin_amdgcn_ballot_w64(valid && h == hs && sc >= thr_s[reg][row]);
            if (m) {
              while (m) {
                const int b = __builtin_ctzll(m);
                m &= m - 1;
                const float cs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), b));
                const int32_t ci = __builtin_amdgcn_readlane(int32_t(v), b);
                row_insert(ls[reg], li[reg], cs, ci, lane, row, K);
              }
              thr_s[reg][row] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls[reg]), 16 * row + K - 1));
            }
          }
        }
      }
    }
  }
  if (wave < rbs && (lane & 15) < K) {
    const int row = lane >> 4;
#pragma unroll
    for (int reg = 0; reg < 8; ++reg) {
      const int qh = 32 * wave + 4 * reg + row;
      if (qh < Qg) {
        const float sig = sigma[(g * rbs + wave) * 32 + 4 * reg + row];
        const int64_t at = ((g * Qg + qh) * int64_t(gridDim.x) + blockIdx.x) * K + (lane & 15);
        tk_s[at] = ls[reg] * sig;
        tk_i[at] = li[reg];
      }
    }
  }
}

}  // namespace

hipError_t launch_encode_wide(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t N,
                              void* packed, hipStream_t s) {
  const int64_t total = G * N;
  if (total == 0) return hipSuccess;
  uint32_t* planes = static_cast<uint32_t*>(packed);
  uint32_t* norms = planes + total * int64_t(cb.bits) * (kD / 32);
  const int grid = int(std::min<int64_t>((total + kEncKeys - 1) / kEncKeys, int64_t(std::max(1, cb.num_cus))));
#define TQ_ENC(BB, BF)                                                                               \
  hipLaunchKernelGGL((encode1024_kernel<BB, BF>), dim3(grid), dim3(kEncThreads), 0, s, keys, total, N, \
                     planes, norms, cb.d_fragW, cb.d_consts)
  const bool bf = dtype == 1;
  switch (cb.bits - 1) {
    case 1: if (bf) TQ_ENC(1, true); else TQ_ENC(1, false); break;
    case 2: if (bf) TQ_ENC(2, true); else TQ_ENC(2, false); break;
    default: if (bf) TQ_ENC(3, true); else TQ_ENC(3, false); break;
  }
#undef TQ_ENC
  return hipGetLastError();
}

size_t score_wide_prep_bytes(int64_t G, int Qg) {
  return size_t(G) * Qg * (2 * kD + 4) * sizeof(float);
}

int64_t score_wide_ranges(const Codebook& cb, int64_t G, int Qg, int64_t N, int64_t* chunk_out) {
  const int nqc = (Qg + 3) / 4;
  const int64_t units = G * nqc;
  const int64_t cus = std::max(1, cb.num_cus);
  int64_t want = std::max<int64_t>(1, (cus + units - 1) / units);
  want = std::min<int64_t>(want, std::max<int64_t>(1, (N + 1023) / 1024));
  const int64_t chunk = ((N + want - 1) / want + 63) / 64 * 64;
  if (chunk_out) *chunk_out = chunk;
  return (N + chunk - 1) / chunk;
}

// Many queries per group take the matrix-core top-k (one row block of 32
// queries per wave); fewer take the table scorer.
static bool use_mq(int Qg) { return Qg >= 32 && Qg <= 32 * kMqMaxRb; }

static int64_t mq_ranges(const Codebook& cb, int64_t G, int64_t N, int64_t* tiles_per_wg) {
  const int64_t ntiles = (N + 127) / 128;
  const int64_t cus = std::max(1, cb.num_cus);
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(ntiles, (cus + G - 1) / G));
  const int64_t per = (ntiles + want - 1) / want;
  if (tiles_per_wg) *tiles_per_wg = per;
  return (ntiles + per - 1) / per;
}

static size_t mq_frag_bytes(int64_t G, int Qg) {
  const int rbs = (Qg + 31) / 32;
  return size_t(G) * rbs * 4 * 64 * 64 * 16 + size_t(G) * rbs * 32 * 4;
}

size_t topk_wide_bytes(const Codebook& cb, int64_t G, int Qg, int64_t N, int K) {
  if (use_mq(Qg))
    return score_wide_prep_bytes(G, Qg) + mq_frag_bytes(G, Qg) +
           size_t(G) * Qg * mq_ranges(cb, G, N, nullptr) * K * 8;
  const int64_t ranges = score_wide_ranges(cb, G, Qg, N, nullptr);
  return score_wide_prep_bytes(G, Qg) + size_t(G) * Qg * ranges * K * 8;
}

static hipError_t prep_wide(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg, float* X,
                            float* sums, hipStream_t s) {
  const int64_t nq = G * Qg;
  if (qdtype == 1)
    hipLaunchKernelGGL(qprep1024_kernel<true>, dim3(unsigned(nq)), dim3(1024), 0, s, q, nq, X, sums,
                       cb.d_consts, cb.d_St);
  else
    hipLaunchKernelGGL(qprep1024_kernel<false>, dim3(unsigned(nq)), dim3(1024), 0, s, q, nq, X, sums,
                       cb.d_consts, cb.d_St);
  return hipGetLastError();
}

template <bool TOPK>
static hipError_t score_wide(const Codebook& cb, const void* packed, int64_t G, int Qg, int64_t N,
                             const float* X, const float* sums, float* logits, int K, float* tk_s,
                             int32_t* tk_i, hipStream_t s) {
  int64_t chunk = 0;
  const int64_t ranges = score_wide_ranges(cb, G, Qg, N, &chunk);
  const dim3 grid{unsigned(G), unsigned((Qg + 3) / 4), unsigned(ranges)};
  const uint4* planes = static_cast<const uint4*>(packed);
  const uint32_t* norms = static_cast<const uint32_t*>(packed) + G * N * int64_t(cb.bits) * (kD / 32);
#define TQ_SW(BB)                                                                                  \
  hipLaunchKernelGGL((score1024_kernel<BB, TOPK>), grid, dim3(kWideThreads), 0, s, planes, norms, N, Qg, \
                     chunk, X, sums, logits, K, tk_s, tk_i, cb.d_consts)
  switch (cb.bits - 1) {
    case 1: TQ_SW(1); break;
    case 2: TQ_SW(2); break;
    default: TQ_SW(3); break;
  }
#undef TQ_SW
  return hipGetLastError();
}

hipError_t launch_score_wide(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                             const void* packed, int64_t N, float* logits, void* ws, hipStream_t s) {
  float* X = static_cast<float*>(ws);
  float* sums = X + G * Qg * 2 * kD;
  hipError_t e = prep_wide(cb, q, qdtype, G, Qg, X, sums, s);
  if (e != hipSuccess) return e;
  return score_wide<false>(cb, packed, G, Qg, N, X, sums, logits, 0, nullptr, nullptr, s);
}

hipError_t launch_topk_wide(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                            const void* packed, int64_t N, int K, int32_t* idx, float* scores,
                            void* ws, hipStream_t s) {
  float* X = static_cast<float*>(ws);
  float* sums = X + G * Qg * 2 * kD;
  if (use_mq(Qg)) {
    const int rbs = (Qg + 31) / 32;
    char* base = static_cast<char*>(ws) + score_wide_prep_bytes(G, Qg);
    uint4* frag = reinterpret_cast<uint4*>(base);
    float* sigma = reinterpret_cast<float*>(base + size_t(G) * rbs * 4 * 64 * 64 * 16);
    int64_t per = 0;
    const int64_t ranges = mq_ranges(cb, G, N, &per);
    float* tk_s = reinterpret_cast<float*>(base + mq_frag_bytes(G, Qg));
    int32_t* tk_i = reinterpret_cast<int32_t*>(tk_s + G * Qg * ranges * K);
    hipError_t e = prep_wide(cb, q, qdtype, G, Qg, X, sums, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mqprep1024_kernel, dim3(unsigned(G * rbs)), dim3(256), 0, s, X, Qg, rbs, frag,
                       sigma, cb.d_consts);
    const dim3 grid{unsigned(ranges), unsigned(G)};
    const uint32_t* pl = static_cast<const uint32_t*>(packed);
    const uint32_t* nr = pl + G * N * int64_t(cb.bits) * (kD / 32);
#define TQ_MQ(BB)                                                                                \
    hipLaunchKernelGGL((mqtopk1024_kernel<BB>), grid, dim3(kMqThreads), 0, s, pl, nr, N, Qg, rbs, \
                       per, frag, sigma, K, tk_s, tk_i, cb.d_consts)
    switch (cb.bits - 1) {
      case 1: TQ_MQ(1); break;
      case 2: TQ_MQ(2); break;
      default: TQ_MQ(3); break;
    }
#undef TQ_MQ
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(unsigned(G * Qg)), dim3(64), 0, s, tk_s, tk_i,
                       int(ranges), K, idx, scores);
    return hipGetLastError();
  }
  const int64_t ranges = score_wide_ranges(cb, G, Qg, N, nullptr);
  float* tk_s = reinterpret_cast<float*>(static_cast<char*>(ws) + score_wide_prep_bytes(G, Qg));
  int32_t* tk_i = reinterpret_cast<int32_t*>(tk_s + G * Qg * ranges * K);
  hipError_t e = prep_wide(cb, q, qdtype, G, Qg, X, sums, s);
  if (e != hipSuccess) return e;
  e = score_wide<true>(cb, packed, G, Qg, N, X, sums, nullptr, K, tk_s, tk_i, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(unsigned(G * Qg)), dim3(64), 0, s, tk_s, tk_i,
                     int(ranges), K, idx, scores);
  return hipGetLastError();
}


hipError_t launch_decode_wide(const Codebook& cb, const void* packed, int64_t G, int64_t N, void* out,
                              int odtype, hipStream_t s) {
  const int64_t total = G * N;
  const uint32_t* planes = static_cast<const uint32_t*>(packed);
  const uint32_t* norms = planes + total * int64_t(cb.bits) * (kD / 32);
  const int grid = int(std::min<int64_t>((total + 3) / 4, int64_t(std::max(1, cb.num_cus)) * 16));
  const bool bf = odtype == 1;
#define TQ_DW(BB, BF)                                                                             \
  hipLaunchKernelGGL((decode1024_kernel<BB, BF>), dim3(grid), dim3(256), 0, s, planes, norms, total, N, \
                     out, cb.d_consts)
  switch (cb.bits - 1) {
    case 1: if (bf) TQ_DW(1, true); else TQ_DW(1, false); break;
    case 2: if (bf) TQ_DW(2, true); else TQ_DW(2, false); break;
    default: if (bf) TQ_DW(3, true); else TQ_DW(3, false); break;
  }
#undef TQ_DW
  return hipGetLastError();
}

}  // namespace tq

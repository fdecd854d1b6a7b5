// HIP kernels (gfx950 / MI355X) of the TurboQuant key path, d = 128.
//
//  encode:  rotation y = H D k / (||k|| sqrt(d)) on the matrix cores (bf16
//           keys) or as a register-resident Hadamard butterfly (float32
//           keys), Lloyd-Max codes by threshold comparison,
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
#include <type_traits>

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

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// x = hi + lo for two values: hi = RTZ_f16(x) packed by one convert, and
// lo = RN_f16(x - hi) (x - hi is exact in float32).  Builtins only: the
// registers feed the matrix cores, and the compiler's hazard checks do not
// see through inline assembly.
// mone must hold -1.0f in a register the compiler cannot see through: then
// x - hi is one mixed-precision fma per value (v_fma_mix_f32 reads the half
// straight from the packed register) instead of a convert and a subtract.
__device__ __forceinline__ void split_f16_pair(float x0, float x1, float mone, uint32_t& hi,
                                               uint32_t& lo) {
  const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  const half2v l = {static_cast<_Float16>(__builtin_fmaf(static_cast<float>(h[0]), mone, x0)),
                    static_cast<_Float16>(__builtin_fmaf(static_cast<float>(h[1]), mone, x1))};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
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
// Two kernels: bf16 keys and values run 16 keys per wave-tile on the matrix
// cores (encode128_bf16_t16_kernel, below); float32 keys and values use the
// two-lane layout described here.
//
// Two-lane layout: a wave encodes 32 keys at a time, two lanes per key.  Lane
// L = 32h + kl holds coordinates [64h, 64h + 64) of key kl in x[0..63].
// Six butterfly stages run inside the register file; the stage across the
// two halves uses v_permlane32_swap on register pairs (r, r + 32), which
// leaves register r of half h holding coordinate
//   (r % 32) + 32 * (h + 2 * (r / 32)),
// i.e. bit-plane word h in x[0..31] and word 2 + h in x[32..63], bit r % 32.
// The residual registers feed the matrix-core B operand directly (K order
// = register order); the host lays S R^T out in the matching A order.

struct EncConsts {
  float tpos[3], cpos[4], sqrt_d;
};

__device__ __forceinline__ void load_enc_consts(const DevConsts* __restrict__ cst, EncConsts& c) {
#pragma unroll
  for (int k = 0; k < 3; ++k) c.tpos[k] = cst->tpos[k];
#pragma unroll
  for (int k = 0; k < 4; ++k) c.cpos[k] = cst->cpos_s[k];
  c.sqrt_d = cst->sqrt_d;
}

// Butterfly stages of strides first_stride..32 inside the lane, then the
// stride-64 stage across the wave halves.
__device__ __forceinline__ void butterfly_rest(float (&x)[64], int first_stride) {
#pragma unroll
  for (int st = 1; st < 64; st <<= 1) {
    if (st < first_stride) continue;
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      if (r & st) continue;
      const float a = x[r], b = x[r + st];
      x[r] = a + b;
      x[r + st] = a - b;
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
}

// Everything after the rotation for the 32 keys of one wave tile: codes and
// code planes, residual and its norm, the matrix-core QJL projection, sign
// words, stores.  x holds u = H D k (unnormalised); nu2 is this lane's half
// of ||k||^2.  Rotated values must carry no -0 (an exact zero counts as
// non-negative).
// Results of one lane for one tile: words (2h, 2h+1) of every plane of key
// (g, n) and, for h = 0, the packed half norms.
struct TileOut {
  uint2 w[4];        // planes 0..B (code planes, then the sign plane at index B)
  uint32_t norm;
  int64_t g, n;
  bool valid;
};

template <int B>
__device__ __forceinline__ void store_tile(const TileOut& o, int lane, int64_t Ncap,
                                           uint32_t* __restrict__ planes,
                                           uint32_t* __restrict__ norms) {
  constexpr int P = B + 1;
  if (!o.valid) return;
  const int h = lane >> 5;
  uint32_t* pl = planes + (o.g * P) * Ncap * 4;
#pragma unroll
  for (int p = 0; p < P; ++p) *reinterpret_cast<uint2*>(pl + (p * Ncap + o.n) * 4 + 2 * h) = o.w[p];
  if (h == 0) norms[o.g * Ncap + o.n] = o.norm;
}

template <int B>
__device__ __forceinline__ void encode_tail(const float (&x)[64], float nu2, const EncConsts& ec,
                                            const uint4* __restrict__ s_frag, int lane, int64_t g,
                                            int64_t n, bool valid, TileOut& out) {
  constexpr int K = 1 << (B - 1);      // levels on the positive half
  constexpr int P = B + 1;             // planes per key
  const int h = lane >> 5;
  nu2 = xor32_sum(nu2);
  // hardware square root and reciprocal (1 ulp): the norms are stored as
  // half, and a relative error of 1e-7 in the residual scale moves no sign
  // or code outside the band where the two roundings may differ anyway
  const float nu = __builtin_amdgcn_sqrtf(nu2);
  const bool zero = !(nu >= 1e-10f);
  const float nsd = nu * ec.sqrt_d;                       // u = y * nu * sqrt(d)
  const float gsc = zero ? 0.f : kResidualScale * __builtin_amdgcn_rcpf(nsd);   // u -> 2^12 y
  float tu[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) tu[k] = ec.tpos[k] * nsd;

  // ---- Lloyd-Max codes (sign bit + magnitude thresholds), residual, hi/lo
  //      split, and the QJL projection p = (S R^T) r_rot on the matrix cores,
  //      interleaved: as soon as the 16 coordinates of chunk kc are split into
  //      fp16 hi/lo, its 8 MFMAs (4 row blocks x (S R^T) r_hi + (S R^T) r_lo;
  //      S R^T is exact in float16, fp32 accumulation) are issued, so the
  //      matrix core runs while the vector ALU quantises the next chunk.
  // The fragment table never changes inside the tile loop; an opaque lane
  // offset keeps the compiler from hoisting its 64 reads out of the loop.
  int fl_off = lane;
  asm volatile("" : "+v"(fl_off));
  const half8* fh = reinterpret_cast<const half8*>(s_frag) + fl_off;
  uint32_t wu[2] = {0u, 0u};
  uint32_t wd[K > 1 ? K - 1 : 1][2];
#pragma unroll
  for (int k = 0; k < (K > 1 ? K - 1 : 1); ++k) wd[k][0] = wd[k][1] = 0u;
  f32x16 acc[4] = {};
  float rho2 = 0.f;
  float mone = -1.0f;
  asm volatile("" : "+v"(mone));
  // codes, residual and fp16 hi/lo split of the 8 registers of chunk kc
  auto quant_chunk = [&](int kc, uint32_t (&bh)[4], uint32_t (&bl)[4]) {
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      float ep[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int rr = 8 * kc + 2 * pr + t, ws = rr >> 5;
        const float u = x[rr];
        const float a = fabsf(u);
        wu[ws] = push_sign(wu[ws], u);
        float mag = ec.cpos[0];
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
          // one compare feeds both the bit push (shift-add with the compare
          // as carry-in) and the level select
          // the lane mask of one compare is the carry-in of a doubling add
          // (pushes the bit) and the select of the level
          const uint64_t below = __builtin_amdgcn_ballot_w64(a < tu[k]);
          uint64_t co;
          const float up = ec.cpos[k + 1];
          asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3"
              : "=v"(wd[k][ws]), "=s"(co) : "v"(wd[k][ws]), "s"(below));
          asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(mag) : "v"(up), "v"(mag), "s"(below));
        }
        const float yh = copysignf(mag, u);
        // the negated residual yh - u g = 2^12 (c[code] - y): one fma with a
        // negated source; the fragment table holds -S R^T, so the products
        // below still come out as +S r
        ep[t] = fmaf(-u, gsc, yh);
        rho2 = fmaf(ep[t], ep[t], rho2);
      }
      split_f16_pair(ep[0], ep[1], mone, bh[pr], bl[pr]);
    }
  };
  // an empty use of the code words (no instruction): their bits are
  // accumulated chunk by chunk instead of being recombined after all the
  // products, which would keep every comparison result live meanwhile
  auto pin_words = [&]() {
    if constexpr (K > 2) {
      asm volatile("" : "+v"(wu[0]), "+v"(wu[1]), "+v"(wd[0][0]), "+v"(wd[0][1]), "+v"(wd[1][0]),
                   "+v"(wd[1][1]), "+v"(wd[2][0]), "+v"(wd[2][1]));
    } else {
      asm volatile("" : "+v"(wu[0]), "+v"(wu[1]), "+v"(wd[0][0]), "+v"(wd[0][1]));
    }
  };
  // Software pipeline over the 8 chunks: the 8 matrix products of chunk kc
  // share one scheduling region with the vector work of chunk kc + 1 and are
  // interleaved with it (one product per twelve vector instructions), so the
  // matrix core runs while this wave quantises instead of stalling its issue.
  uint32_t bh[2][4], bl[2][4];
  half8 ahi[2][4];
  // fragments of chunk kc are read one region ahead, behind a per-chunk
  // opaque offset (no instruction) that keeps them from being hoisted out of
  // the tile loop
  auto read_frag = [&](int kc, half8 (&fhv)[4]) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) fhv[jb] = fh[kc * 4 * 64 + jb * 64];
  };
  read_frag(0, ahi[0]);
  quant_chunk(0, bh[0], bl[0]);
  pin_words();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    const int cur = kc & 1;
    if (kc < 7) {
      read_frag(kc + 1, ahi[cur ^ 1]);
      quant_chunk(kc + 1, bh[cur ^ 1], bl[cur ^ 1]);
    }
    const half8 bhi = __builtin_bit_cast(half8, u32x4{bh[cur][0], bh[cur][1], bh[cur][2], bh[cur][3]});
    const half8 blo = __builtin_bit_cast(half8, u32x4{bl[cur][0], bl[cur][1], bl[cur][2], bl[cur][3]});
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[cur][jb], bhi, acc[jb], 0, 0, 0);
      acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[cur][jb], blo, acc[jb], 0, 0, 0);
    }
    if (kc < 7) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // next chunk's fragment reads first
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // twelve VALU
      }
    }
    pin_words();
    __builtin_amdgcn_sched_barrier(0);
  }
  rho2 = xor32_sum(rho2);
  const float rho = zero ? 0.f : __builtin_amdgcn_sqrtf(rho2) * (nu * (1.0f / kResidualScale));

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
#pragma unroll
  for (int p = 0; p < P - 1; ++p) {
    // (word h, word 2+h) of each lane -> (words 2h, 2h+1): swap across halves
    auto pr = __builtin_amdgcn_permlane32_swap(pw[p][0], pw[p][1], false, false);
    out.w[p] = make_uint2(keep ? uint32_t(pr[0]) : 0u, keep ? uint32_t(pr[1]) : 0u);
  }

  // ---- sign words: lane (kl, h) holds rows j = 32 jb + 8 (v / 4) + 4 h + (v % 4) of key kl
  uint32_t sw[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    uint32_t b16 = 0u;
#pragma unroll
    for (int v = 15; v >= 0; --v) b16 = push_sign(b16, acc[jb][v]);
    uint32_t t = (b16 | (b16 << 8)) & 0x00FF00FFu;
    t = (t | (t << 4)) & 0x0F0F0F0Fu;
    sw[jb] = xor32_or(t << (4 * h));
  }

  const bool keep_s = keep && rho2 > 0.f;
  out.w[P - 1] = make_uint2(keep_s ? (h ? sw[2] : sw[0]) : 0u, keep_s ? (h ? sw[3] : sw[1]) : 0u);
  out.norm = keep ? (uint32_t(f2h_bits(nu)) | (uint32_t(f2h_bits(rho)) << 16)) : 0u;
  out.g = g;
  out.n = n;
  out.valid = valid;
}

// ---- values: MSE-only records (b-bit level index, one half norm).
// Same lane layout and rotation as the keys; each positive threshold is one
// compare whose lane mask is the carry-in of a doubling add (the bit push),
// the sign bit is pushed with v_alignbit, and the level index bits follow
// from the thermometer bits: with d_k = [|y| >= t_k], bit j of the magnitude
// index is the XOR of d_k over k with (k + 1) divisible by 2^j, and the
// stored bit j is that XOR the sign (negative levels mirror the positive
// ones); the top bit is the complement of the sign.
struct ValOut {
  uint2 w[4];        // words (2h, 2h+1) of planes 0..BV-1
  uint32_t norm;     // half(nu) in the low 16 bits
  int64_t g, n;
  bool valid;
};

template <int BV>
__device__ __forceinline__ void store_vtile(const ValOut& o, int lane, int64_t Ncap,
                                            uint32_t* __restrict__ planes,
                                            uint16_t* __restrict__ norms) {
  if (!o.valid) return;
  const int h = lane >> 5;
  uint32_t* pl = planes + (o.g * BV) * Ncap * 4;
#pragma unroll
  for (int p = 0; p < BV; ++p) *reinterpret_cast<uint2*>(pl + (p * Ncap + o.n) * 4 + 2 * h) = o.w[p];
  if (h == 0) norms[o.g * Ncap + o.n] = uint16_t(o.norm);
}

template <int BV>
__device__ __forceinline__ void value_tail(const float (&x)[64], float nu2,
                                           const DevConsts* __restrict__ cst, int lane, int64_t g,
                                           int64_t n, bool valid, ValOut& out) {
  constexpr int KV = 1 << (BV - 1);    // levels on the positive half
  nu2 = xor32_sum(nu2);
  const float nu = __builtin_amdgcn_sqrtf(nu2);
  const bool zero = !(nu >= 1e-10f);
  const float nsd = nu * cst->sqrt_d;
  float tu[KV > 1 ? KV - 1 : 1];
#pragma unroll
  for (int k = 0; k < KV - 1; ++k) tu[k] = cst->vtpos[k] * nsd;
  uint32_t wu[2] = {0u, 0u};
  uint32_t wd[KV > 1 ? KV - 1 : 1][2];
#pragma unroll
  for (int k = 0; k < (KV > 1 ? KV - 1 : 1); ++k) wd[k][0] = wd[k][1] = 0u;
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    const int ws = r >> 5;
    const float u = x[r];
    const float a = fabsf(u);
    wu[ws] = push_sign(wu[ws], u);
#pragma unroll
    for (int k = 0; k < KV - 1; ++k) {
      const uint64_t below = __builtin_amdgcn_ballot_w64(a < tu[k]);
      uint64_t co;
      asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3"
          : "=v"(wd[k][ws]), "=s"(co) : "v"(wd[k][ws]), "s"(below));
    }
  }
  const bool keep = valid && !zero;
  uint32_t pw[BV][2];
#pragma unroll
  for (int ws = 0; ws < 2; ++ws) {
    // words were filled oldest-bit-first: bit (r % 32) sits at 31 - r % 32
    const uint32_t sg = __builtin_bitreverse32(wu[ws]);       // 1 = negative
    pw[BV - 1][ws] = ~sg;
#pragma unroll
    for (int j = 0; j < BV - 1; ++j) {
      uint32_t e = 0u;   // XOR of the "below" bits (complements of d_k); odd count
#pragma unroll
      for (int k = 0; k < KV - 1; ++k)
        if (((k + 1) & ((1 << j) - 1)) == 0) e ^= __builtin_bitreverse32(wd[k][ws]);
      pw[j][ws] = ~(e ^ sg);
    }
  }
#pragma unroll
  for (int p = 0; p < BV; ++p) {
    // (word h, word 2+h) of each lane -> (words 2h, 2h+1): swap across halves
    auto pr = __builtin_amdgcn_permlane32_swap(pw[p][0], pw[p][1], false, false);
    out.w[p] = make_uint2(keep ? uint32_t(pr[0]) : 0u, keep ? uint32_t(pr[1]) : 0u);
  }
  out.norm = keep ? uint32_t(f2h_bits(nu)) : 0u;
  out.g = g;
  out.n = n;
  out.valid = valid;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

// ---- bf16 keys, 16 keys per wave-tile (16 x 16 x 32 matrix products).
// Lane L = 16 w + n serves key n of the tile and owns the coordinates
// [32 w, 32 w + 32): the bits it produces are word w of every bit plane, so
// codes and sign words leave the lane in natural order with no cross-lane
// packing, and each lane holds 32 rotated values instead of 64 (registers
// for three waves per SIMD).
//
// Rotation.  Split coordinates as c = 32 c_hi + c_lo; the Sylvester matrix
// factors as H_128[r][c] = H_4[r_hi][c_hi] H_32[r_lo][c_lo].  Product step t
// feeds the lane's input coordinates 32 w + 8 t + j (K index 8 w + j), and
// output row m of block b is coordinate 32 (m / 4) + 4 b + m % 4.  The A
// operand of (b, t) is then sigma(b / 2, t) P_{b % 2}: two per-lane +-1
// patterns (the H_4 factor of the lane's (m / 4, w) and the low H_32 bits)
// times the wave-uniform sign sigma(s, t) = (-1)^popcount(s & t).  For each
// pattern the four blocks b = p + 2 s are the 4-point Hadamard over t of the
// products P_p B_t, accumulated as a tree with shared prefixes: 11 products
// per pattern, 22 per 16 keys.
constexpr int kEnc16Threads = 256;
constexpr int kEnc16Waves = kEnc16Threads / 64;

// A-operand patterns of this lane (row m = lane % 16, K group lane / 16):
// p[0] = P_0, p[1] = P_1, p[2] = -P_0, p[3] = -P_1 (bf16 +-1).
__device__ __forceinline__ void hadamard_frags16(int lane, u32x4 (&p)[4]) {
  const int m = lane & 15, kg = lane >> 4;
  const int base = __builtin_popcount((m >> 2) & kg) & 1;
  uint32_t w0[4], w1[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t v0 = 0, v1 = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * r + u;
      const int s0 = base ^ (__builtin_popcount((m & 3) & (j & 3)) & 1);
      const int s1 = s0 ^ (j >> 2);
      v0 |= (s0 ? 0xBF80u : 0x3F80u) << (16 * u);
      v1 |= (s1 ? 0xBF80u : 0x3F80u) << (16 * u);
    }
    w0[r] = v0;
    w1[r] = v1;
  }
  p[0] = u32x4{w0[0], w0[1], w0[2], w0[3]};
  p[1] = u32x4{w1[0], w1[1], w1[2], w1[3]};
  p[2] = p[0] ^ 0x80008000u;
  p[3] = p[1] ^ 0x80008000u;
}

// Rows hold din <= 128 elements (din a multiple of 16): a lane whose eight
// coordinates 32 w + 8 t + j lie at or past din reads the row start instead
// (valid memory) and the consumer replaces the data by zeros.
__device__ __forceinline__ void issue_tile_dma16(const uint16_t* __restrict__ keys, uint32_t tile,
                                                 uint32_t tpg, int64_t N, uint32_t din, int lane,
                                                 uint4* buf) {
  const int w = lane >> 4, kl = lane & 15;
  const uint32_t gt = tile / tpg;
  const int64_t g = gt;
  const int64_t n = int64_t(tile - gt * tpg) * 16 + kl;
  const int64_t nl = n < N ? n : N - 1;
  const uint4* src = reinterpret_cast<const uint4*>(keys + (g * N + nl) * din) + 4 * w;
  if (din == 128) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + t), (lds_void*)(buf + t * 64),
                                       16, 0, 0);
  } else {
    const uint4* row = src - 4 * w;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(uint32_t(32 * w + 8 * t) < din ? src + t : row),
          (lds_void*)(buf + t * 64), 16, 0, 0);
  }
}

struct TileOut16 {
  uint32_t w[4];     // word (lane / 16) of planes 0..B (code planes, then the sign plane)
  uint32_t norm;
  int64_t g, n;
  bool valid;
};

template <int B>
__device__ __forceinline__ void store_tile16(const TileOut16& o, int lane, int64_t Ncap,
                                             uint32_t* __restrict__ planes,
                                             uint32_t* __restrict__ norms) {
  constexpr int P = B + 1;
  if (!o.valid) return;
  const int w = lane >> 4;
  uint32_t* pl = planes + (o.g * P) * Ncap * 4;
#pragma unroll
  for (int p = 0; p < P; ++p) pl[(p * Ncap + o.n) * 4 + w] = o.w[p];
  if (w == 0) norms[o.g * Ncap + o.n] = o.norm;
}

// sum over the four lanes of a key (lanes n, n + 16, n + 32, n + 48)
__device__ __forceinline__ float key16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));   // lane ^ 16
  return xor32_sum(v);
}

// A tile between its products and its packing: the sketch accumulators are
// read one iteration later, after the next tile's rotation products are
// issued, so no wave waits for its own matrix products to drain.
struct Pending16 {
  f32x4 acc[8];
  uint32_t wu, wd[3];
  float rho2, nu;
  bool zero, valid;
  int64_t g, n;
};

template <int B>
__device__ __forceinline__ void quant_sketch16(const f32x4 (&y)[8], float nu2, const EncConsts& ec,
                                               const uint4* __restrict__ s_frag, int lane,
                                               int64_t g, int64_t n, bool valid, Pending16& pd) {
  constexpr int K = 1 << (B - 1);      // levels on the positive half
  nu2 = key16_sum(nu2);
  // hardware square root and reciprocal, as in the float32-key encoder
  const float nu = __builtin_amdgcn_sqrtf(nu2);
  const bool zero = !(nu >= 1e-10f);
  const float nsd = nu * ec.sqrt_d;                       // u = y * nu * sqrt(d)
  const float gsc = zero ? 0.f : kResidualScale * __builtin_amdgcn_rcpf(nsd);   // u -> 2^12 y
  float tu[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) tu[k] = ec.tpos[k] * nsd;

  // fragment reads go through a per-tile opaque lane offset (no instruction)
  // so the compiler cannot hoist the loop-invariant table out of the tile loop
  int fl_off = lane;
  asm volatile("" : "+v"(fl_off));
  const half8* fh = reinterpret_cast<const half8*>(s_frag) + fl_off;
  uint32_t wu = 0u;
  uint32_t wd[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int k = 0; k < (K > 1 ? K - 1 : 1); ++k) wd[k] = 0u;
  f32x4 acc[8] = {};
  float rho2 = 0.f;
  float mone = -1.0f;
  asm volatile("" : "+v"(mone));
  // chunk c = rotation blocks 2c, 2c + 1: codes, residual and fp16 hi/lo
  // split of the lane's coordinates 32 w + 8 c + j, j = 0..7 (register pair
  // r holds j = 2r, 2r + 1)
  auto quant_chunk = [&](int c, uint32_t (&bh)[4], uint32_t (&bl)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float ep[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = 2 * r + t;
        const float u = y[2 * c + (j >> 2)][j & 3];
        const float a = fabsf(u);
        wu = push_sign(wu, u);
        float mag = ec.cpos[0];
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
          // the lane mask of one compare is the carry-in of a doubling add
          // (pushes the bit) and the select of the level
          const uint64_t below = __builtin_amdgcn_ballot_w64(a < tu[k]);
          uint64_t co;
          const float up = ec.cpos[k + 1];
          asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(wd[k]), "=s"(co) : "v"(wd[k]), "s"(below));
          asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(mag) : "v"(up), "v"(mag), "s"(below));
        }
        const float yh = copysignf(mag, u);
        // negated residual 2^12 (c[code] - y); the table holds -S R^T
        ep[t] = fmaf(-u, gsc, yh);
        rho2 = fmaf(ep[t], ep[t], rho2);
      }
      split_f16_pair(ep[0], ep[1], mone, bh[r], bl[r]);
    }
  };
  auto pin_words = [&]() {
    if constexpr (K > 2) {
      asm volatile("" : "+v"(wu), "+v"(wd[0]), "+v"(wd[1]), "+v"(wd[2]));
    } else {
      asm volatile("" : "+v"(wu), "+v"(wd[0]));
    }
  };
  // Software pipeline over the 4 chunks: the 16 products of chunk c share a
  // scheduling region with the vector work of chunk c + 1, one product per
  // five vector instructions; the fragment of row block b for chunk c + 1 is
  // read right after the two products of chunk c that use its register.
  uint32_t bh[2][4], bl[2][4];
  half8 f[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) f[b] = fh[b * 64];
  quant_chunk(0, bh[0], bl[0]);
  pin_words();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int cur = c & 1;
    if (c < 3) quant_chunk(c + 1, bh[cur ^ 1], bl[cur ^ 1]);
    const half8 bhi = __builtin_bit_cast(half8, u32x4{bh[cur][0], bh[cur][1], bh[cur][2], bh[cur][3]});
    const half8 blo = __builtin_bit_cast(half8, u32x4{bl[cur][0], bl[cur][1], bl[cur][2], bl[cur][3]});
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[b], bhi, acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[b], blo, acc[b], 0, 0, 0);
      if (c < 3) f[b] = fh[((c + 1) * 8 + b) * 64];
    }
    if (c < 3) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // five VALU
        if (i & 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one fragment read
      }
    }
    pin_words();
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) pd.acc[b] = acc[b];
  pd.wu = wu;
#pragma unroll
  for (int k = 0; k < (K > 1 ? K - 1 : 1); ++k) pd.wd[k] = wd[k];
  pd.rho2 = rho2;
  pd.nu = nu;
  pd.zero = zero;
  pd.valid = valid;
  pd.g = g;
  pd.n = n;
}

template <int B>
__device__ __forceinline__ void finish16(const Pending16& pd, TileOut16& out) {
  constexpr int P = B + 1;
  const float rho2 = key16_sum(pd.rho2);
  const float nu = pd.nu;
  const bool zero = pd.zero, valid = pd.valid;
  const uint32_t wu = pd.wu;
  const uint32_t* wd = pd.wd;
  const f32x4* acc = pd.acc;
  const float rho = zero ? 0.f : __builtin_amdgcn_sqrtf(rho2) * (nu * (1.0f / kResidualScale));

  // words were filled oldest-bit-first: bit r sits at 31 - r
  const bool keep = valid && !zero;
  const uint32_t u_ = __builtin_bitreverse32(wu);
  uint32_t pw[P - 1];
  if constexpr (B == 1) {
    pw[0] = ~u_;
  } else if constexpr (B == 2) {
    pw[1] = ~u_;
    pw[0] = ~(u_ ^ __builtin_bitreverse32(wd[0]));
  } else {
    const uint32_t d0 = __builtin_bitreverse32(wd[0]);
    const uint32_t d1 = __builtin_bitreverse32(wd[1]);
    const uint32_t d2 = __builtin_bitreverse32(wd[2]);
    pw[2] = ~u_;
    pw[1] = ~(u_ ^ d1);
    pw[0] = ~(u_ ^ d0 ^ d1 ^ d2);
  }
#pragma unroll
  for (int p = 0; p < P - 1; ++p) out.w[p] = keep ? pw[p] : 0u;

  // sign word: value i of block b is sketch row 32 w + 4 b + i; pushed from
  // the top row down, row r lands at bit r
  uint32_t sw = 0u;
#pragma unroll
  for (int b = 7; b >= 0; --b)
#pragma unroll
    for (int i = 3; i >= 0; --i) sw = push_sign(sw, acc[b][i]);
  const bool keep_s = keep && rho2 > 0.f;
  out.w[P - 1] = keep_s ? sw : 0u;
  out.norm = keep ? (uint32_t(f2h_bits(nu)) | (uint32_t(f2h_bits(rho)) << 16)) : 0u;
  out.g = pd.g;
  out.n = pd.n;
  out.valid = valid;
}

// Value records in the 16-key layout: each lane's 32 rotated coordinates
// give word w of the b level-index planes (same bit rules as value_tail).
template <int BV>
__device__ __forceinline__ void store_vtile16(const TileOut16& o, int lane, int64_t Ncap,
                                              uint32_t* __restrict__ planes,
                                              uint16_t* __restrict__ norms) {
  if (!o.valid) return;
  const int w = lane >> 4;
  uint32_t* pl = planes + (o.g * BV) * Ncap * 4;
#pragma unroll
  for (int p = 0; p < BV; ++p) pl[(p * Ncap + o.n) * 4 + w] = o.w[p];
  if (w == 0) norms[o.g * Ncap + o.n] = uint16_t(o.norm);
}

template <int BV>
__device__ __forceinline__ void value_tail16(const f32x4 (&y)[8], float nu2,
                                             const DevConsts* __restrict__ cst, int64_t g,
                                             int64_t n, bool valid, TileOut16& out) {
  constexpr int KV = 1 << (BV - 1);    // levels on the positive half
  nu2 = key16_sum(nu2);
  const float nu = __builtin_amdgcn_sqrtf(nu2);
  const bool zero = !(nu >= 1e-10f);
  const float nsd = nu * cst->sqrt_d;
  float tu[KV > 1 ? KV - 1 : 1];
#pragma unroll
  for (int k = 0; k < KV - 1; ++k) tu[k] = cst->vtpos[k] * nsd;
  uint32_t wu = 0u;
  uint32_t wd[KV > 1 ? KV - 1 : 1];
#pragma unroll
  for (int k = 0; k < (KV > 1 ? KV - 1 : 1); ++k) wd[k] = 0u;
#pragma unroll
  for (int r = 0; r < 32; ++r) {   // coordinate 32 w + r is value r % 4 of block r / 4
    const float u = y[r >> 2][r & 3];
    const float a = fabsf(u);
    wu = push_sign(wu, u);
#pragma unroll
    for (int k = 0; k < KV - 1; ++k) {
      const uint64_t below = __builtin_amdgcn_ballot_w64(a < tu[k]);
      uint64_t co;
      asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(wd[k]), "=s"(co) : "v"(wd[k]), "s"(below));
    }
  }
  const bool keep = valid && !zero;
  // words were filled oldest-bit-first: bit r sits at 31 - r
  const uint32_t sg = __builtin_bitreverse32(wu);       // 1 = negative
  out.w[BV - 1] = keep ? ~sg : 0u;
#pragma unroll
  for (int j = 0; j < BV - 1; ++j) {
    uint32_t e = 0u;   // XOR of the "below" bits (complements of d_k); odd count
#pragma unroll
    for (int k = 0; k < KV - 1; ++k)
      if (((k + 1) & ((1 << j) - 1)) == 0) e ^= __builtin_bitreverse32(wd[k]);
    out.w[j] = keep ? ~(e ^ sg) : 0u;
  }
  out.norm = keep ? uint32_t(f2h_bits(nu)) : 0u;
  out.g = g;
  out.n = n;
  out.valid = valid;
}

// VAL: value records (B = value bits, no sketch; norms are uint16 halves).
template <int B, bool VAL>
__global__ __launch_bounds__(kEnc16Threads, VAL ? 4 : 3) void encode128_bf16_t16_kernel(
    const uint16_t* __restrict__ keys, int64_t G, int64_t N, int64_t Ncap, int64_t pos,
    uint32_t* __restrict__ planes, void* __restrict__ norms_,
    const DevConsts* __restrict__ cst, const uint4* __restrict__ frag,
    const uint4* __restrict__ dmask) {
  __shared__ uint4 s_frag[VAL ? 1 : 2048];           // 32 KB: [t 4][b 8][lane 64]
  __shared__ uint4 s_raw[kEnc16Waves][4 * 64];       // 16 KB: per-wave key tile
  __shared__ uint4 s_dm[16];                         // D as bf16 sign bits, [word][k-step]

  const int tid = threadIdx.x, lane = tid & 63, w = lane >> 4, kl = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t tpg = uint32_t((N + 15) / 16);
  const uint64_t ntiles = uint64_t(G) * tpg;   // < 2^32 (the host bounds G x N)
  const uint64_t stride = uint64_t(gridDim.x) * kEnc16Waves;
  uint64_t tile = uint64_t(blockIdx.x) * kEnc16Waves + wave;
  uint4* buf = s_raw[wave];
  const uint32_t din = cst->din;
  if (tile < ntiles) issue_tile_dma16(keys, uint32_t(tile), tpg, N, din, lane, buf);
  if constexpr (!VAL)
    for (int i = tid; i < 2048; i += kEnc16Threads) s_frag[i] = frag[i];
  if (tid < 16) s_dm[tid] = dmask[tid];
  EncConsts ec;
  load_enc_consts(cst, ec);
  u32x4 hp[4];
  hadamard_frags16(lane, hp);
  __syncthreads();

  // Each iteration: wait for this tile's keys (the DMA issued one iteration
  // earlier and the stores of two tiles back are the only vector memory
  // operations in flight), copy them to registers, start the next tile's DMA,
  // issue this tile's rotation products, pack and store the previous tile,
  // then quantise this tile and issue its sketch products.
  Pending16 pend;
  TileOut16 out;
  bool have = false;   // pend holds the previous tile (wave-uniform)
  for (; tile < ntiles; tile += stride) {
    const uint32_t t32 = uint32_t(tile);
    const uint32_t gt = t32 / tpg;
    const int64_t g = gt;
    const int64_t n = int64_t(t32 - gt * tpg) * 16 + kl;
    const bool valid = n < N;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    u32x4 raw[4], dmv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 v = buf[t * 64 + lane];
      raw[t] = u32x4{v.x, v.y, v.z, v.w};
      const uint4 dm = s_dm[w * 4 + t];
      dmv[t] = u32x4{dm.x, dm.y, dm.z, dm.w};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // buffer free again
    if (din < 128) {   // zero padding past din
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (uint32_t(32 * w + 8 * t) >= din) raw[t] = u32x4{0u, 0u, 0u, 0u};
    }
    if (tile + stride < ntiles) issue_tile_dma16(keys, uint32_t(tile + stride), tpg, N, din, lane, buf);

    float nu2 = 0.f;
    bf16x8 kv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bf16x2 q = __builtin_bit_cast(bf16x2, uint32_t(raw[t][r]));
        nu2 = __builtin_amdgcn_fdot2_f32_bf16(q, q, nu2, false);
      }
      kv[t] = __builtin_bit_cast(bf16x8, raw[t] ^ dmv[t]);
    }
    // y[p + 2 s] = sum_t (-1)^popcount(s & t) P_p B_t, as a prefix tree
    f32x4 y[8];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bf16x8 pp = __builtin_bit_cast(bf16x8, hp[p]), pn = __builtin_bit_cast(bf16x8, hp[p + 2]);
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, kv[0], z, 0, 0, 0);
      const f32x4 ap = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, kv[1], a, 0, 0, 0);
      const f32x4 am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pn, kv[1], a, 0, 0, 0);
      const f32x4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, kv[2], ap, 0, 0, 0);
      const f32x4 c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pn, kv[2], ap, 0, 0, 0);
      const f32x4 c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, kv[2], am, 0, 0, 0);
      const f32x4 c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pn, kv[2], am, 0, 0, 0);
      y[p + 0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, kv[3], c0, 0, 0, 0);
      y[p + 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pn, kv[3], c1, 0, 0, 0);
      y[p + 4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pn, kv[3], c2, 0, 0, 0);
      y[p + 6] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, kv[3], c3, 0, 0, 0);
    }
    uint32_t* nk = static_cast<uint32_t*>(norms_);
    uint16_t* nv = static_cast<uint16_t*>(norms_);
    if constexpr (VAL) {
      if (have) store_vtile16<B>(out, lane, Ncap, planes, nv);
      value_tail16<B>(y, nu2, cst, g, pos + n, valid, out);
      have = true;
    } else {
      if (have) {   // the previous tile's packing runs while this tile's rotation products do
        finish16<B>(pend, out);
        store_tile16<B>(out, lane, Ncap, planes, nk);
      }
      // a wave in its vector-heavy stretch issues ahead of waves running
      // rotation products (measured 1-2% faster than equal priorities)
      __builtin_amdgcn_s_setprio(1);
      quant_sketch16<B>(y, nu2, ec, s_frag, lane, g, pos + n, valid, pend);
      __builtin_amdgcn_s_setprio(0);
      have = true;
    }
  }
  if (have) {
    if constexpr (VAL) {
      store_vtile16<B>(out, lane, Ncap, planes, static_cast<uint16_t*>(norms_));
    } else {
      finish16<B>(pend, out);
      store_tile16<B>(out, lane, Ncap, planes, static_cast<uint32_t*>(norms_));
    }
  }
}

// ---- float32 keys (register loads, four waves per workgroup).
constexpr int kEncThreads = 256;
constexpr int kEncWaves = kEncThreads / 64;

template <int B, bool VAL>
__global__ __launch_bounds__(kEncThreads, 2) void encode128_f32_kernel(
    const float* __restrict__ keys, int64_t G, int64_t N, int64_t Ncap, int64_t pos,
    uint32_t* __restrict__ planes,
    void* __restrict__ norms_, const DevConsts* __restrict__ cst,
    const uint4* __restrict__ frag, const uint32_t* __restrict__ flip) {
  __shared__ uint4 s_frag[VAL ? 1 : 2048];       // [kc 8][jb 4][lane 64]
  __shared__ uint32_t s_flip[128];

  const int tid = threadIdx.x;
  if constexpr (!VAL)
    for (int i = tid; i < 2048; i += kEncThreads) s_frag[i] = frag[i];
  for (int i = tid; i < 128; i += kEncThreads) s_flip[i] = flip[i];
  EncConsts ec;
  load_enc_consts(cst, ec);
  __syncthreads();

  const int lane = tid & 63, h = lane >> 5, kl = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t tpg = uint32_t((N + 31) / 32);
  const uint32_t ntiles = uint32_t(G) * tpg;
  const uint32_t din = cst->din;   // row length (128, or less when zero-padded)
  for (uint32_t tile = blockIdx.x * kEncWaves + wave; tile < ntiles; tile += gridDim.x * kEncWaves) {
    const uint32_t gt = tile / tpg;
    const int64_t g = gt;
    const int64_t n = int64_t(tile - gt * tpg) * 32 + kl;
    const bool valid = n < N;
    // lanes past the end of a ragged group load the group's last key; their
    // results are never stored and each key has its own matrix column
    const int64_t nl = valid ? n : N - 1;
    const float* row = keys + (g * N + nl) * din;
    const uint4* src = reinterpret_cast<const uint4*>(row + 64 * h);
    const uint4* fl = reinterpret_cast<const uint4*>(s_flip) + h * 16;
    float x[64];
    float nu2 = 0.f;
    if (din == 128) {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint4 v = src[c];
        const uint4 f = fl[c];
        x[4 * c + 0] = __uint_as_float(v.x ^ f.x);
        x[4 * c + 1] = __uint_as_float(v.y ^ f.y);
        x[4 * c + 2] = __uint_as_float(v.z ^ f.z);
        x[4 * c + 3] = __uint_as_float(v.w ^ f.w);
      }
    } else {
      // zero padding: 4-coordinate chunk c of this lane half is an input
      // coordinate when 64 h + 4 c < din; the others read as +0
      const int cval = std::min(16, std::max(0, (int(din) - 64 * h) / 4));
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint4 v = c < cval ? src[c] : make_uint4(0u, 0u, 0u, 0u);
        const uint4 f = c < cval ? fl[c] : make_uint4(0u, 0u, 0u, 0u);
        x[4 * c + 0] = __uint_as_float(v.x ^ f.x);
        x[4 * c + 1] = __uint_as_float(v.y ^ f.y);
        x[4 * c + 2] = __uint_as_float(v.z ^ f.z);
        x[4 * c + 3] = __uint_as_float(v.w ^ f.w);
      }
    }
#pragma unroll
    for (int r = 0; r < 64; ++r) nu2 = fmaf(x[r], x[r], nu2);
    // the first stage adds +0 to its outputs: sign-flipped zero inputs would
    // otherwise leave -0 behind, and an exact zero must count as non-negative
#pragma unroll
    for (int r = 0; r < 64; r += 2) {
      const float a = x[r], b = x[r + 1];
      x[r] = (a + b) + 0.0f;
      x[r + 1] = (a - b) + 0.0f;
    }
    butterfly_rest(x, 2);
    if constexpr (VAL) {
      ValOut out;
      value_tail<B>(x, nu2, cst, lane, g, pos + n, valid, out);
      store_vtile<B>(out, lane, Ncap, planes, static_cast<uint16_t*>(norms_));
    } else {
      TileOut out;
      encode_tail<B>(x, nu2, ec, s_frag, lane, g, pos + n, valid, out);
      store_tile<B>(out, lane, Ncap, planes, static_cast<uint32_t*>(norms_));
    }
  }
}

// ============================================================== score, d = 128
// Grid (g, chunk of 4 query heads, key range); 1024 threads, 16 waves.
// Set-up:
//  - R q by a butterfly (waves 0-3, one query each; lane L holds coordinates
//    L and L + 64), exchanges through DPP, swizzles and half-wave swaps;
//  - S q: wave w multiplies rows 64 (w & 1) + L of S by columns
//    16 (w >> 1) .. 16 (w >> 1) + 15 of the four queries, which are the same
//    for the whole wave and sit in scalar registers; eight partial sums per row;
//  - byte subset-sum tables  T[ty][idx][pos] = sum over set bits t of idx of
//    2 X_ty[8 pos + t], four queries per 16-byte entry, X_0 = R q (read with
//    code-plane bytes), X_1 = S q (read with sign-plane bytes).
// Entry (ty, idx, pos) lives at byte ty * 64K + idx * 256 + pos * 16, so byte
// position pos is always in LDS bank group pos.  Lane L visits the sixteen
// byte positions of a plane in the order k ^ (L & 15): the sixteen lanes the
// LDS serves together then hit sixteen different bank groups whatever the
// key bytes are, and the random gathers run at the conflict-free rate.
// Each lane scores one key per step: (B + 1) planes (B = 3: plus the parity
// plane) x 16 table reads with 4 adds each.  Every wave keeps D key tiles in
// flight in registers; the first D are requested before the set-up, so the
// key stream starts at once.  All loads are unconditional (clamped to the
// range) so that each wait covers exactly the data it needs.

constexpr int kScoreThreads = 1024;

struct ScoreLds {
  f32x4 tab[2 * 256 * 16];   // 128 KB, first: its byte offsets are the table addresses
  f32x4 x[2][8][16];         // [ty][t][pos] = 2 X_ty[8 pos + t]
  f32x4 part[8][128];        // S q partial sums, [column segment][row]
  f32x4 sum[2];              // sum over all coordinates of 2 X_ty
};

// o[i] = w[i ^ (2 s2 + s1)]: the lane's word order for its position order
__device__ __forceinline__ void permute_words(const uint4 w, bool s2, bool s1, uint32_t (&o)[4]) {
  const uint32_t t0 = s2 ? w.z : w.x, t1 = s2 ? w.w : w.y;
  const uint32_t t2 = s2 ? w.x : w.z, t3 = s2 ? w.y : w.w;
  o[0] = s1 ? t1 : t0;
  o[1] = s1 ? t0 : t1;
  o[2] = s1 ? t3 : t2;
  o[3] = s1 ? t2 : t3;
}

// value of lane L ^ S
template <int S>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __float_as_int(v);
  if constexpr (S == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
  if constexpr (S == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
  if constexpr (S == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x101F));
  if constexpr (S == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));
  if constexpr (S == 16) return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x401F));
}

// one butterfly stage of stride S: (a, b) -> (a + b, a - b) over lanes L, L ^ S
template <int S>
__device__ __forceinline__ float butterfly_lane(float y, bool up) {
  const float p = lane_xor<S>(y);
  return up ? p - y : y + p;
}

__device__ __forceinline__ float butterfly_lane32(float y, bool up) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  const float r0 = __uint_as_float(r[0]), r1 = __uint_as_float(r[1]);
  return up ? r0 - r1 : r0 + r1;   // lanes < 32: (own, partner); lanes >= 32: (partner, own)
}

template <int B, bool QBF16>
__global__ __launch_bounds__(kScoreThreads, 1) void score128_kernel(
    const void* __restrict__ q, const uint4* __restrict__ planes, const uint32_t* __restrict__ norms,
    int64_t N, int64_t Ncap, int Qg, int64_t chunk, float* __restrict__ logits,
    const DevConsts* __restrict__ cst, const uint4* __restrict__ Sh) {
  constexpr int P = B + 1;
  constexpr int NW = B == 3 ? P + 1 : P;   // plane words scored per key (B = 3: + parity)
  constexpr int D = 2;   // key tiles in flight per wave (two measured 2-3% faster than three at b = 3)
  constexpr int64_t kStride = kScoreThreads;   // keys between a wave's consecutive tiles
  __shared__ ScoreLds sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.x;
  const int qc = blockIdx.y;
  const int64_t n0 = int64_t(blockIdx.z) * chunk;
  const int64_t n1 = std::min<int64_t>(N, n0 + chunk);   // n0 < n1: the host sizes the grid so
  // keys [0, N) of a cache holding Ncap records per group; logits [G][Qg][N]
  const uint4* pg = planes + g * P * Ncap;
  const uint32_t* ng = norms + g * Ncap;

  // ---- loads: sixteen S R^T columns (fp16, exact), the R q input, the
  // first D key tiles.  S q = (S R^T)(R q): the scorer needs R q anyway, and
  // the fp16 table is half the bytes every workgroup fetches at its start.
  const int seg = wave >> 1;
  const int jrow = 64 * (wave & 1) + lane;
  uint4 sh[2];   // (S R^T)[jrow][16 seg + m], m = 0..15
  {
    const uint4* sp = Sh + (size_t(seg) * 128 + jrow) * 2;
    sh[0] = sp[0];
    sh[1] = sp[1];
  }
  // query rows hold din <= 128 elements; coordinates at or past din are zero
  // padding (the loads are clamped to the row and their values dropped)
  const int din = int(cst->din);
  uint32_t u0, u1;   // raw bits of the R q input (converted after the pin below)
  {
    const int qr = std::min(qc * 4 + (wave & 3), Qg - 1);
    const int64_t at = (g * Qg + qr) * din;
    const int i0 = std::min(lane, din - 1), i1 = std::min(lane + 64, din - 1);
    if constexpr (QBF16) {
      u0 = static_cast<const uint16_t*>(q)[at + i0];
      u1 = static_cast<const uint16_t*>(q)[at + i1];
    } else {
      u0 = static_cast<const uint32_t*>(q)[at + i0];
      u1 = static_cast<const uint32_t*>(q)[at + i1];
    }
  }
  uint32_t dn0 = cst->dneg[lane >> 5], dn1 = cst->dneg[2 + (lane >> 5)];
  // wave-uniform plane bases + 32-bit lane offsets (key index < 2^28): the
  // loads take the scalar-base form and need no 64-bit address arithmetic
  auto load_tile = [&](int64_t b, uint4 (&wv)[P], uint32_t& nv) {
    const uint32_t n = uint32_t(std::min<int64_t>(b + lane, n1 - 1));
    const uint32_t off16 = n * 16u, off4 = n * 4u;   // byte offsets, < 2^32
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(pg + p * Ncap) + off16));
      wv[p] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    nv = __builtin_nontemporal_load(
        reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(ng) + off4));
  };
  const int64_t first = n0 + int64_t(wave) * 64;
  uint4 w[D][P];
  uint32_t nr[D];
#pragma unroll
  for (int k = 0; k < D; ++k) load_tile(first + k * kStride, w[k], nr[k]);
  // (an empty use outside the branch below keeps these loads ahead of the key
  // tiles: issued later, waiting for them would also wait for the tiles)
  asm volatile("" : "+v"(u0), "+v"(u1), "+v"(dn0), "+v"(dn1));
  const float v0 = lane < din ? __uint_as_float(QBF16 ? u0 << 16 : u0) : 0.f;
  const float v1 = lane + 64 < din ? __uint_as_float(QBF16 ? u1 << 16 : u1) : 0.f;

  // ---- R q = H D q / sqrt(d)
  if (wave < 4) {
    const bool live = qc * 4 + wave < Qg;
    const uint32_t f0 = (dn0 >> (lane & 31)) & 1u;
    const uint32_t f1 = (dn1 >> (lane & 31)) & 1u;
    const float a = live ? (f0 ? -v0 : v0) : 0.f, bq = live ? (f1 ? -v1 : v1) : 0.f;
    float y0 = a + bq, y1 = a - bq;
    y0 = butterfly_lane<1>(y0, lane & 1);   y1 = butterfly_lane<1>(y1, lane & 1);
    y0 = butterfly_lane<2>(y0, lane & 2);   y1 = butterfly_lane<2>(y1, lane & 2);
    y0 = butterfly_lane<4>(y0, lane & 4);   y1 = butterfly_lane<4>(y1, lane & 4);
    y0 = butterfly_lane<8>(y0, lane & 8);   y1 = butterfly_lane<8>(y1, lane & 8);
    y0 = butterfly_lane<16>(y0, lane & 16); y1 = butterfly_lane<16>(y1, lane & 16);
    y0 = butterfly_lane32(y0, lane & 32);   y1 = butterfly_lane32(y1, lane & 32);
    float* xf = reinterpret_cast<float*>(&sm.x[0][0][0]);
    xf[((lane & 7) * 16 + (lane >> 3)) * 4 + wave] = 2.0f * (y0 * cst->inv_sqrt_d);
    xf[((lane & 7) * 16 + 8 + (lane >> 3)) * 4 + wave] = 2.0f * (y1 * cst->inv_sqrt_d);
  }
  __syncthreads();
  // ---- 2 S q partial sums over this wave's sixteen coordinates of 2 R q
  {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint32_t hw[8] = {sh[0].x, sh[0].y, sh[0].z, sh[0].w, sh[1].x, sh[1].y, sh[1].z, sh[1].w};
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float sv = h2f_bits(hw[m >> 1] >> (16 * (m & 1)));
      const f32x4 xv = sm.x[0][m & 7][2 * seg + (m >> 3)];   // coordinate 16 seg + m, 4 queries
      acc[0] = fmaf(sv, xv[0], acc[0]);
      acc[1] = fmaf(sv, xv[1], acc[1]);
      acc[2] = fmaf(sv, xv[2], acc[2]);
      acc[3] = fmaf(sv, xv[3], acc[3]);
    }
    sm.part[seg][jrow] = acc;
  }
  __syncthreads();
  if (tid < 128) {
    f32x4 t = sm.part[0][tid];
#pragma unroll
    for (int k = 1; k < 8; ++k) t += sm.part[k][tid];
    sm.x[1][tid & 7][tid >> 3] = t;
  }
  __syncthreads();
  // ---- tables: thread (pos, ty, hi) writes entries idx = 8 hi + j, j = 0..7
  {
    const int pos = tid & 15, ty = (tid >> 4) & 1, hi = tid >> 5;
    f32x4 xv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) xv[t] = sm.x[ty][t][pos];
    f32x4 bs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 3; t < 8; ++t) {
      const float on = float((hi >> (t - 3)) & 1);
      bs[0] = fmaf(on, xv[t][0], bs[0]);
      bs[1] = fmaf(on, xv[t][1], bs[1]);
      bs[2] = fmaf(on, xv[t][2], bs[2]);
      bs[3] = fmaf(on, xv[t][3], bs[3]);
    }
    f32x4 e[8];
    e[0] = bs;
    e[1] = bs + xv[0];
    e[2] = bs + xv[1];
    e[3] = e[2] + xv[0];
    e[4] = bs + xv[2];
    e[5] = e[4] + xv[0];
    e[6] = e[4] + xv[1];
    e[7] = e[6] + xv[0];
#pragma unroll
    for (int j = 0; j < 8; ++j) sm.tab[(ty * 256 + hi * 8 + j) * 16 + pos] = e[j];
    if (wave == 15) {   // lanes 32..63 hold the full-byte sums (idx 255) of every position
      f32x4 t = e[7];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        t[c] += lane_xor<1>(t[c]);
        t[c] += lane_xor<2>(t[c]);
        t[c] += lane_xor<4>(t[c]);
        t[c] += lane_xor<8>(t[c]);
      }
      if (lane == 32) sm.sum[0] = t;
      if (lane == 48) sm.sum[1] = t;
    }
  }
  __syncthreads();

  // per-query sums (sum R q, sum S q) are the same for every lane
  // (the components are copied to scalars first: a bit cast of a vector
  // element lvalue reads the vector's first component)
  float sr[4], ss[4];
  {
    const f32x4 s0 = sm.sum[0], s1 = sm.sum[1];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float a = s0[qq], b = s1[qq];
      sr[qq] = 0.5f * __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a)));
      ss[qq] = 0.5f * __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(b)));
    }
  }
  const float a0 = cst->alpha[0], a1 = cst->alpha[1], a2 = cst->alpha[2], a3 = cst->alpha[3];
  const float asum = cst->alpha_sum, qs = cst->qjl_scale;
  float* lrow[4];   // logit rows of the chunk's queries (wave-uniform)
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) lrow[qq] = logits + (g * Qg + std::min(qc * 4 + qq, Qg - 1)) * N;

  // Per-lane address pieces.  Lookup (a, c) of a plane reads position
  // (4 a + c) ^ r, which is byte c ^ (r & 3) of permuted word a; one byte
  // permute assembles  ty * 64K + byte * 256 + slot * 16  from the word, a
  // pair of slot bytes (plus a 0x01 byte for ty = 1) and a selector.
  const uint32_t r = lane & 15, rb = r & 3;
  uint32_t bp[4][2], sel[2][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bp[a][h] = (((4u * a + 2 * h) ^ r) << 4) | (((4u * a + 2 * h + 1) ^ r) << 12) | (1u << 16);
      asm volatile("" : "+v"(bp[a][h]));
    }
#pragma unroll
  for (int ty = 0; ty < 2; ++ty)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sel[ty][c] = uint32_t(c & 1) | ((4u + (c ^ rb)) << 8) | ((ty ? 2u : 12u) << 16) | (12u << 24);
      asm volatile("" : "+v"(sel[ty][c]));
    }
  const bool s2 = lane & 8, s1 = lane & 4;
  const char* tabp = reinterpret_cast<const char*>(sm.tab);

  auto add_plane = [&](const uint32_t (&rw)[4], int ty, float* acc) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t ad = __builtin_amdgcn_perm(rw[a], bp[a][c >> 1], sel[ty][c]);
        const f32x4 tv = *reinterpret_cast<const f32x4*>(tabp + ad);
        acc[0] += tv[0]; acc[1] += tv[1]; acc[2] += tv[2]; acc[3] += tv[3];
      }
      // an empty fence (no instruction) that takes the accumulators: this
      // word's adds complete before the next word's table reads are issued
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]) : : "memory");
    }
  };

  auto score_tile = [&](const uint4 (&wt)[P], uint32_t nrm, int64_t b) {
    uint32_t rw[NW][4];
#pragma unroll
    for (int p = 0; p < P; ++p) permute_words(wt[p], s2, s1, rw[p]);
    if constexpr (B == 3) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rw[P][i] = rw[0][i] ^ rw[1][i] ^ rw[2][i];
    }
    float acc[NW][4];
#pragma unroll
    for (int t = 0; t < NW; ++t)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) acc[t][qq] = 0.f;
    // code planes (and parity) against R q, the sign plane (index B) against S q
#pragma unroll
    for (int t = 0; t < B; ++t) add_plane(rw[t], 0, acc[t]);
    if constexpr (B == 3) add_plane(rw[P], 0, acc[P]);
    add_plane(rw[B], 1, acc[B]);

    const float nu = h2f_bits(nrm & 0xffffu), rs = h2f_bits(nrm >> 16) * qs;
    const bool in_range = b + lane < n1;
    uint32_t off4 = (uint32_t(b) + uint32_t(lane)) * 4u;
    asm volatile("" : "+v"(off4));   // keep the offset 32-bit (scalar-base stores)
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
      const int qh = qc * 4 + qq;
      if (in_range && qh < Qg)   // streamed output: no reuse, written past the caches
        __builtin_nontemporal_store(fmaf(nu, mse, rs * (ss[qq] - acc[B][qq])),
                                    reinterpret_cast<float*>(reinterpret_cast<char*>(lrow[qq]) + off4));
    }
  };

  // tiles t = 0, 1, ... of this wave start at first + t * kStride; tile t
  // sits in slot t % D and its slot is refilled with tile t + D right after
  const int64_t ntiles = first < n1 ? (n1 - first + kStride - 1) / kStride : 0;
  for (int64_t t0 = 0; t0 < ntiles; t0 += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      if (t0 + k < ntiles) score_tile(w[k], nr[k], first + (t0 + k) * kStride);
      load_tile(first + (t0 + k + D) * kStride, w[k], nr[k]);
    }
  }
  // the refills past the range are never used: let them land before the wave ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
  // rows of din elements: the coordinates a zero-padded input never had are dropped
  const int din = int(cst->din);
  if constexpr (BF16OUT) {
    __bf16* o = static_cast<__bf16*>(out) + key * din;
    if (lane < din) o[lane] = static_cast<__bf16>(y0);
    if (lane + 64 < din) o[lane + 64] = static_cast<__bf16>(y1);
  } else {
    float* o = static_cast<float*>(out) + key * din;
    if (lane < din) o[lane] = y0;
    if (lane + 64 < din) o[lane + 64] = y1;
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

// ============================================================== decode attention, d = 128
// out[g][h] = sum_n softmax_n(scale * logit[g][h][n]) v_mse[g][n] over packed
// values v_mse = nu~ R^T c_v[code] (value records: b-bit Lloyd-Max codes and
// a half norm).  R^T is linear, so the weighted sum is formed in the rotated
// domain, A = sum_n w_n nu~_n c_v[code_n], and rotated back once per query.
// Split over key ranges (flash-decoding style): each range keeps its own
// maximum m_s, normaliser Z_s = sum exp(scale l - m_s) and A_s; a combine step
// rescales by exp(m_s - M).
constexpr int kAttnThreads = 256;
constexpr int kAttnPart = 8 + 4 * 128;   // m[4], Z[4], A[4][128] per (group, query chunk, range)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Grid (G, query chunks of 4, key ranges).  Thread t: while weighting, key
// t % 64 of a 64-key block for query t / 64; while accumulating, the four
// adjacent coordinates 4 (t % 32) .. 4 (t % 32) + 3 of every eighth key of the
// block, starting at key t / 32.  A 2^(2 BV)-entry table maps the BV plane
// bits of two adjacent coordinates to their two levels, so each pair costs one
// 8-byte LDS read after BV two-bit field extractions.
template <int BV>
__global__ __launch_bounds__(kAttnThreads) void attn_values128_kernel(
    const float* __restrict__ logits, const uint4* __restrict__ vplanes,
    const uint16_t* __restrict__ vnorms, int64_t N, int Qg, int64_t chunk, float scale,
    const DevConsts* __restrict__ cst, float* __restrict__ part) {
  constexpr int NL = 1 << (2 * BV);
  __shared__ f32x4 s_w[2][64];              // weights of a block's keys, 4 queries (double-buffered)
  __shared__ uint32_t s_pl[2][BV][64][4];   // value plane words of a block's keys
  __shared__ float2 s_lut[NL];              // pair of levels by plane-major 2-bit fields
  __shared__ float s_red[8][32][17];        // [key lane][coordinate quad][4 coords x 4 queries]
  __shared__ float s_m[2][4];
  __shared__ float s_f[2][4];               // rescale of the accumulators per block and query
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t g = blockIdx.x;
  const int qc = blockIdx.y;
  const int64_t n0 = int64_t(blockIdx.z) * chunk;
  const int64_t n1 = std::min<int64_t>(N, n0 + chunk);
  for (int j = tid; j < NL; j += kAttnThreads) {
    int ca = 0, cb = 0;
#pragma unroll
    for (int p = 0; p < BV; ++p) {
      ca |= ((j >> (2 * p)) & 1) << p;
      cb |= ((j >> (2 * p + 1)) & 1) << p;
    }
    s_lut[j] = make_float2(cst->vlevels[ca], cst->vlevels[cb]);
  }

  // Online softmax: wave q keeps query q's running maximum mx (the same in
  // every lane) and normaliser; when a block raises the maximum, every
  // accumulator of that query is rescaled by exp(old - new) before the block
  // is added.
  const int qh = qc * 4 + wave;
  const bool qlive = qh < Qg;
  const float* lrow = logits + (g * Qg + (qlive ? qh : 0)) * N;
  float mx = -INFINITY;
  float zs = 0.f;                    // this thread's part of Z for query `wave`
  float acc[4][4] = {};              // [coordinate][query]
  const int cq = tid & 31, kq = tid >> 5;
  const int wsel = cq >> 3, sh = 4 * (cq & 7);   // word and bit of the coordinate quad
  const char* lut = reinterpret_cast<const char*>(s_lut);
  // the next block's logit, norm and plane words are loaded into registers
  // while the current block is accumulated (one barrier per block: a buffer
  // is rewritten only after every thread has passed the next barrier)
  float lg_n = 0.f;
  uint32_t nv_n = 0;
  uint4 pl_n = make_uint4(0, 0, 0, 0);
  auto load_block = [&](int64_t nb) {
    const int64_t nc = std::min<int64_t>(nb + lane, n1 - 1);
    lg_n = lrow[nc];
    nv_n = vnorms[g * N + nc];
    if (wave < BV) pl_n = vplanes[(g * BV + wave) * N + nc];
  };
  load_block(n0);
  int buf = 0;
  for (int64_t nb = n0; nb < n1; nb += 64, buf ^= 1) {
    {
      const bool in = nb + lane < n1 && qlive;
      const float z = scale * lg_n;
      const float mnew = fmaxf(mx, wave_max(in ? z : -INFINITY));
      const float f = qlive ? __expf(mx - mnew) : 1.f;     // exp(-inf) = 0 on the first block
      mx = qlive ? mnew : 0.f;
      float w = 0.f;
      zs *= f;
      if (in) {
        const float e = __expf(z - mx);
        zs += e;
        w = e * h2f_bits(nv_n);
      }
      reinterpret_cast<float*>(&s_w[buf][lane])[wave] = w;
      if (lane == 0) s_f[buf][wave] = f;
      if (wave < BV) *reinterpret_cast<uint4*>(s_pl[buf][wave][lane]) = pl_n;
    }
    __syncthreads();
    {
      const float f0 = s_f[buf][0], f1 = s_f[buf][1], f2 = s_f[buf][2], f3 = s_f[buf][3];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[c][0] *= f0; acc[c][1] *= f1; acc[c][2] *= f2; acc[c][3] *= f3;
      }
    }
    if (nb + 64 < n1) load_block(nb + 64);
#pragma unroll 4
    for (int j = 0; j < 8; ++j) {
      const int kk = kq + 8 * j;
      const f32x4 wv = s_w[buf][kk];
      uint32_t a0 = 0, a1 = 0;   // byte offsets of the two level pairs
#pragma unroll
      for (int p = 0; p < BV; ++p) {
        const uint32_t x = s_pl[buf][p][kk][wsel];
        a0 |= __builtin_amdgcn_ubfe(x, sh, 2) << (2 * p + 3);
        a1 |= __builtin_amdgcn_ubfe(x, sh + 2, 2) << (2 * p + 3);
      }
      const float2 l01 = *reinterpret_cast<const float2*>(lut + a0);
      const float2 l23 = *reinterpret_cast<const float2*>(lut + a1);
      const float lv[4] = {l01.x, l01.y, l23.x, l23.y};
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[c][q] = fmaf(wv[q], lv[c], acc[c][q]);
    }
  }

  // ---- reduce over the eight key lanes, write the range's partial state
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) s_red[kq][cq][4 * c + q] = acc[c][q];
  zs = wave_sum(zs);
  if (lane == 0) { s_m[0][wave] = mx; s_m[1][wave] = zs; }
  __syncthreads();
  float* out = part + ((g * gridDim.y + qc) * gridDim.z + blockIdx.z) * kAttnPart;
  if (tid < 8) out[tid] = s_m[tid >> 2][tid & 3];
  for (int e = tid; e < 512; e += kAttnThreads) {
    const int q = e >> 7, i = e & 127, quad = i >> 2, c = i & 3;
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a += s_red[k][quad][4 * c + q];
    out[8 + e] = a;                 // A[q][i]
  }
}

// One wave per (group, query): merge the ranges, divide by Z, rotate back
// with R^T = D H / sqrt(d).  Lane L holds coordinates L and L + 64.
__global__ __launch_bounds__(64) void attn_combine128_kernel(const float* __restrict__ part,
                                                              int Qg, int nqc, int splits,
                                                              const DevConsts* __restrict__ cst,
                                                              float* __restrict__ out) {
  const int lane = threadIdx.x;
  const int64_t gh = blockIdx.x;
  const int64_t g = gh / Qg;
  const int h = int(gh - g * Qg), qc = h >> 2, q = h & 3;
  const float* base = part + (g * nqc + qc) * int64_t(splits) * kAttnPart;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) M = fmaxf(M, base[s * kAttnPart + q]);
  float Z = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    const float* ps = base + s * kAttnPart;
    const float f = __expf(ps[q] - M);
    Z = fmaf(f, ps[4 + q], Z);
    a0 = fmaf(f, ps[8 + q * 128 + lane], a0);
    a1 = fmaf(f, ps[8 + q * 128 + 64 + lane], a1);
  }
  const float inv = 1.0f / Z;
  float y0 = a0 * inv + a1 * inv, y1 = a0 * inv - a1 * inv;
  y0 = butterfly_lane<1>(y0, lane & 1);   y1 = butterfly_lane<1>(y1, lane & 1);
  y0 = butterfly_lane<2>(y0, lane & 2);   y1 = butterfly_lane<2>(y1, lane & 2);
  y0 = butterfly_lane<4>(y0, lane & 4);   y1 = butterfly_lane<4>(y1, lane & 4);
  y0 = butterfly_lane<8>(y0, lane & 8);   y1 = butterfly_lane<8>(y1, lane & 8);
  y0 = butterfly_lane<16>(y0, lane & 16); y1 = butterfly_lane<16>(y1, lane & 16);
  y0 = butterfly_lane32(y0, lane & 32);   y1 = butterfly_lane32(y1, lane & 32);
  const float sc = cst->inv_sqrt_d;
  const uint32_t f0 = (cst->dneg[lane >> 5] >> (lane & 31)) & 1u;
  const uint32_t f1 = (cst->dneg[2 + (lane >> 5)] >> (lane & 31)) & 1u;
  const int din = int(cst->din);   // output rows keep the input coordinates only
  float* o = out + gh * din;
  if (lane < din) o[lane] = (f0 ? -y0 : y0) * sc;
  if (64 + lane < din) o[64 + lane] = (f1 ? -y1 : y1) * sc;
}

}  // namespace

bool encode_supported(const Codebook& cb) { return cb.d == 128 || cb.d == 1024; }
bool score_supported(const Codebook& cb) { return cb.d == 128 || cb.d == 1024; }

// d = 128: each workgroup prepares its queries itself, no workspace; d = 1024:
// the prepared queries (2 R q, 2 S q and their sums) for all groups.
size_t score_workspace_bytes(const Codebook& cb, int64_t G, int Qg) {
  return cb.d == 1024 ? score_wide_prep_bytes(G, Qg) : 0;
}

hipError_t launch_encode(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t N,
                         int64_t Ncap, int64_t pos, void* packed, hipStream_t s) {
  if (cb.d == 1024) return launch_encode_wide(cb, keys, dtype, G, N, packed, s);
  const int64_t ntiles = G * ((N + 31) / 32);
  uint32_t* planes = static_cast<uint32_t*>(packed);
  uint32_t* norms = planes + G * Ncap * int64_t(cb.bits) * (cb.d / 32);
  if (dtype == 1) {
    const int64_t ntiles16 = G * ((N + 15) / 16);
    const int64_t want = (ntiles16 + kEnc16Waves - 1) / kEnc16Waves;
    const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * 3));
    const uint16_t* kb = static_cast<const uint16_t*>(keys);
#define TQ_ENCB(BB)                                                                              \
  hipLaunchKernelGGL((encode128_bf16_t16_kernel<BB, false>), dim3(grid), dim3(kEnc16Threads), 0, s, kb, G, N, \
                     Ncap, pos, planes, norms, cb.d_consts, cb.d_frag16,                       \
                     reinterpret_cast<const uint4*>(cb.d_dm16))
    switch (cb.bits - 1) {
      case 1: TQ_ENCB(1); break;
      case 2: TQ_ENCB(2); break;
      default: TQ_ENCB(3); break;
    }
#undef TQ_ENCB
  } else {
    const int64_t want = (ntiles + kEncWaves - 1) / kEncWaves;
    const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * 2));
    const float* kf = static_cast<const float*>(keys);
#define TQ_ENCF(BB)                                                                             \
  hipLaunchKernelGGL((encode128_f32_kernel<BB, false>), dim3(grid), dim3(kEncThreads), 0, s, kf, G, N, \
                     Ncap, pos, \
                     planes, norms, cb.d_consts, cb.d_frag, cb.d_flip_f32)
    switch (cb.bits - 1) {
      case 1: TQ_ENCF(1); break;
      case 2: TQ_ENCF(2); break;
      default: TQ_ENCF(3); break;
    }
#undef TQ_ENCF
  }
  return hipGetLastError();
}

hipError_t launch_encode_values(const Codebook& cb, const void* values, int dtype, int64_t G,
                                int64_t N, void* vpacked, hipStream_t s) {
  const int64_t ntiles = G * ((N + 31) / 32);
  uint32_t* planes = static_cast<uint32_t*>(vpacked);
  uint16_t* norms = reinterpret_cast<uint16_t*>(planes + G * N * int64_t(cb.bits) * (cb.d / 32));
  if (dtype == 1) {
    const int64_t ntiles16 = G * ((N + 15) / 16);
    const int64_t want = (ntiles16 + kEnc16Waves - 1) / kEnc16Waves;
    const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * 4));
    const uint16_t* vb = static_cast<const uint16_t*>(values);
#define TQ_VB(BB)                                                                                  \
  hipLaunchKernelGGL((encode128_bf16_t16_kernel<BB, true>), dim3(grid), dim3(kEnc16Threads), 0, s, vb, \
                     G, N, N, int64_t(0), planes, norms, cb.d_consts, cb.d_frag16,                 \
                     reinterpret_cast<const uint4*>(cb.d_dm16))
    switch (cb.bits) {
      case 2: TQ_VB(2); break;
      case 3: TQ_VB(3); break;
      default: TQ_VB(4); break;
    }
#undef TQ_VB
  } else {
    const int64_t want = (ntiles + kEncWaves - 1) / kEncWaves;
    const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * 2));
    const float* vf = static_cast<const float*>(values);
#define TQ_VF(BB)                                                                                \
  hipLaunchKernelGGL((encode128_f32_kernel<BB, true>), dim3(grid), dim3(kEncThreads), 0, s, vf, \
                     G, N, N, int64_t(0), planes, norms, cb.d_consts, cb.d_frag, cb.d_flip_f32)
    switch (cb.bits) {
      case 2: TQ_VF(2); break;
      case 3: TQ_VF(3); break;
      default: TQ_VF(4); break;
    }
#undef TQ_VF
  }
  return hipGetLastError();
}

// Key ranges of the decode-attention value pass: multiples of 64 keys,
// enough (group, query chunk, range) workgroups for four per compute unit.
static void attn_split(int64_t G, int Qg, int64_t N, int64_t& chunk, int64_t& splits) {
  const int64_t units = G * ((Qg + 3) / 4);
  const int64_t want_wg = int64_t(num_cus()) * 4;
  int64_t want = std::max<int64_t>(1, (want_wg + units - 1) / units);
  want = std::min<int64_t>(want, std::max<int64_t>(1, (N + 255) / 256));
  chunk = ((N + want - 1) / want + 63) / 64 * 64;
  splits = (N + chunk - 1) / chunk;
}

size_t attention_workspace_bytes(const Codebook& cb, int64_t G, int Qg, int64_t N) {
  (void)cb;
  int64_t chunk, splits;
  attn_split(G, Qg, N, chunk, splits);
  const size_t lg = (size_t(G) * Qg * N * 4 + 255) / 256 * 256;
  return lg + size_t(G) * ((Qg + 3) / 4) * splits * kAttnPart * 4;
}

hipError_t launch_attention(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                            const void* kpacked, const void* vpacked, int64_t N, float scale,
                            float* out, void* ws, hipStream_t s) {
  int64_t chunk, splits;
  attn_split(G, Qg, N, chunk, splits);
  float* logits = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         (size_t(G) * Qg * N * 4 + 255) / 256 * 256);
  hipError_t e = launch_score(cb, q, qdtype, G, Qg, kpacked, N, N, logits, nullptr, s);
  if (e != hipSuccess) return e;
  const int nqc = (Qg + 3) / 4;
  const uint4* vpl = static_cast<const uint4*>(vpacked);
  const uint16_t* vn = reinterpret_cast<const uint16_t*>(static_cast<const uint32_t*>(vpacked) +
                                                         G * N * int64_t(cb.bits) * (cb.d / 32));
  const dim3 grid{unsigned(G), unsigned(nqc), unsigned(splits)};
#define TQ_AV(BB)                                                                                 \
  hipLaunchKernelGGL((attn_values128_kernel<BB>), grid, dim3(kAttnThreads), 0, s, logits, vpl, vn, \
                     N, Qg, chunk, scale, cb.d_consts, part)
  switch (cb.bits) {
    case 2: TQ_AV(2); break;
    case 3: TQ_AV(3); break;
    default: TQ_AV(4); break;
  }
#undef TQ_AV
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine128_kernel, dim3(unsigned(G * Qg)), dim3(64), 0, s, part, Qg, nqc,
                     int(splits), cb.d_consts, out);
  return hipGetLastError();
}

hipError_t launch_score(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                        const void* packed, int64_t N, int64_t Ncap, float* logits, void* ws,
                        hipStream_t s) {
  if (cb.d == 1024) return launch_score_wide(cb, q, qdtype, G, Qg, packed, N, logits, ws, s);
  // enough workgroups for every CU: split each (group, query chunk) unit's
  // keys into ranges of at least 512 keys, a multiple of 64 each
  const int nqc = (Qg + 3) / 4;
  const int64_t units = G * nqc;
  const int64_t cus = num_cus();
  int64_t want = std::max<int64_t>(1, (cus + units - 1) / units);
  want = std::min<int64_t>(want, std::max<int64_t>(1, (N + 511) / 512));
  const int64_t chunk = ((N + want - 1) / want + 63) / 64 * 64;
  const int64_t splits = (N + chunk - 1) / chunk;
  const dim3 grid{unsigned(G), unsigned(nqc), unsigned(splits)};
  const uint4* planes = static_cast<const uint4*>(packed);
  const uint32_t* norms =
      static_cast<const uint32_t*>(packed) + G * Ncap * int64_t(cb.bits) * (cb.d / 32);
  const bool bf = qdtype == 1;
#define TQ_SC(BB, QB)                                                                   \
  hipLaunchKernelGGL((score128_kernel<BB, QB>), grid, dim3(kScoreThreads), 0, s, q, planes, \
                     norms, N, Ncap, Qg, chunk, logits, cb.d_consts, cb.d_Sh)
  switch (cb.bits - 1) {
    case 1: if (bf) TQ_SC(1, true); else TQ_SC(1, false); break;
    case 2: if (bf) TQ_SC(2, true); else TQ_SC(2, false); break;
    default: if (bf) TQ_SC(3, true); else TQ_SC(3, false); break;
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

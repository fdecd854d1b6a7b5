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
//
// Records are stored per tile of 16 values: slot s of a tile holds
// coordinate 32 (s / 32) + 16 (s % 2) + (s % 32) / 2 for all 16 values, as
// eight groups of two values, bit 2 p + i of group q being bit p of the code
// of value 2 q + i.  The decode attention reads one group as the index of a
// table of level pairs.

// Tile packing, for all 64 lanes of a wave: wp[p] of lane 16 w + n holds bit
// p of the codes of value n of the tile at coordinates 32 w .. 32 w + 31 (bit
// r: coordinate 32 w + r); out receives the lane's BV words of the tile,
// slots 2 (16 w + n) and 2 (16 w + n) + 1.  First a bit transpose inside each
// row of 16 lanes: four exchanges, exchange i trading lane bit i for word bit
// i with lane n ^ 2^i, leave in word bit k + 16 h value k at coordinate
// 32 w + 16 h + n; then each slot's bits are regrouped value group by value
// group.
template <int BV>
__device__ __forceinline__ void vtile_pack(uint32_t (&wp)[BV], int lane, uint32_t (&out)[BV]) {
  const int n = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = 1 << i;
    const uint32_t m = i == 0 ? 0x55555555u : i == 1 ? 0x33333333u : i == 2 ? 0x0F0F0F0Fu : 0x00FF00FFu;
    const bool low = ((n >> i) & 1) == 0;
    const uint32_t own = low ? m : ~m;                  // bits this lane keeps
    const uint32_t rot = low ? uint32_t(32 - s) : uint32_t(s);   // partner's bits move up / down
#pragma unroll
    for (int p = 0; p < BV; ++p) {
      int y;
      if (i == 0) y = __builtin_amdgcn_mov_dpp(int(wp[p]), 0xB1, 0xF, 0xF, false);       // lane ^ 1
      else if (i == 1) y = __builtin_amdgcn_mov_dpp(int(wp[p]), 0x4E, 0xF, 0xF, false);  // lane ^ 2
      else if (i == 2) y = __builtin_amdgcn_ds_swizzle(int(wp[p]), 0x101F);             // lane ^ 4
      else y = __builtin_amdgcn_ds_swizzle(int(wp[p]), 0x201F);                         // lane ^ 8
      const uint32_t z = __builtin_amdgcn_alignbit(uint32_t(y), uint32_t(y), rot);
      wp[p] = (wp[p] & own) | (z & ~own);
    }
  }
  // regrouping: byte j of a word holds the 2-bit units (value pairs) 4 (j % 2)
  // .. + 3 of slot j / 2; two shift-and-mask steps move a byte's four units
  // to stride 2 BV bits, and the planes are ORed in at 2 p: block j (8 BV
  // bits) is then four groups of the slot
  uint32_t blk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t acc = 0u;
#pragma unroll
    for (int p = 0; p < BV; ++p) {
      uint32_t x = __builtin_amdgcn_ubfe(wp[p], 8 * j, 8);
      if constexpr (BV == 2) {
        x = (x | (x << 4)) & 0x0F0Fu;
        x = (x | (x << 2)) & 0x3333u;
      } else if constexpr (BV == 3) {
        x = (x | (x << 8)) & 0xF00Fu;
        x = (x | (x << 4)) & 0xC30C3u;
      } else {
        x = (x | (x << 12)) & 0x000F000Fu;
        x = (x | (x << 6)) & 0x03030303u;
      }
      acc |= x << (2 * p);
    }
    blk[j] = acc;
  }
  // block j sits at bit 8 BV j of the lane's 32 BV bits
  if constexpr (BV == 2) {
    out[0] = blk[0] | (blk[1] << 16);
    out[1] = blk[2] | (blk[3] << 16);
  } else if constexpr (BV == 3) {
    out[0] = blk[0] | (blk[1] << 24);
    out[1] = (blk[1] >> 8) | (blk[2] << 16);
    out[2] = (blk[2] >> 16) | (blk[3] << 8);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = blk[j];
  }
}

// The tile's words: lane L writes words BV L .. BV L + BV - 1 of tile t of
// group g (tpg tiles per group).
template <int BV>
__device__ __forceinline__ void store_vwords(const uint32_t (&ow)[BV], int lane, int64_t g, int64_t tpg,
                                             int64_t t, uint32_t* __restrict__ planes) {
  uint32_t* dst = planes + ((g * tpg + t) * 64 + lane) * BV;
#pragma unroll
  for (int p = 0; p < BV; ++p) dst[p] = ow[p];
}

// float32 values (two-lane layout, 32 values per wave): each lane leaves its
// key's plane words h and 2 + h in the wave's LDS area st ([plane][value][word]),
// and returns half(nu), or 0 for a value below the zero-norm rule.
template <int BV>
__device__ __forceinline__ uint32_t value_tail(const float (&x)[64], float nu2,
                                               const DevConsts* __restrict__ cst, int lane, bool valid,
                                               uint32_t* st) {
  constexpr int KV = 1 << (BV - 1);    // levels on the positive half
  nu2 = xor32_sum(nu2);
  const float nu = __builtin_amdgcn_sqrtf(nu2);
  const bool zero = !(nu >= 1e-10f);
  const float nsd = nu * cst->sqrt_d;
  float tu[KV > 1 ? KV - 1 : 1];
#pragma unroll
  for (int k = 0; k < KV - 1; ++k) tu[k] = cst->vtpos[k] * nsd;
  uint32_t wu[2] = {0u, 0u};
  uint32_t wb[BV - 1][2];   // pushed magnitude index bits, complemented (see value_tail16)
#pragma unroll
  for (int j = 0; j < BV - 1; ++j) wb[j][0] = wb[j][1] = 0u;
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    const int ws = r >> 5;
    const float u = x[r];
    const float a = fabsf(u);
    wu[ws] = push_sign(wu[ws], u);
    uint64_t bx[BV - 1];
#pragma unroll
    for (int j = 0; j < BV - 1; ++j) bx[j] = 0u;
#pragma unroll
    for (int k = 0; k < KV - 1; ++k) {
      const uint64_t below = __builtin_amdgcn_ballot_w64(a < tu[k]);
#pragma unroll
      for (int j = 0; j < BV - 1; ++j)
        if (((k + 1) & ((1 << j) - 1)) == 0) bx[j] ^= below;
    }
#pragma unroll
    for (int j = 0; j < BV - 1; ++j) {
      uint64_t co;
      asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3"
          : "=v"(wb[j][ws]), "=s"(co) : "v"(wb[j][ws]), "s"(bx[j]));
    }
  }
  const bool keep = valid && !zero;
  const int h = lane >> 5, kl = lane & 31;
#pragma unroll
  for (int ws = 0; ws < 2; ++ws) {
    // words were filled oldest-bit-first: bit (r % 32) sits at 31 - r % 32
    const uint32_t sg = __builtin_bitreverse32(wu[ws]);       // 1 = negative
    uint32_t pw[BV];
    pw[BV - 1] = ~sg;
#pragma unroll
    for (int j = 0; j < BV - 1; ++j) pw[j] = ~(__builtin_bitreverse32(wb[j][ws]) ^ sg);
    // x[r] for r < 32 is coordinate 32 h + r (word h), for r >= 32 word 2 + h
#pragma unroll
    for (int p = 0; p < BV; ++p) st[(p * 32 + kl) * 4 + 2 * ws + h] = keep ? pw[p] : 0u;
  }
  return keep ? uint32_t(f2h_bits(nu)) : 0u;
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
    asm volatile("");   // a real branch: if-converted, every tile would pay the selects
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

// Paged cache: a pool of pages, each laid out as one packed group of
// page_size records; table[g * ppg + p] is the pool page that holds logical
// page p of group g.  Appends take rows [G][T] and pos[g], the logical
// position of group g's first new row; scoring takes lens[g], the number of
// records of group g.
struct PageMap {
  const int32_t* table;
  const int32_t* pos;
  const int32_t* lens;
  uint32_t T;
  int32_t ppg;         // table entries per group
  int32_t page_size;   // records per page (a multiple of 64)
  int32_t num_pages;   // pages in the pool
  // append latency kernel only: table == nullptr maps row r of a [G][T]
  // append to page r / T (the group) at slot base + r % T, a contiguous cache
  // of page_size records per group
  int64_t base;
};

// Pool page and slot of row r of a [G][T] append; false when the row's
// logical page lies outside its group's table or the entry outside the pool
// (the row is then not written).
__device__ __forceinline__ bool page_dest(const PageMap& pm, int64_t r, int64_t& page, int64_t& slot) {
  const uint32_t g = uint32_t(r) / pm.T, t = uint32_t(r) - g * pm.T;
  const int64_t lp = int64_t(pm.pos[g]) + t;
  if (lp < 0) return false;
  const int64_t lpage = lp / pm.page_size;
  if (lpage >= pm.ppg) return false;
  const int32_t ph = pm.table[int64_t(g) * pm.ppg + lpage];
  if (ph < 0 || ph >= pm.num_pages) return false;
  page = ph;
  slot = lp - lpage * pm.page_size;
  return true;
}

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
  uint32_t wu, wd[2];   // sign word; magnitude index bits (complemented), pushed
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
  constexpr int NB = B - 1;   // magnitude index bits
  uint32_t wu = 0u;
  uint32_t wd[NB > 0 ? NB : 1];
#pragma unroll
  for (int j = 0; j < (NB > 0 ? NB : 1); ++j) wd[j] = 0u;
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
        // one compare per positive threshold: its lane mask selects the
        // level; bit j of the magnitude index (complemented) is the XOR of
        // the masks over k with (k + 1) divisible by 2^j, formed on the
        // scalar unit and pushed by the carry-in of a doubling add
        uint64_t bx[NB > 0 ? NB : 1];
#pragma unroll
        for (int j = 0; j < (NB > 0 ? NB : 1); ++j) bx[j] = 0u;
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
          const uint64_t below = __builtin_amdgcn_ballot_w64(a < tu[k]);
          const float up = ec.cpos[k + 1];
          asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(mag) : "v"(up), "v"(mag), "s"(below));
#pragma unroll
          for (int j = 0; j < NB; ++j)
            if (((k + 1) & ((1 << j) - 1)) == 0) bx[j] ^= below;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          uint64_t co;
          asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(wd[j]), "=s"(co) : "v"(wd[j]), "s"(bx[j]));
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
    if constexpr (NB > 1) {
      asm volatile("" : "+v"(wu), "+v"(wd[0]), "+v"(wd[1]));
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
  for (int j = 0; j < NB; ++j) pd.wd[j] = wd[j];
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
  // stored bit j = magnitude index bit j XOR the sign; the top plane is the
  // complement of the sign (the pushed bits are complemented, odd counts)
  pw[P - 2] = ~u_;
#pragma unroll
  for (int j = 0; j < P - 2; ++j) pw[j] = ~(u_ ^ __builtin_bitreverse32(wd[j]));
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

// Value records of a 16-value tile: every lane writes its words of the tile
// (the tile's values past N are zero), the lanes of the first quarter the
// half norms of their values.
template <int BV>
__device__ __forceinline__ void store_vtile16(const TileOut16& o, int lane, int64_t Ncap,
                                              uint32_t* __restrict__ planes,
                                              uint16_t* __restrict__ norms) {
  uint32_t ow[BV];
#pragma unroll
  for (int p = 0; p < BV; ++p) ow[p] = o.w[p];
  store_vwords<BV>(ow, lane, o.g, (Ncap + 15) / 16, o.n >> 4, planes);
  if (o.valid && (lane >> 4) == 0) norms[o.g * Ncap + o.n] = uint16_t(o.norm);
}

template <int BV>
__device__ __forceinline__ void value_tail16(const f32x4 (&y)[8], float nu2,
                                             const DevConsts* __restrict__ cst, int lane, int64_t g,
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
  uint32_t wb[BV - 1];
#pragma unroll
  for (int j = 0; j < BV - 1; ++j) wb[j] = 0u;
#pragma unroll
  for (int r = 0; r < 32; ++r) {   // coordinate 32 w + r is value r % 4 of block r / 4
    const float u = y[r >> 2][r & 3];
    const float a = fabsf(u);
    wu = push_sign(wu, u);
    // bit j of the magnitude index, complemented: the XOR of the "below"
    // lane masks over k with (k + 1) divisible by 2^j (an odd count), formed
    // on the scalar unit; one push per bit
    uint64_t bx[BV - 1];
#pragma unroll
    for (int j = 0; j < BV - 1; ++j) bx[j] = 0u;
#pragma unroll
    for (int k = 0; k < KV - 1; ++k) {
      const uint64_t below = __builtin_amdgcn_ballot_w64(a < tu[k]);
#pragma unroll
      for (int j = 0; j < BV - 1; ++j)
        if (((k + 1) & ((1 << j) - 1)) == 0) bx[j] ^= below;
    }
#pragma unroll
    for (int j = 0; j < BV - 1; ++j) {
      uint64_t co;
      asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(wb[j]), "=s"(co) : "v"(wb[j]), "s"(bx[j]));
    }
  }
  const bool keep = valid && !zero;
  // words were filled oldest-bit-first: bit r sits at 31 - r
  const uint32_t sg = __builtin_bitreverse32(wu);       // 1 = negative
  uint32_t wp[BV], ow[BV];
  wp[BV - 1] = keep ? ~sg : 0u;
#pragma unroll
  for (int j = 0; j < BV - 1; ++j) wp[j] = keep ? ~(__builtin_bitreverse32(wb[j]) ^ sg) : 0u;
  vtile_pack<BV>(wp, lane, ow);
#pragma unroll
  for (int j = 0; j < BV; ++j) out.w[j] = ow[j];
  out.norm = keep ? uint32_t(f2h_bits(nu)) : 0u;
  out.g = g;
  out.n = n;
  out.valid = valid;
}

// VAL: value records (B = value bits, no sketch; norms are uint16 halves).
// PAGED: keys are the G = 1 x N rows of a [groups][T] append whose records go
// to the pool pages the page map gives (Ncap = page size); a 16-key tile then
// holds rows of up to 16 different groups.
// Keys run three workgroups per CU (at most 168 VGPRs); the paged form at
// B = 3 (page-map registers beside the extra thresholds) runs two.
template <int B, bool VAL, bool PAGED = false>
__global__ __launch_bounds__(kEnc16Threads, VAL ? 4 : (PAGED && B == 3 ? 2 : 3)) void encode128_bf16_t16_kernel(
    const uint16_t* __restrict__ keys, int64_t G, int64_t N, int64_t Ncap, int64_t pos,
    uint32_t* __restrict__ planes, void* __restrict__ norms_,
    const DevConsts* __restrict__ cst, const uint4* __restrict__ frag,
    const uint4* __restrict__ dmask, PageMap pm) {
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
    // paged rows: the page-map loads go out before the wait for the key tile
    int64_t dg = g, dn = pos + n;
    bool dv = valid;
    if constexpr (PAGED) dv = valid && page_dest(pm, n, dg, dn);
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
      // (a real branch: if-converted, the selects would run on every tile)
      asm volatile("");
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
      value_tail16<B>(y, nu2, cst, lane, g, pos + n, valid, out);
      have = true;
    } else {
      if (have) {   // the previous tile's packing runs while this tile's rotation products do
        finish16<B>(pend, out);
        store_tile16<B>(out, lane, Ncap, planes, nk);
      }
      // a wave in its vector-heavy stretch issues ahead of waves running
      // rotation products (measured 1-2% faster than equal priorities)
      __builtin_amdgcn_s_setprio(1);
      quant_sketch16<B>(y, nu2, ec, s_frag, lane, dg, dn, dv, pend);
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

template <int B, bool VAL, bool PAGED = false>
__global__ __launch_bounds__(kEncThreads, 2) void encode128_f32_kernel(
    const float* __restrict__ keys, int64_t G, int64_t N, int64_t Ncap, int64_t pos,
    uint32_t* __restrict__ planes,
    void* __restrict__ norms_, const DevConsts* __restrict__ cst,
    const uint4* __restrict__ frag, const uint32_t* __restrict__ flip, PageMap pm) {
  __shared__ uint4 s_frag[VAL ? 1 : 2048];       // [kc 8][jb 4][lane 64]
  __shared__ uint32_t s_flip[128];
  __shared__ uint32_t s_vt[VAL ? kEncWaves * 4 * 32 * 4 : 1];   // values: [wave][plane][value][word]

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
      // the wave's 32 values go out as two tiles of 16 (the second only when
      // it holds a value): plane words through LDS into the 16-lane order of
      // the tile packing
      uint32_t* st = s_vt + wave * (4 * 32 * 4);
      const uint32_t nh = value_tail<B>(x, nu2, cst, lane, valid, st);
      if (valid && h == 0) static_cast<uint16_t*>(norms_)[g * Ncap + pos + n] = uint16_t(nh);
      asm volatile("" ::: "memory");
      const int64_t n0 = int64_t(tile - gt * tpg) * 32;   // first value of the 32
      const int64_t tpg16 = (Ncap + 15) / 16;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (n0 + 16 * u >= N) break;
        uint32_t wp[B], ow[B];
#pragma unroll
        for (int p = 0; p < B; ++p) wp[p] = st[(p * 32 + 16 * u + (lane & 15)) * 4 + (lane >> 4)];
        vtile_pack<B>(wp, lane, ow);
        store_vwords<B>(ow, lane, g, tpg16, (pos + n0) / 16 + u, planes);
      }
      asm volatile("" ::: "memory");
    } else {
      TileOut out;
      int64_t dg = g, dn = pos + n;
      bool dv = valid;
      if constexpr (PAGED) dv = valid && page_dest(pm, n, dg, dn);
      encode_tail<B>(x, nu2, ec, s_frag, lane, dg, dn, dv, out);
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
  uint4 bq[4][64];           // 2 R q as fp16 hi + lo: the B operand of the S q products [step][lane]
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

// Decode attention fused into the scorer (BV > 0 below): value records of the
// same keys, the softmax scale and the per-range partial states.
struct AttnArgs {
  const uint4* vplanes;    // value codes: [G][ceil(vcap / 16)] tiles of 16 BV 16-byte units
  const uint16_t* vnorms;  // value half norms [G][vcap]
  float* part;             // per (group, query chunk, range): m[4], Z[4], A[4][128]
  float scale;
  int64_t vcap;            // value records per group (N, or a cache's capacity)
};
constexpr int kAttnPart = 8 + 4 * 128;   // m[4], Z[4], A[4][128] per (group, query chunk, range)

// LDS of the value phase, over the scorer's LDS once its tables are dead.
template <int BV>
struct AttnLds {
  // level table: entry e (a value pair's 2 BV code bits) holds the halves
  // hi, lo of the first level, then hi, lo of the second, in kCopies copies
  // side by side, lane L reading copy L % kCopies: the 8-byte reads of 32
  // lanes hit 64 different banks whatever the codes are (16 copies at 4
  // bits: 32 KB)
  static constexpr int kLutEntries = 1 << (2 * BV);
  static constexpr int kCopies = BV == 4 ? 16 : 32;
  static constexpr int kStage = BV * 256 + 8;   // words per wave: 4 of padding, a 64-key tile's codes, 4
  uint2 lut[kLutEntries * kCopies];
  uint32_t stage[16][kStage];
  // per wave: the scaled weights of the tile's keys as matrix-core A rows,
  // one word per key: row q the half hi twice, row 4 + q the half lo and 0
  uint32_t wt[16][8][64];
  uint32_t wz[64];            // zeros: the A rows 8..15
  float m[16][4], z[16][4];   // per wave: maximum of scale * logit, normaliser
};

// Largest float exponent field of the wave's non-negative values (DPP
// maxima inside each row of 16 lanes, then the four rows), wave-uniform.
__device__ __forceinline__ uint32_t wave_max_exponent(float v) {
  uint32_t m = __float_as_uint(v) >> 23;
  m = std::max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0xB1, 0xF, 0xF, false)));    // lane ^ 1
  m = std::max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0x4E, 0xF, 0xF, false)));    // lane ^ 2
  m = std::max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0x141, 0xF, 0xF, false)));   // 7 - lane in 8
  m = std::max(m, uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0x140, 0xF, 0xF, false)));   // 15 - lane in 16
  const uint32_t a = __builtin_amdgcn_readlane(m, 0), b = __builtin_amdgcn_readlane(m, 16);
  const uint32_t c = __builtin_amdgcn_readlane(m, 32), d = __builtin_amdgcn_readlane(m, 48);
  return std::max(std::max(a, b), std::max(c, d));
}

// Wave-wide maximum and sum, wave-uniform: DPP inside each row of 16 lanes
// (lane ^ 1, lane ^ 2, 7 - lane in 8, 15 - lane in 16), then the four rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_lane(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ float wave_max64(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return fmaxf(fmaxf(row_lane(v, 0), row_lane(v, 16)), fmaxf(row_lane(v, 32), row_lane(v, 48)));
}
__device__ __forceinline__ float wave_sum64(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return (row_lane(v, 0) + row_lane(v, 16)) + (row_lane(v, 32) + row_lane(v, 48));
}

// Loads of one 64-key tile of the value phase (keys from position b, their
// value records from record bv of vn / vq): the lane's logits and value
// norm (clamped to the range), the tile's value codes (BV 16-byte units per
// lane, clamped to the last tile of vq).  The bases are wave-uniform and the
// per-lane offsets 32-bit (a scalar base and one vector offset per load, no
// 64-bit address arithmetic per lane).
template <int BV>
__device__ __forceinline__ void attn_fetch(int64_t b, int64_t bv, int lane, int64_t n1,
                                           const float* const (&lrow)[4], const uint16_t* vn,
                                           const uint4* vq, int64_t vlast, u32x4 (&cv)[BV], float (&lg)[4],
                                           uint32_t& nvb) {
  const uint32_t kn = std::min(uint32_t(lane), uint32_t(std::min<int64_t>(n1 - 1 - b, 63)));
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) lg[qq] = (lrow[qq] + b)[kn];
  nvb = (vn + bv)[kn];
  const int64_t u0 = (bv >> 4) * (16 * BV);   // the tile's first 16-byte unit
  const uint4* vt = vq + u0;
  const uint32_t ul = uint32_t(std::min<int64_t>(vlast - u0, 64 * BV - 1));
#pragma unroll
  for (int j = 0; j < BV; ++j) {
    const uint4 v = vt[std::min(uint32_t(j * 64 + lane), ul)];
    cv[j] = u32x4{v.x, v.y, v.z, v.w};
  }
}

// The value records of the 64-key tile at position b (b < n1): the group's
// own (a cache of aa.vcap records per group), or, paged, those of the pool
// page the page map gives for b (pages of aa.vcap = page_size records).  ok:
// the tile has records; a tile in an invalid page reads page 0 and is
// weighed with nothing (its logits were not written either).
template <int BV, bool PAGED>
__device__ __forceinline__ void attn_fetch_tile(int64_t b, int lane, int64_t n1, int64_t g,
                                                const float* const (&lrow)[4], const AttnArgs& aa,
                                                const PageMap& pm, u32x4 (&cv)[BV], float (&lg)[4],
                                                uint32_t& nvb, bool& ok) {
  const int64_t tpg16 = (aa.vcap + 15) / 16;
  const int64_t vlast = tpg16 * 16 * BV - 1;
  if constexpr (PAGED) {
    const int32_t lpage = int32_t(b / pm.page_size);
    int32_t ph = __builtin_amdgcn_readfirstlane(pm.table[g * pm.ppg + lpage]);
    ok = ph >= 0 && ph < pm.num_pages;
    if (!ok) ph = 0;
    attn_fetch<BV>(b, b - int64_t(lpage) * pm.page_size, lane, n1, lrow, aa.vnorms + int64_t(ph) * aa.vcap,
                   aa.vplanes + int64_t(ph) * tpg16 * 16 * BV, vlast, cv, lg, nvb);
    if (!ok) nvb = 0u;
  } else {
    ok = true;
    attn_fetch<BV>(b, b, lane, n1, lrow, aa.vnorms + g * aa.vcap, aa.vplanes + g * tpg16 * 16 * BV, vlast,
                   cv, lg, nvb);
  }
}

// Value phase of the fused decode attention, after the range's logits of
// queries qc*4 .. qc*4+3 are in `logits` (written by this wave for its own
// tiles) and lmax holds this lane's largest logit per query.  Each wave
// weighs its keys with exp(scale l - M_w), M_w its own exact maximum (no
// wait for the other waves), and the workgroup merges the waves' states
// with exp(M_w - M) at the end.
// v_mse = nu~ R^T c_v, so the weighted sums stay in the rotated domain: per
// query and coordinate, sum over keys of w nu~ c_v[code].  They run on the
// matrix cores, one 16 x 16 x 32 product per 16-value tile and 16 slots: the
// B operand of lane (values 4 kg .. 4 kg + 3, slot 16 cb + n) is two entries
// of a table of level pairs indexed by the lane's two value groups in that
// slot (each level as half hi, lo); the A operand's rows 0..3 hold the
// weights' halves hi twice (against hi and lo), rows 4..7 their lo once
// (against hi), both as written to LDS per key, rows 8..15 zeros: float16
// operands, about 22 bits of every product kept.  The weights w nu~ are
// scaled by a power of 2 that keeps them under 2^14 (from the largest value
// norm the wave has seen; its sums are rescaled when that grows), so that
// the halves lose nothing to the float16 range.  The range's state goes to
// `part` and attn_combine128_kernel rotates back.
template <int BV, bool PAGED>
__device__ __forceinline__ void attn_value_phase(void* lds_raw, const float (&lmax)[4], const AttnArgs& aa,
                                                 const DevConsts* __restrict__ cst, const float* logits,
                                                 int64_t g, int qc, int Qg, int64_t N, int64_t n1,
                                                 int64_t first, int64_t ntiles, int64_t stride,
                                                 const PageMap& pm) {
  using Lds = AttnLds<BV>;
  static_assert(sizeof(Lds) <= sizeof(ScoreLds), "the value phase reuses the scorer's LDS");
  // the per-wave normaliser parts are written while other waves still read
  // the level table, their staging and their weights
  static_assert(offsetof(Lds, z) >= offsetof(Lds, wt) + sizeof(Lds::wt), "z lies past the loop's arrays");
  static_assert(offsetof(Lds, m) >= 16 * 8 * 4 * 16 * 4, "the final sums overlay only table and staging");
  Lds& sm = *reinterpret_cast<Lds*>(lds_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float* lrow[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) lrow[qq] = logits + (g * Qg + std::min(qc * 4 + qq, Qg - 1)) * N;
  // loads of tile t: the key's logits and value norm, the 64 keys' codes;
  // the first tile's go out now, over the barriers below
  u32x4 cv[BV];
  float lg[4];
  uint32_t nvb = 0;
  bool okn = false;
  if (ntiles > 0) attn_fetch_tile<BV, PAGED>(first, lane, n1, g, lrow, aa, pm, cv, lg, nvb, okn);
  // the wave's own maximum of scale * logit per query: its weights
  // exp(scale l - M) are at most 1, and the workgroup's sums merge the
  // waves' states with exp(M_w - M) at the end
  float M[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const float mw = wave_max64(lmax[qq]);
    M[qq] = qc * 4 + qq < Qg ? aa.scale * mw : 0.f;
  }
  // level table: value i of entry e has code bit p at bit 2 p + i of e; the
  // levels are read now, the entries written once the scorer's LDS is free
  constexpr int kLutPer = (Lds::kLutEntries * Lds::kCopies + kScoreThreads - 1) / kScoreThreads;
  float la[kLutPer][2];
#pragma unroll
  for (int j = 0; j < kLutPer; ++j) {
    const int e = (tid + j * kScoreThreads) / Lds::kCopies;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = 0;
#pragma unroll
      for (int p = 0; p < BV; ++p) c |= ((e >> (2 * p + i)) & 1) << p;
      la[j][i] = e < Lds::kLutEntries ? cst->vlevels[c] : 0.f;
    }
  }
  // this LDS overlays the scorer's tables: nothing is written before every
  // wave is past them (and past its logit stores)
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kLutPer; ++j) {
    const int x = tid + j * kScoreThreads;
    if (x < Lds::kLutEntries * Lds::kCopies) {
      const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(la[j][0], la[j][1]));
      const half2v e0 = {h[0], static_cast<_Float16>(la[j][0] - static_cast<float>(h[0]))};
      const half2v e1 = {h[1], static_cast<_Float16>(la[j][1] - static_cast<float>(h[1]))};
      sm.lut[x] = make_uint2(__builtin_bit_cast(uint32_t, e0), __builtin_bit_cast(uint32_t, e1));
    }
  }
  if (tid < 64) sm.wz[tid] = 0u;
  __syncthreads();
  // the weights w nu~ are scaled by 2^(140 - E), E the largest exponent
  // field of the value norms seen so far by this wave: a norm below 2^(E - 126)
  // times a weight of at most 1 stays under 2^14; when a tile raises E, the
  // sums so far are scaled down by the same power of 2 (exact)
  uint32_t erun = 103;   // the smallest non-zero half, 2^-24, has field 103
  uint32_t* stw = sm.stage[wave];
  const uint32_t* l32 = reinterpret_cast<const uint32_t*>(lds_raw);
  uint32_t* wtw = &sm.wt[wave][0][0];
  const int n = lane & 15, kg = lane >> 4;   // B: slot column n, values 4 kg .. 4 kg + 3; A: row n
  // The lane's values 4 kg .. 4 kg + 3 in slot 16 cb + n are the two groups
  // 2 kg, 2 kg + 1: 4 BV bits from bit 64 BV cb + 16 BV n + 4 BV kg of a tile.
  // BV = 3: read 8 bits up in the 32 bits (word rd, word rd + 1) >> sh, so
  // that each 6-bit index masked in place (bits 8..13) or after a shift is
  // an entry's byte offset; a field in the low 8 bits of a word takes the
  // word before it as the low half (the padding covers the first).
  int rd = 0, sh = 0;
  if constexpr (BV == 3) {
    const int bp = 48 * n + 12 * kg, d0 = bp >> 5, o = bp & 31;
    rd = o < 8 ? d0 - 1 : d0;
    sh = o < 8 ? o + 24 : o - 8;
  }
  constexpr int kEntryShift = BV == 4 ? 7 : 8;   // entry stride: kCopies x 8 bytes
  const uint32_t cofs = uint32_t(lane % Lds::kCopies) * 8u;
  const uint32_t* arow = n < 8 ? wtw + n * 64 : sm.wz;   // A rows: 0..3 hi (twice), 4..7 lo, 8..15 zero
  f32x4 acc[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zp[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t t = 0; t < ntiles; ++t) {
    const int64_t b = first + t * stride;
    const bool valid = okn && uint32_t(lane) < uint32_t(std::min<int64_t>(n1 - b, 64));
    const float nvr = h2f_bits(nvb);
    const uint32_t et = wave_max_exponent(nvr);
    if (et > erun) {
      const float down = __uint_as_float((127u - (et - erun)) << 23);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) acc[cb] *= down;
      erun = et;
    }
    const float nv = nvr * __uint_as_float((267u - erun) << 23);
    float wq[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float e = (valid && qc * 4 + qq < Qg) ? __expf(fmaf(aa.scale, lg[qq], -M[qq])) : 0.f;
      zp[qq] += e;
      wq[qq] = e * nv;
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const half2v hh = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(wq[qq], wq[qq]));
      wtw[qq * 64 + lane] = __builtin_bit_cast(uint32_t, hh);
      wtw[(4 + qq) * 64 + lane] =
          uint32_t(__builtin_bit_cast(uint16_t, static_cast<_Float16>(wq[qq] - static_cast<float>(hh[0]))));
    }
#pragma unroll
    for (int j = 0; j < BV; ++j) reinterpret_cast<u32x4*>(stw + 4)[j * 64 + lane] = cv[j];
    // the next tile's loads fly over this tile's products
    attn_fetch_tile<BV, PAGED>(first + std::min<int64_t>(t + 1, ntiles - 1) * stride, lane, n1, g, lrow, aa,
                               pm, cv, lg, nvb, okn);
    // in steps of four products (16-value tile u = k / 2, slots 16 cb + n for
    // cb = 4 (k % 2) .. + 3): the four groups' fields, their table entries,
    // then the products; the next step's fields are requested before this
    // step's products, so the two LDS round trips of a step overlap the
    // previous step's products
    uint32_t fw[4][2];   // BV = 3: the word pair holding the lane's group; else the group itself
    auto read_fields = [&](int k) __attribute__((always_inline)) {
      const int u = k >> 1;
      // BV = 3: one address register per step, the slot blocks at immediate offsets
      // (an index from the start of the LDS, signed: the slot offsets fold into the reads)
      int fi = int(stw - l32) + 4 + u * 192 + 96 * (k & 1) + rd;
      if constexpr (BV == 3) asm volatile("" : "+v"(fi));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cb = 4 * (k & 1) + c;
        if constexpr (BV == 3) {
          fw[c][0] = l32[fi + 24 * c];
          fw[c][1] = l32[fi + 24 * c + 1];
        } else if constexpr (BV == 2) {
          fw[c][0] = reinterpret_cast<const uint8_t*>(stw + 4)[u * 512 + 4 * (16 * cb + n) + kg];
        } else {
          fw[c][0] = reinterpret_cast<const uint16_t*>(stw + 4)[u * 512 + 4 * (16 * cb + n) + kg];
        }
      }
    };
    read_fields(0);
    half8 A;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int u = k >> 1;
      u32x4 bv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t o0, o1;   // byte offsets of the two pairs' entries
        if constexpr (BV == 3) {
          const uint32_t v = __builtin_amdgcn_alignbit(fw[c][1], fw[c][0], sh);
          o0 = (v & 0x3F00u) | cofs;
          o1 = ((v >> 6) & 0x3F00u) | cofs;
        } else if constexpr (BV == 2) {
          o0 = ((fw[c][0] & 0xFu) << kEntryShift) | cofs;
          o1 = ((fw[c][0] >> 4) << kEntryShift) | cofs;
        } else {
          o0 = ((fw[c][0] & 0xFFu) << kEntryShift) | cofs;
          o1 = ((fw[c][0] >> 8) << kEntryShift) | cofs;
        }
        const char* lb = reinterpret_cast<const char*>(sm.lut);
        const uint2 e0 = *reinterpret_cast<const uint2*>(lb + o0);
        const uint2 e1 = *reinterpret_cast<const uint2*>(lb + o1);
        // K order of the lane's 8 products: hi(v0) lo(v0) hi(v1) lo(v1) hi(v2)
        // lo(v2) hi(v3) lo(v3) for its values v0..v3 = 4 kg .. 4 kg + 3
        bv[c] = u32x4{e0.x, e0.y, e1.x, e1.y};
      }
      if ((k & 1) == 0) {
        // the same K order: row q < 4 holds w_hi(v) twice per value (against
        // the level's hi and lo), row 4 + q w_lo(v) and 0 (hi levels only)
        const u32x4 av = *reinterpret_cast<const u32x4*>(arow + 16 * u + 4 * kg);
        A = __builtin_bit_cast(half8, av);
      }
      if (k < 7) read_fields(k + 1);
      __builtin_amdgcn_sched_barrier(0);   // the reads above go out before the products
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cb = 4 * (k & 1) + c;
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8, bv[c]), acc[cb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const float z = wave_sum64(zp[qq]);
    if (lane == 0) {
      sm.z[wave][qq] = z;
      sm.m[wave][qq] = M[qq];
    }
  }
  // rows 0..3 (lanes 0..15) and 4..7 (lanes 16..31) of every block: the sums
  // against the weights' hi and lo halves
  const float unscale = __uint_as_float((erun - 13u) << 23);   // 2^(E - 140)
  float tot[8][4];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      tot[cb][i] = unscale * (acc[cb][i] +
                              __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(acc[cb][i]), 0x401F)));
  __syncthreads();   // every wave is done with the level table and its staging
  float* red = reinterpret_cast<float*>(lds_raw);   // [wave][cb][query][column]: 32 KB
  if (lane < 16) {
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((wave * 8 + cb) * 4 + i) * 16 + lane] = tot[cb][i];
  }
  __syncthreads();
  float* out = aa.part + ((g * gridDim.y + qc) * gridDim.z + blockIdx.z) * kAttnPart;
  if (tid < 516) {
    const int qq = tid < 512 ? tid >> 7 : tid - 512;
    float mm = sm.m[0][qq];
    for (int w = 1; w < 16; ++w) mm = fmaxf(mm, sm.m[w][qq]);
    // waves without keys hold M = -inf and no sums
    auto f = [&](int w) { const float mw = sm.m[w][qq]; return mw == -INFINITY ? 0.f : __expf(mw - mm); };
    if (tid < 512) {
      const int s = tid & 127, cb = s >> 4, col = s & 15;
      float a = 0.f;
      for (int w = 0; w < 16; ++w) a = fmaf(f(w), red[((w * 8 + cb) * 4 + qq) * 16 + col], a);
      const int c = 32 * (s >> 5) + 16 * (s & 1) + ((s & 31) >> 1);   // the coordinate of slot s
      out[8 + qq * 128 + c] = a;
    } else {
      float z = 0.f;
      for (int w = 0; w < 16; ++w) z = fmaf(f(w), sm.z[w][qq], z);
      out[qq] = mm;
      out[4 + qq] = z;
    }
  }
}

// PAGED: records of group g live in the pool pages of the page map
// (planes/norms are the pool's), group g has lens[g] of them (at most
// ppg * page_size), and N is the logit row length; each 64-key tile lies in
// one page.
// BV > 0: decode attention over value records of BV bits (see
// attn_value_phase): logits go to `logits` through the caches and the
// range's partial state to aa.part.
template <int B, bool QBF16, bool PAGED = false, int BV = 0>
__global__ __launch_bounds__(kScoreThreads, 1) void score128_kernel(
    const void* __restrict__ q, const uint4* __restrict__ planes, const uint32_t* __restrict__ norms,
    int64_t N, int64_t Ncap, int Qg, int din, int64_t chunk, float* __restrict__ logits,
    const DevConsts* __restrict__ cst, const uint4* __restrict__ Sfrag, PageMap pm, AttnArgs aa) {
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
  int64_t n1 = std::min<int64_t>(N, n0 + chunk);   // n0 < n1: the host sizes the grid so
  if constexpr (PAGED) {   // group lengths live in device memory: ranges past them have no work
    n1 = std::min<int64_t>(n1, std::min<int64_t>(pm.lens[g], int64_t(pm.ppg) * pm.page_size));
    if (n1 <= n0) {
      if constexpr (BV > 0) {   // attention: the range's state is empty (maximum -inf, no sums)
        float* st = aa.part + ((g * gridDim.y + qc) * gridDim.z + blockIdx.z) * kAttnPart;
        if (tid < kAttnPart) st[tid] = tid < 4 ? -INFINITY : 0.f;
      }
      return;
    }
  }
  // keys [0, N) of a cache holding Ncap records per group; logits [G][Qg][N]
  const uint4* pg = planes + g * P * Ncap;
  const uint32_t* ng = norms + g * Ncap;

  // ---- loads: the S q products' A operands, the R q input, the first key
  // tile.  S q = (S R^T)(R q): the scorer needs R q anyway.  Waves 0..7 form
  // the sixteen sketch rows of block `wave` on the matrix cores from -S R^T
  // in fp16 (exact), in the key encoder's operand order: step t's A operand
  // of row block b at [t][b][lane], matrix row m of block b = sketch row
  // 32 (m / 4) + 4 b + m % 4, K index k of step t = coordinate
  // 32 (k / 8) + 8 t + k % 8.
  uint4 sa[4];
  if (wave < 8) {
#pragma unroll
    for (int t = 0; t < 4; ++t) sa[t] = Sfrag[(t * 8 + wave) * 64 + lane];
  }
  // query rows hold din <= 128 elements (an argument: read from the constant
  // block, it would put an L2 round trip before the query loads); coordinates
  // at or past din are zero padding (the loads are clamped to the row and
  // their values dropped)
  // (waves 0..3 rotate query wave; the others load nothing they would wait for
  // before the first barrier)
  uint32_t u0 = 0, u1 = 0;   // raw bits of the R q input
  uint32_t dn0 = 0, dn1 = 0;
  if (wave < 4) {
    const int qr = std::min(qc * 4 + wave, Qg - 1);
    const int64_t at = (g * Qg + qr) * din;
    const int i0 = std::min(lane, din - 1), i1 = std::min(lane + 64, din - 1);
    if constexpr (QBF16) {
      u0 = static_cast<const uint16_t*>(q)[at + i0];
      u1 = static_cast<const uint16_t*>(q)[at + i1];
    } else {
      u0 = static_cast<const uint32_t*>(q)[at + i0];
      u1 = static_cast<const uint32_t*>(q)[at + i1];
    }
    dn0 = cst->dneg[lane >> 5];
    dn1 = cst->dneg[2 + (lane >> 5)];
  }
  // codebook scalars, read with the setup loads: read where they are used,
  // after the key tiles, they wait behind the whole chip's tile traffic in L2
  float isd = cst->inv_sqrt_d, qs = cst->qjl_scale, asum = cst->alpha_sum;
  float a0 = cst->alpha[0], a1 = cst->alpha[1], a2 = cst->alpha[2], a3 = cst->alpha[3];
  // wave-uniform plane bases + 32-bit lane offsets (key index < 2^28): the
  // loads take the scalar-base form and need no 64-bit address arithmetic
  auto load_tile = [&](int64_t b, uint4 (&wv)[P], uint32_t& nv, bool& ok) {
    uint32_t n = uint32_t(std::min<int64_t>(b + lane, n1 - 1));
    const uint4* pt = pg;
    const uint32_t* nt = ng;
    int64_t stride = Ncap;
    ok = true;
    if constexpr (PAGED) {
      // the tile (or, past the range, the clamped last record) lies in one page
      const int32_t lpage = int32_t(std::min<int64_t>(b, n1 - 1) / pm.page_size);
      int32_t ph = __builtin_amdgcn_readfirstlane(pm.table[g * pm.ppg + lpage]);
      ok = ph >= 0 && ph < pm.num_pages;
      if (!ok) ph = 0;   // read a valid page, store nothing
      pt = planes + int64_t(ph) * P * pm.page_size;
      nt = norms + int64_t(ph) * pm.page_size;
      n -= uint32_t(lpage) * uint32_t(pm.page_size);
      stride = pm.page_size;
    }
    const uint32_t off16 = n * 16u, off4 = n * 4u;   // byte offsets, < 2^32
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(pt + p * stride) + off16));
      wv[p] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    nv = __builtin_nontemporal_load(
        reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(nt) + off4));
  };
  const int64_t first = n0 + int64_t(wave) * 64;
  uint4 w[D][P];
  uint32_t nr[D];
  bool okt[D];
  // Every wave issues the loads above before any wave issues a key tile, and
  // only one tile goes out before the setup (the second later, see below).
  // A CU takes only so many loads in flight: past that, a wave stalls where
  // it issues the next one until earlier data comes back, and the setup's
  // barriers wait for the slowest wave (measured at this scorer's launch on
  // the Llama-3.1-8B decode shape: two tiles per wave up front left the
  // tables ready after ~13,000 cycles, one after ~8,000).  A bare barrier,
  // with no wait for the loads themselves.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  load_tile(first, w[0], nr[0], okt[0]);
  // B operand columns 8..15 of the S q products carry no query: zeros
  if (tid >= 256 && tid < 384) {
    const int i = tid - 256, t = i >> 5, kg = (i >> 3) & 3, c = 8 + (i & 7);
    sm.bq[t][16 * kg + c] = make_uint4(0u, 0u, 0u, 0u);
  }

  // ---- R q = H D q / sqrt(d)
  if (wave < 4) {
    asm volatile("" : "+v"(u0), "+v"(u1), "+v"(dn0), "+v"(dn1), "+s"(isd));
    const float v0 = lane < din ? __uint_as_float(QBF16 ? u0 << 16 : u0) : 0.f;
    const float v1 = lane + 64 < din ? __uint_as_float(QBF16 ? u1 << 16 : u1) : 0.f;
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
    const float x0 = 2.0f * (y0 * isd), x1 = 2.0f * (y1 * isd);   // coordinates lane, lane + 64
    xf[((lane & 7) * 16 + (lane >> 3)) * 4 + wave] = x0;
    xf[((lane & 7) * 16 + 8 + (lane >> 3)) * 4 + wave] = x1;
    // B operand of the S q products: column 2 q + h of K row k holds query
    // q's coordinate 32 (k / 8) + 8 t + k % 8 as fp16 hi (h = 0) and
    // 2^11 x (x - hi) (h = 1, exact in float32 before its rounding)
    uint16_t* bq16 = reinterpret_cast<uint16_t*>(&sm.bq[0][0]);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const float x = h2 ? x1 : x0;
      const int c = lane + 64 * h2;
      const _Float16 hi = static_cast<_Float16>(x);
      const _Float16 lo = static_cast<_Float16>((x - static_cast<float>(hi)) * 2048.0f);
      const int base = (((c >> 3) & 3) * 64 + 16 * (c >> 5) + 2 * wave) * 8 + (c & 7);
      bq16[base] = __builtin_bit_cast(uint16_t, hi);
      bq16[base + 8] = __builtin_bit_cast(uint16_t, lo);
    }
  }
  __syncthreads();
  asm volatile("" : "+s"(qs), "+s"(asum), "+s"(a0), "+s"(a1), "+s"(a2), "+s"(a3));
  // ---- byte subset-sum tables T[ty][idx][pos] = sum over the set bits t of
  // idx of 2 X_ty[8 pos + t], thread (pos, h) writing entries idx = 4 h + j,
  // j = 0..3.  Waves 0..7 first form 2 S q on the matrix cores, then join the
  // other waves on the R q tables; then all build the S q tables.  The
  // full-byte entries (idx 255) of every position give the sums.
  auto build_tables = [&](int ty) {
    const int pos = tid & 15, h = tid >> 4;
    f32x4 xv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) xv[t] = sm.x[ty][t][pos];
    f32x4 bs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 2; t < 8; ++t) {
      const float on = float((h >> (t - 2)) & 1);
      bs[0] = fmaf(on, xv[t][0], bs[0]);
      bs[1] = fmaf(on, xv[t][1], bs[1]);
      bs[2] = fmaf(on, xv[t][2], bs[2]);
      bs[3] = fmaf(on, xv[t][3], bs[3]);
    }
    f32x4 e[4];
    e[0] = bs;
    e[1] = bs + xv[0];
    e[2] = bs + xv[1];
    e[3] = e[2] + xv[0];
#pragma unroll
    for (int j = 0; j < 4; ++j) sm.tab[(ty * 256 + h * 4 + j) * 16 + pos] = e[j];
    if (wave == 15) {   // lanes 48..63 hold idx 255 of positions 0..15
      f32x4 t = e[3];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        t[c] += lane_xor<1>(t[c]);
        t[c] += lane_xor<2>(t[c]);
        t[c] += lane_xor<4>(t[c]);
        t[c] += lane_xor<8>(t[c]);
      }
      if (lane == 48) sm.sum[ty] = t;
    }
  };
  if (wave < 8) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 bv = sm.bq[t][lane];
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, sa[t]),
                                                   __builtin_bit_cast(half8, bv), acc, 0, 0, 0);
    }
    // D[m][col] (m = 4 (lane / 16) + i, col = lane % 16) = -(2 S q) of sketch
    // row 32 (lane / 16) + 4 wave + i for query col / 2, hi (even col) or
    // 2^11 x lo part (odd col, the next lane's)
    float lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lo[i] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc[i]), 0x101, 0xF, 0xF, false));
    if ((lane & 1) == 0 && (lane & 15) < 8) {
      float* xf1 = reinterpret_cast<float*>(&sm.x[1][0][0]);
      const int qq = (lane & 15) >> 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 32 * (lane >> 4) + 4 * wave + i;
        xf1[((j & 7) * 16 + (j >> 3)) * 4 + qq] = -fmaf(lo[i], 1.0f / 2048.0f, acc[i]);
      }
    }
  }
  build_tables(0);
  __syncthreads();
  // The second tile of each wave: at b = 2 here, at b = 3 and 4 after the
  // tables (measured on the Llama-3.1-8B decode shape: 15.6 against 16.0 us
  // at b = 2, 18.6 against 18.9 at b = 3, 25.8 against 27.6 at b = 4; a wave
  // that issues it here stalls until the first tiles free their slots)
  static_assert(D == 2, "the prologue loads one tile, this the second");
  if constexpr (B == 1) load_tile(first + kStride, w[1], nr[1], okt[1]);
  build_tables(1);
  __syncthreads();
  if constexpr (B != 1) load_tile(first + kStride, w[1], nr[1], okt[1]);

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

  float lmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // BV > 0: largest logit per query
  auto score_tile = [&](const uint4 (&wt)[P], uint32_t nrm, int64_t b, bool ok) {
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
    const bool in_range = b + lane < n1 && ok;
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
      const float v = fmaf(nu, mse, rs * (ss[qq] - acc[B][qq]));
      float* dst = reinterpret_cast<float*>(reinterpret_cast<char*>(lrow[qq]) + off4);
      if (in_range && qh < Qg) {
        if constexpr (BV > 0) {   // read back by the value phase: kept in the caches
          *dst = v;
          lmax[qq] = fmaxf(lmax[qq], v);
        } else {                  // streamed output: no reuse, written past the caches
          __builtin_nontemporal_store(v, dst);
        }
      }
    }
  };

  // tiles t = 0, 1, ... of this wave start at first + t * kStride; tile t
  // sits in slot t % D and its slot is refilled with tile t + D right after
  const int64_t ntiles = first < n1 ? (n1 - first + kStride - 1) / kStride : 0;
  for (int64_t t0 = 0; t0 < ntiles; t0 += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      if (t0 + k < ntiles) score_tile(w[k], nr[k], first + (t0 + k) * kStride, okt[k]);
      load_tile(first + (t0 + k + D) * kStride, w[k], nr[k], okt[k]);
    }
  }
  // the refills past the range are never used: let them land before the wave ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (BV > 0)
    attn_value_phase<BV, PAGED>(&sm, lmax, aa, cst, logits, g, qc, Qg, N, n1, first, ntiles, kStride, pm);
}

// ============================================================== append, few rows, d = 128
// Latency path of the paged append: one key per workgroup of four waves.
// Every wave rotates and quantises the whole key (lane L: coordinates L and
// L + 64; a float32 butterfly, stride 64 inside the lane with +0 so that no
// -0 survives, strides 1..32 across lanes; every bit-plane word comes from a
// wave ballot: bit L of the ballot over coordinate L or L + 64 is bit L % 32
// of word L / 32 or 2 + L / 32, the natural order), then forms the sketch
// sums S r of rows L and L + 64 over its own quarter of the coordinates in
// float32 from the exact float16 rows of S R^T; wave 0 adds the four
// quarters in a fixed order and stores the record.  A key's chain is the
// load, the butterfly and 64 products per lane (one wave would take 256).
// Same rules as the tile encoders; the float32 sums differ from theirs only
// in rounding.
constexpr int kAppendThreads = 256;
constexpr int kAppendWaves = kAppendThreads / 64;

// sum over the 64 lanes (DPP, swizzle and a half swap: no LDS round trips)
__device__ __forceinline__ float wave_sum64_fast(float v) {
  v += lane_xor<1>(v);
  v += lane_xor<2>(v);
  v += lane_xor<4>(v);
  v += lane_xor<8>(v);
  v += lane_xor<16>(v);
  return xor32_sum(v);
}

template <int B, bool BF16>
__global__ __launch_bounds__(kAppendThreads) void append_rows128_kernel(
    const void* __restrict__ keys, int64_t rows, uint32_t* __restrict__ planes,
    uint32_t* __restrict__ norms, const DevConsts* __restrict__ cst, const uint4* __restrict__ Sh,
    PageMap pm) {
  constexpr int K = 1 << (B - 1);   // levels on the positive half
  constexpr int P = B + 1;
  __shared__ float s_e[kAppendWaves][128];   // per-wave residual, coordinate order
  __shared__ float2 s_p[kAppendWaves][64];   // per-wave partial sketch sums (rows L, L + 64)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r = blockIdx.x;   // one key per workgroup (the grid has exactly `rows` of them)
  // S R^T[row][16 s + m], rows L and L + 64, segments s = 2 wave, 2 wave + 1
  // (coordinates [32 wave, 32 wave + 32)), as float16 pairs
  uint4 sh[2][2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      const uint4* sp = Sh + (size_t(2 * wave + sg) * 128 + lane + 64 * j) * 2;
      sh[j][sg][0] = sp[0];
      sh[j][sg][1] = sp[1];
    }
  int64_t dg = 0, dn = 0;
  bool ok = false;
  if (wave == 0) {
    if (pm.table) {
      ok = page_dest(pm, r, dg, dn);
    } else {
      dg = r / pm.T;
      dn = pm.base + (r - dg * pm.T);
      ok = true;
    }
  }
  const int din = int(cst->din);
  float a, b;
  if constexpr (BF16) {
    const uint16_t* row = static_cast<const uint16_t*>(keys) + r * din;
    a = lane < din ? __uint_as_float(uint32_t(row[lane]) << 16) : 0.f;
    b = lane + 64 < din ? __uint_as_float(uint32_t(row[lane + 64]) << 16) : 0.f;
  } else {
    const float* row = static_cast<const float*>(keys) + r * din;
    a = lane < din ? row[lane] : 0.f;
    b = lane + 64 < din ? row[lane + 64] : 0.f;
  }
  const float nu2 = wave_sum64_fast(fmaf(a, a, b * b));
  const float fa = ((cst->dneg[lane >> 5] >> (lane & 31)) & 1u) ? -a : a;
  const float fb = ((cst->dneg[2 + (lane >> 5)] >> (lane & 31)) & 1u) ? -b : b;
  float u0 = (fa + fb) + 0.0f, u1 = (fa - fb) + 0.0f;
  u0 = butterfly_lane<1>(u0, lane & 1);   u1 = butterfly_lane<1>(u1, lane & 1);
  u0 = butterfly_lane<2>(u0, lane & 2);   u1 = butterfly_lane<2>(u1, lane & 2);
  u0 = butterfly_lane<4>(u0, lane & 4);   u1 = butterfly_lane<4>(u1, lane & 4);
  u0 = butterfly_lane<8>(u0, lane & 8);   u1 = butterfly_lane<8>(u1, lane & 8);
  u0 = butterfly_lane<16>(u0, lane & 16); u1 = butterfly_lane<16>(u1, lane & 16);
  u0 = butterfly_lane32(u0, lane & 32);   u1 = butterfly_lane32(u1, lane & 32);

  const float nu = __builtin_amdgcn_sqrtf(nu2);
  const bool zero = !(nu >= 1e-10f);
  const float nsd = nu * cst->sqrt_d;                                    // u = y nu sqrt(d)
  const float gsc = zero ? 0.f : kResidualScale * __builtin_amdgcn_rcpf(nsd);   // u -> 2^12 y
  uint64_t neg[2], below[2][K > 1 ? K - 1 : 1];
  float rho2 = 0.f;
  float* sr = s_e[wave];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float u = h ? u1 : u0, au = fabsf(u);
    neg[h] = __builtin_amdgcn_ballot_w64(u < 0.f);
    float mag = cst->cpos_s[0];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
      const bool bl = au < cst->tpos[k] * nsd;
      below[h][k] = __builtin_amdgcn_ballot_w64(bl);
      mag = bl ? mag : cst->cpos_s[k + 1];
    }
    const float e = zero ? 0.f : fmaf(u, gsc, -copysignf(mag, u));    // 2^12 (y - c[code])
    rho2 = fmaf(e, e, rho2);
    sr[lane + 64 * h] = e;
  }
  rho2 = wave_sum64_fast(rho2);
  // partial p_j = sum over this wave's 32 coordinates of (S R^T)_j,c r_c for
  // rows j = L and L + 64, two chains per row (sign only: any positive scale)
  float p0a = 0.f, p0b = 0.f, p1a = 0.f, p1b = 0.f;
  const f32x4* sr4 = reinterpret_cast<const f32x4*>(sr) + 8 * wave;   // coordinates 32 wave ..
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const f32x4 rv = sr4[4 * sg + c4];   // coordinates 32 wave + 16 sg + 4 c4 .. + 3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * c4 + i;
        const uint4 w0 = sh[0][sg][m >> 3], w1 = sh[1][sg][m >> 3];
        const uint32_t x0 = (m & 7) < 2 ? w0.x : (m & 7) < 4 ? w0.y : (m & 7) < 6 ? w0.z : w0.w;
        const uint32_t x1 = (m & 7) < 2 ? w1.x : (m & 7) < 4 ? w1.y : (m & 7) < 6 ? w1.z : w1.w;
        if (i & 1) {
          p0b = fmaf(h2f_bits(x0 >> (16 * (m & 1))), rv[i], p0b);
          p1b = fmaf(h2f_bits(x1 >> (16 * (m & 1))), rv[i], p1b);
        } else {
          p0a = fmaf(h2f_bits(x0 >> (16 * (m & 1))), rv[i], p0a);
          p1a = fmaf(h2f_bits(x1 >> (16 * (m & 1))), rv[i], p1a);
        }
      }
    }
  }
  s_p[wave][lane] = make_float2(p0a + p0b, p1a + p1b);
  __syncthreads();
  if (wave != 0) return;   // no barrier follows
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int q = 0; q < kAppendWaves; ++q) {
    const float2 pq = s_p[q][lane];
    p0 += pq.x;
    p1 += pq.y;
  }
  const float rho = zero ? 0.f : __builtin_amdgcn_sqrtf(rho2) * (nu * (1.0f / kResidualScale));
  const uint64_t sg0 = __builtin_amdgcn_ballot_w64(p0 < 0.f), sg1 = __builtin_amdgcn_ballot_w64(p1 < 0.f);
  if (!ok) return;
  const bool keep = !zero, keep_s = keep && rho2 > 0.f;
  // plane p: ~neg is the top code bit; lower bits XOR the "below" masks (as the tile encoders)
  uint64_t pw[2][P - 1];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (B == 1) {
      pw[h][0] = ~neg[h];
    } else if constexpr (B == 2) {
      pw[h][1] = ~neg[h];
      pw[h][0] = ~(neg[h] ^ below[h][0]);
    } else {
      pw[h][2] = ~neg[h];
      pw[h][1] = ~(neg[h] ^ below[h][1]);
      pw[h][0] = ~(neg[h] ^ below[h][0] ^ below[h][1] ^ below[h][2]);
    }
  }
  uint4* rec = reinterpret_cast<uint4*>(planes) + dg * P * int64_t(pm.page_size) + dn;
  if (lane < P - 1) {
    uint64_t lo = pw[0][0], hi = pw[1][0];
#pragma unroll
    for (int p = 1; p < P - 1; ++p)
      if (lane == p) { lo = pw[0][p]; hi = pw[1][p]; }
    rec[int64_t(lane) * pm.page_size] = keep ? make_uint4(uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi),
                                                          uint32_t(hi >> 32))
                                             : make_uint4(0u, 0u, 0u, 0u);
  } else if (lane == P - 1) {
    rec[int64_t(P - 1) * pm.page_size] =
        keep_s ? make_uint4(uint32_t(sg0), uint32_t(sg0 >> 32), uint32_t(sg1), uint32_t(sg1 >> 32))
               : make_uint4(0u, 0u, 0u, 0u);
  } else if (lane == P) {
    norms[dg * int64_t(pm.page_size) + dn] =
        keep ? (uint32_t(f2h_bits(nu)) | (uint32_t(f2h_bits(rho)) << 16)) : 0u;
  }
}

// ============================================================== decode, d = 128
// One wave per key (grid-stride over keys): lane L reconstructs coordinates
// L and L + 64 of nu~ D H c[code] / sqrt(d)  (= nu~ R^T c[code]).

template <int B, bool BF16OUT>
__global__ __launch_bounds__(256) void decode128_kernel(const uint32_t* __restrict__ planes,
                                                         const uint32_t* __restrict__ norms,
                                                         int64_t G, int64_t N, void* __restrict__ out,
                                                         const DevConsts* __restrict__ cst) {
  constexpr int P = B + 1;
  const int lane = threadIdx.x & 63;
  const int64_t stride = int64_t(gridDim.x) * 4;
  for (int64_t key = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6); key < G * N; key += stride) {
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
// The scorer (score128_kernel with BV > 0) computes each key range's logits,
// maximum m, normaliser Z = sum exp(scale l - m) and A; the combine below
// merges the ranges (flash-decoding rescale by exp(m_s - M)).

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
  // the codebook scalars are requested with the ranges' states
  const float sc = cst->inv_sqrt_d;
  const uint32_t dn0 = cst->dneg[lane >> 5], dn1 = cst->dneg[2 + (lane >> 5)];
  const int din = int(cst->din);   // output rows keep the input coordinates only
  float M = -INFINITY, Z = 0.f, a0 = 0.f, a1 = 0.f;
  if (splits <= 8) {   // one pass: every range's state in registers
    float mv[8], zv[8], x0[8], x1[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < splits) {
        const float* ps = base + s * kAttnPart;
        mv[s] = ps[q];
        zv[s] = ps[4 + q];
        x0[s] = ps[8 + q * 128 + lane];
        x1[s] = ps[8 + q * 128 + 64 + lane];
        M = fmaxf(M, mv[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < splits) {
        const float f = mv[s] == -INFINITY ? 0.f : __expf(mv[s] - M);   // a range without keys
        Z = fmaf(f, zv[s], Z);
        a0 = fmaf(f, x0[s], a0);
        a1 = fmaf(f, x1[s], a1);
      }
    }
  } else {
#pragma unroll 8
    for (int s = 0; s < splits; ++s) M = fmaxf(M, base[s * kAttnPart + q]);
#pragma unroll 8
    for (int s = 0; s < splits; ++s) {
      const float* ps = base + s * kAttnPart;
      const float f = ps[q] == -INFINITY ? 0.f : __expf(ps[q] - M);
      Z = fmaf(f, ps[4 + q], Z);
      a0 = fmaf(f, ps[8 + q * 128 + lane], a0);
      a1 = fmaf(f, ps[8 + q * 128 + 64 + lane], a1);
    }
  }
  const float inv = Z > 0.f ? 1.0f / Z : 0.f;   // no keys at all (a paged group of length 0): zeros
  float y0 = a0 * inv + a1 * inv, y1 = a0 * inv - a1 * inv;
  y0 = butterfly_lane<1>(y0, lane & 1);   y1 = butterfly_lane<1>(y1, lane & 1);
  y0 = butterfly_lane<2>(y0, lane & 2);   y1 = butterfly_lane<2>(y1, lane & 2);
  y0 = butterfly_lane<4>(y0, lane & 4);   y1 = butterfly_lane<4>(y1, lane & 4);
  y0 = butterfly_lane<8>(y0, lane & 8);   y1 = butterfly_lane<8>(y1, lane & 8);
  y0 = butterfly_lane<16>(y0, lane & 16); y1 = butterfly_lane<16>(y1, lane & 16);
  y0 = butterfly_lane32(y0, lane & 32);   y1 = butterfly_lane32(y1, lane & 32);
  const uint32_t f0 = (dn0 >> (lane & 31)) & 1u;
  const uint32_t f1 = (dn1 >> (lane & 31)) & 1u;
  float* o = out + gh * din;
  if (lane < din) o[lane] = (f0 ? -y0 : y0) * sc;
  if (64 + lane < din) o[64 + lane] = (f1 ? -y1 : y1) * sc;
}

// ============================================================== value append, d = 128
// Latency path of the write-time value append: one value per wave.  The wave
// rotates the value (the float32 butterfly of the key append: lane L holds
// coordinates L and L + 64), forms each coordinate's level index by the
// value encoders' rules (compares of |u| against t nu sqrt(d), stored bit j =
// bit j of the magnitude index XOR the sign, the top bit the complement of
// the sign) and writes it into the value's 16-value tile bit by bit with
// atomic OR / AND: the tile's other values are not touched.  Input row r
// goes to record n of group (or pool page) g of a buffer of Ncap records per
// group.
template <int BV, bool BF16>
__device__ __forceinline__ void append_value128(const void* __restrict__ values, int64_t r, int64_t g,
                                                int64_t n, int64_t Ncap, int lane,
                                                uint32_t* __restrict__ codes, uint16_t* __restrict__ norms,
                                                const DevConsts* __restrict__ cst) {
  constexpr int KV = 1 << (BV - 1);   // levels on the positive half
  const int din = int(cst->din);
  float a, b;
  if constexpr (BF16) {
    const uint16_t* row = static_cast<const uint16_t*>(values) + r * din;
    a = lane < din ? __uint_as_float(uint32_t(row[lane]) << 16) : 0.f;
    b = lane + 64 < din ? __uint_as_float(uint32_t(row[lane + 64]) << 16) : 0.f;
  } else {
    const float* row = static_cast<const float*>(values) + r * din;
    a = lane < din ? row[lane] : 0.f;
    b = lane + 64 < din ? row[lane + 64] : 0.f;
  }
  const float nu2 = wave_sum64_fast(fmaf(a, a, b * b));
  const float fa = ((cst->dneg[lane >> 5] >> (lane & 31)) & 1u) ? -a : a;
  const float fb = ((cst->dneg[2 + (lane >> 5)] >> (lane & 31)) & 1u) ? -b : b;
  // the first stage adds +0: no -0 survives, so u < 0 is the sign bit
  float u0 = (fa + fb) + 0.0f, u1 = (fa - fb) + 0.0f;
  u0 = butterfly_lane<1>(u0, lane & 1);   u1 = butterfly_lane<1>(u1, lane & 1);
  u0 = butterfly_lane<2>(u0, lane & 2);   u1 = butterfly_lane<2>(u1, lane & 2);
  u0 = butterfly_lane<4>(u0, lane & 4);   u1 = butterfly_lane<4>(u1, lane & 4);
  u0 = butterfly_lane<8>(u0, lane & 8);   u1 = butterfly_lane<8>(u1, lane & 8);
  u0 = butterfly_lane<16>(u0, lane & 16); u1 = butterfly_lane<16>(u1, lane & 16);
  u0 = butterfly_lane32(u0, lane & 32);   u1 = butterfly_lane32(u1, lane & 32);
  const float nu = __builtin_amdgcn_sqrtf(nu2);
  const bool zero = !(nu >= 1e-10f);
  const float nsd = nu * cst->sqrt_d;
  // the value's tile; value v of the tile is i = v % 2 of group q = v / 2
  uint32_t* tw = codes + ((g * ((Ncap + 15) / 16) + (n >> 4)) * 64) * BV;
  const int v = int(n & 15), q = v >> 1, i = v & 1;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = lane + 64 * h;
    const float u = h ? u1 : u0, au = fabsf(u);
    int m = 0;   // magnitude index: thresholds at or below |u|
#pragma unroll
    for (int k = 0; k < KV - 1; ++k) m += au < cst->vtpos[k] * nsd ? 0 : 1;
    const bool neg = u < 0.f;
    const int code = zero ? 0 : (((m ^ (neg ? KV - 1 : 0)) & (KV - 1)) | (neg ? 0 : KV));
    const int slot = 32 * (c >> 5) + 2 * (c & 15) + ((c >> 4) & 1);   // slot of coordinate c
    const int bit0 = 16 * BV * slot + 2 * BV * q + i;                   // plane p at bit0 + 2 p
#pragma unroll
    for (int p = 0; p < BV; ++p) {
      const int bit = bit0 + 2 * p;
      uint32_t* w = tw + (bit >> 5);
      const uint32_t mask = 1u << (bit & 31);
      if ((code >> p) & 1) atomicOr(w, mask);
      else atomicAnd(w, ~mask);
    }
  }
  if (lane == 0) norms[g * Ncap + n] = zero ? uint16_t(0) : f2h_bits(nu);
}

// PAGED: row r of the [G][T] append goes to the pool page and slot the page
// map gives (pages of pm.page_size records; rows without a valid page are
// not written); else to record pos + r % T of group r / T of a cache of Ncap
// records per group.
template <int BV, bool BF16, bool PAGED>
__global__ __launch_bounds__(256) void append_values128_kernel(
    const void* __restrict__ values, int64_t G, int64_t T, int64_t Ncap, int64_t pos,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ norms, const DevConsts* __restrict__ cst,
    PageMap pm) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wave-uniform grid-stride loop over the G T values (no barriers)
  for (int64_t r = int64_t(blockIdx.x) * 4 + wave; r < G * T; r += int64_t(gridDim.x) * 4) {
    int64_t dg, dn;
    if constexpr (PAGED) {
      if (page_dest(pm, r, dg, dn)) append_value128<BV, BF16>(values, r, dg, dn, pm.page_size, lane, codes, norms, cst);
    } else {
      dg = r / T;
      dn = pos + (r - dg * T);
      append_value128<BV, BF16>(values, r, dg, dn, Ncap, lane, codes, norms, cst);
    }
  }
}

// ============================================================== measurement helpers
// Not part of the method: ceilings and clocks the benchmark reports beside
// the kernels above.

// One wave reads the core-clock cycle counter and the constant-rate
// reference counter, spins until the reference counter has advanced by
// `ticks` (or a cap on iterations), and reads both again.
__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ out, uint32_t ticks) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint64_t r1 = r0, c1 = c0;
  for (uint32_t it = 0; it < (1u << 24); ++it) {
    r1 = __builtin_amdgcn_s_memrealtime();
    c1 = __builtin_amdgcn_s_memtime();
    if (r1 - r0 >= ticks) break;
  }
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

// Streaming ceiling: workgroup w reads its contiguous share of src (16-byte
// non-temporal loads, 1024 threads side by side, four loads in flight per
// thread) and writes its share of dst in between: after each read round
// (four loads per thread) the write rounds that bring the writes up to the
// same fraction of their share.  The written value is a fold of what was
// read; with no writes the fold is kept alive by a store that only happens
// when it equals a constant.
constexpr int kProbeThreads = 1024;
constexpr int kProbeUnroll = 4;
__global__ __launch_bounds__(kProbeThreads) void stream_probe_kernel(const uint4* __restrict__ src,
                                                                     uint64_t nsrc,
                                                                     uint4* __restrict__ dst,
                                                                     uint64_t ndst) {
  constexpr uint64_t kRound = uint64_t(kProbeThreads) * kProbeUnroll;
  const uint64_t wgs = gridDim.x, w = blockIdx.x;
  const uint64_t r0 = nsrc * w / wgs, r1 = nsrc * (w + 1) / wgs;
  const uint64_t w0 = ndst * w / wgs, w1 = ndst * (w + 1) / wgs;
  const uint64_t nr = r1 - r0, nw = w1 - w0;
  const uint32_t tid = threadIdx.x;
  u32x4 fold = {0u, 0u, 0u, 0u};
  const uint64_t rounds_r = (nr + kRound - 1) / kRound;
  const uint64_t rounds_w = (nw + kProbeThreads - 1) / kProbeThreads;
  uint64_t wr = 0;   // write rounds done (1024 stores each)
  for (uint64_t k = 0; k < rounds_r || wr < rounds_w; ++k) {
    if (k < rounds_r) {
      u32x4 v[kProbeUnroll];
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) {
        const uint64_t i = k * kRound + uint64_t(u) * kProbeThreads + tid;
        v[u] = i < nr ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + r0 + i))
                      : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) fold ^= v[u];
    }
    const uint64_t due = rounds_r ? (k + 1 >= rounds_r ? rounds_w : (k + 1) * rounds_w / rounds_r) : rounds_w;
    for (; wr < due; ++wr) {
      const uint64_t j = wr * kProbeThreads + tid;
      if (j < nw) __builtin_nontemporal_store(fold, reinterpret_cast<u32x4*>(dst + w0 + j));
    }
  }
  if (ndst == 0 && dst != nullptr && fold[0] == 0x9E3779B9u && fold[1] == 0x7F4A7C15u)
    dst[0] = make_uint4(fold[0], fold[1], fold[2], fold[3]);
}

// The loads and stores of score128_kernel (same grid, same 64-key tiles per
// wave with two tiles in flight, same record reads and logit writes) without
// the query preparation and without the table arithmetic: each logit is a
// fold of the record.
template <int B>
__global__ __launch_bounds__(kScoreThreads, 1) void score128_stream_kernel(
    const uint4* __restrict__ planes, const uint32_t* __restrict__ norms, int64_t N, int Qg,
    int64_t chunk, float* __restrict__ logits) {
  constexpr int P = B + 1;
  constexpr int D = 2;
  constexpr int64_t kStride = kScoreThreads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.x;
  const int qc = blockIdx.y;
  const int64_t n0 = int64_t(blockIdx.z) * chunk;
  const int64_t n1 = std::min<int64_t>(N, n0 + chunk);
  const uint4* pg = planes + g * P * N;
  const uint32_t* ng = norms + g * N;
  float* lrow[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) lrow[qq] = logits + (g * Qg + std::min(qc * 4 + qq, Qg - 1)) * N;
  auto load_tile = [&](int64_t b) {
    const uint32_t n = uint32_t(std::min<int64_t>(b + lane, n1 - 1));
    uint32_t f = __builtin_nontemporal_load(
        reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(ng) + n * 4u));
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(pg + p * N) + n * 16u));
      f ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    return f;
  };
  const int64_t first = n0 + int64_t(wave) * 64;
  const int64_t ntiles = first < n1 ? (n1 - first + kStride - 1) / kStride : 0;
  uint32_t f[D];
#pragma unroll
  for (int k = 0; k < D; ++k) f[k] = load_tile(first + k * kStride);
  for (int64_t t0 = 0; t0 < ntiles; t0 += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const int64_t b = first + (t0 + k) * kStride;
      if (t0 + k < ntiles && b + lane < n1) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (qc * 4 + qq < Qg) __builtin_nontemporal_store(__uint_as_float(f[k] + qq), lrow[qq] + b + lane);
      }
      f[k] = load_tile(first + (t0 + k + D) * kStride);
    }
  }
}

}  // namespace

bool encode_supported(const Codebook& cb) {
  return cb.d == 128 || cb.d == 1024 || cb.d == 2048 || cb.d == 4096;
}
bool score_supported(const Codebook& cb) { return encode_supported(cb); }

// d = 128: each workgroup prepares its queries itself, no workspace; d = 1024:
// the prepared queries (2 R q, 2 S q and their sums) for all groups.
size_t score_workspace_bytes(const Codebook& cb, int64_t G, int Qg) {
  return cb.d == 1024 ? score_wide_prep_bytes(G, Qg) : cb.d > 1024 ? score_wider_prep_bytes(cb, G, Qg) : 0;
}

hipError_t launch_encode(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t N,
                         int64_t Ncap, int64_t pos, void* packed, hipStream_t s) {
  if (cb.d == 1024) return launch_encode_wide(cb, keys, dtype, G, N, packed, s);
  if (cb.d > 1024) return launch_encode_wider(cb, keys, dtype, G, N, packed, s);
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
                     reinterpret_cast<const uint4*>(cb.d_dm16), PageMap{})
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
                     planes, norms, cb.d_consts, cb.d_frag, cb.d_flip_f32, PageMap{})
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
  // codes: 16-value tiles of 16 * bits * d / 32 words, then the half norms
  uint16_t* norms = reinterpret_cast<uint16_t*>(planes + G * ((N + 15) / 16) * 16 * int64_t(cb.bits) *
                                                             (cb.d / 32));
  if (dtype == 1) {
    const int64_t ntiles16 = G * ((N + 15) / 16);
    const int64_t want = (ntiles16 + kEnc16Waves - 1) / kEnc16Waves;
    const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * 4));
    const uint16_t* vb = static_cast<const uint16_t*>(values);
#define TQ_VB(BB)                                                                                  \
  hipLaunchKernelGGL((encode128_bf16_t16_kernel<BB, true>), dim3(grid), dim3(kEnc16Threads), 0, s, vb, \
                     G, N, N, int64_t(0), planes, norms, cb.d_consts, cb.d_frag16,                 \
                     reinterpret_cast<const uint4*>(cb.d_dm16), PageMap{})
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
                     G, N, N, int64_t(0), planes, norms, cb.d_consts, cb.d_frag, cb.d_flip_f32, PageMap{})
    switch (cb.bits) {
      case 2: TQ_VF(2); break;
      case 3: TQ_VF(3); break;
      default: TQ_VF(4); break;
    }
#undef TQ_VF
  }
  return hipGetLastError();
}

// Value append: whole 16-value tiles (pos and pos + T multiples of 16) take
// the tile encoders, which write only those tiles; other shapes the latency
// kernel above.
hipError_t launch_append_values(const Codebook& cb, const void* values, int dtype, int64_t G, int64_t T,
                                void* vpacked, int64_t Ncap, int64_t pos, hipStream_t s) {
  uint32_t* codes = static_cast<uint32_t*>(vpacked);
  uint16_t* norms = reinterpret_cast<uint16_t*>(codes + G * ((Ncap + 15) / 16) * 16 * int64_t(cb.bits) *
                                                              (cb.d / 32));
  if (pos % 16 == 0 && T % 16 == 0) {
    if (dtype == 1) {
      const int64_t want = (G * (T / 16) + kEnc16Waves - 1) / kEnc16Waves;
      const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * 4));
      const uint16_t* vb = static_cast<const uint16_t*>(values);
#define TQ_VB(BB)                                                                                  \
  hipLaunchKernelGGL((encode128_bf16_t16_kernel<BB, true>), dim3(grid), dim3(kEnc16Threads), 0, s, vb, \
                     G, T, Ncap, pos, codes, norms, cb.d_consts, cb.d_frag16,                       \
                     reinterpret_cast<const uint4*>(cb.d_dm16), PageMap{})
      switch (cb.bits) {
        case 2: TQ_VB(2); break;
        case 3: TQ_VB(3); break;
        default: TQ_VB(4); break;
      }
#undef TQ_VB
    } else {
      const int64_t want = (G * ((T + 31) / 32) + kEncWaves - 1) / kEncWaves;
      const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * 2));
      const float* vf = static_cast<const float*>(values);
#define TQ_VF(BB)                                                                                \
  hipLaunchKernelGGL((encode128_f32_kernel<BB, true>), dim3(grid), dim3(kEncThreads), 0, s, vf, \
                     G, T, Ncap, pos, codes, norms, cb.d_consts, cb.d_frag, cb.d_flip_f32, PageMap{})
      switch (cb.bits) {
        case 2: TQ_VF(2); break;
        case 3: TQ_VF(3); break;
        default: TQ_VF(4); break;
      }
#undef TQ_VF
    }
    return hipGetLastError();
  }
  const unsigned grid = unsigned(std::min<int64_t>((G * T + 3) / 4, int64_t(num_cus()) * 8));
#define TQ_AV(BB, BF)                                                                              \
  hipLaunchKernelGGL((append_values128_kernel<BB, BF, false>), dim3(grid), dim3(256), 0, s, values, G, T, \
                     Ncap, pos, codes, norms, cb.d_consts, PageMap{})
  switch (cb.bits) {
    case 2: if (dtype == 1) TQ_AV(2, true); else TQ_AV(2, false); break;
    case 3: if (dtype == 1) TQ_AV(3, true); else TQ_AV(3, false); break;
    default: if (dtype == 1) TQ_AV(4, true); else TQ_AV(4, false); break;
  }
#undef TQ_AV
  return hipGetLastError();
}

// Device scratch for callers that cannot allocate (tq_attention_decode_noalloc):
// a file-scope device array that every GPU the library runs on holds until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the symbol): its device address is
// looked up once per device with hipGetSymbolAddress and that pointer is used
// everywhere.  Calls that overlap on one device share it and race.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// Grid of the d = 128 scorer: (group, chunk of 4 queries, key range).  One
// workgroup fills a CU, so each (group, query chunk) unit's keys are split
// into as many ranges as fit in one round of workgroups over the CUs (at
// least one; ranges of at least 512 keys, a multiple of 64 each): a second,
// partial round would cost every range another set-up.
static dim3 score_grid(int64_t G, int Qg, int64_t N, int64_t& chunk) {
  const int nqc = (Qg + 3) / 4;
  const int64_t units = G * nqc;
  const int64_t cus = num_cus();
  int64_t want = std::max<int64_t>(1, cus / units);
  want = std::min<int64_t>(want, std::max<int64_t>(1, (N + 511) / 512));
  chunk = ((N + want - 1) / want + 63) / 64 * 64;
  const int64_t splits = (N + chunk - 1) / chunk;
  return dim3{unsigned(G), unsigned(nqc), unsigned(splits)};
}

hipError_t launch_score(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                        const void* packed, int64_t N, int64_t Ncap, float* logits, void* ws,
                        hipStream_t s) {
  if (cb.d == 1024) return launch_score_wide(cb, q, qdtype, G, Qg, packed, N, logits, ws, s);
  if (cb.d > 1024) return launch_score_wider(cb, q, qdtype, G, Qg, packed, N, logits, ws, s);
  int64_t chunk = 0;
  const dim3 grid = score_grid(G, Qg, N, chunk);
  const uint4* planes = static_cast<const uint4*>(packed);
  const uint32_t* norms =
      static_cast<const uint32_t*>(packed) + G * Ncap * int64_t(cb.bits) * (cb.d / 32);
  const bool bf = qdtype == 1;
#define TQ_SC(BB, QB)                                                                   \
  hipLaunchKernelGGL((score128_kernel<BB, QB>), grid, dim3(kScoreThreads), 0, s, q, planes, \
                     norms, N, Ncap, Qg, cb.d_in, chunk, logits, cb.d_consts, cb.d_frag16, PageMap{}, AttnArgs{})
  switch (cb.bits - 1) {
    case 1: if (bf) TQ_SC(1, true); else TQ_SC(1, false); break;
    case 2: if (bf) TQ_SC(2, true); else TQ_SC(2, false); break;
    default: if (bf) TQ_SC(3, true); else TQ_SC(3, false); break;
  }
#undef TQ_SC
  return hipGetLastError();
}

size_t attention_workspace_bytes(const Codebook& cb, int64_t G, int Qg, int64_t N) {
  (void)cb;
  int64_t chunk = 0;
  const dim3 grid = score_grid(G, Qg, N, chunk);
  const size_t lg = (size_t(G) * Qg * N * 4 + 255) / 256 * 256;
  return lg + size_t(grid.x) * grid.y * grid.z * kAttnPart * 4;
}

// Decode attention: the scorer with the value phase (one launch over the
// scorer's grid; logits pass through the caches in the workspace, each key
// range leaves its partial state), then the combine of the ranges.
hipError_t launch_attention(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                            const void* kpacked, const void* vpacked, int64_t N, int64_t Ncap,
                            float scale, float* out, void* ws, hipStream_t s) {
  int64_t chunk = 0;
  const dim3 grid = score_grid(G, Qg, N, chunk);
  float* logits = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         (size_t(G) * Qg * N * 4 + 255) / 256 * 256);
  const uint4* planes = static_cast<const uint4*>(kpacked);
  const uint32_t* norms =
      static_cast<const uint32_t*>(kpacked) + G * Ncap * int64_t(cb.bits) * (cb.d / 32);
  const uint4* vpl = static_cast<const uint4*>(vpacked);
  const uint16_t* vn = reinterpret_cast<const uint16_t*>(
      static_cast<const uint32_t*>(vpacked) + G * ((Ncap + 15) / 16) * 16 * int64_t(cb.bits) * (cb.d / 32));
  const AttnArgs aa{vpl, vn, part, scale, Ncap};
  const bool bf = qdtype == 1;
#define TQ_AT(BB, QB, BVV)                                                                       \
  hipLaunchKernelGGL((score128_kernel<BB, QB, false, BVV>), grid, dim3(kScoreThreads), 0, s, q, planes, \
                     norms, N, Ncap, Qg, cb.d_in, chunk, logits, cb.d_consts, cb.d_frag16, PageMap{}, aa)
  switch (cb.bits) {
    case 2: if (bf) TQ_AT(1, true, 2); else TQ_AT(1, false, 2); break;
    case 3: if (bf) TQ_AT(2, true, 3); else TQ_AT(2, false, 3); break;
    default: if (bf) TQ_AT(3, true, 4); else TQ_AT(3, false, 4); break;
  }
#undef TQ_AT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine128_kernel, dim3(unsigned(G * Qg)), dim3(64), 0, s, part, Qg,
                     int(grid.y), int(grid.z), cb.d_consts, out);
  return hipGetLastError();
}

hipError_t launch_decode(const Codebook& cb, const void* packed, int64_t G, int64_t N, void* out,
                         int odtype, hipStream_t s) {
  if (cb.d == 1024) return launch_decode_wide(cb, packed, G, N, out, odtype, s);
  if (cb.d > 1024) return launch_decode_wider(cb, packed, G, N, out, odtype, s);
  const int64_t keys = G * N;
  const int grid = int(std::min<int64_t>((keys + 3) / 4, int64_t(num_cus()) * 64));
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

hipError_t launch_clock_probe(uint64_t* out, uint32_t ticks, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, s, out, ticks);
  return hipGetLastError();
}

hipError_t launch_stream_probe(const void* src, size_t src_bytes, void* dst, size_t dst_bytes, int grid,
                               hipStream_t s) {
  if (grid <= 0) grid = num_cus() * 4;
  hipLaunchKernelGGL(stream_probe_kernel, dim3(unsigned(grid)), dim3(kProbeThreads), 0, s,
                     static_cast<const uint4*>(src), uint64_t(src_bytes / 16), static_cast<uint4*>(dst),
                     uint64_t(dst_bytes / 16));
  return hipGetLastError();
}

hipError_t launch_score_stream_probe(const Codebook& cb, int64_t G, int Qg, const void* packed, int64_t N,
                                     float* logits, hipStream_t s) {
  int64_t chunk = 0;
  const dim3 grid = score_grid(G, Qg, N, chunk);
  const uint4* planes = static_cast<const uint4*>(packed);
  const uint32_t* norms = static_cast<const uint32_t*>(packed) + G * N * int64_t(cb.bits) * (cb.d / 32);
#define TQ_SP(BB)                                                                                   \
  hipLaunchKernelGGL((score128_stream_kernel<BB>), grid, dim3(kScoreThreads), 0, s, planes, norms, N, Qg, \
                     chunk, logits)
  switch (cb.bits - 1) {
    case 1: TQ_SP(1); break;
    case 2: TQ_SP(2); break;
    default: TQ_SP(3); break;
  }
#undef TQ_SP
  return hipGetLastError();
}

// Paged cache: appends as one [1][G*T] batch of rows whose destinations come
// from the page map (so a 16-key tile packs rows of 16 groups when T = 1);
// scoring with the page map and per-group lengths.
// Appends of at most this many rows take the one-key-per-wave kernel.
constexpr int64_t kAppendRowsMax = 2048;

// The append latency kernel over `rows` keys (rows <= kAppendRowsMax), one
// key per workgroup, destinations from pm.
hipError_t launch_append_rows(const Codebook& cb, const void* keys, int dtype, int64_t rows,
                              uint32_t* planes, uint32_t* norms, const PageMap& pm, hipStream_t s) {
  const int grid = int(rows);
  const bool bf = dtype == 1;
#define TQ_APP(BB)                                                                            \
  if (bf)                                                                                     \
    hipLaunchKernelGGL((append_rows128_kernel<BB, true>), dim3(grid), dim3(kAppendThreads), 0, s, \
                       keys, rows, planes, norms, cb.d_consts, cb.d_Sh, pm);                  \
  else                                                                                        \
    hipLaunchKernelGGL((append_rows128_kernel<BB, false>), dim3(grid), dim3(kAppendThreads), 0, s, \
                       keys, rows, planes, norms, cb.d_consts, cb.d_Sh, pm)
  switch (cb.bits - 1) {
    case 1: TQ_APP(1); break;
    case 2: TQ_APP(2); break;
    default: TQ_APP(3); break;
  }
#undef TQ_APP
  return hipGetLastError();
}

// Write-time append into a contiguous cache of Ncap records per group: such
// a cache is a pool whose page g is group g, Ncap records a page, so up to
// kAppendRowsMax keys take the latency kernel with the contiguous map; larger
// batches the tile encoders.
hipError_t launch_append_keys(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t T,
                              int64_t Ncap, int64_t pos, void* packed, hipStream_t s) {
  const int64_t rows = G * T;
  if (cb.d != 128 || rows > kAppendRowsMax || Ncap > INT32_MAX)
    return launch_encode(cb, keys, dtype, G, T, Ncap, pos, packed, s);
  uint32_t* planes = static_cast<uint32_t*>(packed);
  uint32_t* norms = planes + G * Ncap * int64_t(cb.bits) * (cb.d / 32);
  const PageMap pm{nullptr, nullptr, nullptr, uint32_t(T), 1, int32_t(Ncap), int32_t(G), pos};
  return launch_append_rows(cb, keys, dtype, rows, planes, norms, pm, s);
}

hipError_t launch_encode_paged(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t T,
                               void* pool, int64_t num_pages, int page_size, const int32_t* table,
                               int ppg, const int32_t* pos, hipStream_t s) {
  const int64_t rows = G * T;
  uint32_t* planes = static_cast<uint32_t*>(pool);
  uint32_t* norms = planes + num_pages * int64_t(page_size) * int64_t(cb.bits) * (cb.d / 32);
  const PageMap pm{table, pos, nullptr, uint32_t(T), ppg, page_size, int32_t(num_pages), 0};
  if (rows <= kAppendRowsMax)   // latency path: one key per workgroup
    return launch_append_rows(cb, keys, dtype, rows, planes, norms, pm, s);
  if (dtype == 1) {
    const int64_t want = ((rows + 15) / 16 + kEnc16Waves - 1) / kEnc16Waves;
    const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * (cb.bits == 4 ? 2 : 3)));
    const uint16_t* kb = static_cast<const uint16_t*>(keys);
#define TQ_ENCP(BB)                                                                              \
  hipLaunchKernelGGL((encode128_bf16_t16_kernel<BB, false, true>), dim3(grid), dim3(kEnc16Threads), 0, s, \
                     kb, int64_t(1), rows, int64_t(page_size), int64_t(0), planes, norms, cb.d_consts,     \
                     cb.d_frag16, reinterpret_cast<const uint4*>(cb.d_dm16), pm)
    switch (cb.bits - 1) {
      case 1: TQ_ENCP(1); break;
      case 2: TQ_ENCP(2); break;
      default: TQ_ENCP(3); break;
    }
#undef TQ_ENCP
  } else {
    const int64_t want = ((rows + 31) / 32 + kEncWaves - 1) / kEncWaves;
    const int grid = int(std::min<int64_t>(want, int64_t(num_cus()) * 2));
    const float* kf = static_cast<const float*>(keys);
#define TQ_ENCPF(BB)                                                                               \
  hipLaunchKernelGGL((encode128_f32_kernel<BB, false, true>), dim3(grid), dim3(kEncThreads), 0, s, kf,   \
                     int64_t(1), rows, int64_t(page_size), int64_t(0), planes, norms, cb.d_consts,       \
                     cb.d_frag, cb.d_flip_f32, pm)
    switch (cb.bits - 1) {
      case 1: TQ_ENCPF(1); break;
      case 2: TQ_ENCPF(2); break;
      default: TQ_ENCPF(3); break;
    }
#undef TQ_ENCPF
  }
  return hipGetLastError();
}

hipError_t launch_score_paged(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                              const void* pool, int64_t num_pages, int page_size, const int32_t* table,
                              int ppg, const int32_t* lens, int64_t Lmax, float* logits, hipStream_t s) {
  int64_t chunk = 0;
  const dim3 grid = score_grid(G, Qg, Lmax, chunk);
  const uint4* planes = static_cast<const uint4*>(pool);
  const uint32_t* norms =
      static_cast<const uint32_t*>(pool) + num_pages * int64_t(page_size) * int64_t(cb.bits) * (cb.d / 32);
  const PageMap pm{table, nullptr, lens, 1u, ppg, page_size, int32_t(num_pages)};
  const bool bf = qdtype == 1;
#define TQ_SCP(BB, QB)                                                                          \
  hipLaunchKernelGGL((score128_kernel<BB, QB, true>), grid, dim3(kScoreThreads), 0, s, q, planes, \
                     norms, Lmax, int64_t(page_size), Qg, cb.d_in, chunk, logits, cb.d_consts, cb.d_frag16, pm, AttnArgs{})
  switch (cb.bits - 1) {
    case 1: if (bf) TQ_SCP(1, true); else TQ_SCP(1, false); break;
    case 2: if (bf) TQ_SCP(2, true); else TQ_SCP(2, false); break;
    default: if (bf) TQ_SCP(3, true); else TQ_SCP(3, false); break;
  }
#undef TQ_SCP
  return hipGetLastError();
}

// Value append into a paged value pool (num_pages pages of page_size value
// records, laid out as a value buffer of num_pages groups): the latency
// kernel, one value per wave, for any number of rows.
hipError_t launch_append_values_paged(const Codebook& cb, const void* values, int dtype, int64_t G, int64_t T,
                                      void* pool, int64_t num_pages, int page_size, const int32_t* table,
                                      int ppg, const int32_t* pos, hipStream_t s) {
  uint32_t* codes = static_cast<uint32_t*>(pool);
  uint16_t* norms = reinterpret_cast<uint16_t*>(codes + num_pages * (int64_t(page_size) / 16) * 16 *
                                                              int64_t(cb.bits) * (cb.d / 32));
  const PageMap pm{table, pos, nullptr, uint32_t(T), ppg, page_size, int32_t(num_pages), 0};
  const unsigned grid = unsigned(std::min<int64_t>((G * T + 3) / 4, int64_t(num_cus()) * 8));
#define TQ_AVP(BB, BF)                                                                             \
  hipLaunchKernelGGL((append_values128_kernel<BB, BF, true>), dim3(grid), dim3(256), 0, s, values, G, T, \
                     int64_t(page_size), int64_t(0), codes, norms, cb.d_consts, pm)
  switch (cb.bits) {
    case 2: if (dtype == 1) TQ_AVP(2, true); else TQ_AVP(2, false); break;
    case 3: if (dtype == 1) TQ_AVP(3, true); else TQ_AVP(3, false); break;
    default: if (dtype == 1) TQ_AVP(4, true); else TQ_AVP(4, false); break;
  }
#undef TQ_AVP
  return hipGetLastError();
}

// Decode attention over a paged key pool and a paged value pool that share
// one page table: the scorer in paged form with the value phase (each
// 64-key tile's key and value records from its page), then the combine.
// Logits [G][Qg][Lmax] in the workspace, as for tq_attention_decode with
// N = Lmax.
hipError_t launch_attention_paged(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                                  const void* kpool, const void* vpool, int64_t num_pages, int page_size,
                                  const int32_t* table, int ppg, const int32_t* lens, int64_t Lmax,
                                  float scale, float* out, void* ws, hipStream_t s) {
  int64_t chunk = 0;
  const dim3 grid = score_grid(G, Qg, Lmax, chunk);
  float* logits = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         (size_t(G) * Qg * Lmax * 4 + 255) / 256 * 256);
  const uint4* planes = static_cast<const uint4*>(kpool);
  const uint32_t* norms =
      static_cast<const uint32_t*>(kpool) + num_pages * int64_t(page_size) * int64_t(cb.bits) * (cb.d / 32);
  const uint4* vpl = static_cast<const uint4*>(vpool);
  const uint16_t* vn = reinterpret_cast<const uint16_t*>(
      static_cast<const uint32_t*>(vpool) +
      num_pages * (int64_t(page_size) / 16) * 16 * int64_t(cb.bits) * (cb.d / 32));
  const AttnArgs aa{vpl, vn, part, scale, int64_t(page_size)};
  const PageMap pm{table, nullptr, lens, 1u, ppg, page_size, int32_t(num_pages), 0};
  const bool bf = qdtype == 1;
#define TQ_ATP(BB, QB, BVV)                                                                      \
  hipLaunchKernelGGL((score128_kernel<BB, QB, true, BVV>), grid, dim3(kScoreThreads), 0, s, q, planes, \
                     norms, Lmax, int64_t(page_size), Qg, cb.d_in, chunk, logits, cb.d_consts, cb.d_frag16, pm, aa)
  switch (cb.bits) {
    case 2: if (bf) TQ_ATP(1, true, 2); else TQ_ATP(1, false, 2); break;
    case 3: if (bf) TQ_ATP(2, true, 3); else TQ_ATP(2, false, 3); break;
    default: if (bf) TQ_ATP(3, true, 4); else TQ_ATP(3, false, 4); break;
  }
#undef TQ_ATP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine128_kernel, dim3(unsigned(G * Qg)), dim3(64), 0, s, part, Qg,
                     int(grid.y), int(grid.z), cb.d_consts, out);
  return hipGetLastError();
}

}  // namespace tq

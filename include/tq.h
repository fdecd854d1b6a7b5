/*
 * tq.h — C ABI of the TurboQuant key-path library for AMD Instinct MI355X
 * (gfx950).  Plain pointers and sizes only; device pointers are HIP device
 * allocations (for example torch tensors' data_ptr()), streams are
 * hipStream_t passed as void* (NULL = the default stream).
 *
 * The operation it implements, from the pages:
 *  - keys are normalised, rotated with R = H_d D / sqrt(d) (Sylvester
 *    Hadamard H_d, Rademacher diagonal D), and each rotated coordinate,
 *    approximately N(0, 1/d), is coded by a shared Lloyd-Max scalar quantizer
 *    [ICLR 2026 paper digest (0h-n0.github.io), "Step 1: PolarQuant", eq. for R
 *    and Theorem 1; Qiita explainer (kai_kou), "Stage 1" step 3];
 *  - with b total bits, b-1 bits go to that MSE stage and 1 bit to a QJL sign
 *    sketch of the residual [ai.spot.hk TurboQuant article, "無偏內積估計"];
 *  - a full-precision query is scored against the packed key with
 *      <q,k> ~ <q,k_mse> + ||r|| sqrt(pi/2)/m <S q, sign(S r)>
 *    [Qiita explainer, "Stage 2: QJL", estimator equation];
 *  - the norm is kept on the side and zero vectors (||k|| < 1e-10) give an
 *    all-zero record [ICLR 2026 paper digest, "実装の擬似コード",
 *    "実装のポイント"].
 *
 * Packed key record layout (one buffer for G groups x N keys; D =
 * tq_rotation_dim(d), which is d itself unless d is zero-padded, and m = D):
 *   planes: uint32 [G][bits][N][D/32].  Planes 0..bits-2 hold bit p of the
 *           level index (LSB first; levels ascending, code 0 = most negative
 *           level); plane bits-1 holds the QJL sign bits, 1 = negative.
 *           Bit j of word w is coordinate (or sketch row) 32*w + j.
 *   norms:  uint32 [G][N] = half(||k||) | half(||r||) << 16  (IEEE half, RNE).
 *   Total:  G*N*((bits-1)*D/8 + D/8 + 4) bytes.
 *
 * Dimensions that are not a power of two: the method needs a power of two
 * for the Hadamard transform, and a shorter vector is zero-padded up to the
 * next one [ICLR 2026 paper digest, "実装のポイント": zero padding to the
 * nearest power of two, with negligible accuracy loss reported].  A codebook
 * made for such a d (a multiple of 16) runs in D = tq_rotation_dim(d):
 * delta has D entries, S is m x D with m = D, the levels are those for
 * N(0, 1/D), and records are D-dimensional.  Keys, values and queries are
 * passed as rows of d elements and decoded vectors come back as rows of d
 * elements; the kernels read the missing coordinates as zeros.  Where a call
 * below is limited to some d (128, 1024, 2048, 4096), that names D: a
 * zero-padded codebook follows the rules of its D.
 *
 * Status: every entry point returns TQ_OK (0) or a negative TQ_ERR_* code.
 * No C++ exception crosses this boundary.  Launches are asynchronous on the
 * given stream; device faults surface at the caller's next synchronisation.
 * Inputs are not checked for NaN/Inf (outputs are then unspecified); key
 * norms >= 65520 overflow the half-precision norm and are unsupported.
 * All pointer arguments of the GPU calls must be 16-byte aligned.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TQ_OK = 0,
  TQ_ERR_ARG = -1,          /* null/misaligned pointer, negative size, bad dtype */
  TQ_ERR_UNSUPPORTED = -2,  /* parameter outside what the kernels implement */
  TQ_ERR_ALLOC = -3,        /* host or device allocation failed */
  TQ_ERR_HIP = -4,          /* a HIP runtime call or launch failed; see tq_last_hip_error */
  TQ_ERR_WORKSPACE = -5     /* workspace pointer null or smaller than required */
};

/* Element types of keys, queries and decoded outputs. */
enum { TQ_F32 = 0, TQ_BF16 = 1 };

/* Coordinate law the Lloyd-Max tables are optimal for.  TQ_CODEBOOK_GAUSSIAN:
 * N(0, 1/d), the limit the pages give for a rotated coordinate (the default).
 * TQ_CODEBOOK_BETA: the exact law of one coordinate of a uniformly random
 * unit vector in R^d, density proportional to (1 - y^2)^((d-3)/2) on [-1, 1]
 * (y^2 ~ Beta(1/2, (d-1)/2)) [ai.spot.hk article, "隨機旋轉與Beta分佈";
 * ICLR 2026 paper digest, "Step 1: PolarQuant"].  Both are symmetric with the
 * middle threshold at 0; only the level and threshold values differ. */
enum { TQ_CODEBOOK_GAUSSIAN = 0, TQ_CODEBOOK_BETA = 1 };

typedef struct tq_codebook tq_codebook;

/* The power of two D the method runs in for vectors of d elements: d when d
 * is a power of two in [32, 4096]; otherwise the next power of two >= 32
 * when d is a multiple of 16 below 4096 (zero padding, see above); 0 when d
 * is unsupported.  Pure host function.  (The host tables exist for every such
 * D; the device kernels for D in {128, 1024, 2048, 4096}.) */
int32_t tq_rotation_dim(int32_t d);

/*
 * Host-only: the quantizer tables derived from (d, bits, m, seed), written to
 * caller-owned host arrays (any may be NULL).  Below, d stands for
 * tq_rotation_dim(d) (the same value unless d is zero-padded):
 *   levels[L], thresholds[L-1]  Lloyd-Max levels/boundaries for N(0, 1/d),
 *                               L = 2^(bits-1), ascending, float64;
 *   delta[d]                    Rademacher signs (+1/-1) of D;
 *   S[m*d]                      QJL sketch, row-major, float64: S = S_rot R;
 *   S_rot[m*d]                  S R^T (the sketch seen from the rotated
 *                               domain, S r = S_rot (R r)): N(0,1) draws
 *                               rounded to float16, held in float64.
 * R is orthogonal, so S has the i.i.d. N(0,1) law of the QJL projection
 * [Qiita explainer, "Stage 2: QJL"] up to the float16 rounding of the draws.
 * delta and S_rot come from a counter-based SplitMix64 stream: draw(seed, s, i)
 * = mix64(mix64(seed + s*G) + (i+1)*G), G = 0x9E3779B97F4A7C15; delta_i = +1
 * iff bit 63 of draw(seed,1,i) is 0; S_rot[j][i] = fp16(sqrt(-2 ln u1)
 * cos(2 pi u2)), u1 = ((x>>11)+1) 2^-53, u2 = (y>>11) 2^-53,
 * x,y = draw(seed,2,2(jd+i)+{0,1}).
 * Touches no GPU.  Errors: TQ_ERR_UNSUPPORTED (tq_rotation_dim(d) == 0,
 * bits not in {2,3,4}, m != tq_rotation_dim(d)), TQ_ERR_ALLOC.
 */
int tq_codebook_tables(int32_t d, int32_t bits, int32_t m, uint64_t seed,
                       double* levels, double* thresholds, int8_t* delta,
                       double* S, double* S_rot);

/* tq_codebook_tables for a chosen coordinate law (TQ_CODEBOOK_*) [ai.spot.hk
 * article, "隨機旋轉與Beta分佈": a rotated coordinate follows a Beta law;
 * ICLR 2026 paper digest, "Step 1: PolarQuant": that law, then N(0, 1/d) for
 * large d]; kind
 * TQ_CODEBOOK_GAUSSIAN is tq_codebook_tables.  Errors as above, plus
 * TQ_ERR_ARG for an unknown kind. */
int tq_codebook_tables_ex(int32_t d, int32_t bits, int32_t m, uint64_t seed, int32_t kind,
                          double* levels, double* thresholds, int8_t* delta, double* S,
                          double* S_rot);

/*
 * Build the quantizer state for (d, bits, m, seed) on the current HIP device:
 * the tables above plus the kernels' constant blocks (thresholds and levels in
 * float32, S_rot as float16 laid out for the matrix
 * cores, Walsh coefficients of the levels for the scorer).  The handle owns
 * its device memory (hipMalloc) and is immutable afterwards, so it may be
 * shared by streams and threads; it is valid on the device that was current
 * here.  Supported: tq_rotation_dim(d) in {128, 1024, 2048, 4096}, i.e.
 * d = 128, 1024, 2048 or 4096, or a zero-padded d: 80, 96, 112, or a multiple
 * of 16 in [528, 1008], [1040, 2032] or [2064, 4080]; bits in {2, 3, 4};
 * m == tq_rotation_dim(d).
 * Errors: TQ_ERR_ARG (out NULL), TQ_ERR_UNSUPPORTED, TQ_ERR_ALLOC, TQ_ERR_HIP.
 */
int tq_make_codebook(int32_t d, int32_t bits, int32_t m, uint64_t seed, tq_codebook** out);

/* tq_make_codebook for a chosen coordinate law (TQ_CODEBOOK_*; passages as
 * tq_codebook_tables_ex): every entry point then encodes, scores and
 * decodes with those levels and thresholds (keys: bits-1 bit codes, values:
 * bits bit codes).  Errors as above, plus TQ_ERR_ARG for an unknown kind. */
int tq_make_codebook_ex(int32_t d, int32_t bits, int32_t m, uint64_t seed, int32_t kind,
                        tq_codebook** out);

/* Release a codebook (NULL is a no-op).  The caller must ensure no launch
 * that uses it is still in flight.  (Library bookkeeping: defines no step of
 * the method.) */
void tq_free_codebook(tq_codebook* cb);

/* (Library bookkeeping.)  Host copies of a codebook's tables (same meaning and sizes as
 * tq_codebook_tables: delta has tq_rotation_dim(d) entries; any pointer may
 * be NULL).  Errors: TQ_ERR_ARG (cb NULL). */
int tq_codebook_export(const tq_codebook* cb, double* levels, double* thresholds,
                       int8_t* delta, double* S, double* S_rot);

/* (Library bookkeeping.)  (d, bits, m, seed) of a codebook as passed to tq_make_codebook (d is the
 * caller's vector length, before any zero padding); any pointer may be NULL. */
int tq_codebook_info(const tq_codebook* cb, int32_t* d, int32_t* bits, int32_t* m,
                     uint64_t* seed);

/* Bytes of a packed buffer for G groups of N keys [ICLR 2026 paper digest,
 * implementation notes: the norm kept beside each vector, sign bits eight per
 * byte; Qiita explainer, byte table: bytes per key at each width]; 0 on bad arguments. */
size_t tq_packed_bytes(const tq_codebook* cb, int64_t G, int64_t N);

/*
 * Encode G*N keys (rows of d elements, [G][N][d] contiguous, TQ_F32 or
 * TQ_BF16) into the packed layout above.  Per key k: nu = ||k||; zero record if
 * nu < 1e-10; else y = R k / nu, code_i = #{thresholds <= y_i},
 * residual r = k - nu R^T c[code], rho = ||r||, sign bit_j = [(S r)_j < 0]
 * (S r is evaluated as S_rot (R r) on the matrix cores: S_rot is exact in
 * float16, R r is split into float16 hi + lo, float32 accumulation), norms
 * stored as half.
 * Passages: normalise, rotate with the randomized Hadamard transform and
 * quantise every coordinate with one scalar codebook [ICLR 2026 paper digest,
 * "Step 1: PolarQuant"; Qiita explainer, "Stage 1: PolarQuant" step 3];
 * sign sketch of the residual with a Gaussian projection [Qiita explainer,
 * "Stage 2: QJL"]; (b-1) + 1 bits [ai.spot.hk article, "無偏內積估計"];
 * zero vectors and "0 counts as positive" [ICLR 2026 paper digest,
 * "実装の擬似コード"].
 * keys and packed are device pointers owned by the caller; G*N == 0 is a
 * no-op.  d = 128 and d = 1024 allocate nothing (d = 1024 holds each tile's
 * residuals on chip); d = 2048 and 4096 run in chunks of 2^26 / d keys, each
 * through a float32 temporary of 256 MiB taken from the device's
 * stream-ordered pool (hipMallocAsync / hipFreeAsync on the given stream).
 * Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP (also when that
 * temporary cannot be allocated).
 */
int tq_encode_keys(const tq_codebook* cb, const void* keys, int32_t key_dtype,
                   int64_t G, int64_t N, void* packed, void* stream);

/*
 * Append new keys to a packed cache at write time (compression happens when
 * the cache is written; nothing is retrained [ICLR 2026 paper digest,
 * "実装のポイント"; ai.spot.hk article, online / data-oblivious quantisation]).
 * keys: [G][T][d] device rows (TQ_F32 or TQ_BF16), typically T = 1 new
 * token per (batch, KV head) per decode step.  packed: a device buffer laid
 * out as above for G groups of Ncap records (tq_packed_bytes(cb, G, Ncap)).
 * Key t of group g is encoded by the rules of tq_encode_keys and written to
 * record pos + t of group g; no other record is touched.  Up to 2048 keys
 * (G*T) are encoded by the latency kernel of tq_paged_append_keys, one key
 * per workgroup (float32 rotation and projection: records equal
 * tq_encode_keys's except where a rotated coordinate lies within rounding of
 * a threshold or a projection within rounding of zero, cases the method's
 * parity rules leave open); more keys by the tile encoder of tq_encode_keys
 * (identical records).
 * Requires 0 <= pos and pos + T <= Ncap.  G*T == 0 is a no-op.  d = 128 only.
 * Allocates nothing.  Errors: TQ_ERR_ARG (also pos + T > Ncap),
 * TQ_ERR_UNSUPPORTED (d != 128), TQ_ERR_HIP.
 */
int tq_append_keys(const tq_codebook* cb, const void* keys, int32_t key_dtype, int64_t G,
                   int64_t T, void* packed, int64_t Ncap, int64_t pos, void* stream);

/*
 * Paged key cache: compression at the time the cache is written, as above,
 * into fixed-size pages that a page table maps, so a serving loop grows each
 * sequence's cache page by page and reuses freed pages (a ring or a sliding
 * window is a page table whose entries the caller rotates).
 *
 * Pool: num_pages pages of page_size records; page i is laid out exactly as
 * the packed buffer of one group of page_size keys (planes, then norms), so
 * the pool is tq_packed_bytes(cb, num_pages, page_size) bytes.  page_table:
 * device int32 [G][pages_per_group]; entry (g, p) is the pool page holding
 * logical positions [p * page_size, (p + 1) * page_size) of group g.  The
 * table, pos and lens live in device memory (the host does not read them):
 * a record whose logical page is past pages_per_group, or whose table entry
 * is outside [0, num_pages), is not written (append) and not scored (score).
 * d = 128 only; page_size a multiple of 64 in [64, 2^20].
 *
 * tq_paged_append_keys: keys [G][T][d] (TQ_F32 or TQ_BF16); key t of group g
 * is encoded by the rules of tq_encode_keys and written to logical position
 * pos[g] + t (pos: device int32 [G]).  The G*T rows are encoded as one batch:
 * up to 2048 rows by a latency kernel, one key per workgroup (float32
 * rotation and projection: its records equal tq_encode_keys's except where a
 * rotated coordinate lies within rounding of a threshold or a projection
 * within rounding of zero, cases the method's parity rules leave open), more
 * rows by the tile encoder of tq_encode_keys in paged form (identical
 * records).  G*T == 0 is a no-op; nothing is allocated.
 * Errors: TQ_ERR_ARG (null/misaligned pointer: keys and pool 16-byte,
 * table and pos 4-byte aligned; a size <= 0), TQ_ERR_UNSUPPORTED (d != 128,
 * page_size, G*T >= 2^31, G*pages_per_group >= 2^31), TQ_ERR_HIP.
 *
 * tq_paged_score: logits[g][h][n] (float32 [G][Qg][Lmax]) for n < min(lens[g],
 * Lmax, pages_per_group * page_size), the estimator of tq_score_logits on the
 * record at logical position n of group g; other logits are left untouched.
 * Errors: as tq_paged_append_keys (logits 16-byte aligned, lens 4-byte),
 * TQ_ERR_UNSUPPORTED also for Qg > 256 or Lmax >= 2^28.
 */
int tq_paged_append_keys(const tq_codebook* cb, const void* keys, int32_t key_dtype, int64_t G,
                         int64_t T, void* pool, int64_t num_pages, int32_t page_size,
                         const int32_t* page_table, int32_t pages_per_group, const int32_t* pos,
                         void* stream);
int tq_paged_score(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                   const void* pool, int64_t num_pages, int32_t page_size, const int32_t* page_table,
                   int32_t pages_per_group, const int32_t* lens, int64_t Lmax, float* logits,
                   void* stream);

/*
 * Paged value pool and decode attention over paged caches: the value side of
 * the paged key cache above, for a serving loop whose KV-cache wrapper keeps
 * every token compressed from the moment it is cached [Qiita explainer, API
 * table: the KV-cache wrapper beside the key and value compressors; ICLR
 * 2026 paper digest, "実装のポイント": compression at write time].
 *
 * Value pool: num_pages pages of page_size value records, laid out as the
 * value records (tq_value_packed_bytes layout) of num_pages groups of
 * page_size values, so tq_value_packed_bytes(cb, num_pages, page_size)
 * bytes.  It shares the key pool's page table: entry (g, p) names the page
 * of logical positions [p * page_size, (p + 1) * page_size) of group g in
 * both pools.  page_size as for the key pool (a multiple of 64).
 *
 * tq_paged_append_values: values [G][T][d] (TQ_F32 or TQ_BF16); value t of
 * group g is coded by the rules of tq_encode_values and written to logical
 * position pos[g] + t (pos: device int32 [G]) by the value append latency
 * kernel (one value per wave, float32 rotation: level indices equal
 * tq_encode_values's except where a rotated coordinate lies within rounding
 * of a threshold), which sets the value's bits in its 16-value tile with
 * atomic OR / AND, so the values of one tile may arrive in any calls.  A
 * position whose page is invalid is not written.  G*T == 0 is a no-op;
 * nothing is allocated.  Errors: as tq_paged_append_keys.
 *
 * tq_paged_attention: out[g][h] (float32 [G][Qg][d]) = sum over the
 * positions n < min(lens[g], Lmax, pages_per_group * page_size) whose page
 * entry is valid of softmax_n(scale * logit) * v_mse, with the estimator and
 * the value decode of tq_attention_decode; a group without such positions
 * gets zeros.  kpool: the key pool (its size in pages is num_pages for both
 * pools), vpool: the value pool.  Two launches (the paged scorer with the
 * value phase, then the combine); ws: tq_attention_workspace_bytes(cb, G,
 * Qg, Lmax) bytes of device memory.
 * Errors: TQ_ERR_ARG (as tq_paged_score; also Lmax == 0 with G*Qg > 0, scale
 * not finite and > 0), TQ_ERR_WORKSPACE, TQ_ERR_UNSUPPORTED (as
 * tq_paged_score), TQ_ERR_HIP.
 */
int tq_paged_append_values(const tq_codebook* cb, const void* values, int32_t dtype, int64_t G, int64_t T,
                           void* pool, int64_t num_pages, int32_t page_size, const int32_t* page_table,
                           int32_t pages_per_group, const int32_t* pos, void* stream);
int tq_paged_attention(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                       const void* kpool, const void* vpool, int64_t num_pages, int32_t page_size,
                       const int32_t* page_table, int32_t pages_per_group, const int32_t* lens, int64_t Lmax,
                       float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Value records (MSE-only): the community implementation on the Qiita
 * explainer compresses values with the Stage-1 quantizer alone (API table:
 * value compressor = rotation + Lloyd-Max), and its byte table counts b-bit
 * value codes plus one half norm per value.  A value record uses all `bits`
 * bits of the codebook for a Lloyd-Max code of N(0, 1/d) (2^bits levels),
 * with the same rotation R; no sketch bit.  Layout for G groups x N values,
 * in tiles of 16 consecutive values of a group (T = ceil(N/16) per group):
 *   codes:  uint32 [G][T][bits*D/2]: tile t holds values 16t .. 16t+15
 *           (values past N have code 0); its 16*bits*D bits (bit k = bit
 *           k%32 of word k/32) are D slots of 16*bits bits, slot s holding
 *           coordinate 32*(s/32) + 16*(s%2) + (s%32)/2 of the 16 values, as
 *           8 groups of 2*bits bits: bit 2p+i of group q = bit p of the
 *           level index of value 2q+i;
 *   norms:  uint16 [G][N] = half(||v||) (RNE); zero record if ||v|| < 1e-10.
 *   Total:  G*(16*T*bits*D/8 + 2*N) bytes (bits*D/8 + 2 per value when N is
 *           a multiple of 16).
 * A slot group is the index of a table of level pairs: the decode attention
 * forms its weighted sums on the matrix cores from it (this bit order is the
 * library's, not the pages').  d = 128 only.
 */
size_t tq_value_packed_bytes(const tq_codebook* cb, int64_t G, int64_t N);

/* Encode G*N values ([G][N][d] device rows, TQ_F32 or TQ_BF16) into value
 * records.  Per value: nu = ||v||, y = R v / nu, code_i = #{t_j <= y_i} over
 * the 2^bits - 1 thresholds, nu stored as half.  G*N == 0 is a no-op; nothing
 * is allocated.  Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED (d != 128), TQ_ERR_HIP. */
int tq_encode_values(const tq_codebook* cb, const void* values, int32_t dtype, int64_t G,
                     int64_t N, void* vpacked, void* stream);

/*
 * Append new values to a value cache at write time, the value side of
 * tq_append_keys (the Qiita explainer's API table lists an MSE compressor for
 * value vectors beside the key compressor; the ICLR 2026 paper digest,
 * "実装のポイント", has compression happen when the cache is written).
 * values: [G][T][d] device rows (TQ_F32 or TQ_BF16).  vpacked: a value cache
 * laid out as above for G groups of Ncap records
 * (tq_value_packed_bytes(cb, G, Ncap)).  Value t of group g is coded by the
 * rules of tq_encode_values and written to record pos + t of group g (its
 * level indices into its tile, its half norm); no other record is touched,
 * also not the other values of a tile it shares.  Whole tiles (pos and T
 * multiples of 16) are written by the tile encoder of tq_encode_values
 * (identical records); other shapes by a latency kernel, one value per wave
 * (float32 rotation; its level indices equal tq_encode_values's except where
 * a rotated coordinate lies within rounding of a threshold) that sets the
 * value's bits with atomic OR / AND.  Records pos .. pos+T-1 of one call may
 * share tiles with records another call on another stream writes at the same
 * time: the bit updates do not race, but the caller orders appends before the
 * attention that reads them.  Requires 0 <= pos and pos + T <= Ncap.
 * G*T == 0 is a no-op; nothing is allocated.  d = 128 only.
 * Errors: TQ_ERR_ARG (also pos + T > Ncap), TQ_ERR_UNSUPPORTED (d != 128,
 * G*T >= 2^33), TQ_ERR_HIP.
 */
int tq_append_values(const tq_codebook* cb, const void* values, int32_t dtype, int64_t G, int64_t T,
                     void* vpacked, int64_t Ncap, int64_t pos, void* stream);

/* (Library bookkeeping.)  Workspace bytes of tq_attention_decode (the logits plus per-range partial
 * sums); 0 on bad arguments or d != 128. */
size_t tq_attention_workspace_bytes(const tq_codebook* cb, int64_t G, int32_t Qg, int64_t N);

/*
 * Decode attention over packed keys and values, neither ever dequantised to
 * memory:  out[g][h] = sum_n softmax_n(scale * logit[g][h][n]) * v_mse[g][n],
 * logit = the estimator of tq_score_logits, v_mse = nu~ R^T c_v[code]
 * (scale = 1/sqrt(d) for scaled dot-product attention).  q [G][Qg][d]
 * (TQ_F32/TQ_BF16), kpacked: key records for N keys per group, vpacked: value
 * records for N values per group, out float32 [G][Qg][d].  Two launches on
 * the stream: the score kernel with a value pass over its key range (logits
 * into ws; each range keeps its maximum, normaliser and weighted level sums
 * in the rotated domain, float16 hi/lo operands on the matrix cores), and a
 * combine that merges the ranges and rotates back with R^T.
 * ws: tq_attention_workspace_bytes(cb, G, Qg, N) bytes of device memory.
 * Errors: TQ_ERR_ARG (also N == 0 with G*Qg > 0, scale not finite and > 0),
 * TQ_ERR_WORKSPACE, TQ_ERR_UNSUPPORTED (d != 128, Qg > 256, N >= 2^28), TQ_ERR_HIP.
 */
int tq_attention_decode(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G,
                        int32_t Qg, const void* kpacked, const void* vpacked, int64_t N,
                        float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * tq_attention_decode over the first len records of each group of a key
 * cache and a value cache that hold Ncap records per group (the layouts
 * tq_append_keys and tq_append_values write into): the decode step of a
 * serving loop that compresses each token as it is cached [ICLR 2026 paper
 * digest, "実装のポイント"].  Same launches and same results as
 * tq_attention_decode on a buffer of len records; records past len are not
 * weighed (their codes may hold anything, their norms are not read).
 * ws: tq_attention_workspace_bytes(cb, G, Qg, len) bytes.  Requires
 * 1 <= len <= Ncap when G*Qg > 0.
 * Errors: TQ_ERR_ARG (also len == 0 or len > Ncap), TQ_ERR_WORKSPACE,
 * TQ_ERR_UNSUPPORTED (d != 128, Qg > 256, Ncap >= 2^28), TQ_ERR_HIP.
 */
int tq_attention_cache(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                       const void* kpacked, const void* vpacked, int64_t Ncap, int64_t len, float scale,
                       float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * tq_attention_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same launches, same results as
 * tq_attention_decode; the workspace lives in a static device array of
 * tq_attention_noalloc_max_bytes() bytes (32 MiB) that the library holds on
 * every GPU it runs on until the process ends.  Nothing is allocated and no
 * memory is cleared: every byte the launches read from the array is written
 * by an earlier launch of the same call.  All calls on one GPU share the
 * array, so calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 * Errors: as tq_attention_decode, and TQ_ERR_WORKSPACE when
 * tq_attention_workspace_bytes(cb, G, Qg, N) exceeds the array.
 */
int tq_attention_decode_noalloc(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G,
                                int32_t Qg, const void* kpacked, const void* vpacked, int64_t N,
                                float scale, float* out, void* stream);

/* Size in bytes of the static array tq_attention_decode_noalloc works in
 * (library bookkeeping, for the callers that entry point is for). */
size_t tq_attention_noalloc_max_bytes(void);

/* (Library bookkeeping.)  Workspace bytes tq_score_logits needs for G groups of Qg queries: 0 for
 * d = 128 (each workgroup prepares its queries on chip; ws may be NULL);
 * G*Qg*(2*d + 4)*4 for d = 1024, 2048 and 4096 (the prepared queries 2 R q,
 * 2 S q and their sums). */
size_t tq_score_workspace_bytes(const tq_codebook* cb, int64_t G, int32_t Qg);

/*
 * Estimated logits of full-precision queries against packed keys:
 *   logits[g][h][n] = nu~ <R q, c[code]> + rho~ sqrt(pi/2)/m <S q, 1 - 2 sbit>
 * for query h of group g, q[g][h][0..d) (TQ_F32 or TQ_BF16), against key n of
 * group g (GQA: query head j*Qg + h uses KV head j).  logits is float32
 * [G][Qg][N].  One launch on the stream: each workgroup prepares its queries
 * (R q via a Hadamard butterfly, S q, their sums) and then streams the packed
 * keys of its range.  All buffers are caller-owned device memory; ws must hold
 * tq_score_workspace_bytes(cb, G, Qg) bytes (may be NULL when that is 0).
 * G*N*Qg == 0 is a no-op.  d = 1024, 2048 and 4096 run a query-preparation
 * kernel into ws first, then score with nibble subset-sum tables (same
 * estimator; at 2048 and 4096 in 1024-coordinate slices whose partial logits
 * accumulate in the logits array).
 * Errors: TQ_ERR_ARG, TQ_ERR_WORKSPACE, TQ_ERR_UNSUPPORTED (Qg > 256, G > 2^31 - 1,
 * or N >= 2^28 at d = 128: records and logits of a group are addressed with
 * 32-bit byte offsets), TQ_ERR_HIP.
 */
int tq_score_logits(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G,
                    int32_t Qg, const void* packed, int64_t N, float* logits, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * tq_score_logits over the first len records of each group of a packed cache
 * that holds Ncap records per group (the layout tq_append_keys writes into):
 * logits is float32 [G][Qg][len], same estimator and same kernel as
 * tq_score_logits (which is the case len = Ncap = N).  Requires
 * 0 <= len <= Ncap.  d = 128 only; needs no workspace.
 * Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED (d != 128, Qg > 256,
 * G > 2^31 - 1, Ncap >= 2^28), TQ_ERR_HIP.
 */
int tq_score_cache(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                   const void* packed, int64_t Ncap, int64_t len, float* logits, void* stream);

/*
 * Vector-search top-k by the same estimated inner product as tq_score_logits
 * (nearest-neighbour search over an index of packed vectors [ICLR 2026 paper
 * digest, vector-search results]): for every query h of group g, the k keys
 * of that group with the largest estimate, best first, ties broken by the
 * smaller key index; the logit matrix is never formed.
 *   idx[g][h][k]     int32 key index in [0, N), -1 where N < k (device, caller-owned)
 *   scores[g][h][k]  float32 estimate, -inf where N < k (device, caller-owned)
 * ws must hold tq_score_topk_workspace_bytes(cb, G, Qg, N, k) bytes of device
 * memory (prepared queries plus per-key-range candidate lists).
 * Supported: d == 1024, 1 <= k <= 16, Qg <= 256, N <= 2^31 - 1.
 * Errors: TQ_ERR_ARG (null/misaligned pointer, N == 0), TQ_ERR_UNSUPPORTED,
 * TQ_ERR_WORKSPACE, TQ_ERR_HIP.
 */
size_t tq_score_topk_workspace_bytes(const tq_codebook* cb, int64_t G, int32_t Qg, int64_t N,
                                     int32_t k);
int tq_score_topk(const tq_codebook* cb, const void* q, int32_t q_dtype, int64_t G, int32_t Qg,
                  const void* packed, int64_t N, int32_t k, int32_t* idx, float* scores, void* ws,
                  size_t ws_bytes, void* stream);

/*
 * MSE-only reconstruction of every packed key: out[g][n] = nu~ R^T c[code]
 * as TQ_F32 or TQ_BF16 [G][N][d] (rows of the codebook's d elements; the
 * zero-padded coordinates are dropped).  This is the Stage-1 dequantisation:
 * the level of each code, the inverse rotation R^T = D H / sqrt(d) and the
 * stored norm [ICLR 2026 paper digest, "Step 1: PolarQuant" (R orthogonal,
 * norm kept on the side); Qiita explainer, API table (MSE-only compressor,
 * "TurboQuantMSE")].  Computed in float32, rounded to nearest even for
 * TQ_BF16.  d = 128, 1024, 2048 and 4096 (and the zero-padded d of those D).
 * G*N == 0 is a no-op; nothing is allocated.
 * Errors: TQ_ERR_ARG (null/misaligned pointer, negative size, bad dtype,
 * codebook made on another device), TQ_ERR_UNSUPPORTED (a rotation dimension
 * without device kernels), TQ_ERR_HIP.
 */
int tq_decode_mse(const tq_codebook* cb, const void* packed, int64_t G, int64_t N,
                  void* out, int32_t out_dtype, void* stream);

/*
 * Measurement helper, not part of the method: unquantised logits
 * logits[g][h][n] = q[g][h] . k[g][n] for bf16 q [G][Qg][d] and bf16 keys
 * [G][N][d], float32 accumulation.  The comparator for scoring packed keys.
 * Supported: d == 128, 1 <= Qg <= 8.  Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED,
 * TQ_ERR_HIP.
 */
int tq_dense_logits_bf16(const void* q, const void* keys, int64_t G, int32_t Qg,
                         int64_t N, int32_t d, float* logits, void* stream);

/*
 * Measurement helpers, not part of the method: the ceilings and the clock
 * the benchmark reports beside the kernels.
 *
 * tq_clock_probe: one wave reads the core-clock cycle counter and the
 * constant-rate reference counter, spins until the reference counter has
 * advanced by `ticks`, and writes out[0] = cycles elapsed, out[1] = reference
 * ticks elapsed (device memory, 2 x uint64).  The core clock in MHz is
 * out[0] / out[1] times the reference rate (100 MHz on gfx950).
 * Errors: TQ_ERR_ARG (out NULL or misaligned, ticks <= 0), TQ_ERR_HIP.
 */
int tq_clock_probe(uint64_t* out, int32_t ticks, void* stream);

/*
 * (A measurement helper, as tq_clock_probe.)
 * tq_stream_probe: streams src_bytes from src with 16-byte non-temporal
 * loads and writes dst_bytes to dst with 16-byte non-temporal stores, the
 * writes spread evenly between the reads, over `grid` workgroups of 1024
 * threads (grid <= 0: four per compute unit), each taking a contiguous share
 * of both buffers.  dst_bytes == 0 gives a read-only stream (dst may then be
 * NULL); src_bytes == dst_bytes a copy.  Sizes are multiples of 16; device
 * pointers, 16-byte aligned.  Errors: TQ_ERR_ARG, TQ_ERR_UNSUPPORTED
 * (grid > 2^20), TQ_ERR_HIP.
 */
int tq_stream_probe(const void* src, size_t src_bytes, void* dst, size_t dst_bytes, int32_t grid,
                    void* stream);

/*
 * tq_score_stream_probe: the memory traffic of tq_score_logits at d = 128 in
 * its own launch configuration (same grid, same record loads, same logit
 * stores) without the query preparation and without the estimator's
 * arithmetic: every logit is a fold of its key's record, so the output is
 * meaningless.  The rate it reaches is the ceiling of the scorer's access
 * pattern.  Errors as tq_score_cache.
 */
int tq_score_stream_probe(const tq_codebook* cb, int64_t G, int32_t Qg, const void* packed, int64_t N,
                          float* logits, void* stream);

/* Static description of a status code (library bookkeeping). */
const char* tq_status_string(int status);

/* hipError_t of the last failing HIP call on this thread (0 if none;
 * library bookkeeping). */
int tq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */

// Exercises the host core of the library (tables, codebook set-up and
// teardown, argument validation of every entry point) on the CPU, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against the host stand-ins
// in stubs.cpp.  Prints one line per check group; exits non-zero on the first
// failed expectation.  Test infrastructure, not part of the library.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tq.h"

static int failures = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static void tables(int d, int bits, int kind) {
  const int D = tq_rotation_dim(d), L = 1 << (bits - 1);
  std::vector<double> lv(L), th(L - 1), S(size_t(D) * D), Sr(size_t(D) * D);
  std::vector<int8_t> delta(D);
  EXPECT(tq_codebook_tables_ex(d, bits, D, 7, kind, lv.data(), th.data(), delta.data(), S.data(),
                               Sr.data()) == TQ_OK);
  for (int i = 0; i + 1 < L; ++i) EXPECT(lv[i] < lv[i + 1]);
  for (int i = 0; i + 1 < L; ++i) EXPECT(std::fabs(th[i] - 0.5 * (lv[i] + lv[i + 1])) < 1e-12);
  EXPECT(th[L / 2 - 1] == 0.0);
  for (int i = 0; i < D; ++i) EXPECT(delta[i] == 1 || delta[i] == -1);
  // every row of S has the norm of its row of S R^T (R is orthogonal)
  for (int j = 0; j < D; j += D / 8) {
    double a = 0, b = 0;
    for (int i = 0; i < D; ++i) {
      a += S[size_t(j) * D + i] * S[size_t(j) * D + i];
      b += Sr[size_t(j) * D + i] * Sr[size_t(j) * D + i];
    }
    EXPECT(std::fabs(a - b) < 1e-9 * b);
  }
  // any pointer may be NULL
  EXPECT(tq_codebook_tables_ex(d, bits, D, 7, kind, nullptr, nullptr, nullptr, nullptr, nullptr) == TQ_OK);
}

int main() {
  // rotation dimension rule
  int supported = 0;
  for (int d = -3; d <= 5000; ++d) {
    const int D = tq_rotation_dim(d);
    if (D) {
      ++supported;
      EXPECT(D >= d && (D & (D - 1)) == 0 && D >= 32 && D <= 4096);
    }
  }
  std::printf("rotation_dim: %d supported lengths\n", supported);

  for (int bits = 2; bits <= 4; ++bits) {
    tables(128, bits, TQ_CODEBOOK_GAUSSIAN);
    tables(96, bits, TQ_CODEBOOK_BETA);
  }
  tables(1024, 4, TQ_CODEBOOK_GAUSSIAN);
  tables(1536, 3, TQ_CODEBOOK_GAUSSIAN);
  tables(32, 2, TQ_CODEBOOK_BETA);
  EXPECT(tq_codebook_tables(100, 3, 100, 1, nullptr, nullptr, nullptr, nullptr, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_codebook_tables_ex(128, 3, 128, 1, 9, nullptr, nullptr, nullptr, nullptr, nullptr) == TQ_ERR_ARG);
  std::printf("tables: ok\n");

  // codebook set-up and teardown on the host stand-in device, every size
  const int dims[] = {128, 96, 1024, 768, 2048};
  for (int d : dims)
    for (int bits = 2; bits <= 4; ++bits) {
      tq_codebook* cb = nullptr;
      EXPECT(tq_make_codebook(d, bits, tq_rotation_dim(d), 42, &cb) == TQ_OK && cb);
      int32_t dd = 0, bb = 0, mm = 0;
      uint64_t seed = 0;
      EXPECT(tq_codebook_info(cb, &dd, &bb, &mm, &seed) == TQ_OK && dd == d && bb == bits && seed == 42);
      const int D = tq_rotation_dim(d), L = 1 << (bits - 1);
      std::vector<double> lv(L);
      std::vector<int8_t> delta(D);
      EXPECT(tq_codebook_export(cb, lv.data(), nullptr, delta.data(), nullptr, nullptr) == TQ_OK);
      EXPECT(tq_packed_bytes(cb, 3, 5) == size_t(3) * 5 * ((bits - 1) * D / 8 + D / 8 + 4));
      EXPECT(tq_packed_bytes(cb, -1, 5) == 0);
      tq_free_codebook(cb);
    }
  tq_free_codebook(nullptr);
  {
    tq_codebook* cb = reinterpret_cast<tq_codebook*>(1);
    EXPECT(tq_make_codebook(256, 3, 256, 1, &cb) == TQ_ERR_UNSUPPORTED && cb == nullptr);
    EXPECT(tq_make_codebook(128, 3, 128, 1, nullptr) == TQ_ERR_ARG);
    EXPECT(tq_make_codebook_ex(128, 3, 128, 1, 5, &cb) == TQ_ERR_ARG);
  }
  std::printf("codebooks: ok\n");

  // argument validation of every GPU entry point (nothing is launched: the
  // stand-in launchers would report TQ_ERR_HIP)
  tq_codebook* cb = nullptr;
  EXPECT(tq_make_codebook(128, 3, 128, 42, &cb) == TQ_OK);
  tq_codebook* cw = nullptr;
  EXPECT(tq_make_codebook(1024, 4, 1024, 42, &cw) == TQ_OK);
  alignas(16) static unsigned char buf[1 << 16];
  void* p = buf;
  void* mis = buf + 4;
  float* f = reinterpret_cast<float*>(buf);
  int32_t* i32 = reinterpret_cast<int32_t*>(buf);
  EXPECT(tq_encode_keys(nullptr, p, TQ_F32, 1, 1, p, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_encode_keys(cb, p, 7, 1, 1, p, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_encode_keys(cb, mis, TQ_F32, 1, 1, p, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_encode_keys(cb, nullptr, TQ_F32, 0, 5, nullptr, nullptr) == TQ_OK);
  EXPECT(tq_encode_keys(cb, p, TQ_F32, 1, 1, p, nullptr) == TQ_ERR_HIP);
  EXPECT(tq_append_keys(cb, p, TQ_BF16, 1, 4, p, 3, 0, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_append_keys(cw, p, TQ_BF16, 1, 1, p, 3, 0, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_score_logits(cb, p, TQ_F32, 1, 300, p, 10, f, nullptr, 0, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_score_logits(cb, p, TQ_F32, 1, 4, p, int64_t(1) << 28, f, nullptr, 0, nullptr) ==
         TQ_ERR_UNSUPPORTED);
  EXPECT(tq_score_logits(cw, p, TQ_F32, 1, 4, p, 10, f, nullptr, 0, nullptr) == TQ_ERR_WORKSPACE);
  EXPECT(tq_score_cache(cb, p, TQ_F32, 1, 4, p, 10, 11, f, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_score_topk(cb, p, TQ_F32, 1, 4, p, 10, 5, i32, f, p, 1 << 16, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_score_topk(cw, p, TQ_F32, 1, 4, p, 10, 17, i32, f, p, 1 << 16, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_decode_mse(cb, p, 1, 1, p, 3, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_decode_mse(cb, p, 1, 1, mis, TQ_F32, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_encode_values(cw, p, TQ_F32, 1, 1, p, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_attention_decode(cb, p, TQ_F32, 1, 4, p, p, 0, 0.1f, f, p, 1 << 16, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_attention_decode(cb, p, TQ_F32, 1, 4, p, p, 10, -1.f, f, p, 1 << 16, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_attention_decode(cb, p, TQ_F32, 1, 4, p, p, 10, 0.1f, f, nullptr, 0, nullptr) == TQ_ERR_WORKSPACE);
  EXPECT(tq_append_values(cb, p, TQ_BF16, 1, 4, p, 3, 0, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_append_values(cb, p, TQ_BF16, 1, 2, p, 3, 2, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_append_values(cb, mis, TQ_BF16, 1, 1, p, 3, 0, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_append_values(cw, p, TQ_BF16, 1, 1, p, 3, 0, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_append_values(cb, p, TQ_BF16, 1, 1, p, 3, 2, nullptr) == TQ_ERR_HIP);
  EXPECT(tq_attention_cache(cb, p, TQ_F32, 1, 4, p, p, 10, 11, 0.1f, f, p, 1 << 16, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_attention_cache(cb, p, TQ_F32, 1, 4, p, p, 10, 0, 0.1f, f, p, 1 << 16, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_attention_cache(cb, p, TQ_F32, 1, 4, p, p, 10, 5, 0.1f, f, nullptr, 0, nullptr) ==
         TQ_ERR_WORKSPACE);
  EXPECT(tq_attention_cache(cb, p, TQ_F32, 1, 4, p, p, 10, 5, 0.1f, f, p, 1 << 16, nullptr) == TQ_ERR_HIP);
  EXPECT(tq_attention_decode_noalloc(cb, p, TQ_F32, 1, 4, p, p, 10, NAN, f, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_attention_decode_noalloc(cb, p, TQ_F32, 128, 4, p, p, 20000, 0.1f, f, nullptr) ==
         TQ_ERR_WORKSPACE);
  EXPECT(tq_paged_append_keys(cb, p, TQ_F32, 1, 1, p, 4, 48, i32, 1, i32, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_paged_append_keys(cb, p, TQ_F32, 1, 1, p, 0, 64, i32, 1, i32, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_paged_append_keys(cb, p, TQ_F32, 1, 1, p, 4, 64, reinterpret_cast<int32_t*>(buf + 2), 1, i32,
                              nullptr) == TQ_ERR_ARG);
  EXPECT(tq_paged_score(cw, p, TQ_F32, 1, 4, p, 4, 64, i32, 1, i32, 64, f, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_paged_append_values(cb, p, TQ_F32, 1, 1, p, 4, 48, i32, 1, i32, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_paged_append_values(cb, p, TQ_F32, 1, 1, p, 4, 64, i32, 1, nullptr, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_paged_append_values(cb, p, TQ_F32, 1, 1, p, 4, 64, i32, 1, i32, nullptr) == TQ_ERR_HIP);
  EXPECT(tq_paged_attention(cb, p, TQ_F32, 1, 4, p, p, 4, 64, i32, 1, i32, 0, 0.1f, f, p, 1 << 16, nullptr) ==
         TQ_ERR_ARG);
  EXPECT(tq_paged_attention(cb, p, TQ_F32, 1, 4, p, p, 4, 64, i32, 1, i32, 64, -1.f, f, p, 1 << 16, nullptr) ==
         TQ_ERR_ARG);
  EXPECT(tq_paged_attention(cb, p, TQ_F32, 1, 4, p, p, 4, 64, i32, 1, i32, 64, 0.1f, f, nullptr, 0, nullptr) ==
         TQ_ERR_WORKSPACE);
  EXPECT(tq_paged_attention(cw, p, TQ_F32, 1, 4, p, p, 4, 64, i32, 1, i32, 64, 0.1f, f, p, 1 << 16, nullptr) ==
         TQ_ERR_UNSUPPORTED);
  EXPECT(tq_paged_attention(cb, p, TQ_F32, 1, 4, p, p, 4, 64, i32, 1, i32, 64, 0.1f, f, p, 1 << 16, nullptr) ==
         TQ_ERR_HIP);
  EXPECT(tq_dense_logits_bf16(p, p, 1, 9, 10, 128, f, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_clock_probe(nullptr, 10, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_stream_probe(p, 17, nullptr, 0, 0, nullptr) == TQ_ERR_ARG);
  EXPECT(tq_score_stream_probe(cw, 1, 4, p, 10, f, nullptr) == TQ_ERR_UNSUPPORTED);
  EXPECT(tq_attention_noalloc_max_bytes() > 0);
  for (int s = -6; s <= 1; ++s) EXPECT(tq_status_string(s) != nullptr);
  tq_free_codebook(cb);
  tq_free_codebook(cw);
  std::printf("validation: ok\n");
  if (failures) std::fprintf(stderr, "%d failed expectations\n", failures);
  return failures ? 1 : 0;
}

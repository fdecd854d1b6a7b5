// Internal declarations shared by the host core (tq_host.cpp) and the HIP
// kernels (tq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

namespace tq {

// Constant block the kernels read (one per codebook, device resident).
// Scales: "t" and "c" values are for N(0, 1/d) (unit-vector coordinates).
struct DevConsts {
  float tpos[8];      // positive thresholds t_{L/2}..t_{L-2} (L/2-1 of them), ascending
  float cpos_s[8];    // positive levels c_{L/2}..c_{L-1}, times 2^12 (encoder residual scale)
  float levels[16];   // all L levels, ascending (decoder)
  float alpha[4];     // Walsh coefficients of the levels: s0, s1, s2, s0*s1*s2 terms
  float vtpos[8];     // value quantizer (bits bits): positive thresholds, ascending
  float vlevels[16];  // value quantizer: all 2^bits levels, ascending
  float sqrt_d;       // sqrt(d)
  float inv_sqrt_d;   // 1/sqrt(d)
  float qjl_scale;    // sqrt(pi/2) / m
  float alpha_sum;    // alpha[0] + ... + alpha[3]
  uint32_t dneg[128]; // bit (i % 32) of word i/32 set where delta_i = -1 (d <= 4096)
  uint32_t din;       // length of input rows (and of decoded rows): d, or less when zero-padded to d
  uint32_t pad[3];
};

constexpr float kResidualScale = 4096.0f;  // 2^12: keeps residual hi/lo halves normal

struct Codebook {
  int d = 0, bits = 0, m = 0;   // d: the power of two the method runs in
  int d_in = 0;                 // caller's vector length (d_in <= d; rows are zero-padded to d)
  int kind = 0;               // TQ_CODEBOOK_GAUSSIAN or TQ_CODEBOOK_BETA
  uint64_t seed = 0;
  int device = 0;
  // host tables
  std::vector<double> levels, thresholds, S_rot;
  std::vector<double> vlevels, vthresholds;   // value quantizer: 2^bits levels
  std::vector<int8_t> delta;
  std::vector<double> S;
  DevConsts consts{};
  // device copies
  DevConsts* d_consts = nullptr;
  uint4* d_frag = nullptr;       // -S R^T as float16 (exact), matrix-core A-operand order
  uint4* d_frag16 = nullptr;     // the same for the 16-key bf16 encoder and the scorer's S q: [k-step 4][row block 8][lane 64]
  uint32_t* d_dm16 = nullptr;    // [word 4][k-step 4][4] D as bf16 sign bits for that encoder
  float* d_St = nullptr;         // S transposed, float32 [d][m] (d = 1024)
  uint4* d_Sh = nullptr;         // d = 128 paged append: S R^T as float16 (exact), [column segment 8][row 128][16]
  uint32_t* d_flip_f32 = nullptr;   // [2][d/2] sign-flip words for f32 (d = 128)
  uint4* d_fragW = nullptr;         // S R^T for d >= 1024: [row block d/32][k-step d/16][lane 64]
  float* d_Scol = nullptr;          // column sums of S, float32 [d] (d >= 2048)
  int num_cus = 0;                  // compute units of the device
};

// Launchers (tq_kernels.hip).  Return hipSuccess or the launch error.
// Encode G x N keys into positions [pos, pos + N) of a packed buffer that
// holds Ncap records per group (tq_encode_keys: Ncap = N, pos = 0; d = 1024
// supports only that case).
hipError_t launch_encode(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t N,
                         int64_t Ncap, int64_t pos, void* packed, hipStream_t s);
// Score records [0, N) of a packed buffer holding Ncap per group (d = 1024:
// Ncap = N only).
hipError_t launch_score(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                        const void* packed, int64_t N, int64_t Ncap, float* logits, void* ws,
                        hipStream_t s);
// Paged cache (d = 128): a pool of num_pages pages of page_size records
// (each page laid out as one packed group), a page table [G][ppg] of pool
// page indices, per-group first positions (append) or lengths (score).
// Write-time key append into a contiguous cache of Ncap records per group.
hipError_t launch_append_keys(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t T,
                              int64_t Ncap, int64_t pos, void* packed, hipStream_t s);
// Paged value pool (num_pages pages of page_size value records, the layout
// of a value buffer of num_pages groups) and decode attention over a paged
// key pool and value pool sharing one page table.
hipError_t launch_append_values_paged(const Codebook& cb, const void* values, int dtype, int64_t G, int64_t T,
                                      void* pool, int64_t num_pages, int page_size, const int32_t* table,
                                      int ppg, const int32_t* pos, hipStream_t s);
hipError_t launch_attention_paged(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                                  const void* kpool, const void* vpool, int64_t num_pages, int page_size,
                                  const int32_t* table, int ppg, const int32_t* lens, int64_t Lmax,
                                  float scale, float* out, void* ws, hipStream_t s);
hipError_t launch_encode_paged(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t T,
                               void* pool, int64_t num_pages, int page_size, const int32_t* table,
                               int ppg, const int32_t* pos, hipStream_t s);
hipError_t launch_score_paged(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                              const void* pool, int64_t num_pages, int page_size, const int32_t* table,
                              int ppg, const int32_t* lens, int64_t Lmax, float* logits, hipStream_t s);
hipError_t launch_decode(const Codebook& cb, const void* packed, int64_t G, int64_t N, void* out,
                         int odtype, hipStream_t s);
hipError_t launch_dense_bf16(const void* q, const void* keys, int64_t G, int Qg, int64_t N, int d,
                             float* logits, hipStream_t s);
size_t score_workspace_bytes(const Codebook& cb, int64_t G, int Qg);
// Value records (d = 128): codes in 16-value tiles [G][ceil(N/16)][bits*64] uint32, then uint16
// half norms [G][N].
hipError_t launch_encode_values(const Codebook& cb, const void* values, int dtype, int64_t G,
                                int64_t N, void* vpacked, hipStream_t s);
// Decode attention over packed keys and values (d = 128): logits into the
// workspace, a value pass over key ranges, a combine with the rotation back.
size_t attention_workspace_bytes(const Codebook& cb, int64_t G, int Qg, int64_t N);
// Static device scratch of the no-allocation attention call: its size and the
// current device's address of it (looked up once per device).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_address(void** ptr);
hipError_t launch_attention(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                            const void* kpacked, const void* vpacked, int64_t N, int64_t Ncap,
                            float scale, float* out, void* ws, hipStream_t s);
// Write-time value append (d = 128): T values per group into records pos ..
// pos + T - 1 of a value cache of Ncap records per group.
hipError_t launch_append_values(const Codebook& cb, const void* values, int dtype, int64_t G, int64_t T,
                                void* vpacked, int64_t Ncap, int64_t pos, hipStream_t s);
// d = 1024 (tq_wide.hip)
hipError_t launch_decode_wide(const Codebook& cb, const void* packed, int64_t G, int64_t N, void* out,
                              int odtype, hipStream_t s);
hipError_t launch_encode_wide(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t N,
                              void* packed, hipStream_t s);
size_t score_wide_prep_bytes(int64_t G, int Qg);
// d = 2048 and 4096 (tq_wider.hip)
hipError_t launch_encode_wider(const Codebook& cb, const void* keys, int dtype, int64_t G, int64_t N,
                               void* packed, hipStream_t s);
size_t score_wider_prep_bytes(const Codebook& cb, int64_t G, int Qg);
hipError_t launch_score_wider(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                              const void* packed, int64_t N, float* logits, void* ws, hipStream_t s);
hipError_t launch_decode_wider(const Codebook& cb, const void* packed, int64_t G, int64_t N, void* out,
                               int odtype, hipStream_t s);
size_t topk_wide_bytes(const Codebook& cb, int64_t G, int Qg, int64_t N, int K);
hipError_t launch_score_wide(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                             const void* packed, int64_t N, float* logits, void* ws, hipStream_t s);
hipError_t launch_topk_wide(const Codebook& cb, const void* q, int qdtype, int64_t G, int Qg,
                            const void* packed, int64_t N, int K, int32_t* idx, float* scores,
                            void* ws, hipStream_t s);
// measurement helpers (not part of the method)
hipError_t launch_clock_probe(uint64_t* out, uint32_t ticks, hipStream_t s);
hipError_t launch_stream_probe(const void* src, size_t src_bytes, void* dst, size_t dst_bytes, int grid,
                               hipStream_t s);
hipError_t launch_score_stream_probe(const Codebook& cb, int64_t G, int Qg, const void* packed, int64_t N,
                                     float* logits, hipStream_t s);
constexpr int kMaxTopKAbi = 16;
bool encode_supported(const Codebook& cb);
bool score_supported(const Codebook& cb);

}  // namespace tq

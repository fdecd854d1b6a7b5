// Host-only stand-ins for the HIP runtime calls and the kernel launchers the
// host core (kv_cache_vector_rotate_amd/csrc/tq_host.cpp) uses, so that the
// host core builds as plain C++ and runs on a machine without a GPU under
// AddressSanitizer and UndefinedBehaviorSanitizer: "device" memory is host
// memory, one device with 256 compute units, and every launcher reports
// hipErrorNotSupported (the C ABI turns that into TQ_ERR_HIP).  Test
// infrastructure, not part of the library.
#include "../../kv_cache_vector_rotate_amd/csrc/tq_internal.h"

#include <cstdlib>
#include <cstring>

extern "C" {
hipError_t hipMalloc(void** ptr, size_t size) {
  *ptr = std::malloc(size ? size : 1);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* ptr) {
  std::free(ptr);
  return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind) {
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}
}

namespace tq {
namespace {
constexpr hipError_t kNo = hipErrorNotSupported;
}
bool encode_supported(const Codebook& cb) {
  return cb.d == 128 || cb.d == 1024 || cb.d == 2048 || cb.d == 4096;
}
bool score_supported(const Codebook& cb) { return encode_supported(cb); }
size_t score_workspace_bytes(const Codebook& cb, int64_t G, int Qg) {
  return cb.d >= 1024 ? size_t(G) * Qg * (2 * size_t(cb.d) + 4) * 4 : 0;
}
size_t attention_workspace_bytes(const Codebook&, int64_t G, int Qg, int64_t N) {
  return size_t(G) * Qg * N * 4 + 4096;
}
size_t topk_wide_bytes(const Codebook&, int64_t G, int Qg, int64_t N, int K) {
  return size_t(G) * Qg * (8 * 1024 + size_t(K) * 8 * (N / 1024 + 1));
}
hipError_t scratch_address(void**) { return kNo; }
hipError_t launch_encode(const Codebook&, const void*, int, int64_t, int64_t, int64_t, int64_t, void*,
                         hipStream_t) { return kNo; }
hipError_t launch_score(const Codebook&, const void*, int, int64_t, int, const void*, int64_t, int64_t,
                        float*, void*, hipStream_t) { return kNo; }
hipError_t launch_decode(const Codebook&, const void*, int64_t, int64_t, void*, int, hipStream_t) {
  return kNo;
}
hipError_t launch_dense_bf16(const void*, const void*, int64_t, int, int64_t, int, float*, hipStream_t) {
  return kNo;
}
hipError_t launch_encode_values(const Codebook&, const void*, int, int64_t, int64_t, void*, hipStream_t) {
  return kNo;
}
hipError_t launch_attention(const Codebook&, const void*, int, int64_t, int, const void*, const void*,
                            int64_t, int64_t, float, float*, void*, hipStream_t) { return kNo; }
hipError_t launch_append_values_paged(const Codebook&, const void*, int, int64_t, int64_t, void*, int64_t, int,
                                      const int32_t*, int, const int32_t*, hipStream_t) { return kNo; }
hipError_t launch_attention_paged(const Codebook&, const void*, int, int64_t, int, const void*, const void*,
                                  int64_t, int, const int32_t*, int, const int32_t*, int64_t, float, float*,
                                  void*, hipStream_t) { return kNo; }
hipError_t launch_append_keys(const Codebook&, const void*, int, int64_t, int64_t, int64_t, int64_t, void*,
                              hipStream_t) { return kNo; }
hipError_t launch_append_values(const Codebook&, const void*, int, int64_t, int64_t, void*, int64_t, int64_t,
                                hipStream_t) { return kNo; }
hipError_t launch_topk_wide(const Codebook&, const void*, int, int64_t, int, const void*, int64_t, int,
                            int32_t*, float*, void*, hipStream_t) { return kNo; }
hipError_t launch_encode_paged(const Codebook&, const void*, int, int64_t, int64_t, void*, int64_t, int,
                               const int32_t*, int, const int32_t*, hipStream_t) { return kNo; }
hipError_t launch_score_paged(const Codebook&, const void*, int, int64_t, int, const void*, int64_t, int,
                              const int32_t*, int, const int32_t*, int64_t, float*, hipStream_t) {
  return kNo;
}
hipError_t launch_clock_probe(uint64_t*, uint32_t, hipStream_t) { return kNo; }
hipError_t launch_stream_probe(const void*, size_t, void*, size_t, int, hipStream_t) { return kNo; }
hipError_t launch_score_stream_probe(const Codebook&, int64_t, int, const void*, int64_t, float*,
                                     hipStream_t) { return kNo; }
}  // namespace tq

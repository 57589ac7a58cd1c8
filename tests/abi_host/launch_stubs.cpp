// Host-only stand-ins for the kernel launchers and the two HIP runtime calls
// the C ABI makes, so that the ABI's argument checks, workspace carving and
// pointer handling (api.cpp, host_sizes.cpp) can be built and run under
// AddressSanitizer / UndefinedBehaviorSanitizer on a machine without a GPU.
// Each launcher records that it was reached and the pointers it was given.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>

#include "../../long_context_sparse_apply_amd/csrc/sa_internal.hpp"
#include "launch_stubs.hpp"

StubLog g_log;

// Fake address ranges: [kDevLo, kDevHi) device memory, [kPinLo, kPinHi) pinned
// host memory (its device view is the address + kPinShift), anything else
// unregistered host memory.
extern "C" hipError_t hipPointerGetAttributes(hipPointerAttribute_t* a, const void* p) {
  std::memset(a, 0, sizeof(*a));
  const uintptr_t x = reinterpret_cast<uintptr_t>(p);
  if (x >= kDevLo && x < kDevHi) {
    a->type = hipMemoryTypeDevice;
    a->devicePointer = const_cast<void*>(p);
    return hipSuccess;
  }
  if (x >= kPinLo && x < kPinHi) {
    a->type = hipMemoryTypeHost;
    a->hostPointer = const_cast<void*>(p);
    a->devicePointer = reinterpret_cast<void*>(x + kPinShift);
    return hipSuccess;
  }
  ++g_log.last_error_set;
  return hipErrorInvalidValue;
}

extern "C" hipError_t hipGetLastError(void) {
  g_log.last_error_set = 0;
  return hipSuccess;
}

namespace sa {

static hipError_t hit(const char* name, const void* a = nullptr, const void* b = nullptr,
                      const void* c = nullptr) {
  ++g_log.launches;
  g_log.name = name;
  g_log.p[0] = a;
  g_log.p[1] = b;
  g_log.p[2] = c;
  return g_log.fail ? hipErrorLaunchFailure : hipSuccess;
}

hipError_t launch_rope(const void* x, void* out, int, int, int, int, int, const int32_t*, int,
                       const RopeFreq&, hipStream_t) {
  return hit("rope", x, out);
}
hipError_t launch_kv_append(const void* k_new, const void*, int, int, int, int, int, int,
                            const int32_t*, const RopeFreq&, int, const int32_t*, int, void*,
                            void* k_rest, void* v_out, hipStream_t) {
  return hit("kv_append", k_new, k_rest, v_out);
}
hipError_t launch_rope_pool(const void* q, const void*, int, int, int, int, int, int, int, int,
                            int, const RopeFreq&, void*, float, void*, float* pq, float* pk,
                            hipStream_t) {
  return hit("rope_pool", q, pq, pk);
}
hipError_t launch_block_gemm(const float* pq, const float* pk, int, int, int, int, int, float, int,
                             float* scores, hipStream_t) {
  return hit("block_gemm", pq, pk, scores);
}
hipError_t launch_topk(const float* scores, int64_t, int, const int32_t*, const int32_t*, int, int,
                       int, int32_t* idx, int, int32_t* cnt, hipStream_t) {
  return hit("topk", scores, idx, cnt);
}
hipError_t launch_prefill(const void* q, const void*, const void*, int, int, int, int, int, int,
                          int, const int32_t*, const int32_t*, int, int, float, void* out, float*,
                          hipStream_t) {
  return hit("prefill", q, out);
}
hipError_t launch_token_collect(const void* q, const void*, int, int, int, int, int, int,
                                const int32_t*, const int32_t*, int, int, float,
                                const TokenCollect&, hipStream_t) {
  return hit("token_collect", q);
}
hipError_t launch_token_topk(const void* q, const void* k, int, int, int, int, int, int,
                             const int32_t*, const int32_t*, int, int, float, int, int32_t*, int,
                             int32_t*, void* ws, hipStream_t) {
  return hit("token_topk", q, k, ws);
}
hipError_t launch_token_score(const void* q, const void* k, int, int, int, int, int, int,
                              const int32_t*, const int32_t*, int, int, float, float* scores,
                              hipStream_t) {
  return hit("token_score", q, k, scores);
}
hipError_t launch_decode(const void* q, const void*, const void* k_rest, const void* v, int, int,
                         int, int, int, int, const int32_t*, const int32_t*, int, int,
                         const int32_t*, const int32_t*, int, float, void*, float*, void*,
                         hipStream_t) {
  return hit("decode", q, k_rest, v);
}
hipError_t launch_sfa_sparsify(const void* x, void* out, int, int64_t, int, int, hipStream_t) {
  return hit("sfa", x, out);
}
hipError_t launch_calibrate(const void* q, const void*, int, int, int, int, int, int, int,
                            int32_t*, int32_t*, void* ws, hipStream_t) {
  return hit("calibrate", q, ws);
}

hipError_t decode_static_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(kDevLo + 0x800000);
  return hipSuccess;
}

}  // namespace sa

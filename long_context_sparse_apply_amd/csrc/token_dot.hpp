// The arithmetic of one token's importance score.
//
// "FASA: Frequency-aware Sparse Attention", sec. 2.B item 1: a token's score
// sums, over the dominant frequency chunks only, the products of the query's
// and the key's channels.  Here: one fp32 fused multiply-add per channel, in
// the stored (slab) channel order, starting from zero, with the query slice
// already multiplied by the softmax scale.  Every kernel that scores a token
// uses this function, so their scores agree bit for bit.
#pragma once

#include "sa_common.hpp"

namespace sa {

// q: NDC scaled query channels (16-byte aligned, typically in LDS);
// kv: the key's NDC channels in the same order, as fp32.
template <int NDC>
__device__ __forceinline__ float token_dot(const float* __restrict__ q, const float (&kv)[NDC]) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NDC; j += 4) {
    const float4 qv = *reinterpret_cast<const float4*>(q + j);
    acc = fmaf(qv.x, kv[j], acc);
    acc = fmaf(qv.y, kv[j + 1], acc);
    acc = fmaf(qv.z, kv[j + 2], acc);
    acc = fmaf(qv.w, kv[j + 3], acc);
  }
  return acc;
}

// One stored slab row of NDC channels (16-byte aligned, NDC * sizeof(T) a
// multiple of 16) as fp32, read with 16-byte loads.
template <typename T, int NDC>
__device__ __forceinline__ void load_slab_row(const T* __restrict__ row, float (&kv)[NDC]) {
  constexpr int PER = 16 / static_cast<int>(sizeof(T));  // channels per 16 bytes
  static_assert(NDC % PER == 0, "slab row is whole 16-byte words");
  const uint4* w = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int c = 0; c < NDC / PER; ++c) {
    const uint4 x = w[c];
    if constexpr (sizeof(T) == 2) {
      float tmp[8];
      Elem<uint16_t>::unpack8(x, tmp);
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[c * 8 + e] = tmp[e];
    } else {
      kv[c * 4 + 0] = __uint_as_float(x.x);
      kv[c * 4 + 1] = __uint_as_float(x.y);
      kv[c * 4 + 2] = __uint_as_float(x.z);
      kv[c * 4 + 3] = __uint_as_float(x.w);
    }
  }
}

}  // namespace sa

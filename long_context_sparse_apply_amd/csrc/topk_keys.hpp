// Order-preserving keys of fp32 scores and the (key, column) composite that
// every top-k selection compares: score descending, then column ascending.
//
// "Prism: Spectral-Aware Block-Sparse Attention", sec. 1 (a subset of relevant
// blocks) and "FASA: Frequency-aware Sparse Attention", sec. 2.B (the critical
// token subset T_t) select by score; the order here makes that selection
// unique.  NaN ranks as -inf and -0 equals +0.
#pragma once

#include "sa_common.hpp"

namespace sa {

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN ranks as -inf
  if ((u & 0x7fffffffu) == 0u) u = 0u;                   // -0 equals +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);     // candidates: key >= 0x007fffff
}

// The unique 64-bit composite key << 32 | (0xffffffff - column): its k
// largest values are exactly the k best columns.
__device__ __forceinline__ uint64_t composite(uint32_t key, int idx) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int comp_col(uint64_t c) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(c & 0xffffffffu));
}

// A threshold key as a float test.  For a value that is not NaN, key(v) >=
// t_low is v >= f_low, f_low the float whose key is t_low; a t_low at or
// below the key of -inf takes every value (NaN ranks as -inf), one above the
// key of +inf gives a NaN f_low that no value passes.
struct KeyThreshold {
  bool take_all;
  float f_low;
  __device__ __forceinline__ explicit KeyThreshold(uint32_t t_low)
      : take_all(t_low <= 0x007fffffu),
        f_low((t_low & 0x80000000u) ? __uint_as_float(t_low & 0x7fffffffu) : __uint_as_float(~t_low)) {}
  __device__ __forceinline__ bool qualifies(float v) const { return take_all || v >= f_low; }
};

// A threshold key no score passes (above the key of +inf).
constexpr uint32_t kNoCandidates = 0xffffffffu;

// Candidate lists of the fused token top-k, in its workspace.  The scoring
// work-group of a (batch, KV head) and a tile of kCollectTile tokens gives
// each of its kCollectWaves waves a private list of kCollectSlots entries per
// row (b * Hq + h), so no list is shared and no atomic is needed: per (row,
// tile, wave) the number of qualifying tokens (it may exceed the slots: the
// selection then reads the row again) and the first kCollectSlots of them as
// score bits << 32 | token (the selection forms the composites).
struct TokenCollect {
  const uint32_t* thr;  // [rows] threshold keys
  int* cnt;             // [rows, tiles, kCollectWaves]
  uint64_t* cand;       // [rows, tiles, kCollectWaves, kCollectSlots]
  int tiles;            // ceil(Lmax / kCollectTile)
};

}  // namespace sa

// Host-side size arithmetic of the library: rotation frequencies, workspace
// and LDS sizes.  Plain C++ with no device code, shared by the C ABI's checks
// (api.cpp) and the launchers, and built on its own for the host-only
// sanitizer test of the ABI.
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "sa_internal.hpp"
#include "sa_limits.hpp"

namespace sa {

namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

RopeFreq make_rope_freq(int d, double theta) {
  RopeFreq r{};
  const int P = d / 2;
  for (int i = 0; i < P && i < kMaxPairs; ++i)
    r.f[i] = std::pow(theta, -2.0 * i / d) / (2.0 * M_PI);
  return r;
}

int decode_splits(int max_k) {
  const int s = (max_k + kDecChunk - 1) / kDecChunk;
  return s < 1 ? 1 : s;
}

size_t decode_ws_bytes(int B, int Hq, int max_k) {
  const size_t parts = static_cast<size_t>(B) * Hq * decode_splits(max_k);
  return parts * (2 + 128) * sizeof(float) + 256;
}

DecodePlan decode_plan(int B, int Hq, int max_k) {
  const int nchunks = decode_splits(max_k);
  const int64_t rows = static_cast<int64_t>(B) * Hq;
  const int cpw = rows >= 2 * kChipCUs ? nchunks : 1;
  return DecodePlan{(nchunks + cpw - 1) / cpw, cpw};
}

size_t decode_scratch_bytes(int B, int Hq, int max_k) {
  const DecodePlan p = decode_plan(B, Hq, max_k);
  if (p.splits <= 1) return 0;
  return static_cast<size_t>(B) * Hq * p.splits * (2 + 128) * sizeof(float);
}

// LDS of one long-row top-k work-group: candidate composites, the radix
// histogram, the row's bitmap and per-wave scratch
size_t topk_lds_bytes(int cols, int cap) {
  const size_t words = (static_cast<size_t>(cols) + 31) / 32;
  return static_cast<size_t>(cap) * 8 + kBins * 4 + words * 4 + (kLongThreads / kWave + 4) * 4;
}

// LDS of a fused-selection work-group: the candidate / bitmap region, the
// radix histogram and the scan scalars.
size_t token_select_lds_bytes(int cols, int cap) {
  return static_cast<size_t>(token_select_region(cols, cap)) + kBins * 4 +
         (kLongThreads / kWave + 4) * 4;
}

// Candidate buffer of a long row: k plus a quarter plus 1024 (the sampled
// threshold overshoots k by a few standard deviations), at most kMaxCap.
int topk_cap(int k) {
  int cap = k + k / 4 + 1024;
  cap = ((cap + 63) / 64) * 64;
  return cap > kMaxCap ? kMaxCap : cap;
}

// A row's candidate buffer in the fused token selection: twice k plus 1024
// (a threshold sampled from a few thousand tokens overshoots k by more), at
// most kMaxCap.
int token_topk_cap(int k) {
  int cap = 2 * k + 1024;
  cap = ((cap + 63) / 64) * 64;
  return cap > kMaxCap ? kMaxCap : cap;
}

// Workspace of the fused token top-k: thresholds [rows], list counts
// [rows, tiles, waves], lists [rows, tiles, waves, kCollectSlots] and the
// rows' sample keys [rows, kTokenSampleKeys], each part 256-byte aligned.
size_t token_topk_ws_bytes(int64_t rows, int Lmax) {
  const size_t tiles = static_cast<size_t>((Lmax + kCollectTile - 1) / kCollectTile);
  const size_t lists = static_cast<size_t>(rows) * tiles * kCollectWaves;
  return align256(static_cast<size_t>(rows) * 4) + align256(lists * 4) +
         align256(lists * kCollectSlots * 8) + static_cast<size_t>(rows) * kTokenSampleKeys * 4;
}

// Workspace of the offline calibration: full and pair scores, their
// selections, and the per-pair counts, each part 256-byte aligned.
size_t calib_ws_bytes(int Hq, int M, int L, int d, int Hkv, int kcal) {
  const size_t rows = static_cast<size_t>(Hq) * M;
  const size_t P = static_cast<size_t>(d) / 2;
  return align256(rows * L * 4) + align256(rows * P * L * 4) + align256(rows * kcal * 4) +
         align256(rows * 4) + align256(rows * P * kcal * 4) + align256(rows * P * 4) +
         align256(static_cast<size_t>(Hkv) * P * 4) * 2 + align256(static_cast<size_t>(Hkv) * 4) +
         256;
}

}  // namespace sa

// Sizes shared by the kernels and the host-side size arithmetic (plain C++,
// no device code), so the workspace and LDS sizes the host computes and the
// layouts the kernels assume come from one definition.
#pragma once

namespace sa {

constexpr int kWave = 64;  // wavefront width on gfx950

// split-K decode attention: tokens per work-group chunk, waves per work-group
constexpr int kDecChunk = 256;
constexpr int kDecWaves = 4;
constexpr int kChipCUs = 256;  // MI355X compute units

// long-row top-k: threads per row, radix digit, largest LDS candidate
// buffer (64-bit composites), longest row the host accepts
constexpr int kLongThreads = 512;
constexpr int kDigit = 11;
constexpr int kBins = 1 << kDigit;
constexpr int kMaxCap = 8192;
constexpr int kMaxLongCols = 262144;

// candidate lists of the fused token top-k: tokens a scoring tile covers,
// waves of a scoring work-group (one private list each per row), entries a
// list keeps
constexpr int kCollectTile = 4096;
constexpr int kCollectWaves = 4;
constexpr int kCollectSlots = 256;
// sample keys a row of the fused token top-k keeps in its workspace
constexpr int kTokenSampleKeys = 4096;

// fused selection's LDS region: the candidate buffer (cap 64-bit composites)
// or, on the exact fallback, the row's selection bitmap followed by a buffer
// of at least kSelFallbackBuf composites (bytes, a multiple of 16)
constexpr int kSelFallbackBuf = 2048;
constexpr long long token_select_region(int cols, int cap) {
  const long long bitmap = ((static_cast<long long>(cols) + 31) / 32 * 4 + 15) / 16 * 16;
  const long long a = static_cast<long long>(cap) * 8;
  const long long b = bitmap + static_cast<long long>(kSelFallbackBuf) * 8;
  return a > b ? a : b;
}

}  // namespace sa

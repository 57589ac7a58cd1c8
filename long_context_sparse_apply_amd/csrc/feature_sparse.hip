// k-sparse feature codes for Sparse Feature Attention.
//
// "Scaling Attention via Feature Sparsity", sec. 2: each query and key
// vector keeps its k channels of largest magnitude and zeroes the rest; a
// score then only sums over the channels active in both codes.  The score of
// two zero-filled codes is exactly that sum, so the attention itself runs on
// the matrix unit (the block-sparse prefill kernel with every causal block
// listed): on gfx950 a dense 32x32x16 MFMA over the masked tiles produces the
// intersection scores faster than gathering the active channels would.
//
// One wave per row, the row in registers (channel j*64 + lane in slot j).
// The k-th largest magnitude key is found by a bitwise search with ballot
// counts; ties on it go to the lower channels through a running count in
// channel order.  NaN ranks below every number.  Values are copied bit for
// bit; in-place use is allowed (a wave reads its whole row before writing).
#include "sa_common.hpp"

namespace sa {

template <typename T, int E>
__global__ __launch_bounds__(256) void sfa_sparsify_kernel(const T* __restrict__ x, T* out,
                                                           int64_t rows, int kf) {
  constexpr int D = E * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (row >= rows) return;
  const T* xr = x + row * D;
  T raw[E];
  uint32_t key[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    raw[j] = xr[j * kWave + lane];
    const uint32_t m = __float_as_uint(Elem<T>::load1(&raw[j])) & 0x7fffffffu;
    key[j] = m > 0x7f800000u ? 0u : m;  // NaN ranks lowest
  }
  uint32_t T_ = 0;
  int need = 0;
  if (kf < D) {
    // a bf16 magnitude occupies bits 30..16 of its fp32 pattern: at most 15
    // steps, fewer once exactly kf magnitudes reach the bits fixed so far
    // (they are then the kept channels whatever the lower bits)
    constexpr int kLowBit = sizeof(T) == 2 ? 16 : 0;
    for (int bit = 30; bit >= kLowBit; --bit) {
      const uint32_t t = T_ | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < E; ++j) cnt += __popcll(__ballot(key[j] >= t));
      if (cnt >= kf) T_ = t;
      if (cnt == kf) break;
    }
    int gt = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) gt += __popcll(__ballot(key[j] > T_));
    need = kf - gt;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int eq_seen = 0;
  T* orow = out + row * D;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    bool keep = true;
    if (kf < D) {
      const bool eq = key[j] == T_;
      const uint64_t eqm = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(eqm & below);
      eq_seen += __popcll(eqm);
      keep = key[j] > T_ || (eq && eq_rank < need);
    }
    orow[j * kWave + lane] = keep ? raw[j] : T(0);
  }
}

hipError_t launch_sfa_sparsify(const void* x, void* out, int dtype, int64_t rows, int d, int kf,
                               hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
#define SA_SF(T, E) \
  sfa_sparsify_kernel<T, E><<<grid, 256, 0, st>>>(static_cast<const T*>(x), static_cast<T*>(out), rows, kf)
  if (dtype == kBF16) {
    if (d == 128) { SA_SF(uint16_t, 2); } else { SA_SF(uint16_t, 1); }
  } else {
    if (d == 128) { SA_SF(float, 2); } else { SA_SF(float, 1); }
  }
#undef SA_SF
  return hipGetLastError();
}

}  // namespace sa

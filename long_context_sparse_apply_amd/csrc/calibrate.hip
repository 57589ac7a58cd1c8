// Offline calibration of the dominant rotary pairs.
//
// "FASA: Frequency-aware Sparse Attention", sec. 2.A (a small fixed set of
// dominant frequency chunks reproduces a head's context selection) and sec.
// 2.B item 1 (that set comes from a one-time offline calibration).  The
// pages give no criterion; the one computed here: for each calibration
// query, the overlap between the top-k keys by one pair's partial score
// (q_i k_i + q_{i+P} k_{i+P}) and the top-k keys by the full score, summed
// per KV head over its query heads and calibration queries; the dominant
// set is the n_dom pairs with the largest sums (ties to the lower pair).
//
// Steps (the top-k selections use the library's own top-k kernels):
//   calib_score_kernel   full and pair scores of every (query, key), fp32
//   top-k of every full row and every pair row
//   calib_overlap_kernel per (query head, calibration query): the full
//                        selection as an LDS bitmap, then each pair's hits,
//                        added to the KV head's integer counts
//   the counts as floats, then their top-n_dom per KV head.
// Scores are decided in fp32: the full score adds the channel products in
// ascending channel order, a pair score is one rounding of its two products;
// with bf16 inputs every product is exact, so the scores, the selections and
// the integer counts do not depend on the launch shape.
#include "sa_common.hpp"
#include "sa_internal.hpp"

namespace sa {

// One thread per key, one work-group per (256 keys, calibration query m, query head h).
template <int D>
__global__ __launch_bounds__(256) void calib_score_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k, int Hq,
                                                          int Hkv, int M, int L,
                                                          float* __restrict__ full,
                                                          float* __restrict__ pairs) {
  constexpr int P = D / 2;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int m = blockIdx.y;
  const int h = blockIdx.z;
  const int g = h / (Hq / Hkv);
  __shared__ float s_q[D];
  const int64_t row = static_cast<int64_t>(h) * M + m;
  if (threadIdx.x < D) s_q[threadIdx.x] = bf16_to_f32(q[row * D + threadIdx.x]);
  __syncthreads();
  if (t >= L) return;
  const uint16_t* kr = k + (static_cast<int64_t>(g) * L + t) * D;
  float pa[P];
  float acc = 0.f;
  // first halves of the pairs: channels 0 .. P-1
#pragma unroll
  for (int c8 = 0; c8 < P / 8; ++c8) {
    float kv[8];
    Elem<uint16_t>::load8(kr + 8 * c8, kv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pa[8 * c8 + e] = s_q[8 * c8 + e] * kv[e];  // exact: a product of two bf16 values
      acc += pa[8 * c8 + e];
    }
  }
  // second halves: channels P .. D-1, pair i = channels i and i + P
  float* prow = pairs + row * P * L + t;
#pragma unroll
  for (int c8 = 0; c8 < P / 8; ++c8) {
    float kv[8];
    Elem<uint16_t>::load8(kr + P + 8 * c8, kv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 8 * c8 + e;
      const float pb = s_q[P + i] * kv[e];
      acc += pb;
      prow[static_cast<int64_t>(i) * L] = pa[i] + pb;
    }
  }
  full[row * L + t] = acc;
}

// One work-group per (calibration query m, query head h).
__global__ __launch_bounds__(256) void calib_overlap_kernel(
    const int32_t* __restrict__ full_idx, const int32_t* __restrict__ pair_idx, int Hq, int Hkv,
    int M, int L, int P, int kcal, uint32_t* __restrict__ counts) {
  extern __shared__ uint32_t s_bits[];  // L bits, then P counters
  const int m = blockIdx.x;
  const int h = blockIdx.y;
  const int g = h / (Hq / Hkv);
  const int words = (L + 31) / 32;
  uint32_t* s_cnt = s_bits + words;
  const int64_t row = static_cast<int64_t>(h) * M + m;
  for (int w = threadIdx.x; w < words; w += 256) s_bits[w] = 0u;
  for (int i = threadIdx.x; i < P; i += 256) s_cnt[i] = 0u;
  __syncthreads();
  const int32_t* fi = full_idx + row * kcal;
  for (int e = threadIdx.x; e < kcal; e += 256) {
    const int t = fi[e];
    if (t >= 0 && t < L) atomicOr(&s_bits[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  const int32_t* pi = pair_idx + row * P * kcal;
  for (int e = threadIdx.x; e < P * kcal; e += 256) {
    const int t = pi[e];
    if (t >= 0 && t < L && ((s_bits[t >> 5] >> (t & 31)) & 1u)) atomicAdd(&s_cnt[e / kcal], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < P; i += 256)
    if (s_cnt[i]) atomicAdd(&counts[static_cast<int64_t>(g) * P + i], s_cnt[i]);
}

__global__ void calib_fill_kernel(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ void calib_to_float_kernel(const uint32_t* __restrict__ c, float* __restrict__ f,
                                      int32_t* __restrict__ ci, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    f[i] = static_cast<float>(c[i]);  // exact: counts stay far below 2^24
    if (ci) ci[i] = static_cast<int32_t>(c[i]);
  }
}

static size_t al(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }


hipError_t launch_calibrate(const void* q, const void* k, int Hq, int Hkv, int M, int L, int d,
                            int kcal, int n_dom, int32_t* dom_out, int32_t* counts_out, void* ws,
                            hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(Hq) * M;
  const int P = d / 2;
  char* w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~static_cast<uintptr_t>(255));
  auto take = [&](size_t bytes) { char* p = w; w += al(bytes); return p; };
  float* full = reinterpret_cast<float*>(take(static_cast<size_t>(rows) * L * 4));
  float* pairs = reinterpret_cast<float*>(take(static_cast<size_t>(rows) * P * L * 4));
  int32_t* fidx = reinterpret_cast<int32_t*>(take(static_cast<size_t>(rows) * kcal * 4));
  int32_t* fcnt = reinterpret_cast<int32_t*>(take(static_cast<size_t>(rows) * 4));
  int32_t* pidx = reinterpret_cast<int32_t*>(take(static_cast<size_t>(rows) * P * kcal * 4));
  int32_t* pcnt = reinterpret_cast<int32_t*>(take(static_cast<size_t>(rows) * P * 4));
  uint32_t* counts = reinterpret_cast<uint32_t*>(take(static_cast<size_t>(Hkv) * P * 4));
  float* fcounts = reinterpret_cast<float*>(take(static_cast<size_t>(Hkv) * P * 4));
  int32_t* dcnt = reinterpret_cast<int32_t*>(take(static_cast<size_t>(Hkv) * 4));

  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const dim3 sgrid((L + 255) / 256, M, Hq);
  if (d == 128)
    calib_score_kernel<128><<<sgrid, 256, 0, st>>>(qq, kk, Hq, Hkv, M, L, full, pairs);
  else
    calib_score_kernel<64><<<sgrid, 256, 0, st>>>(qq, kk, Hq, Hkv, M, L, full, pairs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_topk(full, rows, L, nullptr, nullptr, kcal, 0, 0, fidx, kcal, fcnt, st);
  if (e != hipSuccess) return e;
  e = launch_topk(pairs, rows * P, L, nullptr, nullptr, kcal, 0, 0, pidx, kcal, pcnt, st);
  if (e != hipSuccess) return e;
  const int nc = Hkv * P;
  calib_fill_kernel<<<(nc + 255) / 256, 256, 0, st>>>(counts, nc);
  const size_t lds = (static_cast<size_t>(L + 31) / 32 + P) * 4;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&calib_overlap_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  calib_overlap_kernel<<<dim3(M, Hq), 256, lds, st>>>(fidx, pidx, Hq, Hkv, M, L, P, kcal, counts);
  calib_to_float_kernel<<<(nc + 255) / 256, 256, 0, st>>>(counts, fcounts, counts_out, nc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk(fcounts, Hkv, P, nullptr, nullptr, n_dom, 0, 0, dom_out, n_dom, dcnt, st);
}

}  // namespace sa

// Token importance from the dominant frequency chunks only.
//
// "FASA: Frequency-aware Sparse Attention", sec. 2.B item 1 (Token Importance
// Predictor: scores aggregated from the dominant frequency chunks) and sec.
// 2.C (the computation-optimised variant reads only a sparse subset of the
// key states).
//
//   s(b, h, t) = scale * sum_{i in D_g} (q_i k_{t,i} + q_{i+P} k_{t,i+P})
//
// One work-group streams 256 cached tokens of one (batch, KV head) and scores
// them for all Hq/Hkv query heads of the group, so every key byte is read once
// per group.  A token row is split over LPT lanes that each load 16 bytes
// (8 channels, bf16): in the standard layout the whole d-channel row is read
// (the dominant pairs are scattered through it) and multiplied by a query whose
// non-dominant channels are zero; in the slab layout only the 2*n_dom dominant
// channels are stored contiguously and read.  Per-lane partial dots are summed
// across the LPT lanes with xor shuffles; scores are staged in LDS and written
// as contiguous rows.
#include "sa_common.hpp"

namespace sa {

constexpr int kTokPerWG = 256;

template <typename T, int ROW, int GRP>
__global__ __launch_bounds__(256) void token_score_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int Hq, int Hkv, int Lmax, int d,
    const int32_t* __restrict__ cache_len, const int32_t* __restrict__ dom, int n_dom, int slab,
    float scale, float* __restrict__ scores) {
  constexpr int LPT = ROW / 8;          // lanes per token row
  constexpr int TPI = kWave / LPT;      // tokens per wave per step
  constexpr int WAVES = 256 / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int sub = lane % LPT;
  const int tok_in_step = lane / LPT;
  const int t0 = blockIdx.x * kTokPerWG;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int P = d / 2;
  const int L = cache_len[b];

  __shared__ float s_q[GRP][128];
  __shared__ uint64_t s_dmask;
  __shared__ int s_ch[128];
  __shared__ float s_out[GRP][kTokPerWG];

  // channel held by slab/row position c, and the dominant-pair mask
  if (tid == 0) {
    uint64_t m = 0;
    for (int j = 0; j < n_dom; ++j) m |= 1ull << dom[g * n_dom + j];
    s_dmask = m;
  }
  __syncthreads();
  if (tid < ROW) {
    int ch = tid;
    if (slab) {
      const int j = tid % n_dom;
      ch = dom[g * n_dom + j] + (tid >= n_dom ? P : 0);
    }
    s_ch[tid] = ch;
  }
  __syncthreads();
  for (int e = tid; e < GRP * ROW; e += 256) {
    const int hh = e / ROW, c = e % ROW;
    const int ch = s_ch[c];
    const int pair = ch % P;
    const bool dominant = (s_dmask >> pair) & 1ull;
    const float v = Elem<T>::load1(q + (static_cast<int64_t>(b) * Hq + g * GRP + hh) * d + ch);
    s_q[hh][c] = dominant ? v : 0.f;
  }
  __syncthreads();
  float qv[GRP][8];
#pragma unroll
  for (int hh = 0; hh < GRP; ++hh)
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[hh][j] = s_q[hh][sub * 8 + j];

  const T* kb = k + (static_cast<int64_t>(b) * Hkv + g) * static_cast<int64_t>(Lmax) * ROW;
  constexpr int STEPS = kTokPerWG / (WAVES * TPI);
#pragma unroll 4
  for (int it = 0; it < STEPS; ++it) {
    const int tl = (it * WAVES + wid) * TPI + tok_in_step;  // token within the work-group
    const int t = t0 + tl;
    float kv[8];
    const bool live = t < L;
    if (live) {
      Elem<T>::load8(kb + static_cast<int64_t>(t) * ROW + sub * 8, kv);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) kv[j] = 0.f;
    }
    float acc[GRP];
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) a = fmaf(qv[hh][j], kv[j], a);
      acc[hh] = a;
    }
#pragma unroll
    for (int o = LPT / 2; o >= 1; o >>= 1)
#pragma unroll
      for (int hh = 0; hh < GRP; ++hh) acc[hh] += __shfl_xor(acc[hh], o, kWave);
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh)
      if (hh % LPT == sub) s_out[hh][tl] = live ? scale * acc[hh] : -INFINITY;
  }
  __syncthreads();
  for (int e = tid; e < GRP * kTokPerWG; e += 256) {
    const int hh = e / kTokPerWG, tl = e % kTokPerWG;
    const int t = t0 + tl;
    if (t < Lmax)
      scores[(static_cast<int64_t>(b) * Hq + g * GRP + hh) * Lmax + t] = s_out[hh][tl];
  }
}

hipError_t launch_token_score(const void* q, const void* k, int dtype, int B, int Hq, int Hkv,
                              int Lmax, int d, const int32_t* cache_len, const int32_t* dom,
                              int n_dom, int slab, float scale, float* scores, hipStream_t st) {
  const int row = slab ? 2 * n_dom : d;
  const int grp = Hq / Hkv;
  const dim3 grid((Lmax + kTokPerWG - 1) / kTokPerWG, Hkv, B);
#define SA_TS(T, R, G)                                                                       \
  token_score_kernel<T, R, G><<<grid, 256, 0, st>>>(static_cast<const T*>(q),                \
                                                    static_cast<const T*>(k), Hq, Hkv, Lmax, d, \
                                                    cache_len, dom, n_dom, slab, scale, scores)
#define SA_TS_G(T, R)                      \
  switch (grp) {                           \
    case 1: SA_TS(T, R, 1); break;         \
    case 2: SA_TS(T, R, 2); break;         \
    case 4: SA_TS(T, R, 4); break;         \
    case 8: SA_TS(T, R, 8); break;         \
    default: return hipErrorInvalidValue;  \
  }
#define SA_TS_R(T)                                \
  switch (row) {                                  \
    case 8: SA_TS_G(T, 8) break;                  \
    case 16: SA_TS_G(T, 16) break;                \
    case 32: SA_TS_G(T, 32) break;                \
    case 64: SA_TS_G(T, 64) break;                \
    case 128: SA_TS_G(T, 128) break;              \
    default: return hipErrorInvalidValue;         \
  }
  if (dtype == kBF16) {
    SA_TS_R(uint16_t)
  } else {
    SA_TS_R(float)
  }
#undef SA_TS_R
#undef SA_TS_G
#undef SA_TS
  return hipGetLastError();
}

}  // namespace sa

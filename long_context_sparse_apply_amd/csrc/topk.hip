// Per-row top-k selection with forced columns and a deterministic tie-break.
//
// "Prism: Spectral-Aware Block-Sparse Attention", sec. 1: attention runs on a
// subset of relevant blocks; "FASA: Frequency-aware Sparse Attention",
// sec. 2.B: the critical token subset T_t is chosen from predicted scores.
//
// Order used everywhere: score descending, then column ascending.  A score
// maps to an order-preserving 32-bit key (NaN -> -inf, -0 -> +0 first); the
// pair (key, column) becomes the unique 64-bit composite
//     key << 32 | (0xffffffff - column)
// whose k largest values are exactly the k best columns.  Forced columns
// (sink and local window) are always kept and never compete.  Output is
// ascending by column, which falls out of emitting selection flags in column
// order.
//
// Short rows (<= 1024 columns, the prefill block rows): one wave per row, the
// row in registers (slot j of lane l = column 64 j + l), the k-th key found by
// a 32-step bitwise search with ballot counts; ties on that key go to the
// lowest columns through a running count in column order.
//
// Long rows (the decode token rows, up to 262144 columns): one 1024-thread
// work-group per row.  MSB-first radix select on the composite, 11 bits per
// level with an LDS histogram.  Columns decided at a level are set in an LDS
// bitmap; once the undecided columns fit in an LDS buffer (4096 entries) the
// remaining levels run on that buffer, so a row is usually read from memory
// twice.  The bitmap is finally compacted into ascending column indices.
#include "sa_common.hpp"

namespace sa {

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN ranks as -inf
  if ((u & 0x7fffffffu) == 0u) u = 0u;                   // -0 equals +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);     // candidates: key >= 0x007fffff
}

__device__ __forceinline__ void row_params(int64_t row, int cols, const int32_t* valid_len,
                                           const int32_t* k_per_row, int k_const, int& n, int& k) {
  n = valid_len ? valid_len[row] : cols;
  n = n < 0 ? 0 : (n > cols ? cols : n);
  k = k_per_row ? k_per_row[row] : k_const;
  k = k < 0 ? 0 : (k > k_const ? k_const : k);
}

// ------------------------------------------------------------------ short rows
template <int E>
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ scores, int64_t rows,
                                                        int cols, const int32_t* __restrict__ valid_len,
                                                        const int32_t* __restrict__ k_per_row, int k_const,
                                                        int n_sink, int n_local, int32_t* __restrict__ idx_out,
                                                        int max_out, int32_t* __restrict__ count_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (row >= rows) return;
  int n, k;
  row_params(row, cols, valid_len, k_per_row, k_const, n, k);
  const float* s = scores + row * cols;

  uint32_t key[E];
  uint32_t candm = 0, forcm = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int idx = j * kWave + lane;
    key[j] = 0;
    if (idx < n) {
      if (idx < n_sink || idx >= n - n_local) {
        forcm |= 1u << j;
      } else {
        candm |= 1u << j;
        key[j] = order_key(s[idx]);
      }
    }
  }
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) ncand += __popcll(__ballot((candm >> j) & 1u));

  uint32_t T = 0;
  int need = 0;
  if (k < ncand) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < E; ++j) cnt += __popcll(__ballot(((candm >> j) & 1u) && key[j] >= t));
      if (cnt >= k) T = t;
    }
    int gt = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) gt += __popcll(__ballot(((candm >> j) & 1u) && key[j] > T));
    need = k - gt;
  }
  // k >= ncand: T = 0 and every candidate key is > 0, so all are kept

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int32_t* dst = idx_out + row * max_out;
  int out = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (j * kWave < n) {
      const bool cand = (candm >> j) & 1u;
      const bool eq = cand && key[j] == T;
      const uint64_t eqm = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(eqm & below);
      eq_seen += __popcll(eqm);
      const bool sel = ((forcm >> j) & 1u) || (cand && (key[j] > T || (eq && eq_rank < need)));
      const uint64_t sm = __ballot(sel);
      if (sel) dst[out + __popcll(sm & below)] = j * kWave + lane;
      out += __popcll(sm);
    }
  }
  for (int p = out + lane; p < max_out; p += kWave) dst[p] = -1;
  if (lane == 0) count_out[row] = out;
}

// ------------------------------------------------------------------ long rows
constexpr int kLongThreads = 1024;
constexpr int kDigit = 11;
constexpr int kBins = 1 << kDigit;
constexpr int kCap = 4096;
constexpr int kMaxLongCols = 262144;

// exclusive prefix sum over the work-group; returns the prefix, sets total
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  constexpr int NW = kLongThreads / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) s_tmp[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int z = lane < NW ? s_tmp[lane] : 0;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const int y = __shfl_up(z, o, kWave);
      if (lane >= o) z += y;
    }
    if (lane < NW) s_tmp[lane] = z;
  }
  __syncthreads();
  const int base = wid > 0 ? s_tmp[wid - 1] : 0;
  total = s_tmp[NW - 1];
  __syncthreads();
  return base + x - v;
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int idx) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(idx));
}

__global__ __launch_bounds__(kLongThreads) void topk_block_kernel(
    const float* __restrict__ scores, int cols, const int32_t* __restrict__ valid_len,
    const int32_t* __restrict__ k_per_row, int k_const, int n_sink, int n_local,
    int32_t* __restrict__ idx_out, int max_out, int32_t* __restrict__ count_out) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t bitmap[kMaxLongCols / 32];
  __shared__ uint64_t cbuf[kCap];
  __shared__ int s_tmp[kLongThreads / kWave];
  __shared__ int s_pick[2];  // chosen digit, count above it
  __shared__ int s_nbuf;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  int n, k;
  row_params(row, cols, valid_len, k_per_row, k_const, n, k);
  const float* s = scores + row * cols;
  const int nwords = (n + 31) / 32;
  const int fa = n_sink < n ? n_sink : n;          // forced sink: [0, fa)
  const int fb = n - n_local > 0 ? n - n_local : 0;  // forced local: [fb, n)
  const int nforced = fa + (n - fb) - (fa > fb ? fa - fb : 0);
  const int ncand = n - nforced;

  for (int w = tid; w < nwords; w += kLongThreads) bitmap[w] = 0u;
  if (tid == 0) s_nbuf = 0;
  __syncthreads();
  for (int i = tid; i < fa; i += kLongThreads) atomicOr(&bitmap[i >> 5], 1u << (i & 31));
  for (int i = fb + tid; i < n; i += kLongThreads) atomicOr(&bitmap[i >> 5], 1u << (i & 31));

  auto is_cand = [&](int i) { return i >= fa && i < fb; };

  if (k >= ncand) {
    for (int i = fa + tid; i < fb; i += kLongThreads) atomicOr(&bitmap[i >> 5], 1u << (i & 31));
  } else if (k > 0) {
    uint64_t prefix = 0;
    int pbits = 0;
    int need = k;
    bool in_lds = false;
    int nbuf = 0;
    while (true) {
      for (int b = tid; b < kBins; b += kLongThreads) hist[b] = 0u;
      __syncthreads();
      const int pb = pbits;
      const uint64_t pre = prefix;
      auto matches = [&](uint64_t c) { return pb == 0 || (c >> (64 - pb)) == pre; };
      auto digit = [&](uint64_t c) { return static_cast<int>((c << pb) >> (64 - kDigit)); };
      if (!in_lds) {
        for (int i = fa + tid; i < fb; i += kLongThreads) {
          const uint64_t c = composite(order_key(s[i]), i);
          if (matches(c)) atomicAdd(&hist[digit(c)], 1u);
        }
      } else {
        for (int i = tid; i < nbuf; i += kLongThreads) {
          const uint64_t c = cbuf[i];
          if (matches(c)) atomicAdd(&hist[digit(c)], 1u);
        }
      }
      __syncthreads();
      // digit b with count(digit > b) < need <= count(digit >= b), scanning from the top
      {
        constexpr int BPT = kBins / kLongThreads;
        int local = 0;
#pragma unroll
        for (int q = 0; q < BPT; ++q) local += hist[kBins - 1 - (tid * BPT + q)];
        int total;
        int above = block_excl_scan(local, s_tmp, total);
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
          const int bin = kBins - 1 - (tid * BPT + q);
          const int h = hist[bin];
          if (above < need && need <= above + h) {
            s_pick[0] = bin;
            s_pick[1] = above;
          }
          above += h;
        }
      }
      __syncthreads();
      const int bsel = s_pick[0];
      const int gt = s_pick[1];
      const int cntb = hist[bsel];
      need -= gt;
      const bool done = (cntb == need);
      const bool collect = !in_lds && !done && cntb <= kCap;
      if (!in_lds) {
        for (int i = fa + tid; i < fb; i += kLongThreads) {
          const uint64_t c = composite(order_key(s[i]), i);
          if (!matches(c)) continue;
          const int dg = digit(c);
          if (dg > bsel || (done && dg == bsel)) {
            atomicOr(&bitmap[i >> 5], 1u << (i & 31));
          } else if (collect && dg == bsel) {
            const int slot = atomicAdd(&s_nbuf, 1);
            cbuf[slot] = c;
          }
        }
      } else {
        for (int i = tid; i < nbuf; i += kLongThreads) {
          const uint64_t c = cbuf[i];
          if (!matches(c)) continue;
          const int dg = digit(c);
          if (dg > bsel || (done && dg == bsel)) {
            const int col = static_cast<int>(0xffffffffu - static_cast<uint32_t>(c & 0xffffffffu));
            atomicOr(&bitmap[col >> 5], 1u << (col & 31));
          }
        }
      }
      __syncthreads();
      if (done) break;
      prefix = (prefix << kDigit) | static_cast<uint64_t>(bsel);
      pbits += kDigit;
      if (collect) {
        in_lds = true;
        nbuf = s_nbuf;
      }
    }
  }
  (void)is_cand;
  __syncthreads();

  // compact the bitmap into ascending column indices
  const int wpt = (nwords + kLongThreads - 1) / kLongThreads;
  const int w0 = tid * wpt;
  int mine = 0;
  for (int w = w0; w < w0 + wpt && w < nwords; ++w) {
    uint32_t bits = bitmap[w];
    if ((w + 1) * 32 > n) bits &= (n - w * 32 >= 32) ? 0xffffffffu : ((1u << (n - w * 32)) - 1u);
    mine += __popc(bits);
  }
  int total;
  int pos = block_excl_scan(mine, s_tmp, total);
  int32_t* dst = idx_out + row * max_out;
  for (int w = w0; w < w0 + wpt && w < nwords; ++w) {
    uint32_t bits = bitmap[w];
    if ((w + 1) * 32 > n) bits &= (n - w * 32 >= 32) ? 0xffffffffu : ((1u << (n - w * 32)) - 1u);
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      bits &= bits - 1;
      dst[pos++] = w * 32 + bpos;
    }
  }
  for (int p = total + tid; p < max_out; p += kLongThreads) dst[p] = -1;
  if (tid == 0) count_out[row] = total;
}

hipError_t launch_topk(const float* scores, int64_t rows, int cols, const int32_t* valid_len,
                       const int32_t* k_per_row, int k_const, int n_sink, int n_local,
                       int32_t* idx_out, int max_out, int32_t* count_out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (cols <= 1024) {
    const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
#define SA_TOPK_W(E)                                                                         \
  topk_wave_kernel<E><<<grid, 256, 0, st>>>(scores, rows, cols, valid_len, k_per_row, k_const, \
                                            n_sink, n_local, idx_out, max_out, count_out)
    if (cols <= 128) SA_TOPK_W(2);
    else if (cols <= 256) SA_TOPK_W(4);
    else if (cols <= 512) SA_TOPK_W(8);
    else SA_TOPK_W(16);
#undef SA_TOPK_W
  } else {
    topk_block_kernel<<<dim3(static_cast<unsigned>(rows)), kLongThreads, 0, st>>>(
        scores, cols, valid_len, k_per_row, k_const, n_sink, n_local, idx_out, max_out, count_out);
  }
  return hipGetLastError();
}

}  // namespace sa

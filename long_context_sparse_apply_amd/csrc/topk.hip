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
constexpr int kCap = 8192;            // LDS candidate buffer (64-bit composites)
constexpr int kMaxLongCols = 262144;  // LDS bitmap size in columns
constexpr int kSegs = 64;             // sample segments per row
constexpr int kSegLen = 128;          // samples per segment (at most)

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
__device__ __forceinline__ int comp_col(uint64_t c) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(c & 0xffffffffu));
}

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t bitmap[kMaxLongCols / 32];
  uint64_t cbuf[kCap];  // candidate composites; the sample keys live here first
  int tmp[kLongThreads / kWave];
  int pick[2];
  int nbuf;
};

// Histogram level of the MSB-first radix select on 64-bit composites: among
// the values matching the pbits-bit prefix, find the 11-bit digit b with
// count(digit > b) < need <= count(digit >= b).  `each` visits every value.
template <typename Each>
__device__ __forceinline__ void radix_level(TopkShared& sh, int pbits, uint64_t prefix, int need,
                                            Each each, int& bsel, int& above, int& cntb) {
  const int tid = threadIdx.x;
  for (int b = tid; b < kBins; b += kLongThreads) sh.hist[b] = 0u;
  __syncthreads();
  each([&](uint64_t c) {
    if (pbits == 0 || (c >> (64 - pbits)) == prefix)
      atomicAdd(&sh.hist[static_cast<int>((c << pbits) >> (64 - kDigit))], 1u);
  });
  __syncthreads();
  constexpr int BPT = kBins / kLongThreads;
  int local = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) local += sh.hist[kBins - 1 - (tid * BPT + q)];
  int total;
  int run = block_excl_scan(local, sh.tmp, total);
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int bin = kBins - 1 - (tid * BPT + q);
    const int h = sh.hist[bin];
    if (run < need && need <= run + h) {
      sh.pick[0] = bin;
      sh.pick[1] = run;
    }
    run += h;
  }
  __syncthreads();
  bsel = sh.pick[0];
  above = sh.pick[1];
  cntb = sh.hist[bsel];
  __syncthreads();
}

// Exact selection of the `need` largest composites among cbuf[0, nbuf): marks
// their columns in the bitmap.
__device__ void select_in_lds(TopkShared& sh, int nbuf, int need) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int pbits = 0;
  while (true) {
    int bsel, above, cntb;
    auto each = [&](auto f) {
      for (int i = tid; i < nbuf; i += kLongThreads) f(sh.cbuf[i]);
    };
    radix_level(sh, pbits, prefix, need, each, bsel, above, cntb);
    need -= above;
    const bool done = (cntb == need);
    for (int i = tid; i < nbuf; i += kLongThreads) {
      const uint64_t c = sh.cbuf[i];
      if (pbits != 0 && (c >> (64 - pbits)) != prefix) continue;
      const int dg = static_cast<int>((c << pbits) >> (64 - kDigit));
      if (dg > bsel || (done && dg == bsel)) {
        const int col = comp_col(c);
        atomicOr(&sh.bitmap[col >> 5], 1u << (col & 31));
      }
    }
    __syncthreads();
    if (done) break;
    prefix = (prefix << kDigit) | static_cast<uint64_t>(bsel);
    pbits += kDigit;
  }
}

// Fallback: radix select reading the row from memory at each level, moving
// to the LDS buffer once the undecided values fit (always exact).
__device__ void select_from_row(TopkShared& sh, const float* s, int fa, int fb, int need) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int pbits = 0;
  if (tid == 0) sh.nbuf = 0;
  __syncthreads();
  while (true) {
    int bsel, above, cntb;
    auto each = [&](auto f) {
      for (int i = fa + tid; i < fb; i += kLongThreads) f(composite(order_key(s[i]), i));
    };
    radix_level(sh, pbits, prefix, need, each, bsel, above, cntb);
    need -= above;
    const bool done = (cntb == need);
    const bool collect = !done && cntb <= kCap;
    for (int i = fa + tid; i < fb; i += kLongThreads) {
      const uint64_t c = composite(order_key(s[i]), i);
      if (pbits != 0 && (c >> (64 - pbits)) != prefix) continue;
      const int dg = static_cast<int>((c << pbits) >> (64 - kDigit));
      if (dg > bsel || (done && dg == bsel)) {
        atomicOr(&sh.bitmap[i >> 5], 1u << (i & 31));
      } else if (collect && dg == bsel) {
        sh.cbuf[atomicAdd(&sh.nbuf, 1)] = c;
      }
    }
    __syncthreads();
    if (done) return;
    if (collect) {
      const int nb = sh.nbuf;
      // keep only the collected values: the prefix now covers pbits + 11 bits
      select_in_lds(sh, nb, need);
      return;
    }
    prefix = (prefix << kDigit) | static_cast<uint64_t>(bsel);
    pbits += kDigit;
  }
}

// wave-aggregated append of `c` (where pred) to the candidate buffer
__device__ __forceinline__ void append(TopkShared& sh, bool pred, uint64_t c) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int leader = __ffsll(static_cast<long long>(m)) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(&sh.nbuf, __popcll(m));
  base = __shfl(base, leader, kWave);
  if (pred) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int pos = base + __popcll(m & below);
    if (pos < kCap) sh.cbuf[pos] = c;
  }
}

// One 1024-thread work-group per row.
//  1. Samples: kSegs contiguous segments spread over the candidate columns
//     (about 1/16 of them); the threshold t_low is the sample key of rank
//     k * (samples / candidates) plus four standard deviations plus 8, so that
//     with high probability at least k candidates, and not many more, have a
//     key >= t_low.
//  2. One vectorised pass appends every candidate with key >= t_low (as a
//     64-bit composite) to the LDS buffer.
//  3. If the count is in [k, kCap], an exact radix select in LDS marks the k
//     best; otherwise (an unlucky sample) the exact row-reading radix select
//     runs instead.  Either way the result is exact.
//  4. The bitmap (forced + selected columns) is compacted into ascending
//     column indices.
__global__ __launch_bounds__(kLongThreads) void topk_block_kernel(
    const float* __restrict__ scores, int cols, const int32_t* __restrict__ valid_len,
    const int32_t* __restrict__ k_per_row, int k_const, int n_sink, int n_local,
    int32_t* __restrict__ idx_out, int max_out, int32_t* __restrict__ count_out) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int64_t row = blockIdx.x;
  int n, k;
  row_params(row, cols, valid_len, k_per_row, k_const, n, k);
  const float* s = scores + row * cols;
  const int nwords = (n + 31) / 32;
  const int fa = n_sink < n ? n_sink : n;            // forced sink: [0, fa)
  const int fb = n - n_local > fa ? n - n_local : fa;  // forced local: [fb, n)
  const int ncand = fb - fa;

  for (int w = tid; w < nwords; w += kLongThreads) sh.bitmap[w] = 0u;
  if (tid == 0) sh.nbuf = 0;
  __syncthreads();
  for (int i = tid; i < fa; i += kLongThreads) atomicOr(&sh.bitmap[i >> 5], 1u << (i & 31));
  for (int i = fb + tid; i < n; i += kLongThreads) atomicOr(&sh.bitmap[i >> 5], 1u << (i & 31));

  if (k >= ncand) {
    for (int i = fa + tid; i < fb; i += kLongThreads) atomicOr(&sh.bitmap[i >> 5], 1u << (i & 31));
  } else if (k > 0) {
    bool done = false;
    const int seg_len = ncand / kSegs < kSegLen ? ncand / kSegs : kSegLen;
    const int nsamp = seg_len * kSegs;
    const double expect = static_cast<double>(k) * nsamp / ncand;
    int rank = static_cast<int>(expect + 4.0 * sqrt(expect) + 8.0);
    if (nsamp >= 1024 && rank < nsamp) {
      // 1. sample keys -> cbuf as composites (sample index as tie-break)
      uint32_t* samp = reinterpret_cast<uint32_t*>(sh.cbuf);
      const int seg_stride = ncand / kSegs;
      for (int e = tid; e < nsamp; e += kLongThreads) {
        const int seg = e / seg_len, o = e % seg_len;
        samp[e] = order_key(s[fa + seg * seg_stride + o]);
      }
      __syncthreads();
      // widen in place to composites (backwards: the u64 slots overlap the u32 ones)
      for (int base = ((nsamp - 1) / kLongThreads) * kLongThreads; base >= 0; base -= kLongThreads) {
        const int e = base + tid;
        uint32_t kv = 0;
        if (e < nsamp) kv = samp[e];
        __syncthreads();
        if (e < nsamp) sh.cbuf[e] = composite(kv, e);
        __syncthreads();
      }
      // the rank-th largest sample
      uint64_t prefix = 0;
      int pbits = 0, need = rank;
      while (true) {
        int bsel, above, cntb;
        auto each = [&](auto f) {
          for (int i = tid; i < nsamp; i += kLongThreads) f(sh.cbuf[i]);
        };
        radix_level(sh, pbits, prefix, need, each, bsel, above, cntb);
        need -= above;
        prefix = (prefix << kDigit) | static_cast<uint64_t>(bsel);
        pbits += kDigit;
        if (cntb == 1 || pbits >= 33) break;  // the key (top 32 bits) is decided by then
      }
      // top 32 bits of the prefix = the sample key at that rank (or a prefix of it)
      const uint32_t t_low = pbits >= 32 ? static_cast<uint32_t>(prefix >> (pbits - 32))
                                          : static_cast<uint32_t>(prefix << (32 - pbits));
      __syncthreads();
      if (tid == 0) sh.nbuf = 0;
      __syncthreads();
      // 2. collect every candidate with key >= t_low
      const bool aligned = ((reinterpret_cast<uintptr_t>(s) & 15) == 0);
      const int a0 = aligned ? ((fa + 3) & ~3) : fb;
      const int a1 = aligned ? (fb & ~3) : fb;
      for (int i = fa + tid; i < (a0 < fb ? a0 : fb); i += kLongThreads) {
        const uint32_t kv = order_key(s[i]);
        if (kv >= t_low) append(sh, true, composite(kv, i));
      }
      for (int base = a0; base < a1; base += 4 * kLongThreads * 4) {
        float4 v4[4];
        int i4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          i4[u] = base + (u * kLongThreads + tid) * 4;
          v4[u] = i4[u] < a1 ? *reinterpret_cast<const float4*>(s + i4[u])
                             : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float vv[4] = {v4[u].x, v4[u].y, v4[u].z, v4[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t kv = order_key(vv[e]);
            const bool ok = i4[u] < a1 && kv >= t_low;
            append(sh, ok, composite(kv, i4[u] + e));
          }
        }
      }
      for (int i = (a1 > a0 ? a1 : a0) + tid; i < fb; i += kLongThreads) {
        const uint32_t kv = order_key(s[i]);
        if (kv >= t_low) append(sh, true, composite(kv, i));
      }
      (void)lane;
      __syncthreads();
      const int got = sh.nbuf;
      __syncthreads();
      if (got >= k && got <= kCap) {
        select_in_lds(sh, got, k);
        done = true;
      }
    }
    if (!done) select_from_row(sh, s, fa, fb, k);
  }
  __syncthreads();

  // compact the bitmap into ascending column indices
  const int wpt = (nwords + kLongThreads - 1) / kLongThreads;
  const int w0 = tid * wpt;
  int mine = 0;
  for (int w = w0; w < w0 + wpt && w < nwords; ++w) mine += __popc(sh.bitmap[w]);
  int total;
  int pos = block_excl_scan(mine, sh.tmp, total);
  int32_t* dst = idx_out + row * max_out;
  for (int w = w0; w < w0 + wpt && w < nwords; ++w) {
    uint32_t bits = sh.bitmap[w];
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

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
// a bitwise search with ballot counts (at most 32 steps; it stops as soon as
// exactly k keys reach the bits fixed so far); ties on that key go to the
// lowest columns through a running count in column order.
//
// Long rows (the decode token rows, up to 262144 columns): one 512-thread
// work-group per row.  A sampled threshold (the sample keys' rank that
// matches k plus a few standard deviations) lets one vectorised pass collect
// the candidates into an LDS buffer, where an MSB-first radix select (11 bits
// a level, LDS histogram) marks the k best in an LDS bitmap; an unlucky
// sample falls back to the radix select reading the row at each level.  The
// bitmap is finally compacted into ascending column indices.  The LDS is
// sized per launch from the row length and k, so two rows of the decode
// workloads share a CU.
#include "token_dot.hpp"
#include "topk_keys.hpp"

namespace sa {

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
  // the wave's row, in a scalar register: the row's length, k and the
  // search's threshold are then scalars and the search a uniform loop
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wv;
  if (row >= rows) return;
  int n, k;
  row_params(row, cols, valid_len, k_per_row, k_const, n, k);
  const float* s = scores + row * cols;

  // all loads first (a slot past the row reads column 0, which every row
  // has, and is dropped), so they are in flight together
  float val[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int idx = j * kWave + lane;
    val[j] = s[idx < n ? idx : 0];
  }
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
        key[j] = order_key(val[j]);
      }
    }
  }
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) ncand += __popcll(__ballot((candm >> j) & 1u));

  uint32_t T = 0;
  int need = 0;
  if (k < ncand) {
    // T: the largest key with at least k candidates at or above it, bit by
    // bit from the top.  Once exactly k are at or above T the k best are
    // known (they are the keys >= T) and the lower bits cannot change the
    // selection, so the search stops there.  The tests need no candidate
    // mask: every tested t is at least 1, a candidate's key at least
    // 0x007fffff, and every other slot's key 0.
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < E; ++j) cnt += __popcll(__ballot(key[j] >= t));
      if (cnt >= k) T = t;
      if (cnt == k) break;
    }
    int gt = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) gt += __popcll(__ballot(key[j] > T));
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
// (threads a row, radix digit, candidate and row limits: sa_limits.hpp)
constexpr int kSegs = 64;             // sample segments per row
constexpr int kSegLen = 256;          // samples per segment (at most)
constexpr int kCollectVec = 4;        // float4 loads a thread per batch of the collect pass
constexpr int kSampPerThread = kSegs * kSegLen / kLongThreads;

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

// Views into the work-group's dynamic LDS: the candidate buffer (cap 64-bit
// composites), the radix histogram, the selection bitmap (one bit a column)
// and a few scalars.  Sized per launch from the row length and k.
struct TopkShared {
  uint64_t* cbuf;
  uint32_t* hist;
  uint32_t* bitmap;
  int* tmp;
  int* pick;
  int* nbuf;
  int cap;
};


__device__ __forceinline__ TopkShared topk_views(uint8_t* lds, int cols, int cap) {
  TopkShared sh;
  const int words = (cols + 31) / 32;
  sh.cbuf = reinterpret_cast<uint64_t*>(lds);
  sh.hist = reinterpret_cast<uint32_t*>(lds + static_cast<size_t>(cap) * 8);
  sh.bitmap = sh.hist + kBins;
  sh.tmp = reinterpret_cast<int*>(sh.bitmap + words);
  sh.pick = sh.tmp + kLongThreads / kWave;
  sh.nbuf = sh.pick + 2;
  sh.cap = cap;
  return sh;
}

// Histogram level of the MSB-first radix select on 64-bit composites: among
// the values matching the pbits-bit prefix, find the 11-bit digit b with
// count(digit > b) < need <= count(digit >= b).  `each` visits every value.
template <typename Each>
__device__ __forceinline__ void radix_level(const TopkShared& sh, int pbits, uint64_t prefix, int need,
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
// their columns in the bitmap.  Where every composite is known to share its
// top pbits0 bits (prefix0), the first level starts below them.
__device__ void select_in_lds(const TopkShared& sh, int nbuf, int need, uint64_t prefix0 = 0,
                              int pbits0 = 0) {
  const int tid = threadIdx.x;
  uint64_t prefix = prefix0;
  int pbits = pbits0;
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

// Fallback: radix select over the columns [fa, fb) whose scores `val(i)`
// gives (read from the row, or recomputed), taken again at each level, moving
// to the LDS buffer once the undecided values fit (always exact).
template <typename Val>
__device__ void select_from_source(const TopkShared& sh, Val val, int fa, int fb, int need) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int pbits = 0;
  if (tid == 0) *sh.nbuf = 0;
  __syncthreads();
  while (true) {
    int bsel, above, cntb;
    auto each = [&](auto f) {
      for (int i = fa + tid; i < fb; i += kLongThreads) f(composite(order_key(val(i)), i));
    };
    radix_level(sh, pbits, prefix, need, each, bsel, above, cntb);
    need -= above;
    const bool done = (cntb == need);
    const bool collect = !done && cntb <= sh.cap;
    for (int i = fa + tid; i < fb; i += kLongThreads) {
      const uint64_t c = composite(order_key(val(i)), i);
      if (pbits != 0 && (c >> (64 - pbits)) != prefix) continue;
      const int dg = static_cast<int>((c << pbits) >> (64 - kDigit));
      if (dg > bsel || (done && dg == bsel)) {
        atomicOr(&sh.bitmap[i >> 5], 1u << (i & 31));
      } else if (collect && dg == bsel) {
        sh.cbuf[atomicAdd(sh.nbuf, 1)] = c;
      }
    }
    __syncthreads();
    if (done) return;
    if (collect) {
      const int nb = *sh.nbuf;
      // keep only the collected values: the prefix now covers pbits + 11 bits
      select_in_lds(sh, nb, need);
      return;
    }
    prefix = (prefix << kDigit) | static_cast<uint64_t>(bsel);
    pbits += kDigit;
  }
}

__device__ void select_from_row(const TopkShared& sh, const float* s, int fa, int fb, int need) {
  select_from_source(sh, [s](int i) { return s[i]; }, fa, fb, need);
}

// Wave-aggregated append of up to four composites a lane (where ok[e]) to the
// candidate buffer: one LDS atomic per wave for all of them.
__device__ __forceinline__ void append4(const TopkShared& sh, const bool (&ok)[4], const uint64_t (&c)[4]) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t m[4];
  int tot = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[e] = __ballot(ok[e]);
    tot += __popcll(m[e]);
  }
  if (tot == 0) return;
  const int leader = __ffsll(static_cast<long long>(m[0] | m[1] | m[2] | m[3])) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(sh.nbuf, tot);
  base = __shfl(base, leader, kWave);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (ok[e]) {
      const int pos = base + __popcll(m[e] & below);
      if (pos < sh.cap) sh.cbuf[pos] = c[e];
    }
    base += __popcll(m[e]);
  }
}

// Sampling plan of a long row's threshold: up to kSegs segments of kSegLen
// consecutive candidates spread over the ncand candidates (nsamp samples),
// and the rank among them whose key becomes the threshold: the expected rank
// of the k-th best plus four standard deviations plus 8, so that with high
// probability at least k candidates, and not many more, have a key at or
// above it.  False when the row is too short for that.
__device__ __forceinline__ bool sample_plan(int ncand, int k, int& seg_len, int& nsamp, int& rank) {
  seg_len = ncand / kSegs < kSegLen ? ncand / kSegs : kSegLen;
  nsamp = seg_len * kSegs;
  const double expect = static_cast<double>(k) * nsamp / ncand;
  rank = static_cast<int>(expect + 4.0 * sqrt(expect) + 8.0);
  return nsamp >= 1024 && rank < nsamp;
}

// The threshold key from the samples' keys (thread tid holds samples tid +
// j kLongThreads, keys of samples past nsamp are ignored): the radix levels
// find the rank-th largest (sample index as tie-break) to 22 key bits (sign,
// exponent and 13 mantissa bits, within about 1e-4 of that sample: enough);
// the key prefix with its low bits zero is at most that sample's key.
template <int KPT>
__device__ __forceinline__ uint32_t sampled_threshold_t(const TopkShared& sh, const uint32_t (&skey)[KPT],
                                                        int nsamp, int rank) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int pbits = 0, need = rank;
  while (true) {
    int bsel, above, cntb;
    auto each = [&](auto f) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int e = tid + j * kLongThreads;
        if (e < nsamp) f(composite(skey[j], e));
      }
    };
    radix_level(sh, pbits, prefix, need, each, bsel, above, cntb);
    need -= above;
    prefix = (prefix << kDigit) | static_cast<uint64_t>(bsel);
    pbits += kDigit;
    if (cntb == 1 || pbits >= 22) break;
  }
  return pbits >= 32 ? static_cast<uint32_t>(prefix >> (pbits - 32))
                     : static_cast<uint32_t>(prefix << (32 - pbits));
}
__device__ __forceinline__ uint32_t sampled_threshold(const TopkShared& sh,
                                                      const uint32_t (&skey)[kSampPerThread],
                                                      int nsamp, int rank) {
  return sampled_threshold_t<kSampPerThread>(sh, skey, nsamp, rank);
}

// The selection bitmap of a row (nwords words) as ascending column indices
// into dst[0, max_out), padded with -1, and their number into *count.
__device__ void emit_bitmap(const TopkShared& sh, int nwords, int32_t* dst, int max_out, int32_t* count) {
  const int tid = threadIdx.x;
  const int wpt = (nwords + kLongThreads - 1) / kLongThreads;
  const int w0 = tid * wpt;
  int mine = 0;
  for (int w = w0; w < w0 + wpt && w < nwords; ++w) mine += __popc(sh.bitmap[w]);
  int total;
  int pos = block_excl_scan(mine, sh.tmp, total);
  for (int w = w0; w < w0 + wpt && w < nwords; ++w) {
    uint32_t bits = sh.bitmap[w];
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      bits &= bits - 1;
      dst[pos++] = w * 32 + bpos;
    }
  }
  for (int p = total + tid; p < max_out; p += kLongThreads) dst[p] = -1;
  if (tid == 0) *count = total;
}

// The k-th largest composite among cbuf[0, nbuf) (need = k): the MSB-first
// radix levels of select_in_lds, without marking; every composite at or above
// the returned value is selected and no other.
__device__ uint64_t select_bound_in_lds(const TopkShared& sh, int nbuf, int need, uint64_t prefix0,
                                        int pbits0) {
  const int tid = threadIdx.x;
  uint64_t prefix = prefix0;
  int pbits = pbits0;
  while (true) {
    int bsel, above, cntb;
    auto each = [&](auto f) {
      for (int i = tid; i < nbuf; i += kLongThreads) f(sh.cbuf[i]);
    };
    radix_level(sh, pbits, prefix, need, each, bsel, above, cntb);
    need -= above;
    if (cntb == need) {
      // the lowest composite with this prefix and digit (composites are
      // unique, so the levels end by the 64th bit)
      const uint64_t top = pbits == 0 ? 0ull : prefix << (64 - pbits);
      return top | ((static_cast<uint64_t>(bsel) << (64 - kDigit)) >> pbits);
    }
    prefix = (prefix << kDigit) | static_cast<uint64_t>(bsel);
    pbits += kDigit;
  }
}

// The columns of the composites at or above `bound` among cbuf[0, nbuf),
// which is in ascending column order, into dst[0, max_out) in that order,
// padded with -1, and their number into *count: a work-group compaction, each
// thread taking a contiguous run.
__device__ void emit_ordered(const TopkShared& sh, int nbuf, uint64_t bound, int32_t* dst,
                             int max_out, int32_t* count) {
  const int tid = threadIdx.x;
  const int per = (nbuf + kLongThreads - 1) / kLongThreads;
  const int i0 = tid * per < nbuf ? tid * per : nbuf;
  const int i1 = i0 + per < nbuf ? i0 + per : nbuf;
  int mine = 0;
  for (int i = i0; i < i1; ++i) mine += sh.cbuf[i] >= bound ? 1 : 0;
  int total;
  int pos = block_excl_scan(mine, sh.tmp, total);
  for (int i = i0; i < i1; ++i) {
    const uint64_t c = sh.cbuf[i];
    if (c >= bound) dst[pos++] = comp_col(c);
  }
  for (int p = total + tid; p < max_out; p += kLongThreads) dst[p] = -1;
  if (tid == 0) *count = total;
}

// One 512-thread work-group per row.
//  1. Samples: kSegs contiguous segments spread over the candidate columns
//     (up to 16384 values, read once and kept in registers); the
//     threshold t_low is the sample key of rank k * (samples / candidates)
//     plus four standard deviations plus 8, so that with high probability at
//     least k candidates, and not many more, have a key >= t_low.
//  2. One vectorised, software-pipelined pass (two batches of 8 float4 loads
//     a thread) appends every candidate with key >= t_low (as a 64-bit
//     composite) to the LDS buffer.
//  3. If the count is in [k, cap], an exact radix select in LDS marks the k
//     best; otherwise (an unlucky sample) the exact row-reading radix select
//     runs instead.  Either way the result is exact.
//  4. The bitmap (forced + selected columns) is compacted into ascending
//     column indices.
__global__ __launch_bounds__(kLongThreads) void topk_block_kernel(
    const float* __restrict__ scores, int cols, const int32_t* __restrict__ valid_len,
    const int32_t* __restrict__ k_per_row, int k_const, int n_sink, int n_local,
    int32_t* __restrict__ idx_out, int max_out, int32_t* __restrict__ count_out, int cap) {
  extern __shared__ __attribute__((aligned(16))) uint8_t topk_lds[];
  const TopkShared sh = topk_views(topk_lds, cols, cap);
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  int n, k;
  row_params(row, cols, valid_len, k_per_row, k_const, n, k);
  const float* s = scores + row * cols;
  const int nwords = (n + 31) / 32;
  const int fa = n_sink < n ? n_sink : n;            // forced sink: [0, fa)
  const int fb = n - n_local > fa ? n - n_local : fa;  // forced local: [fb, n)
  const int ncand = fb - fa;

  for (int w = tid; w < nwords; w += kLongThreads) sh.bitmap[w] = 0u;
  if (tid == 0) *sh.nbuf = 0;
  __syncthreads();
  for (int i = tid; i < fa; i += kLongThreads) atomicOr(&sh.bitmap[i >> 5], 1u << (i & 31));
  for (int i = fb + tid; i < n; i += kLongThreads) atomicOr(&sh.bitmap[i >> 5], 1u << (i & 31));

  if (k >= ncand) {
    for (int i = fa + tid; i < fb; i += kLongThreads) atomicOr(&sh.bitmap[i >> 5], 1u << (i & 31));
  } else if (k > 0) {
    bool done = false;
    int seg_len, nsamp, rank;
    if (sample_plan(ncand, k, seg_len, nsamp, rank)) {
      // 1. the rank-th largest sample; each thread keeps its samples' keys in
      //    registers for the radix levels
      const int seg_stride = ncand / kSegs;
      // Sample e sits at fa + (e / seg_len) seg_stride + e % seg_len.  The
      // thread's samples are e = tid + j kLongThreads: segment and offset
      // advance by kLongThreads / seg_len and kLongThreads % seg_len a step
      // (one carry at most, the offset staying below seg_len), so no step
      // divides.  Every load is issued before any key is formed, and a
      // sample past nsamp reads column fa instead (its key is dropped), so
      // the loads need no branch and are all in flight together.
      const int seg_step = kLongThreads / seg_len, off_step = kLongThreads % seg_len;
      int seg = tid / seg_len, off = tid % seg_len;
      float sval[kSampPerThread];
#pragma unroll
      for (int j = 0; j < kSampPerThread; ++j) {
        const bool in = tid + j * kLongThreads < nsamp;
        sval[j] = s[in ? fa + seg * seg_stride + off : fa];
        seg += seg_step;
        off += off_step;
        if (off >= seg_len) { off -= seg_len; ++seg; }
      }
      uint32_t skey[kSampPerThread];
#pragma unroll
      for (int j = 0; j < kSampPerThread; ++j)
        skey[j] = tid + j * kLongThreads < nsamp ? order_key(sval[j]) : 0u;
      const uint32_t t_low = sampled_threshold(sh, skey, nsamp, rank);
      __syncthreads();
      if (tid == 0) *sh.nbuf = 0;
      __syncthreads();
      // 2. collect every candidate with key >= t_low (as a float test)
      const KeyThreshold thr(t_low);
      auto qualifies = [&](float v) { return thr.qualifies(v); };
      const bool aligned = ((reinterpret_cast<uintptr_t>(s) & 15) == 0);
      const int a0 = aligned ? ((fa + 3) & ~3) : fb;
      const int a1 = aligned ? (fb & ~3) : fb;
      for (int i = fa + tid; i < (a0 < fb ? a0 : fb); i += kLongThreads) {
        const float v = s[i];
        const bool ok[4] = {qualifies(v), false, false, false};
        const uint64_t c[4] = {composite(order_key(v), i), 0, 0, 0};
        append4(sh, ok, c);
      }
      // Vectorised body, software-pipelined over four named batches of
      // kCollectVec float4 a thread: a batch's loads are issued three batches
      // before it is tested, and no register is copied between batches (a
      // copy would wait for the loads just issued).  The loads take no branch:
      // an index at or past a1 reads column a0 instead (a valid aligned
      // address; a1 > a0 inside the loop) and the value is dropped by the
      // i < a1 test, so the counter waits stay exact.
      constexpr int kStep = 4 * kLongThreads * kCollectVec;
      auto load_batch = [&](float4 (&dst)[kCollectVec], int bbase) {
#pragma unroll
        for (int u = 0; u < kCollectVec; ++u) {
          const int i = bbase + (u * kLongThreads + tid) * 4;
          // (nontemporal: the row is streamed once)
          typedef float v4f __attribute__((ext_vector_type(4)));
          const v4f t4 = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(s + (i < a1 ? i : a0)));
          dst[u] = make_float4(t4.x, t4.y, t4.z, t4.w);
        }
      };
      // the wave's qualifying values of a batch take one LDS atomic for their
      // slots (lane 0's, broadcast by readfirstlane: every lane is active
      // here); a value's slot is the running total plus its rank among the
      // lanes below in its ballot.  Each lane keeps its own qualifying bits
      // and the ballots are taken again when writing, so only one is live at
      // a time.
      auto test_batch = [&](const float4 (&src)[kCollectVec], int bbase) {
        static_assert(4 * kCollectVec <= 32, "one bit a value of the batch");
        uint32_t qbits = 0;
        int tot = 0;
#pragma unroll
        for (int u = 0; u < kCollectVec; ++u) {
          const int i = bbase + (u * kLongThreads + tid) * 4;  // i < a1 covers i + 3 (a1 % 4 == 0)
          const float vv[4] = {src[u].x, src[u].y, src[u].z, src[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = i < a1 && qualifies(vv[e]);
            qbits |= static_cast<uint32_t>(ok) << (4 * u + e);
            tot += __popcll(__ballot(ok));
          }
        }
        if (tot == 0) return;
        const int lane = tid & (kWave - 1);
        int slot = 0;
        if (lane == 0) slot = atomicAdd(sh.nbuf, tot);
        slot = __builtin_amdgcn_readfirstlane(slot);
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
        for (int u = 0; u < kCollectVec; ++u) {
          const int i = bbase + (u * kLongThreads + tid) * 4;
          const float vv[4] = {src[u].x, src[u].y, src[u].z, src[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = (qbits >> (4 * u + e)) & 1u;
            const uint64_t m = __ballot(ok);
            if (ok) {
              const int pos = slot + __popcll(m & below);
              if (pos < sh.cap) sh.cbuf[pos] = composite(order_key(vv[e]), i + e);
            }
            slot += __popcll(m);
          }
        }
      };
      if (a0 < a1) {
        float4 b0[kCollectVec], b1[kCollectVec], b2[kCollectVec], b3[kCollectVec];
        load_batch(b0, a0);
        load_batch(b1, a0 + kStep);
        load_batch(b2, a0 + 2 * kStep);
        for (int base = a0; base < a1; base += 4 * kStep) {
          load_batch(b3, base + 3 * kStep);
          test_batch(b0, base);
          load_batch(b0, base + 4 * kStep);
          test_batch(b1, base + kStep);
          load_batch(b1, base + 5 * kStep);
          test_batch(b2, base + 2 * kStep);
          load_batch(b2, base + 6 * kStep);
          test_batch(b3, base + 3 * kStep);
        }
      }
      for (int i = (a1 > a0 ? a1 : a0) + tid; i < fb; i += kLongThreads) {
        const float v = s[i];
        const bool ok[4] = {qualifies(v), false, false, false};
        const uint64_t c[4] = {composite(order_key(v), i), 0, 0, 0};
        append4(sh, ok, c);
      }
      __syncthreads();
      const int got = *sh.nbuf;
      __syncthreads();
      if (got >= k && got <= cap) {
        select_in_lds(sh, got, k);
        done = true;
      }
    }
    if (!done) select_from_row(sh, s, fa, fb, k);
  }
  __syncthreads();

  emit_bitmap(sh, nwords, idx_out + row * max_out, max_out, count_out + row);
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
    const int cap = topk_cap(k_const);
    const size_t lds = topk_lds_bytes(cols, cap);
    // allow the largest size this kernel ever asks for (above the 64 KB default)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_block_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(topk_lds_bytes(kMaxLongCols, kMaxCap)));
    if (e != hipSuccess) return e;
    topk_block_kernel<<<dim3(static_cast<unsigned>(rows)), kLongThreads, lds, st>>>(
        scores, cols, valid_len, k_per_row, k_const, n_sink, n_local, idx_out, max_out, count_out, cap);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ fused token top-k
// The decode step's token selection without a score array ("FASA:
// Frequency-aware Sparse Attention", sec. 2.B items 1 and 2: token importance
// from the dominant chunks, then the critical subset T_t).  Three kernels:
//  1. token_thr_kernel, one work-group per (batch, KV head): a sampled
//     threshold for each of the group's query heads, from the scores of
//     kSegs x kSegLenF sampled tokens (each sample's row read once for all
//     heads).  Rows with k = 0 or k >= their length get a threshold
//     nothing passes, rows too short to sample one that takes every token.
//     With few groups, four work-groups share a group's samples and
//     token_thr_pick_kernel finishes each row's threshold from their keys.
//  2. the token scoring kernel in collect mode (token_score.hip): the same
//     scores as the scoring entry point; tokens at or above the threshold go
//     to per-wave candidate lists (no atomics).
//  3. token_select_kernel, one work-group per row: the exact top-k of the
//     candidates gathered into LDS; when a list overflowed or their number is
//     not in [k, cap] (an unlucky sample), the exact radix select over all
//     tokens with their scores recomputed by the same arithmetic.  The
//     threshold only steers how many candidates come back, so the result is
//     the top-k of the scores whatever it is.
// The slab row of a token is the 2 n_dom dominant channels (NDC), read as
// 16-byte words; a standard row holds all d channels, of which the scored
// ones are read through the scoring kernel's channel table.

constexpr int kSegLenF = 64;                                  // samples a segment (at most)
constexpr int kSampPerThreadF = kSegs * kSegLenF / kLongThreads;  // 8
constexpr int kSampCap = kTokenSampleKeys;  // sample keys a row
static_assert(kSegs * kSegLenF == kSampCap, "a row's samples fill its key slots");
// With fewer (batch, KV head) groups than this, four work-groups share a
// group's samples and a pick kernel searches each row's keys
constexpr int kThrSplitBelow = 256;


// The scaled dominant query slice of row `row` in slab channel order, as the
// scoring kernel stages it: thread t < NDC writes channel t.
template <typename T, int NDC>
__device__ __forceinline__ void stage_query_slice(float* s_q, const T* __restrict__ q, int64_t row,
                                                  int g, int d, const int32_t* __restrict__ dom,
                                                  int n_dom, float scale) {
  const int tid = threadIdx.x;
  if (tid < NDC) {
    float v = 0.f;
    if (tid < 2 * n_dom) {
      const int qc = (dom[g * n_dom + (tid % n_dom)] + (tid >= n_dom ? d / 2 : 0)) & (d - 1);
      v = Elem<T>::load1(q + row * d + qc) * scale;
    }
    s_q[tid] = v;
  }
}

__device__ __forceinline__ int clamp_len(int L, int Lmax) { return L < 0 ? 0 : (L > Lmax ? Lmax : L); }

// Standard layout: the row channel of scored slot j, as the scoring kernel
// reads it (slots past 2 n_dom read channel 0; their query value is 0).
// Thread t < NDC writes slot t.
template <int NDC>
__device__ __forceinline__ void stage_channels(int* s_ch, int g, int d, const int32_t* __restrict__ dom,
                                               int n_dom) {
  const int tid = threadIdx.x;
  if (tid < NDC)
    s_ch[tid] = tid < 2 * n_dom ? (dom[g * n_dom + (tid % n_dom)] + (tid >= n_dom ? d / 2 : 0)) & (d - 1) : 0;
}

// One token's NDC scored channels from a standard row (all loads issued
// before any use).
template <typename T, int NDC>
__device__ __forceinline__ void load_std_row(const T* __restrict__ row, const int* s_ch, float (&kv)[NDC]) {
#pragma unroll
  for (int j = 0; j < NDC; ++j) kv[j] = Elem<T>::load1(row + s_ch[j]);
}

// The sampling plan of a row with n cached tokens and budget k: the sample
// count and the rank whose key becomes the threshold.  Returns false when the
// row needs no sample (k <= 0 or k >= n: nothing passes; too few samples or a
// rank past them: every token passes), with the threshold in *fixed.
__device__ __forceinline__ bool thr_plan(int n, int k, int& seg_len, int& nsamp, int& rank,
                                         uint32_t& fixed) {
  if (k <= 0 || k >= n) {
    fixed = kNoCandidates;
    return false;
  }
  seg_len = n / kSegs < kSegLenF ? n / kSegs : kSegLenF;
  nsamp = seg_len * kSegs;
  const double expect = static_cast<double>(k) * nsamp / n;
  rank = static_cast<int>(expect + 4.0 * sqrt(expect) + 8.0);
  if (nsamp < 1024 || rank >= nsamp) {
    fixed = 0u;  // take every token
    return false;
  }
  return true;
}

// Sampled thresholds of one (batch, KV head) group's query heads.  PARTS ==
// 1: grid B * Hkv, a work-group scores all the group's samples for every
// query head and runs each head's radix search itself (thr[row]).  PARTS > 1
// (few groups: more work-groups to share the sample loads): grid (B * Hkv,
// PARTS), part p scores rounds [p, p + 1) * KPT / PARTS and stores the keys
// at keys[row][e] (e = sample index) for token_thr_pick_kernel, which runs
// the same search over the same keys.  Rows that need no sample get their
// fixed threshold from the work-group (PARTS == 1) or the pick kernel.
template <typename T, int NDC, int GRP, bool SLAB, int PARTS>
__global__ __launch_bounds__(kLongThreads) void token_thr_kernel(
    const T* __restrict__ q, const T* __restrict__ kdom, int Hq, int Hkv, int Lmax, int d,
    const int32_t* __restrict__ cache_len, const int32_t* __restrict__ dom, int n_dom, float scale,
    int k_top, uint32_t* __restrict__ thr, uint32_t* __restrict__ keys) {
  constexpr int R16 = NDC * static_cast<int>(sizeof(T)) / 16;  // 16-byte words a slab row
  static_assert(!SLAB || (R16 >= 1 && R16 <= 8), "slab rows of 16 to 128 bytes");
  static_assert(kSampPerThreadF % PARTS == 0, "rounds split evenly over the parts");
  constexpr int RPP = kSampPerThreadF / PARTS;  // rounds of this work-group
  __shared__ int s_ch[NDC];
  __shared__ __attribute__((aligned(16))) float s_q[GRP][NDC];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / Hkv;
  const int g = blockIdx.x % Hkv;
  const int j0 = PARTS > 1 ? static_cast<int>(blockIdx.y) * RPP : 0;  // first round
  const int64_t row0 = static_cast<int64_t>(b) * Hq + g * GRP;  // the group's first row
  const int n = clamp_len(cache_len[b], Lmax);
  int seg_len = 0, nsamp = 0, rank = 0;
  uint32_t fixed = 0;
  // uniform over the work-group: all threads return here or none
  if (!thr_plan(n, k_top, seg_len, nsamp, rank, fixed)) {
    if (PARTS == 1 && tid < GRP) thr[row0 + tid] = fixed;
    return;
  }
#pragma unroll
  for (int hh = 0; hh < GRP; ++hh)
    stage_query_slice<T, NDC>(&s_q[hh][0], q, row0 + hh, g, d, dom, n_dom, scale);
  if (!SLAB) stage_channels<NDC>(s_ch, g, d, dom, n_dom);
  __syncthreads();
  const int rowlen = SLAB ? NDC : d;
  const T* kb = kdom + (static_cast<int64_t>(b) * Hkv + g) * Lmax * rowlen;
  // sample e = tid + j kLongThreads sits at (e / seg_len) seg_stride + e % seg_len.
  // The per-load split of e divides by the uniform seg_len (<= kSegLenF) with
  // a multiply-high by m = floor((2^32 - 1) / seg_len) + 1: for e < 2^32 /
  // seg_len its error stays below 1 / seg_len, so the quotient is exact.
  const uint32_t seg_m = 0xFFFFFFFFu / static_cast<uint32_t>(seg_len) + 1u;
  auto seg_of = [&](int e) { return static_cast<int>(__umulhi(static_cast<uint32_t>(e), seg_m)); };
  const int seg_stride = n / kSegs;
  // the token of sample e (a sample past nsamp reads token 0; its key is 0)
  auto sample_tok = [&](int e) {
    const int se = seg_of(e);
    return e < nsamp ? se * seg_stride + (e - se * seg_len) : 0;
  };
  uint32_t skey[GRP][RPP];
  if constexpr (SLAB && R16 <= 4) {
    // slab rows of at most 64 bytes: in round j a wave loads its 64 samples'
    // rows with R16 lanes a row (64 / R16 rows an instruction, so each load
    // touches a few lines, not 64), parks them in its LDS slice, and each
    // lane unpacks and scores its own sample from there
    constexpr int RPI = kWave / R16;           // rows an instruction
    __shared__ uint4 s_rows[kLongThreads / kWave][kWave][R16];
    const int wv = tid / kWave, ln = tid & (kWave - 1);
    const int rsub = ln / R16, part = ln % R16;
#pragma unroll
    for (int jj = 0; jj < RPP; ++jj) {
      const int j = j0 + jj;
      uint4 raw[R16];
#pragma unroll
      for (int i = 0; i < R16; ++i) {
        const int e = j * kLongThreads + wv * kWave + i * RPI + rsub;  // the sample loaded
        raw[i] = reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(sample_tok(e)) * NDC)[part];
      }
#pragma unroll
      for (int i = 0; i < R16; ++i) s_rows[wv][i * RPI + rsub][part] = raw[i];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes landed
      __builtin_amdgcn_wave_barrier();
      float kv[NDC];
      load_slab_row<T, NDC>(reinterpret_cast<const T*>(&s_rows[wv][ln][0]), kv);
      const bool in = tid + j * kLongThreads < nsamp;
#pragma unroll
      for (int hh = 0; hh < GRP; ++hh) skey[hh][jj] = in ? order_key(token_dot<NDC>(&s_q[hh][0], kv)) : 0u;
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the slice's reads done before it is rewritten
      __builtin_amdgcn_wave_barrier();
    }
  } else if constexpr (SLAB) {
    uint4 w[RPP][R16];
#pragma unroll
    for (int jj = 0; jj < RPP; ++jj) {
      const uint4* src = reinterpret_cast<const uint4*>(
          kb + static_cast<int64_t>(sample_tok(tid + (j0 + jj) * kLongThreads)) * NDC);
#pragma unroll
      for (int c = 0; c < R16; ++c) w[jj][c] = src[c];
    }
#pragma unroll
    for (int jj = 0; jj < RPP; ++jj) {
      float kv[NDC];
      load_slab_row<T, NDC>(reinterpret_cast<const T*>(&w[jj][0]), kv);
      const bool in = tid + (j0 + jj) * kLongThreads < nsamp;
#pragma unroll
      for (int hh = 0; hh < GRP; ++hh) skey[hh][jj] = in ? order_key(token_dot<NDC>(&s_q[hh][0], kv)) : 0u;
    }
  } else if constexpr (sizeof(T) == 2 && NDC <= 32) {
    // standard rows, bf16, up to 32 scored channels: in round j a wave loads
    // the scored channels of its 64 samples with NDC lanes a row (64 / NDC
    // rows an instruction, so each load touches a few lines, not 64), parks
    // the raw values in its LDS slice, and each lane then scores its own
    // sample from there with the same sequential arithmetic
    constexpr int RPI = kWave / NDC;           // rows an instruction
    __shared__ uint16_t s_raw[kLongThreads / kWave][kWave][NDC];
    const int wv = tid / kWave, ln = tid & (kWave - 1);
    const int rsub = ln / NDC, slot = ln % NDC;
    const int ch = s_ch[slot];
#pragma unroll
    for (int jj = 0; jj < RPP; ++jj) {
      const int j = j0 + jj;
      uint16_t raw[kWave / RPI];
#pragma unroll
      for (int i = 0; i < kWave / RPI; ++i) {
        const int e = j * kLongThreads + wv * kWave + i * RPI + rsub;  // the sample loaded
        raw[i] = reinterpret_cast<const uint16_t*>(kb)[static_cast<int64_t>(sample_tok(e)) * d + ch];
      }
#pragma unroll
      for (int i = 0; i < kWave / RPI; ++i) s_raw[wv][i * RPI + rsub][slot] = raw[i];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes landed
      __builtin_amdgcn_wave_barrier();
      float kv[NDC];
#pragma unroll
      for (int c = 0; c < NDC; ++c) kv[c] = __uint_as_float(static_cast<uint32_t>(s_raw[wv][ln][c]) << 16);
      const bool in = tid + j * kLongThreads < nsamp;
#pragma unroll
      for (int hh = 0; hh < GRP; ++hh) skey[hh][jj] = in ? order_key(token_dot<NDC>(&s_q[hh][0], kv)) : 0u;
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the slice's reads done before it is rewritten
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    // standard rows: the scored channels of RND samples at a time
    int tok[RPP];
#pragma unroll
    for (int jj = 0; jj < RPP; ++jj) tok[jj] = sample_tok(tid + (j0 + jj) * kLongThreads);
    constexpr int RND = NDC >= 64 ? 1 : (64 / NDC < RPP ? 64 / NDC : RPP);
#pragma unroll
    for (int r0 = 0; r0 < RPP; r0 += RND) {
      float kv[RND][NDC];
#pragma unroll
      for (int jj = 0; jj < RND; ++jj)
        load_std_row<T, NDC>(kb + static_cast<int64_t>(tok[r0 + jj]) * d, s_ch, kv[jj]);
#pragma unroll
      for (int jj = 0; jj < RND; ++jj) {
        const bool in = tid + (j0 + r0 + jj) * kLongThreads < nsamp;
#pragma unroll
        for (int hh = 0; hh < GRP; ++hh)
          skey[hh][r0 + jj] = in ? order_key(token_dot<NDC>(&s_q[hh][0], kv[jj])) : 0u;
      }
    }
  }
  if constexpr (PARTS == 1) {
    __shared__ uint32_t s_hist[kBins];
    __shared__ int s_tmp[kLongThreads / kWave + 4];
    TopkShared sh{};
    sh.hist = s_hist;
    sh.tmp = s_tmp;
    sh.pick = s_tmp + kLongThreads / kWave;
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh) {
      const uint32_t t_low = sampled_threshold_t<RPP>(sh, skey[hh], nsamp, rank);
      if (tid == 0) thr[row0 + hh] = t_low;
    }
  } else {
    // sample e = tid + j kLongThreads of row row0 + hh at keys[(row0 + hh) kSampCap + e]
#pragma unroll
    for (int hh = 0; hh < GRP; ++hh)
#pragma unroll
      for (int jj = 0; jj < RPP; ++jj)
        keys[(row0 + hh) * kSampCap + tid + (j0 + jj) * kLongThreads] = skey[hh][jj];
  }
}

// The sampled threshold of each (batch, query head) row from its sample keys
// (one work-group a row): the same radix search over the same keys, in the
// same per-thread layout, as when one work-group scored and selected a
// group's samples itself.
__global__ __launch_bounds__(kLongThreads) void token_thr_pick_kernel(
    int Hq, int Lmax, const int32_t* __restrict__ cache_len, int k_top,
    const uint32_t* __restrict__ keys, uint32_t* __restrict__ thr) {
  constexpr int KPT = kSampPerThreadF;
  __shared__ uint32_t s_hist[kBins];
  __shared__ int s_tmp[kLongThreads / kWave + 4];
  TopkShared sh{};
  sh.hist = s_hist;
  sh.tmp = s_tmp;
  sh.pick = s_tmp + kLongThreads / kWave;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / Hq);
  const int n = clamp_len(cache_len[b], Lmax);
  int seg_len = 0, nsamp = 0, rank = 0;
  uint32_t fixed = 0;
  if (!thr_plan(n, k_top, seg_len, nsamp, rank, fixed)) {
    if (tid == 0) thr[row] = fixed;
    return;
  }
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = keys[row * kSampCap + tid + j * kLongThreads];
  const uint32_t t_low = sampled_threshold_t<KPT>(sh, key, nsamp, rank);
  if (tid == 0) thr[row] = t_low;
}

template <typename T, int NDC, bool SLAB>
__global__ __launch_bounds__(kLongThreads) void token_select_kernel(
    const T* __restrict__ q, const T* __restrict__ kdom, int Hq, int Hkv, int Lmax, int d,
    const int32_t* __restrict__ cache_len, const int32_t* __restrict__ dom, int n_dom, float scale,
    int k_top, TokenCollect col, int cap, int32_t* __restrict__ idx_out, int max_out,
    int32_t* __restrict__ count_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t topk_lds[];
  __shared__ __attribute__((aligned(16))) float s_q[NDC];
  __shared__ int s_ch[NDC];
  constexpr int kMaxLists = kMaxLongCols / kCollectTile * kCollectWaves;
  static_assert(kMaxLists <= kLongThreads, "a thread a list in the count scan");
  __shared__ int s_at[kMaxLists], s_cn[kMaxLists];  // each list's place and length
  __shared__ uint64_t s_lo[kLongThreads / kWave], s_hi[kLongThreads / kWave];
  // LDS: the region (candidates, or bitmap + buffer on the fallback), the
  // radix histogram, the scan scalars
  const int region = static_cast<int>(token_select_region(Lmax, cap));
  TopkShared sh;
  sh.cbuf = reinterpret_cast<uint64_t*>(topk_lds);
  sh.hist = reinterpret_cast<uint32_t*>(topk_lds + region);
  sh.bitmap = nullptr;
  sh.tmp = reinterpret_cast<int*>(sh.hist + kBins);
  sh.pick = sh.tmp + kLongThreads / kWave;
  sh.nbuf = sh.pick + 2;
  sh.cap = cap;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>(row / Hq);
  const int g = static_cast<int>(row % Hq) / (Hq / Hkv);
  const int n = clamp_len(cache_len[b], Lmax);
  const int k = k_top;
  int32_t* dst = idx_out + row * max_out;
  // (n <= k <= max_out here)
  if (k >= n) {
    for (int p = tid; p < max_out; p += kLongThreads) dst[p] = p < n ? p : -1;
    if (tid == 0) count_out[row] = n;
    return;
  }
  if (k <= 0) {
    for (int p = tid; p < max_out; p += kLongThreads) dst[p] = -1;
    if (tid == 0) count_out[row] = 0;
    return;
  }
  // gather the (tile, wave) lists: thread j < nsub owns list j
  const int nsub = col.tiles * kCollectWaves;  // <= kLongThreads (Lmax <= 262144)
  const int cj = tid < nsub ? col.cnt[row * nsub + tid] : 0;
  const bool over = __syncthreads_or(cj > kCollectSlots);
  int total;
  const int at = block_excl_scan(cj, sh.tmp, total);
  if (!over && total >= k && total <= cap) {
    // Four threads a list, each taking every fourth entry; a round issues
    // all its loads before any store (a list past 64 entries takes more
    // rounds; a round's reads stay in the list's kCollectSlots slots).  The
    // lists, taken in order, are in ascending token order, and so is the
    // buffer.  The smallest and largest composite come along for the select.
    if (tid < nsub) {
      s_at[tid] = at;
      s_cn[tid] = cj;
    }
    __syncthreads();
    uint64_t lo = ~0ull, hi = 0ull;
    for (int j = tid >> 2; j < nsub; j += kLongThreads / 4) {
      const int nj = s_cn[j], aj = s_at[j];
      const uint64_t* src = col.cand + (row * nsub + j) * kCollectSlots + (tid & 3);
      for (int base = 0; base < nj; base += 64) {
        uint64_t v[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) v[m] = src[base + 4 * m];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          const int i = base + (tid & 3) + 4 * m;
          if (i < nj) {
            // (score bits, token) -> the composite the selection compares
            const uint64_t c = composite(order_key(__uint_as_float(static_cast<uint32_t>(v[m] >> 32))),
                                         static_cast<int>(static_cast<uint32_t>(v[m])));
            sh.cbuf[aj + i] = c;
            lo = c < lo ? c : lo;
            hi = c > hi ? c : hi;
          }
        }
      }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const uint64_t a = __shfl_xor(lo, o, kWave), c = __shfl_xor(hi, o, kWave);
      lo = a < lo ? a : lo;
      hi = c > hi ? c : hi;
    }
    if ((tid & (kWave - 1)) == 0) {
      s_lo[tid / kWave] = lo;
      s_hi[tid / kWave] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kLongThreads / kWave; ++w) {
      lo = s_lo[w] < lo ? s_lo[w] : lo;
      hi = s_hi[w] > hi ? s_hi[w] : hi;
    }
    // every candidate lies in [lo, hi], so all share the bits above the
    // highest bit where lo and hi differ (composites are unique: lo < hi
    // unless there is one candidate)
    int pb = __clzll(static_cast<long long>(lo ^ hi));
    pb = pb > 63 ? 63 : pb;
    const uint64_t bound = select_bound_in_lds(sh, total, k, pb > 0 ? hi >> (64 - pb) : 0ull, pb);
    emit_ordered(sh, total, bound, dst, max_out, count_out + row);
    return;
  }
  // Fallback (a list overflowed, or the candidates are not in [k, cap]: an
  // unlucky sample): every token, its score recomputed exactly as the scoring
  // kernel has it.  The row's bitmap sits at the end of the region, the
  // buffer before it.
  const int nwords = (n + 31) / 32;
  const int bm_bytes = ((Lmax + 31) / 32 * 4 + 15) / 16 * 16;
  sh.bitmap = reinterpret_cast<uint32_t*>(topk_lds + region - bm_bytes);
  sh.cap = (region - bm_bytes) / 8;
  for (int w = tid; w < nwords; w += kLongThreads) sh.bitmap[w] = 0u;
  stage_query_slice<T, NDC>(s_q, q, row, g, d, dom, n_dom, scale);
  if (!SLAB) stage_channels<NDC>(s_ch, g, d, dom, n_dom);
  __syncthreads();
  const int rowlen = SLAB ? NDC : d;
  const T* kb = kdom + (static_cast<int64_t>(b) * Hkv + g) * Lmax * rowlen;
  auto val = [&](int i) {
    if constexpr (SLAB) {
      float kv[NDC];
      load_slab_row<T, NDC>(kb + static_cast<int64_t>(i) * NDC, kv);
      return token_dot<NDC>(s_q, kv);
    } else {
      // token_dot's chain (one fused multiply-add a channel, in slot order,
      // from zero) four channels at a time: the same score bit for bit, with
      // four scattered loads live instead of NDC, so this rare path does not
      // set the register count of the whole kernel
      const T* rowp = kb + static_cast<int64_t>(i) * d;
      float acc = 0.f;
#pragma unroll 1
      for (int j = 0; j < NDC; j += 4) {
        const float4 qv = *reinterpret_cast<const float4*>(s_q + j);
        const float k0 = Elem<T>::load1(rowp + s_ch[j]);
        const float k1 = Elem<T>::load1(rowp + s_ch[j + 1]);
        const float k2 = Elem<T>::load1(rowp + s_ch[j + 2]);
        const float k3 = Elem<T>::load1(rowp + s_ch[j + 3]);
        acc = fmaf(qv.x, k0, acc);
        acc = fmaf(qv.y, k1, acc);
        acc = fmaf(qv.z, k2, acc);
        acc = fmaf(qv.w, k3, acc);
      }
      return acc;
    }
  };
  select_from_source(sh, val, 0, n, k);
  __syncthreads();
  emit_bitmap(sh, nwords, dst, max_out, count_out + row);
}

// Workspace (sized by token_topk_ws_bytes): thresholds [rows], list counts
// [rows, tiles, waves], lists [rows, tiles, waves, kCollectSlots] and sample
// keys [rows, kSampCap], each part 256-byte aligned.
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

hipError_t launch_token_topk(const void* q, const void* k, int dtype, int B, int Hq, int Hkv,
                             int Lmax, int d, const int32_t* cache_len, const int32_t* dom,
                             int n_dom, int slab, float scale, int k_top, int32_t* idx_out,
                             int max_out, int32_t* count_out, void* ws, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(B) * Hq;
  if (rows == 0) return hipSuccess;
  const int cap = token_topk_cap(k_top);
  const int tiles = (Lmax + kCollectTile - 1) / kCollectTile;
  const size_t lists = static_cast<size_t>(rows) * tiles * kCollectWaves;
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint32_t* thr = reinterpret_cast<uint32_t*>(w);
  int* cnt = reinterpret_cast<int*>(w + align256(static_cast<size_t>(rows) * 4));
  uint64_t* cand = reinterpret_cast<uint64_t*>(w + align256(static_cast<size_t>(rows) * 4) + align256(lists * 4));
  uint32_t* skeys = reinterpret_cast<uint32_t*>(w + align256(static_cast<size_t>(rows) * 4) + align256(lists * 4) +
                                                align256(lists * kCollectSlots * 8));
  const TokenCollect col{thr, cnt, cand, tiles};
  const bool split = static_cast<int64_t>(B) * Hkv < kThrSplitBelow;
  const size_t lds = token_select_lds_bytes(Lmax, cap);
  // scored slots: exactly 2 n_dom in the slab, a power of two of at least 8
  // covering them in the standard layout (as the scoring kernel has it)
  const int need = 2 * n_dom;
  const int ndc = slab ? need : (need <= 8 ? 8 : need <= 16 ? 16 : need <= 32 ? 32 : need <= 64 ? 64 : 128);
  const int grp = Hq / Hkv;
#define SA_TT_G(T, C, SL, G)                                                                        \
  if (split)                                                                                        \
    token_thr_kernel<T, C, G, SL, 4><<<dim3(static_cast<unsigned>(B * Hkv), 4), kLongThreads, 0,   \
                                       st>>>(qq, kk, Hq, Hkv, Lmax, d, cache_len, dom, n_dom, scale,  \
                                             k_top, thr, skeys);                                     \
  else                                                                                              \
    token_thr_kernel<T, C, G, SL, 1><<<dim3(static_cast<unsigned>(B * Hkv)), kLongThreads, 0, st>>>( \
        qq, kk, Hq, Hkv, Lmax, d, cache_len, dom, n_dom, scale, k_top, thr, skeys)
#define SA_TT(T, C, SL)                                                                             \
  do {                                                                                              \
    const auto* qq = static_cast<const T*>(q);                                                      \
    const auto* kk = static_cast<const T*>(k);                                                      \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&token_select_kernel<T, C, SL>), \
                                       hipFuncAttributeMaxDynamicSharedMemorySize,                  \
                                       static_cast<int>(token_select_lds_bytes(kMaxLongCols, kMaxCap))); \
    if (e != hipSuccess) return e;                                                                  \
    switch (grp) {                                                                                  \
      case 1: SA_TT_G(T, C, SL, 1); break;                                                          \
      case 2: SA_TT_G(T, C, SL, 2); break;                                                          \
      case 4: SA_TT_G(T, C, SL, 4); break;                                                          \
      case 8: SA_TT_G(T, C, SL, 8); break;                                                          \
      default: return hipErrorInvalidValue;                                                         \
    }                                                                                               \
    e = hipGetLastError();                                                                          \
    if (e != hipSuccess) return e;                                                                  \
    if (split) {                                                                                    \
      token_thr_pick_kernel<<<dim3(static_cast<unsigned>(rows)), kLongThreads, 0, st>>>(            \
          Hq, Lmax, cache_len, k_top, skeys, thr);                                                  \
      e = hipGetLastError();                                                                        \
      if (e != hipSuccess) return e;                                                                \
    }                                                                                               \
    e = launch_token_collect(q, k, dtype, B, Hq, Hkv, Lmax, d, cache_len, dom, n_dom, slab, scale,  \
                             col, st);                                                              \
    if (e != hipSuccess) return e;                                                                  \
    token_select_kernel<T, C, SL><<<dim3(static_cast<unsigned>(rows)), kLongThreads, lds, st>>>(    \
        qq, kk, Hq, Hkv, Lmax, d, cache_len, dom, n_dom, scale, k_top, col, cap, idx_out, max_out,  \
        count_out);                                                                                 \
  } while (0)
  if (dtype == kBF16) {
    if (slab) {
      switch (ndc) {
        case 8: SA_TT(uint16_t, 8, true); break;
        case 16: SA_TT(uint16_t, 16, true); break;
        case 32: SA_TT(uint16_t, 32, true); break;
        case 64: SA_TT(uint16_t, 64, true); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (ndc) {
        case 8: SA_TT(uint16_t, 8, false); break;
        case 16: SA_TT(uint16_t, 16, false); break;
        case 32: SA_TT(uint16_t, 32, false); break;
        case 64: SA_TT(uint16_t, 64, false); break;
        default: SA_TT(uint16_t, 128, false); break;
      }
    }
  } else {
    if (slab) {
      switch (ndc) {
        case 8: SA_TT(float, 8, true); break;
        case 16: SA_TT(float, 16, true); break;
        case 32: SA_TT(float, 32, true); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (ndc) {
        case 8: SA_TT(float, 8, false); break;
        case 16: SA_TT(float, 16, false); break;
        case 32: SA_TT(float, 32, false); break;
        case 64: SA_TT(float, 64, false); break;
        default: SA_TT(float, 128, false); break;
      }
    }
  }
#undef SA_TT
#undef SA_TT_G
  return hipGetLastError();
}

}  // namespace sa

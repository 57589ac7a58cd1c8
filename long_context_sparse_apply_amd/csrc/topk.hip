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
// Long rows (the decode token rows, up to 262144 columns): one 512-thread
// work-group per row.  A sampled threshold (the sample keys' rank that
// matches k plus a few standard deviations) lets one vectorised pass collect
// the candidates into an LDS buffer, where an MSB-first radix select (11 bits
// a level, LDS histogram) marks the k best in an LDS bitmap; an unlucky
// sample falls back to the radix select reading the row at each level.  The
// bitmap is finally compacted into ascending column indices.  The LDS is
// sized per launch from the row length and k, so two rows of the decode
// workloads share a CU.
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
constexpr int kLongThreads = 512;
constexpr int kDigit = 11;
constexpr int kBins = 1 << kDigit;
constexpr int kMaxCap = 8192;         // largest LDS candidate buffer (64-bit composites)
constexpr int kMaxLongCols = 262144;  // longest row (the host rejects longer ones)
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

__device__ __forceinline__ uint64_t composite(uint32_t key, int idx) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int comp_col(uint64_t c) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(c & 0xffffffffu));
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

size_t topk_lds_bytes(int cols, int cap) {
  const size_t words = (static_cast<size_t>(cols) + 31) / 32;
  return static_cast<size_t>(cap) * 8 + kBins * 4 + words * 4 + (kLongThreads / kWave + 4) * 4;
}

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
// their columns in the bitmap.
__device__ void select_in_lds(const TopkShared& sh, int nbuf, int need) {
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
__device__ void select_from_row(const TopkShared& sh, const float* s, int fa, int fb, int need) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int pbits = 0;
  if (tid == 0) *sh.nbuf = 0;
  __syncthreads();
  while (true) {
    int bsel, above, cntb;
    auto each = [&](auto f) {
      for (int i = fa + tid; i < fb; i += kLongThreads) f(composite(order_key(s[i]), i));
    };
    radix_level(sh, pbits, prefix, need, each, bsel, above, cntb);
    need -= above;
    const bool done = (cntb == need);
    const bool collect = !done && cntb <= sh.cap;
    for (int i = fa + tid; i < fb; i += kLongThreads) {
      const uint64_t c = composite(order_key(s[i]), i);
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
    const int seg_len = ncand / kSegs < kSegLen ? ncand / kSegs : kSegLen;
    const int nsamp = seg_len * kSegs;
    const double expect = static_cast<double>(k) * nsamp / ncand;
    int rank = static_cast<int>(expect + 4.0 * sqrt(expect) + 8.0);
    if (nsamp >= 1024 && rank < nsamp) {
      // 1. the rank-th largest sample (sample index as tie-break); each thread
      //    keeps its samples' keys in registers for the radix levels
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
      uint64_t prefix = 0;
      int pbits = 0, need = rank;
      while (true) {
        int bsel, above, cntb;
        auto each = [&](auto f) {
#pragma unroll
          for (int j = 0; j < kSampPerThread; ++j) {
            const int e = tid + j * kLongThreads;
            if (e < nsamp) f(composite(skey[j], e));
          }
        };
        radix_level(sh, pbits, prefix, need, each, bsel, above, cntb);
        need -= above;
        prefix = (prefix << kDigit) | static_cast<uint64_t>(bsel);
        pbits += kDigit;
        // 22 key bits (sign, exponent and 13 mantissa bits) place the
        // threshold within about 1e-4 of the sample at that rank: enough
        if (cntb == 1 || pbits >= 22) break;
      }
      // the key prefix, low bits zero: at most the sample key at that rank
      const uint32_t t_low = pbits >= 32 ? static_cast<uint32_t>(prefix >> (pbits - 32))
                                          : static_cast<uint32_t>(prefix << (32 - pbits));
      __syncthreads();
      if (tid == 0) *sh.nbuf = 0;
      __syncthreads();
      // 2. collect every candidate with key >= t_low.  For a value that is not
      //    NaN, key(v) >= t_low is v >= f_low, f_low the float whose key is
      //    t_low; a t_low at or below the key of -inf takes every value (NaN
      //    ranks as -inf), one above the key of +inf gives a NaN f_low that
      //    no value passes.
      const bool take_all = t_low <= 0x007fffffu;
      const float f_low = (t_low & 0x80000000u) ? __uint_as_float(t_low & 0x7fffffffu)
                                                : __uint_as_float(~t_low);
      auto qualifies = [&](float v) { return take_all || v >= f_low; };
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
          dst[u] = *reinterpret_cast<const float4*>(s + (i < a1 ? i : a0));
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
    // candidate buffer: k plus a quarter plus 1024 (the sampled threshold
    // overshoots k by a few standard deviations), at most kMaxCap
    int cap = k_const + k_const / 4 + 1024;
    cap = ((cap + 63) / 64) * 64;
    if (cap > kMaxCap) cap = kMaxCap;
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

}  // namespace sa

// Token importance from the dominant frequency chunks only.
//
// "FASA: Frequency-aware Sparse Attention", sec. 2.B item 1 (Token Importance
// Predictor: scores aggregated from the dominant frequency chunks) and sec.
// 2.C (the computation-optimised variant reads only a sparse subset of the
// key states).
//
//   s(b, h, t) = scale * sum_{i in D_g} (q_i k_{t,i} + q_{i+P} k_{t,i+P})
//
// A work-group walks a range of cached tokens of one (batch, KV head) in
// chunks of CT tokens and scores them for all Hq/Hkv query heads of the group,
// so every key byte is read once per group.  Each chunk's stored rows (the
// whole d-channel row in the standard layout, where the dominant pairs are
// scattered through it; only the 2*n_dom-channel dominant slab otherwise)
// stream into LDS with direct-to-LDS loads, double-buffered: chunk c + 1 loads
// while chunk c is scored.  Row r's 16-byte chunk j sits at chunk position
// j ^ (r % CPR).  A thread scores one token for its share of the query heads:
// it reads the token's dominant channels from LDS once (2-byte reads in the
// standard layout, 16-byte reads of the slab) and takes the query slices,
// staged once per work-group in LDS, as broadcast reads.
#include "sa_common.hpp"
#include "token_dot.hpp"
#include "topk_keys.hpp"

namespace sa {

template <typename T> struct TokElem;
template <> struct TokElem<uint16_t> {
  static __device__ __forceinline__ float lds(const uint8_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16);
  }
};
template <> struct TokElem<float> {
  static __device__ __forceinline__ float lds(const uint8_t* p) {
    return *reinterpret_cast<const float*>(p);
  }
};

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt not waited on): the LDS stores
// before a barrier complete too, which the barrier does not wait for.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// ROW: channels per stored row (d, or 2*n_dom for the slab); NDC: dominant
// channels per head (2*n_dom) rounded up; GRP: query heads per KV head.
template <typename T, int ROW, int GRP, int NDC>
struct TokenScoreShape {
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int ROWB = ROW * ES;
  static constexpr int CPR = ROWB / 16;
  static constexpr int CT0 = 32768 / ROWB;
  static constexpr int CT = CT0 < 256 ? CT0 : 256;           // tokens per chunk
  static constexpr int HGS0 = 256 / CT;                        // threads per token
  static constexpr int HGS = HGS0 < GRP ? HGS0 : GRP;
  static constexpr int HPT = GRP / HGS;                        // heads per thread
  static constexpr int CHB = CT * ROWB;                        // chunk bytes
  static constexpr int LPW = CHB / 1024 / 4;                   // DMA per wave per chunk
  static_assert(LPW * 4096 == CHB, "chunk must split over 4 waves");
};

// COLLECT: instead of storing the scores, append each token whose score
// passes its row's threshold key (and lies below cache_len) to the wave's own
// candidate list of that row and tile (blockIdx.x), as (score bits << 32 |
// token); the wave counts in scalars and writes its counts at the end
// (entries past the slots are dropped, the count stays true).  In this mode
// a chunk's CT rows are CT/64 runs of 64 tokens, run s from segment s of the
// tile (the tile split into CT/64 equal segments, walked 64 tokens a chunk),
// and row r belongs to wave (r / 64) mod (CT / 64) of its head group, so each
// wave's list is in ascending token order and a row's lists, taken in (tile,
// wave) order, are too.
template <typename T, int ROW, int GRP, int NDC, bool SLAB, bool COLLECT>
__global__ __launch_bounds__(256) void token_score_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int Hq, int Hkv, int Lmax, int d,
    const int32_t* __restrict__ cache_len, const int32_t* __restrict__ dom, int n_dom,
    float scale, float* __restrict__ scores, int chunks_per_wg, TokenCollect col) {
  using Sh = TokenScoreShape<T, ROW, GRP, NDC>;
  constexpr int ES = Sh::ES, ROWB = Sh::ROWB, CPR = Sh::CPR, CT = Sh::CT, HPT = Sh::HPT;
  constexpr int CHB = Sh::CHB, LPW = Sh::LPW;
  static_assert(!SLAB || ROW == NDC, "the slab row is exactly the dominant channels");
  static_assert(!COLLECT || CT % 64 == 0, "collect mode takes chunks of whole 64-token runs");
  __shared__ __attribute__((aligned(1024))) uint8_t sk0[CHB];
  __shared__ __attribute__((aligned(1024))) uint8_t sk1[CHB];
  // collect mode with chunks of at most 16 KB: a third stage
  constexpr bool THREE = COLLECT && CHB <= 16384;
  __shared__ __attribute__((aligned(1024))) uint8_t sk2[THREE ? CHB : 16];
  __shared__ __attribute__((aligned(16))) float s_q[GRP][NDC];
  __shared__ int s_off[NDC];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int P = d / 2;
  const int L = cache_len[b];
  const int ndc = 2 * n_dom;
  const int tb = blockIdx.x * chunks_per_wg * CT;                   // first token of this WG
  // chunks holding a token below Lmax (collect mode: segment 0 has the most)
  int nch = COLLECT ? (Lmax - tb + 63) / 64 : (Lmax - tb + CT - 1) / CT;
  nch = nch < chunks_per_wg ? nch : chunks_per_wg;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(k + (static_cast<int64_t>(b) * Hkv + g) * Lmax * ROW);

  // the token in row `row` of chunk c (collect mode: runs of 64 tokens from
  // the tile's CT/64 segments; scoring: CT consecutive tokens)
  const int seg_tokens = chunks_per_wg * 64;
  auto chunk_token = [&](int c, int row) {
    if constexpr (COLLECT)
      return tb + (row >> 6) * seg_tokens + c * 64 + (row & 63);
    else
      return tb + c * CT + row;
  };
  // stage chunk c's rows (tokens past the cache end re-read its last row);
  // the collect instances load through a buffer resource over this (b, KV
  // head)'s rows (at most 64 MiB), whose LDS writes the compiler tracks per
  // buffer.  Both forms load with the nontemporal hint: every key row is read
  // once, and the candidate lists written between the reads are small
  // partial lines.  With the hint the collect pass reads at 5.9-6.2 TB/s
  // instead of 5.2 (kernel traces: standard rows at 64K 413 -> 344 us, the
  // 128K slab 826 -> 730 us, the same selections)
  const auto rsrc = buffer_rsrc(kb, Lmax * ROWB);
  auto issue_one = [&](int c, int j, uint8_t* buf) {
    const int ins = wid * LPW + j;
    const int off = ins * 1024 + lane * 16;
    const int row = off / ROWB;
    const int pos = (off % ROWB) >> 4;
    const int tok = chunk_token(c, row);
    const int src = tok < Lmax ? tok : Lmax - 1;
    const int byte = src * ROWB + ((pos ^ (row % CPR)) << 4);
    if constexpr (COLLECT)
      lds_dma16_buf_nt(rsrc, byte, buf + ins * 1024);
    else
      lds_dma16_nt(kb + byte, buf + ins * 1024);
  };
  auto issue = [&](int c, uint8_t* buf) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) issue_one(c, j, buf);
  };
  if (!THREE && nch > 0) issue(0, sk0);

  // query slices (dominant channels, pre-scaled) and the stored channel of each
  for (int e = tid; e < GRP * NDC; e += 256) {
    const int hh = e / NDC, j = e % NDC;
    float v = 0.f;
    if (j < ndc) {
      // (a pair outside [0, d/2) gives undefined scores, never a read outside the row)
      const int qc = (dom[g * n_dom + (j % n_dom)] + (j >= n_dom ? P : 0)) & (d - 1);
      v = Elem<T>::load1(q + (static_cast<int64_t>(b) * Hq + g * GRP + hh) * d + qc) * scale;
    }
    s_q[hh][j] = v;
  }
  if (tid < NDC) {
    int c = 0;
    if (tid < ndc) c = SLAB ? tid : (dom[g * n_dom + (tid % n_dom)] + (tid >= n_dom ? P : 0)) & (d - 1);
    s_off[tid] = c * ES;  // byte offset of the channel within an unswizzled row
  }

  static_assert(CT * Sh::HGS0 == 256, "a chunk's tokens times the head groups fill the work-group");
  const int r = tid % CT;              // this thread's token within a chunk
  const int hg = tid / CT;             // its head group (HGS groups of HPT heads)
  // (one head group: every thread scores; known to the compiler in collect mode)
  const bool active = (COLLECT && Sh::HGS0 == 1) || hg * HPT < GRP;
  const int hh0 = active ? hg * HPT : 0;  // the group's first head (a valid one when idle)
  // collect mode, per head of the thread's group (uniform over the wave):
  // candidates so far, the threshold as a float test, and the wave's list
  int wcnt[HPT];
  float f_low[HPT];
  bool take_all[HPT];
  uint64_t* lst[HPT];
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    wcnt[u] = 0;
    if constexpr (COLLECT) {
      const int64_t srow = static_cast<int64_t>(b) * Hq + g * GRP + (hh0 + u < GRP ? hh0 + u : 0);
      const KeyThreshold kt(col.thr[srow]);
      f_low[u] = kt.f_low;
      take_all[u] = kt.take_all;
      lst[u] = col.cand + ((srow * col.tiles + blockIdx.x) * kCollectWaves + wid) * kCollectSlots;
    }
  }
  const int rx = r % CPR;

  // collect mode: a chunk's candidates wait in registers (pend_*) and are
  // stored at the start of the next step, before its loads
  uint64_t pend_v[COLLECT ? HPT : 1];
  int pend_s[COLLECT ? HPT : 1];
  bool pend_p[COLLECT ? HPT : 1];
#pragma unroll
  for (int u = 0; u < (COLLECT ? HPT : 1); ++u) pend_p[u] = false;
  auto flush = [&]() {
    if constexpr (COLLECT) {
#pragma unroll
      for (int u = 0; u < HPT; ++u)
        if (pend_p[u]) lst[u][static_cast<uint32_t>(pend_s[u])] = pend_v[u];
    }
  };
  auto score_chunk = [&](int c, const uint8_t* buf) {
    if (!active) return;
    const int t = chunk_token(c, r);
    const uint8_t* rowp = buf + r * ROWB;
    float kv[NDC];
    if constexpr (SLAB) {
#pragma unroll
      for (int j = 0; j < CPR; ++j) {
        const uint4 w = *reinterpret_cast<const uint4*>(rowp + ((j ^ rx) << 4));
        float tmp[8];
        if constexpr (ES == 2) {
          Elem<uint16_t>::unpack8(w, tmp);
#pragma unroll
          for (int e = 0; e < 8; ++e) kv[j * 8 + e] = tmp[e];
        } else {
          kv[j * 4 + 0] = __uint_as_float(w.x); kv[j * 4 + 1] = __uint_as_float(w.y);
          kv[j * 4 + 2] = __uint_as_float(w.z); kv[j * 4 + 3] = __uint_as_float(w.w);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NDC; ++j) {
        const int byte = s_off[j];
        kv[j] = TokElem<T>::lds(rowp + ((((byte >> 4) ^ rx)) << 4) + (byte & 15));
      }
    }
    // (t < Lmax too: the selection's row length is cache_len clamped to Lmax)
    const bool tin = t < L && t < Lmax;
#pragma unroll
    for (int u = 0; u < HPT; ++u) {
      const int hh = hg * HPT + u;
      const float acc = token_dot<NDC>(&s_q[hh][0], kv);
      const int64_t srow = static_cast<int64_t>(b) * Hq + g * GRP + hh;
      if constexpr (COLLECT) {
        // (KeyThreshold::qualifies with the test's parts held per head)
        const bool ok = tin & (take_all[u] | (acc >= f_low[u]));
        const uint64_t m = __ballot(ok);
        const int pos = wcnt[u] + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                      static_cast<uint32_t>(m >> 32),
                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
        pend_p[u] = ok & (pos < kCollectSlots);
        pend_s[u] = pos;
        pend_v[u] = (static_cast<uint64_t>(__float_as_uint(acc)) << 32) | static_cast<uint32_t>(t);
        wcnt[u] += __popcll(m);
      } else {
        if (t < Lmax) scores[srow * Lmax + t] = (t < L) ? acc : -INFINITY;
      }
    }
  };

  if constexpr (THREE) {
    // Three stages, two chunks in flight.  Step c: wait for chunk c's loads,
    // barrier (every share landed; chunk c - 1's buffer is free), store
    // chunk c - 1's candidates, issue chunk c + 2 into the free buffer, score
    // chunk c.  A wave's vector memory operations complete in issue order,
    // and after chunk c's loads it issued only chunk c - 2's stores and
    // chunk c + 1's loads (LPW, if any): waiting until LPW remain covers
    // chunk c (and those stores, one step after they were issued).
    if (nch > 0) issue(0, sk0);
    if (nch > 1) issue(1, sk1);
    auto step = [&](int c, const uint8_t* cur, uint8_t* ahead) {
      if (c + 1 < nch)
        wait_vm_lgkm0<LPW>();
      else
        wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      flush();
      if (c + 2 < nch) issue(c + 2, ahead);
      score_chunk(c, cur);
    };
    for (int c = 0; c < nch; c += 3) {
      step(c, sk0, sk2);
      if (c + 1 >= nch) break;
      step(c + 1, sk1, sk0);
      if (c + 2 >= nch) break;
      step(c + 2, sk2, sk1);
    }
    flush();
  } else {
    // wait for chunk c, barrier (every share landed; every thread is done
    // with chunk c - 1, whose buffer is free), issue chunk c + 1, score c
    // (collect mode: each chunk's candidates are stored at once)
    for (int c = 0; c < nch; c += 2) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (c + 1 < nch) issue(c + 1, sk1);
      score_chunk(c, sk0);
      flush();
      if (c + 1 >= nch) break;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (c + 2 < nch) issue(c + 2, sk0);
      score_chunk(c + 1, sk1);
      flush();
    }
  }

  // collect mode: the wave's counts of this tile for every head of the
  // group (zero for the heads of other waves' groups, whose lists it leaves)
  if constexpr (COLLECT) {
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < GRP; ++hh) {
        int v = 0;
#pragma unroll
        for (int u = 0; u < HPT; ++u)
          if (active && hg * HPT + u == hh) v = wcnt[u];
        col.cnt[((static_cast<int64_t>(b) * Hq + g * GRP + hh) * col.tiles + blockIdx.x) * kCollectWaves + wid] = v;
      }
    }
  }
}

// Scoring (COLLECT false: every score into `scores`) or candidate collection
// for the fused token top-k (COLLECT true).
template <bool COLLECT>
static hipError_t launch_scoring(const void* q, const void* k, int dtype, int B, int Hq, int Hkv,
                                 int Lmax, int d, const int32_t* cache_len, const int32_t* dom,
                                 int n_dom, int slab, float scale, float* scores,
                                 const TokenCollect& col, hipStream_t st) {
  const int row = slab ? 2 * n_dom : d;
  const int grp = Hq / Hkv;
  const int ndc_need = 2 * n_dom;
  const int ndc = ndc_need <= 8 ? 8 : ndc_need <= 16 ? 16 : ndc_need <= 32 ? 32 : ndc_need <= 64 ? 64 : 128;
  const int es = dtype == kBF16 ? 2 : 4;
  const int ct0 = 32768 / (row * es);
  const int ct = ct0 < 256 ? ct0 : 256;
  // about 4096 tokens per work-group, fewer when that leaves under ~2048 work-groups
  const int per_head_chunks = (Lmax + ct - 1) / ct;
  int cpw = 4096 / ct;
  // (collect mode keeps tiles of kCollectTile tokens: its lists are laid out per tile)
  while (!COLLECT && cpw > 1 &&
         static_cast<int64_t>(B) * Hkv * ((per_head_chunks + cpw - 1) / cpw) < 2048)
    cpw /= 2;
  if (COLLECT && cpw * ct != kCollectTile) return hipErrorInvalidValue;
  const dim3 grid((per_head_chunks + cpw - 1) / cpw, Hkv, B);
#define SA_TS(T, R, G, C, SL)                                                                  \
  token_score_kernel<T, R, G, C, SL, COLLECT><<<grid, 256, 0, st>>>(                            \
      static_cast<const T*>(q), static_cast<const T*>(k), Hq, Hkv, Lmax, d, cache_len, dom,     \
      n_dom, scale, scores, cpw, col)
#define SA_TS_G(T, R, C, SL)                  \
  switch (grp) {                              \
    case 1: SA_TS(T, R, 1, C, SL); break;     \
    case 2: SA_TS(T, R, 2, C, SL); break;     \
    case 4: SA_TS(T, R, 4, C, SL); break;     \
    case 8: SA_TS(T, R, 8, C, SL); break;     \
    default: return hipErrorInvalidValue;     \
  }
#define SA_TS_STD(T, D)                             \
  switch (ndc) {                                    \
    case 8: SA_TS_G(T, D, 8, false) break;          \
    case 16: SA_TS_G(T, D, 16, false) break;        \
    case 32: SA_TS_G(T, D, 32, false) break;        \
    case 64: SA_TS_G(T, D, 64, false) break;        \
    default: SA_TS_G(T, D, 128, false) break;       \
  }
#define SA_TS_DT(T)                                                    \
  if (slab) {                                                          \
    switch (row) {                                                     \
      case 8: SA_TS_G(T, 8, 8, true) break;                            \
      case 16: SA_TS_G(T, 16, 16, true) break;                         \
      case 32: SA_TS_G(T, 32, 32, true) break;                         \
      case 64: SA_TS_G(T, 64, 64, true) break;                         \
      case 128: SA_TS_G(T, 128, 128, true) break;                      \
      default: return hipErrorInvalidValue;                            \
    }                                                                  \
  } else if (d == 128) {                                               \
    SA_TS_STD(T, 128)                                                  \
  } else {                                                             \
    if (ndc > 64) return hipErrorInvalidValue;                         \
    SA_TS_STD(T, 64)                                                   \
  }
  if (dtype == kBF16) {
    SA_TS_DT(uint16_t)
  } else {
    SA_TS_DT(float)
  }
#undef SA_TS_DT
#undef SA_TS_STD
#undef SA_TS_G
#undef SA_TS
  return hipGetLastError();
}

hipError_t launch_token_score(const void* q, const void* k, int dtype, int B, int Hq, int Hkv,
                              int Lmax, int d, const int32_t* cache_len, const int32_t* dom,
                              int n_dom, int slab, float scale, float* scores, hipStream_t st) {
  return launch_scoring<false>(q, k, dtype, B, Hq, Hkv, Lmax, d, cache_len, dom, n_dom, slab, scale,
                               scores, TokenCollect{}, st);
}

hipError_t launch_token_collect(const void* q, const void* k, int dtype, int B, int Hq, int Hkv,
                                int Lmax, int d, const int32_t* cache_len, const int32_t* dom,
                                int n_dom, int slab, float scale, const TokenCollect& col,
                                hipStream_t st) {
  return launch_scoring<true>(q, k, dtype, B, Hq, Hkv, Lmax, d, cache_len, dom, n_dom, slab, scale,
                              nullptr, col, st);
}

}  // namespace sa

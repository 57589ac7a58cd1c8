// Focused decode attention over the selected tokens, split-K across CUs.
//
// "FASA: Frequency-aware Sparse Attention", sec. 2.B item 2 (full-dimension
// attention over the selected subset T_t, at the tokens' original positions)
// and sec. 2.C (both variants read only the selected key/value rows).
//
// Grid: (splits, B*Hq).  A work-group walks cpw chunks of 256 consecutive
// entries of one (b, h) selection list; each of its 4 waves takes 64 entries
// of a chunk and keeps a running softmax over its chunks.  With at least two
// lists per CU a work-group takes a whole list (cpw = all chunks, one pass);
// with fewer, each takes one chunk and a merge pass combines the splits.
// A token row (d channels) is spread over LPT = d/8 lanes with one 16-byte
// load each, so a wave gathers 4 rows per instruction; for each chunk the
// wave first loads its 64 indices with one coalesced load and hands them out
// by shuffle, then issues all its key and value loads together before using
// any (32 KB in flight per wave).
// A one-pass work-group writes the output itself; otherwise each leaves
// (max, sum, unnormalised output) for its split in the workspace and a
// second kernel merges the splits with the log-sum-exp rule
//     M = max m_s,  L = sum l_s e^{m_s - M},  o = sum o_s e^{m_s - M} / L.
//
// With the dominant-slab key layout the key row is the concatenation of its
// k_dom part (read by the first 2*n_dom/8 lanes) and its k_rest part (the
// other lanes); the query is permuted to the same channel order, since the
// dot product does not depend on the order of channels.
#include <mutex>

#include "sa_common.hpp"

namespace sa {

// (chunk and wave counts: sa_limits.hpp; splits and workspace size: host_sizes.cpp)
constexpr int kDecPerWave = kDecChunk / kDecWaves;

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ k_rest,
    const T* __restrict__ v, int Hq, int Hkv, int Lmax, const int32_t* __restrict__ dom,
    int n_dom, int slab, const int32_t* __restrict__ tok_idx, const int32_t* __restrict__ tok_cnt,
    int max_k, float scale, int splits, int cpw, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, T* __restrict__ out, float* __restrict__ lse) {
  constexpr int LPT = D / 8;
  constexpr int TPI = kWave / LPT;
  constexpr int STEPS = kDecPerWave / TPI;
  constexpr int P = D / 2;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int sub = lane % LPT;
  const int grp_tok = lane / LPT;
  const int split = blockIdx.x;
  // one pass over a multiple of 8 lists: list ids in XCD-contiguous ranges
  // (work-groups go to the 8 XCDs in turn), so the query heads of a KV group
  // share an XCD and a row that two of them select can come from its L2
  int bh = blockIdx.y;
  if (gridDim.x == 1 && (gridDim.y & 7) == 0) bh = (bh & 7) * (gridDim.y >> 3) + (bh >> 3);
  const int h = bh % Hq;
  const int b = bh / Hq;
  const int g = h / (Hq / Hkv);
  // the count is clamped to the list width, so a count above it (a caller's
  // stale buffer) never reads past the row of indices
  const int cnt = min(max(tok_cnt[bh], 0), max_k);

  __shared__ int s_ch[D];
  __shared__ unsigned long long s_dmask[(D + 63) / 64];
  __shared__ float s_m[kDecWaves], s_l[kDecWaves];
  __shared__ float s_o[kDecWaves][D];

  // channel order of the key row as the lanes read it: identity, or with the
  // slab layout the dominant channels (in slab order) followed by the others
  // in ascending order.  Built in parallel: thread t < D tests channel t
  // against the dominant set, a ballot gives the set as a bit mask, and a
  // non-dominant channel's slot is 2 n_dom + the number of non-dominant
  // channels below it.
  const int dom_w = slab ? 2 * n_dom : D;  // channels stored in `k`
  if (slab) {
    bool isdom = false;
    if (tid < D) {
      for (int j = 0; j < n_dom; ++j) {
        const int c = dom[g * n_dom + j];
        isdom |= (tid == c) || (tid == c + P);
      }
    }
    const unsigned long long m = __ballot(isdom);
    if (tid < D && lane == 0) s_dmask[wid] = m;
    // (pairs outside [0, d/2) or repeated give undefined output, never an
    // access outside the query row or s_ch)
    if (tid < 2 * n_dom) s_ch[tid] = (dom[g * n_dom + (tid % n_dom)] + (tid >= n_dom ? P : 0)) & (D - 1);
    __syncthreads();
    if (tid < D && !isdom) {
      int below = __popcll(~s_dmask[wid] & ((1ull << lane) - 1ull));
      if (wid == 1) below += __popcll(~s_dmask[0]);
      if (2 * n_dom + below < D) s_ch[2 * n_dom + below] = tid;
    }
    __syncthreads();
  }
  float qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = slab ? s_ch[sub * 8 + j] : sub * 8 + j;
    qv[j] = Elem<T>::load1(q + static_cast<int64_t>(bh) * D + c) * scale;
  }

  const int64_t head_rows = (static_cast<int64_t>(b) * Hkv + g) * Lmax;
  const T* krow_base;
  int kstride, kofs;
  if (!slab || sub * 8 < dom_w) {
    krow_base = k;
    kstride = dom_w;
    kofs = sub * 8;
  } else {
    krow_base = k_rest;
    kstride = D - dom_w;
    kofs = sub * 8 - dom_w;
  }

  using Raw = typename Elem<T>::Raw;
  // running softmax state of this wave over its share of cpw chunks
  float m_run = -INFINITY, lsum = 0.f;
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.f;
  for (int ci = 0; ci < cpw; ++ci) {
    const int first = (split * cpw + ci) * kDecChunk + wid * kDecPerWave;
    if (first >= cnt) break;
    // this wave's 64 indices, one per lane (every later load needs them)
    const int my_pos = first + lane;
    const int my_idx = (my_pos < cnt) ? tok_idx[static_cast<int64_t>(bh) * max_k + my_pos] : -1;
    int tok[STEPS];
#pragma unroll
    for (int it = 0; it < STEPS; ++it) {
      const int t = __shfl(my_idx, it * TPI + grp_tok, kWave);
      tok[it] = (t >= 0 && t < Lmax) ? t : -1;  // out-of-range entries are ignored
    }
    // gather every key and value row of the wave before using any of them,
    // with the nontemporal hint (the decode attention at batch 16 / 64K cache
    // 98-101 -> 92-93 us and at batch 64 / 128K 703-707 -> 655-656 us with
    // it, outputs unchanged)
    Raw kr[STEPS], vr[STEPS];
#pragma unroll
    for (int it = 0; it < STEPS; ++it) {
      kr[it] = tok[it] >= 0 ? Elem<T>::load_raw8_nt(krow_base + (head_rows + tok[it]) * kstride + kofs)
                            : Elem<T>::zero_raw8();
      vr[it] = tok[it] >= 0 ? Elem<T>::load_raw8_nt(v + (head_rows + tok[it]) * D + sub * 8)
                            : Elem<T>::zero_raw8();
    }
    float logit[STEPS];
#pragma unroll
    for (int it = 0; it < STEPS; ++it) {
      float kv[8];
      Elem<T>::unpack8(kr[it], kv);
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) a = fmaf(qv[j], kv[j], a);
#pragma unroll
      for (int sh = LPT / 2; sh >= 1; sh >>= 1) a += __shfl_xor(a, sh, kWave);
      logit[it] = tok[it] >= 0 ? a : -INFINITY;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int it = 0; it < STEPS; ++it) mloc = fmaxf(mloc, logit[it]);
    const float mw = wave_max(mloc);
    if (mw > -INFINITY) {
      const float m_new = fmaxf(m_run, mw);
      const float alpha = (m_run == -INFINITY) ? 0.f : __expf(m_run - m_new);
      lsum *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] *= alpha;
      m_run = m_new;
#pragma unroll
      for (int it = 0; it < STEPS; ++it) {
        const float p = tok[it] >= 0 ? __expf(logit[it] - m_run) : 0.f;
        lsum += p;
        float vv[8];
        Elem<T>::unpack8(vr[it], vv);
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = fmaf(p, vv[j], o[j]);
      }
    }
  }
  const float mw = m_run;
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
    lsum += __shfl_xor(lsum, off, kWave);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] += __shfl_xor(o[j], off, kWave);
  }
  if (lane == 0) {
    s_m[wid] = mw;
    s_l[wid] = lsum;
  }
  if (lane < LPT) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s_o[wid][lane * 8 + j] = o[j];
  }
  __syncthreads();
  if (tid < D) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, s_m[w]);
    float L = 0.f, O = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float f = (s_m[w] > -INFINITY) ? __expf(s_m[w] - M) : 0.f;
        L += s_l[w] * f;
        O += s_o[w][tid] * f;
      }
    }
    if (splits == 1) {
      // the work-group saw every selected token: final output, no merge pass
      Elem<T>::store1(out + static_cast<int64_t>(bh) * D + tid, (L > 0.f) ? O / L : 0.f);
      if (lse && tid == 0) lse[bh] = (L > 0.f) ? M + logf(L) : -INFINITY;
    } else {
      const int64_t part = static_cast<int64_t>(bh) * splits + split;
      ws_o[part * D + tid] = O;
      if (tid == 0) {
        ws_m[part] = M;
        ws_l[part] = L;
      }
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ ws_m,
                                                         const float* __restrict__ ws_l,
                                                         const float* __restrict__ ws_o, int splits,
                                                         T* __restrict__ out, float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t base = static_cast<int64_t>(bh) * splits;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ws_m[base + s]);
  float L = 0.f, O = 0.f;
  if (M > -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float m = ws_m[base + s];
      if (m == -INFINITY) continue;
      const float f = __expf(m - M);
      L += ws_l[base + s] * f;
      O += ws_o[(base + s) * D + t] * f;
    }
  }
  const float res = (L > 0.f) ? O / L : 0.f;
  Elem<T>::store1(out + static_cast<int64_t>(bh) * D + t, res);
  if (lse && t == 0) lse[bh] = (L > 0.f) ? M + logf(L) : -INFINITY;
}

// Split-K partials of the allocation-free entry point: one array per GPU,
// held until the process ends, located once per device with
// hipGetSymbolAddress (in host code the array's name is not its device
// address).  Calls that overlap on one GPU share it and race.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_static_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const void* q, const void* k, const void* k_rest, const void* v,
                         int dtype, int B, int Hq, int Hkv, int Lmax, int d,
                         const int32_t* cache_len, const int32_t* dom, int n_dom, int slab,
                         const int32_t* tok_idx, const int32_t* tok_cnt, int max_k, float scale,
                         void* out, float* lse, void* ws, hipStream_t st) {
  (void)cache_len;
  const DecodePlan plan = decode_plan(B, Hq, max_k);
  const int cpw = plan.cpw;
  const int splits = plan.splits;
  const int64_t parts = static_cast<int64_t>(B) * Hq * splits;
  float* ws_m = static_cast<float*>(ws);
  float* ws_l = ws_m + parts;
  float* ws_o = ws_l + parts;
  const dim3 grid(splits, B * Hq);
#define SA_DEC(T, D)                                                                              \
  decode_partial_kernel<T, D><<<grid, 256, 0, st>>>(                                              \
      static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(k_rest),          \
      static_cast<const T*>(v), Hq, Hkv, Lmax, dom, n_dom, slab, tok_idx, tok_cnt, max_k, scale,  \
      splits, cpw, ws_m, ws_l, ws_o, static_cast<T*>(out), lse);                                  \
  if (splits > 1)                                                                                 \
    decode_merge_kernel<T, D><<<dim3(B * Hq), D, 0, st>>>(ws_m, ws_l, ws_o, splits,               \
                                                          static_cast<T*>(out), lse)
  if (dtype == kBF16) {
    if (d == 128) { SA_DEC(uint16_t, 128); } else { SA_DEC(uint16_t, 64); }
  } else {
    if (d == 128) { SA_DEC(float, 128); } else { SA_DEC(float, 64); }
  }
#undef SA_DEC
  return hipGetLastError();
}

}  // namespace sa

// Block-sparse prefill attention over the selected key blocks.
//
// "Prism: Spectral-Aware Block-Sparse Attention", sec. 1: attention is
// computed only for a subset of relevant key blocks.  For a query at position
// t in query block I of head h, the keys are those of the blocks listed for
// (h, I); with the causal mask only keys s <= t count.  K/V come from KV head
// h / (Hq/Hkv).
//
// bf16 path (d in {64, 128}, block in {64, 128}): one work-group per
// (b, h, I) with one wave per 32 queries.  For every selected key block the
// work-group stages K (row-major) and V (transposed, [d][key]) in LDS; each
// wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS,
// B = Q^T held in registers for the whole block list), so the C layout leaves
// one query per lane column and 16 keys per lane.  The online softmax (fp32,
// base-2 exponent with the scale folded in) runs on those registers; the
// probabilities are rounded to bf16 and used directly as the B operand of
// O^T += V^T P^T (the k-slot order of P^T matches the C layout of S^T, and
// V^T is read from LDS in the same key order), so P never leaves registers.
//
// Work order: large query blocks first (their lists are the longest) and all
// work of one KV group placed on one XCD when the grid divides evenly, so the
// four query heads that read the same K/V blocks share that XCD's L2.
//
// fp32 path: a plain kernel, one query per LPT = d/8 lanes, online softmax
// over the selected keys in order, fp32 throughout.
#include "sa_common.hpp"

namespace sa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// map a flat work-group id to (b, h, I): heavy query blocks first, one KV
// group per XCD chunk when the grid splits evenly over the 8 XCDs
__device__ __forceinline__ void prefill_work_item(int x, int nwg, int B, int Hq, int Hkv, int N,
                                                  int& b, int& h, int& I) {
  int w = x;
  if ((nwg & 7) == 0) w = (x & 7) * (nwg >> 3) + (x >> 3);
  const int grp = Hq / Hkv;
  const int hh = w % grp;
  w /= grp;
  const int Ir = w % N;
  w /= N;
  const int g = w % Hkv;
  b = w / Hkv;
  h = g * grp + hh;
  I = N - 1 - Ir;
}

// ------------------------------------------------------------------ bf16 MFMA kernel
// LDS tile: ROWS rows (keys) x D bf16, row-major, rows unpadded; the 16-byte
// chunk c of row r sits at chunk position c ^ sw(r), with
// sw(r) = 2 (r mod CPR/2) + (r div CPR/2 mod 2).  sw is one-to-one on r mod CPR,
// so the 16 consecutive rows of a K operand read land on 16 distinct bank
// groups; and for the 4 consecutive rows x 2 adjacent chunks of a V transpose
// read it yields 8 distinct positions.  Tiles are filled by direct-to-LDS
// loads (global_load_lds_dwordx4): one wave instruction writes 1 KB of
// consecutive LDS bytes, lane i its 16 bytes at offset 16 i, and each lane
// fetches the global chunk that belongs there.
template <int D, int ROWS, int NW>
struct LdsTile {
  static constexpr int ROWB = D * 2;                 // bytes per row
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int LPW = BYTES / 1024 / NW;      // load instructions per wave per tile
  static_assert(LPW * NW * 1024 == BYTES, "tile must split evenly over the waves");

  static __device__ __forceinline__ int sw(int row) {
    return ((row % (CPR / 2)) << 1) | ((row / (CPR / 2)) & 1);
  }
  static __device__ __forceinline__ int phys(int row, int chunk) {
    return row * ROWB + ((chunk ^ sw(row)) << 4);
  }
  // issue this wave's share of the tile's direct-to-LDS loads (asynchronous)
  static __device__ __forceinline__ void issue(const uint16_t* g, uint8_t* lds, int wid, int lane) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int ins = wid * LPW + j;
      const int off = ins * 1024 + lane * 16;
      const int row = off / ROWB;
      const int pos = (off % ROWB) >> 4;
      const int chunk = pos ^ sw(row);
      const uint8_t* src = reinterpret_cast<const uint8_t*>(g) + row * ROWB + chunk * 16;
      lds_dma16(src, lds + ins * 1024);
    }
  }
};

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left at their maxima (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ u32x2 lds_read_tr(const uint8_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) uint8_t*)(p)));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Per-lane state of the online softmax of one wave (32 queries, one per lane
// column; lanes l and l ^ 32 hold the two key halves of the same query).
template <int DT>
struct SoftmaxState {
  f32x16 acc_o[DT];
  float m_ref;   // reference max (base 2)
  float l_part;  // this lane's half of the denominator
};

// One 64-key chunk: S^T = K Q^T, masked and exponentiated in place, then
// O^T += V^T P^T.  kbuf / vbuf hold the chunk's K and V rows (swizzled).
template <int D>
__device__ __forceinline__ void prefill_chunk(const uint8_t* kbuf, const uint8_t* vbuf,
                                              const bf16x8 (&qf)[D / 16],
                                              SoftmaxState<D / 32>& st, float sl2, int key0,
                                              int qloc, bool diag, int l32, int hi, int grp16,
                                              int i16) {
  using Tile = LdsTile<D, 64, 1>;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr float kRescale = 8.f;
  f32x16 sacc[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint4 w = *reinterpret_cast<const uint4*>(&kbuf[Tile::phys(kt * 32 + l32, 2 * s + hi)]);
      u32x4 t = {w.x, w.y, w.z, w.w};
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, t), qf[s],
                                                          sacc[kt], 0, 0, 0);
    }
  float mblk = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (diag && key0 + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3) > qloc) sacc[kt][r] = -INFINITY;
      mblk = fmaxf(mblk, sacc[kt][r]);
    }
  mblk = fmaxf(mblk, __shfl_xor(mblk, 32, 64)) * sl2;
  const bool raise = mblk > st.m_ref + kRescale;
  if (__ballot(raise)) {
    const float m_new = raise ? mblk : st.m_ref;
    const float alpha = (st.m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m_ref - m_new);
    st.l_part *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc_o[dt][r] *= alpha;
    st.m_ref = m_new;
  }
  const float m_use = (st.m_ref == -INFINITY) ? 0.f : st.m_ref;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], sl2, -m_use));
      sacc[kt][r] = p;
      st.l_part += p;
    }
  // O^T += V^T P^T, 16 keys per k-step.  P^T k-slots 0-3 hold keys 16s + 4hi + i
  // (registers 8u + i of tile s/2), slots 4-7 keys 16s + 8 + 4hi + i (registers
  // 8u + 4 + i): registers 8u .. 8u + 7 in order.  The V^T operand (row d = dt*32 +
  // l32, the same key slots) comes from the transpose read: lane (group G, index i)
  // addresses key row 16s + 4(G/2) + i/4 [+8] at channels dt*32 + (G%2)*16 + 4(i%4),
  // and the hardware hands each lane its own column.
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int kt = s >> 1, u = s & 1;
    u32x4 pw;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pw[i] = cvt_pk_bf16(sacc[kt][8 * u + 2 * i], sacc[kt][8 * u + 2 * i + 1]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
    const int vrow = 16 * s + 4 * (grp16 >> 1) + (i16 >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int col = dt * 32 + (grp16 & 1) * 16 + 4 * (i16 & 3);
      const int chunk = col >> 3, within = (col & 7) * 2;
      const u32x2 v0 = lds_read_tr(&vbuf[Tile::phys(vrow, chunk) + within]);
      const u32x2 v1 = lds_read_tr(&vbuf[Tile::phys(vrow + 8, chunk) + within]);
      u32x4 vw = {v0[0], v0[1], v1[0], v1[1]};
      st.acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pf,
                                                              st.acc_o[dt], 0, 0, 0);
    }
  }
}

// One work-group per (b, h, I), one wave per 32 queries.  The selected key
// blocks are walked as 64-key chunks; chunk c's K and V rows live in LDS
// buffer c % 2 and chunk c + 1 streams into the other buffer (direct-to-LDS,
// asynchronous) while chunk c is computed, so loads overlap the matrix work.
// The loop is unrolled by two so each half names its buffers statically.
// Per chunk each wave computes S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K
// from LDS, B = Q^T in registers), the online softmax on the accumulators
// (base 2, scale folded into one FMA, the reference max raised only when a
// chunk exceeds it by more than 8, so p <= 2^8), and O^T += V^T P^T with P^T
// taken straight from the S^T registers and V^T from the LDS transpose read.
template <int D, int BS>
__global__ __launch_bounds__(BS * 2) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int B, int Hq, int Hkv, int S, const int32_t* __restrict__ blk_idx,
    const int32_t* __restrict__ blk_cnt, int max_sel, int causal, float scale,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int NW = BS / 32;
  using Tile = LdsTile<D, 64, NW>;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPB = BS / 64;         // 64-key chunks per block
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[Tile::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[Tile::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[Tile::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[Tile::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp16 = lane >> 4;
  const int i16 = lane & 15;
  const int N = S / BS;
  int b, h, I;
  prefill_work_item(blockIdx.x, gridDim.x, B, Hq, Hkv, N, b, h, I);
  const int g = h / (Hq / Hkv);
  const int64_t qrow0 = (static_cast<int64_t>(b) * Hq + h) * S + static_cast<int64_t>(I) * BS;
  const uint16_t* kbase = k + (static_cast<int64_t>(b) * Hkv + g) * S * D;
  const uint16_t* vbase = v + (static_cast<int64_t>(b) * Hkv + g) * S * D;
  const int64_t sel0 = ((static_cast<int64_t>(b) * Hq + h) * N + I);

  // the block list, read with uniform (scalar) loads; entries out of range or
  // above the diagonal (causal) are skipped
  const int cnt = blk_cnt[sel0];
  const int32_t* sel = blk_idx + sel0 * max_sel;
  auto next_valid = [&](int from) {
    for (int t = from; t < cnt; ++t) {
      const int J = sel[t];
      if (J >= 0 && J < N && !(causal && J > I)) return t;
    }
    return cnt;
  };

  // Q^T fragments: this lane's query and 8 channels per k-step
  const int qloc = wid * 32 + l32;
  bf16x8 qf[KS];
  {
    const uint16_t* qp = q + (qrow0 + qloc) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 w = *reinterpret_cast<const uint4*>(qp + 16 * s);
      u32x4 t = {w.x, w.y, w.z, w.w};
      qf[s] = __builtin_bit_cast(bf16x8, t);
    }
  }
  const float sl2 = scale * kLog2e;
  SoftmaxState<DT> st;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc_o[dt][r] = 0.f;
  st.m_ref = -INFINITY;
  st.l_part = 0.f;

  // chunk cursor: list position t, chunk c within the block
  int t = next_valid(0), c = 0;
  auto issue_chunk = [&](int tt, int cc, uint8_t* kb, uint8_t* vb) {
    const int64_t row0 = static_cast<int64_t>(sel[tt]) * BS + cc * 64;
    Tile::issue(kbase + row0 * D, kb, wid, lane);
    Tile::issue(vbase + row0 * D, vb, wid, lane);
  };
  auto advance = [&](int& tt, int& cc) {
    if (cc + 1 < CPB) { ++cc; } else { tt = next_valid(tt + 1); cc = 0; }
  };
  // Per chunk: wait for this wave's share of chunk c, barrier (every share has
  // landed and every wave has finished chunk c - 1, whose buffers are free),
  // issue chunk c + 1 into those buffers, compute chunk c.
  if (t < cnt) issue_chunk(t, c, sK0, sV0);
  while (t < cnt) {
    // ---- even half: chunk in buffers 0, next chunk into buffers 1
    {
      int tn = t, cn = c;
      advance(tn, cn);
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (tn < cnt) issue_chunk(tn, cn, sK1, sV1);
      const int J = sel[t];
      prefill_chunk<D>(sK0, sV0, qf, st, sl2, c * 64, qloc, causal && J == I, l32, hi, grp16, i16);
      t = tn;
      c = cn;
    }
    if (t >= cnt) break;
    // ---- odd half: chunk in buffers 1, next chunk into buffers 0
    {
      int tn = t, cn = c;
      advance(tn, cn);
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (tn < cnt) issue_chunk(tn, cn, sK0, sV0);
      const int J = sel[t];
      prefill_chunk<D>(sK1, sV1, qf, st, sl2, c * 64, qloc, causal && J == I, l32, hi, grp16, i16);
      t = tn;
      c = cn;
    }
  }

  // normalise and store: lane holds query qloc, channels dt*32 + 8j + 4hi + i
  const float l_run = st.l_part + __shfl_xor(st.l_part, 32, 64);
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  uint16_t* op = out + (qrow0 + qloc) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 w = {cvt_pk_bf16(st.acc_o[dt][4 * j + 0] * inv, st.acc_o[dt][4 * j + 1] * inv),
                 cvt_pk_bf16(st.acc_o[dt][4 * j + 2] * inv, st.acc_o[dt][4 * j + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * j + 4 * hi) = w;
    }
  if (lse && hi == 0)
    lse[qrow0 + qloc] = (l_run > 0.f) ? (st.m_ref * kLn2 + logf(l_run)) : -INFINITY;
}

// ------------------------------------------------------------------ plain kernel (fp32)
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_plain_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int B, int Hq,
    int Hkv, int S, int block, const int32_t* __restrict__ blk_idx,
    const int32_t* __restrict__ blk_cnt, int max_sel, int causal, float scale, T* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int LPT = D / 8;
  constexpr int QPW = kWave / LPT;
  constexpr int QPG = QPW * 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int sub = lane % LPT;
  const int N = S / block;
  int b, h, I;
  prefill_work_item(blockIdx.x, gridDim.x, B, Hq, Hkv, N, b, h, I);
  const int g = h / (Hq / Hkv);
  const int64_t qrow0 = (static_cast<int64_t>(b) * Hq + h) * S;
  const int64_t kvrow0 = (static_cast<int64_t>(b) * Hkv + g) * S;
  const int64_t sel0 = (static_cast<int64_t>(b) * Hq + h) * N + I;
  const int cnt = blk_cnt[sel0];
  const int32_t* sel = blk_idx + sel0 * max_sel;

  for (int qb = 0; qb < block; qb += QPG) {
    const int qi = qb + wid * QPW + lane / LPT;
    const bool qvalid = qi < block;
    const int t = I * block + (qvalid ? qi : 0);
    float qv[8];
    Elem<T>::load8(q + (qrow0 + t) * D + sub * 8, qv);
    float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.f;
    for (int si = 0; si < cnt; ++si) {
      const int J = sel[si];
      if (J < 0 || J >= N || (causal && J > I)) continue;
      for (int kk = 0; kk < block; ++kk) {
        const int s = J * block + kk;
        float kv[8], vv[8];
        Elem<T>::load8(k + (kvrow0 + s) * D + sub * 8, kv);
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) dot = fmaf(qv[j], kv[j], dot);
#pragma unroll
        for (int off = LPT / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, kWave);
        const bool vis = qvalid && (!causal || s <= t);
        if (vis) {
          const float x = dot * scale;
          const float mn = fmaxf(m, x);
          const float a = (m == -INFINITY) ? 0.f : expf(m - mn);
          const float p = expf(x - mn);
          Elem<T>::load8(v + (kvrow0 + s) * D + sub * 8, vv);
          l = l * a + p;
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] = o[j] * a + p * vv[j];
          m = mn;
        }
      }
    }
    if (qvalid) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = o[j] * inv;
      Elem<T>::store8(out + (qrow0 + t) * D + sub * 8, r);
      if (lse && sub == 0) lse[qrow0 + t] = l > 0.f ? m + logf(l) : -INFINITY;
    }
  }
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, int dtype, int B, int Hq,
                          int Hkv, int S, int d, int block, const int32_t* blk_idx,
                          const int32_t* blk_cnt, int max_sel, int causal, float scale,
                          void* out, float* lse, hipStream_t st) {
  const int N = S / block;
  const dim3 grid(static_cast<unsigned>(B * Hq * N));
  if (dtype == kBF16 && (block == 64 || block == 128)) {
    const auto* qq = static_cast<const uint16_t*>(q);
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    auto* oo = static_cast<uint16_t*>(out);
#define SA_PF(D, BS)                                                                           \
  prefill_mfma_kernel<D, BS><<<grid, BS * 2, 0, st>>>(qq, kk, vv, B, Hq, Hkv, S, blk_idx, blk_cnt, \
                                                      max_sel, causal, scale, oo, lse)
    if (d == 128) { if (block == 128) SA_PF(128, 128); else SA_PF(128, 64); }
    else { if (block == 128) SA_PF(64, 128); else SA_PF(64, 64); }
#undef SA_PF
  } else if (dtype == kBF16) {
    if (d == 128)
      prefill_plain_kernel<uint16_t, 128><<<grid, 256, 0, st>>>(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
          B, Hq, Hkv, S, block, blk_idx, blk_cnt, max_sel, causal, scale, static_cast<uint16_t*>(out), lse);
    else
      prefill_plain_kernel<uint16_t, 64><<<grid, 256, 0, st>>>(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
          B, Hq, Hkv, S, block, blk_idx, blk_cnt, max_sel, causal, scale, static_cast<uint16_t*>(out), lse);
  } else {
    if (d == 128)
      prefill_plain_kernel<float, 128><<<grid, 256, 0, st>>>(
          static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
          B, Hq, Hkv, S, block, blk_idx, blk_cnt, max_sel, causal, scale, static_cast<float*>(out), lse);
    else
      prefill_plain_kernel<float, 64><<<grid, 256, 0, st>>>(
          static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
          B, Hq, Hkv, S, block, blk_idx, blk_cnt, max_sel, causal, scale, static_cast<float*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace sa

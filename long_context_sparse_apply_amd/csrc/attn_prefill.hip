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
template <int D, int BS>
__global__ __launch_bounds__(BS * 2) void prefill_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int B, int Hq, int Hkv, int S, const int32_t* __restrict__ blk_idx,
    const int32_t* __restrict__ blk_cnt, int max_sel, int causal, float scale,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int NT = BS * 2;          // threads: one wave per 32 queries
  constexpr int KS = D / 16;          // k-steps of the QK^T product
  constexpr int KT = BS / 32;         // 32-key tiles per block
  constexpr int DT = D / 32;          // 32-wide d tiles of the output
  constexpr int KROW = D + 8;         // LDS row pitch of K (bf16), padded
  constexpr int VROW = BS + 8;        // LDS row pitch of V^T (bf16), padded
  __shared__ __attribute__((aligned(16))) uint16_t sK[BS * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int N = S / BS;
  int b, h, I;
  prefill_work_item(blockIdx.x, gridDim.x, B, Hq, Hkv, N, b, h, I);
  const int g = h / (Hq / Hkv);
  const int64_t qrow0 = (static_cast<int64_t>(b) * Hq + h) * S + static_cast<int64_t>(I) * BS;
  const int64_t kvrow0 = (static_cast<int64_t>(b) * Hkv + g) * S;
  const int64_t sel0 = ((static_cast<int64_t>(b) * Hq + h) * N + I);
  const int cnt = blk_cnt[sel0];
  const int32_t* sel = blk_idx + sel0 * max_sel;

  // Q^T fragments: this lane's query (row wid*32 + l32) and 8 channels per k-step
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

  f32x16 acc_o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;
  float m_run = -INFINITY;  // running max (base-2 units) of this lane's query
  float l_run = 0.f;

  for (int si = 0; si < cnt; ++si) {
    const int J = sel[si];
    if (J < 0 || J >= N || (causal && J > I)) continue;  // uniform across the work-group
    __syncthreads();  // previous block's LDS reads are done
    // stage K rows (16-byte chunks) and V transposed (4 keys x 8 channels per chunk)
    {
      const uint16_t* kp = k + (kvrow0 + static_cast<int64_t>(J) * BS) * D;
      constexpr int KCH = BS * D / 8;
#pragma unroll
      for (int c = tid; c < KCH; c += NT) {
        const int row = c / (D / 8), col8 = c % (D / 8);
        const uint4 w = *reinterpret_cast<const uint4*>(kp + static_cast<int64_t>(row) * D + col8 * 8);
        *reinterpret_cast<uint4*>(&sK[row * KROW + col8 * 8]) = w;
      }
      const uint16_t* vp = v + (kvrow0 + static_cast<int64_t>(J) * BS) * D;
      constexpr int VCH = (BS / 4) * (D / 8);
#pragma unroll
      for (int c = tid; c < VCH; c += NT) {
        const int col8 = c % (D / 8), kq = c / (D / 8);
        uint4 w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          w[r] = *reinterpret_cast<const uint4*>(vp + static_cast<int64_t>(kq * 4 + r) * D + col8 * 8);
        // element e of row r: channel col8*8 + e, key kq*4 + r
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t vals[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t word = (e < 2) ? w[r].x : (e < 4) ? w[r].y : (e < 6) ? w[r].z : w[r].w;
            vals[r] = (e & 1) ? (word >> 16) : (word & 0xffffu);
          }
          u32x2 pk = {vals[0] | (vals[1] << 16), vals[2] | (vals[3] << 16)};
          *reinterpret_cast<u32x2*>(&sV[(col8 * 8 + e) * VROW + kq * 4]) = pk;
        }
      }
    }
    __syncthreads();

    // S^T = K Q^T for the block: KT tiles of 32 keys x 32 queries
    f32x16 sacc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint4 w = *reinterpret_cast<const uint4*>(&sK[(kt * 32 + l32) * KROW + 16 * s + 8 * hi]);
        u32x4 t = {w.x, w.y, w.z, w.w};
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, t), qf[s],
                                                            sacc[kt], 0, 0, 0);
      }
    }
    // scale to base-2 units, causal mask on the diagonal block, block max
    const bool diag = causal && (J == I);
    float mblk = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        float x = sacc[kt][r] * sl2;
        if (diag && key > qloc) x = -INFINITY;
        sacc[kt][r] = x;
        mblk = fmaxf(mblk, x);
      }
    mblk = fmaxf(mblk, __shfl_xor(mblk, 32, 64));
    const float m_new = fmaxf(m_run, mblk);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);  // m_run = -inf -> 0
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sacc[kt][r] - m_use);
        sacc[kt][r] = p;
        psum += p;
      }
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[dt][r] *= alpha;

    // O^T += V^T P^T, 16 keys per k-step
#pragma unroll
    for (int s = 0; s < BS / 16; ++s) {
      const int kt = s >> 1, u = s & 1;
      // P^T k-slots 0-3 hold keys 16s + 4hi + i (registers 8u + i) and slots 4-7 keys
      // 16s + 8 + 4hi + i (registers 8u + 4 + i): registers 8u .. 8u + 7 in order
      u32x4 pw;
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = pack_bf16(sacc[kt][8 * u + 2 * i], sacc[kt][8 * u + 2 * i + 1]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* vr = &sV[(dt * 32 + l32) * VROW + 16 * s + 4 * hi];
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(vr + 8);
        u32x4 vw = {v0[0], v0[1], v1[0], v1[1]};
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pf,
                                                             acc_o[dt], 0, 0, 0);
      }
    }
  }

  // normalise and store: lane holds query qloc, channels dt*32 + 8j + 4hi + i
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  uint16_t* op = out + (qrow0 + qloc) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 w = {pack_bf16(acc_o[dt][4 * j + 0] * inv, acc_o[dt][4 * j + 1] * inv),
                 pack_bf16(acc_o[dt][4 * j + 2] * inv, acc_o[dt][4 * j + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * j + 4 * hi) = w;
    }
  if (lse && hi == 0)
    lse[qrow0 + qloc] = (l_run > 0.f) ? (m_run * kLn2 + logf(l_run)) : -INFINITY;
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

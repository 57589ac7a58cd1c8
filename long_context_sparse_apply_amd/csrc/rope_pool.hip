// Rotary position encoding, and the fused pass that rotates Q and K and
// pools them into calibrated dual-band block vectors.
//
// "Prism: Spectral-Aware Block-Sparse Attention", sec. 1 (mean-pooled block
// importance), sec. 3 item 1 (high- and low-frequency bands pooled apart) and
// sec. 3 item 2 (temperature from the RMS energy density); "FASA:
// Frequency-aware Sparse Attention", sec. 2.A (RoPE frequency chunks).
//
// Data layout: x[B, H, S, d] row-major.  A thread owns 8 consecutive rotary
// pairs of one token row: channels [8c, 8c+8) and their partners
// [P+8c, P+8c+8), read as two 16-byte (bf16) or 32-byte (fp32) accesses, so a
// wave reads whole 256-byte rows with full coalescing.
#include "sa_common.hpp"

#include <cmath>

namespace sa {


// ------------------------------------------------------------------ rotation only
template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(const T* __restrict__ x, T* __restrict__ out,
                                                   int H, int S, const int32_t* __restrict__ pos,
                                                   int pos0, int64_t rows, RopeFreq fr) {
  constexpr int P = D / 2;
  constexpr int CH = P / 8;  // threads per row
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = gid / CH;
  const int c = static_cast<int>(gid % CH);
  if (row >= rows) return;
  const int s = static_cast<int>(row % S);
  const int64_t b = row / (static_cast<int64_t>(H) * S);
  const int64_t p = pos ? static_cast<int64_t>(pos[b * S + s]) : static_cast<int64_t>(pos0) + s;
  const T* src = x + row * D;
  float a[8], bb[8];
  Elem<T>::load8(src + 8 * c, a);
  Elem<T>::load8(src + P + 8 * c, bb);
  // the 8 frequencies are read together, before the first rotation
  double fj[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) fj[j] = fr.f[8 * c + j];
  float ra[8], rb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float cs, sn;
    rot_cos_sin(p, fj[j], cs, sn);
    ra[j] = a[j] * cs - bb[j] * sn;
    rb[j] = bb[j] * cs + a[j] * sn;
  }
  T* dst = out + row * D;
  Elem<T>::store8(dst + 8 * c, ra);
  Elem<T>::store8(dst + P + 8 * c, rb);
}

hipError_t launch_rope(const void* x, void* out, int dtype, int B, int H, int S, int d,
                       const int32_t* pos, int pos0, const RopeFreq& fr, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(B) * H * S;
  const int CH = d / 16;
  const int64_t threads = rows * CH;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (dtype == kBF16) {
    if (d == 128)
      rope_kernel<uint16_t, 128><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x),
                                                       static_cast<uint16_t*>(out), H, S, pos, pos0, rows, fr);
    else
      rope_kernel<uint16_t, 64><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x),
                                                      static_cast<uint16_t*>(out), H, S, pos, pos0, rows, fr);
  } else {
    if (d == 128)
      rope_kernel<float, 128><<<grid, 256, 0, st>>>(static_cast<const float*>(x),
                                                    static_cast<float*>(out), H, S, pos, pos0, rows, fr);
    else
      rope_kernel<float, 64><<<grid, 256, 0, st>>>(static_cast<const float*>(x),
                                                   static_cast<float*>(out), H, S, pos, pos0, rows, fr);
  }
  return hipGetLastError();
}

// Store 8 rotated elements with the nontemporal hint: the rotated rows are
// written once here and read back only by a later kernel, so they stream past
// the caches instead of displacing the rows still being read.
template <typename T> __device__ __forceinline__ void stream_store8(T* p, const float* v);
template <> __device__ __forceinline__ void stream_store8<uint16_t>(uint16_t* p, const float* v) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t a = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                     pack_bf16(v[6], v[7])};
  __builtin_nontemporal_store(a, reinterpret_cast<u32x4_t*>(p));
}
template <> __device__ __forceinline__ void stream_store8<float>(float* p, const float* v) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const f32x4_t a = {v[0], v[1], v[2], v[3]};
  const f32x4_t b = {v[4], v[5], v[6], v[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(p + 4));
}

// ------------------------------------------------------------------ rotation + pooling
// One work-group per (batch b, query block I, KV group g).  It walks the
// group's head rows -- KV head g, then its Hq/Hkv query heads -- over the
// block's `block` tokens, so the cos/sin of the block's (position, pair)
// grid are computed once and kept in registers for all of them.
//
// Per head row it rotates every token (fp32), optionally stores the rotated
// row, sums the rotated channels and the per-band squared norms, then forms
//   m = sum / block,  e_tok = sqrt(E_band / (block |band|)),
//   e_pool = sqrt(|m_band|^2 / |band|),  pooled = m * e_tok / e_pool.
// The sums use the fp32 rotated values before any bf16 rounding.  Stored
// query rows are multiplied by q_scale first (the pooled vectors are not).
//
// NT threads (256 or 512); a thread owns 8 rotary pairs of MAXR rows, RP =
// NT / (D/16) rows apart.  Head row 0's loads are issued before the cos/sin
// grid is computed, and head row hr+1's loads as soon as head row hr's have
// been taken into registers, so a wave always has a head row in flight.  The reduction takes
// two barriers per head row: the row-group partial sums go to LDS column-major
// (conflict-free both ways), LPC = NT / D adjacent lanes then sum one column
// (16 partials each) and combine by lane shuffles; the band sums of the
// energies and of the squared means go through small per-wave arrays that
// alternate between head rows, so the next head row's writes never meet this
// one's reads.
template <typename T, int D, int NT, int MAXR>
__global__ __launch_bounds__(NT) void rope_pool_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int Hq, int Hkv, int S, int block,
    int split, int calibrate, RopeFreq fr, T* __restrict__ q_rope, float q_scale,
    T* __restrict__ k_rope, float* __restrict__ pq, float* __restrict__ pk) {
  constexpr int P = D / 2;
  constexpr int CH = P / 8;     // threads per token row
  constexpr int RP = NT / CH;   // rows per pass
  constexpr int NW = NT / kWave;
  constexpr int LPC = NT / D;   // lanes per column in the column reduction
  constexpr int RPL = RP / LPC; // row-group partials each of them sums
  static_assert(RPL * LPC == RP && (LPC & (LPC - 1)) == 0 && LPC <= kWave, "reduction shape");
  const int tid = threadIdx.x;
  const int c = tid % CH;
  const int r0 = tid / CH;
  const int N = S / block;
  const int I = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int grp = Hq / Hkv;
  const int wid = tid / kWave;

  __shared__ float s_colT[D][RP + 1];   // [channel][row group]
  __shared__ float s_red[2][4][NW];     // [head parity][e_hi, e_lo, m2_hi, m2_lo][wave]

  // the block's rows of head row hr (KV head first, then the group's query heads)
  auto head_src = [&](int hr) {
    const bool is_k = (hr == 0);
    const int h = is_k ? g : g * grp + (hr - 1);
    const int H = is_k ? Hkv : Hq;
    return (is_k ? k : q) + ((static_cast<int64_t>(b) * H + h) * S + static_cast<int64_t>(I) * block) * D;
  };
  // this thread's raw elements of one head row, loaded one head row ahead
  using Raw = typename Elem<T>::Raw;
  Raw nxt_a[MAXR], nxt_b[MAXR];
  auto load_head = [&](int hr) {
    const T* src = head_src(hr);
#pragma unroll
    for (int ri = 0; ri < MAXR; ++ri) {
      const int r = r0 + ri * RP;
      if (r < block) {
        nxt_a[ri] = Elem<T>::load_raw8(src + static_cast<int64_t>(r) * D + 8 * c);
        nxt_b[ri] = Elem<T>::load_raw8(src + static_cast<int64_t>(r) * D + P + 8 * c);
      } else {
        nxt_a[ri] = Elem<T>::zero_raw8();
        nxt_b[ri] = Elem<T>::zero_raw8();
      }
    }
  };
  load_head(0);

  // cos / sin of this thread's (row, pair) grid (rows past the block are
  // computed too and never used); the 8 frequencies are read once, together
  double fj[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) fj[j] = fr.f[8 * c + j];
  float cs[MAXR][8], sn[MAXR][8];
#pragma unroll
  for (int ri = 0; ri < MAXR; ++ri) {
    const int64_t p = static_cast<int64_t>(I) * block + r0 + ri * RP;
#pragma unroll
    for (int j = 0; j < 8; ++j) rot_cos_sin(p, fj[j], cs[ri][j], sn[ri][j]);
  }

  // barrier for the LDS reductions only: waits for this wave's LDS accesses,
  // not for its global loads (the next head's rows stay in flight)
  auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  // column reduced by this lane, and its share of the row-group partials
  const int rcol = tid / LPC;
  const int rpart = tid % LPC;
  const bool rhi = (rcol % P) < split;
  const float inv_block = 1.f / static_cast<float>(block);

  for (int hr = 0; hr <= grp; ++hr) {
    const bool is_k = (hr == 0);
    const int h = is_k ? g : g * grp + (hr - 1);
    const int H = is_k ? Hkv : Hq;
    const int par = hr & 1;
    T* dst = is_k ? k_rope : q_rope;
    const float osc = is_k ? 1.f : q_scale;
    if (dst) dst += ((static_cast<int64_t>(b) * H + h) * S + static_cast<int64_t>(I) * block) * D;
    float* pool_out = (is_k ? pk : pq) + ((static_cast<int64_t>(b) * H + h) * N + I) * D;
    Raw cur_a[MAXR], cur_b[MAXR];
#pragma unroll
    for (int ri = 0; ri < MAXR; ++ri) { cur_a[ri] = nxt_a[ri]; cur_b[ri] = nxt_b[ri]; }
    if (hr < grp) load_head(hr + 1);

    float col[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) col[j] = 0.f;
    float e_hi = 0.f, e_lo = 0.f;
#pragma unroll
    for (int ri = 0; ri < MAXR; ++ri) {
      const int r = r0 + ri * RP;
      if (r < block) {
        float a[8], bb[8], ra[8], rb[8];
        Elem<T>::unpack8(cur_a[ri], a);
        Elem<T>::unpack8(cur_b[ri], bb);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          ra[j] = a[j] * cs[ri][j] - bb[j] * sn[ri][j];
          rb[j] = bb[j] * cs[ri][j] + a[j] * sn[ri][j];
          col[j] += ra[j];
          col[8 + j] += rb[j];
          const float e = ra[j] * ra[j] + rb[j] * rb[j];
          if (8 * c + j < split) e_hi += e; else e_lo += e;
        }
        if (dst) {
          float oa[8], ob[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) { oa[j] = ra[j] * osc; ob[j] = rb[j] * osc; }
          stream_store8<T>(dst + static_cast<int64_t>(r) * D + 8 * c, oa);
          stream_store8<T>(dst + static_cast<int64_t>(r) * D + P + 8 * c, ob);
        }
      }
    }
    // row-group partials of the column sums, and the per-wave band energies
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s_colT[8 * c + j][r0] = col[j];
      s_colT[P + 8 * c + j][r0] = col[8 + j];
    }
    e_hi = wave_sum(e_hi);
    e_lo = wave_sum(e_lo);
    if ((tid & (kWave - 1)) == 0) {
      s_red[par][0][wid] = e_hi;
      s_red[par][1][wid] = e_lo;
    }
    lds_barrier();
    // column mean: LPC adjacent lanes sum RPL partials each, then combine
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) sum += s_colT[rcol][rpart * RPL + i];
#pragma unroll
    for (int o = 1; o < LPC; o <<= 1) sum += __shfl_xor(sum, o, kWave);
    const float m = sum * inv_block;
    // band sums of the squared means (one lane per column contributes)
    float m2_hi = (rpart == 0 && rhi) ? m * m : 0.f;
    float m2_lo = (rpart == 0 && !rhi) ? m * m : 0.f;
    m2_hi = wave_sum(m2_hi);
    m2_lo = wave_sum(m2_lo);
    if ((tid & (kWave - 1)) == 0) {
      s_red[par][2][wid] = m2_hi;
      s_red[par][3][wid] = m2_lo;
    }
    lds_barrier();
    if (rpart == 0) {
      const int band = rhi ? 0 : 1;
      float e = 0.f, m2 = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        e += s_red[par][band][w];
        m2 += s_red[par][2 + band][w];
      }
      const int nch = 2 * (band == 0 ? split : P - split);
      float fac = 1.f;
      if (calibrate) {
        if (nch == 0 || m2 <= 0.f) {
          fac = 0.f;
        } else {
          const float e_tok = sqrtf(e / (static_cast<float>(block) * nch));
          const float e_pool = sqrtf(m2 / nch);
          fac = e_tok / e_pool;
        }
      }
      pool_out[rcol] = m * fac;
    }
  }
}

hipError_t launch_rope_pool(const void* q, const void* k, int dtype, int B, int Hq, int Hkv, int S,
                            int d, int block, int split, int calibrate, const RopeFreq& fr,
                            void* q_rope, float q_scale, void* k_rope, float* pq, float* pk,
                            hipStream_t st) {
  const dim3 grid(S / block, Hkv, B);
  const int CH = d / 16;
  // 512 threads when the block fills them (block * CH >= 512), else 256
  const int nt = block * CH >= 512 ? 512 : 256;
  const int RP = nt / CH;
  const int rows_per_thread = (block + RP - 1) / RP;
#define SA_RP_LAUNCH(T, D, NT, R)                                                                 \
  rope_pool_kernel<T, D, NT, R><<<grid, NT, 0, st>>>(                                             \
      static_cast<const T*>(q), static_cast<const T*>(k), Hq, Hkv, S, block, split, calibrate, fr, \
      static_cast<T*>(q_rope), q_scale, static_cast<T*>(k_rope), pq, pk)
#define SA_RP_R(T, D)                                   \
  if (nt == 256) SA_RP_LAUNCH(T, D, 256, 1);            \
  else if (rows_per_thread <= 1) SA_RP_LAUNCH(T, D, 512, 1); \
  else if (rows_per_thread <= 2) SA_RP_LAUNCH(T, D, 512, 2); \
  else SA_RP_LAUNCH(T, D, 512, 4);
  if (dtype == kBF16) {
    if (d == 128) { SA_RP_R(uint16_t, 128) } else { SA_RP_R(uint16_t, 64) }
  } else {
    if (d == 128) { SA_RP_R(float, 128) } else { SA_RP_R(float, 64) }
  }
#undef SA_RP_R
#undef SA_RP_LAUNCH
  return hipGetLastError();
}

}  // namespace sa

// Block-sparse prefill attention over the selected key blocks.
//
// "Prism: Spectral-Aware Block-Sparse Attention", sec. 1: attention is
// computed only for a subset of relevant key blocks.  For a query at position
// t in query block I of head h, the keys are those of the blocks listed for
// (h, I); with the causal mask only keys s <= t count.  K/V come from KV head
// h / (Hq/Hkv).
//
// bf16 path (d in {64, 128}, block in {64, 128}): one work-group per
// (b, h, I) with one wave per 32 queries.  The selected key blocks are walked
// as 64-key chunks staged in LDS (K and V both row-major, swizzled) by
// direct-to-LDS loads.  Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in registers for the
// whole block list), so the C layout leaves one query per lane column and 16
// keys per lane.  The online softmax (fp32, base-2 exponent with the scale
// folded in) runs on those registers; the probabilities are rounded to bf16
// and used directly as the B operand of O^T += V^T P^T (the k-slot order of
// P^T matches the C layout of S^T; V^T comes from LDS transpose reads in the
// same key order), so P never leaves registers.
//
// Work order: large query blocks first (their lists are the longest) and all
// work of one KV group placed on one XCD when the grid divides evenly, so the
// four query heads that read the same K/V blocks share that XCD's L2.
//
// fp32 path: a plain kernel, one query per LPT = d/8 lanes, online softmax
// over the selected keys in order, fp32 throughout.
#include <cmath>

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
// chunk c of row r sits at chunk position c ^ sw(r).  With r = 4b + a
// (a, b in 0..3, bits a0 a1 b0 b1), sw(r) has bits
//   bit 0 = b0, bit 1 = a0 ^ b1, bit 2 = a1, bit 3 = a0   (bit 3 only when D = 128)
// It depends on r mod 16 only, so rows 16 and 32 further on use the same
// pattern.  It makes both read patterns conflict-free whether the LDS serves
// 128 or 256 bytes a cycle:
//  - a K operand read (16 bytes a lane, rows r..r+7 or r..r+15 at one chunk,
//    r aligned) hits distinct 16-byte bank groups, since sw is one-to-one on
//    (a0, a1, b0) and, for 16 rows, on r mod 16 (D = 128) or on the 8 rows of
//    one parity (D = 64, two rows per 256 bytes);
//  - a V transpose read (8 bytes a lane, 4 aligned rows x 2 or 4 adjacent
//    chunks) does too, since bits 1-2 and bits 2-3 of sw are one-to-one on
//    (a0, a1).
// Tiles are filled by direct-to-LDS loads (buffer_load_dwordx4 ... lds): one
// wave instruction writes 1 KB of consecutive LDS bytes, lane i its 16 bytes
// at offset 16 i, and each lane fetches the global chunk that belongs there.
// The buffer form, not the global one: while a global-form load to LDS is in
// flight the compiler waits for every outstanding LDS read before each use,
// which would undo the operand reads the step plan issues ahead.
template <int D, int ROWS, int NW>
struct LdsTile {
  static constexpr int ROWB = D * 2;                 // bytes per row
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int LPW = BYTES / 1024 / NW;      // load instructions per wave per tile
  static_assert(LPW * NW * 1024 == BYTES, "tile must split evenly over the waves");
  static_assert(CPR == 8 || CPR == 16, "the swizzle is laid out for D = 64 or 128");

  static __device__ __forceinline__ int sw(int row) {
    const int a0 = row & 1, a1 = (row >> 1) & 1, b0 = (row >> 2) & 1, b1 = (row >> 3) & 1;
    return (b0 | ((a0 ^ b1) << 1) | (a1 << 2) | (a0 << 3)) & (CPR - 1);
  }
  static __device__ __forceinline__ int phys(int row, int chunk) {
    return row * ROWB + ((chunk ^ sw(row)) << 4);
  }
  // issue this wave's share of the tile's direct-to-LDS loads (asynchronous)
  static __device__ __forceinline__ void issue(const uint16_t* g, uint8_t* lds, int wid, int lane) {
    const auto rsrc = buffer_rsrc(g, BYTES);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int ins = wid * LPW + j;
      const int off = ins * 1024 + lane * 16;
      const int row = off / ROWB;
      const int pos = (off % ROWB) >> 4;
      const int chunk = pos ^ sw(row);
      lds_dma16_buf(rsrc, row * ROWB + chunk * 16, lds + ins * 1024);
    }
  }
};

// Pointer to uniform, read-only data in the constant address space (its loads
// are scalar).
typedef const __attribute__((address_space(4))) int32_t* uniform_i32p;

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

// Maximum of two scores.  Scores are never NaN, so the NaN-propagating
// maximum (v_maximum3_f32 on this target) gives the same value as fmaxf
// without fmaxf's canonicalising of every MFMA result first.
__device__ __forceinline__ float max_nn(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Max / sum of a value over lanes l and l ^ 32 (the two key halves of a
// query) with v_permlane32_swap, which trades the wave's 32-lane halves
// without an LDS round trip: for lane l < 32 the pair is (x[l], x[l + 32]),
// for lane l >= 32 it is (x[l - 32], x[l]).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Per-lane LDS byte offsets of a wave's reads of a 64-key tile.  The swizzle
// repeats every 16 rows, so one offset per (k-step) for K and per (d-tile,
// half) for V covers every read; rows 32 (K) and 16 (V) further on are fixed
// byte distances away and go into the instructions' immediate offsets.
template <int D>
struct ChunkOffsets {
  int k[D / 16];      // K row l32, 16-byte chunk 2s + hi
  int v[D / 32][2];   // V row 4(G/2) + i/4 (+8), channels dt*32 + (G%2)*16 + 4(i%4)
  __device__ __forceinline__ void init(int l32, int hi, int grp16, int i16) {
    using Tile = LdsTile<D, 64, 1>;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) k[s] = Tile::phys(l32, 2 * s + hi);
    const int vrow = 4 * (grp16 >> 1) + (i16 >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int col = dt * 32 + (grp16 & 1) * 16 + 4 * (i16 & 3);
      v[dt][0] = Tile::phys(vrow, col >> 3) + (col & 7) * 2;
      v[dt][1] = Tile::phys(vrow + 8, col >> 3) + (col & 7) * 2;
    }
  }
  // an empty asm that claims to rewrite the offsets: address arithmetic that
  // uses them cannot be hoisted out of the caller's loop, so each read keeps
  // the form offset-register + immediate instead of a register per address
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) asm volatile("" : "+v"(k[s]));
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) asm volatile("" : "+v"(v[dt][0]), "+v"(v[dt][1]));
  }
};

// S^T = K Q^T for one 64-key chunk (K tile kbuf): two 32-key tiles, D/16
// k-steps each.
template <int D>
__device__ __forceinline__ void chunk_scores(const uint8_t* kbuf, const ChunkOffsets<D>& off,
                                             const bf16x8 (&qf)[D / 16], f32x16 (&sacc)[2]) {
  constexpr int ROWB = 2 * D;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint4 w = *reinterpret_cast<const uint4*>(kbuf + off.k[s] + kt * 32 * ROWB);
      u32x4 t = {w.x, w.y, w.z, w.w};
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, t), qf[s],
                                                          sacc[kt], 0, 0, 0);
    }
}

// Causal mask of a chunk of the diagonal block: key > query is dropped.
__device__ __forceinline__ void chunk_mask(f32x16 (&sacc)[2], int key0, int qloc, int hi) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0 + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3) > qloc) sacc[kt][r] = -INFINITY;
}

// Chunk max (base 2) of this lane's query, over both key halves.
__device__ __forceinline__ float chunk_maxval(const f32x16 (&sacc)[2], float sl2) {
  float mblk = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mblk = max_nn(mblk, sacc[kt][r]);
  return pair_max(mblk) * sl2;
}

// Lazy rescale: when a chunk's max exceeds the reference by more than 8 (base
// 2), O and l move to the new reference, so every p = 2^(x - m_ref) <= 2^8.
template <int DT>
__device__ __forceinline__ void chunk_rescale(SoftmaxState<DT>& st, float mblk, bool valid) {
  constexpr float kRescale = 8.f;
  const bool raise = valid && mblk > st.m_ref + kRescale;
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
}

// Unit mode (q pre-multiplied by sm_scale * log2 e, so scores are base-2
// exponents): the S MFMAs start from -m_ref, so the scores come out relative
// to the reference and p = 2^s needs no further instruction.  The reference
// lives on the grid of multiples of 64 and moves only when a chunk's max
// (relative) exceeds 64: then O and l scale by an exact power of two, the
// pending scores and the -m_ref tile shift by the same multiple of 64, and
// every p stays <= 2^64 (fp32 and bf16 keep their relative precision).  For
// ordinary logits the reference stays 0.
__device__ __forceinline__ float grid64(float m) { return 64.f * rintf(m * (1.f / 64.f)); }

template <int DT>
__device__ __forceinline__ void chunk_rescale_unit(SoftmaxState<DT>& st, float mrel, bool valid,
                                                   f32x16 (&snext)[2], f32x16& negm) {
  const bool raise = valid && mrel > 64.f;
  if (__ballot(raise)) {
    const float delta = raise ? grid64(mrel) : 0.f;
    const float alpha = ldexpf(1.f, -static_cast<int>(delta));  // exact power of two
    st.l_part *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc_o[dt][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      snext[0][r] -= delta;
      snext[1][r] -= delta;
      negm[r] -= delta;
    }
    st.m_ref += delta;
  }
}

// Slot plan of one pipelined step (NS = 2 D/16 S MFMAs, NP = 4 D/32 P V
// MFMAs, NT = NS + NP slots, one MFMA per slot):
//   S(c + 1) keys 0-31 | P V k-steps 0, 1 | S(c + 1) keys 32-63 | P V k-steps 2, 3
// MFMAs that accumulate into the same registers run back to back where they
// can (the matrix unit issues such a chain faster than it switches between
// accumulators): each S half is one chain over the D/16 k-steps, and each P V
// half goes d-tile by d-tile with its two k-steps together.  The vector work
// is spread over the slots: P words 0-7 (k-steps 0, 1) over the first S half,
// words 8-15 over the next S1 slots, each before the first P V MFMA that
// reads it; the max of the 16 scores of S(c + 1) key half kt (two per unit)
// follows two slots after that half's last S MFMA.
template <int D>
struct StepPlan {
  static constexpr int DT = D / 32;
  static constexpr int NS = 2 * (D / 16);
  static constexpr int NP = 4 * DT;
  static constexpr int NT = NS + NP;
  static constexpr int S1 = NS / 2 + NP / 2;   // first slot of the second S half
  static constexpr int PFD = 2;                // LDS operand reads run this many slots ahead
  static constexpr bool is_s(int j) { return j < NS / 2 || (j >= S1 && j < S1 + NS / 2); }
  static constexpr int s_kt(int j) { return j < NS / 2 ? 0 : 1; }
  static constexpr int s_step(int j) { return j < NS / 2 ? j : j - S1; }
  static constexpr int pv_local(int j) { return j < S1 ? j - NS / 2 : j - NS; }
  static constexpr int pv_s(int j) { return 2 * (pv_local(j) / (NP / 2)) + pv_local(j) % 2; }
  static constexpr int pv_dt(int j) { return (pv_local(j) % (NP / 2)) / 2; }
  static constexpr int word_slot(int u) { return u < 8 ? u * (NS / 2) / 8 : NS / 2 + (u - 8) * S1 / 8; }
  static constexpr int max_slot(int kt, int m) {
    const int start = kt == 0 ? NS / 2 + 1 : S1 + NS / 2 + 1;
    return start + m * (NT - start) / 8;
  }
};

// One pipelined step of a wave, written slot by slot: each slot issues the
// LDS reads of the MFMA PFD slots ahead, its MFMA, and its share of the vector
// work; a scheduling fence after each slot keeps that order, so the matrix
// unit runs while the vector unit works.  P word u is p = 2^(x sl2 - m) for
// two keys, packed to bf16 for the P V MFMA; the denominator sums the fp32
// values.  Returns the max (base 2) of S(c + 1) for this lane's query,
// before any causal mask (the caller masks a diagonal chunk and takes its max
// again).
template <int D, bool UNIT>
__device__ __forceinline__ float chunk_step(const uint8_t* kbuf, const uint8_t* vbuf,
                                            const ChunkOffsets<D>& off, const bf16x8 (&qf)[D / 16],
                                            const f32x16 (&sacc)[2], f32x16 (&snext)[2],
                                            SoftmaxState<D / 32>& st, float sl2,
                                            const f32x16& negm) {
  using Plan = StepPlan<D>;
  constexpr int ROWB = 2 * D;
  constexpr int DT = Plan::DT, NT = Plan::NT;
  const float neg_m = (st.m_ref == -INFINITY) ? 0.f : -st.m_ref;
  u32x4 pw[4];
  float lsum = st.l_part;
  float mx = -INFINITY;
  auto pword = [&](int u) {
    const int s = u >> 2, i = u & 3;
    const float x0 = sacc[s >> 1][8 * (s & 1) + 2 * i];
    const float x1 = sacc[s >> 1][8 * (s & 1) + 2 * i + 1];
    // unit mode: the scores already are the base-2 exponents (the S MFMAs
    // start from -m_ref)
    const float a0 = UNIT ? x0 : fmaf(x0, sl2, neg_m);
    const float a1 = UNIT ? x1 : fmaf(x1, sl2, neg_m);
    const float p0 = __builtin_amdgcn_exp2f(a0);
    const float p1 = __builtin_amdgcn_exp2f(a1);
    const uint32_t w = cvt_pk_bf16(p0, p1);
    pw[s][i] = w;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, lsum, false);
    asm volatile("" : "+v"(lsum));  // keep the sum in its slot (see max_unit)
  };
  // the empty asm keeps each unit in its slot: without it the compiler sinks
  // the whole max to the end of the step, behind the last MFMA
  auto max_unit = [&](int kt, int m) {
    mx = max_nn(mx, max_nn(snext[kt][2 * m], snext[kt][2 * m + 1]));
    asm volatile("" : "+v"(mx));
  };
  auto operand = [&](int j) {
    u32x4 t;
    if (Plan::is_s(j)) {
      const uint4 w = *reinterpret_cast<const uint4*>(kbuf + off.k[Plan::s_step(j)] +
                                                      Plan::s_kt(j) * 32 * ROWB);
      t = u32x4{w.x, w.y, w.z, w.w};
    } else {
      const int s = Plan::pv_s(j), dt = Plan::pv_dt(j);
      const u32x2 v0 = lds_read_tr(vbuf + off.v[dt][0] + 16 * s * ROWB);
      const u32x2 v1 = lds_read_tr(vbuf + off.v[dt][1] + 16 * s * ROWB);
      t = u32x4{v0[0], v0[1], v1[0], v1[1]};
    }
    return t;
  };

#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) snext[kt][r] = UNIT ? negm[r] : 0.f;
  constexpr int PFD = Plan::PFD;
  u32x4 op[NT];
#pragma unroll
  for (int j = 0; j < PFD; ++j) op[j] = operand(j);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (j + PFD < NT) op[j + PFD] = operand(j + PFD);
    if (Plan::is_s(j)) {
      const int kt = Plan::s_kt(j);
      snext[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, op[j]),
                                                           qf[Plan::s_step(j)], snext[kt], 0, 0, 0);
    } else {
      const int s = Plan::pv_s(j), dt = Plan::pv_dt(j);
      st.acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, op[j]), __builtin_bit_cast(bf16x8, pw[s]), st.acc_o[dt], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (Plan::word_slot(u) == j) pword(u);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int m = 0; m < 8; ++m)
        if (Plan::max_slot(kt, m) == j) max_unit(kt, m);
    __builtin_amdgcn_sched_barrier(0);
  }
  st.l_part = lsum;
  return UNIT ? pair_max(mx) : pair_max(mx) * sl2;
}

// The slot plan's promises, checked at compile time: every P word is ready
// before the first P V MFMA that reads it, and each max unit comes at least
// two slots after the last S MFMA of its key half and inside the step.
template <int D>
constexpr bool step_plan_ok() {
  using Plan = StepPlan<D>;
  for (int u = 0; u < 16; ++u) {
    const int s = u / 4;
    int first = -1;
    for (int j = 0; j < Plan::NT && first < 0; ++j)
      if (!Plan::is_s(j) && Plan::pv_s(j) == s) first = j;
    if (!(Plan::word_slot(u) < first)) return false;
  }
  for (int kt = 0; kt < 2; ++kt) {
    int last = -1;
    for (int j = 0; j < Plan::NT; ++j)
      if (Plan::is_s(j) && Plan::s_kt(j) == kt) last = j;
    for (int m = 0; m < 8; ++m)
      if (Plan::max_slot(kt, m) < last + 2 || Plan::max_slot(kt, m) >= Plan::NT) return false;
  }
  return true;
}
static_assert(step_plan_ok<64>() && step_plan_ok<128>(), "prefill step slot plan");

// One work-group per (b, h, I), one wave per 32 queries.  The selected key
// blocks are walked as 64-key chunks.  K runs one chunk ahead of V: while a
// wave exponentiates chunk c, it already computes S for chunk c + 1, so the
// matrix unit and the vector unit of a SIMD work at the same time.  LDS holds
// two K buffers and two V buffers; at the start of step c (one barrier: K(c+1)
// and V(c) have landed for every wave, and every wave is done with step c - 1)
// the work-group issues K(c+2) into the K buffer that held K(c) and V(c+1)
// into the V buffer that held V(c-1), asynchronously (direct-to-LDS), then
// runs the slot plan above: S(c+1) = K(c+1) Q^T and O += V(c)^T P(c)^T on the
// matrix unit, P(c) and the max of S(c+1) on the vector unit, followed by the
// causal mask of a diagonal chunk and the lazy rescale.  The loop is unrolled
// by two so each half names its buffers statically.
template <int D, int BS, bool UNIT>
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
  // four 64-key tiles.  Separate arrays, not one: the compiler then sees that
  // the direct-to-LDS loads into one buffer cannot alias the reads of another
  // and does not wait for them before the reads.
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[Tile::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[Tile::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[Tile::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[Tile::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index, in a scalar register: the tile loads' LDS bases derive
  // from it and then need no per-step move from a vector register
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // read through the constant address space: the reads are uniform and become
  // scalar loads, which the vector-load counter the tile waits use does not see
  // clamped to the list width: a count above it never reads past the row
  const int cnt = min(max(((uniform_i32p)blk_cnt)[sel0], 0), max_sel);
  const uniform_i32p sel = (uniform_i32p)(blk_idx + sel0 * max_sel);
  // the first entry is read beside the count, not after it (one scalar
  // round trip less before the first tile load)
  const int J0 = max_sel > 0 ? sel[0] : -1;
  auto usable = [&](int J) { return J >= 0 && J < N && !(causal && J > I); };
  // the first usable entry at or after `from` (cnt: none), its block in jj
  auto next_valid = [&](int from, int& jj) {
    for (int t = from; t < cnt; ++t) {
      const int j = sel[t];
      if (usable(j)) {
        jj = j;
        return t;
      }
    }
    jj = -1;
    return cnt;
  };
  // chunk cursor: list position t, chunk c within the block (t == cnt: none)
  // and the block's index jj, read from the list once per block, so a step
  // issues its tile loads without waiting for a scalar load of the list
  auto advance = [&](int& tt, int& cc, int& jj) {
    if (tt >= cnt) return;
    if (cc + 1 < CPB) { ++cc; } else { tt = next_valid(tt + 1, jj); cc = 0; }
  };
  auto chunk_row0 = [&](int jj, int cc) { return static_cast<int64_t>(jj) * BS + cc * 64; };

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
  // unit mode: q arrives pre-multiplied by sm_scale * log2(e), so the scores
  // are already exponents in base 2
  const float sl2 = UNIT ? 1.f : scale * kLog2e;
  SoftmaxState<DT> st;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc_o[dt][r] = 0.f;
  st.m_ref = -INFINITY;
  st.l_part = 0.f;

  // cursors: (t0, c0) = chunk c (scores in sacc), (t1, c1) = chunk c + 1, (t2, c2) = chunk c + 2
  int j0 = J0;
  int t0 = (cnt > 0 && usable(J0)) ? 0 : next_valid(1, j0), c0 = 0;
  int t1 = t0, c1 = 0, j1 = j0;
  advance(t1, c1, j1);
  int t2 = t1, c2 = c1, j2 = j1;
  advance(t2, c2, j2);

  ChunkOffsets<D> off;
  off.init(l32, hi, grp16, i16);
  f32x16 negm;  // unit mode: -m_ref in every slot, the S MFMAs' starting value
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = 0.f;
  f32x16 sacc[2];
  if (t0 < cnt) {
    // prologue: K(0) -> K0, K(1) -> K1 and V(0) -> V0 issued together; S(0)
    // waits for Q and K(0) only (the loads complete in order), so K(1) and
    // V(0) land while it is computed
    Tile::issue(kbase + chunk_row0(j0, c0) * D, sK0, wid, lane);
    if (t1 < cnt) Tile::issue(kbase + chunk_row0(j1, c1) * D, sK1, wid, lane);
    Tile::issue(vbase + chunk_row0(j0, c0) * D, sV0, wid, lane);
    if (t1 < cnt) wait_vmcnt<2 * Tile::LPW>();
    else wait_vmcnt<Tile::LPW>();
    __builtin_amdgcn_s_barrier();
    chunk_scores<D>(sK0, off, qf, sacc);
    if (causal && j0 == I) chunk_mask(sacc, c0 * 64, qloc, hi);
    // O and l are still zero: nothing to rescale
    st.m_ref = chunk_maxval(sacc, sl2);
    if (UNIT) {
      // reference on the 64-grid (0 when no key is visible: every p is then 0)
      st.m_ref = st.m_ref == -INFINITY ? 0.f : grid64(st.m_ref);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[0][r] -= st.m_ref;
        sacc[1][r] -= st.m_ref;
        negm[r] = -st.m_ref;
      }
    }
  }
  // One step: chunk c's P and P V with V in vread, chunk c + 1's S with K in
  // kread; K(c + 2) goes to kwrite, V(c + 1) to vwrite.  S(c + 1) is computed
  // even past the last chunk (stale but in-bounds LDS; its max is then
  // ignored) so that the step body is one straight-line region.
  auto step = [&](const uint8_t* kread, uint8_t* kwrite, const uint8_t* vread, uint8_t* vwrite) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (t2 < cnt) Tile::issue(kbase + chunk_row0(j2, c2) * D, kwrite, wid, lane);
    if (t1 < cnt) Tile::issue(vbase + chunk_row0(j1, c1) * D, vwrite, wid, lane);
    off.pin();
    const bool next = t1 < cnt;
    f32x16 snext[2];
    float mblk = chunk_step<D, UNIT>(kread, vread, off, qf, sacc, snext, st, sl2, negm);
    if (causal && next && j1 == I) {  // uniform: chunk c + 1 is on the diagonal
      chunk_mask(snext, c1 * 64, qloc, hi);
      mblk = chunk_maxval(snext, sl2);
    }
    if (UNIT) chunk_rescale_unit<DT>(st, mblk, next, snext, negm);
    else chunk_rescale<DT>(st, mblk, next);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) sacc[kt] = snext[kt];
    t0 = t1; c0 = c1;
    t1 = t2; c1 = c2; j1 = j2;
    advance(t2, c2, j2);
  };
  while (t0 < cnt) {
    step(sK1, sK0, sV0, sV1);  // c even: K(c+1) in K1, V(c) in V0
    if (t0 >= cnt) break;
    step(sK0, sK1, sV1, sV0);  // c odd
  }

  // normalise and store: lane holds query qloc, channels dt*32 + 8j + 4hi + i
  const float l_run = pair_sum(st.l_part);
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
  // read through the constant address space: the reads are uniform and become
  // scalar loads, which the vector-load counter the tile waits use does not see
  // clamped to the list width: a count above it never reads past the row
  const int cnt = min(max(((uniform_i32p)blk_cnt)[sel0], 0), max_sel);
  const uniform_i32p sel = (uniform_i32p)(blk_idx + sel0 * max_sel);

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
    // sm_scale = ln 2 (the float nearest): the logits are base-2 exponents as
    // they stand (the caller folded sm_scale * log2 e into q)
    const bool unit = scale == kLn2;
#define SA_PF(D, BS)                                                                               \
  do {                                                                                             \
    if (unit)                                                                                      \
      prefill_mfma_kernel<D, BS, true><<<grid, BS * 2, 0, st>>>(qq, kk, vv, B, Hq, Hkv, S, blk_idx, \
                                                                blk_cnt, max_sel, causal, scale,   \
                                                                oo, lse);                          \
    else                                                                                           \
      prefill_mfma_kernel<D, BS, false><<<grid, BS * 2, 0, st>>>(qq, kk, vv, B, Hq, Hkv, S,        \
                                                                 blk_idx, blk_cnt, max_sel, causal, \
                                                                 scale, oo, lse);                  \
  } while (0)
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

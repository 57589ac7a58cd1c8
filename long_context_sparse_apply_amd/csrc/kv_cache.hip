// Appending tokens to a decode KV cache: keys rotated at their absolute
// positions, in the standard layout, the dominant-slab layout (slab + rest)
// or the slab plus full rows, plus values.
//
// "FASA: Frequency-aware Sparse Attention", sec. 2.B item 2 (attention over
// the selected tokens keeps their original absolute positions, so the cache
// holds keys rotated at those positions) and sec. 2.C (the
// computation-optimised variant scores from a sparse subset of the key
// state: the dominant channels, kept together).
//
// One work-group per (row chunk, KV head, batch).  A thread owns 8 rotary
// pairs of one new token (channels [8c, 8c+8) and [P+8c, P+8c+8)), rotates
// them at position start[b] + s with the fp64-reduced angle.  In the
// standard layout it writes the 16 channels straight to the row of that
// position.  In the slab layout the work-group's rotated rows are staged in
// LDS; since consecutive new tokens land in consecutive cache rows, the
// work-group's part of each slab is one contiguous run, written with
// coalesced stores that gather channels through a slot -> channel table:
// slot j < n_dom holds D[j], slot n_dom + j holds D[j] + P, and the rest slab
// holds every other channel in ascending order.  With slab + full rows
// (layout 2) the whole rotated row also goes, in the standard channel order,
// to the full-row cache, which the attention gathers as aligned 256-byte rows.
// Values are copied unrotated.
#include "sa_common.hpp"

namespace sa {

template <typename T, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new, int Hkv, int S, int Lmax,
    const int32_t* __restrict__ start, RopeFreq fr, int slab, const int32_t* __restrict__ dom,
    int n_dom, T* __restrict__ k_out, T* __restrict__ k_rest, T* __restrict__ v_out) {
  constexpr int P = D / 2;
  constexpr int CH = P / 8;         // threads per token row
  constexpr int RPW = 256 / CH;     // rows per work-group
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int c = tid % CH;
  const int rl = tid / CH;
  const int r0 = blockIdx.x * RPW;
  const int r = r0 + rl;

  // rows of this work-group that land inside the cache: [r_lo, r_hi)
  const int64_t st = start[b];
  const int64_t r_lo = max(static_cast<int64_t>(r0), -st);
  const int64_t r_hi = min(min(static_cast<int64_t>(r0) + RPW, static_cast<int64_t>(S)),
                           static_cast<int64_t>(Lmax) - st);
  if (r_lo >= r_hi) return;  // uniform over the work-group: no barrier is skipped by part of it

  __shared__ int s_chan[D];                      // slab slot -> channel
  __shared__ unsigned long long s_dmask[(D + 63) / 64];
  __shared__ float s_rows[RPW][D];               // rotated rows (slab layout only)
  const int ndc = 2 * n_dom;
  const int nrest = D - ndc;
  if (slab) {
    int slot = -1;
    if (tid < D) {
      for (int j = 0; j < n_dom; ++j) {
        const int ch = dom[g * n_dom + j];
        if (tid == ch) slot = j;
        if (tid == ch + P) slot = n_dom + j;
      }
    }
    const bool isdom = slot >= 0;
    const unsigned long long m = __ballot(isdom);
    if (tid < D && lane == 0) s_dmask[wid] = m;
    __syncthreads();
    if (tid < D) {
      if (!isdom) {
        int below = __popcll(~s_dmask[wid] & ((1ull << lane) - 1ull));
        if (wid == 1) below += __popcll(~s_dmask[0]);
        slot = ndc + below;
      }
      // a malformed dominant set leaves slots unset; reads clamp the channel
      if (slot < D) s_chan[slot] = tid;
    }
  }

  const bool live = r >= r_lo && r < r_hi;
  if (live) {
    const int64_t src = (static_cast<int64_t>(b) * Hkv + g) * S + r;
    const int64_t dst = (static_cast<int64_t>(b) * Hkv + g) * Lmax + st + r;
    // every load (the key row, the value row, the 8 frequencies) is issued
    // before the rotation uses any of them
    float a[8], bb[8], ra[8], rb[8], va[8], vb[8];
    Elem<T>::load8(k_new + src * D + 8 * c, a);
    Elem<T>::load8(k_new + src * D + P + 8 * c, bb);
    Elem<T>::load8(v_new + src * D + 8 * c, va);
    Elem<T>::load8(v_new + src * D + P + 8 * c, vb);
    double fj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) fj[j] = fr.f[8 * c + j];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float cs, sn;
      rot_cos_sin(st + r, fj[j], cs, sn);
      ra[j] = a[j] * cs - bb[j] * sn;
      rb[j] = bb[j] * cs + a[j] * sn;
    }
    if (slab != 1) {
      T* full = slab == 0 ? k_out : k_rest;  // layout 2: k_rest holds the full rows
      Elem<T>::store8(full + dst * D + 8 * c, ra);
      Elem<T>::store8(full + dst * D + P + 8 * c, rb);
    }
    if (slab) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        s_rows[rl][8 * c + j] = ra[j];
        s_rows[rl][P + 8 * c + j] = rb[j];
      }
    }
    Elem<T>::store8(v_out + dst * D + 8 * c, va);
    Elem<T>::store8(v_out + dst * D + P + 8 * c, vb);
  }
  if (!slab) return;
  __syncthreads();

  // each slab's rows [r_lo, r_hi) form one contiguous run of nr * width elements
  const int nr = static_cast<int>(r_hi - r_lo);
  const int row_off = static_cast<int>(r_lo) - r0;
  const int64_t row0 = (static_cast<int64_t>(b) * Hkv + g) * Lmax + st + r_lo;
  auto write_run = [&](T* __restrict__ base, int width, int slot0) {
    const int total = nr * width;
    if ((width & 7) == 0) {
      for (int e = tid * 8; e < total; e += 256 * 8) {
        const int rr = e / width, sl = e - rr * width;
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = s_rows[row_off + rr][s_chan[slot0 + sl + j] & (D - 1)];
        Elem<T>::store8(base + e, x);
      }
    } else {
      for (int e = tid; e < total; e += 256) {
        const int rr = e / width, sl = e - rr * width;
        Elem<T>::store1(base + e, s_rows[row_off + rr][s_chan[slot0 + sl] & (D - 1)]);
      }
    }
  };
  write_run(k_out + row0 * ndc, ndc, 0);
  if (slab == 1 && nrest > 0) write_run(k_rest + row0 * nrest, nrest, ndc);
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, int dtype, int B, int Hkv,
                            int S, int d, int Lmax, const int32_t* start, const RopeFreq& fr,
                            int slab, const int32_t* dom, int n_dom, void* k_out, void* k_rest,
                            void* v_out, hipStream_t st) {
  const int rpw = 256 / (d / 16);
  const dim3 grid((S + rpw - 1) / rpw, Hkv, B);
#define SA_KVA(T, D)                                                                             \
  kv_append_kernel<T, D><<<grid, 256, 0, st>>>(                                                  \
      static_cast<const T*>(k_new), static_cast<const T*>(v_new), Hkv, S, Lmax, start, fr, slab,  \
      dom, n_dom, static_cast<T*>(k_out), static_cast<T*>(k_rest), static_cast<T*>(v_out))
  if (dtype == kBF16) {
    if (d == 128) { SA_KVA(uint16_t, 128); } else { SA_KVA(uint16_t, 64); }
  } else {
    if (d == 128) { SA_KVA(float, 128); } else { SA_KVA(float, 64); }
  }
#undef SA_KVA
  return hipGetLastError();
}

}  // namespace sa

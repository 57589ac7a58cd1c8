// Block-score matrix product: scores[b, h, I, J] = scale * <pq[b, h, I], pk[b, g(h), J]>,
// -inf above the diagonal when causal.
//
// "Prism: Spectral-Aware Block-Sparse Attention", sec. 3 item 2 and sec. 5:
// the importance estimate is a block-level matrix product only.  The summed
// calibrated band logits are one dot product over all channels of the
// calibrated pooled vectors.
//
// The work is small next to attention (Hq * N^2 / 2 * d MACs) and runs on
// the bf16 matrix cores in split form (below); tiles strictly above the
// diagonal are filled with -inf without loading anything.
#include "sa_common.hpp"

namespace sa {

// ------------------------------------------------------------------ split-bf16 matrix-core form
// Pooled vectors are fp32; each value x is split into three bf16 parts
// hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid), so that
// x = hi + mid + lo to within 2^-27 |x| (each rounding keeps 8 significant
// bits of what is left), and the product <a, b> is summed from the six part
// products down to 2^-18 of |a b| (hi.hi, hi.mid, mid.hi, hi.lo, lo.hi,
// mid.mid; the dropped ones are below 2^-27 |a b|) on the matrix cores with
// fp32 accumulation, smallest first: the split-bf16 scheme of Henry, Tang &
// Heinecke (2019).  A channel product is then within about 2^-25 of exact,
// like an fp32 product.  Two parts (the three-product form) leave 2^-17 of
// |a b| per channel, which a score that nearly cancels can amplify past a
// 1e-4 relative bound.  One work-group per 64 x 64 output tile: its 64
// pooled query rows and 64 pooled key rows are staged in LDS 64 channels at
// a time with coalesced 16-byte loads (rows padded so a fragment read is
// bank-conflict free; 34 KB of LDS, four work-groups a CU), and after each
// stage one wave per 32 x 32 quarter runs v_mfma_f32_32x32x16_bf16 with A = query
// rows (lane l: row l % 32, channels 8 (l / 32) .. + 7 of the k-step) and
// B = key rows (lane l: row l % 32); the C layout gives lane l the output
// column l % 32 and rows 8 (r / 4) + 4 (l / 32) + r % 4.  Reading fragments
// straight from global memory instead (32 rows per load instruction) took
// as long as the fp32 FMA form.
typedef __attribute__((ext_vector_type(8))) __bf16 bs_bf16x8;
typedef __attribute__((ext_vector_type(16))) float bs_f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int bs_u32x4;

__device__ __forceinline__ uint32_t bs_pack(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// 8 fp32 values -> their bf16 high, middle and low parts (RNE each); the
// subtractions are exact (each removes the leading bits just rounded off)
__device__ __forceinline__ void bs_split(const float4& x, const float4& y, bs_bf16x8& hi,
                                         bs_bf16x8& mid, bs_bf16x8& lo) {
  float v[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
  bs_u32x4 part[3];
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = bs_pack(v[2 * j], v[2 * j + 1]);
      part[p][j] = w;
      if (p < 2) {
        v[2 * j] -= __uint_as_float(w << 16);
        v[2 * j + 1] -= __uint_as_float(w & 0xffff0000u);
      }
    }
  hi = __builtin_bit_cast(bs_bf16x8, part[0]);
  mid = __builtin_bit_cast(bs_bf16x8, part[1]);
  lo = __builtin_bit_cast(bs_bf16x8, part[2]);
}

template <int D>
__global__ __launch_bounds__(256) void block_gemm_mfma_kernel(const float* __restrict__ pq,
                                                              const float* __restrict__ pk, int Hq,
                                                              int Hkv, int N, float scale,
                                                              int causal,
                                                              float* __restrict__ scores) {
  // the tiles of a head in one XCD-contiguous range of work-group ids
  // (work-groups go to the 8 XCDs in turn), so the head's pooled rows are
  // fetched into one L2, not eight
  const int64_t gx = gridDim.x, gy = gridDim.y;
  const int64_t nwg = gx * gy * gridDim.z;
  int64_t wl = (blockIdx.z * gy + blockIdx.y) * gx + blockIdx.x;
  if ((nwg & 7) == 0) wl = (wl & 7) * (nwg >> 3) + (wl >> 3);
  const int ti = static_cast<int>(wl % gx), tj = static_cast<int>((wl / gx) % gy);
  const int bh = static_cast<int>(wl / (gx * gy));
  const int h = bh % Hq, b = bh / Hq, g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int ti0 = ti * 64, tj0 = tj * 64;
  float* out = scores + static_cast<int64_t>(bh) * N * N;
  if (causal && tj0 > ti0 + 63) {  // the whole tile lies above the diagonal: no loads
    for (int e = tid; e < 64 * 64; e += 256) {
      const int i = ti0 + e / 64, j = tj0 + e % 64;
      if (i < N && j < N) out[static_cast<int64_t>(i) * N + j] = -INFINITY;
    }
    return;
  }
  // the tile's 64 query rows and 64 key rows, staged KC channels at a time
  // with coalesced 16-byte loads (64 channels: two stages at d = 128)
  constexpr int KC = D < 64 ? D : 64;
  constexpr int LD = KC + 4;        // padded row: 16 rows of a fragment read hit distinct banks
  constexpr int F4 = KC / 4;        // float4 per staged row
  __shared__ __attribute__((aligned(16))) float sA[64 * LD];
  __shared__ __attribute__((aligned(16))) float sB[64 * LD];
  const float* A = pq + (static_cast<int64_t>(b) * Hq + h) * N * D;
  const float* Bm = pk + (static_cast<int64_t>(b) * Hkv + g) * N * D;
  const int i0 = ti0 + 32 * (w >> 1);   // this wave's 32 rows (I)
  const int j0 = tj0 + 32 * (w & 1);    // and 32 columns (J)
  const bool live = !(causal && j0 > i0 + 31);  // this quarter lies on or below the diagonal
  const float* ar = sA + (32 * (w >> 1) + l32) * LD + 8 * hi;
  const float* br = sB + (32 * (w & 1) + l32) * LD + 8 * hi;
  bs_f32x16 acc = {};
#pragma unroll
  for (int c0 = 0; c0 < D; c0 += KC) {
    if (c0 > 0) __syncthreads();  // every wave is done with the previous stage
    float4 a[64 * F4 / 256], c[64 * F4 / 256];
#pragma unroll
    for (int u = 0; u < 64 * F4 / 256; ++u) {
      const int e = tid + 256 * u, r = e / F4, q4 = e % F4;
      a[u] = *reinterpret_cast<const float4*>(A + static_cast<int64_t>(min(ti0 + r, N - 1)) * D + c0 + 4 * q4);
      c[u] = *reinterpret_cast<const float4*>(Bm + static_cast<int64_t>(min(tj0 + r, N - 1)) * D + c0 + 4 * q4);
    }
#pragma unroll
    for (int u = 0; u < 64 * F4 / 256; ++u) {
      const int e = tid + 256 * u, r = e / F4, q4 = e % F4;
      *reinterpret_cast<float4*>(sA + r * LD + 4 * q4) = a[u];
      *reinterpret_cast<float4*>(sB + r * LD + 4 * q4) = c[u];
    }
    __syncthreads();
    {
      // (a quarter above the diagonal, only on diagonal tiles, computes too
      // and writes -inf below: no branch around the matrix products)
#pragma unroll
      for (int s = 0; s < KC / 16; ++s) {
        bs_bf16x8 ah, am, al, bh_, bm, bl;
        bs_split(*reinterpret_cast<const float4*>(ar + 16 * s), *reinterpret_cast<const float4*>(ar + 16 * s + 4),
                 ah, am, al);
        bs_split(*reinterpret_cast<const float4*>(br + 16 * s), *reinterpret_cast<const float4*>(br + 16 * s + 4),
                 bh_, bm, bl);
        // C[m = I row][n = J column]: A = query rows, B = key rows; small parts first
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bm, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh_, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bh_, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bm, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh_, acc, 0, 0, 0);
      }
    }
  }
  if (!live) {  // a quarter above the diagonal
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + 8 * (r >> 2) + 4 * hi + (r & 3), j = j0 + l32;
      if (i < N && j < N) out[static_cast<int64_t>(i) * N + j] = -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + 8 * (r >> 2) + 4 * hi + (r & 3), j = j0 + l32;
    if (i < N && j < N)
      out[static_cast<int64_t>(i) * N + j] = (causal && j > i) ? -INFINITY : scale * acc[r];
  }
}

hipError_t launch_block_gemm(const float* pq, const float* pk, int B, int Hq, int Hkv, int N,
                             int d, float scale, int causal, float* scores, hipStream_t st) {
  const int t = (N + 63) / 64;
  const dim3 grid(t, t, static_cast<unsigned>(B * Hq));
  if (d == 128)
    block_gemm_mfma_kernel<128><<<grid, 256, 0, st>>>(pq, pk, Hq, Hkv, N, scale, causal, scores);
  else
    block_gemm_mfma_kernel<64><<<grid, 256, 0, st>>>(pq, pk, Hq, Hkv, N, scale, causal, scores);
  return hipGetLastError();
}

}  // namespace sa

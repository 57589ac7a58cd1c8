// Block-score matrix product: scores[b, h, I, J] = scale * <pq[b, h, I], pk[b, g(h), J]>,
// -inf above the diagonal when causal.
//
// "Prism: Spectral-Aware Block-Sparse Attention", sec. 3 item 2 and sec. 5:
// the importance estimate is a block-level matrix product only.  The summed
// calibrated band logits are one dot product over all channels of the
// calibrated pooled vectors.
//
// fp32 FMA keeps the scores well inside 1e-4 relative of an fp64 evaluation.
// The work is tiny next to attention (Hq * N^2 / 2 * d MACs), so this is a
// plain LDS-tiled 64x64 kernel; tiles strictly above the diagonal are filled
// with -inf without loading anything.  The accumulation order over channels
// is ascending, as before.
#include "sa_common.hpp"

namespace sa {

constexpr int kTile = 64;
constexpr int kKc = 64;   // channels per LDS stage
constexpr int kLd = kKc + 4;

// One work-group per 64 x 64 output tile.  The two 64-row slabs of pooled
// vectors go through LDS in stages of 64 channels with 16-byte loads; each
// thread accumulates a 4 x 4 block, channels in ascending order.  Rows are
// padded by 4 floats so the 16 row groups of a read fall in different bank
// quads.
__global__ __launch_bounds__(256) void block_gemm_kernel(const float* __restrict__ pq,
                                                         const float* __restrict__ pk, int Hq,
                                                         int Hkv, int N, int d, float scale,
                                                         int causal, float* __restrict__ scores) {
  const int ti = blockIdx.x;  // tile of I
  const int tj = blockIdx.y;  // tile of J
  const int bh = blockIdx.z;
  const int h = bh % Hq;
  const int b = bh / Hq;
  const int g = h / (Hq / Hkv);
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int i0 = ti * kTile, j0 = tj * kTile;
  float* out = scores + static_cast<int64_t>(bh) * N * N;

  if (causal && j0 > i0 + kTile - 1) {
    for (int e = threadIdx.x; e < kTile * kTile; e += 256) {
      const int i = i0 + e / kTile, j = j0 + e % kTile;
      if (i < N && j < N) out[static_cast<int64_t>(i) * N + j] = -INFINITY;
    }
    return;
  }

  __shared__ __attribute__((aligned(16))) float sa_[kTile * kLd];
  __shared__ __attribute__((aligned(16))) float sb_[kTile * kLd];
  const float* A = pq + (static_cast<int64_t>(b) * Hq + h) * N * d;
  const float* Bm = pk + (static_cast<int64_t>(b) * Hkv + g) * N * d;

  float acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;

  constexpr int q4 = kKc / 4;  // float4 per staged row
  for (int k0 = 0; k0 < d; k0 += kKc) {
    for (int e = threadIdx.x; e < kTile * q4; e += 256) {
      const int r = e / q4, c4 = e % q4;
      const int i = i0 + r, j = j0 + r;
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 av = i < N ? *reinterpret_cast<const float4*>(A + static_cast<int64_t>(i) * d + k0 + 4 * c4) : z;
      const float4 bv = j < N ? *reinterpret_cast<const float4*>(Bm + static_cast<int64_t>(j) * d + k0 + 4 * c4) : z;
      *reinterpret_cast<float4*>(sa_ + r * kLd + 4 * c4) = av;
      *reinterpret_cast<float4*>(sb_ + r * kLd + 4 * c4) = bv;
    }
    __syncthreads();
#pragma unroll 4
    for (int cc = 0; cc < kKc; cc += 4) {
      float4 av[4], bv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) av[x] = *reinterpret_cast<const float4*>(sa_ + (ty + 16 * x) * kLd + cc);
#pragma unroll
      for (int y = 0; y < 4; ++y) bv[y] = *reinterpret_cast<const float4*>(sb_ + (tx + 16 * y) * kLd + cc);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          acc[x][y] = fmaf(av[x].x, bv[y].x, acc[x][y]);
          acc[x][y] = fmaf(av[x].y, bv[y].y, acc[x][y]);
          acc[x][y] = fmaf(av[x].z, bv[y].z, acc[x][y]);
          acc[x][y] = fmaf(av[x].w, bv[y].w, acc[x][y]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int i = i0 + ty + 16 * x;
    if (i >= N) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int j = j0 + tx + 16 * y;
      if (j >= N) continue;
      out[static_cast<int64_t>(i) * N + j] = (causal && j > i) ? -INFINITY : scale * acc[x][y];
    }
  }
}

hipError_t launch_block_gemm(const float* pq, const float* pk, int B, int Hq, int Hkv, int N,
                             int d, float scale, int causal, float* scores, hipStream_t st) {
  const int t = (N + kTile - 1) / kTile;
  const dim3 grid(t, t, static_cast<unsigned>(B * Hq));
  block_gemm_kernel<<<grid, 256, 0, st>>>(pq, pk, Hq, Hkv, N, d, scale, causal, scores);
  return hipGetLastError();
}

}  // namespace sa

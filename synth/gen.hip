// Device-side seeded generator for the synthetic workloads.
//
// Same definition as the host generator in synth/__init__.py, written again
// here for the GPU: element n of tensor `tid` under `seed` takes the first
// three SplitMix64 outputs (Steele, Lea & Flood 2014) of the stream started at
// key = seed * 2^40 ^ tid * 2^36 ^ n, sums their twelve 16-bit lanes exactly,
// and scales (sum - 6*65535) by the fp32 constant 1/sqrt(65536^2 - 1) with one
// fp32 multiply (Irwin-Hall(12) normal).  Stored as fp32 or bf16 (nearest,
// ties to even).  This library makes inputs only; it is not part of the
// attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float gauss(uint64_t key, float c) {
  uint64_t s = key;
  int64_t total = 0;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    s += 0x9E3779B97F4A7C15ull;
    const uint64_t z = mix64(s);
#pragma unroll
    for (int j = 0; j < 4; ++j) total += static_cast<int64_t>((z >> (16 * j)) & 0xFFFFull);
  }
  const float centred = static_cast<float>(total - 6 * 65535);
  return centred * c;
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// out[r, j] = gen(base + r * logical_d + ch(r, j)), ch = chmap[head(r)][j] or j
__global__ void fill_kernel(void* out, int bf16, int64_t rows, int out_cols, int logical_d,
                            uint64_t base, uint64_t key_hi, float c, const int32_t* chmap,
                            int64_t rows_per_head, int n_heads) {
  const int64_t total = rows * out_cols;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = e / out_cols;
    const int j = static_cast<int>(e % out_cols);
    int ch = j;
    if (chmap) {
      const int head = static_cast<int>((r / rows_per_head) % n_heads);
      ch = chmap[head * out_cols + j];
    }
    const uint64_t n = base + static_cast<uint64_t>(r) * logical_d + ch;
    const float z = gauss(key_hi ^ n, c);
    if (bf16) static_cast<uint16_t*>(out)[e] = to_bf16(z);
    else static_cast<float*>(out)[e] = z;
  }
}

}  // namespace

extern "C" int synth_fill(void* out, int bf16, int64_t rows, int out_cols, int logical_d,
                          uint64_t base, int seed, int tid, float c, const int32_t* chmap,
                          int64_t rows_per_head, int n_heads, void* stream) {
  if (!out || rows < 0 || out_cols < 1) return 1;
  const uint64_t key_hi = (static_cast<uint64_t>(seed) << 40) ^ (static_cast<uint64_t>(tid) << 36);
  const int64_t total = rows * out_cols;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  fill_kernel<<<static_cast<unsigned>(blocks), 256, 0, static_cast<hipStream_t>(stream)>>>(
      out, bf16, rows, out_cols, logical_d, base, key_hi, c, chmap, rows_per_head, n_heads);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

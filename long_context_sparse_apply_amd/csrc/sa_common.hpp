// Device-side helpers shared by the kernels of the sparse-attention library.
// gfx950 only: wave64, bf16 stored as the upper 16 bits of an IEEE fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.hpp"
#include "sa_limits.hpp"

namespace sa {

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest, ties to even; NaN -> quiet NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// two bf16 packed in a uint32 (element 0 in the low half)
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// load / store 8 consecutive elements as fp32 (bf16: one 16-byte access; fp32: two)
template <typename T> struct Elem;
template <> struct Elem<float> {
  struct Raw { float4 a, b; };
  static __device__ __forceinline__ Raw load_raw8(const float* p) {
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  // the same with the nontemporal hint (data read once: its lines are the
  // first the L2 gives up)
  static __device__ __forceinline__ Raw load_raw8_nt(const float* p) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f a = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    const v4f b = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p + 4));
    return Raw{make_float4(a.x, a.y, a.z, a.w), make_float4(b.x, b.y, b.z, b.w)};
  }
  static __device__ __forceinline__ Raw zero_raw8() {
    return Raw{make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  }
  static __device__ __forceinline__ void unpack8(const Raw& r, float* v) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
  static __device__ __forceinline__ void load8(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store8(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  using Raw = uint4;
  static __device__ __forceinline__ Raw load_raw8(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
  static __device__ __forceinline__ Raw load_raw8_nt(const uint16_t* p) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  static __device__ __forceinline__ Raw zero_raw8() { return make_uint4(0u, 0u, 0u, 0u); }
  static __device__ __forceinline__ void unpack8(const Raw& a, float* v) {
    v[0] = lo_bf16(a.x); v[1] = hi_bf16(a.x); v[2] = lo_bf16(a.y); v[3] = hi_bf16(a.y);
    v[4] = lo_bf16(a.z); v[5] = hi_bf16(a.z); v[6] = lo_bf16(a.w); v[7] = hi_bf16(a.w);
  }
  static __device__ __forceinline__ void load8(const uint16_t* p, float* v) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    v[0] = lo_bf16(a.x); v[1] = hi_bf16(a.x); v[2] = lo_bf16(a.y); v[3] = hi_bf16(a.y);
    v[4] = lo_bf16(a.z); v[5] = hi_bf16(a.z); v[6] = lo_bf16(a.w); v[7] = hi_bf16(a.w);
  }
  static __device__ __forceinline__ void store8(uint16_t* p, const float* v) {
    uint4 a;
    a.x = pack_bf16(v[0], v[1]); a.y = pack_bf16(v[2], v[3]);
    a.z = pack_bf16(v[4], v[5]); a.w = pack_bf16(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = a;
  }
  static __device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store1(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

// ---------------------------------------------------------------- rotary angle
// cos / sin of 2*pi*frac(p * f) where f = omega / (2*pi) is given in fp64.
// The product and the reduction to one revolution are exact to ~1e-16
// revolutions for |p| < 2^31; the remaining angle (|a| <= pi) is evaluated in
// fp32.
__device__ __forceinline__ void rot_cos_sin(int64_t p, double f, float& c, float& s) {
  const double rev = static_cast<double>(p) * f;
  const double frac = rev - rint(rev);
  const float ang = static_cast<float>(frac * 6.283185307179586476925286766559);
  sincosf(ang, &s, &c);
}

// ---------------------------------------------------------------- direct-to-LDS load
// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane i of the wave writes lds_wave_base + 16 i; lds_wave_base must be uniform.
// Completion is tracked by vmcnt.  Kept in a __device__ function so host
// compilation of the calling kernels never sees the builtin.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}
// the same with the nontemporal hint (cache-policy bit 1, `nt`)
__device__ __forceinline__ void lds_dma16_nt(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 2);
}

// The same through a buffer resource (buffer_load_dwordx4 ... lds): lane i
// fetches base + voffset and writes lds_wave_base + 16 i; offsets at or past
// `bytes` read zeros.  The compiler keeps exact counts for LDS reads issued
// while such a load is in flight (with the global form above it waits for
// all of them before any use), so a wave can keep several operand reads in
// flight across the tile loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  // dword 3 = 0x00020000: raw (untyped) 32-bit buffer access on this family
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, int voffset,
                                              void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, voffset, 0, 0, 0);
}
// The same with the nontemporal hint (cache-policy bit 1, `nt`), for data a
// kernel streams through once: its lines are the first the L2 gives up.
__device__ __forceinline__ void lds_dma16_buf_nt(__amdgpu_buffer_rsrc_t r, int voffset,
                                                 void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, voffset, 0, 0, 2);
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace sa

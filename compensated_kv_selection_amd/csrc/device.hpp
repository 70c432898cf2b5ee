// Device helpers shared by the CompKV kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckv {

// ---- storage formats -------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16 bits, nearest with ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Eight consecutive elements as float (16-byte load for bf16, 2 x 16 for f32).
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store8(uint16_t* p, const float (&x)[8]) {
  uint4 w;
  w.x = bf16_rne(x[0]) | (bf16_rne(x[1]) << 16);
  w.y = bf16_rne(x[2]) | (bf16_rne(x[3]) << 16);
  w.z = bf16_rne(x[4]) | (bf16_rne(x[5]) << 16);
  w.w = bf16_rne(x[6]) | (bf16_rne(x[7]) << 16);
  *reinterpret_cast<uint4*>(p) = w;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

__device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }
__device__ __forceinline__ float load1(const float* p) { return *p; }

// ---- cross-lane reductions --------------------------------------------------

// Sum over aligned groups of W lanes (butterfly).  Addition is commutative,
// so every lane of a group ends with the same bits.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Dot products of G query rows with one 8-element slice (fp32, fixed order).
template <int G>
__device__ __forceinline__ void dot8(const float (&q)[G][8], const float (&x)[8], float (&out)[G]) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaf(q[j][e], x[e], a);
    out[j] = a;
  }
}

// exp(a - m) with an empty state (m = -inf) giving 0.
__device__ __forceinline__ float scale_from(float a, float m) {
  return a == -INFINITY ? 0.f : expf(a - m);
}

}  // namespace ckv

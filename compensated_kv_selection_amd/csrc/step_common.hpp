// Device pieces shared by the decode-step kernels: coherent workspace access,
// arrival counters, raw element loads, radix selection of the k largest keys
// and the ascending selection list.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "internal.hpp"

namespace ckv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// ---- coherent access to workspace written inside the same launch -----------
// The XCDs of the device have separate L2 caches.  Words that one workgroup
// writes and another reads during the same launch are written and read with
// the device-scope cache policy (sc1): such stores write through and such
// loads do not hit stale lines.  Counters use relaxed agent-scope atomics;
// bulk data uses plain buffer instructions with the same policy, which the
// compiler batches like ordinary loads and stores.

template <typename T>
__device__ __forceinline__ void st_c(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_c(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor, 32-bit elements
constexpr int kSc1 = 16;                // cache-policy operand: device scope

// A buffer view of `bytes` bytes at `base`; element indices are in units of
// the accessed type.  Accesses past `bytes` read 0 and drop writes.
struct Coh {
  __amdgpu_buffer_rsrc_t r;
  __device__ Coh(const void* base, size_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                            (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                            kRsrcWord3)) {}
  __device__ float f32(int i) const {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * i, 0, kSc1));
  }
  __device__ float4 f32x4(int i) const {  // i: float index, multiple of 4
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, 4 * i, 0, kSc1);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
  }
  __device__ uint64_t u64(int i) const {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, 8 * i, 0, kSc1);
    return ((uint64_t)v.y << 32) | v.x;
  }
  __device__ void put(int i, float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, 4 * i, 0, kSc1);
  }
  __device__ void put4(int i, float4 v) const {
    u32x4_t w;
    w.x = __float_as_uint(v.x); w.y = __float_as_uint(v.y);
    w.z = __float_as_uint(v.z); w.w = __float_as_uint(v.w);
    __builtin_amdgcn_raw_buffer_store_b128(w, r, 4 * i, 0, kSc1);
  }
  __device__ void put_u64(int i, uint64_t v) const {
    u32x2_t w;
    w.x = (uint32_t)v;
    w.y = (uint32_t)(v >> 32);
    __builtin_amdgcn_raw_buffer_store_b64(w, r, 8 * i, 0, kSc1);
  }
};

// Wait until *p >= target (bounded; running out sets the error word).
__device__ __forceinline__ void wait_at_least(uint32_t* p, uint32_t target, uint32_t* err) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (ld_c(p) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins == kSpinLimit) {
        st_c(err, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Count this workgroup in *p once all its memory operations have completed;
// returns the previous count (same value in every thread).
__device__ __forceinline__ uint32_t arrive(uint32_t* p, uint32_t* slot) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) *slot = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *slot;
}

// ---- eight consecutive elements kept as raw words until used ----------------
template <typename KV> struct Raw8;
template <> struct Raw8<uint16_t> { uint4 a; };
template <> struct Raw8<float> { uint4 a, b; };
__device__ __forceinline__ void raw_load(const uint16_t* p, Raw8<uint16_t>& r) {
  r.a = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void raw_load(const float* p, Raw8<float>& r) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  r.a = q[0];
  r.b = q[1];
}
__device__ __forceinline__ void raw_zero(Raw8<uint16_t>& r) { r.a = make_uint4(0u, 0u, 0u, 0u); }
__device__ __forceinline__ void raw_zero(Raw8<float>& r) { r.a = r.b = make_uint4(0u, 0u, 0u, 0u); }
__device__ __forceinline__ void raw_float(const Raw8<uint16_t>& r, float (&x)[8]) {
  x[0] = bf16_lo(r.a.x); x[1] = bf16_hi(r.a.x); x[2] = bf16_lo(r.a.y); x[3] = bf16_hi(r.a.y);
  x[4] = bf16_lo(r.a.z); x[5] = bf16_hi(r.a.z); x[6] = bf16_lo(r.a.w); x[7] = bf16_hi(r.a.w);
}
__device__ __forceinline__ void raw_float(const Raw8<float>& r, float (&x)[8]) {
  x[0] = __uint_as_float(r.a.x); x[1] = __uint_as_float(r.a.y);
  x[2] = __uint_as_float(r.a.z); x[3] = __uint_as_float(r.a.w);
  x[4] = __uint_as_float(r.b.x); x[5] = __uint_as_float(r.b.y);
  x[6] = __uint_as_float(r.b.z); x[7] = __uint_as_float(r.b.w);
}

// ---- selection keys -----------------------------------------------------------
// A block's key orders by score, then by lower block index: the float bits of
// a non-negative score compare like the score, and the complemented index
// puts the lower index first among equal scores.  Real keys are never 0 or 1.
__device__ __forceinline__ uint64_t make_key(float score, int idx) {
  return ((uint64_t)__float_as_uint(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int key_index(uint64_t key) {
  return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
}

struct LdsKeys {
  const uint64_t* p;
  __device__ uint64_t operator()(int i) const { return p[i]; }
};

// Radix select of the k-th largest of n 64-bit keys (distinct among the k
// largest), 8 bits per pass from the top, by the NT threads of the
// workgroup.  Returns T such that exactly k keys are >= T; 1 <= k <= n.
// hist: 512 words of LDS (two histograms used alternately), sh: 4 words.
template <int NT, class KeyAt>
__device__ uint64_t radix_kth_largest(const KeyAt key_at, int n, int k, uint32_t* hist, uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t prefix = 0, pmask = 0;
  uint32_t krem = (uint32_t)k;
  for (int e = tid; e < 512; e += NT) hist[e] = 0u;
  __syncthreads();
  for (int shift = 56, pass = 0; shift >= 0; shift -= 8, ++pass) {
    uint32_t* h = hist + 256 * (pass & 1);
    uint32_t* h_next = hist + 256 * ((pass + 1) & 1);
    for (int e = tid; e < 256; e += NT) h_next[e] = 0u;
    for (int i = tid; i < n; i += NT) {
      const uint64_t key = key_at(i);
      if ((key & pmask) == prefix) atomicAdd(&h[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t cs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) cs[e] = h[255 - 4 * lane - e];  // descending digits
      const uint32_t loc = cs[0] + cs[1] + cs[2] + cs[3];
      uint32_t inc = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      uint32_t cum = inc - loc;  // keys with a larger digit
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (cum < krem && cum + cs[e] >= krem) {
          sh[0] = 255u - 4u * lane - e;
          sh[1] = cum;
          sh[2] = cs[e];
        }
        cum += cs[e];
      }
    }
    __syncthreads();
    const uint32_t digit = sh[0], above = sh[1], cnt = sh[2];
    krem -= above;
    prefix |= (uint64_t)digit << shift;
    pmask |= (uint64_t)255u << shift;
    if (cnt == krem) break;  // every key with this prefix is taken
  }
  __syncthreads();  // sh and the histograms may be reused by the caller
  return prefix;
}

// Walk the selection bitmap (M bits) in ascending block order.  Writes the
// first `cap` entries of the ascending list to `out` when given, and the
// blocks at list positions [share_lo, share_hi) to share[0..).  wsum: NT/64
// words of LDS.
template <int NT>
__device__ void emit_selection(int M, const uint32_t* bitmap, uint32_t* wsum, int32_t* out, int cap,
                               int* share, int share_lo, int share_hi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int words = (M + 31) / 32;
  const int per = (words + NT - 1) / NT;
  const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
  uint32_t cnt = 0;
  for (int e = w0; e < w1; ++e) cnt += __popc(bitmap[e]);
  uint32_t inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t pos = inc - cnt;
  for (int v = 0; v < wave; ++v) pos += wsum[v];
  for (int e = w0; e < w1; ++e) {
    uint32_t bits = bitmap[e];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      const int idx = 32 * e + bit;
      if (out && (int)pos < cap) out[pos] = idx;
      if ((int)pos >= share_lo && (int)pos < share_hi) share[pos - share_lo] = idx;
      ++pos;
    }
  }
  __syncthreads();
}

// Online softmax update of one query head's state with one weighted logit.
template <int G>
__device__ __forceinline__ void online_add(float (&m)[G], float (&l)[G], float (&acc)[G][8], int j,
                                           float logit, float weight, const float (&val)[8]) {
  if (logit > m[j]) {
    const float sc = scale_from(m[j], logit);
    l[j] *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] *= sc;
    m[j] = logit;
  }
  const float p = weight * expf(logit - m[j]);
  l[j] += p;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(p, val[e], acc[j][e]);
}

}  // namespace
}  // namespace ckv

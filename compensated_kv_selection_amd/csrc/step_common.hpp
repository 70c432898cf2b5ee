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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// e^x and ln x through the hardware's base-2 instructions (v_exp_f32,
// v_log_f32): within a few units in the last place, denormal results flushed
// to zero.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float flog(float x) { return __builtin_amdgcn_logf(x) * 0.693147180559945309f; }
// exp(a - m), 0 for an empty state (a = -inf)
__device__ __forceinline__ float fscale(float a, float m) { return a == -INFINITY ? 0.f : fexp(a - m); }

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
// With `local` set, 64-bit words are stored with the default policy: they
// stay in the writer's L2, where device-scope loads from workgroups on the
// same XCD find them (much sooner than a write-through store reaches memory);
// workgroups on other XCDs may not see them before the launch ends.
struct Coh {
  __amdgpu_buffer_rsrc_t r;
  bool local;
  __device__ Coh(const void* base, size_t bytes, bool local_ = false)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                            (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                            kRsrcWord3)),
        local(local_) {}
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
    if (local) __builtin_amdgcn_raw_buffer_store_b64(w, r, 8 * i, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b64(w, r, 8 * i, 0, kSc1);
  }
};

// A read-only buffer view of `bytes` bytes at `base` for plain loads (byte
// offsets).  Reads past the end return 0 without touching memory, so range
// checks need no branches and every load of a batch is issued unconditionally.
struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ Buf(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                            (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu), kRsrcWord3)) {}
  __device__ uint4 u128(uint32_t off) const {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ float4 f128(uint32_t off) const {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  }
  __device__ uint32_t u32(uint32_t off) const { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
};

// A word that no workgroup writes during the launch, read through the scalar
// cache (uniform address): the wait for it does not hold vector loads.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  typedef const __attribute__((address_space(4))) T* const_p;
  return *(const_p)p;
}

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
// Eight elements at element offset e of a buffer view.
__device__ __forceinline__ void raw_load(const Buf& b, uint32_t e, Raw8<uint16_t>& r) { r.a = b.u128(2 * e); }
__device__ __forceinline__ void raw_load(const Buf& b, uint32_t e, Raw8<float>& r) {
  r.a = b.u128(4 * e);
  r.b = b.u128(4 * e + 16);
}
__device__ __forceinline__ void raw_store(uint16_t* p, const Raw8<uint16_t>& r) {
  *reinterpret_cast<uint4*>(p) = r.a;
}
__device__ __forceinline__ void raw_store(float* p, const Raw8<float>& r) {
  uint4* q = reinterpret_cast<uint4*>(p);
  q[0] = r.a;
  q[1] = r.b;
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

// ---- wave-wide cross-lane operations (DPP and permlane swaps, no LDS) -----------
__device__ __forceinline__ uint32_t dpp_quad_xor1(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t dpp_quad_xor2(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ uint32_t dpp_row_ror4(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_ror8(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_half_mirror(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_mirror(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false);
}
// Combine 16-lane rows pairwise (rows 0-1, 2-3), then wave halves; each
// result lane sees (low operand, high operand) in the same order.
template <class Op>
__device__ __forceinline__ uint32_t across_rows(uint32_t x, Op op) {
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op((uint32_t)p[0], (uint32_t)p[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op((uint32_t)h[0], (uint32_t)h[1]);
}
// Reduction over all 64 lanes; every lane receives the result.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, Op op) {
  x = op(x, dpp_quad_xor1(x));
  x = op(x, dpp_quad_xor2(x));
  x = op(x, dpp_row_ror4(x));
  x = op(x, dpp_row_ror8(x));
  return across_rows(x, op);
}
struct OpOr { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; } };
struct OpAnd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a & b; } };
struct OpFmax {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    const float x = __uint_as_float(a), y = __uint_as_float(b);
    return __float_as_uint(x > y ? x : y);
  }
};
struct OpFadd {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }
};
// Sum over each group of LPT consecutive lanes (LPT = 4, 8, 16) by DPP
// swaps within a row; every lane of a group receives the same value.
template <int LPT>
__device__ __forceinline__ float token_row_sum(float x) {
  uint32_t u = __float_as_uint(x);
  u = OpFadd{}(u, dpp_quad_xor1(u));
  u = OpFadd{}(u, dpp_quad_xor2(u));
  if (LPT >= 8) u = OpFadd{}(u, dpp_row_half_mirror(u));
  if (LPT >= 16) u = OpFadd{}(u, dpp_row_mirror(u));
  return __uint_as_float(u);
}
__device__ __forceinline__ float wave_max_dpp(float x) { return __uint_as_float(wave_reduce(__float_as_uint(x), OpFmax{})); }
__device__ __forceinline__ float wave_sum_dpp(float x) { return __uint_as_float(wave_reduce(__float_as_uint(x), OpFadd{})); }

// Inclusive prefix sum over the 64 lanes (rows of 16 by shifts, then row
// totals broadcast to the following rows).
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false); // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false); // row_bcast:31
  return x;
}

// Radix select of the k-th largest of n 64-bit keys (distinct among the k
// largest), by the NT threads of the workgroup.  Bits shared by every key
// are skipped; the rest is resolved 8 bits per pass from the top.  Returns T
// such that exactly k keys are >= T; 1 <= k <= n.
// hist: 512 words of LDS (two histograms used alternately), sh: 64 words.
template <int NT, class KeyAt>
__device__ uint64_t radix_kth_largest(const KeyAt key_at, int n, int k, uint32_t* hist, uint32_t* sh) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 12, "scratch words");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // keys are read four per thread at a time, all requested before the first
  // is used (one round trip per four instead of per key)
  constexpr int KB = 4;
  uint64_t kor = 0, kand = ~0ull;
  for (int i0 = tid; i0 < n; i0 += KB * NT) {
    uint64_t kb[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) kb[u] = i0 + u * NT < n ? key_at(i0 + u * NT) : 0ull;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (i0 + u * NT < n) {
        kor |= kb[u];
        kand &= kb[u];
      }
    }
  }
  const uint32_t ohi = wave_reduce((uint32_t)(kor >> 32), OpOr{}), olo = wave_reduce((uint32_t)kor, OpOr{});
  const uint32_t ahi = wave_reduce((uint32_t)(kand >> 32), OpAnd{}), alo = wave_reduce((uint32_t)kand, OpAnd{});
  if (lane == 0) {
    sh[16 + 4 * wave] = ohi;
    sh[17 + 4 * wave] = olo;
    sh[18 + 4 * wave] = ahi;
    sh[19 + 4 * wave] = alo;
  }
  for (int e = tid; e < 512; e += NT) hist[e] = 0u;
  __syncthreads();
  uint64_t all_or = 0, all_and = ~0ull;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    all_or |= ((uint64_t)sh[16 + 4 * v] << 32) | sh[17 + 4 * v];
    all_and &= ((uint64_t)sh[18 + 4 * v] << 32) | sh[19 + 4 * v];
  }
  const uint64_t diff = all_or ^ all_and;
  if (diff == 0) {  // every key equal
    __syncthreads();
    return all_and;
  }
  const int hb = 63 - __clzll((long long)diff);
  const uint64_t below = hb == 63 ? ~0ull : ((1ull << (hb + 1)) - 1);
  uint64_t prefix = all_and & ~below, pmask = ~below;
  uint32_t krem = (uint32_t)k;
  for (int top = hb, pass = 0; top >= 0; top -= 8, ++pass) {
    const int lo = top - 7;  // lowest bit of this digit (may be below bit 0)
    uint32_t* h = hist + 256 * (pass & 1);
    uint32_t* h_next = hist + 256 * ((pass + 1) & 1);
    for (int e = tid; e < 256; e += NT) h_next[e] = 0u;
    for (int i0 = tid; i0 < n; i0 += KB * NT) {
      uint64_t kb[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) kb[u] = i0 + u * NT < n ? key_at(i0 + u * NT) : 0ull;
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        if (i0 + u * NT < n && (kb[u] & pmask) == prefix) {
          const uint32_t d = (uint32_t)((lo >= 0 ? kb[u] >> lo : kb[u] << -lo) & 255u);
          atomicAdd(&h[d], 1u);
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t cs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) cs[e] = h[255 - 4 * lane - e];  // descending digits
      const uint32_t loc = cs[0] + cs[1] + cs[2] + cs[3];
      uint32_t cum = wave_scan_incl(loc) - loc;  // keys with a larger digit
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
    prefix |= lo >= 0 ? (uint64_t)digit << lo : (uint64_t)digit >> -lo;
    pmask |= lo >= 0 ? 255ull << lo : 255ull >> -lo;
    if (cnt == krem) break;  // every key with this prefix is taken
  }
  __syncthreads();  // sh and the histograms may be reused by the caller
  return prefix;
}

// ---- wave-wide sorting of 64-bit keys, one per lane ----------------------------
// Value of lane (lane ^ J) for J = 1, 2, 4, 8 (DPP within a row of 16 lanes;
// row_ror:n brings lane (i - n) mod 16) and 16, 32 (permlane swaps, which
// return the even/odd row, resp. low/high half, of each pair).
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  const uint32_t lane = __lane_id();
  if constexpr (J == 1) {
    return dpp_quad_xor1(x);
  } else if constexpr (J == 2) {
    return dpp_quad_xor2(x);
  } else if constexpr (J == 4) {
    const uint32_t below = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xF, 0xF, false);  // i - 4
    const uint32_t above = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x12C, 0xF, 0xF, false);  // i + 4
    return (lane & 4u) ? below : above;
  } else if constexpr (J == 8) {
    return dpp_row_ror8(x);
  } else if constexpr (J == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16u) ? (uint32_t)p[0] : (uint32_t)p[1];
  } else {
    static_assert(J == 32, "lane distance");
    const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32u) ? (uint32_t)h[0] : (uint32_t)h[1];
  }
}

// ---- one block's summary, per 8-channel slice (shared by the summary build
// and the single-launch step's decode append, so both give the same bits) ----
// Mean of rows 0..n-1 of a 16-row block, accumulated on data shifted by row
// 0 (a block of equal rows gets exactly that row as mean).
template <typename KV>
__device__ __forceinline__ void slice_mean(const Raw8<KV> (&raw)[kBlockSize], int n, float (&mu)[8]) {
  float x0[8], sx[8], x[8];
  raw_float(raw[0], x0);
#pragma unroll
  for (int e = 0; e < 8; ++e) sx[e] = 0.f;
#pragma unroll
  for (int t = 1; t < kBlockSize; ++t) {
    if (t < n) {
      raw_float(raw[t], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sx[e] += x[e] - x0[e];
    }
  }
  const float fn = (float)n;
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = x0[e] + sx[e] / fn;
}
// Sum over rows 0..n-1 of the squared deviations from mu (second pass).
template <typename KV>
__device__ __forceinline__ void slice_sqdev(const Raw8<KV> (&raw)[kBlockSize], int n, const float (&mu)[8],
                                            float (&var)[8]) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) var[e] = 0.f;
#pragma unroll
  for (int t = 0; t < kBlockSize; ++t) {
    if (t < n) {
      raw_float(raw[t], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dl = x[e] - mu[e];
        var[e] = fmaf(dl, dl, var[e]);
      }
    }
  }
}
// The grouped variance of a group of gs channels that spans wl = gs / 8
// adjacent, aligned lanes (each lane passing the sum of its slice's squared
// deviations): the sum across the group's lanes over n * gs.
__device__ __forceinline__ float group_variance_lanes(float vs, int gs, int n) {
  const int wl = gs / 8;
  float gsum = vs;
  if (wl > 1) gsum += __uint_as_float(lane_xor<1>(__float_as_uint(gsum)));
  if (wl > 2) gsum += __uint_as_float(lane_xor<2>(__float_as_uint(gsum)));
  if (wl > 4) gsum += __uint_as_float(lane_xor<4>(__float_as_uint(gsum)));
  if (wl > 8) gsum += __uint_as_float(lane_xor<8>(__float_as_uint(gsum)));
  return gsum / ((float)n * (float)gs);
}

// Compare-exchange with lane ^ J: this lane keeps the larger key if
// keep_max, else the smaller.
template <int J>
__device__ __forceinline__ uint64_t cmpx(uint64_t k, bool keep_max) {
  const uint64_t o = ((uint64_t)lane_xor<J>((uint32_t)(k >> 32)) << 32) | lane_xor<J>((uint32_t)k);
  return (k > o) == keep_max ? k : o;
}

// Bitonic merge steps J, J/2, ..., 1 of stage K (K = 64: the final,
// descending stage).  Runs of K lanes alternate direction below K = 64.
template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_steps(uint64_t k) {
  const uint32_t lane = __lane_id();
  k = cmpx<J>(k, ((lane & (uint32_t)K) == 0) == ((lane & (uint32_t)J) == 0));
  if constexpr (J > 1) return bitonic_steps<K, J / 2>(k);
  else return k;
}

// The 64 keys of the wave, one per lane, sorted in descending order across
// lanes (lane 0 the largest).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t k) {
  k = bitonic_steps<2, 1>(k);
  k = bitonic_steps<4, 2>(k);
  k = bitonic_steps<8, 4>(k);
  k = bitonic_steps<16, 8>(k);
  k = bitonic_steps<32, 16>(k);
  return bitonic_steps<64, 32>(k);
}

// Two descending 64-key lists, a in lane order and b in reversed lane order
// (lane i holds b[63 - i]): the 64 largest of their union, descending.
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t a, uint64_t b_reversed) {
  return bitonic_steps<64, 32>(a > b_reversed ? a : b_reversed);
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
  const uint32_t inc = wave_scan_incl(cnt);
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

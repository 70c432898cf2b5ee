// CompKV decode-step kernels for gfx950 (MI355X).
//
// The method (CompKV abstract, shd-paper.top listing; CompKV review,
// evolve.pub, "Summary" and FAQ): keys and values are split into blocks;
// every block keeps its mean key, grouped key variance and mean value; each
// block is ranked by a practical residual score - a second-order attention
// mass estimate times the estimated within-block logit variance (paper
// Section 3, Eqs. 4-7); the top-k blocks under a token budget are attended
// exactly, and every omitted block enters the softmax once, with its
// block-mean logit, weighted by its token count, carrying its mean value.
//
// Workgroup roles of the step kernel (a role is fixed by blockIdx):
//   scan   (sequence, KV head, chunk of 256 blocks).  Issues every load of
//          its chunk up front: mean keys and grouped variances (pass A) and
//          mean values (pass B).  Pass A computes block-mean logits on the
//          matrix cores - the G query heads of the KV head are the rows of a
//          16x16x32 bf16 MFMA tile - and the per-head log-scores; pass B sums
//          the compensation terms of all blocks of the chunk.
//   slice  (sequence, KV head, 1024 blocks).  Forms the ranked score of
//          each block of its slice and keeps the slice's top-k candidates.
//          In the fused launch every slice then computes the same global
//          top-k from all candidates and attends exactly to its share of
//          the selected blocks; in the select launch the last slice to
//          arrive does the global top-k and writes the selection.
//   gather (sequence, KV head, split of the selected blocks; attend-only and
//          dense launches) attends exactly to a split of the blocks.
//   merge  run by the workgroup that arrives last for its (sequence, KV
//          head): log-sum-exp combination of the exact partials with the
//          compensation of the omitted blocks (all-block sums minus the
//          selected blocks' own terms) into the output.
// Only the fused launch waits: slices wait for their KV head's scans and for
// each other.  The host launches it only when fewer waiting workgroups than
// half the device's resident capacity exist, so free slots always remain
// for the workgroups being waited on; every spin is bounded as well and sets
// an error flag if the bound is hit.  Otherwise the step runs as separate
// launches that never wait.  Hand-offs between workgroups use L2-coherent
// atomic loads and stores, ordered by s_waitcnt and the workgroup barrier.

#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace ckv {

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kSpinLimit = 1u << 22;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Agent-scope relaxed atomic loads and stores: L2-coherent across the XCDs.
template <typename T>
__device__ __forceinline__ void st_c(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_c(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t* ctr_scan_a(const Work& w, int bg) { return w.ctrl + kCtrlHeader + 4 * bg; }
__device__ __forceinline__ uint32_t* ctr_select(const Work& w, int bg) { return w.ctrl + kCtrlHeader + 4 * bg + 1; }
__device__ __forceinline__ uint32_t* ctr_merge(const Work& w, int bg) { return w.ctrl + kCtrlHeader + 4 * bg + 2; }

// Wait until *p >= target (bounded; the bound sets the error word).
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

// Count this workgroup in *p once all its stores have completed; returns the
// previous count (same value in every thread).
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

// ---------------------------------------------------------------------------
// Summary build: mean key, mean value, grouped key variance, count of one
// block for every KV head.  One workgroup per (sequence, block); threads over
// (KV head, 8-channel slice).  Summaries are stored by logical block.
// ---------------------------------------------------------------------------
template <typename KV, int D>
__global__ __launch_bounds__(kThreads) void summary_kernel(
    Shape s, const KV* __restrict__ kc, const KV* __restrict__ vc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ sl, int append_only, KV* __restrict__ mk, KV* __restrict__ mv,
    float* __restrict__ gv, int32_t* __restrict__ cnt) {
  extern __shared__ float var_sh[];  // [Hkv][D] per-channel variances
  constexpr int LPR = D / 8;
  const int b = append_only ? (int)blockIdx.x : (int)blockIdx.x / s.max_blocks;
  const int L = clamp_len(sl[b], s.max_blocks * s.bs);
  const int M = (L + s.bs - 1) / s.bs;
  const int i = append_only ? M - 1 : (int)blockIdx.x % s.max_blocks;
  if (i < 0 || i >= M) return;
  const int page = bt[(size_t)b * s.max_blocks + i];
  if (page < 0 || page >= s.P) return;
  const int n = min(s.bs, L - i * s.bs);
  const float fn = (float)n;

  for (int item = threadIdx.x; item < s.Hkv * LPR; item += blockDim.x) {
    const int g = item / LPR, c = item % LPR;
    const size_t tile = ((size_t)page * s.Hkv + g) * s.bs * D + c * 8;
    const KV* kp = kc + tile;
    const KV* vp = vc + tile;
    // Means on data shifted by the first token: a block of equal tokens gets
    // exactly that token as mean and zero variance.
    float k0[8], v0[8], sk[8], sv[8], x[8];
    load8(kp, k0);
    load8(vp, v0);
#pragma unroll
    for (int e = 0; e < 8; ++e) { sk[e] = 0.f; sv[e] = 0.f; }
    for (int t = 1; t < n; ++t) {
      load8(kp + t * D, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sk[e] += x[e] - k0[e];
      load8(vp + t * D, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] += x[e] - v0[e];
    }
    float mu[8], nu[8], var[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mu[e] = k0[e] + sk[e] / fn;
      nu[e] = v0[e] + sv[e] / fn;
      var[e] = 0.f;
    }
    for (int t = 0; t < n; ++t) {  // second pass: population variance
      load8(kp + t * D, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dl = x[e] - mu[e];
        var[e] = fmaf(dl, dl, var[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) var_sh[g * D + c * 8 + e] = var[e] / fn;
    const size_t row = (((size_t)b * s.Hkv + g) * s.max_blocks + i) * D + c * 8;
    store8(mk + row, mu);
    store8(mv + row, nu);
  }
  __syncthreads();
  const int gs = D / s.r;
  for (int item = threadIdx.x; item < s.Hkv * s.r; item += blockDim.x) {
    const int g = item / s.r, t = item % s.r;
    float acc = 0.f;
    for (int c = 0; c < gs; ++c) acc += var_sh[g * D + t * gs + c];
    gv[(((size_t)b * s.Hkv + g) * s.max_blocks + i) * s.r + t] = acc / (float)gs;
  }
  if (threadIdx.x == 0) cnt[(size_t)b * s.max_blocks + i] = n;
}

// ---------------------------------------------------------------------------
// Shared memory of the step kernel: one union, each role uses its member.
// ---------------------------------------------------------------------------
template <int D, int G>
struct ScanLds {
  static constexpr int RS = kThreads / (D / 8);
  float qf[G * D];         // this KV head's query rows
  float qn[G * D];         // |q_h restricted to channel group t|^2, [G][r]
  float sb[G][kChunk];     // block-mean logit
  float vh[G][kChunk];     // estimated within-block logit variance
  float lam[G][kChunk];    // log of the ranked per-head score
  float w[G][kChunk];      // compensation weight n e^{s_bar - chunk max}
  float acc[RS * D];       // row-slot sums for the final reduction
};
struct SelLds {
  uint64_t keys[kCandLds];           // slice keys, then second-level candidates
  uint32_t hist[256];
  uint32_t bitmap[kMaxBlocks / 32];
  float hm[(kMaxBlocks / kChunk + 1) * 8];  // chunk headers: max s_bar, z, max log score
  float hz[(kMaxBlocks / kChunk + 1) * 8];
  float hc[(kMaxBlocks / kChunk + 1) * 8];
  float lnz[8];
  float f[kSlice / kChunk][8];
  uint32_t sh[4];
  uint32_t count;
};
template <int D, int G>
struct GathLds {
  static constexpr int RS = kThreads / (D / 8);
  int pg[kShareMax];
  int n[kShareMax];
  float st[2 * RS * G];
  float acc[RS * D];
};
struct MergeLds {
  float f[kMergeFactors];
  float head[8][8];
};
template <int D, int G>
union StepLds {
  ScanLds<D, G> scan;
  SelLds sel;
  GathLds<D, G> gath;
  MergeLds merge;
};

// ---------------------------------------------------------------------------
// Scan
// ---------------------------------------------------------------------------
template <typename KV, int D, int G, int MODE>
__device__ int scan_role(const Shape& s, const StepIO& io, const Work& w, int t, ScanLds<D, G>& L,
                         uint32_t* slot) {
  constexpr int LPR = D / 8, RS = kThreads / LPR, PST = kPartStride(D);
  constexpr int RPL = kChunk / RS;  // pass-B rows per lane
  const int chunk = t % s.n_chunks, bg = t / s.n_chunks;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rs = tid / LPR, c = tid % LPR;
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int start = chunk * kChunk;
  const int nrows = max(0, min(M, start + kChunk) - start);
  const size_t row0 = (size_t)bg * s.max_blocks + start;  // logical summary row of the chunk
  const KV* q = static_cast<const KV*>(io.q) + ((size_t)b * s.Hq + g * G) * D;
  const KV* mk = static_cast<const KV*>(io.summ.mean_k) + row0 * D;
  const KV* mv = static_cast<const KV*>(io.summ.mean_v) + row0 * D;
  const int r = s.r, gs = D / r;
  const float* gv = io.summ.gvar + row0 * r;

  // ---- every load of the chunk, issued first ----
  constexpr bool MF = std::is_same<KV, uint16_t>::value;
  constexpr int KT = D / 32;
  uint4 mu[4][KT];      // pass A (matrix path): 4 groups of 16 rows per wave
  float4 gpre[4];       // grouped variances of those rows (r == 4)
  bf16x8_t qa[KT];
  Raw8<KV> nu[RPL];     // pass B: mean values of this lane's rows
  const bool holder = (lane >> 4) * 4 < G;
  if constexpr (MF) {
    const int head = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (head < G) v = *reinterpret_cast<const uint4*>(q + (size_t)head * D + 32 * kt + 8 * kq);
      qa[kt] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ri = (wave + 4 * u) * 16 + (lane & 15);
      const bool ok = ri < nrows;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        mu[u][kt] = ok ? *reinterpret_cast<const uint4*>(mk + (size_t)ri * D + 32 * kt + 8 * (lane >> 4))
                       : make_uint4(0u, 0u, 0u, 0u);
      gpre[u] = (ok && holder && r == 4) ? *reinterpret_cast<const float4*>(gv + (size_t)ri * 4)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int jj = 0; jj < RPL; ++jj) {
    const int ri = rs + jj * RS;
    if (ri < nrows) raw_load(mv + (size_t)ri * D + c * 8, nu[jj]);
    else raw_zero(nu[jj]);
  }
  for (int e = tid; e < G * D; e += kThreads) L.qf[e] = load1(q + e);
  __syncthreads();
  for (int item = tid; item < G * r; item += kThreads) {
    const int j = item / r, tg = item % r;
    const float* qh = L.qf + j * D + tg * gs;
    float a = 0.f;
    for (int cc = 0; cc < gs; ++cc) a = fmaf(qh[cc], qh[cc], a);
    L.qn[item] = a;
  }
  __syncthreads();

  // ---- pass A: block-mean logits and variance estimates ----
  if constexpr (MF) {
    // D[head][row] = sum_k Q[head][k] mean_k[row][k]; lane l holds Q[l%16][8(l/16)..+7]
    // of each 32-wide k-slice (zero rows past G), mean_k of row l%16 at the same
    // k, and receives D[4(l/16)+i][l%16].
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kt], __builtin_bit_cast(bf16x8_t, mu[u][kt]), acc,
                                                       0, 0, 0);
      const int ri = (wave + 4 * u) * 16 + (lane & 15);
      if (ri < nrows && holder) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * (lane >> 4) + i;
          if (j < G) {
            float sig = 0.f;
            if (r == 4) {
              sig = fmaf(L.qn[j * 4 + 0], gpre[u].x, sig);
              sig = fmaf(L.qn[j * 4 + 1], gpre[u].y, sig);
              sig = fmaf(L.qn[j * 4 + 2], gpre[u].z, sig);
              sig = fmaf(L.qn[j * 4 + 3], gpre[u].w, sig);
            } else {
              for (int e = 0; e < r; ++e) sig = fmaf(L.qn[j * r + e], gv[(size_t)ri * r + e], sig);
            }
            L.sb[j][ri] = acc[i] * s.tau;
            L.vh[j][ri] = sig * s.tau2;
          }
        }
      }
    }
  } else {
    // f32 storage: vector ALU, D/8 lanes per row.
    float qv[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[j][e] = L.qf[j * D + c * 8 + e];
    for (int ri = rs; ri < nrows; ri += RS) {
      float mu8[8], dot[G], sig[G];
      load8(mk + (size_t)ri * D + c * 8, mu8);
      dot8<G>(qv, mu8, dot);
#pragma unroll
      for (int j = 0; j < G; ++j) sig[j] = 0.f;
      for (int e = c; e < r; e += LPR) {
        const float gve = gv[(size_t)ri * r + e];
#pragma unroll
        for (int j = 0; j < G; ++j) sig[j] = fmaf(L.qn[j * r + e], gve, sig[j]);
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float d = group_sum<LPR>(dot[j]);
        const float v = group_sum<LPR>(sig[j]);
        if (c == 0) {
          L.sb[j][ri] = d * s.tau;
          L.vh[j][ri] = v * s.tau2;
        }
      }
    }
  }
  __syncthreads();

  // ---- log-scores, chunk maxima, compensation weights, Z_hat partial ----
  float* part = w.cpart + ((size_t)bg * s.n_chunks + chunk) * G * PST;
  for (int j = wave; j < G; j += 4) {
    float mx = -INFINITY, cx = -INFINITY;
    for (int ri = lane; ri < nrows; ri += 64) {
      const int n = min(s.bs, Lseq - (start + ri) * s.bs);
      const float sb = L.sb[j][ri], half = 0.5f * L.vh[j][ri];
      const float massf = (float)n * (1.f + half);  // second-order mass estimate / e^{s_bar}
      const float lam = io.score_mode == kScoreMass ? sb + logf(massf) : sb + logf(massf * half);
      L.lam[j][ri] = lam;
      mx = fmaxf(mx, sb);
      cx = fmaxf(cx, lam);
    }
    mx = wave_max(mx);
    cx = wave_max(cx);
    float lsum = 0.f, zsum = 0.f;
    float* xrow = w.xs + ((size_t)b * s.Hq + g * G + j) * s.max_blocks + start;
    for (int ri = lane; ri < nrows; ri += 64) {
      const int n = min(s.bs, Lseq - (start + ri) * s.bs);
      const float wt = (float)n * expf(L.sb[j][ri] - mx);
      lsum += wt;
      zsum = fmaf(wt, 1.f + 0.5f * L.vh[j][ri], zsum);
      const float lam = L.lam[j][ri];
      L.w[j][ri] = wt;
      st_c(xrow + ri, lam == -INFINITY ? 0.f : expf(lam - cx));
    }
    lsum = wave_sum(lsum);
    zsum = wave_sum(zsum);
    if (lane == 0) {
      float* h = part + (size_t)j * PST;
      st_c(h, mx);
      st_c(h + 1, lsum);
      st_c(h + 2, zsum);
      st_c(h + 3, cx);
    }
  }
  if (MODE == kModeFused) arrive(ctr_scan_a(w, bg), slot);
  else __syncthreads();

  // ---- pass B: compensation sums over the chunk's mean values ----
  float acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
#pragma unroll
  for (int jj = 0; jj < RPL; ++jj) {
    const int ri = rs + jj * RS;
    if (ri < nrows) {
      float x[8];
      raw_float(nu[jj], x);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float wt = L.w[j][ri];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(wt, x[e], acc[j][e]);
      }
    }
  }
  // every row slot shares the chunk maximum: plain sums across slots
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) L.acc[rs * D + c * 8 + e] = acc[j][e];
    __syncthreads();
    for (int d = tid; d < D; d += kThreads) {
      float a = 0.f;
      for (int r2 = 0; r2 < RS; ++r2) a += L.acc[r2 * D + d];
      st_c(part + (size_t)j * PST + 4 + d, a);
    }
    __syncthreads();
  }
  if (MODE == kModeFused) {
    const uint32_t prev = arrive(ctr_merge(w, bg), slot);
    return prev == (uint32_t)(s.n_chunks + s.n_slices - 1) ? bg : -1;
  }
  return -1;
}

// ---------------------------------------------------------------------------
// Radix select of the k-th largest of n distinct 64-bit keys, 8 bits per pass
// from the top.  Returns T such that exactly k keys are >= T.  1 <= k <= n.
// ---------------------------------------------------------------------------
struct LdsKeys {
  const uint64_t* p;
  __device__ uint64_t operator()(int i) const { return p[i]; }
};
// Candidates of all slices in memory: slice s holds its kk keys at s * stride.
struct SliceKeys {
  const uint64_t* p;
  int kk, stride;
  __device__ uint64_t operator()(int e) const { return ld_c(p + (size_t)(e / kk) * stride + (e % kk)); }
};

template <class KeyAt>
__device__ uint64_t radix_kth_largest(const KeyAt key_at, int n, int k, uint32_t* hist, uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t prefix = 0, pmask = 0;
  uint32_t krem = (uint32_t)k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int e = tid; e < 256; e += kThreads) hist[e] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint64_t key = key_at(i);
      if ((key & pmask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t cs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) cs[e] = hist[255 - 4 * lane - e];  // descending digits
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
    __syncthreads();
    if (cnt == krem) break;  // every key with this prefix is taken
  }
  return prefix;
}

__device__ __forceinline__ uint64_t make_key(float score, int idx) {
  return ((uint64_t)__float_as_uint(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int key_index(uint64_t key) {
  return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
}

// Global top-k of (sequence, KV head) from the slices' candidates: marks the
// selected blocks in L.bitmap and returns after a barrier.
__device__ void global_topk(const Shape& s, const Work& w, int bg, int kk, int M, SelLds& L) {
  const int tid = threadIdx.x;
  const uint64_t* all = w.cand + (size_t)bg * s.n_slices * s.kmax;
  const int n2 = s.n_slices * kk;
  const int words = (M + 31) / 32;
  for (int e = tid; e < words; e += kThreads) L.bitmap[e] = 0u;
  if (n2 <= kCandLds) {
    for (int e = tid; e < n2; e += kThreads) L.keys[e] = ld_c(all + (size_t)(e / kk) * s.kmax + (e % kk));
    __syncthreads();
    const uint64_t T = radix_kth_largest(LdsKeys{L.keys}, n2, kk, L.hist, L.sh);
    for (int e = tid; e < n2; e += kThreads) {
      const uint64_t key = L.keys[e];
      if (key >= T) atomicOr(&L.bitmap[key_index(key) >> 5], 1u << (key_index(key) & 31));
    }
  } else {
    __syncthreads();
    const SliceKeys keys{all, kk, s.kmax};
    const uint64_t T = radix_kth_largest(keys, n2, kk, L.hist, L.sh);
    for (int e = tid; e < n2; e += kThreads) {
      const uint64_t key = keys(e);
      if (key >= T) atomicOr(&L.bitmap[key_index(key) >> 5], 1u << (key_index(key) & 31));
    }
  }
  __syncthreads();
}

// Walk the selection bitmap in ascending block order.  Writes the output
// selection when `out` is given, and the blocks at positions
// [share_lo, share_hi) of the ascending list into `share`.
__device__ void emit_selection(int M, SelLds& L, int32_t* out, int* share, int share_lo, int share_hi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int words = (M + 31) / 32;
  const int per = (words + kThreads - 1) / kThreads;
  const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
  uint32_t cnt = 0;
  for (int e = w0; e < w1; ++e) cnt += __popc(L.bitmap[e]);
  uint32_t inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) L.hist[wave] = inc;
  __syncthreads();
  uint32_t pos = inc - cnt;
  for (int v = 0; v < wave; ++v) pos += L.hist[v];
  for (int e = w0; e < w1; ++e) {
    uint32_t bits = L.bitmap[e];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      const int idx = 32 * e + bit;
      if (out) st_c(out + pos, (int32_t)idx);
      if ((int)pos >= share_lo && (int)pos < share_hi) share[pos - share_lo] = idx;
      ++pos;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Gather core: exact attention over a list of blocks of one (sequence, KV
// head), and (comp) those blocks' own compensation terms.  Writes
// [m, l, -, -, acc[D]] per query head at part (head stride `slot`); the
// compensation partial follows at part + D + 4 unless slot == D + 4.
// ---------------------------------------------------------------------------
template <int D, int G, int RS>
__device__ void combine_online(const float (&m)[G], const float (&l)[G], const float (&acc)[G][8],
                               float* part, int head_stride, float* st, float* sacc) {
  constexpr int LPR = D / 8;
  const int tid = threadIdx.x, rs = tid / LPR, c = tid % LPR;
  if (c == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      st[rs * G + j] = m[j];
      st[RS * G + rs * G + j] = l[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float Mj = -INFINITY;
    for (int r2 = 0; r2 < RS; ++r2) Mj = fmaxf(Mj, st[r2 * G + j]);
    const float f = scale_from(m[j], Mj);
#pragma unroll
    for (int e = 0; e < 8; ++e) sacc[rs * D + c * 8 + e] = acc[j][e] * f;
    __syncthreads();
    float* pj = part + (size_t)j * head_stride;
    for (int d = tid; d < D; d += kThreads) {
      float a = 0.f;
      for (int r2 = 0; r2 < RS; ++r2) a += sacc[r2 * D + d];
      st_c(pj + 4 + d, a);
    }
    if (tid == 0) {
      float ls = 0.f;
      for (int r2 = 0; r2 < RS; ++r2) ls += st[RS * G + r2 * G + j] * scale_from(st[r2 * G + j], Mj);
      st_c(pj, Mj);
      st_c(pj + 1, ls);
    }
    __syncthreads();
  }
}

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

template <typename KV, int D, int G>
__device__ void gather_core(const Shape& s, const StepIO& io, int b, int g, const int* blk, int nb,
                            bool comp, float* part, int slot, GathLds<D, G>& L) {
  constexpr int LPR = D / 8, RS = kThreads / LPR, PST = kPartStride(D);
  constexpr int UG = 4;  // rows per lane per batch
  const int bg = b * s.Hkv + g;
  const int tid = threadIdx.x, rs = tid / LPR, c = tid % LPR;
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const KV* q = static_cast<const KV*>(io.q) + ((size_t)b * s.Hq + g * G) * D;
  const KV* kc = static_cast<const KV*>(io.k_cache);
  const KV* vc = static_cast<const KV*>(io.v_cache);

  for (int e = tid; e < nb; e += kThreads) {
    const int i = blk[e];
    int p = -1, n = 0;
    if (i >= 0 && i < M) {
      p = io.block_table[(size_t)b * s.max_blocks + i];
      if (p < 0 || p >= s.P) p = -1;
      else n = min(s.bs, Lseq - i * s.bs);
    }
    L.pg[e] = p;
    L.n[e] = n;
  }
  float qv[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) load8(q + (size_t)j * D + c * 8, qv[j]);
  __syncthreads();

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  const int nrows = nb * kBlockSize;
  const int nbatch = (nrows + RS * UG - 1) / (RS * UG);
  Raw8<KV> kr[UG], vr[UG];
  bool ok[UG];
  // software pipeline: the next batch is in flight while this one is used
#define CKV_ISSUE(BI)                                                                     \
  _Pragma("unroll") for (int u = 0; u < UG; ++u) {                                        \
    const int R = ((BI) * UG + u) * RS + rs;                                              \
    const int bl = R / kBlockSize, tok = R % kBlockSize;                                  \
    ok[u] = R < nrows && L.pg[bl] >= 0 && tok < L.n[bl];                                  \
    if (ok[u]) {                                                                          \
      const size_t off = (((size_t)L.pg[bl] * s.Hkv + g) * s.bs + tok) * D + c * 8;       \
      raw_load(kc + off, kr[u]);                                                          \
      raw_load(vc + off, vr[u]);                                                          \
    }                                                                                     \
  }
  if (nbatch > 0) { CKV_ISSUE(0) }
  for (int bi = 0; bi < nbatch; ++bi) {
    float k8[UG][8], v8[UG][8];
    bool okc[UG];
#pragma unroll
    for (int u = 0; u < UG; ++u) {
      okc[u] = ok[u];
      if (ok[u]) {
        raw_float(kr[u], k8[u]);
        raw_float(vr[u], v8[u]);
      }
    }
    if (bi + 1 < nbatch) { CKV_ISSUE(bi + 1) }
#pragma unroll
    for (int u = 0; u < UG; ++u) {
      if (okc[u]) {  // uniform across the row's lanes
        float dot[G];
        dot8<G>(qv, k8[u], dot);
#pragma unroll
        for (int j = 0; j < G; ++j) online_add<G>(m, l, acc, j, group_sum<LPR>(dot[j]) * s.tau, 1.f, v8[u]);
      }
    }
  }
#undef CKV_ISSUE
  combine_online<D, G, RS>(m, l, acc, part, slot, L.st, L.acc);
  if (slot == PST) return;  // dense: no compensation slot

#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  if (comp) {
    const KV* mk = static_cast<const KV*>(io.summ.mean_k);
    const KV* mv = static_cast<const KV*>(io.summ.mean_v);
    for (int e = rs; e < nb; e += RS) {
      if (L.n[e] == 0) continue;  // uniform across the row's lanes
      const size_t row = ((size_t)bg * s.max_blocks + blk[e]) * D + c * 8;
      float mu8[8], nu8[8], dot[G];
      load8(mk + row, mu8);
      load8(mv + row, nu8);
      dot8<G>(qv, mu8, dot);
      const float fn = (float)L.n[e];
#pragma unroll
      for (int j = 0; j < G; ++j) online_add<G>(m, l, acc, j, group_sum<LPR>(dot[j]) * s.tau, fn, nu8);
    }
  }
  combine_online<D, G, RS>(m, l, acc, part + PST, slot, L.st, L.acc);
}

// ---------------------------------------------------------------------------
// Slice: ranked scores, slice top-k, global top-k, and (fused) a share of the
// exact attention.
// ---------------------------------------------------------------------------
template <typename KV, int D, int G, int MODE>
__device__ int slice_role(const Shape& s, const StepIO& io, const Work& w, int t, StepLds<D, G>& U,
                          int* share, uint32_t* slot) {
  constexpr int PST = kPartStride(D);
  SelLds& L = U.sel;
  const int slice = t % s.n_slices, bg = t / s.n_slices;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (MODE == kModeFused) wait_at_least(ctr_scan_a(w, bg), (uint32_t)s.n_chunks, w.ctrl + 2);

  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = min(M, s.kmax);
  const float* parts = w.cpart + (size_t)bg * s.n_chunks * G * PST;
  const int i0 = slice * kSlice;
  const int nloc = max(0, min(M, i0 + kSlice) - i0);

  // chunk headers and this slice's per-head scores, all loads issued together
  for (int item = tid; item < s.n_chunks * G; item += kThreads) {
    const float* h = parts + (size_t)item * PST;
    L.hm[item] = ld_c(h);
    L.hz[item] = ld_c(h + 2);
    L.hc[item] = ld_c(h + 3);
  }
  constexpr int XPT = kSlice / kThreads;
  float xv[XPT][G];
#pragma unroll
  for (int u = 0; u < XPT; ++u) {
    const int i = tid + u * kThreads;
#pragma unroll
    for (int j = 0; j < G; ++j)
      xv[u][j] = i < nloc ? ld_c(w.xs + ((size_t)b * s.Hq + g * G + j) * s.max_blocks + i0 + i) : 0.f;
  }
  __syncthreads();
  // log Z_hat per query head: Z_hat = sum over chunks of z e^{max s_bar}
  for (int j = wave; j < G; j += 4) {
    float mz = -INFINITY;
    for (int ch = lane; ch < s.n_chunks; ch += 64) mz = fmaxf(mz, L.hm[ch * G + j]);
    mz = wave_max(mz);
    float zs = 0.f;
    for (int ch = lane; ch < s.n_chunks; ch += 64) zs += L.hz[ch * G + j] * scale_from(L.hm[ch * G + j], mz);
    zs = wave_sum(zs);
    if (lane == 0) L.lnz[j] = zs > 0.f ? mz + logf(zs) : -INFINITY;
  }
  __syncthreads();
  constexpr int CPS = kSlice / kChunk;
  for (int item = tid; item < CPS * G; item += kThreads) {
    const int cc = item / G, j = item % G;
    const int ch = i0 / kChunk + cc;
    const float cmax = ch < s.n_chunks ? L.hc[ch * G + j] : -INFINITY;
    L.f[cc][j] = (cmax == -INFINITY || L.lnz[j] == -INFINITY) ? 0.f : expf(cmax - L.lnz[j]);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < XPT; ++u) {
    const int i = tid + u * kThreads;
    if (i < nloc) {
      const int cc = i / kChunk;
      float S = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) S = fmaf(xv[u][j], L.f[cc][j], S);
      L.keys[i] = make_key(S, i0 + i);
      if (io.group_scores) io.group_scores[(size_t)bg * s.max_blocks + i0 + i] = S;
    }
  }
  __syncthreads();

  uint64_t* cand = w.cand + ((size_t)bg * s.n_slices + slice) * s.kmax;
  if (kk > 0 && kk < M) {
    const int k1 = min(kk, nloc);
    if (k1 > 0) {
      const uint64_t T = radix_kth_largest(LdsKeys{L.keys}, nloc, k1, L.hist, L.sh);
      if (tid == 0) L.count = 0;
      __syncthreads();
      for (int i = tid; i < nloc; i += kThreads) {
        const uint64_t key = L.keys[i];
        if (key >= T) st_c(cand + atomicAdd(&L.count, 1u), key);
      }
    }
    for (int e = k1 + tid; e < kk; e += kThreads) st_c(cand + e, (uint64_t)0);  // below every real key
  }
  const uint32_t prev = arrive(ctr_select(w, bg), slot);

  if (MODE == kModeSelectOnly) {
    // the last slice of this (sequence, KV head) does the global top-k
    if (prev != (uint32_t)(s.n_slices - 1)) return -1;
    int32_t* out = io.selected + (size_t)bg * s.kmax;
    if (tid == 0) st_c(io.num_selected + bg, (int32_t)kk);
    for (int e = kk + tid; e < s.kmax; e += kThreads) st_c(out + e, (int32_t)-1);
    if (kk == M) {
      for (int i = tid; i < M; i += kThreads) st_c(out + i, (int32_t)i);
    } else if (kk > 0) {
      global_topk(s, w, bg, kk, M, L);
      emit_selection(M, L, out, share, 0, 0);
    }
    if (tid == 0) st_c(ctr_select(w, bg), 0u);
    return -1;
  }

  // fused: every slice computes the global top-k and attends to its share
  wait_at_least(ctr_select(w, bg), (uint32_t)s.n_slices, w.ctrl + 2);
  const int lo = slice * s.share, hi = min(kk, lo + s.share);
  const int nb = max(0, hi - lo);
  int32_t* out = slice == 0 ? io.selected + (size_t)bg * s.kmax : nullptr;
  if (slice == 0) {
    if (tid == 0) st_c(io.num_selected + bg, (int32_t)kk);
    for (int e = kk + tid; e < s.kmax; e += kThreads) st_c(out + e, (int32_t)-1);
  }
  if (kk == M) {
    for (int i = tid; i < M; i += kThreads) {
      if (out) st_c(out + i, (int32_t)i);
      if (i >= lo && i < hi) share[i - lo] = i;
    }
    __syncthreads();
  } else if (kk > 0) {
    global_topk(s, w, bg, kk, M, L);
    emit_selection(M, L, out, share, lo, hi);
  }
  constexpr int SLOT = 2 * PST;
  float* gp = w.gpart + ((size_t)bg * s.n_slices + slice) * G * SLOT;
  gather_core<KV, D, G>(s, io, b, g, share, nb, io.compensate != 0, gp, SLOT, U.gath);
  const uint32_t prev_m = arrive(ctr_merge(w, bg), slot);
  return prev_m == (uint32_t)(s.n_chunks + s.n_slices - 1) ? bg : -1;
}

// ---------------------------------------------------------------------------
// Gather (attend-only and dense launches)
// ---------------------------------------------------------------------------
template <typename KV, int D, int G, int MODE>
__device__ int gather_role(const Shape& s, const StepIO& io, const Work& w, int t, GathLds<D, G>& L,
                           int* blk, uint32_t* slot) {
  constexpr int PST = kPartStride(D);
  constexpr bool DENSE = MODE == kModeDense;
  constexpr int SLOT = (DENSE ? 1 : 2) * PST;
  const int split = t % s.n_splits, bg = t / s.n_splits;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = DENSE ? M : min(min(ld_c(io.num_selected + bg), s.kmax), M);
  const int first = split * s.pages_per_split;
  const int nb = max(0, min(kk, first + s.pages_per_split) - first);
  for (int e = threadIdx.x; e < nb; e += kThreads)
    blk[e] = DENSE ? first + e : ld_c(io.selected + (size_t)bg * s.kmax + first + e);
  __syncthreads();
  float* gp = w.gpart + ((size_t)bg * s.n_splits + split) * G * SLOT;
  gather_core<KV, D, G>(s, io, b, g, blk, nb, !DENSE && io.compensate != 0, gp, SLOT, L);
  const uint32_t prev = arrive(ctr_merge(w, bg), slot);
  return prev == (uint32_t)(s.n_splits - 1) ? bg : -1;
}

// ---------------------------------------------------------------------------
// Merge: out = (exact + omitted compensation) / (their weights), lse.
// omitted = all-block compensation sums (scan) - the selected blocks' terms.
// ---------------------------------------------------------------------------
template <int D, int G, int MODE>
__device__ void merge_role(const Shape& s, const StepIO& io, const Work& w, int bg, MergeLds& L) {
  constexpr int PST = kPartStride(D);
  constexpr bool DENSE = MODE == kModeDense;
  constexpr int SLOT = (DENSE ? 1 : 2) * PST;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = DENSE ? M : min(min(ld_c(io.num_selected + bg), s.kmax), M);
  const bool comp = !DENSE && io.compensate && kk < M;
  const int nch = comp ? s.n_chunks : 0;
  const int nsp = MODE == kModeFused ? s.n_slices : s.n_splits;
  const float* cp = w.cpart + (size_t)bg * s.n_chunks * G * PST;
  const float* gp = w.gpart + (size_t)bg * nsp * G * SLOT;
  float* f_ch = L.f;                    // [G][nch]
  float* f_ex = L.f + G * nch;          // [G][nsp]
  float* f_sc = L.f + G * (nch + nsp);  // [G][nsp]

  for (int j = wave; j < G; j += 4) {
    float Ma = -INFINITY, Me = -INFINITY, Ms = -INFINITY;
    for (int ch = lane; ch < nch; ch += 64) Ma = fmaxf(Ma, ld_c(cp + ((size_t)ch * G + j) * PST));
    for (int sp = lane; sp < nsp; sp += 64) {
      Me = fmaxf(Me, ld_c(gp + ((size_t)sp * G + j) * SLOT));
      if (comp) Ms = fmaxf(Ms, ld_c(gp + ((size_t)sp * G + j) * SLOT + PST));
    }
    Ma = wave_max(Ma);
    Me = wave_max(Me);
    Ms = wave_max(Ms);
    float la = 0.f, le = 0.f, ls = 0.f;
    for (int ch = lane; ch < nch; ch += 64) {
      const float* h = cp + ((size_t)ch * G + j) * PST;
      const float f = scale_from(ld_c(h), Ma);
      f_ch[j * nch + ch] = f;
      la += ld_c(h + 1) * f;
    }
    for (int sp = lane; sp < nsp; sp += 64) {
      const float* h = gp + ((size_t)sp * G + j) * SLOT;
      const float f = scale_from(ld_c(h), Me);
      f_ex[j * nsp + sp] = f;
      le += ld_c(h + 1) * f;
      if (comp) {
        const float f2 = scale_from(ld_c(h + PST), Ms);
        f_sc[j * nsp + sp] = f2;
        ls += ld_c(h + PST + 1) * f2;
      }
    }
    la = wave_sum(la);
    le = wave_sum(le);
    ls = wave_sum(ls);
    if (lane == 0) {
      const float fs = scale_from(Ms, Ma);  // selected terms in the all-block frame (Ms <= Ma)
      float lo = comp ? la - ls * fs : 0.f;
      if (lo < 0.f) lo = 0.f;              // omitted mass below the rounding of the selected mass
      const float Mo = comp ? Ma : -INFINITY;
      const float Mx = fmaxf(Me, Mo);
      const float fe = scale_from(Me, Mx), fo = scale_from(Mo, Mx);
      L.head[j][0] = fe;
      L.head[j][1] = fo;
      L.head[j][2] = fs;
      L.head[j][3] = le * fe + lo * fo;
      L.head[j][4] = Mx;
    }
  }
  __syncthreads();
  for (int o = tid; o < G * D; o += kThreads) {
    const int j = o / D, d = o % D;
    float ae = 0.f;
#pragma unroll 16
    for (int sp = 0; sp < nsp; ++sp) ae = fmaf(ld_c(gp + ((size_t)sp * G + j) * SLOT + 4 + d), f_ex[j * nsp + sp], ae);
    float ao = 0.f;
    if (comp) {
      float aa = 0.f, as = 0.f;
#pragma unroll 16
      for (int ch = 0; ch < nch; ++ch) aa = fmaf(ld_c(cp + ((size_t)ch * G + j) * PST + 4 + d), f_ch[j * nch + ch], aa);
#pragma unroll 16
      for (int sp = 0; sp < nsp; ++sp)
        as = fmaf(ld_c(gp + ((size_t)sp * G + j) * SLOT + PST + 4 + d), f_sc[j * nsp + sp], as);
      ao = aa - as * L.head[j][2];
    }
    const float den = L.head[j][3];
    const int h = g * G + j;
    const size_t oi = ((size_t)b * s.Hq + h) * D + d;
    io.out[oi] = den > 0.f ? (ae * L.head[j][0] + ao * L.head[j][1]) / den : 0.f;
    if (io.lse && d == 0) io.lse[(size_t)b * s.Hq + h] = den > 0.f ? L.head[j][4] + logf(den) : -INFINITY;
  }
  if (tid == 0) {
    st_c(ctr_merge(w, bg), 0u);
    if (MODE == kModeFused) {
      st_c(ctr_scan_a(w, bg), 0u);
      st_c(ctr_select(w, bg), 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// The step kernel.  blockIdx.x: [scans][slices] (fused), [scans], [slices]
// or [gathers], by mode.
// ---------------------------------------------------------------------------
template <typename KV, int D, int G, int MODE>
__global__ __launch_bounds__(kThreads) void step_kernel(Shape s, StepIO io, Work w, int n_scan) {
  __shared__ StepLds<D, G> lds;
  __shared__ int share[kShareMax];
  __shared__ uint32_t slot;
  const int t = (int)blockIdx.x;
  int merge_bg = -1;
  if (MODE == kModeFused) {
    if (t < n_scan) merge_bg = scan_role<KV, D, G, MODE>(s, io, w, t, lds.scan, &slot);
    else merge_bg = slice_role<KV, D, G, MODE>(s, io, w, t - n_scan, lds, share, &slot);
  } else if (MODE == kModeScanOnly) {
    scan_role<KV, D, G, MODE>(s, io, w, t, lds.scan, &slot);
  } else if (MODE == kModeSelectOnly) {
    slice_role<KV, D, G, MODE>(s, io, w, t, lds, share, &slot);
  } else {
    merge_bg = gather_role<KV, D, G, MODE>(s, io, w, t, lds.gath, share, &slot);
  }
  if (merge_bg >= 0) {
    __syncthreads();
    merge_role<D, G, MODE>(s, io, w, merge_bg, lds.merge);
  }
}

}  // namespace

// ---- launchers --------------------------------------------------------------

hipError_t launch_build_summaries(const Shape& s, const void* k_cache, const void* v_cache,
                                  const int32_t* bt, const int32_t* sl, int append_only,
                                  const Summ& o, hipStream_t st) {
  const int LPR = s.D / 8;
  int threads = ((s.Hkv * LPR + 63) / 64) * 64;
  threads = threads > kThreads ? kThreads : threads;
  const dim3 grid(append_only ? s.B : s.B * s.max_blocks);
  const size_t lds = (size_t)s.Hkv * s.D * sizeof(float);
#define CKV_SUMM(KV, DD)                                                                        \
  hipLaunchKernelGGL((summary_kernel<KV, DD>), grid, dim3(threads), lds, st, s,                 \
                     (const KV*)k_cache, (const KV*)v_cache, bt, sl, append_only, (KV*)o.mean_k, \
                     (KV*)o.mean_v, o.gvar, o.count)
  if (s.dtype == 0) {
    if (s.D == 128) CKV_SUMM(uint16_t, 128); else CKV_SUMM(uint16_t, 64);
  } else {
    if (s.D == 128) CKV_SUMM(float, 128); else CKV_SUMM(float, 64);
  }
#undef CKV_SUMM
  return hipGetLastError();
}

// Calls f(kernel) with the step-kernel instance for (dtype, D, G) in MODE.
template <int MODE, class F>
static auto with_kernel(const Shape& s, F&& f) {
#define CKV_G(KV, DD)                                                  \
  switch (s.G) {                                                       \
    case 1: return f(&step_kernel<KV, DD, 1, MODE>);                   \
    case 2: return f(&step_kernel<KV, DD, 2, MODE>);                   \
    case 4: return f(&step_kernel<KV, DD, 4, MODE>);                   \
    default: return f(&step_kernel<KV, DD, 8, MODE>);                  \
  }
  if (s.dtype == 0) {
    if (s.D == 128) { CKV_G(uint16_t, 128) } else { CKV_G(uint16_t, 64) }
  } else {
    if (s.D == 128) { CKV_G(float, 128) } else { CKV_G(float, 64) }
  }
#undef CKV_G
}

int waiting_workgroups(const Shape& s, int mode) {
  return mode == kModeFused ? s.B * s.Hkv * s.n_slices : 0;
}

int resident_workgroups(const Shape& s, int mode) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  auto occ = [&](auto fn) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, 0) != hipSuccess) n = 0;
    return n;
  };
  switch (mode) {
    case kModeFused: per_cu = with_kernel<kModeFused>(s, occ); break;
    case kModeScanOnly: per_cu = with_kernel<kModeScanOnly>(s, occ); break;
    case kModeSelectOnly: per_cu = with_kernel<kModeSelectOnly>(s, occ); break;
    case kModeAttendOnly: per_cu = with_kernel<kModeAttendOnly>(s, occ); break;
    default: per_cu = with_kernel<kModeDense>(s, occ); break;
  }
  return per_cu * cus;
}

template <int MODE>
static hipError_t launch_mode(const Shape& s, const StepIO& io, const Work& w, hipStream_t st) {
  const int bgs = s.B * s.Hkv;
  const int n_scan = (MODE == kModeFused || MODE == kModeScanOnly) ? bgs * s.n_chunks : 0;
  const int n_rest = MODE == kModeScanOnly ? 0
                     : (MODE == kModeFused || MODE == kModeSelectOnly) ? bgs * s.n_slices
                                                                       : bgs * s.n_splits;
  const dim3 grid(n_scan + n_rest);
  return with_kernel<MODE>(s, [&](auto fn) {
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), 0, st, s, io, w, n_scan);
    return hipGetLastError();
  });
}

hipError_t launch_step(const Shape& s, int mode, const StepIO& io, const Work& w, hipStream_t st) {
  switch (mode) {
    case kModeFused: return launch_mode<kModeFused>(s, io, w, st);
    case kModeScanOnly: return launch_mode<kModeScanOnly>(s, io, w, st);
    case kModeSelectOnly: return launch_mode<kModeSelectOnly>(s, io, w, st);
    case kModeAttendOnly: return launch_mode<kModeAttendOnly>(s, io, w, st);
    default: return launch_mode<kModeDense>(s, io, w, st);
  }
}

}  // namespace ckv

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
// One launch runs a whole decode step.  Workgroups take a ticket from an
// atomic counter and the ticket decides the role:
//   scan    (sequence, KV head, chunk of 256 blocks): pass A reads the mean
//           keys and grouped variances, computes block-mean logits on the
//           matrix cores (the G query heads of the KV head are the rows of
//           a 16x16x32 bf16 MFMA tile) and the log-scores; pass B streams the
//           mean values and accumulates the compensation sums of all blocks.
//   select  (sequence, KV head, slice of 1024 blocks): waits for pass A of
//           its KV head, forms the ranked score of each block and keeps the
//           slice's top-k; the last slice merges the candidates.
//   gather  (sequence, KV head, split of the selected blocks): waits for the
//           selection and attends exactly to the selected tokens; it also
//           forms the selected blocks' own compensation terms, which the
//           merge removes from the all-block sums.
//   merge   run by whichever workgroup arrives last for its (sequence, KV
//           head): log-sum-exp combination into the output.
// A workgroup only ever waits for workgroups with smaller tickets, which are
// already running and never wait on larger tickets, so the waits end; each
// spin is also bounded and records an error flag if the bound is hit.
// Hand-offs between workgroups use L2-coherent atomic loads and stores (see
// st_c / ld_c), ordered by s_waitcnt and the workgroup barrier.
// Selection and gather overlap pass B of the scan.

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

// Control words of the workspace.
__device__ __forceinline__ uint32_t* ctr_scan_a(const Work& w, int bg) { return w.ctrl + kCtrlHeader + 4 * bg; }
__device__ __forceinline__ uint32_t* ctr_select(const Work& w, int bg) { return w.ctrl + kCtrlHeader + 4 * bg + 1; }
__device__ __forceinline__ uint32_t* flag_selected(const Work& w, int bg) { return w.ctrl + kCtrlHeader + 4 * bg + 2; }
__device__ __forceinline__ uint32_t* ctr_merge(const Work& w, int bg) { return w.ctrl + kCtrlHeader + 4 * bg + 3; }

// Data that one workgroup hands to another within a launch goes through
// agent-scope relaxed atomic loads and stores: on gfx950 these are L2-coherent
// accesses across the eight XCDs, so no whole-cache writeback or invalidate
// (what an agent-scope fence costs) is ever needed.
template <typename T>
__device__ __forceinline__ void st_c(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_c(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until *p >= target (bounded; the bound sets the error word).
__device__ __forceinline__ void wait_at_least(uint32_t* p, uint32_t target, uint32_t* err) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (ld_c(p) < target) {
      __builtin_amdgcn_s_sleep(4);
      if (++spins == kSpinLimit) {
        st_c(err, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Count this workgroup in *p once all its coherent stores have completed;
// returns the previous count (same value in every thread).
__device__ __forceinline__ uint32_t arrive(uint32_t* p, uint32_t* slot) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) *slot = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *slot;
}

// ---------------------------------------------------------------------------
// Summary build: mean key, mean value, grouped key variance, count.
// One workgroup per (sequence, block); threads over (KV head, 8-channel slice).
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
    const size_t row = ((size_t)page * s.Hkv + g) * D + c * 8;
    store8(mk + row, mu);
    store8(mv + row, nu);
  }
  __syncthreads();
  const int gs = D / s.r;
  for (int item = threadIdx.x; item < s.Hkv * s.r; item += blockDim.x) {
    const int g = item / s.r, t = item % s.r;
    float acc = 0.f;
    for (int c = 0; c < gs; ++c) acc += var_sh[g * D + t * gs + c];
    gv[((size_t)page * s.Hkv + g) * s.r + t] = acc / (float)gs;
  }
  if (threadIdx.x == 0) cnt[page] = n;
}

// ---------------------------------------------------------------------------
// Shared memory of the step kernel: one union, each role uses its member.
// ---------------------------------------------------------------------------
template <int D, int G>
struct ScanLds {
  static constexpr int RS = kThreads / (D / 8);
  int pg[kChunk];          // page of each block of the chunk (-1: skip)
  float sb[G][kChunk];     // block-mean logit
  float vh[G][kChunk];     // estimated within-block logit variance
  float lam[G][kChunk];    // log of the ranked per-head score
  float w[G][kChunk];      // compensation weight n e^{s_bar - chunk max}
  float qn[G * D];         // |q_h restricted to channel group t|^2
  float acc[RS * D];       // row-slot sums for the final reduction
};
struct SelLds {
  uint64_t keys[kSlice];
  uint32_t hist[256];
  uint32_t bitmap[kMaxBlocks / 32];
  float lnz[8];
  float f[kSlice / kChunk][8];
  uint32_t sh[4];
  uint32_t count;
};
template <int D, int G>
struct GathLds {
  static constexpr int RS = kThreads / (D / 8);
  int pg[256];
  int n[256];
  float st[2 * RS * G];
  float acc[RS * D];
};
struct MergeLds {
  float f[kMergeFactors];
  float head[8][8];  // per head: fe, fo, fs, den, Mx
};
template <int D, int G>
union StepLds {
  ScanLds<D, G> scan;
  SelLds sel;
  GathLds<D, G> gath;
  MergeLds merge;
};

// ---------------------------------------------------------------------------
// Scan: pass A (mean keys -> scores), pass B (mean values -> compensation).
// ---------------------------------------------------------------------------
template <typename KV, int D, int G, int MODE>
__device__ int scan_role(const Shape& s, const StepIO& io, const Work& w, int t,
                         ScanLds<D, G>& L, uint32_t* slot) {
  constexpr int LPR = D / 8, RS = kThreads / LPR, PST = kPartStride(D);
  const int chunk = t % s.n_chunks, bg = t / s.n_chunks;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rs = tid / LPR, c = tid % LPR;
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int start = chunk * kChunk;
  const int nrows = max(0, min(M, start + kChunk) - start);
  const KV* q = static_cast<const KV*>(io.q) + (size_t)b * s.Hq * D;
  const KV* mk = static_cast<const KV*>(io.summ.mean_k);
  const KV* mv = static_cast<const KV*>(io.summ.mean_v);
  const float* gv = io.summ.gvar;
  const int r = s.r, gs = D / r;

  for (int i = tid; i < nrows; i += kThreads) {
    const int p = io.block_table[(size_t)b * s.max_blocks + start + i];
    L.pg[i] = (p >= 0 && p < s.P) ? p : -1;
  }
  for (int item = tid; item < G * r; item += kThreads) {
    const int j = item / r, tg = item % r;
    const KV* qh = q + (size_t)(g * G + j) * D + tg * gs;
    float a = 0.f;
    for (int cc = 0; cc < gs; ++cc) {
      const float x = load1(qh + cc);
      a = fmaf(x, x, a);
    }
    L.qn[item] = a;
  }
  __syncthreads();

  // ---- pass A: block-mean logits and variance estimates ----
  if constexpr (std::is_same<KV, uint16_t>::value) {
    // Matrix cores: D[head][row] = sum_k Q[head][k] mean_k[row][k] on
    // 16x16x32 bf16 tiles; lane l holds Q[l%16][8(l/16)..+7] of each 32-wide
    // k-slice (zero rows past G), mean_k of row l%16 at the same k, and gets
    // D[4(l/16)+i][l%16].
    constexpr int KT = D / 32;
    bf16x8_t qa[KT];
    {
      const int head = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (head < G) v = *reinterpret_cast<const uint4*>(q + (size_t)(g * G + head) * D + 32 * kt + 8 * kq);
        qa[kt] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    const bool holder = (lane >> 4) * 4 < G;  // lanes whose accumulators hold real heads
    const int ngroups = (nrows + 15) / 16;
    for (int g0 = wave; g0 < ngroups; g0 += 8) {
      uint4 bv[2][KT];
      float gpre[2][8];
      int rowi[2];
      bool ok[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int grp = g0 + 4 * u;
        rowi[u] = grp * 16 + (lane & 15);
        ok[u] = grp < ngroups && rowi[u] < nrows && L.pg[rowi[u]] >= 0;
        const size_t row = ok[u] ? ((size_t)L.pg[rowi[u]] * s.Hkv + g) : 0;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          bv[u][kt] = ok[u] ? *reinterpret_cast<const uint4*>(mk + row * D + 32 * kt + 8 * (lane >> 4))
                            : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int e = 0; e < 8; ++e) gpre[u][e] = (ok[u] && holder && e < r) ? gv[row * r + e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kt], __builtin_bit_cast(bf16x8_t, bv[u][kt]),
                                                         acc, 0, 0, 0);
        if (ok[u] && holder) {
          const int ri = rowi[u];
          const float* gvr = gv + ((size_t)L.pg[ri] * s.Hkv + g) * r;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 4 * (lane >> 4) + i;
            if (j < G) {
              float sig = 0.f;
              if (r <= 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                  if (e < r) sig = fmaf(L.qn[j * r + e], gpre[u][e], sig);
              } else {
                for (int e = 0; e < r; ++e) sig = fmaf(L.qn[j * r + e], gvr[e], sig);
              }
              L.sb[j][ri] = acc[i] * s.tau;
              L.vh[j][ri] = sig * s.tau2;
            }
          }
        }
      }
    }
  } else {
    // f32 storage: vector ALU, D/8 lanes per row.
    float qv[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) load8(q + (size_t)(g * G + j) * D + c * 8, qv[j]);
    for (int ri = rs; ri < nrows; ri += RS) {
      if (L.pg[ri] < 0) continue;  // uniform across the row's lanes
      const size_t row = (size_t)L.pg[ri] * s.Hkv + g;
      float mu8[8], dot[G], sig[G];
      load8(mk + row * D + c * 8, mu8);
      dot8<G>(qv, mu8, dot);
#pragma unroll
      for (int j = 0; j < G; ++j) sig[j] = 0.f;
      for (int e = c; e < r; e += LPR) {
        const float gve = gv[row * r + e];
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
      if (L.pg[ri] < 0) { L.lam[j][ri] = -INFINITY; continue; }
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
      float wt = 0.f, x = 0.f;
      if (L.pg[ri] >= 0) {
        const int n = min(s.bs, Lseq - (start + ri) * s.bs);
        wt = (float)n * expf(L.sb[j][ri] - mx);
        lsum += wt;
        zsum = fmaf(wt, 1.f + 0.5f * L.vh[j][ri], zsum);
        const float lam = L.lam[j][ri];
        x = lam == -INFINITY ? 0.f : expf(lam - cx);
      }
      L.w[j][ri] = wt;
      st_c(&xrow[ri], x);
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
  if (MODE == kModeFused || MODE == kModeSelectOnly) arrive(ctr_scan_a(w, bg), slot);
  else __syncthreads();

  // ---- pass B: compensation sums over the chunk's mean values ----
  float acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  constexpr int UB = 4;
  for (int base = 0; base < nrows; base += RS * UB) {
    float nu[UB][8];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int ri = base + u * RS + rs;
      if (ri < nrows && L.pg[ri] >= 0) {
        load8(mv + ((size_t)L.pg[ri] * s.Hkv + g) * D + c * 8, nu[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) nu[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int ri = base + u * RS + rs;
      if (ri < nrows) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float wt = L.w[j][ri];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(wt, nu[u][e], acc[j][e]);
        }
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
      st_c(&part[(size_t)j * PST + 4 + d], a);
    }
    __syncthreads();
  }
  if (MODE == kModeFused) {
    const uint32_t prev = arrive(ctr_merge(w, bg), slot);
    return prev == (uint32_t)(s.n_chunks + s.n_splits - 1) ? bg : -1;
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
// Candidate keys of all slices: slice s holds its kk keys at s * stride.
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

// ---------------------------------------------------------------------------
// Select: ranked score S_i = sum_h S_{h,i} / Z_hat_h of every block of the
// slice, slice top-k, and (last slice) the global top-k in ascending order.
// ---------------------------------------------------------------------------
template <int D, int G, int MODE>
__device__ void select_role(const Shape& s, const StepIO& io, const Work& w, int t, SelLds& L,
                            uint32_t* slot) {
  constexpr int PST = kPartStride(D);
  const int slice = t % s.n_slices, bg = t / s.n_slices;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  wait_at_least(ctr_scan_a(w, bg), (uint32_t)s.n_chunks, w.ctrl + 2);

  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = min(M, s.kmax);
  const float* parts = w.cpart + (size_t)bg * s.n_chunks * G * PST;

  // log Z_hat per query head: Z_hat = sum over chunks of z e^{max s_bar}
  for (int j = wave; j < G; j += 4) {
    float mz = -INFINITY;
    for (int ch = lane; ch < s.n_chunks; ch += 64) mz = fmaxf(mz, ld_c(parts + ((size_t)ch * G + j) * PST));
    mz = wave_max(mz);
    float zs = 0.f;
    for (int ch = lane; ch < s.n_chunks; ch += 64) {
      const float* h = parts + ((size_t)ch * G + j) * PST;
      zs += ld_c(h + 2) * scale_from(ld_c(h), mz);
    }
    zs = wave_sum(zs);
    if (lane == 0) L.lnz[j] = zs > 0.f ? mz + logf(zs) : -INFINITY;
  }
  __syncthreads();
  const int i0 = slice * kSlice;
  const int nloc = max(0, min(M, i0 + kSlice) - i0);
  constexpr int CPS = kSlice / kChunk;
  for (int item = tid; item < CPS * G; item += kThreads) {
    const int cc = item / G, j = item % G;
    const int ch = i0 / kChunk + cc;
    const float cmax = ch < s.n_chunks ? ld_c(parts + ((size_t)ch * G + j) * PST + 3) : -INFINITY;
    L.f[cc][j] = (cmax == -INFINITY || L.lnz[j] == -INFINITY) ? 0.f : expf(cmax - L.lnz[j]);
  }
  __syncthreads();
  for (int i = tid; i < nloc; i += kThreads) {
    const int ib = i0 + i, cc = i / kChunk;
    float S = 0.f;
#pragma unroll
    for (int j = 0; j < G; ++j)
      S = fmaf(ld_c(w.xs + ((size_t)b * s.Hq + g * G + j) * s.max_blocks + ib), L.f[cc][j], S);
    L.keys[i] = make_key(S, ib);
    if (io.group_scores) io.group_scores[(size_t)bg * s.max_blocks + ib] = S;
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
  if (prev != (uint32_t)(s.n_slices - 1)) return;

  // ---- last slice of this (sequence, KV head): global top-k ----
  int32_t* out = io.selected + (size_t)bg * s.kmax;
  if (tid == 0) st_c(io.num_selected + bg, (int32_t)kk);
  for (int e = kk + tid; e < s.kmax; e += kThreads) st_c(out + e, (int32_t)-1);
  if (kk == M) {
    for (int i = tid; i < M; i += kThreads) st_c(out + i, (int32_t)i);
  } else if (kk > 0) {
    const int n2 = s.n_slices * kk;
    const SliceKeys key2{w.cand + (size_t)bg * s.n_slices * s.kmax, kk, s.kmax};
    const uint64_t T = radix_kth_largest(key2, n2, kk, L.hist, L.sh);
    const int words = (M + 31) / 32;
    for (int e = tid; e < words; e += kThreads) L.bitmap[e] = 0u;
    __syncthreads();
    for (int e = tid; e < n2; e += kThreads) {
      const uint64_t key = key2(e);
      if (key >= T) {
        const int i = key_index(key);
        atomicOr(&L.bitmap[i >> 5], 1u << (i & 31));
      }
    }
    __syncthreads();
    // ascending order: prefix sums of the bitmap's popcounts
    const int per = (words + kThreads - 1) / kThreads;
    const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
    uint32_t cnt = 0;
    for (int e = w0; e < w1; ++e) cnt += __popc(L.bitmap[e]);
    // block exclusive scan of cnt
    uint32_t inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) L.hist[wave] = inc;
    __syncthreads();
    uint32_t base = 0;
    for (int v = 0; v < wave; ++v) base += L.hist[v];
    uint32_t pos = base + inc - cnt;
    for (int e = w0; e < w1; ++e) {
      uint32_t bits = L.bitmap[e];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        st_c(out + pos, (int32_t)(32 * e + bit));
        ++pos;
      }
    }
  }
  // reset this (sequence, KV head)'s select counters for the next launch
  if (tid == 0) {
    st_c(ctr_scan_a(w, bg), 0u);
    st_c(ctr_select(w, bg), 0u);
  }
  if (MODE == kModeFused) {
    __builtin_amdgcn_s_waitcnt(0);  // the selection is stored before the flag goes up
    __syncthreads();
    if (tid == 0) st_c(flag_selected(w, bg), 1u);
  }
}

// ---------------------------------------------------------------------------
// Gather: exact attention over a split of the selected blocks (every block,
// for the dense baseline) and the selected blocks' compensation terms.
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

template <typename KV, int D, int G, int MODE>
__device__ int gather_role(const Shape& s, const StepIO& io, const Work& w, int t, GathLds<D, G>& L,
                           uint32_t* slot) {
  constexpr int LPR = D / 8, RS = kThreads / LPR, PST = kPartStride(D);
  constexpr bool DENSE = MODE == kModeDense;
  const int split = t % s.n_splits, bg = t / s.n_splits;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, rs = tid / LPR, c = tid % LPR;
  if (MODE == kModeFused) wait_at_least(flag_selected(w, bg), 1u, w.ctrl + 2);

  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = DENSE ? M : min(min(ld_c(io.num_selected + bg), s.kmax), M);
  const int PPS = s.pages_per_split;
  const int first = split * PPS;
  const int nb = max(0, min(kk, first + PPS) - first);
  for (int e = tid; e < nb; e += kThreads) {
    const int i = DENSE ? first + e : ld_c(io.selected + (size_t)bg * s.kmax + first + e);
    int p = -1, n = 0;
    if (i >= 0 && i < M) {
      p = io.block_table[(size_t)b * s.max_blocks + i];
      if (p < 0 || p >= s.P) p = -1;
      else n = min(s.bs, Lseq - i * s.bs);
    }
    L.pg[e] = p;
    L.n[e] = n;
  }
  __syncthreads();

  const KV* q = static_cast<const KV*>(io.q) + (size_t)b * s.Hq * D;
  const KV* kc = static_cast<const KV*>(io.k_cache);
  const KV* vc = static_cast<const KV*>(io.v_cache);
  float qv[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) load8(q + (size_t)(g * G + j) * D + c * 8, qv[j]);

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  constexpr int UG = 4;
  const int nrows = nb * kBlockSize;
  for (int base = 0; base < nrows; base += RS * UG) {
    float k8[UG][8], v8[UG][8];
    bool ok[UG];
#pragma unroll
    for (int u = 0; u < UG; ++u) {
      const int R = base + u * RS + rs;
      const int bl = R / kBlockSize, tok = R % kBlockSize;
      ok[u] = R < nrows && L.pg[bl] >= 0 && tok < L.n[bl];
      if (ok[u]) {
        const size_t off = (((size_t)L.pg[bl] * s.Hkv + g) * s.bs + tok) * D + c * 8;
        load8(kc + off, k8[u]);
        load8(vc + off, v8[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < UG; ++u) {
      if (ok[u]) {  // uniform across the row's lanes
        float dot[G];
        dot8<G>(qv, k8[u], dot);
#pragma unroll
        for (int j = 0; j < G; ++j) online_add<G>(m, l, acc, j, group_sum<LPR>(dot[j]) * s.tau, 1.f, v8[u]);
      }
    }
  }
  constexpr int SLOT = (DENSE ? 1 : 2) * PST;
  float* base_part = w.gpart + ((size_t)bg * s.n_splits + split) * G * SLOT;
  combine_online<D, G, RS>(m, l, acc, base_part, SLOT, L.st, L.acc);

  if (!DENSE) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
    }
    if (io.compensate) {
      const KV* mk = static_cast<const KV*>(io.summ.mean_k);
      const KV* mv = static_cast<const KV*>(io.summ.mean_v);
      for (int bl = rs; bl < nb; bl += RS) {
        if (L.pg[bl] < 0) continue;
        const size_t row = ((size_t)L.pg[bl] * s.Hkv + g) * D + c * 8;
        float mu8[8], nu8[8], dot[G];
        load8(mk + row, mu8);
        load8(mv + row, nu8);
        dot8<G>(qv, mu8, dot);
        const float fn = (float)L.n[bl];
#pragma unroll
        for (int j = 0; j < G; ++j) online_add<G>(m, l, acc, j, group_sum<LPR>(dot[j]) * s.tau, fn, nu8);
      }
    }
    combine_online<D, G, RS>(m, l, acc, base_part + PST, SLOT, L.st, L.acc);
  }
  const uint32_t target = MODE == kModeFused ? (uint32_t)(s.n_chunks + s.n_splits) : (uint32_t)s.n_splits;
  const uint32_t prev = arrive(ctr_merge(w, bg), slot);
  return prev == target - 1 ? bg : -1;
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
  const int nch = comp ? s.n_chunks : 0, nsp = s.n_splits;
  const float* cp = w.cpart + (size_t)bg * s.n_chunks * G * PST;
  const float* gp = w.gpart + (size_t)bg * s.n_splits * G * SLOT;
  float* f_ch = L.f;                  // [G][nch]
  float* f_ex = L.f + G * nch;        // [G][nsp]
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
#pragma unroll 8
    for (int sp = 0; sp < nsp; ++sp) ae = fmaf(ld_c(gp + ((size_t)sp * G + j) * SLOT + 4 + d), f_ex[j * nsp + sp], ae);
    float ao = 0.f;
    if (comp) {
      float aa = 0.f, as = 0.f;
#pragma unroll 8
      for (int ch = 0; ch < nch; ++ch) aa = fmaf(ld_c(cp + ((size_t)ch * G + j) * PST + 4 + d), f_ch[j * nch + ch], aa);
#pragma unroll 8
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
    if (MODE == kModeFused) st_c(flag_selected(w, bg), 0u);
  }
}

// ---------------------------------------------------------------------------
// The step kernel.
// ---------------------------------------------------------------------------
template <typename KV, int D, int G, int MODE>
__global__ __launch_bounds__(kThreads) void step_kernel(Shape s, StepIO io, Work w, int n_scan,
                                                        int n_sel) {
  __shared__ StepLds<D, G> lds;
  __shared__ uint32_t slot;
  if (threadIdx.x == 0) slot = __hip_atomic_fetch_add(w.ctrl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int t = (int)slot;
  __syncthreads();
  int merge_bg = -1;
  if (MODE == kModeFused || MODE == kModeSelectOnly) {
    if (t < n_scan) merge_bg = scan_role<KV, D, G, MODE>(s, io, w, t, lds.scan, &slot);
    else if (t < n_scan + n_sel) select_role<D, G, MODE>(s, io, w, t - n_scan, lds.sel, &slot);
    else if (MODE == kModeFused) merge_bg = gather_role<KV, D, G, MODE>(s, io, w, t - n_scan - n_sel, lds.gath, &slot);
  } else {
    merge_bg = gather_role<KV, D, G, MODE>(s, io, w, t, lds.gath, &slot);
  }
  if (merge_bg >= 0) {
    __syncthreads();
    merge_role<D, G, MODE>(s, io, w, merge_bg, lds.merge);
  }
  // the last workgroup resets the ticket and completion counters
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t done = __hip_atomic_fetch_add(w.ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      st_c(w.ctrl, 0u);
      st_c(w.ctrl + 1, 0u);
    }
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

template <int MODE>
static void launch_mode(const Shape& s, const StepIO& io, const Work& w, hipStream_t st) {
  const int bgs = s.B * s.Hkv;
  const int n_scan = (MODE == kModeFused || MODE == kModeSelectOnly) ? bgs * s.n_chunks : 0;
  const int n_sel = (MODE == kModeFused || MODE == kModeSelectOnly) ? bgs * s.n_slices : 0;
  const int n_gath = (MODE == kModeSelectOnly) ? 0 : bgs * s.n_splits;
  const dim3 grid(n_scan + n_sel + n_gath);
#define CKV_STEP(KV, DD, GG) \
  hipLaunchKernelGGL((step_kernel<KV, DD, GG, MODE>), grid, dim3(kThreads), 0, st, s, io, w, n_scan, n_sel)
#define CKV_G(KV, DD)                   \
  switch (s.G) {                        \
    case 1: CKV_STEP(KV, DD, 1); break; \
    case 2: CKV_STEP(KV, DD, 2); break; \
    case 4: CKV_STEP(KV, DD, 4); break; \
    default: CKV_STEP(KV, DD, 8); break; \
  }
  if (s.dtype == 0) {
    if (s.D == 128) { CKV_G(uint16_t, 128) } else { CKV_G(uint16_t, 64) }
  } else {
    if (s.D == 128) { CKV_G(float, 128) } else { CKV_G(float, 64) }
  }
#undef CKV_G
#undef CKV_STEP
}

hipError_t launch_step(const Shape& s, int mode, const StepIO& io, const Work& w, hipStream_t st) {
  switch (mode) {
    case kModeFused: launch_mode<kModeFused>(s, io, w, st); break;
    case kModeSelectOnly: launch_mode<kModeSelectOnly>(s, io, w, st); break;
    case kModeAttendOnly: launch_mode<kModeAttendOnly>(s, io, w, st); break;
    default: launch_mode<kModeDense>(s, io, w, st); break;
  }
  return hipGetLastError();
}

}  // namespace ckv

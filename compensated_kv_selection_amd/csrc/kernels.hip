// CompKV decode-step kernels for gfx950 (MI355X): summary build, block
// scoring scan, top-k selection, split-K gather attention, and the
// log-sum-exp merge that folds in Mean compensation.
//
// The method (CompKV abstract, shd-paper.top listing; CompKV review,
// evolve.pub, "Summary" and FAQ): keys and values are split into blocks;
// every block keeps its mean key, grouped key variance and mean value; blocks
// are ranked by a practical residual score (second-order mass estimate times
// the estimated within-block logit variance, paper Section 3, Eqs. 4-7); the
// top-k blocks are attended exactly and every omitted block enters the
// softmax with its block-mean logit, weighted by its token count, carrying
// its mean value.
//
// Work mapping shared by the scan and the gather: a "row" is one
// (block-or-token, KV head) vector of d elements; D/8 consecutive lanes own a
// row, each lane 8 consecutive elements (16-byte loads of bf16).  A
// workgroup of 256 lanes holds 256/(D/8) row slots.  Each lane keeps the G
// query heads of its KV head (GQA packing) for its 8 elements in registers,
// so one pass over a row serves all G heads.

#include "device.hpp"
#include "internal.hpp"

namespace ckv {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

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
// Scan: score every block from its summary and accumulate, over all blocks,
// the partial sums that compensation and the normalizer Z_hat need.
// One workgroup per (sequence, KV head, chunk of kScanChunk blocks).
// ---------------------------------------------------------------------------
template <typename KV, int D, int G>
__device__ __forceinline__ void load_q(const Shape& s, const KV* __restrict__ q, int b, int g, int c,
                                       float (&qv)[G][8]) {
#pragma unroll
  for (int j = 0; j < G; ++j) load8(q + ((size_t)b * s.Hq + g * G + j) * D + c * 8, qv[j]);
}

// Write per-head partial states of all row slots, combined, to `part`
// (stride `slot` floats between heads): [max, sum l, sum z, 0, acc[D]].
template <int D, int G, int RS>
__device__ __forceinline__ void combine_rows(const float (&m)[G], const float (&l)[G],
                                             const float (&z)[G], const float (&acc)[G][8],
                                             float* part, int slot, float* sm_state,
                                             float* sm_acc) {
  constexpr int LPR = D / 8;
  const int tid = threadIdx.x, rs = tid / LPR, c = tid % LPR;
  float* sm_m = sm_state;
  float* sm_l = sm_state + RS * G;
  float* sm_z = sm_state + 2 * RS * G;
  if (c == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      sm_m[rs * G + j] = m[j];
      sm_l[rs * G + j] = l[j];
      sm_z[rs * G + j] = z[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float Mj = -INFINITY;
    for (int r2 = 0; r2 < RS; ++r2) Mj = fmaxf(Mj, sm_m[r2 * G + j]);
    const float f = scale_from(m[j], Mj);
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[rs * D + c * 8 + e] = acc[j][e] * f;
    __syncthreads();
    float* pj = part + (size_t)j * slot;
    for (int t = tid; t < D; t += blockDim.x) {
      float a = 0.f;
      for (int r2 = 0; r2 < RS; ++r2) a += sm_acc[r2 * D + t];
      pj[4 + t] = a;
    }
    if (tid == 0) {
      float ls = 0.f, zs = 0.f;
      for (int r2 = 0; r2 < RS; ++r2) {
        const float f2 = scale_from(sm_m[r2 * G + j], Mj);
        ls += sm_l[r2 * G + j] * f2;
        zs += sm_z[r2 * G + j] * f2;
      }
      pj[0] = Mj;
      pj[1] = ls;
      pj[2] = zs;
      pj[3] = 0.f;
    }
    __syncthreads();
  }
}

template <typename KV, int D, int G>
__global__ __launch_bounds__(kThreads) void scan_kernel(
    Shape s, const KV* __restrict__ q, const KV* __restrict__ mk, const KV* __restrict__ mv,
    const float* __restrict__ gv, const int32_t* __restrict__ bt, const int32_t* __restrict__ sl,
    int mode, float* __restrict__ comp, float* __restrict__ lam) {
  constexpr int LPR = D / 8, RS = kThreads / LPR;
  __shared__ float qn_sh[G * D];  // |q_h restricted to group t|^2, [G][r]
  __shared__ float sm_state[3 * RS * G];
  __shared__ float sm_acc[RS * D];

  const int chunk = blockIdx.x % s.n_chunks;
  const int bg = blockIdx.x / s.n_chunks;
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int L = clamp_len(sl[b], s.max_blocks * s.bs);
  const int M = (L + s.bs - 1) / s.bs;
  const int start = chunk * kScanChunk, end = min(M, start + kScanChunk);
  const int tid = threadIdx.x, rs = tid / LPR, c = tid % LPR;

  float qv[G][8];
  load_q<KV, D, G>(s, q, b, g, c, qv);
  const int gs = D / s.r;
  for (int item = tid; item < G * s.r; item += kThreads) {
    const int j = item / s.r, t = item % s.r;
    const KV* qh = q + ((size_t)b * s.Hq + g * G + j) * D + t * gs;
    float a = 0.f;
    for (int cc = 0; cc < gs; ++cc) {
      const float x = load1(qh + cc);
      a = fmaf(x, x, a);
    }
    qn_sh[item] = a;
  }
  __syncthreads();

  float m[G], l[G], z[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY; l[j] = 0.f; z[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }

  for (int i = start + rs; i < end; i += RS) {
    const int page = bt[(size_t)b * s.max_blocks + i];
    if (page < 0 || page >= s.P) continue;  // uniform across the row's lanes
    const int n = min(s.bs, L - i * s.bs);
    const size_t row = ((size_t)page * s.Hkv + g) * D + c * 8;
    float mu8[8], nu8[8];
    load8(mk + row, mu8);
    load8(mv + row, nu8);
    float dot[G], sig[G];
    dot8<G>(qv, mu8, dot);
#pragma unroll
    for (int j = 0; j < G; ++j) sig[j] = 0.f;
    const float* gvr = gv + ((size_t)page * s.Hkv + g) * s.r;
    for (int t = c; t < s.r; t += LPR) {
      const float gvt = gvr[t];
#pragma unroll
      for (int j = 0; j < G; ++j) sig[j] = fmaf(qn_sh[j * s.r + t], gvt, sig[j]);
    }
    const float fn = (float)n;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float sbar = group_sum<LPR>(dot[j]) * s.tau;       // block-mean logit
      const float vh = group_sum<LPR>(sig[j]) * s.tau2;        // estimated logit variance
      const float half = 0.5f * vh;
      const float massf = fn * (1.f + half);                   // A / e^{s_bar}
      const float lv = (mode == kScoreMass) ? sbar + logf(massf) : sbar + logf(massf * half);
      if (c == 0) lam[((size_t)b * s.Hq + g * G + j) * s.max_blocks + i] = lv;
      if (sbar > m[j]) {
        const float sc = scale_from(m[j], sbar);
        l[j] *= sc; z[j] *= sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] *= sc;
        m[j] = sbar;
      }
      const float w = fn * expf(sbar - m[j]);
      l[j] += w;
      z[j] = fmaf(w, 1.f + half, z[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(w, nu8[e], acc[j][e]);
    }
  }
  float* part = comp + ((size_t)bg * s.n_chunks + chunk) * G * kPartStride(D);
  combine_rows<D, G, RS>(m, l, z, acc, part, kPartStride(D), sm_state, sm_acc);
}

// ---------------------------------------------------------------------------
// Select: per (sequence, KV head), the ranked score of every block
//   S_i = sum over the group's heads of exp(lam_{h,i} - log Z_hat_h)
// and the k largest by radix select on the float bits (S >= 0, so the bits
// order like the values), ties to the lower block id, ascending output.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan of one value per thread over the workgroup; also the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wave_tot, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < kSelWaves ? wave_tot[lane] : 0u;
    t = wave_incl_scan(t, lane);
    if (lane < kSelWaves) wave_tot[lane] = t;
  }
  __syncthreads();
  const uint32_t base = wave ? wave_tot[wave - 1] : 0u;
  total = wave_tot[kSelWaves - 1];
  __syncthreads();
  return base + inc - v;
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    Shape s, const int32_t* __restrict__ sl, const float* __restrict__ comp,
    const float* __restrict__ lam, int32_t* __restrict__ sel, int32_t* __restrict__ nsel,
    float* __restrict__ gscores, int D) {
  extern __shared__ uint32_t keys[];  // [max_blocks] float bits of S
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[kSelWaves];
  __shared__ float lnz[G];
  __shared__ uint32_t sh_digit, sh_above;

  const int bg = blockIdx.x;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = clamp_len(sl[b], s.max_blocks * s.bs);
  const int M = (L + s.bs - 1) / s.bs;
  const int kk = min(M, s.kmax);
  int32_t* out = sel + (size_t)bg * s.kmax;
  if (tid == 0) nsel[bg] = kk;
  for (int e = kk + tid; e < s.kmax; e += kSelThreads) out[e] = -1;

  // log Z_hat per query head of the group, from the scan's chunk partials.
  const int PST = D + 4;
  if (wave < G) {
    const float* base = comp + (size_t)bg * s.n_chunks * G * PST + wave * PST;
    float mx = -INFINITY;
    for (int ch = lane; ch < s.n_chunks; ch += 64) mx = fmaxf(mx, base[(size_t)ch * G * PST]);
    mx = wave_max(mx);
    float zs = 0.f;
    for (int ch = lane; ch < s.n_chunks; ch += 64) {
      const float* p = base + (size_t)ch * G * PST;
      zs += p[2] * scale_from(p[0], mx);
    }
    zs = wave_sum(zs);
    if (lane == 0) lnz[wave] = zs > 0.f ? mx + logf(zs) : -INFINITY;
  }
  __syncthreads();

  for (int i = tid; i < M; i += kSelThreads) {
    float S = 0.f;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float lv = lam[((size_t)b * s.Hq + g * G + j) * s.max_blocks + i];
      S += (lv == -INFINITY) ? 0.f : expf(lv - lnz[j]);
    }
    keys[i] = __float_as_uint(S);
    if (gscores) gscores[(size_t)bg * s.max_blocks + i] = S;
  }
  __syncthreads();
  if (kk == 0) return;
  if (kk == M) {
    for (int i = tid; i < M; i += kSelThreads) out[i] = i;
    return;
  }

  // Radix select of the kk-th largest key, 8 bits at a time from the top.
  uint32_t prefix = 0u, pmask = 0u, krem = (uint32_t)kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int e = tid; e < 256; e += kSelThreads) hist[e] = 0u;
    __syncthreads();
    for (int i = tid; i < M; i += kSelThreads) {
      const uint32_t key = keys[i];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t cs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) cs[e] = hist[255 - 4 * lane - e];  // descending bins
      const uint32_t loc = cs[0] + cs[1] + cs[2] + cs[3];
      uint32_t cum = wave_incl_scan(loc, lane) - loc;              // keys in higher bins
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (cum < krem && cum + cs[e] >= krem) {
          sh_digit = 255u - 4u * lane - e;
          sh_above = cum;
        }
        cum += cs[e];
      }
    }
    __syncthreads();
    krem -= sh_above;
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // prefix = the kk-th largest key T; take every key > T and the krem lowest
  // block ids among keys == T.
  const uint32_t T = prefix;
  const int per = (M + kSelThreads - 1) / kSelThreads;
  const int lo = min(M, tid * per), hi = min(M, lo + per);
  uint32_t eq = 0;
  for (int i = lo; i < hi; ++i) eq += (keys[i] == T);
  uint32_t tot;
  uint32_t eq_rank = block_excl_scan(eq, wave_tot, tot);
  uint32_t take = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = keys[i];
    if (key > T) ++take;
    else if (key == T) { take += (eq_rank < krem); ++eq_rank; }
  }
  uint32_t pos = block_excl_scan(take, wave_tot, tot);
  eq_rank -= eq;
  for (int i = lo; i < hi; ++i) {
    const uint32_t key = keys[i];
    bool t = false;
    if (key > T) t = true;
    else if (key == T) { t = eq_rank < krem; ++eq_rank; }
    if (t) out[pos++] = i;
  }
}

// ---------------------------------------------------------------------------
// Gather: exact attention over a slice of the selected blocks (or, for the
// dense baseline, of all blocks), and - for compensation - the selected
// blocks' own block-mean terms, which the merge removes from the all-block
// compensation sum of the scan.
// One workgroup per (sequence, KV head, split).
// ---------------------------------------------------------------------------
template <typename KV, int D, int G, bool DENSE>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    Shape s, const KV* __restrict__ q, const KV* __restrict__ kc, const KV* __restrict__ vc,
    const KV* __restrict__ mk, const KV* __restrict__ mv, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ sl, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ nsel, int compensate, int pages_per_split,
    float* __restrict__ part) {
  constexpr int LPR = D / 8, RS = kThreads / LPR;
  constexpr int SLOT = (DENSE ? 1 : 2) * kPartStride(D);
  __shared__ float sm_state[3 * RS * G];
  __shared__ float sm_acc[RS * D];

  const int split = blockIdx.x % s.n_splits;
  const int bg = blockIdx.x / s.n_splits;
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int L = clamp_len(sl[b], s.max_blocks * s.bs);
  const int M = (L + s.bs - 1) / s.bs;
  const int tid = threadIdx.x, rs = tid / LPR, c = tid % LPR;

  int first, nblk;
  const int32_t* ids = nullptr;
  if (DENSE) {
    first = split * pages_per_split;
    nblk = max(0, min(M, first + pages_per_split) - first);
  } else {
    const int kk = min(min(nsel[bg], s.kmax), M);
    first = split * pages_per_split;
    nblk = max(0, min(kk, first + pages_per_split) - first);
    ids = sel + (size_t)bg * s.kmax + first;
  }

  float qv[G][8];
  load_q<KV, D, G>(s, q, b, g, c, qv);

  float m[G], l[G], zz[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY; l[j] = 0.f; zz[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  // Exact tokens: rows enumerate (block of the slice, token).
  for (int R = rs; R < nblk * s.bs; R += RS) {
    const int bl = R / s.bs, t = R % s.bs;
    const int i = DENSE ? first + bl : ids[bl];
    if (i < 0 || i >= M) continue;
    const int page = bt[(size_t)b * s.max_blocks + i];
    if (page < 0 || page >= s.P) continue;
    if (t >= min(s.bs, L - i * s.bs)) continue;
    const size_t off = (((size_t)page * s.Hkv + g) * s.bs + t) * D + c * 8;
    float k8[8], v8[8], dot[G];
    load8(kc + off, k8);
    load8(vc + off, v8);
    dot8<G>(qv, k8, dot);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float sj = group_sum<LPR>(dot[j]) * s.tau;
      if (sj > m[j]) {
        const float sc = scale_from(m[j], sj);
        l[j] *= sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] *= sc;
        m[j] = sj;
      }
      const float w = expf(sj - m[j]);
      l[j] += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(w, v8[e], acc[j][e]);
    }
  }
  float* base = part + ((size_t)bg * s.n_splits + split) * G * SLOT;
  combine_rows<D, G, RS>(m, l, zz, acc, base, SLOT, sm_state, sm_acc);
  if (DENSE) return;

  // The selected blocks' compensation terms n e^{s_bar} mean_v, computed
  // exactly as the scan computes them (same lanes, same order).
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY; l[j] = 0.f; zz[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  if (compensate) {
    for (int bl = rs; bl < nblk; bl += RS) {
      const int i = ids[bl];
      if (i < 0 || i >= M) continue;
      const int page = bt[(size_t)b * s.max_blocks + i];
      if (page < 0 || page >= s.P) continue;
      const int n = min(s.bs, L - i * s.bs);
      const size_t row = ((size_t)page * s.Hkv + g) * D + c * 8;
      float mu8[8], nu8[8], dot[G];
      load8(mk + row, mu8);
      load8(mv + row, nu8);
      dot8<G>(qv, mu8, dot);
      const float fn = (float)n;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float sbar = group_sum<LPR>(dot[j]) * s.tau;
        if (sbar > m[j]) {
          const float sc = scale_from(m[j], sbar);
          l[j] *= sc;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j][e] *= sc;
          m[j] = sbar;
        }
        const float w = fn * expf(sbar - m[j]);
        l[j] += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(w, nu8[e], acc[j][e]);
      }
    }
  }
  combine_rows<D, G, RS>(m, l, zz, acc, base + kPartStride(D), SLOT, sm_state, sm_acc);
}

// ---------------------------------------------------------------------------
// Merge: per (sequence, query head), combine the gather partials of the
// exact tokens with the omitted blocks' compensation,
//   omitted = (scan sum over all blocks) - (selected blocks' terms),
// then out = numerator / denominator and lse = log denominator.
// ---------------------------------------------------------------------------
template <int D, bool DENSE>
__global__ __launch_bounds__(D) void merge_kernel(Shape s, const int32_t* __restrict__ sl,
                                                  const int32_t* __restrict__ nsel, int compensate,
                                                  const float* __restrict__ comp,
                                                  const float* __restrict__ gath,
                                                  float* __restrict__ out, float* __restrict__ lse) {
  constexpr int PST = kPartStride(D);
  constexpr int SLOT = (DENSE ? 1 : 2) * PST;
  const int bh = blockIdx.x;
  const int b = bh / s.Hq, h = bh % s.Hq;
  const int g = h / s.G, j = h % s.G;
  const int bg = b * s.Hkv + g;
  const int t = threadIdx.x;
  const int L = clamp_len(sl[b], s.max_blocks * s.bs);
  const int M = (L + s.bs - 1) / s.bs;

  // exact part
  float Me = -INFINITY;
  for (int sp = 0; sp < s.n_splits; ++sp)
    Me = fmaxf(Me, gath[(((size_t)bg * s.n_splits + sp) * s.G + j) * SLOT]);
  float le = 0.f, ae = 0.f;
  for (int sp = 0; sp < s.n_splits; ++sp) {
    const float* p = gath + (((size_t)bg * s.n_splits + sp) * s.G + j) * SLOT;
    const float f = scale_from(p[0], Me);
    le += p[1] * f;
    ae += p[4 + t] * f;
  }
  float Mo = -INFINITY, lo = 0.f, ao = 0.f;
  if (!DENSE && compensate) {
    const int kk = min(min(nsel[bg], s.kmax), M);
    if (kk < M) {
      float Ma = -INFINITY;
      for (int ch = 0; ch < s.n_chunks; ++ch)
        Ma = fmaxf(Ma, comp[(((size_t)bg * s.n_chunks + ch) * s.G + j) * PST]);
      float la = 0.f, aa = 0.f;
      for (int ch = 0; ch < s.n_chunks; ++ch) {
        const float* p = comp + (((size_t)bg * s.n_chunks + ch) * s.G + j) * PST;
        const float f = scale_from(p[0], Ma);
        la += p[1] * f;
        aa += p[4 + t] * f;
      }
      float Ms = -INFINITY;
      for (int sp = 0; sp < s.n_splits; ++sp)
        Ms = fmaxf(Ms, gath[(((size_t)bg * s.n_splits + sp) * s.G + j) * SLOT + PST]);
      float ls = 0.f, as = 0.f;
      for (int sp = 0; sp < s.n_splits; ++sp) {
        const float* p = gath + (((size_t)bg * s.n_splits + sp) * s.G + j) * SLOT + PST;
        const float f = scale_from(p[0], Ms);
        ls += p[1] * f;
        as += p[4 + t] * f;
      }
      const float fs = scale_from(Ms, Ma);  // selected terms in the all-block frame (Ms <= Ma)
      lo = la - ls * fs;
      ao = aa - as * fs;
      if (lo < 0.f) lo = 0.f;  // omitted mass below rounding of the selected mass
      Mo = Ma;
    }
  }
  const float Mx = fmaxf(Me, Mo);
  const float fe = scale_from(Me, Mx), fo = scale_from(Mo, Mx);
  const float den = le * fe + lo * fo;
  const size_t o = (size_t)bh * D + t;
  if (den > 0.f) {
    out[o] = (ae * fe + ao * fo) / den;
    if (lse && t == 0) lse[bh] = Mx + logf(den);
  } else {
    out[o] = 0.f;
    if (lse && t == 0) lse[bh] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Dispatch helpers
// ---------------------------------------------------------------------------
template <template <typename, int, int> class F, typename... A>
hipError_t dispatch(const Shape& s, A&&... args);

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

#define CKV_DISPATCH_G(MACRO, KV, DD) \
  switch (s.G) {                      \
    case 1: MACRO(KV, DD, 1); break;  \
    case 2: MACRO(KV, DD, 2); break;  \
    case 4: MACRO(KV, DD, 4); break;  \
    default: MACRO(KV, DD, 8); break; \
  }
#define CKV_DISPATCH(MACRO)                                                   \
  if (s.dtype == 0) {                                                         \
    if (s.D == 128) { CKV_DISPATCH_G(MACRO, uint16_t, 128) }                  \
    else { CKV_DISPATCH_G(MACRO, uint16_t, 64) }                              \
  } else {                                                                    \
    if (s.D == 128) { CKV_DISPATCH_G(MACRO, float, 128) }                     \
    else { CKV_DISPATCH_G(MACRO, float, 64) }                                 \
  }

hipError_t launch_scan(const Shape& s, const void* q, const Summ& sm, const int32_t* bt,
                       const int32_t* sl, int mode, const Work& w, hipStream_t st) {
  const dim3 grid(s.B * s.Hkv * s.n_chunks);
#define CKV_SCAN(KV, DD, GG)                                                                 \
  hipLaunchKernelGGL((scan_kernel<KV, DD, GG>), grid, dim3(kThreads), 0, st, s, (const KV*)q, \
                     (const KV*)sm.mean_k, (const KV*)sm.mean_v, (const float*)sm.gvar, bt, sl, \
                     mode, w.comp, w.lam)
  CKV_DISPATCH(CKV_SCAN)
#undef CKV_SCAN
  return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const int32_t* sl, const Work& w, int32_t* selected,
                         int32_t* num_selected, float* group_scores, hipStream_t st) {
  const dim3 grid(s.B * s.Hkv);
  const size_t lds = (size_t)s.max_blocks * sizeof(uint32_t);
#define CKV_SEL(GG)                                                                          \
  hipLaunchKernelGGL((select_kernel<GG>), grid, dim3(kSelThreads), lds, st, s, sl, w.comp, \
                     w.lam, selected, num_selected, group_scores, s.D)
  switch (s.G) {
    case 1: CKV_SEL(1); break;
    case 2: CKV_SEL(2); break;
    case 4: CKV_SEL(4); break;
    default: CKV_SEL(8); break;
  }
#undef CKV_SEL
  return hipGetLastError();
}

hipError_t launch_gather(const Shape& s, const void* q, const void* k_cache, const void* v_cache,
                         const Summ& sm, const int32_t* bt, const int32_t* sl,
                         const int32_t* selected, const int32_t* num_selected, int compensate,
                         const Work& w, hipStream_t st) {
  if (s.n_splits == 0) return hipSuccess;
  const dim3 grid(s.B * s.Hkv * s.n_splits);
#define CKV_GATH(KV, DD, GG)                                                                  \
  hipLaunchKernelGGL((gather_kernel<KV, DD, GG, false>), grid, dim3(kThreads), 0, st, s,      \
                     (const KV*)q, (const KV*)k_cache, (const KV*)v_cache, (const KV*)sm.mean_k, \
                     (const KV*)sm.mean_v, bt, sl, selected, num_selected, compensate,         \
                     kGatherPages, w.gath)
  CKV_DISPATCH(CKV_GATH)
#undef CKV_GATH
  return hipGetLastError();
}

hipError_t launch_merge(const Shape& s, const int32_t* sl, const int32_t* num_selected,
                        int compensate, const Work& w, float* out, float* lse, hipStream_t st) {
  const dim3 grid(s.B * s.Hq);
  if (s.D == 128)
    hipLaunchKernelGGL((merge_kernel<128, false>), grid, dim3(128), 0, st, s, sl, num_selected,
                       compensate, w.comp, w.gath, out, lse);
  else
    hipLaunchKernelGGL((merge_kernel<64, false>), grid, dim3(64), 0, st, s, sl, num_selected,
                       compensate, w.comp, w.gath, out, lse);
  return hipGetLastError();
}

hipError_t launch_dense(const Shape& s, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* bt, const int32_t* sl, float* part, float* out, float* lse,
                        hipStream_t st) {
  const dim3 grid(s.B * s.Hkv * s.n_splits);
#define CKV_DENSE(KV, DD, GG)                                                                 \
  hipLaunchKernelGGL((gather_kernel<KV, DD, GG, true>), grid, dim3(kThreads), 0, st, s,       \
                     (const KV*)q, (const KV*)k_cache, (const KV*)v_cache, (const KV*)nullptr, \
                     (const KV*)nullptr, bt, sl, (const int32_t*)nullptr,                      \
                     (const int32_t*)nullptr, 0, kDensePages, part)
  CKV_DISPATCH(CKV_DENSE)
#undef CKV_DENSE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid(s.B * s.Hq);
  if (s.D == 128)
    hipLaunchKernelGGL((merge_kernel<128, true>), mgrid, dim3(128), 0, st, s, sl,
                       (const int32_t*)nullptr, 0, (const float*)nullptr, part, out, lse);
  else
    hipLaunchKernelGGL((merge_kernel<64, true>), mgrid, dim3(64), 0, st, s, sl,
                       (const int32_t*)nullptr, 0, (const float*)nullptr, part, out, lse);
  return hipGetLastError();
}

}  // namespace ckv

// CompKV kernels for gfx950 (MI355X): summary build, and the decode step as
// separate launches that never wait on each other (score, select, attend)
// plus dense attention.  The single-launch step lives in fused.hip.
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
// Workgroup roles of the step kernel (a role is fixed by the launch mode and
// blockIdx):
//   scan   (sequence, KV head, chunk of 256 blocks).  Pass A computes
//          block-mean logits on the matrix cores - the G query heads of the
//          KV head are the rows of a 16x16x32 bf16 MFMA tile - and the
//          per-head log-scores; pass B sums the compensation terms of all
//          blocks of the chunk.
//   slice  (sequence, KV head, 1024 blocks).  Forms the ranked score of each
//          block of its slice and keeps the slice's top-k candidates; the
//          last slice of a (sequence, KV head) to arrive computes the top-k
//          from all candidates and writes the selection.
//   gather (sequence, KV head, split of the selected blocks; attend and
//          dense launches) attends exactly to a split of the blocks.
//   merge  run by the gather workgroup that arrives last for its (sequence,
//          KV head): log-sum-exp combination of the exact partials with the
//          compensation of the omitted blocks (all-block sums minus the
//          selected blocks' own terms) into the output.
// No workgroup waits for another.  What one workgroup hands to another in
// the same launch goes through device-coherent (sc1) stores and loads and a
// completion count; what the previous launch wrote is read with plain loads.

#include <type_traits>

#include "step_common.hpp"

namespace ckv {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Summary build: mean key, mean value, grouped key variance, count of one
// block for every KV head.  One workgroup per (sequence, block); threads over
// (KV head, 8-channel slice).  Summaries are stored by logical block.
// With kn (append only): the sequence's last token is new; its key and value
// rows (kn, vn: [B][Hkv][D]) are written into the page and used in place of
// what the page held there.
// ---------------------------------------------------------------------------
// Streaming loads of the caches (each page is read once per build).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load16(const void* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void raw_load_nt(const uint16_t* p, Raw8<uint16_t>& r) { r.a = nt_load16(p); }
__device__ __forceinline__ void raw_load_nt(const float* p, Raw8<float>& r) {
  r.a = nt_load16(p);
  r.b = nt_load16(p + 4);
}

template <typename KV, int D>
__global__ __launch_bounds__(kThreads) void summary_kernel(
    Shape s, KV* kc, KV* vc, const int32_t* __restrict__ bt, const int32_t* __restrict__ sl,
    int append_only, const KV* __restrict__ kn, const KV* __restrict__ vn, KV* __restrict__ mk,
    KV* __restrict__ mv, float* __restrict__ gv, int32_t* __restrict__ cnt) {
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

  // One item per (K or V, KV head, 8-channel slice): the first Hkv * LPR
  // items take the keys, the rest the values.  All 16 rows of the page are
  // requested at once (rows past the sequence lie in the page and are not
  // used).  Means on data shifted by the first token: a block of equal tokens
  // gets exactly that token as mean and zero variance.
  static_assert(kBlockSize == 16, "one page holds 16 tokens");
  const int nk = s.Hkv * LPR;
  const int gs = D / s.r;                     // channels per group
  const bool lanes_sum = gs % 8 == 0;         // a group is whole 8-channel slices of adjacent lanes
  for (int item = threadIdx.x; item < 2 * nk; item += blockDim.x) {
    const bool isv = item >= nk;
    const int it = isv ? item - nk : item;
    const int g = it / LPR, c = it % LPR;
    KV* p = (isv ? vc : kc) + ((size_t)page * s.Hkv + g) * s.bs * D + c * 8;
    Raw8<KV> raw[kBlockSize];
#pragma unroll
    for (int t = 0; t < kBlockSize; ++t) raw_load_nt(p + t * D, raw[t]);
    if (kn) {  // the new token is row n - 1; only this thread touches its 8 channels
      Raw8<KV> nr;
      raw_load((isv ? vn : kn) + ((size_t)b * s.Hkv + g) * D + c * 8, nr);
      raw_store(p + (n - 1) * D, nr);
#pragma unroll
      for (int t = 0; t < kBlockSize; ++t)
        if (t == n - 1) raw[t] = nr;
    }
    float mu[8];
    slice_mean(raw, n, mu);
    const size_t row = (((size_t)b * s.Hkv + g) * s.max_blocks + i) * D + c * 8;
    float vs = 0.f;  // keys: the slice's squared deviations summed
    if (isv) {
      store8(mv + row, mu);
    } else {
      float var[8];
      slice_sqdev(raw, n, mu, var);
      if (lanes_sum) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vs += var[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) var_sh[g * D + c * 8 + e] = var[e] / fn;
      }
      store8(mk + row, mu);
    }
    if (lanes_sum) {
      // the group's slices are adjacent lanes of one row (gs / 8 of them,
      // aligned): sum them across lanes
      const float gvv = group_variance_lanes(vs, gs, n);
      if (!isv && c % (gs / 8) == 0) gv[(((size_t)b * s.Hkv + g) * s.max_blocks + i) * s.r + c / (gs / 8)] = gvv;
    }
  }
  if (!lanes_sum) {
    __syncthreads();
    for (int item = threadIdx.x; item < s.Hkv * s.r; item += blockDim.x) {
      const int g = item / s.r, t = item % s.r;
      float acc = 0.f;
      for (int c = 0; c < gs; ++c) acc += var_sh[g * D + t * gs + c];
      gv[(((size_t)b * s.Hkv + g) * s.max_blocks + i) * s.r + t] = acc / (float)gs;
    }
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
  float w[G][kChunk];      // compensation weight n e^{s_bar - chunk max}
  float acc[RS * D];       // row-slot sums for the final reduction
};
struct SelLds {
  uint64_t keys[kCandLds];           // slice keys, then second-level candidates
  uint32_t hist[512];
  uint32_t bitmap[kMaxBlocks / 32];
  float hm[kMaxChunks * 8];          // chunk headers: max s_bar, z, max log score
  float hz[kMaxChunks * 8];
  float hc[kMaxChunks * 8];
  float lnz[8];
  float f[kSlice / kChunk][8];
  uint32_t sh[64];
  uint32_t wsum[kThreads / 64];
  uint32_t count;
};
template <int D, int G>
struct GathLds {
  static constexpr int RS = kThreads / (D / 8);
  int pg[kShareMax];
  int n[kShareMax];
  float st[2 * RS * G];
  float acc[RS * D];
  float red[kThreads / 64][G][D + 4];  // the exact tokens' per-wave states
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
// Scan: per-block log-scores (to xs), chunk headers and compensation sums
// (to cpart).  Everything it writes is read by the next launch.
// ---------------------------------------------------------------------------
template <typename KV, int D, int G>
__device__ void scan_role(const Shape& s, const StepIO& io, const Work& w, int t, ScanLds<D, G>& L) {
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

  // ---- every load of the chunk, issued first (q oldest) ----
  constexpr bool MF = std::is_same<KV, uint16_t>::value;
  constexpr int KT = D / 32;
  Raw8<KV> qraw;
  const bool qld = tid < G * D / 8;
  if (qld) raw_load(q + tid * 8, qraw);
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
        mu[u][kt] = ok ? *reinterpret_cast<const uint4*>(mk + (size_t)ri * D + 32 * kt + 8 * kq)
                       : make_uint4(0u, 0u, 0u, 0u);
      gpre[u] = (ok && holder && r == 4) ? *reinterpret_cast<const float4*>(gv + (size_t)ri * 4)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  if (qld) {
    float x[8];
    raw_float(qraw, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) L.qf[tid * 8 + e] = x[e];
  }
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
  // pass B's mean values, requested once pass A has consumed the mean keys:
  // holding both in registers from entry would halve the workgroups a CU can
  // hold; their round trip overlaps the log-scores below
#pragma unroll
  for (int jj = 0; jj < RPL; ++jj) {
    const int ri = rs + jj * RS;
    if (ri < nrows) raw_load(mv + (size_t)ri * D + c * 8, nu[jj]);
    else raw_zero(nu[jj]);
  }

  // ---- log-scores, chunk maxima, compensation weights, Z_hat partial ----
  float* part = w.cpart + ((size_t)bg * s.n_chunks + chunk) * G * PST;
  for (int j = wave; j < G; j += 4) {
    float mx = -INFINITY, cx = -INFINITY;
    float lamv[kChunk / 64];
#pragma unroll
    for (int u = 0; u < kChunk / 64; ++u) {
      const int ri = lane + 64 * u;
      lamv[u] = -INFINITY;
      if (ri < nrows) {
        const int n = min(s.bs, Lseq - (start + ri) * s.bs);
        const float sb = L.sb[j][ri], half = 0.5f * L.vh[j][ri];
        const float massf = (float)n * (1.f + half);  // second-order mass estimate / e^{s_bar}
        lamv[u] = io.score_mode == kScoreMass ? sb + flog(massf) : sb + flog(massf * half);
        mx = fmaxf(mx, sb);
        cx = fmaxf(cx, lamv[u]);
      }
    }
    mx = wave_max(mx);
    cx = wave_max(cx);
    float lsum = 0.f, zsum = 0.f;
    float* xrow = w.xs + ((size_t)b * s.Hq + g * G + j) * s.max_blocks + start;
#pragma unroll
    for (int u = 0; u < kChunk / 64; ++u) {
      const int ri = lane + 64 * u;
      if (ri < nrows) {
        const int n = min(s.bs, Lseq - (start + ri) * s.bs);
        const float wt = (float)n * fexp(L.sb[j][ri] - mx);
        lsum += wt;
        zsum = fmaf(wt, 1.f + 0.5f * L.vh[j][ri], zsum);
        L.w[j][ri] = wt;
        xrow[ri] = lamv[u] == -INFINITY ? 0.f : fexp(lamv[u] - cx);
      }
    }
    lsum = wave_sum(lsum);
    zsum = wave_sum(zsum);
    if (lane == 0) {
      float* h = part + (size_t)j * PST;
      h[0] = mx;
      h[1] = lsum;
      h[2] = zsum;
      h[3] = cx;
    }
  }
  __syncthreads();

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
      part[(size_t)j * PST + 4 + d] = a;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Slice: ranked scores of 1024 blocks and their top-k; the last slice of a
// (sequence, KV head) selects the top-k of all candidates.
// ---------------------------------------------------------------------------
template <typename KV, int D, int G>
__device__ void slice_role(const Shape& s, const StepIO& io, const Work& w, int t, SelLds& L, uint32_t* slot) {
  constexpr int PST = kPartStride(D);
  const int slice = t % s.n_slices, bg = t / s.n_slices;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = min(M, s.kmax);
  const float* parts = w.cpart + (size_t)bg * s.n_chunks * G * PST;
  const int i0 = slice * kSlice;
  const int nloc = max(0, min(M, i0 + kSlice) - i0);

  // chunk headers and this slice's per-head scores, all loads issued together
  for (int item = tid; item < s.n_chunks * G; item += kThreads) {
    const float* h = parts + (size_t)item * PST;
    L.hm[item] = h[0];
    L.hz[item] = h[2];
    L.hc[item] = h[3];
  }
  constexpr int XPT = kSlice / kThreads;
  float xv[XPT][G];
#pragma unroll
  for (int u = 0; u < XPT; ++u) {
    const int i = tid + u * kThreads;
#pragma unroll
    for (int j = 0; j < G; ++j)
      xv[u][j] = i < nloc ? w.xs[((size_t)b * s.Hq + g * G + j) * s.max_blocks + i0 + i] : 0.f;
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

  const Coh cand(w.cand + (size_t)bg * s.n_slices * s.kmax, (size_t)s.n_slices * s.kmax * 8);
  if (kk > 0 && kk < M) {
    const int k1 = min(kk, nloc);
    if (k1 > 0) {
      const uint64_t T = radix_kth_largest<kThreads>(LdsKeys{L.keys}, nloc, k1, L.hist, L.sh);
      if (tid == 0) L.count = 0;
      __syncthreads();
      for (int i = tid; i < nloc; i += kThreads) {
        const uint64_t key = L.keys[i];
        if (key >= T) cand.put_u64(slice * s.kmax + (int)atomicAdd(&L.count, 1u), key);
      }
    }
    for (int e = k1 + tid; e < kk; e += kThreads) cand.put_u64(slice * s.kmax + e, 0u);  // below every real key
  }
  const uint32_t prev = arrive(w.ctrl + kCtrlHeader + kCtrlPerPair * bg + 1, slot);
  if (prev != (uint32_t)(s.n_slices - 1)) return;

  // the last slice of this (sequence, KV head): global top-k and the selection
  int32_t* out = io.selected + (size_t)bg * s.kmax;
  if (tid == 0) io.num_selected[bg] = kk;
  for (int e = kk + tid; e < s.kmax; e += kThreads) out[e] = -1;
  if (kk == M) {
    for (int i = tid; i < M; i += kThreads) out[i] = i;
  } else if (kk > 0) {
    const int n2 = s.n_slices * kk;
    const int words = (M + 31) / 32;
    for (int e = tid; e < words; e += kThreads) L.bitmap[e] = 0u;
    if (n2 <= kCandLds) {
      for (int e = tid; e < n2; e += kThreads) L.keys[e] = cand.u64((e / kk) * s.kmax + e % kk);
      __syncthreads();
      const uint64_t T = radix_kth_largest<kThreads>(LdsKeys{L.keys}, n2, kk, L.hist, L.sh);
      for (int e = tid; e < n2; e += kThreads) {
        const uint64_t key = L.keys[e];
        const int idx = key_index(key);
        if (key >= T && idx >= 0 && idx < M) atomicOr(&L.bitmap[idx >> 5], 1u << (idx & 31));
      }
    } else {
      __syncthreads();
      struct MemKeys {
        Coh c;
        int kk, stride;
        __device__ uint64_t operator()(int e) const { return c.u64((e / kk) * stride + e % kk); }
      };
      const MemKeys keys{cand, kk, s.kmax};
      const uint64_t T = radix_kth_largest<kThreads>(keys, n2, kk, L.hist, L.sh);
      for (int e = tid; e < n2; e += kThreads) {
        const uint64_t key = keys(e);
        const int idx = key_index(key);
        if (key >= T && idx >= 0 && idx < M) atomicOr(&L.bitmap[idx >> 5], 1u << (idx & 31));
      }
    }
    __syncthreads();
    emit_selection<kThreads>(M, L.bitmap, L.wsum, out, kk, nullptr, 0, 0);
  }
  if (tid == 0) st_c(w.ctrl + kCtrlHeader + kCtrlPerPair * bg + 1, 0u);
}

// ---------------------------------------------------------------------------
// Gather core: exact attention over a list of blocks of one (sequence, KV
// head), and (comp) those blocks' own compensation terms.  Writes
// [m, l, -, -, acc[D]] per query head at part (head stride `slot`) with
// coherent stores; the compensation partial follows at part + D + 4 unless
// slot == D + 4.
// ---------------------------------------------------------------------------
template <int D, int G, int RS>
__device__ void combine_online(const float (&m)[G], const float (&l)[G], const float (&acc)[G][8],
                               float* part, int head_stride, float* st, float* sacc) {
  constexpr int LPR = D / 8;
  const int tid = threadIdx.x, rs = tid / LPR, c = tid % LPR;
  const Coh out(part, (size_t)G * head_stride * 4);
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
    for (int d = tid; d < D; d += kThreads) {
      float a = 0.f;
      for (int r2 = 0; r2 < RS; ++r2) a += sacc[r2 * D + d];
      out.put(j * head_stride + 4 + d, a);
    }
    if (tid == 0) {
      float ls = 0.f;
      for (int r2 = 0; r2 < RS; ++r2) ls += st[RS * G + r2 * G + j] * scale_from(st[r2 * G + j], Mj);
      out.put(j * head_stride, Mj);
      out.put(j * head_stride + 1, ls);
    }
    __syncthreads();
  }
}

template <int D, int G>
struct DenseCfg {
  static constexpr int CPL = G == 8 ? 8 : 16;   // channels per lane
  static constexpr int LPT = D / CPL;           // lanes per token row: 4, 8 or 16
  static constexpr int TPW = 64 / LPT;          // token rows per wave pass
  static constexpr int RPP = kBlockSize / TPW;  // rows per lane per page
  static constexpr int NR = CPL / 8;            // eight-element loads per row
};

// Reduction over the lanes that hold the same channels (lane % LPT) in the
// wave's 64 / LPT token slots.
template <int LPT, class Op>
__device__ __forceinline__ uint32_t token_slot_reduce(uint32_t x, Op op) {
  if (LPT == 4) x = op(x, dpp_row_ror4(x));
  if (LPT <= 8) x = op(x, dpp_row_ror8(x));
  return across_rows(x, op);
}
__device__ __forceinline__ float exp2_from(float a, float m) {  // 2^(a - m), 0 for a = -inf
  return a == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(a - m);
}

template <typename KV, int D, int G>
__device__ __forceinline__ void dense_issue(const Shape& s, const KV* kc, const KV* vc, int g, int pg, int n,
                                            int ts, int c, Raw8<KV> (&kr)[DenseCfg<D, G>::RPP][DenseCfg<D, G>::NR],
                                            Raw8<KV> (&vr)[DenseCfg<D, G>::RPP][DenseCfg<D, G>::NR],
                                            bool (&ok)[DenseCfg<D, G>::RPP]) {
  using C = DenseCfg<D, G>;
#pragma unroll
  for (int r = 0; r < C::RPP; ++r) {
    const int tok = r * C::TPW + ts;
    ok[r] = pg >= 0 && tok < n;
    if (ok[r]) {
      const size_t off = (((size_t)pg * s.Hkv + g) * s.bs + tok) * D + c * C::CPL;
#pragma unroll
      for (int u = 0; u < C::NR; ++u) {
        raw_load(kc + off + 8 * u, kr[r][u]);
        raw_load(vc + off + 8 * u, vr[r][u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < C::NR; ++u) {
        raw_zero(kr[r][u]);
        raw_zero(vr[r][u]);
      }
    }
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ uint32_t raw_word(const Raw8<uint16_t>& r, int i) {
  return i == 0 ? r.a.x : i == 1 ? r.a.y : i == 2 ? r.a.z : r.a.w;
}

// qv: the G query rows' CPL channels as float (f32 caches); qp: the same as
// bf16 pairs (bf16 caches, whose logits use the two-term bf16 dot product).
template <typename KV, int D, int G>
__device__ __forceinline__ void dense_page(const float (&qv)[G][DenseCfg<D, G>::CPL],
                                           const uint32_t (&qp)[G][DenseCfg<D, G>::CPL / 2], float tl,
                                           const Raw8<KV> (&kr)[DenseCfg<D, G>::RPP][DenseCfg<D, G>::NR],
                                           const Raw8<KV> (&vr)[DenseCfg<D, G>::RPP][DenseCfg<D, G>::NR],
                                           const bool (&ok)[DenseCfg<D, G>::RPP], float (&m)[G], float (&l)[G],
                                           float (&acc)[G][DenseCfg<D, G>::CPL]) {
  using C = DenseCfg<D, G>;
  constexpr int CPL = C::CPL, RPP = C::RPP;
  float sc[RPP][G];
#pragma unroll
  for (int r = 0; r < RPP; ++r) {
    float dd[G];
    if constexpr (sizeof(KV) == 2) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = 0.f;
#pragma unroll
        for (int u = 0; u < C::NR; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) d = dot2_bf16(raw_word(kr[r][u], i), qp[j][4 * u + i], d);
        dd[j] = d;
      }
    } else {
      float kf[CPL];
#pragma unroll
      for (int u = 0; u < C::NR; ++u) raw_float(kr[r][u], *reinterpret_cast<float(*)[8]>(kf + 8 * u));
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) d = fmaf(qv[j][e], kf[e], d);
        dd[j] = d;
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float d = token_row_sum<C::LPT>(dd[j]);
      sc[r][j] = ok[r] ? d * tl : -INFINITY;
    }
  }
  float p[RPP][G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float mx = sc[0][j];
#pragma unroll
    for (int r = 1; r < RPP; ++r) mx = fmaxf(mx, sc[r][j]);
    if (__ballot(mx > m[j]) != 0) {  // uniform over the wave
      const float mn = fmaxf(m[j], mx);
      const float f = exp2_from(m[j], mn);
      l[j] *= f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[j][e] *= f;
      m[j] = mn;
    }
#pragma unroll
    for (int r = 0; r < RPP; ++r) {
      p[r][j] = ok[r] ? __builtin_amdgcn_exp2f(sc[r][j] - m[j]) : 0.f;
      l[j] += p[r][j];
    }
  }
#pragma unroll
  for (int r = 0; r < RPP; ++r) {
    float vf[CPL];
#pragma unroll
    for (int u = 0; u < C::NR; ++u) raw_float(vr[r][u], *reinterpret_cast<float(*)[8]>(vf + 8 * u));
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[j][e] = fmaf(p[r][j], vf[e], acc[j][e]);
  }
}

// Exact attention of the G query heads of KV head g of sequence b over nb
// pages (page ids pg[], -1 = none, and token counts n[], in LDS, written
// before a barrier) into one partial per head at part: [max (natural log
// units), sum, -, -, acc[D]], head stride head_stride floats, device-coherent
// stores.  The waves take pages wave, wave + 4, ...; each lane holds CPL
// channels of one token row and keeps its own online softmax for the G heads
// (maximum in log2 units), raised only when some lane of the wave meets a
// larger logit; the lanes' states are combined once, at the end, through
// red (LDS).
template <typename KV, int D, int G>
__device__ __forceinline__ void dense_span(const Shape& s, const StepIO& io, int b, int g, const int* pg,
                                           const int* n, int nb, float (*red)[G][D + 4], float* part,
                                           int head_stride) {
  using C = DenseCfg<D, G>;
  constexpr int CPL = C::CPL, LPT = C::LPT, RPP = C::RPP, NR = C::NR, PST = kPartStride(D);
  constexpr int NW = kThreads / 64;
  // bf16 pages are double-buffered in registers up to G = 4; otherwise pages
  // are loaded one at a time
  constexpr bool kPrefetch = sizeof(KV) == 2 && G <= 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane % LPT, ts = lane / LPT;
  const KV* q = static_cast<const KV*>(io.q) + ((size_t)b * s.Hq + g * G) * D + c * CPL;
  float qv[G][CPL];
  uint32_t qp[G][CPL / 2];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      if constexpr (sizeof(KV) == 2) {
        Raw8<KV> rq;
        raw_load(q + (size_t)j * D + 8 * u, rq);
#pragma unroll
        for (int i = 0; i < 4; ++i) qp[j][4 * u + i] = raw_word(rq, i);
      } else {
        load8(q + (size_t)j * D + 8 * u, *reinterpret_cast<float(*)[8]>(&qv[j][8 * u]));
      }
    }
  const float tl = s.tau * 1.44269504088896340736f;  // logits in log2 units
  float m[G], l[G], acc[G][CPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[j][e] = 0.f;
  }

  const KV* kc = static_cast<const KV*>(io.k_cache);
  const KV* vc = static_cast<const KV*>(io.v_cache);
  const int np = nb > wave ? (nb - 1 - wave) / NW + 1 : 0;  // this wave's pages: wave + NW i
  Raw8<KV> ka[RPP][NR], va[RPP][NR];
  bool oka[RPP];
  if constexpr (kPrefetch) {
    Raw8<KV> kb[RPP][NR], vb[RPP][NR];
    bool okb[RPP];
    if (np > 0) dense_issue<KV, D, G>(s, kc, vc, g, pg[wave], n[wave], ts, c, ka, va, oka);
    for (int pi = 0; pi < np; pi += 2) {
      if (pi + 1 < np) {
        const int bl = wave + NW * (pi + 1);
        dense_issue<KV, D, G>(s, kc, vc, g, pg[bl], n[bl], ts, c, kb, vb, okb);
      }
      dense_page<KV, D, G>(qv, qp, tl, ka, va, oka, m, l, acc);
      if (pi + 1 < np) {
        if (pi + 2 < np) {
          const int bl = wave + NW * (pi + 2);
          dense_issue<KV, D, G>(s, kc, vc, g, pg[bl], n[bl], ts, c, ka, va, oka);
        }
        dense_page<KV, D, G>(qv, qp, tl, kb, vb, okb, m, l, acc);
      }
    }
  } else {
    for (int pi = 0; pi < np; ++pi) {
      const int bl = wave + NW * pi;
      dense_issue<KV, D, G>(s, kc, vc, g, pg[bl], n[bl], ts, c, ka, va, oka);
      dense_page<KV, D, G>(qv, qp, tl, ka, va, oka, m, l, acc);
    }
  }

  // combine the token slots of the wave, then the waves, into one partial
  // per head: [max (natural log units), sum, -, -, acc[D]]
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float mw = __uint_as_float(token_slot_reduce<LPT>(__float_as_uint(m[j]), OpFmax{}));
    const float f = exp2_from(m[j], mw);
    const float lw = __uint_as_float(token_slot_reduce<LPT>(__float_as_uint(l[j] * f), OpFadd{}));
    float a[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) a[e] = __uint_as_float(token_slot_reduce<LPT>(__float_as_uint(acc[j][e] * f), OpFadd{}));
    if (lane < LPT) {
      float* rw = red[wave][j];
#pragma unroll
      for (int e = 0; e < CPL; ++e) rw[4 + c * CPL + e] = a[e];
      if (c == 0) {
        rw[0] = mw;
        rw[1] = lw;
      }
    }
  }
  __syncthreads();
  const Coh out(part, (size_t)(G - 1) * head_stride * 4 + (size_t)PST * 4);
  for (int o = tid; o < G * D; o += kThreads) {
    const int j = o / D, d = o % D;
    float Mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) Mx = fmaxf(Mx, red[v][j][0]);
    float a = 0.f, ls = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float f = exp2_from(red[v][j][0], Mx);
      a = fmaf(red[v][j][4 + d], f, a);
      ls = fmaf(red[v][j][1], f, ls);
    }
    out.put(j * head_stride + 4 + d, a);
    if (d == 0) {
      out.put(j * head_stride, Mx * 0.69314718055994530942f);  // -inf stays -inf
      out.put(j * head_stride + 1, ls);
    }
  }
}

template <typename KV, int D, int G>
__device__ void gather_core(const Shape& s, const StepIO& io, int b, int g, const int* blk, int nb,
                            bool comp, float* part, int slot, GathLds<D, G>& L) {
  constexpr int LPR = D / 8, RS = kThreads / LPR, PST = kPartStride(D);
  const int bg = b * s.Hkv + g;
  const int tid = threadIdx.x, rs = tid / LPR, c = tid % LPR;
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const KV* q = static_cast<const KV*>(io.q) + ((size_t)b * s.Hq + g * G) * D;

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

  // exact tokens of the listed pages
  dense_span<KV, D, G>(s, io, b, g, L.pg, L.n, nb, L.red, part, slot);
  float m[G], l[G], acc[G][8];
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
// Gather (attend and dense launches)
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
  const int kk = DENSE ? M : min(min(io.num_selected[bg], s.kmax), M);
  const int first = split * s.pages_per_split;
  const int nb = max(0, min(kk, first + s.pages_per_split) - first);
  for (int e = threadIdx.x; e < nb; e += kThreads)
    blk[e] = DENSE ? first + e : io.selected[(size_t)bg * s.kmax + first + e];
  __syncthreads();
  float* gp = w.gpart + ((size_t)bg * s.n_splits + split) * G * SLOT;
  gather_core<KV, D, G>(s, io, b, g, blk, nb, !DENSE && io.compensate != 0, gp, SLOT, L);
  const uint32_t prev = arrive(w.ctrl + kCtrlHeader + kCtrlPerPair * bg + 2, slot);
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
  const int kk = DENSE ? M : min(min(io.num_selected[bg], s.kmax), M);
  const bool comp = !DENSE && io.compensate && kk < M;
  const int nch = comp ? s.n_chunks : 0;
  const int nsp = s.n_splits;
  const float* cp = w.cpart + (size_t)bg * s.n_chunks * G * PST;  // previous launch: plain loads
  const Coh gp(w.gpart + (size_t)bg * nsp * G * SLOT, (size_t)nsp * G * SLOT * 4);
  float* f_ch = L.f;                    // [G][nch]
  float* f_ex = L.f + G * nch;          // [G][nsp]
  float* f_sc = L.f + G * (nch + nsp);  // [G][nsp]

  for (int j = wave; j < G; j += 4) {
    float Ma = -INFINITY, Me = -INFINITY, Ms = -INFINITY;
    for (int ch = lane; ch < nch; ch += 64) Ma = fmaxf(Ma, cp[((size_t)ch * G + j) * PST]);
    for (int sp = lane; sp < nsp; sp += 64) {
      Me = fmaxf(Me, gp.f32((sp * G + j) * SLOT));
      if (comp) Ms = fmaxf(Ms, gp.f32((sp * G + j) * SLOT + PST));
    }
    Ma = wave_max(Ma);
    Me = wave_max(Me);
    Ms = wave_max(Ms);
    float la = 0.f, le = 0.f, ls = 0.f;
    for (int ch = lane; ch < nch; ch += 64) {
      const float* h = cp + ((size_t)ch * G + j) * PST;
      const float f = scale_from(h[0], Ma);
      f_ch[j * nch + ch] = f;
      la += h[1] * f;
    }
    for (int sp = lane; sp < nsp; sp += 64) {
      const int h = (sp * G + j) * SLOT;
      const float f = scale_from(gp.f32(h), Me);
      f_ex[j * nsp + sp] = f;
      le += gp.f32(h + 1) * f;
      if (comp) {
        const float f2 = scale_from(gp.f32(h + PST), Ms);
        f_sc[j * nsp + sp] = f2;
        ls += gp.f32(h + PST + 1) * f2;
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
    for (int sp = 0; sp < nsp; ++sp) ae = fmaf(gp.f32((sp * G + j) * SLOT + 4 + d), f_ex[j * nsp + sp], ae);
    float ao = 0.f;
    if (comp) {
      float aa = 0.f, as = 0.f;
#pragma unroll 16
      for (int ch = 0; ch < nch; ++ch) aa = fmaf(cp[((size_t)ch * G + j) * PST + 4 + d], f_ch[j * nch + ch], aa);
#pragma unroll 16
      for (int sp = 0; sp < nsp; ++sp) as = fmaf(gp.f32((sp * G + j) * SLOT + PST + 4 + d), f_sc[j * nsp + sp], as);
      ao = aa - as * L.head[j][2];
    }
    const float den = L.head[j][3];
    const int h = g * G + j;
    const size_t oi = ((size_t)b * s.Hq + h) * D + d;
    io.out[oi] = den > 0.f ? (ae * L.head[j][0] + ao * L.head[j][1]) / den : 0.f;
    if (io.lse && d == 0) io.lse[(size_t)b * s.Hq + h] = den > 0.f ? L.head[j][4] + logf(den) : -INFINITY;
  }
  if (tid == 0) st_c(w.ctrl + kCtrlHeader + kCtrlPerPair * bg + 2, 0u);
}

// ---------------------------------------------------------------------------
// Dense decode attention (the baseline the sparse step is measured against):
// exact attention over every block, split over the blocks of each (sequence,
// KV head) pair, one workgroup per split.  A wave takes whole pages (waves
// take pages wave, wave + 4, ... of the split).  Each lane holds CPL channels
// of one token row of the page and keeps its own online-softmax state for
// the G query heads (maximum in log2 units, sum, CPL accumulators), so the
// only cross-lane step per token is the LPT-lane sum of each logit.  A
// lane's maximum is raised only when some lane of the wave meets a larger
// logit (a wave-uniform branch).  The lanes' states are combined once, at
// the end of the split; the last split of a pair to arrive merges the
// splits' partials (the dense mode of merge_role).
// ---------------------------------------------------------------------------
template <int D, int G>
struct DenseLds {
  int pg[kDensePages];
  int n[kDensePages];
  union {
    float red[kThreads / 64][G][D + 4];
    MergeLds merge;
  } u;
};

template <typename KV, int D, int G>
__global__ __launch_bounds__(kThreads, 2) void dense_kernel(Shape s, StepIO io, Work w) {
  constexpr int PST = kPartStride(D);
  __shared__ DenseLds<D, G> L;
  __shared__ uint32_t slot;
  const int t = (int)blockIdx.x, split = t % s.n_splits, bg = t / s.n_splits;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x;
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int first = split * s.pages_per_split;
  const int nb = max(0, min(M, first + s.pages_per_split) - first);
  for (int e = tid; e < nb; e += kThreads) {
    const int i = first + e;
    int p = io.block_table[(size_t)b * s.max_blocks + i];
    int n = 0;
    if (p < 0 || p >= s.P) p = -1;
    else n = min(s.bs, Lseq - i * s.bs);
    L.pg[e] = p;
    L.n[e] = n;
  }
  __syncthreads();
  dense_span<KV, D, G>(s, io, b, g, L.pg, L.n, nb, L.u.red,
                      w.gpart + ((size_t)bg * s.n_splits + split) * G * PST, PST);
  const uint32_t prev = arrive(w.ctrl + kCtrlHeader + kCtrlPerPair * bg + 2, &slot);
  if (prev == (uint32_t)(s.n_splits - 1)) merge_role<D, G, kModeDense>(s, io, w, bg, L.u.merge);
}

// ---------------------------------------------------------------------------
// The step kernel.  blockIdx.x: [scans], [slices] or [gathers], by mode.
// ---------------------------------------------------------------------------
// The bf16 scan is a streaming pass over every chunk: it is held to 128
// registers so that four workgroups share a CU; the other roles keep what
// they need.
template <typename KV, int D, int G, int MODE>
__global__ __launch_bounds__(kThreads, MODE == kModeScanOnly && sizeof(KV) == 2 && G <= 4 ? 4 : 1) void step_kernel(
    Shape s, StepIO io, Work w) {
  __shared__ StepLds<D, G> lds;
  __shared__ int blk[kShareMax];
  __shared__ uint32_t slot;
  const int t = (int)blockIdx.x;
  if (MODE == kModeScanOnly) {
    scan_role<KV, D, G>(s, io, w, t, lds.scan);
  } else if (MODE == kModeSelectOnly) {
    slice_role<KV, D, G>(s, io, w, t, lds.sel, &slot);
  } else {
    const int merge_bg = gather_role<KV, D, G, MODE>(s, io, w, t, lds.gath, blk, &slot);
    if (merge_bg >= 0) {
      __syncthreads();
      merge_role<D, G, MODE>(s, io, w, merge_bg, lds.merge);
    }
  }
}

}  // namespace

// ---- launchers --------------------------------------------------------------

static hipError_t launch_summary(const Shape& s, void* k_cache, void* v_cache, const int32_t* bt,
                                 const int32_t* sl, int append_only, const void* k_new,
                                 const void* v_new, const Summ& o, hipStream_t st) {
  const int LPR = s.D / 8;
  int threads = ((s.Hkv * LPR + 63) / 64) * 64;
  threads = threads > kThreads ? kThreads : threads;
  const dim3 grid(append_only ? s.B : s.B * s.max_blocks);
  const size_t lds = (size_t)s.Hkv * s.D * sizeof(float);
#define CKV_SUMM(KV, DD)                                                                          \
  hipLaunchKernelGGL((summary_kernel<KV, DD>), grid, dim3(threads), lds, st, s, (KV*)k_cache,     \
                     (KV*)v_cache, bt, sl, append_only, (const KV*)k_new, (const KV*)v_new,       \
                     (KV*)o.mean_k, (KV*)o.mean_v, o.gvar, o.count)
  if (s.dtype == 0) {
    if (s.D == 128) CKV_SUMM(uint16_t, 128); else CKV_SUMM(uint16_t, 64);
  } else {
    if (s.D == 128) CKV_SUMM(float, 128); else CKV_SUMM(float, 64);
  }
#undef CKV_SUMM
  return hipGetLastError();
}

hipError_t launch_build_summaries(const Shape& s, const void* k_cache, const void* v_cache,
                                  const int32_t* bt, const int32_t* sl, int append_only,
                                  const Summ& o, hipStream_t st) {
  // read only: the caches are written only when new tokens are given
  return launch_summary(s, const_cast<void*>(k_cache), const_cast<void*>(v_cache), bt, sl, append_only,
                        nullptr, nullptr, o, st);
}

hipError_t launch_append_tokens(const Shape& s, const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, const int32_t* bt, const int32_t* sl, const Summ& o,
                                hipStream_t st) {
  return launch_summary(s, k_cache, v_cache, bt, sl, 1, k_new, v_new, o, st);
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

template <int MODE>
static hipError_t launch_mode(const Shape& s, const StepIO& io, const Work& w, hipStream_t st) {
  const int bgs = s.B * s.Hkv;
  const int n = MODE == kModeScanOnly ? bgs * s.n_chunks
                : MODE == kModeSelectOnly ? bgs * s.n_slices
                                          : bgs * s.n_splits;
  return with_kernel<MODE>(s, [&](auto fn) {
    hipLaunchKernelGGL(fn, dim3(n), dim3(kThreads), 0, st, s, io, w);
    return hipGetLastError();
  });
}

static hipError_t launch_dense(const Shape& s, const StepIO& io, const Work& w, hipStream_t st) {
  const dim3 grid(s.B * s.Hkv * s.n_splits);
#define CKV_DG(KV, DD)                                                                                  \
  switch (s.G) {                                                                                        \
    case 1: hipLaunchKernelGGL((dense_kernel<KV, DD, 1>), grid, dim3(kThreads), 0, st, s, io, w); break; \
    case 2: hipLaunchKernelGGL((dense_kernel<KV, DD, 2>), grid, dim3(kThreads), 0, st, s, io, w); break; \
    case 4: hipLaunchKernelGGL((dense_kernel<KV, DD, 4>), grid, dim3(kThreads), 0, st, s, io, w); break; \
    default: hipLaunchKernelGGL((dense_kernel<KV, DD, 8>), grid, dim3(kThreads), 0, st, s, io, w); break; \
  }
  if (s.dtype == 0) {
    if (s.D == 128) { CKV_DG(uint16_t, 128) } else { CKV_DG(uint16_t, 64) }
  } else {
    if (s.D == 128) { CKV_DG(float, 128) } else { CKV_DG(float, 64) }
  }
#undef CKV_DG
  return hipGetLastError();
}

hipError_t launch_step(const Shape& s, int mode, const StepIO& io, const Work& w, hipStream_t st) {
  switch (mode) {
    case kModeScanOnly: return launch_mode<kModeScanOnly>(s, io, w, st);
    case kModeSelectOnly: return launch_mode<kModeSelectOnly>(s, io, w, st);
    case kModeAttendOnly: return launch_mode<kModeAttendOnly>(s, io, w, st);
    case kModeDense: return launch_dense(s, io, w, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ckv

// Fused CompKV decode step for gfx950 (MI355X): one launch scores every
// block, selects the top-k under the token budget, attends exactly to the
// selected blocks and merges in the Mean compensation of the omitted ones.
//
// The method (CompKV abstract, shd-paper.top listing; CompKV review,
// evolve.pub, "Summary" and FAQ; paper Section 3, Eqs. 4-7): a block's
// residual score is its second-order attention-mass estimate
// n e^{s_bar} (1 + var_hat/2) times var_hat/2, where s_bar is the logit of
// the mean key and var_hat the logit variance estimated from the grouped key
// variances; for GQA the ranked score of a block is the sum over the KV
// head's query heads of score / Z_hat.  The top-k blocks are attended
// exactly; each omitted block enters the softmax once with weight
// n e^{s_bar} and value mean_v.
//
// Organisation.  One workgroup per (sequence, KV head, chunk of 256 blocks).
// The grid covers bg_round (sequence, KV head) pairs at once and walks the
// rest in rounds; every workgroup of the grid is resident, so the workgroups
// of a pair can wait for each other.  A workgroup has 8 waves:
//   control waves 0-3 load the chunk's mean keys and grouped variances,
//     compute the block-mean logits on the matrix cores (the G query heads
//     are the rows of a 16x16x32 bf16 MFMA tile), publish the chunk header
//     (max logit, partial Z_hat per head), read every header of the pair,
//     rank the chunk's blocks, publish the chunk's top-k candidates, read
//     every candidate of the pair, find the pair's top-k, and attend exactly
//     to the workgroup's share of the selected blocks;
//   value waves 4-7 stream the chunk's mean values from the start and, once
//     the selection is known, sum the compensation terms of the chunk's
//     omitted blocks.
// A wave's memory counter drains in issue order, so a wave that waits for a
// load waits for every load it issued before.  Value waves therefore never
// read what other workgroups publish, and control waves never hold the
// long mean-value stream.  Headers and candidates are 64-bit words that are
// never 0 once written; readers poll them until nonzero, so publishing
// needs no completion wait and no counter.  Each workgroup then publishes
// one (max, sum, acc[d]) partial per query head and counts itself; the last
// to arrive merges the pair's partials into the output and clears the pair's
// headers and candidates, which leaves the workspace ready for the next call.
#include <type_traits>

#include "step_common.hpp"

namespace ckv {

namespace {

constexpr int NT = kFusedThreads;  // threads per workgroup
constexpr int NCTL = NT / 2;       // control threads
constexpr int kPollBatch = 8;      // published words read per thread per round trip
constexpr uint32_t kPollLimit = 1u << 20;  // re-reads per thread and call

template <int D, int G>
struct FusedLds {
  static constexpr int NW = NT / 64;
  float qf[G * D];        // this KV head's query rows
  float qn[G * D];        // |q_h restricted to channel group t|^2, [G][r]
  float sb[G][kChunk];    // block-mean logit tau q.mean_k
  float lam[G][kChunk];   // estimated logit variance, then log of the per-head score
  float wt[G][kChunk];    // compensation weight n e^{s_bar - chunk max}
  float mx[G];            // chunk max of s_bar per head
  float lnz[G];           // log Z_hat per head
  float hdr[kMaxChunks * G * 2];  // merge: (max, sum) of every partial
  union {
    uint64_t keys[kFusedCand];    // headers, chunk keys, then the pair's candidates
    float red[NW][G][D + 4];      // per-wave partial states
    float fac[kMaxChunks * G];    // merge factors
  } u;
  float mtot[G], ltot[G];
  uint32_t hist[512];
  uint32_t bitmap[kMaxBlocks / 32];
  int blk[kShareMax];
  int pg[kShareMax];
  int nn[kShareMax];
  uint32_t sh[4];
  uint32_t wsum[NW];
  uint32_t count;
  uint32_t slot;
};

// Copy n published 64-bit words into dst, waiting for each to become
// nonzero.  Word e is read at index (e / per) * stride + e % per.  Run by
// the control threads; each thread's re-reads are bounded in total, and
// running out sets the error word.
__device__ void read_published(const Coh& src, int n, int per, int stride, uint64_t* dst, uint32_t* err) {
  const int t = threadIdx.x;
  uint32_t spins = 0;
  for (int base = 0; base < n; base += NCTL * kPollBatch) {
    uint64_t v[kPollBatch];
#pragma unroll
    for (int u = 0; u < kPollBatch; ++u) {
      const int e = base + t + u * NCTL;
      v[u] = e < n ? src.u64((e / per) * stride + e % per) : 1u;
    }
#pragma unroll
    for (int u = 0; u < kPollBatch; ++u) {
      const int e = base + t + u * NCTL;
      while (v[u] == 0 && spins < kPollLimit) {
        __builtin_amdgcn_s_sleep(1);
        v[u] = src.u64((e / per) * stride + e % per);
        if (++spins == kPollLimit) st_c(err, 1u);
      }
      if (e < n) dst[e] = v[u];
    }
  }
}

// Returns true in the workgroup that arrived last for this pair.
template <typename KV, int D, int G>
__device__ bool fused_chunk(const Shape& s, const StepIO& io, const Work& w, int bg, int chunk,
                            FusedLds<D, G>& L) {
  constexpr int LPR = D / 8, RS = NCTL / LPR, PST = kPartStride(D), RPL = kChunk / RS;
  constexpr int KT = D / 32, NW = NT / 64;
  constexpr bool MF = std::is_same<KV, uint16_t>::value;
  constexpr int RW = sizeof(KV) / 2;                     // uint4 words per 8 elements
  constexpr int NBUF = (MF ? 4 * KT : 0) > RPL * RW ? 4 * KT : RPL * RW;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform values live in scalar registers, so branches on them do not
  // serialise the two halves of the workgroup
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool ctl = wave < NCTL / 64;
  const int ct = ctl ? tid : tid - NCTL;  // thread index within its half
  const int cw = ctl ? wave : wave - NCTL / 64;  // wave index within its half
  const int rs = ct / LPR, c = ct % LPR;  // row slot, 8-channel slice
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = min(M, s.kmax);
  const bool ranked = kk > 0 && kk < M;
  const bool need_mu = kk < M;               // logits of omitted blocks are needed
  const bool comp = need_mu && io.compensate;
  const int start = chunk * kChunk;
  const int nrows = max(0, min(M, start + kChunk) - start);
  const size_t row0 = (size_t)bg * s.max_blocks + start;  // logical summary row of the chunk
  const KV* q = static_cast<const KV*>(io.q) + ((size_t)b * s.Hq + g * G) * D;
  const KV* mk = static_cast<const KV*>(io.summ.mean_k) + row0 * D;
  const KV* mv = static_cast<const KV*>(io.summ.mean_v) + row0 * D;
  const int r = s.r, gs = D / r;
  const float* gv = io.summ.gvar + row0 * r;
  uint32_t* err = w.ctrl + 2;

  // ---- loads: q; control: mean keys and variances; value: mean values ----
  Raw8<KV> qraw;
  const bool qld = tid < G * D / 8;  // control threads only (G * D / 8 <= 128)
  if (qld) raw_load(q + tid * 8, qraw);
  uint4 buf[NBUF];  // control: mean-key MFMA operands; value: raw mean values
  float4 gpre[4];
  bf16x8_t qa[KT];
  const bool holder = (lane >> 4) * 4 < G;
  if (ctl) {
    if constexpr (MF) {
      if (need_mu) {
        const int head = lane & 15, kq = lane >> 4;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if (head < G) v = *reinterpret_cast<const uint4*>(q + (size_t)head * D + 32 * kt + 8 * kq);
          qa[kt] = __builtin_bit_cast(bf16x8_t, v);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ri = (cw + 4 * u) * 16 + (lane & 15);
          const bool ok = ri < nrows;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
            buf[u * KT + kt] = ok ? *reinterpret_cast<const uint4*>(mk + (size_t)ri * D + 32 * kt + 8 * kq)
                                  : make_uint4(0u, 0u, 0u, 0u);
          gpre[u] = (ok && holder && r == 4 && ranked) ? *reinterpret_cast<const float4*>(gv + (size_t)ri * 4)
                                                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  } else if (comp) {
#pragma unroll
    for (int jj = 0; jj < RPL; ++jj) {
      const int ri = rs + jj * RS;
      Raw8<KV> x;
      if (ri < nrows) raw_load(mv + (size_t)ri * D + c * 8, x);
      else raw_zero(x);
      if constexpr (MF) {
        buf[jj] = x.a;
      } else {
        buf[2 * jj] = x.a;
        buf[2 * jj + 1] = x.b;
      }
    }
  }
  if (qld) {
    float x[8];
    raw_float(qraw, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) L.qf[tid * 8 + e] = x[e];
  }
  __syncthreads();
  for (int item = tid; item < G * r; item += NT) {
    const int j = item / r, tg = item % r;
    const float* qh = L.qf + j * D + tg * gs;
    float a = 0.f;
    for (int cc = 0; cc < gs; ++cc) a = fmaf(qh[cc], qh[cc], a);
    L.qn[item] = a;
  }
  __syncthreads();

  // ---- block-mean logits and variance estimates (control waves) ----
  if (ctl && need_mu) {
    if constexpr (MF) {
      // D[head][row] = sum_k Q[head][k] mean_k[row][k]; lane l holds Q[l%16][8(l/16)..+7]
      // of each 32-wide k-slice (zero rows past G), mean_k of row l%16 at the same
      // k, and receives D[4(l/16)+i][l%16].
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kt], __builtin_bit_cast(bf16x8_t, buf[u * KT + kt]),
                                                         acc, 0, 0, 0);
        const int ri = (cw + 4 * u) * 16 + (lane & 15);
        if (ri < nrows && holder) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 4 * (lane >> 4) + i;
            if (j < G) {
              float sig = 0.f;
              if (ranked) {
                if (r == 4) {
                  sig = fmaf(L.qn[j * 4 + 0], gpre[u].x, sig);
                  sig = fmaf(L.qn[j * 4 + 1], gpre[u].y, sig);
                  sig = fmaf(L.qn[j * 4 + 2], gpre[u].z, sig);
                  sig = fmaf(L.qn[j * 4 + 3], gpre[u].w, sig);
                } else {
                  for (int e = 0; e < r; ++e) sig = fmaf(L.qn[j * r + e], gv[(size_t)ri * r + e], sig);
                }
              }
              L.sb[j][ri] = acc[i] * s.tau;
              L.lam[j][ri] = sig * s.tau2;
            }
          }
        }
      }
    } else {
      // f32 storage: vector ALU, D/8 lanes per row
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
        if (ranked) {
          for (int e = c; e < r; e += LPR) {
            const float gve = gv[(size_t)ri * r + e];
#pragma unroll
            for (int j = 0; j < G; ++j) sig[j] = fmaf(L.qn[j * r + e], gve, sig[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float d = group_sum<LPR>(dot[j]);
          const float v = group_sum<LPR>(sig[j]);
          if (c == 0) {
            L.sb[j][ri] = d * s.tau;
            L.lam[j][ri] = v * s.tau2;
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- per head: chunk max, Z_hat part, compensation weights, log-scores ----
  if (need_mu) {
    const Coh hdr(w.fhdr + (size_t)bg * s.n_chunks * G, (size_t)s.n_chunks * G * 8);
    for (int j = wave; j < G; j += NW) {
      float mx = -INFINITY;
      for (int ri = lane; ri < nrows; ri += 64) mx = fmaxf(mx, L.sb[j][ri]);
      mx = wave_max(mx);
      float z = 0.f;
      for (int ri = lane; ri < nrows; ri += 64) {
        const int n = min(s.bs, Lseq - (start + ri) * s.bs);
        const float sb = L.sb[j][ri], half = 0.5f * L.lam[j][ri];
        const float massf = (float)n * (1.f + half);  // second-order mass estimate / e^{s_bar}
        const float wt = (float)n * expf(sb - mx);
        z = fmaf(wt, 1.f + half, z);
        L.wt[j][ri] = wt;
        L.lam[j][ri] = io.score_mode == kScoreMass ? sb + logf(massf) : sb + logf(massf * half);
      }
      z = wave_sum(z);
      if (lane == 0) {
        L.mx[j] = mx;
        if (ranked)
          hdr.put_u64(chunk * G + j, ((uint64_t)__float_as_uint(z) << 32) | __float_as_uint(mx));
      }
    }
  }
  __syncthreads();

  // ---- selection ----
  const int lo = chunk * s.share, hi = min(kk, lo + s.share);
  const int nb = max(0, hi - lo);
  int32_t* sel_out = (chunk == 0 && io.selected) ? io.selected + (size_t)bg * s.kmax : nullptr;
  if (ranked) {
    // log Z_hat per head from every chunk header of the pair
    const int nh = s.n_chunks * G;
    if (ctl) {
      const Coh hdr(w.fhdr + (size_t)bg * nh, (size_t)nh * 8);
      read_published(hdr, nh, nh, 0, L.u.keys, err);
    }
    __syncthreads();
    for (int j = wave; j < G; j += NW) {
      float mz = -INFINITY;
      for (int ch = lane; ch < s.n_chunks; ch += 64) mz = fmaxf(mz, __uint_as_float((uint32_t)L.u.keys[ch * G + j]));
      mz = wave_max(mz);
      float zs = 0.f;
      for (int ch = lane; ch < s.n_chunks; ch += 64) {
        const uint64_t h = L.u.keys[ch * G + j];
        zs += __uint_as_float((uint32_t)(h >> 32)) * scale_from(__uint_as_float((uint32_t)h), mz);
      }
      zs = wave_sum(zs);
      if (lane == 0) L.lnz[j] = zs > 0.f ? mz + logf(zs) : -INFINITY;
    }
    __syncthreads();
    // ranked score of each block of the chunk
    for (int i = tid; i < nrows; i += NT) {
      float S = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float lam = L.lam[j][i], lz = L.lnz[j];
        if (lam != -INFINITY && lz != -INFINITY) S += expf(lam - lz);
      }
      L.u.keys[i] = make_key(S, start + i);
    }
    __syncthreads();
    // the chunk's top-k candidates
    const Coh cand(w.fcand + (size_t)bg * s.n_chunks * s.kmax, (size_t)s.n_chunks * s.kmax * 8);
    const int k1 = min(kk, nrows);
    if (k1 > 0) {
      const uint64_t T1 = k1 == nrows ? 0 : radix_kth_largest<NT>(LdsKeys{L.u.keys}, nrows, k1, L.hist, L.sh);
      if (tid == 0) L.count = 0u;
      __syncthreads();
      for (int i = tid; i < nrows; i += NT) {
        const uint64_t key = L.u.keys[i];
        if (key >= T1) cand.put_u64(chunk * s.kmax + (int)atomicAdd(&L.count, 1u), key);
      }
    }
    for (int e = k1 + tid; e < kk; e += NT) cand.put_u64(chunk * s.kmax + e, 1u);  // below every real key
    __syncthreads();
    // the pair's top-k from every chunk's candidates
    const int n2 = s.n_chunks * kk;
    if (ctl) read_published(cand, n2, kk, s.kmax, L.u.keys, err);
    const int words = (M + 31) / 32;
    for (int e = tid; e < words; e += NT) L.bitmap[e] = 0u;
    __syncthreads();
    const uint64_t T = radix_kth_largest<NT>(LdsKeys{L.u.keys}, n2, kk, L.hist, L.sh);
    for (int e = tid; e < n2; e += NT) {
      const uint64_t key = L.u.keys[e];
      const int idx = key_index(key);
      if (key >= T && idx >= 0 && idx < M) atomicOr(&L.bitmap[idx >> 5], 1u << (idx & 31));
    }
    __syncthreads();
    emit_selection<NT>(M, L.bitmap, L.wsum, sel_out, kk, L.blk, lo, hi);
  } else {
    // every block selected (kk == M), or none (kk == 0)
    for (int e = tid; e < nb; e += NT) L.blk[e] = lo + e;
    if (sel_out)
      for (int i = tid; i < kk; i += NT) sel_out[i] = i;
    __syncthreads();
  }
  if (chunk == 0) {
    if (tid == 0 && io.num_selected) io.num_selected[bg] = kk;
    if (sel_out)
      for (int e = kk + tid; e < s.kmax; e += NT) sel_out[e] = -1;
  }

  // ---- pages of this workgroup's share of the selected blocks ----
  if (ctl) {
    for (int e = ct; e < nb; e += NCTL) {
      const int i = L.blk[e];
      int p = -1, n = 0;
      if (i >= 0 && i < M) {
        p = io.block_table[(size_t)b * s.max_blocks + i];
        if (p < 0 || p >= s.P) p = -1;
        else n = min(s.bs, Lseq - i * s.bs);
      }
      L.pg[e] = p;
      L.nn[e] = n;
    }
  }
  __syncthreads();

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  if (ctl) {
    // ---- exact attention over the share's tokens (control waves) ----
    constexpr int UG = 2;  // token rows per lane per batch
    const KV* kc = static_cast<const KV*>(io.k_cache);
    const KV* vc = static_cast<const KV*>(io.v_cache);
    float qv[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[j][e] = L.qf[j * D + c * 8 + e];
    const int ntok = nb * kBlockSize;
    const int nbatch = (ntok + RS * UG - 1) / (RS * UG);
    Raw8<KV> kr[UG], vr[UG];
    bool ok[UG];
    // software pipeline: the next batch is in flight while this one is used
#define CKV_ISSUE(BI)                                                                   \
  _Pragma("unroll") for (int u = 0; u < UG; ++u) {                                      \
    const int R = ((BI) * UG + u) * RS + rs;                                            \
    const int bl = R / kBlockSize, tok = R % kBlockSize;                                \
    ok[u] = R < ntok && L.pg[bl] >= 0 && tok < L.nn[bl];                                \
    if (ok[u]) {                                                                        \
      const size_t off = (((size_t)L.pg[bl] * s.Hkv + g) * s.bs + tok) * D + c * 8;     \
      raw_load(kc + off, kr[u]);                                                        \
      raw_load(vc + off, vr[u]);                                                        \
    }                                                                                   \
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
  } else if (comp) {
    // ---- compensation of the chunk's omitted blocks (value waves) ----
#pragma unroll
    for (int j = 0; j < G; ++j) m[j] = L.mx[j];
#pragma unroll
    for (int jj = 0; jj < RPL; ++jj) {
      const int ri = rs + jj * RS;
      if (ri < nrows) {
        const int blk = start + ri;
        const bool taken = ranked && ((L.bitmap[blk >> 5] >> (blk & 31)) & 1u);
        if (!taken) {
          Raw8<KV> raw;
          if constexpr (MF) {
            raw.a = buf[jj];
          } else {
            raw.a = buf[2 * jj];
            raw.b = buf[2 * jj + 1];
          }
          float x[8];
          raw_float(raw, x);
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const float wt = L.wt[j][ri];
            l[j] += wt;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(wt, x[e], acc[j][e]);
          }
        }
      }
    }
  }

  // ---- one partial per head: combine row slots, then waves ----
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float mw = m[j];
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) mw = fmaxf(mw, __shfl_xor(mw, o, 64));
    const float f = scale_from(m[j], mw);
    float lj = l[j] * f;
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = acc[j][e] * f;
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      lj += __shfl_xor(lj, o, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += __shfl_xor(a[e], o, 64);
    }
    if (lane < LPR) {
      float* rw = L.u.red[wave][j];
#pragma unroll
      for (int e = 0; e < 8; ++e) rw[4 + c * 8 + e] = a[e];
      if (c == 0) {
        rw[0] = mw;
        rw[1] = lj;
      }
    }
  }
  __syncthreads();
  {
    const Coh part(w.cpart + ((size_t)bg * s.n_chunks + chunk) * G * PST, (size_t)G * PST * 4);
    for (int o = tid; o < G * D / 4; o += NT) {
      const int j = o / (D / 4), d4 = o % (D / 4);
      float Mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < NW; ++v) Mx = fmaxf(Mx, L.u.red[v][j][0]);
      float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
      float Ls = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const float* rw = L.u.red[v][j];
        const float f = scale_from(rw[0], Mx);
        A.x = fmaf(rw[4 + 4 * d4 + 0], f, A.x);
        A.y = fmaf(rw[4 + 4 * d4 + 1], f, A.y);
        A.z = fmaf(rw[4 + 4 * d4 + 2], f, A.z);
        A.w = fmaf(rw[4 + 4 * d4 + 3], f, A.w);
        Ls = fmaf(rw[1], f, Ls);
      }
      part.put4(j * PST + 4 + 4 * d4, A);
      if (d4 == 0) {
        part.put(j * PST, Mx);
        part.put(j * PST + 1, Ls);
      }
    }
  }
  return arrive(w.ctrl + kCtrlHeader + 4 * bg + 2, &L.slot) == (uint32_t)(s.n_chunks - 1);
}

// Merge the pair's chunk partials into out and lse; clear the pair's
// published words and counter.
template <int D, int G>
__device__ void fused_merge(const Shape& s, const StepIO& io, const Work& w, int bg, FusedLds<D, G>& L) {
  constexpr int PST = kPartStride(D), NV = G * D / 4, TPO = NT / NV, NW = NT / 64;
  constexpr int PB = 8;   // partials per thread per round trip
  static_assert(NV <= NT && TPO <= 64, "one float4 output per group of lanes");
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = s.n_chunks;
  const Coh part(w.cpart + (size_t)bg * nch * G * PST, (size_t)nch * G * PST * 4);
  const int o = tid / TPO, sub = tid % TPO;
  const int j = o / (D / 4), d4 = o % (D / 4);
  // (max, sum) of every partial and the first batch of accumulators, together
  float mi = 0.f, li = 0.f;
  if (tid < nch * G) {
    mi = part.f32(tid * PST);
    li = part.f32(tid * PST + 1);
  }
  float4 av[PB];
#pragma unroll
  for (int u = 0; u < PB; ++u) {
    const int p = sub + u * TPO;
    av[u] = p < nch ? part.f32x4((p * G + j) * PST + 4 + 4 * d4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (tid < nch * G) {
    L.hdr[2 * tid] = mi;
    L.hdr[2 * tid + 1] = li;
  }
  __syncthreads();
  for (int jj = wave; jj < G; jj += NW) {
    float Mx = -INFINITY;
    for (int p = lane; p < nch; p += 64) Mx = fmaxf(Mx, L.hdr[2 * (p * G + jj)]);
    Mx = wave_max(Mx);
    float Ls = 0.f;
    for (int p = lane; p < nch; p += 64) {
      const float f = scale_from(L.hdr[2 * (p * G + jj)], Mx);
      L.u.fac[p * G + jj] = f;
      Ls = fmaf(L.hdr[2 * (p * G + jj) + 1], f, Ls);
    }
    Ls = wave_sum(Ls);
    if (lane == 0) {
      L.mtot[jj] = Mx;
      L.ltot[jj] = Ls;
    }
  }
  __syncthreads();
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int base = 0; base < nch; base += PB * TPO) {
    if (base > 0) {
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int p = base + sub + u * TPO;
        av[u] = p < nch ? part.f32x4((p * G + j) * PST + 4 + 4 * d4) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int p = base + sub + u * TPO;
      if (p < nch) {
        const float f = L.u.fac[p * G + j];
        a.x = fmaf(av[u].x, f, a.x);
        a.y = fmaf(av[u].y, f, a.y);
        a.z = fmaf(av[u].z, f, a.z);
        a.w = fmaf(av[u].w, f, a.w);
      }
    }
  }
#pragma unroll
  for (int x = 1; x < TPO; x <<= 1) {
    a.x += __shfl_xor(a.x, x, 64);
    a.y += __shfl_xor(a.y, x, 64);
    a.z += __shfl_xor(a.z, x, 64);
    a.w += __shfl_xor(a.w, x, 64);
  }
  if (sub == 0) {
    const float den = L.ltot[j];
    const int h = g * G + j;
    float* op = io.out + ((size_t)b * s.Hq + h) * D + 4 * d4;
    op[0] = den > 0.f ? a.x / den : 0.f;
    op[1] = den > 0.f ? a.y / den : 0.f;
    op[2] = den > 0.f ? a.z / den : 0.f;
    op[3] = den > 0.f ? a.w / den : 0.f;
    if (d4 == 0 && io.lse) io.lse[(size_t)b * s.Hq + h] = den > 0.f ? L.mtot[j] + logf(den) : -INFINITY;
  }
  // leave the pair's published words cleared for the next call
  const int Lseq = clamp_len(io.seq_lens[b], s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = min(M, s.kmax);
  if (kk > 0 && kk < M) {
    const Coh hdr(w.fhdr + (size_t)bg * nch * G, (size_t)nch * G * 8);
    for (int e = tid; e < nch * G; e += NT) hdr.put_u64(e, 0u);
    const Coh cand(w.fcand + (size_t)bg * nch * s.kmax, (size_t)nch * s.kmax * 8);
    for (int e = tid; e < nch * kk; e += NT) cand.put_u64((e / kk) * s.kmax + e % kk, 0u);
  }
  if (tid == 0) st_c(w.ctrl + kCtrlHeader + 4 * bg + 2, 0u);
}

template <typename KV, int D, int G>
__global__ __launch_bounds__(NT) void fused_step_kernel(Shape s, StepIO io, Work w) {
  __shared__ FusedLds<D, G> lds;
  const int chunk = (int)blockIdx.x % s.n_chunks;
  for (int bg = (int)blockIdx.x / s.n_chunks; bg < s.B * s.Hkv; bg += s.bg_round) {
    if (fused_chunk<KV, D, G>(s, io, w, bg, chunk, lds)) fused_merge<D, G>(s, io, w, bg, lds);
    __syncthreads();
  }
}

// Calls f(kernel) with the fused kernel instance for (dtype, D, G).
template <class F>
auto with_fused(const Shape& s, F&& f) {
#define CKV_G(KV, DD)                                          \
  switch (s.G) {                                               \
    case 1: return f(&fused_step_kernel<KV, DD, 1>, 0);        \
    case 2: return f(&fused_step_kernel<KV, DD, 2>, 1);        \
    case 4: return f(&fused_step_kernel<KV, DD, 4>, 2);        \
    default: return f(&fused_step_kernel<KV, DD, 8>, 3);       \
  }
  if (s.dtype == 0) {
    if (s.D == 128) { CKV_G(uint16_t, 128) } else { CKV_G(uint16_t, 64) }
  } else {
    if (s.D == 128) { CKV_G(float, 128) } else { CKV_G(float, 64) }
  }
#undef CKV_G
}

}  // namespace

int fused_resident_workgroups(const Shape& s) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  // occupancy per (device, kernel instance), computed once
  constexpr int kDevices = 64;
  static int cache[kDevices][16];
  const int variant = (s.dtype == 0 ? 0 : 8) + (s.D == 128 ? 0 : 4);
  return with_fused(s, [&](auto fn, int gi) {
    int* slot = dev < kDevices ? &cache[dev][variant + gi] : nullptr;
    int per_cu = slot ? __atomic_load_n(slot, __ATOMIC_RELAXED) : 0;
    if (per_cu <= 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, 0) != hipSuccess) per_cu = 0;
      if (slot && per_cu > 0) __atomic_store_n(slot, per_cu, __ATOMIC_RELAXED);
    }
    return per_cu * cus;
  });
}

hipError_t launch_fused(const Shape& s, const StepIO& io, const Work& w, hipStream_t st) {
  const dim3 grid(s.bg_round * s.n_chunks);
  return with_fused(s, [&](auto fn, int) {
    hipLaunchKernelGGL(fn, grid, dim3(NT), 0, st, s, io, w);
    return hipGetLastError();
  });
}

}  // namespace ckv

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
// Organisation.  Every (sequence, KV head) pair is split into chunks of 256
// blocks.  Every chunk gets a control workgroup of 4 waves, and the pair gets
// n_val value workgroups of 4 waves: one per chunk when the whole grid fits on
// the device at once, else as few as make it fit (down to one per four
// chunks), value workgroup v taking chunks v, v + n_val, ... in turn:
//   a control workgroup loads the chunk's mean keys, grouped variances and
//     page-table entries, computes the block-mean logits on the matrix cores
//     (the G query heads are the rows of a 16x16x32 bf16 MFMA tile),
//     publishes the chunk's header (max logit, partial Z_hat per head; for
//     f32 and the appending instance also its compensation weights), reads
//     every header of the pair, ranks the
//     chunk's blocks, publishes the chunk's top-k candidates, reads every
//     candidate of the pair, finds the pair's top-k, attends exactly to its
//     share of the selected blocks (ranks chunk, chunk + n_chunks, ... of the
//     pair's selection), takes back the compensation terms of the selected
//     blocks of its chunk, folds in the chunk's value sums and publishes
//     one (max, sum, acc[d]) partial per query head;
//   a value workgroup forms the chunk's compensation weights n e^{s_bar - max}
//     itself (bf16 without append: the same matrix-core logits from the same
//     mean keys, which the control workgroup's loads bring into L2, so the
//     same bits; otherwise it waits for the control workgroup's), streams the
//     chunk's mean values, sums the compensation terms of all the chunk's
//     blocks and publishes them for the chunk's control workgroup.
// Then every control workgroup of the pair merges its slice of the pair's
// output from the control workgroups' partials, and chunk 0's advances the
// pair's epoch.
// A wave's memory counter drains in issue order, so the long mean-value
// stream lives in workgroups that never wait on small hand-offs; it starts
// once the mean keys have arrived, so that the ranking does not wait behind
// it, and it is paced, so that it does not slow the hand-offs.
// Hand-offs are 64-bit words read with device-scope loads: headers and
// candidates are never 0 once written (double-buffered by the parity of the
// call's tag, each half cleared during the call after the one that used it);
// weights and partials carry the call's tag in their upper half.  Readers poll such
// words directly, so publishing needs no completion wait.  When the device
// sends workgroups to its XCDs round robin, all workgroups of a pair run on
// one XCD and the words are stored with the default policy, so they are
// handed over in that XCD's L2; otherwise they are written through.
//
// The grid covers bg_round pairs at once and walks the rest in rounds; the
// host launches it only when the whole grid can be resident, so the
// workgroups of a pair can wait for each other.  Every wait is bounded and
// sets the error word when it runs out.
#include <atomic>
#include <type_traits>

#include "step_common.hpp"

namespace ckv {

namespace {

constexpr int NT = 256;                    // threads per workgroup
constexpr int NW = NT / 64;                // waves per workgroup
#ifdef CKV_PHASE_TRACE
// Phase trace, compiled only into a separately built library for timing
// studies: thread 0 of a workgroup stores the constant-rate clock at mark i
// into the sparse-step workspace's per-block score region, which the single
// launch does not otherwise use (32 words per workgroup slot: marks below 24,
// notes from 24; control slots 0..n_chunks-1, value slots n_chunks + chunk).
// Needs that region to hold B * Hkv * 2 * n_chunks * 32 words (true for long
// sequences).
#define CKV_NOTE(slot, i, v)                                                                            \
  do {                                                                                                  \
    if (threadIdx.x == 0)                                                                               \
      reinterpret_cast<uint64_t*>(w.xs)[((size_t)bg * (2 * s.n_chunks) + (slot)) * 32 + (i)] = (v);    \
  } while (0)
#define CKV_MARK(slot, i) CKV_NOTE(slot, i, __builtin_amdgcn_s_memrealtime())
// a slot's mark row, for marks set inside helpers
#define CKV_ROW(slot) (reinterpret_cast<uint64_t*>(w.xs) + ((size_t)bg * (2 * s.n_chunks) + (slot)) * 32)
#define CKV_ROW_MARK(row, i)                                                   \
  do {                                                                          \
    if (threadIdx.x == 0 && (row) != nullptr) (row)[i] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define CKV_ROW(slot) nullptr
#define CKV_ROW_MARK(row, i) \
  do {                       \
    (void)(row);             \
  } while (0)
#define CKV_NOTE(slot, i, v) \
  do {                       \
  } while (0)
#define CKV_MARK(slot, i) CKV_NOTE(slot, i, 0)
#endif

constexpr int kTier1 = 32;  // k > 32: each chunk's candidates read first (plus the next key)
constexpr int kCtrlTail = 4;  // per-pair control words 4-5: the appended tail summary is stored (tagged)
constexpr int kPollBatch = 8;              // published words read per thread per round trip
constexpr uint32_t kPollLimit = 1u << 20;  // re-reads per thread and wait
constexpr int kWStride = kChunk + 1;       // tagged words per head: weights, then the chunk max
constexpr int kXccProbeBlocks = 256;       // workgroups of the XCD placement check
constexpr uint32_t kErrPlacement = 2u;     // error word: a workgroup ran on an XCD it was not placed on

template <int D, int G>
struct CtlLds {
  static constexpr int CPR = D / 8;  // 16-byte pieces per mean-key row
  float qf[NT * 8];       // this KV head's query rows (G * D), then zeros
  float qn[G * D];        // |q_h restricted to channel group t|^2, [G][r]
  float qsq[NT];          // per-thread 8-channel partials of |q|^2
  float sb[G][kChunk];    // block-mean logit tau q.mean_k
  float lam[G][kChunk];   // estimated logit variance, then log of the per-head score
  float wt[G][kChunk];    // compensation weight n e^{s_bar - chunk max}
  float mx[G];            // chunk max of s_bar per head
  float lnz[G];           // log Z_hat per head
  union {
    uint64_t keys[kFusedCand];  // headers, chunk keys, then the pair's candidates
    uint4 stage[NW][16 * CPR];  // mean-key rows in matrix-operand order, per wave
    float red[NW][G][D + 4];    // per-wave partial states
  } u;
  uint32_t hist[512];
  uint32_t bitmap[kMaxBlocks / 32];
  int pgt[kChunk];        // page of each block of the chunk
  int own[kChunk];        // selected blocks of this chunk (local rows, ascending)
  int gblk[kShareMax];    // selected blocks this workgroup attends to, and their pages
  int gpg[kShareMax];
  uint32_t sh[64];
  uint32_t wsum[NW];
  uint32_t count;
  uint32_t wcnt[NW];      // per-wave counts of the tier-2 candidates
  uint64_t tlo;           // lower bound of the pair's k-th largest candidate
  uint64_t surv[64];      // candidates at or above it
  uint32_t nown;          // selected blocks of this chunk
  uint4 tmk[D / 8];       // decode append: the tail block's new mean key (stored bits),
  float tgv[4];           //   its grouped variances (r = 4)
  float tmv[D];           //   and its new mean value as stored
};

template <int D, int G>
struct ValLds {
  float w[G][kChunk];
  float mx[G];
  float red[NW][G][D + 4];
  float sb[G][kChunk];          // bf16 without append: the block-mean logits, formed here
  uint4 stage[NW][16 * D / 8];  //   through the same matrix-operand tiles as the control's
  uint4 tmk[D / 8];             // decode append: the tail block's new mean key (stored bits)
  float tmv[D];                 //   and mean value, as stored
};

template <int D, int G>
struct MergeLds {
  float pm[NT], pl[NT];
  float4 pa[NT];
};

template <int D, int G>
union FusedLds {
  CtlLds<D, G> c;
  ValLds<D, G> v;
  MergeLds<D, G> m;
};

__device__ __forceinline__ uint32_t* ctr_epoch(const Work& w, int bg) { return w.ctrl + kCtrlHeader + kCtrlPerPair * bg + 3; }

__device__ __forceinline__ uint64_t tagged(float x, uint32_t tag) {
  return ((uint64_t)tag << 32) | __float_as_uint(x);
}

// Candidate keys of the step carry the block's page, so that the workgroup
// that attends to a selected block needs no page-table read: score bits (32),
// complemented block index (14), page (18).  They order like make_key - by
// score, then lower block index first - since distinct blocks differ in the
// index bits; the page bits never decide.  Real keys are never 0 or 1.
constexpr uint32_t kNoPage = (1u << kFusedPageBits) - 1;
__device__ __forceinline__ uint64_t fused_key(float score, int idx, int page) {
  return ((uint64_t)__float_as_uint(score) << 32) |
         ((uint64_t)(0x3FFFu - (uint32_t)idx) << kFusedPageBits) | (uint32_t)(page >= 0 ? page : (int)kNoPage);
}
__device__ __forceinline__ int fused_key_index(uint64_t key) {
  return 0x3FFF - (int)((uint32_t)key >> kFusedPageBits);
}
__device__ __forceinline__ int fused_key_page(uint64_t key) {
  const uint32_t p = (uint32_t)key & kNoPage;
  return p == kNoPage ? -1 : (int)p;
}

// Chunk headers and candidates are double-buffered by the parity of the
// call's tag: a call publishes into its own half, and its value workgroups
// clear the other half, which the previous call used and the next call uses.
__device__ __forceinline__ uint64_t* hdr_half(const Shape& s, const Work& w, uint32_t tag) {
  return w.fhdr + (size_t)(tag & 1u) * s.B * s.Hkv * s.n_chunks * s.G;
}
__device__ __forceinline__ uint64_t* cand_half(const Shape& s, const Work& w, uint32_t tag) {
  return w.fcand + (size_t)(tag & 1u) * s.B * s.Hkv * s.n_chunks * max(s.kmax, 1);
}

// Copy n published 64-bit words into dst, waiting for each to become
// nonzero.  Word e is read at index (e / per) * stride + e % per.  Each
// thread's re-reads are bounded in total; running out sets the error word.
__device__ void read_published(const Coh& src, int n, int per, int stride, uint64_t* dst, uint32_t* err) {
  const int t = threadIdx.x;
  uint32_t spins = 0;
  for (int base = 0; base < n; base += NT * kPollBatch) {
    uint64_t v[kPollBatch];
#pragma unroll
    for (int u = 0; u < kPollBatch; ++u) {
      const int e = base + t + u * NT;
      v[u] = e < n ? src.u64((e / per) * stride + e % per) : 1u;
    }
#pragma unroll
    for (int u = 0; u < kPollBatch; ++u) {
      const int e = base + t + u * NT;
      while (v[u] == 0 && spins < kPollLimit) {
        __builtin_amdgcn_s_sleep(1);
        v[u] = src.u64((e / per) * stride + e % per);
        if (++spins == kPollLimit) st_c(err, 1u);
      }
      if (e < n) dst[e] = v[u];
    }
  }
}

// Wait until word i of src carries this call's tag; returns its float.
__device__ __forceinline__ float read_tagged(const Coh& src, int i, uint64_t v, uint32_t tag, uint32_t& spins,
                                             uint32_t* err) {
  while ((uint32_t)(v >> 32) != tag && spins < kPollLimit) {
    __builtin_amdgcn_s_sleep(1);
    v = src.u64(i);
    if (++spins == kPollLimit) st_c(err, 1u);
  }
  return __uint_as_float((uint32_t)v);
}

// Per-thread attention state of G query heads -> one partial per head at
// `part` ([G][D + 2] tagged words: max, sum, acc[D]), combining the row
// slots of each wave with lane swaps, then the waves through LDS.
// With `extra`, the partial published there by another workgroup (same
// layout and tag) is folded in first.
template <int D, int G>
__device__ void publish_partial(float (&m)[G], float (&l)[G], float (&acc)[G][8], float (*red)[G][D + 4],
                                const Coh& part, uint32_t tag, const Coh* extra, uint32_t* err,
                                uint64_t* trace_row = nullptr) {
  constexpr int LPR = D / 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = tid % LPR;
  // the other partial's words for this thread's first output, requested
  // before the reductions so that their round trip overlaps them
  uint64_t x[4] = {0u, 0u, 0u, 0u};
  if (extra && tid < G * D / 2) {
    const int h = (tid / (D / 2)) * (D + 2), d2 = tid % (D / 2);
    x[0] = extra->u64(h);
    x[1] = extra->u64(h + 1);
    x[2] = extra->u64(h + 2 + 2 * d2);
    x[3] = extra->u64(h + 3 + 2 * d2);
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    uint32_t mb = __float_as_uint(m[j]);
    if (LPR == 8) mb = OpFmax{}(mb, dpp_row_ror8(mb));
    const float mw = __uint_as_float(across_rows(mb, OpFmax{}));
    const float f = fscale(m[j], mw);
    uint32_t lb = __float_as_uint(l[j] * f);
    if (LPR == 8) lb = OpFadd{}(lb, dpp_row_ror8(lb));
    const float lw = __uint_as_float(across_rows(lb, OpFadd{}));
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t ab = __float_as_uint(acc[j][e] * f);
      if (LPR == 8) ab = OpFadd{}(ab, dpp_row_ror8(ab));
      a[e] = __uint_as_float(across_rows(ab, OpFadd{}));
    }
    if (lane < LPR) {
      float* rw = red[wave][j];
#pragma unroll
      for (int e = 0; e < 8; ++e) rw[4 + c * 8 + e] = a[e];
      if (c == 0) {
        rw[0] = mw;
        rw[1] = lw;
      }
    }
  }
  __syncthreads();
  CKV_ROW_MARK(trace_row, 10);
  for (int o = tid; o < G * D / 2; o += NT) {
    const int j = o / (D / 2), d2 = o % (D / 2);
    float Mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) Mx = fmaxf(Mx, red[v][j][0]);
    float a0 = 0.f, a1 = 0.f, Ls = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float* rw = red[v][j];
      const float f = fscale(rw[0], Mx);
      a0 = fmaf(rw[4 + 2 * d2], f, a0);
      a1 = fmaf(rw[4 + 2 * d2 + 1], f, a1);
      Ls = fmaf(rw[1], f, Ls);
    }
    const int h = j * (D + 2);
    if (extra) {
      uint32_t spins = 0;
      const bool first = o == tid;
      const uint64_t w0 = first ? x[0] : extra->u64(h), w1 = first ? x[1] : extra->u64(h + 1),
                     w2 = first ? x[2] : extra->u64(h + 2 + 2 * d2), w3 = first ? x[3] : extra->u64(h + 3 + 2 * d2);
      const float me = read_tagged(*extra, h, w0, tag, spins, err);
      const float le = read_tagged(*extra, h + 1, w1, tag, spins, err);
      const float e0 = read_tagged(*extra, h + 2 + 2 * d2, w2, tag, spins, err);
      const float e1 = read_tagged(*extra, h + 3 + 2 * d2, w3, tag, spins, err);
      const float M = fmaxf(Mx, me), f1 = fscale(Mx, M), f2 = fscale(me, M);
      a0 = a0 * f1 + e0 * f2;
      a1 = a1 * f1 + e1 * f2;
      Ls = Ls * f1 + le * f2;
      Mx = M;
      if (o == tid) CKV_ROW_MARK(trace_row, 15);
    }
    part.put_u64(h + 2 + 2 * d2, tagged(a0, tag));
    part.put_u64(h + 3 + 2 * d2, tagged(a1, tag));
    if (d2 == 0) {
      part.put_u64(h, tagged(Mx, tag));
      part.put_u64(h + 1, tagged(Ls, tag));
    }
  }
}

// This thread's 8-channel slice of the G query rows, as the dot products
// with a key slice want it: bf16 pairs for bf16 keys (multiplied exactly,
// summed in fp32 by v_dot2), fp32 otherwise.
template <typename KV, int G> struct QSlice;
template <int G> struct QSlice<uint16_t, G> {
  uint32_t p[G][4];
  __device__ __forceinline__ void set(const float* qf, int D, int c) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)  // the floats hold bf16 values: their upper halves are the bf16 bits
        p[j][e] = (__float_as_uint(qf[j * D + c * 8 + 2 * e]) >> 16) |
                  (__float_as_uint(qf[j * D + c * 8 + 2 * e + 1]) & 0xFFFF0000u);
  }
  __device__ __forceinline__ void dot(const Raw8<uint16_t>& k, float (&d)[G]) const {
    const uint32_t kw[4] = {k.a.x, k.a.y, k.a.z, k.a.w};
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw[e]), __builtin_bit_cast(bf16x2_t, p[j][e]),
                                            a, false);
      d[j] = a;
    }
  }
};
template <int G> struct QSlice<float, G> {
  float q[G][8];
  __device__ __forceinline__ void set(const float* qf, int D, int c) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) q[j][e] = qf[j * D + c * 8 + e];
  }
  __device__ __forceinline__ void dot(const Raw8<float>& k, float (&d)[G]) const {
    float x[8];
    raw_float(k, x);
    dot8<G>(q, x, d);
  }
};

// Exact attention to up to N token rows (row slot u in use on every lane of
// its row, or on none): the logits of all of them first, then one online
// update per head, so that the state's max moves once per batch.
template <typename KV, int G, int LPR, int N>
__device__ __forceinline__ void attend_rows(float (&m)[G], float (&l)[G], float (&acc)[G][8], const QSlice<KV, G>& q,
                                            const Raw8<KV> (&kr)[N], const Raw8<KV> (&vr)[N], const bool (&use)[N],
                                            float tau) {
  float x[N][G], mn[G];
#pragma unroll
  for (int j = 0; j < G; ++j) mn[j] = m[j];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    if (use[u]) {
      float d[G];
      q.dot(kr[u], d);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        x[u][j] = token_row_sum<LPR>(d[j]) * tau;
        mn[j] = fmaxf(mn[j], x[u][j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float sc = fscale(m[j], mn[j]);
    l[j] *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] *= sc;
    m[j] = mn[j];
  }
#pragma unroll
  for (int u = 0; u < N; ++u) {
    if (use[u]) {
      float v8[8];
      raw_float(vr[u], v8);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float p = fexp(x[u][j] - m[j]);
        l[j] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(p, v8[e], acc[j][e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Control workgroup of chunk `chunk` of pair bg.
// ---------------------------------------------------------------------------
template <typename KV, int D, int G, bool kR4, bool kApp>
__device__ void ctl_chunk(const Shape& s, const StepIO& io, const Work& w, int bg, int chunk, uint32_t tag,
                          CtlLds<D, G>& L) {
  constexpr int LPR = D / 8, RS = NT / LPR;
  constexpr int KT = D / 32, CPR = D / 8, RPI = 64 / CPR, NMU = CPR;  // NMU: 64 rows per wave / RPI
  constexpr bool MF = std::is_same<KV, uint16_t>::value;
  constexpr bool kOwnW = MF && !kApp;  // the value workgroups form the weights themselves
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rs = tid / LPR, c = tid % LPR;  // row slot, 8-channel slice
  const int start = chunk * kChunk;
  const size_t row0 = (size_t)bg * s.max_blocks + start;  // logical summary row of the chunk
  const KV* mk = static_cast<const KV*>(io.summ.mean_k) + row0 * D;
  const KV* mv = static_cast<const KV*>(io.summ.mean_v) + row0 * D;
  const int r = s.r, gs = D / r;
  const float* gv = io.summ.gvar + row0 * r;
  uint32_t* err = w.ctrl + 2;

  // ---- loads, all issued at once, oldest first: q, page-table entries, the
  // matrix-operand rows of q, then the chunk's mean keys and variances.
  // They do not wait for the sequence length: the views end at the chunk's
  // last row of the summary store (max_blocks rows per pair, all allocated),
  // rows at or past the sequence's end are read but never used, and rows
  // past the store read 0. ----
  const int nmax = max(0, min(s.max_blocks, start + kChunk) - start);
  const Buf qb(static_cast<const KV*>(io.q) + ((size_t)b * s.Hq + g * G) * D, G * D * sizeof(KV));
  const Buf btb(io.block_table + (size_t)b * s.max_blocks + start, nmax * 4);
  const Buf mkb(mk, MF ? nmax * D * sizeof(KV) : 0);
  const Buf gvb(gv, nmax * r * 4);
  Raw8<KV> qraw;
  raw_load(qb, tid * 8, qraw);  // threads past G * D / 8 read 0
  const int pge = (int)btb.u32(4 * tid);
  bf16x8_t qa[KT];
  uint4 mu[NMU];
  // Grouped variances in registers: with r = 4 the four rows of this lane's
  // matrix-core results (16 bytes each); otherwise this thread's block row
  // (row tid of the chunk) when r <= 16, else read later from memory.
  constexpr int kRReg = 16;
  float gvr[kRReg];
  const bool holder = (lane >> 4) * 4 < G;
  if constexpr (MF) {
    const int head = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
      qa[kt] = __builtin_bit_cast(bf16x8_t, qb.u128(2 * (head * D + 32 * kt + 8 * kq)));  // 0 past G
#pragma unroll
    for (int u = 0; u < NMU; ++u) {
      const int row = 64 * wave + RPI * u + lane / CPR;
      mu[u] = mkb.u128(2 * (row * D + (lane % CPR) * 8));
    }
    if constexpr (kR4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 v = gvb.f128(16 * (64 * wave + 16 * u + (lane & 15)));
        gvr[4 * u] = v.x;
        gvr[4 * u + 1] = v.y;
        gvr[4 * u + 2] = v.z;
        gvr[4 * u + 3] = v.w;
      }
    } else if (r < 4) {  // r in {1, 2}: the row's r floats
#pragma unroll
      for (int e = 0; e < kRReg; ++e) gvr[e] = e < r ? __uint_as_float(gvb.u32(4 * (tid * r + e))) : 0.f;
    } else {  // r a multiple of 4: up to 16 floats in 16-byte pieces
#pragma unroll
      for (int q = 0; q < kRReg / 4; ++q) {
        const float4 v = 4 * q < r && r <= kRReg ? gvb.f128(4 * (tid * r + 4 * q)) : make_float4(0.f, 0.f, 0.f, 0.f);
        gvr[4 * q] = v.x;
        gvr[4 * q + 1] = v.y;
        gvr[4 * q + 2] = v.z;
        gvr[4 * q + 3] = v.w;
      }
    }
  }

  const int Lseq = clamp_len(ld_uniform(io.seq_lens + b), s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = min(M, s.kmax);
  const bool ranked = kk > 0 && kk < M;
  const bool need_mu = kk < M;  // logits of omitted blocks are needed
  const bool comp = need_mu && io.compensate;
  const int nrows = max(0, min(M, start + kChunk) - start);
  // Decode append (kApp): the sequence's last token is new.  The value
  // workgroup of the chunk holding its block (row ti of the chunk) writes it
  // into its page slot and recomputes and stores the block's summary
  // (append_tail); this control workgroup reads that summary back and forms
  // the row's logits again.
  static_assert(!kApp || (MF && kR4 && D == 128), "the appending instance is bf16, d = 128, r = 4");
  bool app = false;
  int ti = 0;
  if constexpr (kApp) {
    if (M > 0 && chunk == (M - 1) / kChunk) {
      const int tpage = ld_uniform(io.block_table + (size_t)b * s.max_blocks + M - 1);
      app = tpage >= 0 && tpage < s.P;
      ti = M - 1 - start;
    }
  }

  CKV_MARK(chunk, 0);
  CKV_NOTE(chunk, 25, __builtin_amdgcn_s_memtime());
  // q rows to LDS; partial |q|^2 of each thread's 8 channels
  {
    float x[8];
    raw_float(qraw, x);
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sq = fmaf(x[e], x[e], sq);
    // every thread stores (zeros past G * D / 8), so the load is not sunk
    // below the mean-key loads into a branch
#pragma unroll
    for (int e = 0; e < 8; ++e) L.qf[tid * 8 + e] = x[e];
    L.qsq[tid] = sq;
  }
  L.pgt[tid] = tid < nrows && pge >= 0 && pge < s.P ? pge : -1;
  __syncthreads();
  // |q_h restricted to channel group t|^2, from the 8-channel partials when
  // a group spans whole partials
  for (int item = tid; item < G * r; item += NT) {
    const int j = item / r, tg = item % r;
    float a = 0.f;
    if (gs >= 8) {
      const float* part = L.qsq + (j * D + tg * gs) / 8;
      for (int cc = 0; cc < gs / 8; ++cc) a += part[cc];
    } else {
      const float* qh = L.qf + j * D + tg * gs;
      for (int cc = 0; cc < gs; ++cc) a = fmaf(qh[cc], qh[cc], a);
    }
    L.qn[item] = a;
  }
  __syncthreads();
  CKV_MARK(chunk, 1);

  // ---- block-mean logits and variance estimates ----
  if (need_mu) {
    if constexpr (MF) {
      // Each wave turns its 64 rows, 16 at a time, into matrix operands through
      // its own LDS tile (16-byte pieces swizzled by row, conflict-free both
      // ways).  D[head][row] = sum_k Q[head][k] mean_k[row][k]; lane l holds
      // Q[l%16][8(l/16)..+7] of each 32-wide k-slice (zero rows past G), mean_k
      // of row l%16 at the same k, and receives D[4(l/16)+i][l%16].
      uint4* st = L.u.stage[wave];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
        for (int v = 0; v < 16 / RPI; ++v) {
          const int rr = RPI * v + lane / CPR, ch = lane % CPR;
          st[rr * CPR + (ch ^ (rr & (CPR - 1)))] = mu[g4 * (16 / RPI) + v];
        }
        __builtin_amdgcn_wave_barrier();
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int rr = lane & 15, ch = 4 * kt + (lane >> 4);
          const uint4 bv = st[rr * CPR + (ch ^ (rr & (CPR - 1)))];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kt], __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
        const int ri = 64 * wave + 16 * g4 + (lane & 15);
        if (ri < nrows && holder) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 4 * (lane >> 4) + i;
            if (j < G) {
              L.sb[j][ri] = acc[i] * s.tau;
              if constexpr (kR4) {  // variance estimate: sum_t |q_t|^2 gvar_t
                float sig = 0.f;
                if (ranked) {
                  sig = fmaf(L.qn[j * 4 + 0], gvr[4 * g4 + 0], sig);
                  sig = fmaf(L.qn[j * 4 + 1], gvr[4 * g4 + 1], sig);
                  sig = fmaf(L.qn[j * 4 + 2], gvr[4 * g4 + 2], sig);
                  sig = fmaf(L.qn[j * 4 + 3], gvr[4 * g4 + 3], sig);
                }
                L.lam[j][ri] = sig * s.tau2;
              }
            }
          }
        }
      }
      if constexpr (!kR4) {
        // the variance estimate of row tid for every head, from the row's
        // variances in registers (r <= 16) or memory
        if (tid < nrows) {
#pragma unroll
          for (int j = 0; j < G; ++j) {
            float sig = 0.f;
            if (ranked) {
              if (r <= kRReg) {
#pragma unroll
                for (int e = 0; e < kRReg; ++e)
                  if (e < r) sig = fmaf(L.qn[j * r + e], gvr[e], sig);
              } else {
                for (int q = 0; q < r / 4; ++q) {
                  const float4 v = gvb.f128(4 * (tid * r + 4 * q));
                  sig = fmaf(L.qn[j * r + 4 * q], v.x, sig);
                  sig = fmaf(L.qn[j * r + 4 * q + 1], v.y, sig);
                  sig = fmaf(L.qn[j * r + 4 * q + 2], v.z, sig);
                  sig = fmaf(L.qn[j * r + 4 * q + 3], v.w, sig);
                }
              }
            }
            L.lam[j][tid] = sig * s.tau2;
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
  CKV_MARK(chunk, 2);

  // ---- decode append: the tail block's new summary, then its logits again ----
  if constexpr (kApp) {
    if (app) {
      // the tail chunk's value workgroup wrote the new token into its page
      // slot and the block's new summary, then raised the pair's tail word
      const Coh tw(w.ctrl + kCtrlHeader + kCtrlPerPair * bg + kCtrlTail, 8, s.n_xcd > 0);
      if (tid == 0) {
        uint32_t spins = 0;
        read_tagged(tw, 0, tw.u64(0), tag, spins, err);
        tw.put_u64(0, 0u);  // the word's only reader: it ends the call zero
      }
      __syncthreads();
      const size_t srow = (size_t)bg * s.max_blocks + M - 1;
      const Coh smk(static_cast<const KV*>(io.summ.mean_k) + srow * D, D * sizeof(KV), false);
      const Coh smv(static_cast<const KV*>(io.summ.mean_v) + srow * D, D * sizeof(KV), false);
      const Coh sgv(io.summ.gvar + srow * 4, 16, false);
      if (tid < LPR) {
        const float4 v = smk.f32x4(4 * tid);
        L.tmk[tid] = make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                                __float_as_uint(v.w));
      } else if (tid < 2 * LPR) {
        const float4 v = smv.f32x4(4 * (tid - LPR));
        const uint32_t wv[4] = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                                __float_as_uint(v.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          L.tmv[(tid - LPR) * 8 + 2 * e] = __uint_as_float(wv[e] << 16);
          L.tmv[(tid - LPR) * 8 + 2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
        }
      } else if (tid < 2 * LPR + 4) {
        L.tgv[tid - 2 * LPR] = sgv.f32(tid - 2 * LPR);
      }
      __syncthreads();
      if (need_mu && wave == ti / 64) {
        // the tail row's block-mean logits and variance estimates again, on
        // the same matrix-core path (other rows of the tile are not used)
        const int rr = ti % 16;
        uint4* st = L.u.stage[wave];
        if (lane < CPR) st[rr * CPR + (lane ^ (rr & (CPR - 1)))] = L.tmk[lane];
        __builtin_amdgcn_wave_barrier();
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          // this lane's q operand again, from the float copy in LDS (exact
          // bf16 values; zeros past G), as the loads gave it
          const float* qp = L.qf + (lane & 15) * D + 32 * kt + 8 * (lane >> 4);
          uint4 qw;
          qw.x = (__float_as_uint(qp[0]) >> 16) | (__float_as_uint(qp[1]) & 0xffff0000u);
          qw.y = (__float_as_uint(qp[2]) >> 16) | (__float_as_uint(qp[3]) & 0xffff0000u);
          qw.z = (__float_as_uint(qp[4]) >> 16) | (__float_as_uint(qp[5]) & 0xffff0000u);
          qw.w = (__float_as_uint(qp[6]) >> 16) | (__float_as_uint(qp[7]) & 0xffff0000u);
          const int r2 = lane & 15, ch = 4 * kt + (lane >> 4);
          const uint4 bv = st[r2 * CPR + (ch ^ (r2 & (CPR - 1)))];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qw), __builtin_bit_cast(bf16x8_t, bv),
                                                        acc, 0, 0, 0);
        }
        if ((lane & 15) == rr && holder) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 4 * (lane >> 4) + i;
            if (j < G) {
              L.sb[j][ti] = acc[i] * s.tau;
              float sig = 0.f;
              if (ranked) {
                sig = fmaf(L.qn[j * 4 + 0], L.tgv[0], sig);
                sig = fmaf(L.qn[j * 4 + 1], L.tgv[1], sig);
                sig = fmaf(L.qn[j * 4 + 2], L.tgv[2], sig);
                sig = fmaf(L.qn[j * 4 + 3], L.tgv[3], sig);
              }
              L.lam[j][ti] = sig * s.tau2;
            }
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- per head: chunk max, Z_hat part, compensation weights, log-scores ----
  if (need_mu) {
    const Coh hdr(hdr_half(s, w, tag) + (size_t)bg * s.n_chunks * G, (size_t)s.n_chunks * G * 8, s.n_xcd > 0);
    const Coh wts(w.fw + ((size_t)bg * s.n_chunks + chunk) * G * kWStride, (size_t)G * kWStride * 8, s.n_xcd > 0);
    for (int j = wave; j < G; j += NW) {
      float mx = -INFINITY;
      for (int ri = lane; ri < nrows; ri += 64) mx = fmaxf(mx, L.sb[j][ri]);
      mx = wave_max_dpp(mx);
      float z = 0.f;
      for (int ri = lane; ri < nrows; ri += 64) {
        const int n = min(s.bs, Lseq - (start + ri) * s.bs);
        const float sb = L.sb[j][ri], half = 0.5f * L.lam[j][ri];
        const float massf = (float)n * (1.f + half);  // second-order mass estimate / e^{s_bar}
        const float wt = (float)n * fexp(sb - mx);
        z = fmaf(wt, 1.f + half, z);
        L.wt[j][ri] = wt;
        L.lam[j][ri] = io.score_mode == kScoreMass ? sb + flog(massf) : sb + flog(massf * half);
        if (comp && !kOwnW) wts.put_u64(j * kWStride + ri, tagged(wt, tag));
      }
      z = wave_sum_dpp(z);
      if (lane == 0) {
        L.mx[j] = mx;
        if (ranked) hdr.put_u64(chunk * G + j, ((uint64_t)__float_as_uint(z) << 32) | __float_as_uint(mx));
        if (comp && !kOwnW) wts.put_u64(j * kWStride + kChunk, tagged(mx, tag));
      }
    }
  }
  __syncthreads();
  CKV_MARK(chunk, 3);

  // ---- selection: which blocks this workgroup attends to exactly, and
  // which of the chunk's blocks were selected ----
  int n_own = 0, n_gather = 0;
  bool listed = false;  // selection list (and output) made by the one-wave path
  if (ranked) {
    // log Z_hat per head from every chunk header of the pair
    const int nh = s.n_chunks * G;
    {
      const Coh hdr(hdr_half(s, w, tag) + (size_t)bg * nh, (size_t)nh * 8, s.n_xcd > 0);
      read_published(hdr, nh, nh, 0, L.u.keys, err);
    }
    __syncthreads();
    CKV_MARK(chunk, 4);
    for (int j = wave; j < G; j += NW) {
      float mz = -INFINITY;
      for (int ch = lane; ch < s.n_chunks; ch += 64) mz = fmaxf(mz, __uint_as_float((uint32_t)L.u.keys[ch * G + j]));
      mz = wave_max_dpp(mz);
      float zs = 0.f;
      for (int ch = lane; ch < s.n_chunks; ch += 64) {
        const uint64_t h = L.u.keys[ch * G + j];
        zs += __uint_as_float((uint32_t)(h >> 32)) * fscale(__uint_as_float((uint32_t)h), mz);
      }
      zs = wave_sum_dpp(zs);
      if (lane == 0) L.lnz[j] = zs > 0.f ? mz + flog(zs) : -INFINITY;
    }
    __syncthreads();
    // ranked score of block tid of the chunk (nrows <= NT)
    uint64_t mykey = 0;
    if (tid < nrows) {
      float S = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float lam = L.lam[j][tid], lz = L.lnz[j];
        if (lam != -INFINITY && lz != -INFINITY) S += fexp(lam - lz);
      }
      mykey = fused_key(S, start + tid, L.pgt[tid]);
    }
    // the chunk's top-k candidates, published largest first
    const Coh cand(cand_half(s, w, tag) + (size_t)bg * s.n_chunks * s.kmax, (size_t)s.n_chunks * s.kmax * 8,
                   s.n_xcd > 0);
    const int k1 = min(kk, nrows);
    // k <= 32: the one-wave selection from every chunk's top k.  Larger k
    // (measured: from 33 to 64 blocks too) goes through the two tiers below.
    const bool fast = kk <= 32;
    // k > 32 with room to spare in tier 1 (below): tier 2 is published only
    // when the pair's tier 1 turns out not to hold its top k
    const bool tiered = !fast && s.n_chunks * kTier1 >= 2 * kk && s.n_chunks * (2 * kTier1 + 2) <= kFusedCand;
    // tier 2: the chunk's keys ranked kTier1 + 2 .. k1 (below k_next, its
    // (kTier1 + 1)-th largest), into slots kTier1 + 1.., in row order, then
    // sentinels up to slot k - 1; the chunk's keys are in L.u.keys[0..nrows)
    auto publish_tier2 = [&](uint64_t k_next) {
      const uint64_t T1 = k1 >= nrows ? 0 : radix_kth_largest<NT>(LdsKeys{L.u.keys}, nrows, k1, L.hist, L.sh);
      const bool t2 = tid < nrows && mykey >= T1 && mykey < k_next;
      const uint64_t bt = __ballot(t2);
      if (lane == 0) L.wcnt[wave] = (uint32_t)__popcll(bt);
      __syncthreads();
      int pos = kTier1 + 1 + (int)__popcll(bt & ((1ull << lane) - 1ull));
#pragma unroll
      for (int v = 0; v < NW; ++v) pos += v < wave ? (int)L.wcnt[v] : 0;
      if (t2) cand.put_u64(chunk * s.kmax + pos, mykey);
      for (int e = max(k1, kTier1 + 1) + tid; e < kk; e += NT) cand.put_u64(chunk * s.kmax + e, 1u);
    };
    static_assert(NW == 4, "the chunk's four sorted lists are merged in two rounds");
    // each wave sorts its 64 blocks (L.u.keys[0..nrows) then holds the
    // chunk's keys); waves 0 and 2 merge pairs of lists (the 64 largest of
    // each pair, wave 2's past the chunk's keys), then wave 0 the two results.
    // The appending instance merges the four lists one after another on wave
    // 0 (fewer registers live at once).
    auto chunk_top = [&]() -> uint64_t {
      uint64_t top = wave_sort_desc(mykey);
      L.u.keys[tid] = top;
      __syncthreads();
      if constexpr (kApp) {
        if (wave == 0)
          for (int v = 1; v < NW; ++v) top = wave_merge_desc(top, L.u.keys[64 * v + 63 - lane]);
        return top;
      }
      if ((wave & 1) == 0) {
        top = wave_merge_desc(top, L.u.keys[64 * (wave + 1) + 63 - lane]);
        if (wave == 2) L.u.keys[NT + lane] = top;
      }
      __syncthreads();
      if (wave == 0) top = wave_merge_desc(top, L.u.keys[NT + 63 - lane]);
      return top;  // wave 0: the chunk's 64 largest keys, descending
    };
    if (fast) {
      const uint64_t top = chunk_top();
      if (wave == 0) {
        if (lane < kk) cand.put_u64(chunk * s.kmax + lane, lane < k1 ? top : 1u);  // 1: below every real key
      }
    } else {
      // Two tiers (k > 32).  Tier 1: the chunk's kTier1 largest keys, largest
      // first, in slots 0..kTier1-1, and its next largest key (the largest it
      // leaves out of tier 1) in slot kTier1, from the one-wave path's sorts.
      // Tier 2: the rest of its top k, in slots kTier1+1.., in row order.
      // A pair whose every slot kTier1 lies below the k-th largest tier-1 key
      // needs tier 1 only.
      const uint64_t top = chunk_top();
      if (wave == 0) {
        if (lane <= kTier1) cand.put_u64(chunk * s.kmax + lane, lane < k1 ? top : 1u);  // 1: below every real key
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)top, kTier1);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(top >> 32), kTier1);
        if (lane == 0) L.tlo = k1 > kTier1 + 1 ? ((uint64_t)hi << 32) | lo : 0ull;  // tier 2 lies below it
      }
      __syncthreads();
      if (!tiered) publish_tier2(L.tlo);
    }
    __syncthreads();
    // the pair's top-k from every chunk's candidates
    CKV_MARK(chunk, 5);
    const int n2 = s.n_chunks * kk;
    // k > 32 with room to spare in tier 1: read tier 1 and the slots kTier1
    // first; the full candidates only if some chunk may hold more
    bool tier_ok = false;
    uint64_t T_tier = 0;
    if (tiered) {
      const uint64_t k_next = L.tlo;  // this chunk's (kTier1 + 1)-th largest key
      // slots 0..kTier1 of every chunk in one read (staged past the packed
      // arrays), then tier 1 packed and each chunk's slot kTier1 set aside
      const int n1 = s.n_chunks * kTier1;
      uint64_t* nxt = L.u.keys + n1;              // [n_chunks] each chunk's slot kTier1
      uint64_t* raw = nxt + s.n_chunks;           // [n_chunks][kTier1 + 1]
      read_published(cand, s.n_chunks * (kTier1 + 1), kTier1 + 1, s.kmax, raw, err);
      __syncthreads();
      for (int e = tid; e < s.n_chunks * (kTier1 + 1); e += NT) {
        const int c = e / (kTier1 + 1), i = e % (kTier1 + 1);
        if (i < kTier1) L.u.keys[c * kTier1 + i] = raw[e];
        else nxt[c] = raw[e];
      }
      __syncthreads();
      T_tier = radix_kth_largest<NT>(LdsKeys{L.u.keys}, n1, kk, L.hist, L.sh);
      if (tid == 0) L.count = 0u;
      __syncthreads();
      for (int c = tid; c < s.n_chunks; c += NT)
        if (nxt[c] > T_tier) atomicOr(&L.count, 1u);
      __syncthreads();
      tier_ok = L.count == 0u;  // every key left out of tier 1 lies below T_tier: it is the pair's T
      if (!tier_ok) {
        // the same decision in every workgroup of the pair: each publishes
        // its tier 2 now, then reads every candidate
        if (tid < nrows) L.u.keys[tid] = mykey;
        __syncthreads();
        publish_tier2(k_next);
      }
    }
    if (!tier_ok) {
      read_published(cand, n2, kk, s.kmax, L.u.keys, err);
      __syncthreads();
    }
    const int nc = tier_ok ? s.n_chunks * kTier1 : n2;  // candidate keys in L.u.keys
    CKV_MARK(chunk, 6);
    if (fast) {
      // A lower bound of the k-th largest candidate: the k-th largest of the
      // first m candidates of every chunk (at most 64 keys).  The keys at or
      // above it hold the top k; when they fit in one wave they are sorted
      // there, then re-sorted by block index, which gives every block's rank.
      if (wave == 0) {
        const int m = min(kk, max(1, 64 / s.n_chunks));
        const int c = lane / m, e = lane % m;
        const uint64_t v = c < s.n_chunks ? L.u.keys[c * kk + e] : 0ull;
        const uint64_t srt = wave_sort_desc(v);
        const int kth = s.n_chunks * m >= kk ? kk - 1 : 63;  // too few keys: no bound (lane 63 holds 0)
        const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)srt, kth);
        const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(srt >> 32), kth);
        if (lane == 0) {
          L.tlo = (hi << 32) | lo;
          L.count = 0u;
        }
      }
      __syncthreads();
      const uint64_t tlo = L.tlo;
      for (int e = tid; e < n2; e += NT) {
        const uint64_t key = L.u.keys[e];
        if (key >= tlo) {
          const uint32_t pos = atomicAdd(&L.count, 1u);
          if (pos < 64) L.surv[pos] = key;
        }
      }
      __syncthreads();
      const uint32_t nsurv = L.count;
      if (nsurv <= 64) {
        listed = true;
        if (wave == 0) {
          // lane e < kk holds the pair's e-th largest key; the chunks' workgroups
          // attend to them round robin in that order
          const uint64_t top = wave_sort_desc(lane < (int)nsurv ? L.surv[lane] : 0ull);
          const int ti = fused_key_index(top);
          const bool real = lane < kk && ti >= 0 && ti < M;
          if (real && lane % s.n_chunks == chunk) {
            L.gblk[lane / s.n_chunks] = ti;
            L.gpg[lane / s.n_chunks] = fused_key_page(top);
          }
          const bool mine = real && ti >= start && ti < start + nrows;
          const uint64_t mb = __ballot(mine);
          if (mine) L.own[__popcll(mb & ((1ull << lane) - 1ull))] = ti - start;
          if (lane == 0) L.nown = (uint32_t)__popcll(mb);
          L.surv[lane] = real ? (uint64_t)ti : ~0ull;  // for the selection output, written last
        }
        __syncthreads();
        n_own = (int)L.nown;
        n_gather = kk > chunk ? (kk - 1 - chunk) / s.n_chunks + 1 : 0;
      }
    }
    if (!listed) {
      const int words = (M + 31) / 32;
      for (int e = tid; e < words; e += NT) L.bitmap[e] = 0u;
      __syncthreads();
      CKV_MARK(chunk, 12);
      const uint64_t T = tier_ok ? T_tier : radix_kth_largest<NT>(LdsKeys{L.u.keys}, n2, kk, L.hist, L.sh);
      CKV_MARK(chunk, 13);
      for (int e0 = tid; e0 < nc; e0 += 4 * NT) {  // four keys requested at a time
        uint64_t kb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kb[u] = e0 + u * NT < nc ? L.u.keys[e0 + u * NT] : 0ull;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = fused_key_index(kb[u]);
          if (e0 + u * NT < nc && kb[u] >= T && idx >= 0 && idx < M) atomicOr(&L.bitmap[idx >> 5], 1u << (idx & 31));
        }
      }
      __syncthreads();
      // selected blocks before each bitmap word (words <= 2 NT), into hist
      {
        const uint32_t w0 = 2 * tid < words ? L.bitmap[2 * tid] : 0u;
        const uint32_t w1 = 2 * tid + 1 < words ? L.bitmap[2 * tid + 1] : 0u;
        const uint32_t c0 = __popc(w0), tot = c0 + __popc(w1);
        const uint32_t inc = wave_scan_incl(tot);
        if (lane == 63) L.sh[wave] = inc;
        __syncthreads();
        uint32_t off = inc - tot;
        for (int v = 0; v < wave; ++v) off += L.sh[v];
        L.hist[2 * tid] = off;
        L.hist[2 * tid + 1] = off + c0;
      }
      CKV_MARK(chunk, 14);
      // this chunk's selected blocks, ascending (kChunk / 32 bitmap words)
      if (wave == 0) {
        const int wd = start / 32 + lane;
        const uint32_t bits = (lane < kChunk / 32 && wd < words) ? L.bitmap[wd] : 0u;
        const uint32_t cnt = __popc(bits);
        const uint32_t inc = wave_scan_incl(cnt);
        uint32_t pos = inc - cnt;
        for (uint32_t x = bits; x; x &= x - 1) L.own[pos++] = 32 * lane + __ffs(x) - 1;
        if (lane == 63) L.count = inc;
      }
      __syncthreads();
      n_own = (int)L.count;
      // The pair's selected blocks are attended to round robin over its chunks
      // in ascending order: this workgroup takes ranks chunk, chunk + n_chunks, ...
      for (int e0 = tid; e0 < nc; e0 += 4 * NT) {  // four keys requested at a time
        uint64_t kb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kb[u] = e0 + u * NT < nc ? L.u.keys[e0 + u * NT] : 0ull;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint64_t key = kb[u];
          const int idx = fused_key_index(key);
          if (e0 + u * NT < nc && key >= T && idx >= 0 && idx < M) {
            const int rank = (int)(L.hist[idx >> 5] + __popc(L.bitmap[idx >> 5] & ((1u << (idx & 31)) - 1u)));
            if (rank % s.n_chunks == chunk) {
              L.gblk[rank / s.n_chunks] = idx;
              L.gpg[rank / s.n_chunks] = fused_key_page(key);
            }
          }
        }
      }
      n_gather = kk > chunk ? (kk - 1 - chunk) / s.n_chunks + 1 : 0;
      __syncthreads();
    }
  } else if (kk == M) {
    // every block selected: each chunk attends to its own
    n_gather = nrows;
    L.gblk[tid] = start + tid;
    L.gpg[tid] = L.pgt[tid];
    __syncthreads();
  }

  CKV_MARK(chunk, 7);
  // ---- exact attention over this workgroup's share of the selected blocks ----
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  {
    // one batch covers UG tokens per row slot (RS * UG tokens), all its loads
    // issued together; the same in every instance, since the rounding of the
    // batched update depends on it
    constexpr int UG = 4;
    const KV* kc = static_cast<const KV*>(io.k_cache);
    const KV* vc = static_cast<const KV*>(io.v_cache);
    QSlice<KV, G> qs;
    qs.set(L.qf, D, c);
    const int ntok = n_gather * kBlockSize;
    // The value workgroup sums the compensation terms of every block of the
    // chunk; the terms of the chunk's selected blocks are taken back here,
    // before any exact term, in the frame of the chunk max.
    const bool take_back = comp && n_own > 0;
    if (take_back) {
#pragma unroll
      for (int j = 0; j < G; ++j) m[j] = L.mx[j];
    }
    for (int t0 = 0; t0 < max(ntok, take_back ? 1 : 0); t0 += RS * UG) {
      Raw8<KV> kr[UG], vr[UG];
      bool ok[UG];
#pragma unroll
      for (int u = 0; u < UG; ++u) {
        const int R = t0 + u * RS + rs;
        const int gi = R < ntok ? R / kBlockSize : 0, tok = R % kBlockSize;
        const int blk = L.gblk[gi], pg = L.gpg[gi];
        ok[u] = R < ntok && pg >= 0 && tok < Lseq - blk * s.bs;
        if (ok[u]) {
          const size_t off = (((size_t)pg * s.Hkv + g) * s.bs + tok) * D + c * 8;
          raw_load(kc + off, kr[u]);
          raw_load(vc + off, vr[u]);
        }
      }
      if (t0 == 0 && take_back) {
        for (int e = rs; e < n_own; e += RS) {
          const int ri = L.own[e];
          float nv[8];
          load8(mv + (size_t)ri * D + c * 8, nv);
          if constexpr (kApp) {
            if (app && ri == ti) {
#pragma unroll
              for (int e2 = 0; e2 < 8; ++e2) nv[e2] = L.tmv[c * 8 + e2];
            }
          }
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const float wt = L.wt[j][ri];
            l[j] -= wt;
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) acc[j][e2] = fmaf(-wt, nv[e2], acc[j][e2]);
          }
        }
      }
      attend_rows<KV, G, LPR, UG>(m, l, acc, qs, kr, vr, ok, s.tau);  // ok: uniform across the row
    }
  }
  CKV_MARK(chunk, 8);
  const Coh part(w.fpart + ((size_t)bg * 2 * s.n_chunks + chunk) * G * (D + 2), (size_t)G * (D + 2) * 8,
                 s.n_xcd > 0);
  // the value workgroup of this chunk publishes its compensation sums first;
  // they are folded into this partial, so the merge reads one per chunk
  const Coh vpart(w.fpart + ((size_t)bg * 2 * s.n_chunks + s.n_chunks + chunk) * G * (D + 2),
                  (size_t)G * (D + 2) * 8, s.n_xcd > 0);
  publish_partial<D, G>(m, l, acc, L.u.red, part, tag, &vpart, err, CKV_ROW(chunk));
  CKV_MARK(chunk, 9);
  CKV_NOTE(chunk, 26, __builtin_amdgcn_s_memtime());

  // ---- the selection outputs ----
  if (chunk == 0) {
    int32_t* out = io.selected ? io.selected + (size_t)bg * s.kmax : nullptr;
    if (tid == 0 && io.num_selected) io.num_selected[bg] = kk;
    if (out) {
      for (int e = kk + tid; e < s.kmax; e += NT) out[e] = -1;
      if (ranked) {
        if (!listed) {
          emit_selection<NT>(M, L.bitmap, L.wsum, out, kk, nullptr, 0, 0);
        } else if (wave == 0) {
          // by ascending block index: a block's place is the number of selected
          // blocks with a lower index (the indices differ)
          const uint64_t sv = L.surv[lane];
          const bool real = lane < kk && sv != ~0ull;
          const int ti = (int)(uint32_t)sv;
          const int nreal = __popcll(__ballot(real));  // the real entries come first
          int rank = 0;
          for (int e = 0; e < nreal; ++e) rank += (int)(uint32_t)L.surv[e] < ti ? 1 : 0;  // LDS broadcast
          if (real) out[rank] = ti;
          else if (lane >= nreal && lane < kk) out[lane] = -1;
        }
      } else
        for (int i = tid; i < kk; i += NT) out[i] = i;
    }
  }
}

// ---------------------------------------------------------------------------
// Decode append, run by the value workgroup that sums the tail chunk of pair
// bg before it starts on any chunk: the sequence's last token (row tn - 1 of
// its tail block, in page tpage) is new.  Its key and value rows go into
// their page slot, and the tail block's summary (mean key and value,
// grouped variances, count) is recomputed from the page with the summary
// build's arithmetic and stored; then the pair's tail word is raised with
// this call's tag.  The tail chunk's control workgroup waits for that word
// and reads the summary back.
// ---------------------------------------------------------------------------
template <typename KV, int D, int G>
__device__ void append_tail(const Shape& s, const StepIO& io, const Work& w, int bg, uint32_t tag, ValLds<D, G>& L) {
  static_assert(std::is_same<KV, uint16_t>::value && D == 128, "the appending instance is bf16, d = 128");
  constexpr int LPR = D / 8;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x;
  const int rs = tid / LPR, c = tid % LPR;  // row rs, 8-channel slice c of the 16-row page
  const int Lseq = clamp_len(ld_uniform(io.seq_lens + b), s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  if (M == 0) return;
  const int tpage = ld_uniform(io.block_table + (size_t)b * s.max_blocks + M - 1);
  if (tpage < 0 || tpage >= s.P) return;
  const int tn = Lseq - (M - 1) * s.bs;
  // row rs, slice c of the tail page's keys and values, the new token's row
  // taken from k_new / v_new (the page slot it goes to is not read)
  Raw8<KV> tkr, tvr;
  {
    const KV* ks;
    const KV* vs;
    if (rs == tn - 1) {
      const size_t o = ((size_t)b * s.Hkv + g) * D + c * 8;
      ks = static_cast<const KV*>(io.k_new) + o;
      vs = static_cast<const KV*>(io.v_new) + o;
    } else {
      const size_t o = (((size_t)tpage * s.Hkv + g) * s.bs + rs) * D + c * 8;
      ks = static_cast<const KV*>(io.k_cache) + o;
      vs = static_cast<const KV*>(io.v_cache) + o;
    }
    raw_load(ks, tkr);
    raw_load(vs, tvr);
  }
  L.stage[0][tid] = tkr.a;  // row rs, slice c: row-major, channels in order
  L.stage[1][tid] = tvr.a;
  if (rs == tn - 1) {  // the new token into its page slot
    const size_t o = (((size_t)tpage * s.Hkv + g) * s.bs + rs) * D + c * 8;
    raw_store(static_cast<KV*>(const_cast<void*>(io.k_cache)) + o, tkr);
    raw_store(static_cast<KV*>(const_cast<void*>(io.v_cache)) + o, tvr);
  }
  __syncthreads();
  // one channel per thread (keys, then values), each with the summary
  // build's arithmetic and order for that channel
  float* tvar = reinterpret_cast<float*>(L.stage[2]);  // per-channel key sums of squares
  {
    const bool isv = tid >= D;
    const int ch = tid & (D - 1);
    const uint16_t* rows = reinterpret_cast<const uint16_t*>(L.stage[isv ? 1 : 0]) + ch;
    const float x0 = __uint_as_float((uint32_t)rows[0] << 16);
    float sx = 0.f;
#pragma unroll
    for (int t = 1; t < kBlockSize; ++t)
      if (t < tn) sx += __uint_as_float((uint32_t)rows[t * D] << 16) - x0;
    const float mu = x0 + sx / (float)tn;
    const uint32_t mb = bf16_rne(mu);
    if (isv) {
      L.tmv[ch] = __uint_as_float(mb << 16);
    } else {
      reinterpret_cast<uint16_t*>(L.tmk)[ch] = (uint16_t)mb;
      float var = 0.f;
#pragma unroll
      for (int t = 0; t < kBlockSize; ++t) {
        if (t < tn) {
          const float dl = __uint_as_float((uint32_t)rows[t * D] << 16) - mu;
          var = fmaf(dl, dl, var);
        }
      }
      tvar[ch] = var;
    }
  }
  __syncthreads();
  const size_t srow = (size_t)bg * s.max_blocks + M - 1;
  if (tid < LPR) {
    *reinterpret_cast<uint4*>(static_cast<KV*>(io.summ.mean_k) + srow * D + tid * 8) = L.tmk[tid];
  } else if (tid < 2 * LPR) {
    const float* tv = L.tmv + (tid - LPR) * 8;
    uint4 wb;
    wb.x = (__float_as_uint(tv[0]) >> 16) | (__float_as_uint(tv[1]) & 0xffff0000u);
    wb.y = (__float_as_uint(tv[2]) >> 16) | (__float_as_uint(tv[3]) & 0xffff0000u);
    wb.z = (__float_as_uint(tv[4]) >> 16) | (__float_as_uint(tv[5]) & 0xffff0000u);
    wb.w = (__float_as_uint(tv[6]) >> 16) | (__float_as_uint(tv[7]) & 0xffff0000u);
    *reinterpret_cast<uint4*>(static_cast<KV*>(io.summ.mean_v) + srow * D + (tid - LPR) * 8) = wb;
  } else if (tid < 2 * LPR + 4) {
    // group t of 32 channels: each 8-channel slice summed in order, then
    // the four slices pairwise, as the build sums across its lanes
    const int t = tid - 2 * LPR;
    float sl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sl[i] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sl[i] += tvar[(4 * t + i) * 8 + e];
    }
    io.summ.gvar[srow * 4 + t] = ((sl[0] + sl[1]) + (sl[2] + sl[3])) / ((float)tn * (float)(D / 4));
  } else if (tid == 2 * LPR + 4 && g == 0) {
    io.summ.count[(size_t)b * s.max_blocks + M - 1] = tn;
  }
  // every store of the workgroup in L2 before the tail word
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const Coh tw(w.ctrl + kCtrlHeader + kCtrlPerPair * bg + kCtrlTail, 8, s.n_xcd > 0);
    tw.put_u64(0, tagged(1.f, tag));
  }
}

// ---------------------------------------------------------------------------
// Value workgroup of chunk `chunk` of pair bg: the compensation terms of every
// block of the chunk, n e^{s_bar} mean_v, with the control workgroup's weights.
// ---------------------------------------------------------------------------
template <typename KV, int D, int G, bool kApp>
__device__ void val_chunk(const Shape& s, const StepIO& io, const Work& w, int bg, int chunk, uint32_t tag,
                          ValLds<D, G>& L) {
  constexpr int LPR = D / 8, RS = NT / LPR, RPL = kChunk / RS;
  constexpr int KT = D / 32, CPR = D / 8, RPI = 64 / CPR, NMU = CPR;
  // bf16 without append: the weights are formed here from the chunk's mean
  // keys (in L2, which the control workgroup's loads of the same rows fill),
  // with the control workgroup's arithmetic and so its bits; no hand-off
  constexpr bool kOwn = std::is_same<KV, uint16_t>::value && !kApp;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rs = tid / LPR, c = tid % LPR;
  const int Lseq = clamp_len(ld_uniform(io.seq_lens + b), s.max_blocks * s.bs);
  const int M = (Lseq + s.bs - 1) / s.bs;
  const int kk = min(M, s.kmax);
  const bool comp = kk < M && io.compensate;
  const int start = chunk * kChunk;
  const int nrows = max(0, min(M, start + kChunk) - start);
  const Buf mvb(static_cast<const KV*>(io.summ.mean_v) + ((size_t)bg * s.max_blocks + start) * D,
                nrows * D * sizeof(KV));
  uint32_t* err = w.ctrl + 2;

  float m[G], l[G], acc[G][8];
  CKV_MARK(s.n_chunks + chunk, 0);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  if (comp && kOwn) {
    const Buf qb(static_cast<const KV*>(io.q) + ((size_t)b * s.Hq + g * G) * D, G * D * sizeof(KV));
    const Buf mkb(static_cast<const KV*>(io.summ.mean_k) + ((size_t)bg * s.max_blocks + start) * D,
                  nrows * D * sizeof(KV));
    bf16x8_t qa[KT];
    uint4 mu[NMU];
    const int head = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
      qa[kt] = __builtin_bit_cast(bf16x8_t, qb.u128(2 * (head * D + 32 * kt + 8 * kq)));  // 0 past G
#pragma unroll
    for (int u = 0; u < NMU; ++u) {
      const int row = 64 * wave + RPI * u + lane / CPR;
      mu[u] = mkb.u128(2 * (row * D + (lane % CPR) * 8));
    }
    uint4* st = L.stage[wave];
    const bool holder = (lane >> 4) * 4 < G;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
      for (int v = 0; v < 16 / RPI; ++v) {
        const int rr = RPI * v + lane / CPR, ch = lane % CPR;
        st[rr * CPR + (ch ^ (rr & (CPR - 1)))] = mu[g4 * (16 / RPI) + v];
      }
      __builtin_amdgcn_wave_barrier();
      f32x4_t a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int rr = lane & 15, ch = 4 * kt + (lane >> 4);
        const uint4 bv = st[rr * CPR + (ch ^ (rr & (CPR - 1)))];
        a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kt], __builtin_bit_cast(bf16x8_t, bv), a4, 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
      const int ri = 64 * wave + 16 * g4 + (lane & 15);
      if (ri < nrows && holder) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * (lane >> 4) + i;
          if (j < G) L.sb[j][ri] = a4[i] * s.tau;
        }
      }
    }
    __syncthreads();
    for (int j = wave; j < G; j += NW) {
      float mx = -INFINITY;
      for (int ri = lane; ri < nrows; ri += 64) mx = fmaxf(mx, L.sb[j][ri]);
      mx = wave_max_dpp(mx);
      for (int ri = lane; ri < nrows; ri += 64) {
        const int n = min(s.bs, Lseq - (start + ri) * s.bs);
        L.w[j][ri] = (float)n * fexp(L.sb[j][ri] - mx);
      }
      if (lane == 0) L.mx[j] = mx;
    }
    __syncthreads();
  } else if (comp) {
    const Coh wts(w.fw + ((size_t)bg * s.n_chunks + chunk) * G * kWStride, (size_t)G * kWStride * 8, s.n_xcd > 0);
    uint32_t spins = 0;
    if (tid < G) L.mx[tid] = read_tagged(wts, tid * kWStride + kChunk, wts.u64(tid * kWStride + kChunk), tag, spins, err);
    __syncthreads();
    // this thread's weights: row tid of every head, all requested together
    uint64_t wv[G];
#pragma unroll
    for (int j = 0; j < G; ++j) wv[j] = tid < nrows ? wts.u64(j * kWStride + tid) : 0u;
    if (tid < nrows) {
#pragma unroll
      for (int j = 0; j < G; ++j) L.w[j][tid] = read_tagged(wts, j * kWStride + tid, wv[j], tag, spins, err);
    }
    __syncthreads();
  }
  if (comp) {
#pragma unroll
    for (int j = 0; j < G; ++j) m[j] = L.mx[j];
    CKV_MARK(s.n_chunks + chunk, 1);
    // The mean values stream kValRows rows per thread at a time.  Their sums
    // are needed late (when the control workgroup publishes, some 10 us on),
    // and requesting every row at once floods the memory system while the
    // control workgroups hand headers and candidates to each other: measured,
    // 4 rows at a time beat 2, 8 and all 16.
    constexpr int kValRows = RPL < 4 ? RPL : 4;
#pragma unroll 1
    for (int g0 = 0; g0 < RPL; g0 += kValRows) {
      Raw8<KV> nu[kValRows];
#pragma unroll
      for (int jj = 0; jj < kValRows; ++jj) raw_load(mvb, (rs + (g0 + jj) * RS) * D + c * 8, nu[jj]);  // 0 past the chunk
#pragma unroll
      for (int jj = 0; jj < kValRows; ++jj) {
        const int ri = rs + (g0 + jj) * RS;
        if (ri < nrows) {
          float x[8];
          raw_float(nu[jj], x);
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const float wt = L.w[j][ri];
            l[j] += wt;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(wt, x[e], acc[j][e]);
          }
        }
      }
      asm volatile("" ::: "memory");
    }
  }
  CKV_MARK(s.n_chunks + chunk, 2);
  const Coh part(w.fpart + ((size_t)bg * 2 * s.n_chunks + s.n_chunks + chunk) * G * (D + 2),
                 (size_t)G * (D + 2) * 8, s.n_xcd > 0);
  publish_partial<D, G>(m, l, acc, L.red, part, tag, nullptr, err);
  CKV_MARK(s.n_chunks + chunk, 3);
}

// ---------------------------------------------------------------------------
// Control workgroup `slot` of the pair merges its slice of the pair's output
// from the partials of all the pair's control workgroups (each holding its
// chunk's compensation sums too), waiting for each to carry this call's tag.
// The value workgroups take no part: once their sums are published they
// leave, instead of polling beside the control workgroups on the same CUs.
// ---------------------------------------------------------------------------
template <int D, int G>
__device__ void merge_slice(const Shape& s, const StepIO& io, const Work& w, int bg, int slot, uint32_t epoch,
                            MergeLds<D, G>& L) {
  constexpr int NV = G * D / 4;
  const int b = bg / s.Hkv, g = bg % s.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t tag = epoch + 1u;
  uint32_t* err = w.ctrl + 2;
  const int nm = s.n_chunks;  // merging workgroups of the pair
  const int np = s.n_chunks;  // partials: one per chunk (value sums folded in)
  const int per = (NV + nm - 1) / nm;  // float4 outputs of this workgroup
  const int step = max(1, NT / np);    // outputs merged per pass
  const int o0 = slot * per, o1 = min(NV, o0 + per);
  const Coh part(w.fpart + (size_t)bg * 2 * s.n_chunks * G * (D + 2), (size_t)np * G * (D + 2) * 8,
                 s.n_xcd > 0);
  uint32_t spins = 0;
  for (int base = o0; base < o1; base += step) {
    // the (output, partial) items of this pass: six words each, read together
    const int nout = min(o1 - base, step);
    for (int it = tid; it < nout * np; it += NT) {
      const int o = base + it / np, p = it % np;
      const int j = o / (D / 4), d4 = o % (D / 4);
      const int h = (p * G + j) * (D + 2);
      uint64_t v[6];
      v[0] = part.u64(h);
      v[1] = part.u64(h + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[2 + e] = part.u64(h + 2 + 4 * d4 + e);
      L.pm[it] = read_tagged(part, h, v[0], tag, spins, err);
      L.pl[it] = read_tagged(part, h + 1, v[1], tag, spins, err);
      float4 a;
      a.x = read_tagged(part, h + 2 + 4 * d4, v[2], tag, spins, err);
      a.y = read_tagged(part, h + 3 + 4 * d4, v[3], tag, spins, err);
      a.z = read_tagged(part, h + 4 + 4 * d4, v[4], tag, spins, err);
      a.w = read_tagged(part, h + 5 + 4 * d4, v[5], tag, spins, err);
      L.pa[it] = a;
    }
    __syncthreads();
    if (base == o0) CKV_MARK(slot, 16);
    for (int oo = wave; oo < nout; oo += NW) {
      const int o = base + oo;
      const int j = o / (D / 4), d4 = o % (D / 4);
      float Mx = -INFINITY;
      for (int p = lane; p < np; p += 64) Mx = fmaxf(Mx, L.pm[oo * np + p]);
      Mx = wave_max_dpp(Mx);
      float Ls = 0.f;
      float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int p = lane; p < np; p += 64) {
        const int it = oo * np + p;
        const float f = fscale(L.pm[it], Mx);
        Ls = fmaf(L.pl[it], f, Ls);
        A.x = fmaf(L.pa[it].x, f, A.x);
        A.y = fmaf(L.pa[it].y, f, A.y);
        A.z = fmaf(L.pa[it].z, f, A.z);
        A.w = fmaf(L.pa[it].w, f, A.w);
      }
      Ls = wave_sum_dpp(Ls);
      A.x = wave_sum_dpp(A.x);
      A.y = wave_sum_dpp(A.y);
      A.z = wave_sum_dpp(A.z);
      A.w = wave_sum_dpp(A.w);
      if (lane == 0) {
        const int h = g * G + j;
        float* op = io.out + ((size_t)b * s.Hq + h) * D + 4 * d4;
        op[0] = Ls > 0.f ? A.x / Ls : 0.f;
        op[1] = Ls > 0.f ? A.y / Ls : 0.f;
        op[2] = Ls > 0.f ? A.z / Ls : 0.f;
        op[3] = Ls > 0.f ? A.w / Ls : 0.f;
        if (d4 == 0 && io.lse) io.lse[(size_t)b * s.Hq + h] = Ls > 0.f ? Mx + flog(Ls) : -INFINITY;
      }
    }
    __syncthreads();
  }
  // Every partial of the pair carries this call's tag, so every workgroup of
  // the pair has read the epoch: the workgroup of slot 0 (which reads every
  // partial) advances it for the next call, without waiting for the others.
  if (slot == 0 && tid == 0) st_c(ctr_epoch(w, bg), epoch + 1u);
}

// Brings every 64-byte line of the kernel's explicit arguments into the
// scalar cache with one round of independent loads.  Left to itself the
// compiler loads arguments where they are first used, behind branches on
// other arguments, which costs one memory round trip per line.
__device__ __forceinline__ void warm_kernel_args() {
  typedef const __attribute__((address_space(4))) uint32_t* KArg;
  const KArg ka = (KArg)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int kBytes = (int)(sizeof(Shape) + sizeof(StepIO) + sizeof(Work));
  uint32_t x = 0;
#pragma unroll
  for (int o = 0; o < kBytes; o += 64) x ^= ka[o / 4];
  asm volatile("" ::"s"(x));
}

template <typename KV, int D, int G, bool kR4, bool kApp>
__global__ __launch_bounds__(NT, 2) void fused_step_kernel(Shape s_arg, StepIO io, Work w) {
  __shared__ FusedLds<D, G> lds;
  warm_kernel_args();
  Shape s = s_arg;
  // This workgroup's pair (of the round) and role: control workgroup of
  // chunk `role` (role < n_chunks), else value workgroup role - n_chunks.
  // Kept on one XCD (n_xcd > 0): the device sends workgroup i to XCD
  // (i + c) % n_xcd, with c the same for every workgroup of a launch but not
  // always 0 (it moves between launches).  So the workgroups i / n_xcd = t on
  // XCD x are one each per t, and the one running on XCD x with t takes
  // role t % wpp of pair x + n_xcd * (t / wpp): a pair's workgroups share an
  // XCD whatever c is.  Otherwise control workgroups come first.
  const int wpp = s.n_chunks + s.n_val;  // workgroups per pair
  int pair, role;
  if (s.n_xcd > 0) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
    int x = (int)xcc;
    if (x >= s.n_xcd) {  // not one of the XCDs found at the check: record it, write through
      if (threadIdx.x == 0) st_c(w.ctrl + 2, kErrPlacement);
      x = (int)blockIdx.x % s.n_xcd;
      s.n_xcd = -1;
    }
    const int t = (int)blockIdx.x / s_arg.n_xcd;
    pair = x + s_arg.n_xcd * (t / wpp);
    role = t % wpp;
    if (pair >= s.bg_round) return;
  } else {
    const int half = s.bg_round * s.n_chunks;
    if ((int)blockIdx.x < half) {
      pair = (int)blockIdx.x / s.n_chunks;
      role = (int)blockIdx.x % s.n_chunks;
    } else {
      const int t = (int)blockIdx.x - half;
      pair = t / s.n_val;
      role = s.n_chunks + t % s.n_val;
    }
  }
  for (int bg = pair; bg < s.B * s.Hkv; bg += s.bg_round) {
    const uint32_t epoch = ld_uniform(ctr_epoch(w, bg));  // advanced by the previous call
    if (role < s.n_chunks) {
      ctl_chunk<KV, D, G, kR4, kApp>(s, io, w, bg, role, epoch + 1u, lds.c);
      __syncthreads();
      merge_slice<D, G>(s, io, w, bg, role, epoch, lds.m);
      CKV_MARK(role, 11);
    } else {
      if constexpr (kApp) {
        // the tail chunk's value workgroup appends the new token first
        const int Lq = clamp_len(ld_uniform(io.seq_lens + bg / s.Hkv), s.max_blocks * s.bs);
        const int Mq = (Lq + s.bs - 1) / s.bs;
        if (Mq > 0 && ((Mq - 1) / kChunk) % s.n_val == role - s.n_chunks) {
          append_tail<KV, D, G>(s, io, w, bg, epoch + 1u, lds.v);
          __syncthreads();
        }
      }
      // value workgroup v sums chunks v, v + n_val, ... in turn
      for (int chunk = role - s.n_chunks; chunk < s.n_chunks; chunk += s.n_val) {
        val_chunk<KV, D, G, kApp>(s, io, w, bg, chunk, epoch + 1u, lds.v);
        __syncthreads();
      }
      // then clear its chunks' rows of the previous call's headers and
      // candidates (tag `epoch`), for the next call
      const int kc = max(s.kmax, 1);
      for (int chunk = role - s.n_chunks; chunk < s.n_chunks; chunk += s.n_val) {
        const Coh hdr(hdr_half(s, w, epoch) + ((size_t)bg * s.n_chunks + chunk) * G, (size_t)G * 8, s.n_xcd > 0);
        if ((int)threadIdx.x < G) hdr.put_u64((int)threadIdx.x, 0u);
        const Coh cand(cand_half(s, w, epoch) + ((size_t)bg * s.n_chunks + chunk) * kc, (size_t)kc * 8,
                       s.n_xcd > 0);
        for (int e = (int)threadIdx.x; e < kc; e += NT) cand.put_u64(e, 0u);
      }
    }
    __syncthreads();
  }
}

// Calls f(kernel, index) with the fused kernel instance for (dtype, D, G,
// r == 4, append); index < 32.  bf16 has a separate instance for r == 4,
// which keeps the variances of the rows of its matrix-core results in
// registers; f32 scores on the vector ALU and reads them from memory
// whatever r is.  The appending instances exist for bf16, D = 128, r = 4.
template <class F>
auto with_fused(const Shape& s, F&& f) {
#define CKV_G(KV, DD, R4, I, APP)                                           \
  switch (s.G) {                                                            \
    case 1: return f(&fused_step_kernel<KV, DD, 1, R4, APP>, (I) + 0);      \
    case 2: return f(&fused_step_kernel<KV, DD, 2, R4, APP>, (I) + 1);      \
    case 4: return f(&fused_step_kernel<KV, DD, 4, R4, APP>, (I) + 2);      \
    default: return f(&fused_step_kernel<KV, DD, 8, R4, APP>, (I) + 3);     \
  }
  if (s.append) { CKV_G(uint16_t, 128, true, 24, true) }
  if (s.dtype == 0) {
    if (s.r == 4) {
      if (s.D == 128) { CKV_G(uint16_t, 128, true, 0, false) } else { CKV_G(uint16_t, 64, true, 4, false) }
    } else {
      if (s.D == 128) { CKV_G(uint16_t, 128, false, 8, false) } else { CKV_G(uint16_t, 64, false, 12, false) }
    }
  } else {
    if (s.D == 128) { CKV_G(float, 128, true, 16, false) } else { CKV_G(float, 64, true, 20, false) }
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
  static int cache[kDevices][32];
  return with_fused(s, [&](auto fn, int vi) {
    int* slot = dev < kDevices ? &cache[dev][vi] : nullptr;
    int per_cu = slot ? __atomic_load_n(slot, __ATOMIC_RELAXED) : 0;
    if (per_cu <= 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, 0) != hipSuccess) per_cu = 0;
      if (slot && per_cu > 0) __atomic_store_n(slot, per_cu, __ATOMIC_RELAXED);
    }
    return per_cu * cus;
  });
}

__device__ uint32_t g_xcc_of_block[kXccProbeBlocks];

__global__ void xcc_probe_kernel() {
  if (threadIdx.x == 0) {
    uint32_t id;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(id));
    g_xcc_of_block[blockIdx.x] = id;
  }
}

int fused_xcd_count(hipStream_t st) {
  constexpr int kDevices = 64;
  static std::atomic<int> known[kDevices];  // 0 unknown, -1 not round robin, else XCDs
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 0;
  const int k = known[dev].load(std::memory_order_relaxed);
  if (k != 0) return k > 0 ? k : 0;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return 0;
  uint32_t ids[kXccProbeBlocks];
  hipLaunchKernelGGL(xcc_probe_kernel, dim3(kXccProbeBlocks), dim3(64), 0, st);
  if (hipGetLastError() != hipSuccess ||
      hipMemcpyFromSymbolAsync(ids, HIP_SYMBOL(g_xcc_of_block), sizeof ids, 0, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  // round robin from any starting XCD: workgroup i on XCD (i + c) % n
  uint32_t n = 0;
  for (int i = 0; i < kXccProbeBlocks; ++i) n = ids[i] + 1 > n ? ids[i] + 1 : n;
  bool rr = n >= 1 && n <= 16;
  for (int i = 0; rr && i < kXccProbeBlocks; ++i) rr = ids[i] == (ids[0] + (uint32_t)i) % n;
  known[dev].store(rr ? (int)n : -1, std::memory_order_relaxed);
  return rr ? (int)n : 0;
}

hipError_t launch_fused(const Shape& s, const StepIO& io, const Work& w, hipStream_t st) {
  const int wpp = s.n_chunks + s.n_val;
  const dim3 grid(s.n_xcd > 0 ? s.n_xcd * ((s.bg_round + s.n_xcd - 1) / s.n_xcd) * wpp : s.bg_round * wpp);
  return with_fused(s, [&](auto fn, int) {
    hipLaunchKernelGGL(fn, grid, dim3(NT), 0, st, s, io, w);
    return hipGetLastError();
  });
}

}  // namespace ckv

// C ABI of libcompkv.so: host-side argument checks, workspace carving and
// launch order.  Every check runs before anything is enqueued.
#include <algorithm>
#include <math.h>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/compkv.h"
#include "internal.hpp"
#include "plan.hpp"

// The workspace of ckv_decode_step_noalloc: one copy per device, held until
// the process ends.  Host code never passes this name to a kernel or a copy
// (on the host it is only a stand-in for the symbol): it uses the device
// address that hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) unsigned char scratch[CKV_NOALLOC_WORKSPACE_BYTES];

namespace {

thread_local char g_last_error[256] = "";

ckv_status fail(ckv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

ckv_status ok() {
  g_last_error[0] = '\0';
  return CKV_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Validate dims and fill the kernel-side shape (budget < 0 means "no budget").
ckv_status make_shape(const ckv_dims* d, int32_t budget_tokens, ckv::Shape* s) {
  if (!d) return fail(CKV_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 1) return fail(CKV_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", d->batch);
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(CKV_ERR_INVALID_ARG, "head counts must be >= 1");
  if (d->num_q_heads % d->num_kv_heads)
    return fail(CKV_ERR_INVALID_ARG, "num_q_heads %% num_kv_heads != 0 (%d, %d)", d->num_q_heads,
                d->num_kv_heads);
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(CKV_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", G);
  if (d->num_kv_heads > ckv::kMaxKvHeads)
    return fail(CKV_ERR_UNSUPPORTED, "num_kv_heads > %d", ckv::kMaxKvHeads);
  if (d->head_dim < 1) return fail(CKV_ERR_INVALID_ARG, "head_dim must be >= 1");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(CKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
  if (d->block_size < 1) return fail(CKV_ERR_INVALID_ARG, "block_size must be >= 1");
  if (d->block_size != ckv::kBlockSize)
    return fail(CKV_ERR_UNSUPPORTED, "block_size must be %d (got %d)", ckv::kBlockSize,
                d->block_size);
  if (d->r_groups < 1 || d->head_dim % d->r_groups)
    return fail(CKV_ERR_INVALID_ARG, "r_groups must divide head_dim (r=%d, d=%d)", d->r_groups,
                d->head_dim);
  if (d->num_pages < 1) return fail(CKV_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (d->max_blocks_per_seq < 1)
    return fail(CKV_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  if (d->max_blocks_per_seq > ckv::kMaxBlocks)
    return fail(CKV_ERR_UNSUPPORTED, "max_blocks_per_seq > %d", ckv::kMaxBlocks);
  if (d->kv_dtype != CKV_BF16 && d->kv_dtype != CKV_F32)
    return fail(CKV_ERR_INVALID_ARG, "kv_dtype must be CKV_BF16 or CKV_F32");
  ckv::Shape& x = *s;
  x.B = d->batch;
  x.Hq = d->num_q_heads;
  x.Hkv = d->num_kv_heads;
  x.G = G;
  x.D = d->head_dim;
  x.bs = d->block_size;
  x.r = d->r_groups;
  x.P = d->num_pages;
  x.max_blocks = d->max_blocks_per_seq;
  const int kb = budget_tokens < 0 ? 0 : budget_tokens / d->block_size;
  x.kmax = kb < x.max_blocks ? kb : x.max_blocks;
  x.n_chunks = (x.max_blocks + ckv::kChunk - 1) / ckv::kChunk;
  x.n_slices = (x.max_blocks + ckv::kSlice - 1) / ckv::kSlice;
  x.share = x.kmax > 0 ? (x.kmax + x.n_chunks - 1) / x.n_chunks : 1;
  x.bg_round = 0;
  x.n_xcd = 0;
  x.n_val = x.n_chunks;
  int splits = (x.kmax + ckv::kGatherPages - 1) / ckv::kGatherPages;
  splits = std::min(splits, std::max(1, ckv::kGatherGroups / (x.B * x.Hkv)));
  splits = std::max(splits, (x.kmax + ckv::kShareMax - 1) / ckv::kShareMax);  // a split's blocks fit its LDS
  splits = splits < 1 ? 1 : (splits > ckv::kMaxSplits ? ckv::kMaxSplits : splits);
  x.n_splits = splits;
  x.pages_per_split = x.kmax > 0 ? (x.kmax + splits - 1) / splits : 1;
  x.dtype = d->kv_dtype;
  x.append = 0;
  x.tau = (float)(1.0 / sqrt((double)d->head_dim));
  x.tau2 = (float)(1.0 / (double)d->head_dim);
  if (G * (x.n_chunks + 2 * x.n_splits) > ckv::kMergeFactors)
    return fail(CKV_ERR_UNSUPPORTED, "too many partials for the merge");
  return CKV_OK;
}

struct Layout {
  size_t ctrl, xs, cpart, cand, gpart, fhdr, fcand, fw, fpart, total;
};

size_t ctrl_bytes(const ckv::Shape& s) {
  return align_up((size_t)(ckv::kCtrlHeader + ckv::kCtrlPerPair * s.B * s.Hkv) * sizeof(uint32_t));
}

// Sparse-step workspace: control words, per-block scores, chunk partials,
// first-level select candidates, gather partials, and what the fused step
// hands between workgroups: chunk headers and candidates (zero between
// calls), tagged compensation weights and chunk partials.
Layout layout(const ckv::Shape& s) {
  Layout L;
  const size_t pst = ckv::kPartStride(s.D);
  const size_t bg = (size_t)s.B * s.Hkv;
  const size_t kcap = (size_t)(s.kmax > 0 ? s.kmax : 1);
  size_t off = 0;
  L.ctrl = off;
  off += ctrl_bytes(s);
  L.xs = off;
  off += align_up((size_t)s.B * s.Hq * s.max_blocks * sizeof(float));
  L.cpart = off;
  off += align_up(bg * s.n_chunks * s.G * pst * sizeof(float));
  L.cand = off;
  off += align_up(bg * s.n_slices * kcap * sizeof(uint64_t));
  L.gpart = off;
  off += align_up(bg * s.n_splits * s.G * 2 * pst * sizeof(float));
  L.fhdr = off;
  off += align_up(2 * bg * s.n_chunks * s.G * sizeof(uint64_t));
  L.fcand = off;
  off += align_up(2 * bg * s.n_chunks * kcap * sizeof(uint64_t));
  L.fw = off;
  off += align_up(bg * s.n_chunks * s.G * (ckv::kChunk + 1) * sizeof(uint64_t));
  L.fpart = off;
  off += align_up(bg * 2 * s.n_chunks * s.G * (size_t)(s.D + 2) * sizeof(uint64_t));
  L.total = off;
  return L;
}

ckv::Work carve(const ckv::Shape& s, void* ws) {
  const Layout L = layout(s);
  char* base = static_cast<char*>(ws);
  return ckv::Work{reinterpret_cast<uint32_t*>(base + L.ctrl), reinterpret_cast<float*>(base + L.xs),
                   reinterpret_cast<float*>(base + L.cpart), reinterpret_cast<uint64_t*>(base + L.cand),
                   reinterpret_cast<float*>(base + L.gpart), reinterpret_cast<uint64_t*>(base + L.fhdr),
                   reinterpret_cast<uint64_t*>(base + L.fcand), reinterpret_cast<uint64_t*>(base + L.fw),
                   reinterpret_cast<uint64_t*>(base + L.fpart)};
}

// Dense splits: about 256 workgroups in all (one per CU), a
// multiple of 4 blocks (one per wave) between 8 and kDensePages blocks each,
// and at most 256 splits per (sequence, KV head) so that the merge's factors
// fit its LDS.  Depends on the dims only, so the workspace size does too.
void set_dense(ckv::Shape& s) {
  const long long pairs = (long long)s.B * s.Hkv;
  long long pps = (pairs * s.max_blocks + 255) / 256;
  pps = (pps + 3) / 4 * 4;
  const long long floor_pps = std::max<long long>(8, (s.max_blocks + 255) / 256);
  pps = std::max(pps, (floor_pps + 3) / 4 * 4);
  pps = std::min<long long>(pps, ckv::kDensePages);
  s.pages_per_split = (int)pps;
  s.n_splits = (s.max_blocks + s.pages_per_split - 1) / s.pages_per_split;
}

size_t dense_bytes(const ckv::Shape& s) {
  return ctrl_bytes(s) + align_up((size_t)s.B * s.Hkv * s.n_splits * s.G * ckv::kPartStride(s.D) *
                                  sizeof(float));
}

ckv_status check_summaries(const ckv_summaries* sm) {
  if (!sm) return fail(CKV_ERR_INVALID_ARG, "summaries is NULL");
  if (!sm->mean_k || !sm->mean_v || !sm->gvar || !sm->count)
    return fail(CKV_ERR_INVALID_ARG, "a summaries field is NULL");
  return CKV_OK;
}

ckv_status check_workspace(const ckv::Shape& s, const void* ws, size_t bytes) {
  const size_t need = layout(s).total;
  if (!ws) return fail(CKV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (bytes < need) return fail(CKV_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(CKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return CKV_OK;
}

ckv_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define CKV_TRY(expr)                  \
  do {                                 \
    ckv_status st_ = (expr);           \
    if (st_ != CKV_OK) return st_;     \
  } while (0)

ckv::Summ to_summ(const ckv_summaries* sm) {
  return ckv::Summ{sm->mean_k, sm->mean_v, sm->gvar, sm->count};
}

// The single launch's layout on the current device (see plan.hpp).  Whether
// blocks go to the device's XCDs round robin is checked once per device, and
// not while `stream` is capturing.  Sets s->bg_round, s->n_val and s->n_xcd.
bool plan_fused(ckv::Shape* s, hipStream_t stream, bool probe) {
  ckv::plan::Inputs in;
  in.n_chunks = s->n_chunks;
  in.kmax = s->kmax;
  in.share = s->share;
  in.share_max = ckv::kShareMax;
  in.cand_max = ckv::kFusedCand;
  in.num_pages = s->P;
  in.page_limit = 1 << ckv::kFusedPageBits;
  in.pairs = s->B * s->Hkv;
  in.xcds = 0;
  in.max_rounds = ckv::kFusedMaxRounds;
  // the shape rules first, so that a shape that never fuses queries nothing
  in.resident = 1 << 30;
  if (!ckv::plan::single_launch(in).single) return false;
  in.resident = ckv::fused_resident_workgroups(*s);
  const char* off = getenv("CKV_FUSED_ACROSS_XCDS");
  in.xcds = probe && !(off && off[0] == '1') ? ckv::fused_xcd_count(stream) : 0;
  const ckv::plan::Layout L = ckv::plan::single_launch(in);
  if (!L.single) return false;
  s->n_val = L.n_val;
  s->bg_round = L.bg_round;
  s->n_xcd = L.n_xcd;
  return true;
}

// The single launch that also appends the new tokens: bf16, d = 128, r = 4,
// and every pair's workgroups on one XCD, so that the new token's rows and
// the tail block's summary reach the pair's readers through that XCD's L2.
bool plan_fused_append(ckv::Shape* s, hipStream_t stream, bool probe) {
  if (s->dtype != CKV_BF16 || s->D != 128 || s->r != 4) return false;
  s->append = 1;
  if (plan_fused(s, stream, probe) && s->n_xcd > 0) return true;
  s->append = 0;
  return false;
}

// The arguments of ckv_decode_step other than the workspace.
ckv_status check_step_args(const ckv_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                           const ckv_summaries* summaries, const int32_t* block_table, const int32_t* seq_lens,
                           int32_t budget_tokens, int32_t score_mode, const int32_t* selected,
                           const int32_t* num_selected, const float* out, ckv::Shape* s) {
  if (budget_tokens < 0) return fail(CKV_ERR_INVALID_ARG, "budget_tokens must be >= 0");
  CKV_TRY(make_shape(dims, budget_tokens, s));
  if (!q || !k_cache || !v_cache) return fail(CKV_ERR_INVALID_ARG, "q, k_cache or v_cache is NULL");
  if (!block_table || !seq_lens) return fail(CKV_ERR_INVALID_ARG, "block_table or seq_lens is NULL");
  if (!num_selected || (!selected && s->kmax > 0))
    return fail(CKV_ERR_INVALID_ARG, "selected or num_selected is NULL");
  if (!out) return fail(CKV_ERR_INVALID_ARG, "out is NULL");
  if (score_mode != CKV_SCORE_COMPKV && score_mode != CKV_SCORE_MASS)
    return fail(CKV_ERR_INVALID_ARG, "unknown score_mode %d", score_mode);
  return check_summaries(summaries);
}

// One decode step on checked arguments and a workspace of the step's layout.
ckv_status decode_step_launches(ckv::Shape s, const void* q, const void* k_cache, const void* v_cache,
                                const ckv_summaries* summaries, const int32_t* block_table,
                                const int32_t* seq_lens, int32_t score_mode, int32_t* selected,
                                int32_t* num_selected, float* out, float* lse, void* workspace, hipStream_t st) {
  ckv::StepIO io{q, k_cache, v_cache, to_summ(summaries), block_table, seq_lens, selected,
                 num_selected, nullptr, out, lse, score_mode, 1};
  const ckv::Work w = carve(s, workspace);
  if (plan_fused(&s, st, true)) return hip_status(ckv::launch_fused(s, io, w, st), "decode step launch");
  hipError_t e = ckv::launch_step(s, ckv::kModeScanOnly, io, w, st);
  if (e == hipSuccess) e = ckv::launch_step(s, ckv::kModeSelectOnly, io, w, st);
  if (e == hipSuccess) e = ckv::launch_step(s, ckv::kModeAttendOnly, io, w, st);
  return hip_status(e, "decode step launches");
}

// ---- the built-in workspace of ckv_decode_step_noalloc ----
constexpr int kScratchDevices = 64;
struct ScratchState {
  void* ptr = nullptr;    // this device's copy of `scratch`
  bool laid_out = false;  // holds the clean state of the last call's layout:
  ckv_dims dims{};        //   these dims
  int32_t budget = -1;    //   and this budget
};
std::mutex g_scratch_mu;
ScratchState g_scratch[kScratchDevices];

bool same_dims(const ckv_dims& a, const ckv_dims& b) {
  return a.batch == b.batch && a.num_q_heads == b.num_q_heads && a.num_kv_heads == b.num_kv_heads &&
         a.head_dim == b.head_dim && a.block_size == b.block_size && a.r_groups == b.r_groups &&
         a.num_pages == b.num_pages && a.max_blocks_per_seq == b.max_blocks_per_seq && a.kv_dtype == b.kv_dtype;
}

__global__ void zero_fill_kernel(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's state, its scratch address looked up on first use
// (with the device current).  Called with g_scratch_mu held.
ckv_status scratch_state(ScratchState** out) {
  int dev = 0;
  CKV_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kScratchDevices)
    return fail(CKV_ERR_UNSUPPORTED, "device %d: the built-in workspace serves devices 0..%d", dev,
                kScratchDevices - 1);
  ScratchState& z = g_scratch[dev];
  if (!z.ptr) {
    void* p = nullptr;
    CKV_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p || reinterpret_cast<uintptr_t>(p) % 256)
      return fail(CKV_ERR_HIP, "hipGetSymbolAddress(scratch) gave an unusable address %p", p);
    z.ptr = p;
  }
  *out = &z;
  return CKV_OK;
}

}  // namespace

extern "C" {

const char* ckv_status_string(ckv_status st) {
  switch (st) {
    case CKV_OK: return "CKV_OK";
    case CKV_ERR_INVALID_ARG: return "CKV_ERR_INVALID_ARG";
    case CKV_ERR_UNSUPPORTED: return "CKV_ERR_UNSUPPORTED";
    case CKV_ERR_WORKSPACE: return "CKV_ERR_WORKSPACE";
    case CKV_ERR_HIP: return "CKV_ERR_HIP";
    case CKV_ERR_INCOMPLETE: return "CKV_ERR_INCOMPLETE";
  }
  return "CKV_ERR_UNKNOWN";
}

const char* ckv_last_error(void) { return g_last_error; }

ckv_status ckv_build_summaries(const ckv_dims* dims, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               int32_t append_only, const ckv_summaries* summaries,
                               void* stream) {
  ckv::Shape s;
  CKV_TRY(make_shape(dims, 0, &s));
  if (!k_cache || !v_cache) return fail(CKV_ERR_INVALID_ARG, "k_cache or v_cache is NULL");
  if (!block_table || !seq_lens) return fail(CKV_ERR_INVALID_ARG, "block_table or seq_lens is NULL");
  CKV_TRY(check_summaries(summaries));
  return hip_status(ckv::launch_build_summaries(s, k_cache, v_cache, block_table, seq_lens,
                                                append_only ? 1 : 0, to_summ(summaries),
                                                static_cast<hipStream_t>(stream)),
                    "summary build launch");
}

ckv_status ckv_append_tokens(const ckv_dims* dims, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* block_table,
                             const int32_t* seq_lens, const ckv_summaries* summaries, void* stream) {
  ckv::Shape s;
  CKV_TRY(make_shape(dims, 0, &s));
  if (!k_new || !v_new) return fail(CKV_ERR_INVALID_ARG, "k_new or v_new is NULL");
  if (!k_cache || !v_cache) return fail(CKV_ERR_INVALID_ARG, "k_cache or v_cache is NULL");
  if (!block_table || !seq_lens) return fail(CKV_ERR_INVALID_ARG, "block_table or seq_lens is NULL");
  CKV_TRY(check_summaries(summaries));
  return hip_status(ckv::launch_append_tokens(s, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                              to_summ(summaries), static_cast<hipStream_t>(stream)),
                    "append launch");
}

size_t ckv_workspace_bytes(const ckv_dims* dims, int32_t budget_tokens) {
  ckv::Shape s;
  if (budget_tokens < 0 || make_shape(dims, budget_tokens, &s) != CKV_OK) return 0;
  return layout(s).total;
}

ckv_status ckv_score_select(const ckv_dims* dims, const void* q, const ckv_summaries* summaries,
                            const int32_t* block_table, const int32_t* seq_lens,
                            int32_t budget_tokens, int32_t score_mode, int32_t* selected,
                            int32_t* num_selected, float* group_scores, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (budget_tokens < 0) return fail(CKV_ERR_INVALID_ARG, "budget_tokens must be >= 0");
  ckv::Shape s;
  CKV_TRY(make_shape(dims, budget_tokens, &s));
  if (!q) return fail(CKV_ERR_INVALID_ARG, "q is NULL");
  if (!block_table || !seq_lens) return fail(CKV_ERR_INVALID_ARG, "block_table or seq_lens is NULL");
  if (!num_selected || (!selected && s.kmax > 0))
    return fail(CKV_ERR_INVALID_ARG, "selected or num_selected is NULL");
  if (score_mode != CKV_SCORE_COMPKV && score_mode != CKV_SCORE_MASS)
    return fail(CKV_ERR_INVALID_ARG, "unknown score_mode %d", score_mode);
  CKV_TRY(check_summaries(summaries));
  CKV_TRY(check_workspace(s, workspace, workspace_bytes));
  ckv::StepIO io{q, nullptr, nullptr, to_summ(summaries), block_table, seq_lens, selected,
                 num_selected, group_scores, nullptr, nullptr, score_mode, 1};
  const ckv::Work w = carve(s, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = ckv::launch_step(s, ckv::kModeScanOnly, io, w, st);
  if (e != hipSuccess) return hip_status(e, "scan launch");
  return hip_status(ckv::launch_step(s, ckv::kModeSelectOnly, io, w, st), "select launch");
}

ckv_status ckv_compensated_decode_attention(const ckv_dims* dims, const void* q,
                                            const void* k_cache, const void* v_cache,
                                            const ckv_summaries* summaries,
                                            const int32_t* block_table, const int32_t* seq_lens,
                                            int32_t budget_tokens, const int32_t* selected,
                                            const int32_t* num_selected, int32_t compensate,
                                            float* out, float* lse, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  if (budget_tokens < 0) return fail(CKV_ERR_INVALID_ARG, "budget_tokens must be >= 0");
  ckv::Shape s;
  CKV_TRY(make_shape(dims, budget_tokens, &s));
  if (!q || !k_cache || !v_cache) return fail(CKV_ERR_INVALID_ARG, "q, k_cache or v_cache is NULL");
  if (!block_table || !seq_lens) return fail(CKV_ERR_INVALID_ARG, "block_table or seq_lens is NULL");
  if (!num_selected || (!selected && s.kmax > 0))
    return fail(CKV_ERR_INVALID_ARG, "selected or num_selected is NULL");
  if (!out) return fail(CKV_ERR_INVALID_ARG, "out is NULL");
  CKV_TRY(check_summaries(summaries));
  CKV_TRY(check_workspace(s, workspace, workspace_bytes));
  ckv::StepIO io{q, k_cache, v_cache, to_summ(summaries), block_table, seq_lens,
                 const_cast<int32_t*>(selected), const_cast<int32_t*>(num_selected), nullptr, out,
                 lse, 0, compensate ? 1 : 0};
  return hip_status(ckv::launch_step(s, ckv::kModeAttendOnly, io, carve(s, workspace),
                                     static_cast<hipStream_t>(stream)),
                    "attention launch");
}

ckv_status ckv_decode_step(const ckv_dims* dims, const void* q, const void* k_cache,
                           const void* v_cache, const ckv_summaries* summaries,
                           const int32_t* block_table, const int32_t* seq_lens,
                           int32_t budget_tokens, int32_t score_mode, int32_t* selected,
                           int32_t* num_selected, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  ckv::Shape s;
  CKV_TRY(check_step_args(dims, q, k_cache, v_cache, summaries, block_table, seq_lens, budget_tokens,
                          score_mode, selected, num_selected, out, &s));
  CKV_TRY(check_workspace(s, workspace, workspace_bytes));
  return decode_step_launches(s, q, k_cache, v_cache, summaries, block_table, seq_lens, score_mode, selected,
                              num_selected, out, lse, workspace, static_cast<hipStream_t>(stream));
}

ckv_status ckv_decode_step_append(const ckv_dims* dims, const void* q, const void* k_new,
                                  const void* v_new, void* k_cache, void* v_cache,
                                  const ckv_summaries* summaries, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t budget_tokens, int32_t score_mode,
                                  int32_t* selected, int32_t* num_selected, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (budget_tokens < 0) return fail(CKV_ERR_INVALID_ARG, "budget_tokens must be >= 0");
  ckv::Shape s;
  CKV_TRY(make_shape(dims, budget_tokens, &s));
  if (!q || !k_cache || !v_cache) return fail(CKV_ERR_INVALID_ARG, "q, k_cache or v_cache is NULL");
  if (!k_new || !v_new) return fail(CKV_ERR_INVALID_ARG, "k_new or v_new is NULL");
  if (!block_table || !seq_lens) return fail(CKV_ERR_INVALID_ARG, "block_table or seq_lens is NULL");
  if (!num_selected || (!selected && s.kmax > 0))
    return fail(CKV_ERR_INVALID_ARG, "selected or num_selected is NULL");
  if (!out) return fail(CKV_ERR_INVALID_ARG, "out is NULL");
  if (score_mode != CKV_SCORE_COMPKV && score_mode != CKV_SCORE_MASS)
    return fail(CKV_ERR_INVALID_ARG, "unknown score_mode %d", score_mode);
  CKV_TRY(check_summaries(summaries));
  CKV_TRY(check_workspace(s, workspace, workspace_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  ckv::Shape sa = s;
  if (plan_fused_append(&sa, st, true)) {
    ckv::StepIO io{q, k_cache, v_cache, to_summ(summaries), block_table, seq_lens, selected,
                   num_selected, nullptr, out, lse, score_mode, 1, k_new, v_new};
    return hip_status(ckv::launch_fused(sa, io, carve(s, workspace), st), "decode step launch");
  }
  const hipError_t e = ckv::launch_append_tokens(s, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                                 to_summ(summaries), st);
  if (e != hipSuccess) return hip_status(e, "append launch");
  return ckv_decode_step(dims, q, k_cache, v_cache, summaries, block_table, seq_lens, budget_tokens,
                         score_mode, selected, num_selected, out, lse, workspace, workspace_bytes, stream);
}

ckv_status ckv_workspace_status(void* workspace, size_t workspace_bytes, uint32_t* error_word,
                                void* stream) {
  if (error_word) *error_word = 0u;
  if (!workspace && workspace_bytes == 0) {
    // the built-in workspace of ckv_decode_step_noalloc on the current device
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchState* z = nullptr;
    CKV_TRY(scratch_state(&z));
    const ckv_status st = ckv_workspace_status(z->ptr, CKV_NOALLOC_WORKSPACE_BYTES, error_word, stream);
    if (st == CKV_ERR_INCOMPLETE) z->laid_out = false;  // the next call starts from a cleared workspace
    return st;
  }
  if (!workspace) return fail(CKV_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < 3 * sizeof(uint32_t))
    return fail(CKV_ERR_INVALID_ARG, "workspace has %zu bytes, the error word needs 12", workspace_bytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  CKV_TRY(hip_status(hipStreamIsCapturing(st, &cs), "hipStreamIsCapturing"));
  if (cs != hipStreamCaptureStatusNone)
    return fail(CKV_ERR_INVALID_ARG, "ckv_workspace_status synchronizes; the stream is capturing a graph");
  uint32_t* word = static_cast<uint32_t*>(workspace) + 2;
  uint32_t v = 0u;
  CKV_TRY(hip_status(hipMemcpyAsync(&v, word, sizeof v, hipMemcpyDeviceToHost, st), "error word copy"));
  CKV_TRY(hip_status(hipStreamSynchronize(st), "hipStreamSynchronize"));
  if (v == 0u) return ok();
  if (error_word) *error_word = v;
  CKV_TRY(hip_status(hipMemsetAsync(word, 0, sizeof v, st), "error word clear"));
  return fail(CKV_ERR_INCOMPLETE, "error word %u: %s", v,
              v == 1u ? "a bounded wait between workgroups ran out"
                      : "a workgroup ran on an XCD it was not placed on");
}

ckv_status ckv_decode_step_noalloc(const ckv_dims* dims, const void* q, const void* k_cache,
                                   const void* v_cache, const ckv_summaries* summaries,
                                   const int32_t* block_table, const int32_t* seq_lens, int32_t budget_tokens,
                                   int32_t score_mode, int32_t* selected, int32_t* num_selected, float* out,
                                   float* lse, void* stream) {
  ckv::Shape s;
  CKV_TRY(check_step_args(dims, q, k_cache, v_cache, summaries, block_table, seq_lens, budget_tokens,
                          score_mode, selected, num_selected, out, &s));
  const size_t need = layout(s).total;
  if (need > CKV_NOALLOC_WORKSPACE_BYTES)
    return fail(CKV_ERR_WORKSPACE, "the step needs %zu bytes of workspace; the built-in one holds %zu", need,
                (size_t)CKV_NOALLOC_WORKSPACE_BYTES);
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchState* z = nullptr;
  CKV_TRY(scratch_state(&z));
  if (!z->laid_out || z->budget != budget_tokens || !same_dims(z->dims, *dims)) {
    // a new layout: its control and hand-off words start at zero, as in a
    // freshly cleared workspace
    const size_t n = need / sizeof(uint4);  // need is a multiple of 256
    const unsigned grid = (unsigned)std::min<size_t>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, st, static_cast<uint4*>(z->ptr), n);
    CKV_TRY(hip_status(hipGetLastError(), "workspace clear launch"));
    z->dims = *dims;
    z->budget = budget_tokens;
    z->laid_out = true;
  }
  return decode_step_launches(s, q, k_cache, v_cache, summaries, block_table, seq_lens, score_mode, selected,
                              num_selected, out, lse, z->ptr, st);
}

int32_t ckv_decode_step_append_launches(const ckv_dims* dims, int32_t budget_tokens) {
  ckv::Shape s;
  if (budget_tokens < 0 || make_shape(dims, budget_tokens, &s) != CKV_OK) return 0;
  if (plan_fused_append(&s, nullptr, true)) return 1;
  return 1 + (plan_fused(&s, nullptr, false) ? 1 : 3);
}

int32_t ckv_decode_step_launches(const ckv_dims* dims, int32_t budget_tokens) {
  ckv::Shape s;
  if (budget_tokens < 0 || make_shape(dims, budget_tokens, &s) != CKV_OK) return 0;
  return plan_fused(&s, nullptr, false) ? 1 : 3;
}

size_t ckv_dense_workspace_bytes(const ckv_dims* dims) {
  ckv::Shape s;
  if (make_shape(dims, 0, &s) != CKV_OK) return 0;
  set_dense(s);
  return dense_bytes(s);
}

ckv_status ckv_dense_decode_attention(const ckv_dims* dims, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_table,
                                      const int32_t* seq_lens, float* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  ckv::Shape s;
  CKV_TRY(make_shape(dims, 0, &s));
  if (!q || !k_cache || !v_cache) return fail(CKV_ERR_INVALID_ARG, "q, k_cache or v_cache is NULL");
  if (!block_table || !seq_lens) return fail(CKV_ERR_INVALID_ARG, "block_table or seq_lens is NULL");
  if (!out) return fail(CKV_ERR_INVALID_ARG, "out is NULL");
  set_dense(s);
  const size_t need = dense_bytes(s);
  if (!workspace) return fail(CKV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(CKV_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(CKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  char* base = static_cast<char*>(workspace);
  ckv::Work w{reinterpret_cast<uint32_t*>(base), nullptr, nullptr, nullptr,
              reinterpret_cast<float*>(base + ctrl_bytes(s)), nullptr, nullptr, nullptr, nullptr};
  ckv::StepIO io{q, k_cache, v_cache, ckv::Summ{nullptr, nullptr, nullptr, nullptr}, block_table,
                 seq_lens, nullptr, nullptr, nullptr, out, lse, 0, 0};
  return hip_status(ckv::launch_step(s, ckv::kModeDense, io, w, static_cast<hipStream_t>(stream)),
                    "dense launch");
}

}  // extern "C"

// C ABI of libcompkv.so: host-side argument checks, workspace carving and
// launch order.  Every check runs before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/compkv.h"
#include "internal.hpp"

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
  x.n_chunks = (x.max_blocks + ckv::kScanChunk - 1) / ckv::kScanChunk;
  x.n_splits = (x.kmax + ckv::kGatherPages - 1) / ckv::kGatherPages;
  x.dtype = d->kv_dtype;
  x.tau = (float)(1.0 / sqrt((double)d->head_dim));
  x.tau2 = (float)(1.0 / (double)d->head_dim);
  return CKV_OK;
}

struct Layout {
  size_t comp, lam, gath, total;
};

Layout layout(const ckv::Shape& s) {
  Layout L;
  const size_t pst = ckv::kPartStride(s.D);
  L.comp = 0;
  size_t off = align_up((size_t)s.B * s.Hkv * s.n_chunks * s.G * pst * sizeof(float));
  L.lam = off;
  off += align_up((size_t)s.B * s.Hq * s.max_blocks * sizeof(float));
  L.gath = off;
  off += align_up((size_t)s.B * s.Hkv * s.n_splits * s.G * 2 * pst * sizeof(float));
  L.total = off;
  return L;
}

ckv::Work carve(const ckv::Shape& s, void* ws) {
  const Layout L = layout(s);
  char* base = static_cast<char*>(ws);
  return ckv::Work{reinterpret_cast<float*>(base + L.comp), reinterpret_cast<float*>(base + L.lam),
                   reinterpret_cast<float*>(base + L.gath)};
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

}  // namespace

extern "C" {

const char* ckv_status_string(ckv_status st) {
  switch (st) {
    case CKV_OK: return "CKV_OK";
    case CKV_ERR_INVALID_ARG: return "CKV_ERR_INVALID_ARG";
    case CKV_ERR_UNSUPPORTED: return "CKV_ERR_UNSUPPORTED";
    case CKV_ERR_WORKSPACE: return "CKV_ERR_WORKSPACE";
    case CKV_ERR_HIP: return "CKV_ERR_HIP";
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
  const ckv::Work w = carve(s, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = ckv::launch_scan(s, q, to_summ(summaries), block_table, seq_lens, score_mode, w, st);
  if (e != hipSuccess) return hip_status(e, "scan launch");
  return hip_status(ckv::launch_select(s, seq_lens, w, selected, num_selected, group_scores, st),
                    "select launch");
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
  const ckv::Work w = carve(s, workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = ckv::launch_gather(s, q, k_cache, v_cache, to_summ(summaries), block_table,
                                    seq_lens, selected, num_selected, compensate ? 1 : 0, w, st);
  if (e != hipSuccess) return hip_status(e, "gather launch");
  return hip_status(
      ckv::launch_merge(s, seq_lens, num_selected, compensate ? 1 : 0, w, out, lse, st),
      "merge launch");
}

ckv_status ckv_decode_step(const ckv_dims* dims, const void* q, const void* k_cache,
                           const void* v_cache, const ckv_summaries* summaries,
                           const int32_t* block_table, const int32_t* seq_lens,
                           int32_t budget_tokens, int32_t score_mode, int32_t* selected,
                           int32_t* num_selected, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!k_cache || !v_cache) return fail(CKV_ERR_INVALID_ARG, "k_cache or v_cache is NULL");
  if (!out) return fail(CKV_ERR_INVALID_ARG, "out is NULL");
  CKV_TRY(ckv_score_select(dims, q, summaries, block_table, seq_lens, budget_tokens, score_mode,
                           selected, num_selected, nullptr, workspace, workspace_bytes, stream));
  return ckv_compensated_decode_attention(dims, q, k_cache, v_cache, summaries, block_table,
                                          seq_lens, budget_tokens, selected, num_selected, 1, out,
                                          lse, workspace, workspace_bytes, stream);
}

size_t ckv_dense_workspace_bytes(const ckv_dims* dims) {
  ckv::Shape s;
  if (make_shape(dims, 0, &s) != CKV_OK) return 0;
  const int splits = (s.max_blocks + ckv::kDensePages - 1) / ckv::kDensePages;
  return align_up((size_t)s.B * s.Hkv * splits * s.G * ckv::kPartStride(s.D) * sizeof(float));
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
  const size_t need = ckv_dense_workspace_bytes(dims);
  if (!workspace) return fail(CKV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(CKV_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(CKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  s.n_splits = (s.max_blocks + ckv::kDensePages - 1) / ckv::kDensePages;
  return hip_status(ckv::launch_dense(s, q, k_cache, v_cache, block_table, seq_lens,
                                      static_cast<float*>(workspace), out, lse,
                                      static_cast<hipStream_t>(stream)),
                    "dense launch");
}

}  // extern "C"

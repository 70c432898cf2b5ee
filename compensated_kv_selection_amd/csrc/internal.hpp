// Launch interface between the C ABI (argument checks, workspace carving) and
// the kernels.  Host-side only; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ckv {

constexpr int kBlockSize = 16;      // tokens per block = tokens per page
constexpr int kScanChunk = 256;     // blocks scored by one scan workgroup
constexpr int kGatherPages = 4;     // selected blocks attended by one gather workgroup
constexpr int kDensePages = 32;     // blocks attended by one dense workgroup
constexpr int kMaxBlocks = 15872;   // select keeps one 32-bit key per block in LDS
constexpr int kMaxKvHeads = 64;
constexpr int kPartStride(int d) { return d + 4; }  // [m, l, z, pad, acc[d]]

enum ScoreMode { kScoreCompKV = 0, kScoreMass = 1 };

// Problem shape as the kernels see it.
struct Shape {
  int B, Hq, Hkv, G, D, bs, r, P, max_blocks;
  int kmax;      // selected-block capacity per (sequence, KV head)
  int n_chunks;  // scan workgroups per (sequence, KV head)
  int n_splits;  // gather workgroups per (sequence, KV head)
  int dtype;     // 0 = bf16, 1 = f32
  float tau;     // 1 / sqrt(d)
  float tau2;    // 1 / d
};

// Device pointers carved from the caller's workspace.
struct Work {
  float* comp;  // [B][Hkv][n_chunks][G][D+4]   scan partials over all blocks: max s_bar, sum n e^{s_bar},
                //                                sum n e^{s_bar}(1 + var_hat/2), sum n e^{s_bar} mean_v
  float* lam;   // [B][Hq][max_blocks]          log of each block's per-head ranked score
  float* gath;  // [B][Hkv][n_splits][G][2][D+4] gather partials: exact tokens, and the
                //                                selected blocks' own compensation terms
};

struct Summ {
  void* mean_k;
  void* mean_v;
  float* gvar;
  int32_t* count;
};

hipError_t launch_build_summaries(const Shape& s, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  int append_only, const Summ& out, hipStream_t stream);

hipError_t launch_scan(const Shape& s, const void* q, const Summ& summ, const int32_t* block_table,
                       const int32_t* seq_lens, int score_mode, const Work& w, hipStream_t stream);

hipError_t launch_select(const Shape& s, const int32_t* seq_lens, const Work& w, int32_t* selected,
                         int32_t* num_selected, float* group_scores, hipStream_t stream);

hipError_t launch_gather(const Shape& s, const void* q, const void* k_cache, const void* v_cache,
                         const Summ& summ, const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* selected, const int32_t* num_selected, int compensate,
                         const Work& w, hipStream_t stream);

hipError_t launch_merge(const Shape& s, const int32_t* seq_lens, const int32_t* num_selected,
                        int compensate, const Work& w, float* out, float* lse, hipStream_t stream);

// Dense: every block, no compensation.  `part` is [B][Hkv][n_splits][G][D+4].
hipError_t launch_dense(const Shape& s, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const int32_t* seq_lens, float* part,
                        float* out, float* lse, hipStream_t stream);

}  // namespace ckv

// Launch interface between the C ABI (argument checks, workspace carving) and
// the kernels.  Host-side only; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ckv {

constexpr int kBlockSize = 16;      // tokens per block = tokens per page
constexpr int kChunk = 256;         // blocks scored by one scan workgroup
constexpr int kSlice = 1024;        // blocks ranked by one select workgroup
constexpr int kGatherPages = 4;     // selected blocks per gather workgroup (unfused path)
constexpr int kMaxSplits = 64;      // gather workgroups per (sequence, KV head), unfused path
constexpr int kGatherGroups = 256;  // gather workgroups of one attend launch at most, one per CU of
                                    //   MI355X (measured: 256 beat 128, 512 and 1024 on 128 pairs)
constexpr int kDensePages = 128;    // blocks per dense workgroup
constexpr int kMaxBlocks = 15872;   // blocks per sequence (page-table width)
constexpr int kMaxKvHeads = 64;
constexpr int kMergeFactors = 4096; // LDS floats for merge factors: G * (chunks + 2 * parts)
constexpr int kCandLds = 2048;      // second-level candidates kept in LDS (else read from memory)
constexpr int kShareMax = 256;      // selected blocks one fused workgroup attends to
constexpr int kFusedMaxRounds = 2;  // rounds of pairs the single launch takes at most (measured: at
                                    //   three rounds and more the three launches are faster)
constexpr int kMaxChunks = (kMaxBlocks + kChunk - 1) / kChunk;
constexpr int kFusedCand = 4608;    // fused step: candidates of all chunks held in LDS
constexpr int kFusedPageBits = 18;  // fused step: page ids carried in selection keys (P < 2^18)
constexpr int kPartStride(int d) { return d + 4; }  // [m, l, z, c, acc[d]]
constexpr int kCtrlHeader = 64;     // uint32 words before the per-(sequence, KV head) counters
constexpr int kCtrlPerPair = 8;     // control words per (sequence, KV head)

enum ScoreMode { kScoreCompKV = 0, kScoreMass = 1 };

// What one launch of the step kernel does.
enum StepMode {
  kModeFused = 0,       // score, select, gather and merge in one launch
  kModeScanOnly = 1,    // score every block; scores and compensation partials stay in the workspace
  kModeSelectOnly = 2,  // top-k from the scores of a previous scan launch
  kModeAttendOnly = 3,  // gather and merge, using the partials of previous scan/select launches
  kModeDense = 4        // exact attention over every block, no compensation
};

// Problem shape as the kernels see it.
struct Shape {
  int B, Hq, Hkv, G, D, bs, r, P, max_blocks;
  int kmax;           // selected-block capacity per (sequence, KV head)
  int n_chunks;       // scan workgroups per (sequence, KV head)
  int n_slices;       // select workgroups per (sequence, KV head)
  int share;          // selected blocks attended by one chunk workgroup (fused)
  int bg_round;       // (sequence, KV head) pairs processed at once by the fused grid
  int n_xcd;          // fused: > 0 = XCDs of the device, each pair kept on one XCD; 0 = spread
  int n_val;          // fused: value workgroups per pair, 1..n_chunks; value workgroup v sums
                      //   the compensation terms of chunks v, v + n_val, ...
  int n_splits;       // gather workgroups per (sequence, KV head) (attend-only, dense)
  int pages_per_split;
  int dtype;          // 0 = bf16, 1 = f32
  float tau;          // 1 / sqrt(d)
  float tau2;         // 1 / d
  int append;         // fused, host side: 1 = the instance that also appends each sequence's
                      //   new token (StepIO k_new, v_new)
};

// Device pointers carved from the caller's workspace.
struct Work {
  uint32_t* ctrl;  // [kCtrlHeader + kCtrlPerPair * B * Hkv]: error flag at 2; per (b, g):
                   //   (spare), select arrivals, attend arrivals, fused epoch, the fused
                   //   append's tail word (64 bits, tagged; cleared by its reader), (spare x2)
  float* xs;       // [B][Hq][max_blocks]  exp(log score - chunk max of log score)
  float* cpart;    // [B][Hkv][n_chunks][G][D+4]  per chunk and head: max s_bar, sum w,
                   //   sum w (1 + var_hat/2), max log score, sum w mean_v; w = n e^{s_bar - max}
  uint64_t* cand;  // [B][Hkv][n_slices][kmax] first-level top-k candidates
  float* gpart;    // [B][Hkv][n_splits][G][2][D+4] exact-token partials and the selected
                   //   blocks' own compensation terms
  uint64_t* fhdr;  // [2][B][Hkv][n_chunks][G] fused: chunk header (max s_bar, Z_hat part),
                   //   0 = unset; half = parity of the call's tag
  uint64_t* fcand; // [2][B][Hkv][n_chunks][kmax] fused: chunk candidates, 0 = unset
  uint64_t* fw;    // [B][Hkv][n_chunks][G][kChunk + 1] fused: compensation weights and chunk
                   //   max, tagged
  uint64_t* fpart; // [B][Hkv][2 * n_chunks][G][D+2] fused: control and value partials
                   //   (max, sum, acc[D]), tagged
};

struct Summ {
  void* mean_k;   // [B][Hkv][max_blocks][D]
  void* mean_v;   // [B][Hkv][max_blocks][D]
  float* gvar;    // [B][Hkv][max_blocks][r]
  int32_t* count; // [B][max_blocks]
};

struct StepIO {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  Summ summ;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t* selected;
  int32_t* num_selected;
  float* group_scores;
  float* out;
  float* lse;
  int score_mode;
  int compensate;
  // Fused step with append only: the new key and value rows, [B][Hkv][D];
  // k_cache, v_cache and the summaries are then written.
  const void* k_new;
  const void* v_new;
};

hipError_t launch_build_summaries(const Shape& s, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  int append_only, const Summ& out, hipStream_t stream);

// Decode append: writes the new key and value rows (k_new, v_new:
// [B][Hkv][D]) of every sequence's last token into its page and recomputes
// that block's summary.
hipError_t launch_append_tokens(const Shape& s, const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                const Summ& out, hipStream_t stream);

// One launch of the decode-step kernel in the given mode (not kModeFused).
hipError_t launch_step(const Shape& s, int mode, const StepIO& io, const Work& w, hipStream_t stream);

// Workgroups of the fused step kernel that fit on the current device at once
// (0 if the kernel cannot run with this shape).
int fused_resident_workgroups(const Shape& s);

// One launch of the fused step kernel; s.bg_round and s.n_val must be set,
// with W = n_chunks + n_val workgroups per pair:
// s.bg_round * W <= fused_resident_workgroups(s), and with n_xcd > 0
// ceil(bg_round / n_xcd) * W <= fused_resident_workgroups(s) / n_xcd.
hipError_t launch_fused(const Shape& s, const StepIO& io, const Work& w, hipStream_t stream);

// Number of XCDs if the device sends workgroup i of a launch to XCD
// (i + c) % (number of XCDs), c the same for every workgroup of the launch,
// else 0.  Checked once per device with a small kernel
// on `stream` (waits for it); returns 0 without checking while `stream` is
// capturing a graph.
int fused_xcd_count(hipStream_t stream);

}  // namespace ckv

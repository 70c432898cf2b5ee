/*
 * compkv.h - C ABI of libcompkv.so: compensation-aware block-sparse decode
 * attention (CompKV) on AMD Instinct MI355X (gfx950).
 *
 * One decode step of one attention layer, for a batch of sequences whose
 * keys and values live in a paged cache on the GPU:
 *
 *   1. ckv_build_summaries: per block (= page) and KV head, the mean key,
 *      the grouped key variance (r channel groups), the mean value and the
 *      token count.  CompKV review (evolve.pub), "Summary" and the FAQ: the
 *      method keeps mean key, grouped key variances (4 groups by default)
 *      and mean value, 2d + r + 1 scalars per block, updated as tokens enter
 *      the cache.
 *   2. ckv_score_select: score every block from its summary with the
 *      practical residual criterion - a second-order attention-mass estimate
 *      times the estimated within-block logit variance - and keep the top-k
 *      blocks under a token budget.  CompKV abstract (shd-paper.top
 *      listing): the error a block leaves behind under mean compensation
 *      depends on the attention it draws and on how far its logits spread,
 *      and small per-block statistics estimate it; review "Summary", paper
 *      Section 3, Eqs. 4-7.
 *   3. ckv_compensated_decode_attention: exact attention over the selected
 *      blocks' tokens; every omitted block enters the softmax once, with its
 *      block-mean logit, weighted by its token count, carrying its mean
 *      value ("Mean compensation", review "Summary").
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array arguments are DEVICE pointers owned by the caller.  The
 *   library allocates no device memory.  State it keeps between calls: a
 *   thread-local text describing the last argument error (ckv_last_error);
 *   per device, the occupancy of each kernel instance (queried once) and
 *   whether the device sends workgroup i of a launch to XCD i % (number of
 *   XCDs) (checked once, see ckv_decode_step).
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Work is enqueued asynchronously on it.  Nothing synchronizes the host,
 *   except ckv_workspace_status and the first ckv_decode_step /
 *   ckv_decode_step_append (and their *_launches queries) on a device, which
 *   run the one-time XCD check and wait for it.
 * - Arguments are validated on the host before anything is enqueued.  An
 *   invalid or unsupported argument returns an error status and enqueues
 *   nothing.  A failed kernel launch returns CKV_ERR_HIP.  Faults inside a
 *   kernel surface at the caller's next synchronization.
 * - Device-side contents (seq_lens, block_table, selected) cannot be checked
 *   on the host.  Kernels clamp seq_lens[b] to [0, max_blocks_per_seq *
 *   block_size] and skip page ids outside [0, num_pages) and block ids
 *   outside [0, num_blocks), so invalid contents give unspecified results
 *   but never an out-of-bounds access.
 * - A step may read a pair's whole row of block_table and summaries (all
 *   max_blocks_per_seq entries, which the layouts below allocate) before
 *   it knows seq_lens; entries past a sequence's end are never used, so
 *   they may hold anything.
 * - Inputs must be finite; non-finite inputs give unspecified results.
 * - The library is reentrant; calls on different streams with disjoint
 *   outputs and workspaces may overlap, except that the single launch of
 *   ckv_decode_step / ckv_decode_step_append (see there) needs the device to
 *   itself while it runs.
 * - Kernels whose workgroups wait for each other bound every wait.  A wait
 *   that runs out, or a workgroup that finds itself on an XCD it was not
 *   placed on, sets the workspace's error word: the call's outputs are then
 *   unspecified, although it returned CKV_OK.  ckv_workspace_status reports
 *   and clears that word; check it where results matter.
 *
 * Layouts (row-major, innermost last)
 * -----------------------------------
 *   q           [B][Hq][d]                 kv_dtype
 *   k_cache     [P][Hkv][block_size][d]    kv_dtype  (one page = one block)
 *   v_cache     [P][Hkv][block_size][d]    kv_dtype
 *   block_table [B][max_blocks_per_seq]    int32     logical block -> page
 *   seq_lens    [B]                        int32     tokens per sequence
 *   mean_k      [B][Hkv][max_blocks][d]    kv_dtype  (summaries by logical block)
 *   mean_v      [B][Hkv][max_blocks][d]    kv_dtype
 *   gvar        [B][Hkv][max_blocks][r]    float32
 *   count       [B][max_blocks]            int32
 *   selected    [B][Hkv][k_max]            int32, k_max = min(max_blocks_per_seq, budget/block_size)
 *   out         [B][Hq][d]                 float32
 *   lse         [B][Hq]                    float32 (natural log)
 * Query head h reads KV head h / (Hq / Hkv).  Block i of a sequence holds
 * tokens [i*block_size, min((i+1)*block_size, L)).
 */
#ifndef COMPKV_H
#define COMPKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CKV_OK = 0,
  CKV_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent dims */
  CKV_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement */
  CKV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  CKV_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  CKV_ERR_INCOMPLETE = 5   /* ckv_workspace_status: a call on this workspace did not
                              complete its work (see there); its outputs are unspecified */
} ckv_status;

typedef enum { CKV_BF16 = 0, CKV_F32 = 1 } ckv_dtype;

/* Which score ranks the blocks.
 *   CKV_SCORE_COMPKV: practical residual score, S = A * var_hat / 2 with the
 *     second-order mass estimate A = n exp(s_bar) (1 + var_hat / 2)
 *     (review "Summary"; abstract).
 *   CKV_SCORE_MASS: estimated attention mass A alone - the score that
 *     remains when compensation is removed from the objective (review "Key
 *     claims", App. A.5).
 * For GQA the ranked score of a block is the sum over the KV head's query
 * heads of score / Z_hat, Z_hat = sum over the sequence's blocks of A. */
typedef enum { CKV_SCORE_COMPKV = 0, CKV_SCORE_MASS = 1 } ckv_score_mode;

typedef struct {
  int32_t batch;              /* B >= 1 */
  int32_t num_q_heads;        /* Hq >= 1 */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0; G = Hq / Hkv in {1, 2, 4, 8} */
  int32_t head_dim;           /* d in {64, 128} */
  int32_t block_size;         /* tokens per block and per page; 16 */
  int32_t r_groups;           /* r >= 1, d % r == 0: channel groups of the key variance */
  int32_t num_pages;          /* P >= 1: pages of the cache and of the summary store */
  int32_t max_blocks_per_seq; /* columns of block_table, 1 .. 15872 */
  int32_t kv_dtype;           /* ckv_dtype of q, k_cache, v_cache, mean_k, mean_v */
} ckv_dims;

/* The summary store is indexed by (sequence, KV head, logical block), head
 * major, so that scoring one KV head of one sequence streams contiguous
 * memory; the keys and values themselves stay in the paged cache. */
typedef struct {
  void* mean_k;   /* [B][Hkv][max_blocks][d] kv_dtype: mean key of the block's tokens */
  void* mean_v;   /* [B][Hkv][max_blocks][d] kv_dtype: mean value */
  float* gvar;    /* [B][Hkv][max_blocks][r]: per channel group, the mean of the
                     channels' population variances of the keys */
  int32_t* count; /* [B][max_blocks]: tokens in the block */
} ckv_summaries;

/* Build block summaries from the paged cache (review "Summary", FAQ).
 *
 * append_only == 0 (prefill, bulk): every block of every sequence.
 * append_only != 0 (decode): only the block holding each sequence's last
 *   token, i.e. the block a newly appended token entered.  It is recomputed
 *   from its raw tokens, so bulk and append give identical bits.
 * Means are accumulated in float32 and rounded to kv_dtype (nearest, ties to
 * even); variances are two-pass (population, divide by n) in float32.
 * Entries of blocks not touched are left unchanged.
 * Errors: CKV_ERR_INVALID_ARG / CKV_ERR_UNSUPPORTED for bad dims or null
 * pointers (nothing enqueued); CKV_ERR_HIP if the launch fails. */
ckv_status ckv_build_summaries(const ckv_dims* dims, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               int32_t append_only, const ckv_summaries* summaries,
                               void* stream);

/* Decode append in one launch (review FAQ: summaries are updated as tokens
 * enter the cache): the last token of every sequence b, at position
 * seq_lens[b] - 1 (seq_lens already count it), is new.  Its key
 * k_new[b][g][0..d) and value v_new[b][g][0..d) (kv_dtype, [B][Hkv][d],
 * contiguous) are written into slot (seq_lens[b] - 1) % block_size of page
 * block_table[b][(seq_lens[b] - 1) / block_size] of k_cache and v_cache, and
 * that block's summary is recomputed from its tokens.  Gives the same caches
 * and summaries, bit for bit, as writing the token and then calling
 * ckv_build_summaries with append_only != 0.  Sequences with seq_lens[b] == 0
 * or a negative page id are left alone.  k_new and v_new must not overlap the
 * caches; the caller owns every buffer.
 * Errors: CKV_ERR_INVALID_ARG / CKV_ERR_UNSUPPORTED for bad dims or null
 * pointers (nothing enqueued); CKV_ERR_HIP if the launch fails. */
ckv_status ckv_append_tokens(const ckv_dims* dims, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* block_table,
                             const int32_t* seq_lens, const ckv_summaries* summaries, void* stream);

/* Bytes of device workspace that ckv_score_select,
 * ckv_compensated_decode_attention and ckv_decode_step need for these dims
 * and this budget (0 when dims are invalid).  The same workspace must be
 * passed to both calls of one decode step.
 * The workspace must be zero-filled before its first use, and it serves one
 * (dims, budget_tokens) pair: its layout depends on both, so zero it again
 * before using it with other dims or another budget.  Its first
 * 64 + 8 * B * Hkv uint32 words are control words.  Word 2 is an error flag
 * that a call sets, and leaves set, if one of its bounded waits ever ran out
 * (results are then unspecified).  Word 64 + 8 * (b * Hkv + g) + 3 counts
 * the ckv_decode_step calls of sequence b, KV head g; every other control
 * word is zero again after each call, and so is the half of the single-launch
 * step's published words that its next call publishes into.  Calls that
 * share a workspace must not overlap. */
size_t ckv_workspace_bytes(const ckv_dims* dims, int32_t budget_tokens);

/* Score every block and select the top-k per (sequence, KV head) under a
 * token budget (abstract; review "Summary", Section 3 Eqs. 4-7).
 *
 * k = min(num_blocks, budget_tokens / block_size), num_blocks =
 * ceil(seq_lens[b] / block_size); a partial tail block counts as one block.
 * Ties go to the lower block index.  selected[b][g][0..k) receives the
 * chosen logical block ids in ascending order; entries k..k_max-1 are set to
 * -1.  num_selected[b][g] = k.
 * group_scores: optional (may be NULL); if given, [B][Hkv][max_blocks_per_seq]
 * float32 receives the ranked score of each block (entries past num_blocks
 * are not written).  The workspace keeps, for the attention call that
 * follows, the per-block log-scores and the compensation partials of all
 * blocks.
 * Errors: as ckv_build_summaries, plus CKV_ERR_WORKSPACE. */
ckv_status ckv_score_select(const ckv_dims* dims, const void* q, const ckv_summaries* summaries,
                            const int32_t* block_table, const int32_t* seq_lens,
                            int32_t budget_tokens, int32_t score_mode, int32_t* selected,
                            int32_t* num_selected, float* group_scores, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Exact attention over the selected blocks plus Mean compensation of the
 * omitted ones (abstract; review "Summary").
 *
 * For query head h: every token j of a selected block contributes weight
 * exp(tau q.k_j) and value v_j (tau = 1/sqrt(d)); if `compensate` != 0 every
 * omitted block i contributes weight n_i exp(tau q.mean_k_i) and value
 * mean_v_i.  out = weighted mean of the values, lse = log of the total
 * weight.  When every block is selected the result is dense attention; with
 * nothing to attend to, out = 0 and lse = -inf.
 * `selected`/`num_selected` are as written by ckv_score_select (any set of
 * distinct ascending block ids is accepted).  The workspace must hold what
 * ckv_score_select wrote in this step for the same q and summaries.
 * lse may be NULL.  Errors: as ckv_score_select. */
ckv_status ckv_compensated_decode_attention(const ckv_dims* dims, const void* q,
                                            const void* k_cache, const void* v_cache,
                                            const ckv_summaries* summaries,
                                            const int32_t* block_table, const int32_t* seq_lens,
                                            int32_t budget_tokens, const int32_t* selected,
                                            const int32_t* num_selected, int32_t compensate,
                                            float* out, float* lse, void* workspace,
                                            size_t workspace_bytes, void* stream);

/* One whole decode step: ckv_score_select followed by
 * ckv_compensated_decode_attention with compensation on, same arguments and
 * results (group scores are not written).
 *
 * When every chunk of 256 blocks of a (sequence, KV head) pair can be
 * resident at once (see ckv_decode_step_launches), the step is one
 * persistent launch whose workgroups hand data to each other through memory
 * and wait for each other (bounded waits).  The launch is sized to the whole
 * device, so it must not share the device with other work while it runs:
 * a kernel running beside it on another stream can keep some of its
 * workgroups from becoming resident; the waits of the others then run out,
 * the outputs are unspecified and the workspace's error word is set
 * (ckv_workspace_status).  Work on the same stream, before or after, is
 * fine.
 * The first call on a device (or the first *_launches query) checks, once,
 * whether the device sends the workgroups of a launch to its XCDs in turn
 * (workgroup i to XCD (i + c) % (number of XCDs), c fixed within a launch):
 * a small kernel on `stream`, waited for with hipStreamSynchronize (skipped,
 * and the pairs spread over XCDs, if `stream` is capturing a graph).  If so,
 * every workgroup reads the XCD it runs on and takes a role of a pair placed
 * on that XCD, so that a pair's workgroups hand data over in one L2. */
ckv_status ckv_decode_step(const ckv_dims* dims, const void* q, const void* k_cache,
                           const void* v_cache, const ckv_summaries* summaries,
                           const int32_t* block_table, const int32_t* seq_lens,
                           int32_t budget_tokens, int32_t score_mode, int32_t* selected,
                           int32_t* num_selected, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Reads and clears the error word of a workspace used by ckv_score_select,
 * ckv_compensated_decode_attention, ckv_decode_step, ckv_decode_step_append
 * or ckv_dense_decode_attention (uint32 word 2 of the workspace).  Waits for
 * the work enqueued on `stream` so far, then reads the word.
 *   CKV_OK: no call on this workspace since the last check (or since it was
 *     zero-filled) left the word set.
 *   CKV_ERR_INCOMPLETE: at least one did; the word is cleared (on `stream`)
 *     and its value stored in *error_word when error_word is not NULL:
 *     1 = a bounded wait between workgroups ran out (another kernel running
 *     beside the single launch kept some of its workgroups from becoming
 *     resident, or the device stopped sending workgroups to its XCDs in
 *     turn), 2 = a workgroup of the single launch ran on an XCD that the
 *     one-time check did not see.  Outputs of the calls since the last
 *     check are unspecified.
 *   CKV_ERR_INVALID_ARG: workspace NULL (with workspace_bytes > 0) or
 *     smaller than 12 bytes, or `stream` is capturing a graph (the call
 *     synchronizes).
 *   CKV_ERR_HIP: the copy or the synchronization failed.
 * workspace NULL with workspace_bytes 0 names the built-in workspace of
 * ckv_decode_step_noalloc on the current device (CKV_OK if no call has used
 * it); after it reports CKV_ERR_INCOMPLETE, the next ckv_decode_step_noalloc
 * call on the device clears that workspace before it starts.
 * On CKV_OK *error_word (if given) is set to 0. */
ckv_status ckv_workspace_status(void* workspace, size_t workspace_bytes, uint32_t* error_word,
                                void* stream);

/* Size of the workspace built into the library for ckv_decode_step_noalloc:
 * one per device the library runs on, held until the process ends. */
#define CKV_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/* ckv_decode_step for callers that cannot allocate device memory: code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as ckv_decode_step, except that there
 * is no workspace argument: the step runs in a workspace built into the
 * library, CKV_NOALLOC_WORKSPACE_BYTES on each device, which covers, for
 * example, 16 sequences of 64K tokens with 8 KV heads, d = 128 and a budget
 * of 1024 tokens (49 MiB).  The call allocates nothing.
 *   CKV_ERR_WORKSPACE: ckv_workspace_bytes(dims, budget_tokens) is larger
 *     than CKV_NOALLOC_WORKSPACE_BYTES (checked before anything is enqueued).
 *   CKV_ERR_UNSUPPORTED: the current device's ordinal is 64 or more.
 * Every call on a device shares that device's built-in workspace, which
 * keeps the state the last call left: calls on one stream are ordered, but
 * calls that overlap on one device (other streams, other threads) race, and
 * their outputs are unspecified.  The first call on a device, and every call
 * whose dims or budget differ from the previous call's there, first clears
 * the bytes the step uses with a fill kernel on `stream` (inside a captured
 * graph that clear is captured too; an eager call with the same dims and
 * budget before the capture keeps it out).  The first call on a device looks
 * up the built-in workspace's address on it.  ckv_workspace_status(NULL, 0,
 * ...) reads its error word. */
ckv_status ckv_decode_step_noalloc(const ckv_dims* dims, const void* q, const void* k_cache,
                                   const void* v_cache, const ckv_summaries* summaries,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int32_t budget_tokens, int32_t score_mode, int32_t* selected,
                                   int32_t* num_selected, float* out, float* lse, void* stream);

/* Number of kernel launches ckv_decode_step makes for these dims and budget:
 * 1 when the whole step runs as one persistent launch (every chunk of a
 * (sequence, KV head) pair resident at once and the pair's candidates fit in
 * shared memory), 3 otherwise (score, select, attend), 0 if the arguments are
 * invalid.  Reads the current device's compute-unit count and the kernel's
 * occupancy on it (3 when no device is present); launches nothing. */
int32_t ckv_decode_step_launches(const ckv_dims* dims, int32_t budget_tokens);

/* One decode step that first appends the new token of every sequence
 * (review FAQ: summaries are kept current as tokens enter the cache), then
 * scores, selects and attends as ckv_decode_step.  Same results, bit for
 * bit, as ckv_append_tokens(dims, k_new, v_new, k_cache, v_cache,
 * block_table, seq_lens, summaries) followed by ckv_decode_step with the
 * remaining arguments: seq_lens already count the new token, k_new and
 * v_new are [B][Hkv][d] in kv_dtype, and k_cache, v_cache and the summaries
 * are written.  With bf16, d = 128, r_groups = 4, and when the single-launch
 * step applies and the device keeps each (sequence, KV head) pair's
 * workgroups on one XCD, it is one launch: the workgroup that scores the
 * tail block also writes the new token into its page and recomputes that
 * block's summary.  Otherwise it makes exactly those calls.
 * k_new and v_new must not overlap the caches or the summaries; the caller
 * owns every buffer.  Errors: as ckv_decode_step, plus CKV_ERR_INVALID_ARG
 * for a NULL k_new or v_new. */
ckv_status ckv_decode_step_append(const ckv_dims* dims, const void* q, const void* k_new,
                                  const void* v_new, void* k_cache, void* v_cache,
                                  const ckv_summaries* summaries, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t budget_tokens,
                                  int32_t score_mode, int32_t* selected, int32_t* num_selected,
                                  float* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Number of kernel launches ckv_decode_step_append makes for these dims and
 * budget on the current device (0 if the arguments are invalid).  The first
 * call on a device may run the one-time XCD placement check (a small kernel
 * on the null stream, waited for). */
int32_t ckv_decode_step_append_launches(const ckv_dims* dims, int32_t budget_tokens);

/* Dense decode attention over every token (the baseline the method is
 * measured against: review "Summary", speed-up over full attention).
 * Workspace from ckv_dense_workspace_bytes, zero-filled before first use
 * (same control words as above).  lse may be NULL. */
size_t ckv_dense_workspace_bytes(const ckv_dims* dims);
ckv_status ckv_dense_decode_attention(const ckv_dims* dims, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_table,
                                      const int32_t* seq_lens, float* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* ckv_status_string(ckv_status status);

/* Text describing the last argument error returned on this thread ("" if none). */
const char* ckv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* COMPKV_H */

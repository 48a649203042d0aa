/*
 * ddtree.h -- C ABI of the MI355X (gfx950) tree-verify MLA-absorb attention library.
 *
 * Two operations of a DDTree speculative-decoding step, both described on
 * "Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine":
 *
 *   ddtree_verify_attn   the tree-verify attention in MLA-absorb form with visibility masking
 *                        (section "The Mission: A Native DDTree Engine");
 *   ddtree_compact_kv    the post-accept gather of the kept tree rows into the prefix, free of
 *                        the in-place aliasing race (section "The Cache Compaction Problem");
 *
 * and the step between them, described on "The Microsecond Verdict: Validating a DDTree
 * Kernel Fix Under Time Pressure":
 *
 *   ddtree_tree_accept   greedy acceptance of the verified tree (sections "The Crash That
 *                        Demanded a Fix" and "What Was Learned");
 *   ddtree_accept_compact  acceptance and compaction in one launch;
 *   ddtree_compact_kv_layers, ddtree_accept_compact_layers
 *                        the same for every layer's cache of a model, in one launch;
 *   ddtree_append_tree_kv  the tree's rows written into the cache at the tree's offset;
 *
 * and the step before them, described on "Building the Foundation: Architecting a Native CUDA
 * DDTree Inference Engine":
 *
 *   ddtree_tree_build    best-first construction of the draft tree from the drafter's
 *                        per-position top-k (sections "Tie-Breaking and Numerical Precision"
 *                        and "The Single-Threaded Heap Design").
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor arguments are DEVICE pointers owned by the caller.  The library allocates
 *   nothing and keeps no pointer after the call returns; buffers must stay alive until the
 *   given HIP stream has executed the work.
 * - bf16 tensors are passed as raw 16-bit storage (`const void*`), row-major, densely packed.
 * - Calls are asynchronous on `stream` (NULL = the default stream) and never synchronise.
 *   Host-side validation reads no device memory.  There is no global mutable state: calls are
 *   re-entrant across host threads and streams.
 * - Every call returns DDTREE_OK (0) or a negative DDTREE_ERR_* code.  Nothing throws, aborts
 *   or exits across the ABI.  On error nothing is launched.
 * - Data errors that only the device can see (a malformed `parents` or `keep`) never cause an
 *   out-of-bounds access; they set a bit in the optional `dev_status` word (device int32,
 *   bits OR-ed in; the caller clears it).
 */
#ifndef DDTREE_H
#define DDTREE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDTREE_VERSION 1

/* Model geometry of the absorbed MLA attention (DeepSeek-V3 / Kimi style). */
#define DDTREE_HEADS 64      /* query heads sharing one latent cache                    */
#define DDTREE_D_LATENT 512  /* c_kv / q_lat width; also the value and output width     */
#define DDTREE_D_ROPE 64     /* k_pe / q_pe width                                        */
#define DDTREE_MAX_Q_LEN 64  /* tree nodes per stream (one 64-bit ancestor mask)         */

/* Return codes. */
#define DDTREE_OK 0
#define DDTREE_ERR_NULL (-1)      /* a required pointer is NULL                               */
#define DDTREE_ERR_SHAPE (-2)     /* a size is out of range                                   */
#define DDTREE_ERR_ALIGN (-3)     /* a tensor pointer is not 16-byte aligned                  */
#define DDTREE_ERR_ALIAS (-4)     /* an output range overlaps an input range                  */
#define DDTREE_ERR_WORKSPACE (-5) /* workspace missing or smaller than the size query says     */
#define DDTREE_ERR_HIP (-6)       /* the HIP runtime reported an error at launch              */

/* Bits of the optional device status word. */
#define DDTREE_STATUS_BAD_PARENTS 1 /* a parents[] entry is not an earlier node; that node's
                                       ancestor chain stops there (attention), the stream is
                                       skipped (acceptance, tree rows)                         */
#define DDTREE_STATUS_BAD_KEEP 2    /* keep[]/n_keep of a stream invalid; that stream untouched */
#define DDTREE_STATUS_BAD_PREFIX 4  /* a per-stream prefix length out of range; see the ragged calls */
#define DDTREE_STATUS_BAD_POSITION 8 /* a tree position past the rotary tables; see ddtree_append_tree_kv */

/*
 * ddtree_verify_attn -- tree-verify attention, absorbed MLA form, one launch for all streams.
 *
 * For every stream s, tree node i < q_len and head h < 64, with P = prefix_len, L = P + q_len:
 *
 *   visible(i)   = cache rows [0, P)  U  { P + j : j is i or an ancestor of i in parents[s] }
 *   score(t)     = scale * ( q_lat[s,i,h,:] . ckv[s,t,:] + q_pe[s,i,h,:] . kpe[s,t,:] )
 *   lse[s,i,h]   = ln( sum_{t in visible(i)} exp(score(t)) )
 *   out_lat[s,i,h,:] = sum_{t in visible(i)} exp(score(t) - lse[s,i,h]) * ckv[s,t,:]
 *
 * with scale = 1/sqrt(192).  Row P + i of the cache holds tree node i, and every parent index
 * is smaller than its child's (page above, section "The Cache Compaction Problem").
 *
 * Arguments (all device pointers, densely packed, 16-byte aligned):
 *   q_lat    bf16  [n_streams][q_len][64][512]   per-head queries mapped into the latent space
 *   q_pe     bf16  [n_streams][q_len][64][64]    rotary query part (already rotated)
 *   ckv      bf16  [n_streams][prefix_len+q_len][512]  shared latent rows (keys and values)
 *   kpe      bf16  [n_streams][prefix_len+q_len][64]   shared rotary key rows
 *   parents  int32 [n_streams][q_len]            parents[s][0] = -1, else 0 <= p < node
 *   out_lat  fp32  [n_streams][q_len][64][512]   written
 *   lse      fp32  [n_streams][q_len][64]        written (natural log)
 * Sizes: 0 <= prefix_len, 1 <= q_len <= 64, 1 <= n_streams.
 * Errors: DDTREE_ERR_NULL / _SHAPE / _ALIGN / _ALIAS / _HIP.  No workspace: the whole key
 * range of a (stream, query pair) is processed by one workgroup.
 */
int ddtree_verify_attn(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                       int prefix_len, const int32_t* parents, int q_len, int n_streams,
                       float* out_lat, float* lse, hipStream_t stream);

/*
 * ddtree_verify_attn_ex -- as ddtree_verify_attn, plus:
 *   kv_rows          per-stream row stride of ckv/kpe, >= prefix_len + q_len (rows past
 *                    prefix_len + q_len are never read)
 *   scale            softmax scale; <= 0 selects 1/sqrt(192)
 *   num_splits       key-range splits per (stream, query pair): 0 = automatic (enough
 *                    workgroups to fill the GPU), 1 = none, n > 1 = at most n.  Splits are
 *                    merged by their log-sum-exp in a second kernel.
 *   workspace        device scratch for split partials (may be NULL when the size query
 *   workspace_bytes  returns 0 for these arguments)
 *   dev_status       optional device int32 status word (may be NULL)
 */
int ddtree_verify_attn_ex(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                          int prefix_len, const int32_t* parents, int q_len, int n_streams,
                          float* out_lat, float* lse, int kv_rows, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, int32_t* dev_status,
                          hipStream_t stream);

/*
 * ddtree_verify_attn_noalloc -- ddtree_verify_attn_ex without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The call itself allocates nothing: the split partials go
 * to a scratch array inside the library, DDTREE_NOALLOC_SCRATCH_BYTES on every GPU the library
 * runs on, held until the process ends; the first call for a GPU (the GPU of `stream`) looks
 * up that GPU's address of the array, with that GPU made current for the lookup only.
 *   num_splits  0 = the best automatic plan whose partials fit in the scratch array (the
 *               unsplit plan needs none); a forced count (n >= 1) whose partials do not fit
 *               returns DDTREE_ERR_WORKSPACE (ddtree_verify_attn_workspace_size gives the bytes).
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents: calls
 * that can overlap on one GPU (issued to different streams without ordering) race and must not
 * be made.  All other arguments, results and errors are those of ddtree_verify_attn_ex, plus
 * DDTREE_ERR_HIP when the array's device address cannot be obtained.
 */
#define DDTREE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ddtree_verify_attn_noalloc(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                               int prefix_len, const int32_t* parents, int q_len, int n_streams,
                               float* out_lat, float* lse, int kv_rows, float scale, int num_splits,
                               int32_t* dev_status, hipStream_t stream);

/* Bytes of workspace ddtree_verify_attn_ex needs for these arguments (0 when no split is
 * used).  Returns 0 for invalid sizes as well; the launch call then reports the error. */
size_t ddtree_verify_attn_workspace_size(int prefix_len, int q_len, int n_streams,
                                         int num_splits);

/* The number of splits ddtree_verify_attn_ex will use for these arguments (>= 1), or a
 * negative DDTREE_ERR_SHAPE for invalid sizes. */
int ddtree_verify_attn_num_splits(int prefix_len, int q_len, int n_streams, int num_splits);

/* The latent KV cache of n_streams streams: ckv bf16 [n_streams][kv_rows][512] and
 * kpe bf16 [n_streams][kv_rows][64], one logical row = 576 bf16 values. */
typedef struct ddtree_kv_cache {
  void* ckv;
  void* kpe;
  int kv_rows;
  int n_streams;
} ddtree_kv_cache;

/*
 * ddtree_compact_kv -- post-accept KV compaction, in place and race-free.
 *
 * For every stream s with n = n_keep[s] and every i < n:
 *   row prefix_len + i of ckv and kpe  <-  the ORIGINAL row prefix_len + keep[s][i]
 * All other rows are left bit-identical.  keep[s] must be strictly increasing with
 * keep[s][0] >= 0 and prefix_len + keep[s][n-1] < kv_rows (so keep[i] >= i: an accepted
 * root-to-node path, page above, section "The Cache Compaction Problem").
 * One workgroup per stream reads every kept row before any row is written, so the reader/
 * writer race that section analyses cannot occur.  The copy is bitwise.
 *
 * Arguments:
 *   cache        host pointer to the cache descriptor (device data pointers inside)
 *   prefix_len   committed rows before the tree block, >= 0
 *   keep         device int32 [n_streams][keep_stride], positions within the tree block
 *   n_keep       device int32 [n_streams], each 0 <= n_keep[s] <= min(keep_stride, 64)
 *   keep_stride  >= 1
 *   dev_status   optional device int32 status word (DDTREE_STATUS_BAD_KEEP), may be NULL
 * Errors: DDTREE_ERR_NULL / _SHAPE / _ALIGN / _HIP.  A stream whose keep/n_keep is invalid is
 * skipped and flagged in dev_status.
 */
int ddtree_compact_kv(const ddtree_kv_cache* cache, int prefix_len, const int32_t* keep,
                      const int32_t* n_keep, int keep_stride, int32_t* dev_status,
                      hipStream_t stream);

/*
 * ddtree_tree_accept -- greedy acceptance of the verified draft trees, one launch for all
 * streams.
 *
 * For every stream s the walk starts at the root (node 0, always accepted).  From the current
 * node c it moves to the lowest-index child j (parents[s][j] == c) with
 * draft_tokens[s][j] == target_tokens[s][c], and stops when no child matches.  The walk visits
 * strictly increasing nodes, so it ends within q_len nodes for any input (the bound that page
 * adds against cyclic links).
 *
 * Arguments (device pointers, 4-byte aligned, densely packed):
 *   parents        int32 [n_streams][q_len]   the tree, as for ddtree_verify_attn
 *   draft_tokens   int32 [n_streams][q_len]   the drafter's token of each node (the root's
 *                                             entry is not read)
 *   target_tokens  int32 [n_streams][q_len]   the target model's greedy token after each node
 *   keep           int32 [n_streams][keep_stride], keep_stride >= q_len: entries [0, n_keep[s])
 *                  receive the accepted nodes (keep[s][0] = 0, strictly increasing); later
 *                  entries are left unchanged.  This is the keep array of ddtree_compact_kv.
 *   n_keep         int32 [n_streams]          the number of accepted nodes, 1..q_len
 *   next_token     int32 [n_streams] or NULL  target_tokens[s][last accepted node]: the target's
 *                                             token for the position after the accepted run
 *   dev_status     optional device int32 status word, may be NULL
 * A stream whose parents[] is not a valid tree (parents[0] == -1 and 0 <= parents[i] < i) gets
 * n_keep = 0 and next_token = -1 and sets DDTREE_STATUS_BAD_PARENTS.
 * Sizes: 1 <= q_len <= 64, 1 <= n_streams, keep_stride >= q_len.
 * Errors: DDTREE_ERR_NULL / _SHAPE / _ALIGN / _ALIAS (an output overlapping an input or another
 * output) / _HIP.
 */
int ddtree_tree_accept(const int32_t* parents, const int32_t* draft_tokens, const int32_t* target_tokens,
                       int q_len, int n_streams, int32_t* keep, int keep_stride, int32_t* n_keep,
                       int32_t* next_token, int32_t* dev_status, hipStream_t stream);

/*
 * ddtree_accept_compact -- ddtree_tree_accept and then ddtree_compact_kv on its keep / n_keep,
 * in one launch (no host round trip, no second kernel).  Same arguments and results as the two
 * calls in sequence, with the tree block of every stream at rows [prefix_len, prefix_len + q_len)
 * of the cache: prefix_len + q_len <= cache->kv_rows and cache->n_streams == n_streams.
 * A stream with a malformed tree keeps its cache rows bit-identical.
 * Errors: as ddtree_tree_accept, plus the cache checks of ddtree_compact_kv (keep / n_keep /
 * next_token must not overlap the cache either).
 */
int ddtree_accept_compact(const ddtree_kv_cache* cache, int prefix_len, const int32_t* parents,
                          const int32_t* draft_tokens, const int32_t* target_tokens, int q_len,
                          int32_t* keep, int keep_stride, int32_t* n_keep, int32_t* next_token,
                          int32_t* dev_status, hipStream_t stream);

/*
 * Per-stream (ragged) prefix lengths.  After compaction every stream's committed prefix grows by
 * its own accepted count, so the streams of a batch soon hold different prefix lengths.  These
 * calls take them as a device array prefix_lens [n_streams] (int32, 4-byte aligned); stream s's
 * tree block is at rows [prefix_lens[s], prefix_lens[s] + q_len) of its cache rows.  A value the
 * device finds out of range sets DDTREE_STATUS_BAD_PREFIX in dev_status (when given).
 */

/*
 * ddtree_verify_attn_ragged -- ddtree_verify_attn_ex with prefix_lens instead of one prefix_len.
 *   max_prefix_len  host bound: 0 <= prefix_lens[s] <= max_prefix_len for every stream; the launch,
 *                   the split plan and the workspace (ddtree_verify_attn_workspace_size with
 *                   max_prefix_len) are sized for it, and kv_rows >= max_prefix_len + q_len.
 * A stream whose prefix_lens entry is outside [0, max_prefix_len] gets NaN in out_lat and lse and
 * sets DDTREE_STATUS_BAD_PREFIX; the other streams are unaffected.  Shorter streams leave part
 * of the launch idle; all results are those of ddtree_verify_attn_ex with that stream's prefix.
 */
int ddtree_verify_attn_ragged(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                              const int32_t* prefix_lens, int max_prefix_len, const int32_t* parents,
                              int q_len, int n_streams, float* out_lat, float* lse, int kv_rows,
                              float scale, int num_splits, void* workspace, size_t workspace_bytes,
                              int32_t* dev_status, hipStream_t stream);

/*
 * ddtree_compact_kv_ragged -- ddtree_compact_kv with prefix_lens (read only) instead of one
 * prefix_len.  A stream whose prefix_lens entry is negative or above kv_rows is skipped and flagged
 * (DDTREE_STATUS_BAD_PREFIX); keep entries are checked against that stream's own prefix.
 */
int ddtree_compact_kv_ragged(const ddtree_kv_cache* cache, const int32_t* prefix_lens, const int32_t* keep,
                             const int32_t* n_keep, int keep_stride, int32_t* dev_status,
                             hipStream_t stream);

/*
 * ddtree_accept_compact_ragged -- ddtree_accept_compact with prefix_lens, which it also ADVANCES:
 * for every stream whose compaction ran, prefix_lens[s] += n_keep[s] (the accepted rows are now
 * committed and the next tree goes right after them).  So verify -> accept -> compact -> the next
 * verify run on the device without a host round trip.  A stream with
 * prefix_lens[s] + q_len > kv_rows (or a negative entry) keeps its cache and prefix unchanged and
 * sets DDTREE_STATUS_BAD_PREFIX; its keep / n_keep / next_token are still written.
 * Requires q_len <= cache->kv_rows.
 */
int ddtree_accept_compact_ragged(const ddtree_kv_cache* cache, int32_t* prefix_lens, const int32_t* parents,
                                 const int32_t* draft_tokens, const int32_t* target_tokens, int q_len,
                                 int32_t* keep, int keep_stride, int32_t* n_keep, int32_t* next_token,
                                 int32_t* dev_status, hipStream_t stream);

/*
 * Multi-layer compaction.  A model keeps one latent cache per layer, and the accepted path moves
 * the same rows in every one of them ("Race Conditions, Buffer Aliasing, and the Architecture of
 * a Native DDTree Inference Engine": section "The Cache Compaction Problem" for the gather, and
 * the closing section, which defers fusing it).  These calls compact all layers in one launch.
 *
 *   caches      HOST array [n_layers] of cache descriptors; every entry has the same kv_rows
 *               and n_streams, and no two caches overlap.  Read during the call only.
 *   n_layers    1 .. DDTREE_MAX_LAYERS
 *   prefix_len  the prefix of every stream when prefix_lens is NULL (ignored otherwise)
 *   prefix_lens NULL, or device int32 [n_streams]: per-stream prefixes
 * For each layer the result is bit-identical to the single-cache call on that layer with the
 * same arguments.  Each layer's gather is race-free on its own (all reads of a stream's kept
 * rows precede its writes); layers never share memory.
 */
#define DDTREE_MAX_LAYERS 128

/*
 * ddtree_compact_kv_layers -- ddtree_compact_kv (prefix_lens NULL) or ddtree_compact_kv_ragged
 * (prefix_lens given, read only) applied to every layer.  A stream whose keep / n_keep or prefix
 * is invalid is skipped in every layer and flagged once (DDTREE_STATUS_BAD_KEEP / _BAD_PREFIX).
 */
int ddtree_compact_kv_layers(const ddtree_kv_cache* caches, int n_layers, int prefix_len, const int32_t* prefix_lens,
                             const int32_t* keep, const int32_t* n_keep, int keep_stride, int32_t* dev_status,
                             hipStream_t stream);

/*
 * ddtree_accept_compact_layers -- acceptance (as ddtree_tree_accept: keep, n_keep, next_token
 * written once) and the compaction of every layer, one step.  With prefix_lens NULL it matches
 * ddtree_accept_compact on each layer; with prefix_lens it matches ddtree_accept_compact_ragged,
 * including the advance prefix_lens[s] += n_keep[s] for every stream whose rows moved (done by a
 * second, small launch on the same stream, after every layer has read the old value).
 * Requires prefix_len + q_len <= kv_rows (prefix_lens NULL) or q_len <= kv_rows.
 */
int ddtree_accept_compact_layers(const ddtree_kv_cache* caches, int n_layers, int prefix_len, int32_t* prefix_lens,
                                 const int32_t* parents, const int32_t* draft_tokens, const int32_t* target_tokens,
                                 int q_len, int32_t* keep, int keep_stride, int32_t* n_keep, int32_t* next_token,
                                 int32_t* dev_status, hipStream_t stream);

/*
 * ddtree_append_tree_kv -- the draft tree's cache rows, written straight into the cache at the
 * tree's offset ("Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree
 * Inference Engine", section "Scratch Buffer Architecture: Managing Transformer Activations":
 * the key/value projection's output goes through RMSNorm directly into the cache; the model is
 * MLA with RMSNorm and NeoX rotary embeddings per section "Assumptions, Input Knowledge, and
 * Output Knowledge").
 *
 * For every stream s (P = prefix_lens[s], or prefix_len when prefix_lens is NULL) and tree node
 * i < q_len, with x = kv[s][i] (576 fp32: 512 latent, then 64 rotary) and pos = P + depth(i):
 *   ckv[s][P + i][k]    = bf16( x[k] / sqrt(mean_k'(x[k']^2) + eps) * norm_weight[k] ), k < 512
 *   kpe[s][P + i][j]    = bf16( x[512 + j] cos[pos][j] - x[544 + j] sin[pos][j] ),    j < 32
 *   kpe[s][P + i][32+j] = bf16( x[544 + j] cos[pos][j] + x[512 + j] sin[pos][j] )
 * rounded to nearest, ties to even; the sums are computed in fp32.  depth(root) = 0, so the root
 * sits at position P, right after the P committed rows; siblings share a position.  No other
 * cache row is touched.
 *
 * Arguments (device pointers):
 *   cache        the latent cache (as for ddtree_compact_kv); written
 *   parents      int32 [n_streams][q_len], parents[s][0] = -1, else an earlier node
 *   kv           fp32 [n_streams][q_len][576], 16-byte aligned
 *   norm_weight  fp32 [512], 16-byte aligned
 *   rope_cos     fp32 [rope_rows][32], rope_sin likewise (4-byte aligned)
 *   eps          >= 0, finite
 * Requires 1 <= q_len <= 64 and, with one prefix_len, prefix_len + q_len <= kv_rows.
 * A stream with a malformed tree (DDTREE_STATUS_BAD_PARENTS), a block outside the cache
 * (DDTREE_STATUS_BAD_PREFIX) or a position >= rope_rows (DDTREE_STATUS_BAD_POSITION) is left
 * untouched and flagged in dev_status.
 */
int ddtree_append_tree_kv(const ddtree_kv_cache* cache, int prefix_len, const int32_t* prefix_lens,
                          const int32_t* parents, int q_len, const float* kv, const float* norm_weight, float eps,
                          const float* rope_cos, const float* rope_sin, int rope_rows, int32_t* dev_status,
                          hipStream_t stream);

/*
 * ddtree_tree_build -- best-first draft trees, one launch for all requests (streams).
 *
 * For every stream s, with lp = logprobs[s] ([depth][topk], each row in decreasing order) and
 * tok = topk_tokens[s] ([depth][topk]): node 0 is the root (depth 0, token root_tokens[s] or -1,
 * log-weight 0).  A heap of candidates starts with the root's first child (depth 1, rank 0,
 * log-weight lp[0][0]).  Each of up to `budget` steps pops the candidate with the highest
 * log-weight (equal weights: the earliest inserted), appends it as the next node (token
 * tok[d-1][r]) and inserts, in this order, its next sibling when r + 1 < topk (log-weight
 * (logw - lp[d-1][r]) + lp[d-1][r+1], float32, in that order) and its first child when d < depth
 * (log-weight logw + lp[d][0]).  The heap runs empty early only when topk == 1 and
 * depth < budget.
 *
 * Arguments (device pointers, 4-byte aligned; anc 8-byte aligned; Q = budget + 1):
 *   logprobs      fp32  [n_streams][depth][topk]
 *   topk_tokens   int32 [n_streams][depth][topk]
 *   root_tokens   int32 [n_streams] or NULL
 *   parents       int32 [n_streams][Q]    written: the tree for ddtree_verify_attn (parents[0] = -1)
 *   node_tokens   int32 [n_streams][Q]    written: the draft tokens for ddtree_tree_accept
 *   n_nodes       int32 [n_streams]       written: nodes built (budget + 1 unless the heap ran
 *                                         empty); entries from n_nodes on are left unchanged
 *   depths        int32 [n_streams][Q]    or NULL
 *   logw          fp32  [n_streams][Q]    or NULL
 *   first_child   int32 [n_streams][Q]    or NULL (-1: none)
 *   next_sibling  int32 [n_streams][Q]    or NULL (-1: none)
 *   anc           uint64 [n_streams][Q]   or NULL: bit j of anc[s][i] set iff node j is i or an
 *                                         ancestor of i (the visibility relation)
 * Sizes: 1 <= depth <= 64, 1 <= topk <= 64, 1 <= budget <= 63 (a tree of at most 64 nodes, the
 * verify attention's limit), 1 <= n_streams.
 * Errors: DDTREE_ERR_NULL / _SHAPE / _ALIGN / _ALIAS (an output overlapping an input or another
 * output) / _HIP.  Non-finite or unsorted log-probabilities give a well-defined expansion of the
 * same rule; no input value causes an out-of-bounds access.
 */
int ddtree_tree_build(const float* logprobs, const int32_t* topk_tokens, const int32_t* root_tokens, int depth,
                      int topk, int budget, int n_streams, int32_t* parents, int32_t* node_tokens,
                      int32_t* n_nodes, int32_t* depths, float* logw, int32_t* first_child,
                      int32_t* next_sibling, uint64_t* anc, hipStream_t stream);

/* Static text for a return code. */
const char* ddtree_status_string(int code);

/* DDTREE_VERSION of the built library. */
int ddtree_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DDTREE_H */

/*
 * fastar.h -- C ABI of libfastar: the attention hot path of FAST-AR
 * ("Fast Autoregressive Video Diffusion and World Models with Temporal Cache
 * Compression and Sparse Attention") as hand-written HIP kernels for AMD
 * MI355X (gfx950).
 *
 * Four operations, after the method's three modules and their shared hashing:
 *   fastar_hash             SimHash bucket ids (+ bucket-contiguous index)
 *   fastar_hash_multi       the ids of several tensors in one launch
 *   fastar_tempcache_merge  TempCache: merge new frames into the compressed cache
 *   fastar_prune_prompt     AnnCA: drop prompt tokens no query shares a bucket with
 *   fastar_bucket_attention AnnSA / AnnCA attention, online softmax on MFMA
 *   fastar_chunk            one chunk of the layer sequence, all of the above
 * and around them: several LSH tables (fastar_bucket_attention_tables,
 * fastar_prune_prompt_tables), TempCache variants (fastar_tempcache_merge_ex),
 * attention recall (fastar_attention_recall[_counts]), the cache's status
 * word (fastar_cache_status) and an allocation-free chunk
 * (fastar_chunk_noalloc).
 *
 * Conventions shared by every call
 * - All tensor and array arguments are DEVICE pointers owned by the caller.
 *   The library allocates nothing and keeps no state between calls.
 * - Every call is enqueued on `stream` and returns without synchronising
 *   (fastar_chunk forks part of its work to a second stream and joins it
 *   back on `stream`).
 *   Counts produced on the device (groups, kept tokens) stay on the device.
 * - Arguments are validated on the host before any launch; a failed check
 *   returns FASTAR_ERR_INVALID or FASTAR_ERR_UNSUPPORTED and launches nothing.
 *   A launch failure returns FASTAR_ERR_HIP.  fastar_last_error() gives a
 *   message for the last failure in the calling thread.
 * - Float inputs must be finite.  bf16 and fp32 are the supported dtypes;
 *   the head dimension must be 64 or 128.
 * - Integer decisions taken from float comparisons (hash signs, the probes'
 *   order, TempCache's arg-max, threshold and conflict tests) follow the exact
 *   real value of the stored inputs: a decision the fast float32 evaluation
 *   cannot certify is re-evaluated in float64 (and for hash signs, exactly).
 *   Counters of these events accumulate in an optional fastar_diag_t.
 */
#ifndef FASTAR_H
#define FASTAR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FASTAR_OK = 0,
  FASTAR_ERR_INVALID = 1,      /* bad pointer, size or combination of arguments */
  FASTAR_ERR_UNSUPPORTED = 2,  /* valid request outside what the kernels cover   */
  FASTAR_ERR_WORKSPACE = 3,    /* ws_bytes below what the *_workspace query says */
  FASTAR_ERR_HIP = 4,          /* a HIP launch failed                            */
  FASTAR_ERR_CAPACITY = 5      /* a merge dropped groups: the cache was full
                                  (reported by fastar_cache_status only)          */
} fastar_status_t;

typedef enum { FASTAR_F32 = 0, FASTAR_BF16 = 1 } fastar_dtype_t;

/* A [heads][tokens][dim] tensor; dim is contiguous, strides are in elements. */
typedef struct {
  const void* data;
  int32_t dtype;          /* fastar_dtype_t */
  int32_t heads;
  int64_t tokens;
  int32_t dim;
  int32_t reserved;
  int64_t stride_head;
  int64_t stride_token;
} fastar_tensor_t;

/* Device-side event counters.  The caller zeroes the struct; calls add. */
typedef struct {
  uint32_t hash_fallback_rows;   /* rows whose hash was re-evaluated in float64    */
  uint32_t hash_exact_signs;     /* signs settled by exact expansion arithmetic     */
  uint32_t merge_fallbacks;      /* TempCache decisions re-evaluated in float64    */
  uint32_t unresolved;           /* decisions float64 could not certify (0 expected) */
  uint32_t capacity_overflow;    /* new groups dropped because the cache was full  */
  uint32_t reserved[3];
} fastar_diag_t;

/* Limits: probes per LSH table and tables of the multi-table calls. */
#define FASTAR_MAX_PROBES 8
#define FASTAR_MAX_TABLES 4

const char* fastar_status_string(int status);
const char* fastar_last_error(void);
int fastar_version(void);

/* ------------------------------------------------------------------------
 * fastar_hash -- SimHash of the rows of x (paperlayer.ai section 5 "ANN
 * Attention" and section 2 "Approximate nearest neighbor search"; one
 * hashing shared by TempCache, AnnCA and AnnSA, paper.rainbus.top "technical
 * novelty").
 *
 *   x        [H][N][d], bf16 or fp32.
 *   planes   [n_bits][d], same dtype as x, contiguous: hyperplane normals r_j.
 *   n_bits   0..15.  Bit j of an id is 1 iff x . r_j > 0 (exact value).
 *   n_probes 1 .. min(FASTAR_MAX_PROBES, n_bits + 1).  Probe p >= 1 flips
 *            the bit of the p-th nearest hyperplane to x by distance
 *            |x . r_j| / |r_j| (ascending, ties to the smaller j): the second
 *            probe is the Hamming-1 neighbour across the nearest hyperplane,
 *            later ones are multi-probe LSH's next neighbours (paperlayer.ai
 *            section 2, approximate nearest neighbor search: bucket probing).
 *   bucket   out [H][N][n_probes] int32.
 *   offsets  out [H][2^n_bits + 1] int32, or NULL (no index).
 *   perm     out [H][N] int32, or NULL (together with offsets).
 *            perm lists token indices sorted by bucket (with several
 *            probes, the smallest of the token's probe buckets; each token
 *            once), ascending token within a bucket; offsets[B] = number of
 *            tokens whose (smallest) bucket is < B.
 *   ws       device workspace of at least fastar_hash_workspace() bytes,
 *            used by the index only (may be NULL when offsets is NULL).
 *   diag     optional device counters (may be NULL).
 * ---------------------------------------------------------------------- */
size_t fastar_hash_workspace(int heads, int64_t n, int n_bits, int n_probes);
fastar_status_t fastar_hash(const fastar_tensor_t* x, const void* planes, int n_bits,
                            int n_probes, int32_t* bucket, int32_t* offsets, int32_t* perm,
                            void* ws, size_t ws_bytes, fastar_diag_t* diag,
                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * fastar_hash_multi -- the ids of fastar_hash (no index) for up to four
 * tensors hashed with the same planes, in one launch for bf16 (the chunk's
 * queries, new keys and prompt keys share one hashing: paper.rainbus.top
 * "technical novelty").
 *   count     1..4.
 *   x         [count] tensors [H_i][N_i][d], one dtype and d.
 *   n_probes  [count] host ints, each as for fastar_hash.
 *   bucket    [count] device outputs [H_i][N_i][n_probes[i]] int32.
 *   planes, n_bits, diag: as for fastar_hash.  Build an index of any of the
 *   ids with fastar_bucket_index.
 * ---------------------------------------------------------------------- */
fastar_status_t fastar_hash_multi(int count, const fastar_tensor_t* const* x, const int* n_probes,
                                  int32_t* const* bucket, const void* planes, int n_bits,
                                  fastar_diag_t* diag, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fastar_bucket_index -- the bucket-contiguous index of fastar_hash on its
 * own, for ids already computed (e.g. the representatives of a cache).
 *   bucket  [H][n][n_probes] int32.
 *   n_valid optional device [H]: only the first min(n_valid[h], n) entries of
 *           head h are indexed (NULL: all n).
 *   offsets [H][2^n_bits + 1], perm [H][n]: as for fastar_hash.
 * ---------------------------------------------------------------------- */
size_t fastar_bucket_index_workspace(int heads, int64_t n);
fastar_status_t fastar_bucket_index(const int32_t* bucket, int heads, int64_t n, int n_probes,
                                    int n_bits, const int32_t* n_valid, int32_t* offsets,
                                    int32_t* perm, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * TempCache compressed cache (paperlayer.ai section 5 "TempCache" and
 * appendix A, Lemma 5.1: a group of m identical keys is attended exactly
 * through one key with the group-mean value and logit + log m).
 * Every buffer is caller-owned device memory, head-major:
 *   rep_k      [H][capacity][dim]  representative (most recent) key, dtype
 *   v_mean     [H][capacity][dim]  group mean value, dtype (rounded once)
 *   v_sum      [H][capacity][dim]  float32 running value sum
 *   count      [H][capacity]       int32 group size m
 *   log_count  [H][capacity]       float32 ln m (the attention bias)
 *   rep_bucket [H][capacity]       int32 bucket id of the representative
 *   n_groups   [H]                 int32 groups in use (0 = empty cache)
 *   frontier   [H][tokens_per_frame] int32 group of each token of the last
 *                                  merged frame
 *   status     [1]                 int32 device status word: a merge that has
 *                                  to drop groups for lack of capacity sets
 *                                  bit 0 (FASTAR_CACHE_OVERFLOW), whether or
 *                                  not the call had a diag buffer; nothing
 *                                  clears it but fastar_cache_status(clear)
 *   k_sum      [H][capacity][dim]  float64 running key sum, 8-byte aligned:
 *                                  read and written only by merges with the
 *                                  mean or medoid representative (NULL
 *                                  otherwise allowed).  A sum that leaves
 *                                  float64's exact range (keys of one group
 *                                  whose magnitudes span more than about 50
 *                                  binary orders) is counted in
 *                                  diag->unresolved
 * An empty cache is one with n_groups all 0 and status 0; nothing else needs
 * clearing.  tokens_per_frame must be in [1, 2048]; capacity >=
 * tokens_per_frame.
 *
 * Capacity overflow is an error state, not a supported mode: the groups that
 * do not fit are dropped (group_of_new = -1, and n_groups stays at
 * capacity), and which groups survive can then depend on how the frames were
 * split into calls (within one call a dropped frame f - 1 token is still a
 * candidate of frame f; across calls it is not).  Size the capacity for the
 * worst case (frames merged times tokens per frame) or check
 * fastar_cache_status.
 * ---------------------------------------------------------------------- */
#define FASTAR_CACHE_OVERFLOW 1
typedef struct {
  int32_t heads, dim, capacity, tokens_per_frame, n_bits, dtype;
  void* rep_k;
  void* v_mean;
  float* v_sum;
  int32_t* count;
  float* log_count;
  int32_t* rep_bucket;
  int32_t* n_groups;
  int32_t* frontier;
  int32_t* status;
  double* k_sum;
} fastar_cache_t;

/* fastar_cache_status -- the one call that synchronises: waits for `stream`,
 * reads the cache's status word and returns FASTAR_ERR_CAPACITY if a merge
 * since it was last cleared dropped groups, FASTAR_OK otherwise (or
 * FASTAR_ERR_INVALID / FASTAR_ERR_HIP).  With clear != 0 the word is then
 * reset to 0 (stream-ordered, also waited for).  Not for use under graph
 * capture. */
fastar_status_t fastar_cache_status(const fastar_cache_t* cache, int clear, hipStream_t stream);

/* TempCache variants (paperlayer.ai section 5 "ANN Attention" and appendix C;
 * gist.science and paper.rainbus.top on the query-driven correspondence).
 *   match           FASTAR_MATCH_LSH (default): a new key's candidates are
 *                   the previous frame's tokens with its bucket; similarity is
 *                   the exact cosine.
 *                   FASTAR_MATCH_QUANT: every previous-frame token is a
 *                   candidate; similarity is the cosine of per-row
 *                   symmetric code_bits-bit scalar codes of the two keys
 *                   (c_i = round_half_even(Q x_i / max|x|), Q = 2^(bits-1) - 1:
 *                   the pages' quantized ANN, 8 bits by default), decided
 *                   exactly on the integer codes.
 *   code_bits       2..8 with FASTAR_MATCH_QUANT (0 means 8).
 *   representative  FASTAR_REP_LAST (default): a group keeps its most recent
 *                   key.  FASTAR_REP_MEAN: the mean of its keys, rounded once
 *                   to the cache dtype.  FASTAR_REP_MEDOID: of the previous
 *                   representative and the new key, the one of larger cosine
 *                   with the group's key sum (an online medoid; ties keep the
 *                   previous one).  Mean and medoid need cache->k_sum, and
 *                   merge the frames of a call one at a time (a frame's
 *                   candidates are the representatives of the previous
 *                   frame's groups); a group's bucket is its newest key's.
 *                   The mean is rounded exactly from the float64 sum; the
 *                   medoid's cosine comparison is certified in float64, and
 *                   one it cannot certify (other than identical keys, a tie)
 *                   takes the float64 answer and counts in diag->unresolved.
 *   match_queries   NULL (key-driven), or [H][n_frames * T][d] queries of the
 *                   new frames' tokens, cache dtype: the new side of the
 *                   similarity is the token's query (query-driven
 *                   correspondence); the token joins with its key and value.
 *                   FASTAR_MATCH_QUANT only.
 * Everything else (threshold, one-to-one rule, value means, ln m bias) is
 * the same for every variant. */
typedef enum { FASTAR_MATCH_LSH = 0, FASTAR_MATCH_QUANT = 1 } fastar_match_t;
typedef enum { FASTAR_REP_LAST = 0, FASTAR_REP_MEAN = 1, FASTAR_REP_MEDOID = 2 } fastar_rep_t;
typedef struct {
  int32_t match;
  int32_t code_bits;
  int32_t representative;
  int32_t reserved;
  const fastar_tensor_t* match_queries;
  void* reserved_ptr;
} fastar_merge_opts_t;

/* fastar_tempcache_merge -- merge n_frames new frames, in order.
 *   k_new, v_new  [H][n_frames * tokens_per_frame][dim], cache dtype.
 *   k_new_bucket  [H][n_frames * tokens_per_frame] int32 (fastar_hash, one
 *                 probe, same planes as the queries).
 *   tau           cosine threshold (compared as its float32 value).
 * For each new key j of frame f: candidates are frame f-1's tokens with j's
 * bucket; j proposes to the candidate of largest cosine (ties to the smaller
 * index) if that cosine >= tau; each candidate accepts its proposer of
 * largest cosine (ties to smaller j); accepted keys extend the candidate's
 * group (count+1, value sum += v_j, representative := k_j), all others open
 * new groups in ascending j.
 *   group_of_new  out [H][n_frames * tokens_per_frame] or NULL: group id of
 *                 each new token (-1 if dropped for lack of capacity).
 *   rep_offsets   out [H][2^n_bits + 1], rep_perm out [H][capacity], or both
 *                 NULL: bucket index of the representatives after the merge.
 */
size_t fastar_tempcache_workspace(const fastar_cache_t* cache, int n_frames);
/* the same with options (opts NULL: the defaults, as fastar_tempcache_merge) */
size_t fastar_tempcache_workspace_ex(const fastar_cache_t* cache, int n_frames,
                                     const fastar_merge_opts_t* opts);
fastar_status_t fastar_tempcache_merge_ex(const fastar_cache_t* cache, const fastar_tensor_t* k_new,
                                          const fastar_tensor_t* v_new, const int32_t* k_new_bucket,
                                          int n_frames, float tau, const fastar_merge_opts_t* opts,
                                          int32_t* group_of_new, int32_t* rep_offsets,
                                          int32_t* rep_perm, void* ws, size_t ws_bytes,
                                          fastar_diag_t* diag, hipStream_t stream);

/* fastar_scalar_codes -- the per-row symmetric b-bit codes of FASTAR_MATCH_QUANT
 * (bits 2..8) of x [H][N][d]: codes out [H][N][d] int8 (contiguous),
 * norm2 out [H][N] int32, the sum of squared codes. */
fastar_status_t fastar_scalar_codes(const fastar_tensor_t* x, int bits, int8_t* codes, int32_t* norm2,
                                    hipStream_t stream);
fastar_status_t fastar_tempcache_merge(const fastar_cache_t* cache, const fastar_tensor_t* k_new,
                                       const fastar_tensor_t* v_new,
                                       const int32_t* k_new_bucket, int n_frames, float tau,
                                       int32_t* group_of_new, int32_t* rep_offsets,
                                       int32_t* rep_perm, void* ws, size_t ws_bytes,
                                       fastar_diag_t* diag, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fastar_prune_prompt -- AnnCA (gist.science technical summary, AnnCA; the
 * Chinese summary's method steps): per head, keep the prompt tokens whose
 * bucket is occupied by at least one probe of at least one query.
 *   q_bucket [H][n_q][n_probes], p_bucket [H][n_prompt] int32.
 *   keep     out [H][n_prompt] uint8 (0/1).
 *   kept_idx out [H][n_prompt] int32: kept indices ascending, first n_kept[h].
 *   n_kept   out [H] int32.
 * ---------------------------------------------------------------------- */
fastar_status_t fastar_prune_prompt(const int32_t* q_bucket, int heads, int64_t n_q,
                                    int n_probes, const int32_t* p_bucket, int64_t n_prompt,
                                    int n_bits, uint8_t* keep, int32_t* kept_idx,
                                    int32_t* n_kept, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fastar_bucket_attention -- o_q = sum_j softmax_j(scale * q.k_j + bias_j) v_j
 * over a per-query key set (AnnSA: paperlayer.ai section 5 "AnnSA",
 * gist.science AnnSA; bias ln m from Lemma 5.1).  Three modes:
 *   bucket  k_offsets and k_perm given: query t attends to the keys listed in
 *           the segments of its bucket(s) q_bucket[h][t][0..n_probes).  Rows
 *           are visited in q_perm order (the index from fastar_hash).
 *   list    key_list and n_key_list given: every query attends to
 *           key_list[h][0 .. n_key_list[h]) (AnnCA over the kept prompt).
 *   dense   neither: every query attends to all k->tokens keys; with
 *           n_key_list alone, to keys 0 .. n_key_list[h] of head h (e.g. the
 *           n_groups of a compressed cache).
 *   q      [H][Nq][d]; k, v [H][Nk][d], all the same dtype.
 *   key_bias [H][Nk] float32 or NULL (k's head stride is not used for it:
 *           the bias row of head h starts at h * k->tokens).
 *   out    [H][Nq][d] contiguous, dtype of q.
 *   lse    [H][Nq] float32 natural-log normaliser, or NULL.
 *   A query with an empty key set gets out = 0 and lse = -inf.
 *   bf16: one head's k rows (and v rows) must lie within 4 GiB of its first
 *   row, else FASTAR_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
fastar_status_t fastar_bucket_attention(const fastar_tensor_t* q, const int32_t* q_bucket,
                                        const int32_t* q_perm, int n_probes,
                                        const fastar_tensor_t* k, const fastar_tensor_t* v,
                                        const float* key_bias, const int32_t* k_offsets,
                                        const int32_t* k_perm, int n_bits,
                                        const int32_t* key_list, const int32_t* n_key_list,
                                        float scale, void* out, float* lse,
                                        hipStream_t stream);

/* ------------------------------------------------------------------------
 * fastar_bucket_attention_tables -- AnnSA with n_tables LSH tables of
 * n_probes probes each (hash-based retrieval probing buckets in several
 * tables: paperlayer.ai section 2, approximate nearest neighbor search).
 * Query t attends to A(t) = the union over tables u of the keys whose
 * table-u bucket is one of t's table-u probes; a key in several tables'
 * sets is attended once.  With n_tables = 1 this is fastar_bucket_attention's
 * bucket mode (any n_probes).
 *   n_tables   1 .. FASTAR_MAX_TABLES; n_tables * n_probes <= FASTAR_MAX_PROBES.
 *   q_bucket   [n_tables][H][Nq][n_probes] int32 (fastar_hash with each
 *              table's planes); q_perm [H][Nq] the rows' visit order (e.g.
 *              table 0's index; any permutation is correct).
 *   k_bucket   [n_tables][H][Nk] int32: every key's bucket in each table
 *              (read for tables 0 .. n_tables - 2; may be NULL with one).
 *   k_offsets  [n_tables][H][2^n_bits + 1], k_perm [n_tables][H][Nk]: each
 *              table's key index (fastar_bucket_index; a compressed cache's
 *              with n_valid = n_groups).
 *   q, k, v, key_bias, scale, out, lse: as for fastar_bucket_attention.
 *   n_attended out [H][Nq] int32 |A(t)|, or NULL.
 *   n_tables * H * Nk must be < 2^31.
 * ---------------------------------------------------------------------- */
fastar_status_t fastar_bucket_attention_tables(const fastar_tensor_t* q, int n_tables, const int32_t* q_bucket,
                                               const int32_t* q_perm, int n_probes, const fastar_tensor_t* k,
                                               const fastar_tensor_t* v, const float* key_bias,
                                               const int32_t* k_bucket, const int32_t* k_offsets,
                                               const int32_t* k_perm, int n_bits, float scale, void* out,
                                               float* lse, int32_t* n_attended, hipStream_t stream);

/* fastar_prune_prompt_tables -- AnnCA with n_tables LSH tables: a prompt
 * token is kept if, in some table u, its table-u bucket is one of the
 * table-u probes of any query.  q_bucket [n_tables][H][n_q][n_probes],
 * p_bucket [n_tables][H][n_prompt]; keep, kept_idx, n_kept as for
 * fastar_prune_prompt (which this is with n_tables = 1). */
fastar_status_t fastar_prune_prompt_tables(const int32_t* q_bucket, int n_tables, int heads, int64_t n_q,
                                           int n_probes, const int32_t* p_bucket, int64_t n_prompt, int n_bits,
                                           uint8_t* keep, int32_t* kept_idx, int32_t* n_kept,
                                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * fastar_attention_recall -- attention recall and density of a sparse
 * attention against the dense one over the same keys (paperlayer.ai section 4
 * "Motivation", attention sparsity: the dense-attention mass the retained
 * entries keep; section 3: about 85% at 30% density).  For query q with
 * retained key set A(q):
 *   recall(q)  = sum_{j in A(q)} softmax_j(logits over all keys)
 *              = exp(lse_sparse(q) - lse_dense(q))
 *   density(q) = |A(q)| / n_keys[h]
 * lse_sparse, lse_dense [H][n_q] float32: the lse outputs of
 * fastar_bucket_attention over A(q) and over all keys (same scale and bias).
 * |A(q)| comes from
 *   bucket mode  q_bucket [H][n_q][n_probes] and k_offsets [H][2^n_bits + 1]
 *                (the keys of q's distinct probe buckets), or
 *   list mode    n_retained [H] (q_bucket and k_offsets NULL): the same list
 *                for every query of the head (AnnCA's kept prompt).
 * n_keys [H] int32 device: keys the dense attention ran over.
 * recall out [H][n_q] float32, or NULL; stats out [H][2] float32: the mean
 * recall and the mean density over the head's queries.  An empty retained
 * set has recall 0.  One launch; nothing synchronises.
 * ---------------------------------------------------------------------- */
fastar_status_t fastar_attention_recall(const float* lse_sparse, const float* lse_dense, int heads,
                                        int64_t n_q, const int32_t* q_bucket, int n_probes,
                                        const int32_t* k_offsets, int n_bits,
                                        const int32_t* n_retained, const int32_t* n_keys,
                                        float* recall, float* stats, hipStream_t stream);

/* fastar_attention_recall_counts -- the same with |A(q)| given per query:
 * n_attended [H][n_q] int32 device (e.g. fastar_bucket_attention_tables'
 * n_attended).  Every other argument as for fastar_attention_recall. */
fastar_status_t fastar_attention_recall_counts(const float* lse_sparse, const float* lse_dense, int heads,
                                               int64_t n_q, const int32_t* n_attended, const int32_t* n_keys,
                                               float* recall, float* stats, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fastar_chunk -- one chunk of the per-layer sequence in one call, work
 * that does not depend on a launch's own work carried by extra workgroups of
 * it: the new keys (and prompt keys) hashed; the TempCache merge of the new
 * frames, whose match launch also hashes bf16 queries (one hashing serves
 * every module: paper.rainbus.top "technical novelty"); the representatives'
 * bucket index, whose launch also builds the queries' index (when both use
 * the single counting pass); AnnSA over the merged cache; then, with a
 * prompt, AnnCA pruning and cross-attention over the kept prompt tokens.
 * The part that does not touch the cache (prune, cross-attention, and the
 * queries' hashing when it does not ride on the match) runs on a second
 * stream of the library's own (one per device, default priority, created on
 * the device's first chunk call that is not under stream capture), forked
 * from `stream` with an event after the work it needs and joined back before
 * the call's last launch: in stream order of `stream` the call is one unit,
 * also under graph capture.  Calls on one device share that stream, so
 * concurrent calls on different streams serialise their second branches.
 * Equal to fastar_hash_multi, fastar_bucket_index, fastar_tempcache_merge,
 * fastar_bucket_attention (bucket mode, keys rep_k, values v_mean, bias
 * log_count) and, with a prompt, fastar_prune_prompt and
 * fastar_bucket_attention (list mode, kept_idx), called in that order on the
 * same arguments.
 * ---------------------------------------------------------------------- */
typedef struct {
  /* the chunk */
  const fastar_tensor_t* q;         /* [H][Nq][d] queries                       */
  int n_probes;                     /* 1 .. FASTAR_MAX_PROBES                   */
  const fastar_tensor_t* k_new;     /* [H][n_frames * T][d] new frames' keys    */
  const fastar_tensor_t* v_new;     /* and values                               */
  int n_frames;                     /* > 0                                      */
  const fastar_tensor_t* prompt_k;  /* [H][Np][d], or NULL: no cross-attention  */
  const fastar_tensor_t* prompt_v;
  /* parameters */
  const void* planes;               /* [n_bits][d], as for fastar_hash          */
  int n_bits;                       /* the cache's n_bits                       */
  float tau;                        /* TempCache threshold                      */
  float scale;                      /* softmax scale                            */
  /* state: the compressed cache, merged in place */
  const fastar_cache_t* cache;
  /* outputs (device) */
  int32_t* q_bucket;                /* [H][Nq][n_probes]                        */
  int32_t* q_offsets;               /* [H][2^n_bits + 1]                        */
  int32_t* q_perm;                  /* [H][Nq]                                  */
  int32_t* k_bucket;                /* [H][n_frames * T]                        */
  int32_t* group_of_new;            /* [H][n_frames * T], or NULL               */
  int32_t* rep_offsets;             /* [H][2^n_bits + 1]                        */
  int32_t* rep_perm;                /* [H][capacity]                            */
  void* out;                        /* [H][Nq][d] self-attention, q's dtype     */
  float* lse;                       /* [H][Nq] or NULL                          */
  int32_t* p_bucket;                /* [H][Np]      (with a prompt)             */
  uint8_t* keep;                    /* [H][Np]                                  */
  int32_t* kept_idx;                /* [H][Np]                                  */
  int32_t* n_kept;                  /* [H]                                      */
  void* out_cross;                  /* [H][Nq][d]                               */
  float* lse_cross;                 /* [H][Nq] or NULL                          */
  /* TempCache variant (NULL: the defaults) */
  const fastar_merge_opts_t* merge_opts;
} fastar_chunk_t;

size_t fastar_chunk_workspace(const fastar_chunk_t* args);
fastar_status_t fastar_chunk(const fastar_chunk_t* args, void* ws, size_t ws_bytes,
                             fastar_diag_t* diag, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fastar_chunk_noalloc -- fastar_chunk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same launches on the same arguments, with the
 * workspace taken from a scratch array the library holds on each GPU it runs
 * on (FASTAR_NOALLOC_SCRATCH_BYTES, held until the process ends) instead of
 * a caller buffer.  The caller still passes every input and output.
 * - Returns FASTAR_ERR_WORKSPACE, launching nothing, when the call needs more
 *   than FASTAR_NOALLOC_SCRATCH_BYTES (fastar_chunk_workspace(args) says how
 *   much it needs).
 * - Allocates nothing: no hipMalloc, no allocating library routine.  The
 *   first call on a device looks up that device's scratch address once.
 * - Every call on one GPU shares that GPU's scratch: calls that overlap on
 *   one GPU (different streams, or different host threads) race and must be
 *   ordered by the caller.  The scratch keeps the last call's contents; the
 *   kernels write every scratch word before they read it, so nothing needs
 *   clearing between calls.
 * ---------------------------------------------------------------------- */
#define FASTAR_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
fastar_status_t fastar_chunk_noalloc(const fastar_chunk_t* args, fastar_diag_t* diag,
                                     hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FASTAR_H */

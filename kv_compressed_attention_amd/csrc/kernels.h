// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fastar.h"
#include "merge_args.h"

namespace fastar {

// hash.hip ------------------------------------------------------------------
struct HashJob {  // one tensor [H][N][d] hashed into bucket [H][N][P]
  const void* x;
  int64_t sh, st, N;
  int H, P;
  int32_t* bucket;
};
constexpr int kMaxHashJobs = 4;
struct HashJobs {
  HashJob j[kMaxHashJobs];
  int64_t tile_end[kMaxHashJobs];  // filled by launch_hash_multi
  int count;
};
hipError_t launch_hash(const fastar_tensor_t& x, const void* planes, int n_bits, int n_probes,
                       int32_t* bucket, fastar_diag_t* diag, hipStream_t s);
// all tensors share dim and dtype; one launch for bf16
hipError_t launch_hash_multi(HashJobs jobs, int dim, int dtype, const void* planes, int n_bits,
                             fastar_diag_t* diag, hipStream_t s);

// index.hip -----------------------------------------------------------------
// a bucket index (n items per head, ids [H][n][P] sorted by their first
// probe) that another index launch of the same heads and bits builds in
// extra workgroups (the chunk sequence's queries, next to the
// representatives)
struct IndexJob {
  const int32_t* bucket;
  int64_t n;
  int n_bits;
  int P;
  int32_t* offsets;
  int32_t* perm;
};
// With extra (the single counting pass only, which must apply to both), the
// launch also builds that index.
hipError_t launch_bucket_index(const int32_t* bucket, int heads, int64_t n, int n_probes,
                               int n_bits, const int32_t* n_valid, int32_t* offsets,
                               int32_t* perm, int32_t* ws, hipStream_t s,
                               const IndexJob* extra = nullptr);

// whether launch_bucket_index uses the single counting pass for n items (and,
// with n_extra > 0, can build an IndexJob of n_extra items in the same launch)
bool direct_index_supported(int64_t n, int n_probes, int n_bits, int64_t n_extra = 0,
                            int extra_probes = 1);

// prune.hip -----------------------------------------------------------------
hipError_t launch_prune(const int32_t* q_bucket, int heads, int64_t n_q, int n_probes,
                        const int32_t* p_bucket, int64_t n_prompt, int n_bits, uint8_t* keep,
                        int32_t* kept_idx, int32_t* n_kept, hipStream_t s, int n_tables = 1);

// attention.hip -------------------------------------------------------------
struct AttnArgs {
  const void* q; int64_t q_sh, q_st, nq;
  const int32_t* q_bucket; const int32_t* q_perm; int n_probes;
  const void* k; int64_t k_sh, k_st;
  const void* v; int64_t v_sh, v_st; int64_t nk;
  const float* key_bias; const int32_t* k_offsets; const int32_t* k_perm; int n_bits;
  const int32_t* key_list; const int32_t* n_key_list;
  float scale; void* out; float* lse;
  int heads, dim, dtype, mode;  // mode: 0 bucket, 1 list, 2 dense, 3 tables
  // mode 3: n_tables LSH tables of n_probes probes each; q_bucket
  // [n_tables][H][nq][n_probes], k_offsets / k_perm / k_bucket per table
  // ([n_tables][H][...]), n_attended [H][nq] out or NULL
  int n_tables = 1;
  const int32_t* k_bucket = nullptr;
  int32_t* n_attended = nullptr;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// recall.hip ----------------------------------------------------------------
hipError_t launch_recall(const float* lse_s, const float* lse_d, int heads, int64_t nq,
                         const int32_t* q_bucket, int P, const int32_t* k_offsets, int nbits,
                         const int32_t* n_retained, const int32_t* n_keys, float* recall, float* stats,
                         hipStream_t s, const int32_t* n_per_query = nullptr);

// tempcache.hip -------------------------------------------------------------
struct MergeWs {
  int32_t* off;       // [H][n_frames+1][2^b+1] bucket offsets per table (see tempcache.hip)
  int32_t* tok;       // [H][n_frames+1][T] tokens sorted by bucket
  int32_t* tbk;       // [H][n_frames+1][T] their buckets
  int32_t* candg;     // [H][T]
  int32_t* link;      // [H][n_frames][T]
  int32_t* ocnt;      // [H][ceil(n_frames T / 64) + 1]
  int32_t* nextj;     // [H][n_frames][T]
  int32_t* prop;      // [H][n_frames][3][T]
  int32_t* mrange;    // [H][n_frames][ceil(T / 64)][4]
  int32_t* index_ws;  // bucket index scratch
  const IndexJob* also_index = nullptr;  // direct-index job for the representatives' index launch, or none
  // bf16 rows (the queries, one or two probes) that extra workgroups of the match launch hash
  // with hash_planes and hash_bits (same dim as the cache), or none
  const HashJobs* also_hash = nullptr;
  const void* hash_planes = nullptr;
  int hash_bits = 0;
  int rep = FASTAR_REP_LAST;  // representative kind (mean and medoid: one frame per call)
  int64_t kb_stride = 0;      // row stride of k_new_bucket and group_of_new (0: n_frames * T)
  // an event the stream waits for before the representatives' index launch
  // (the job in also_index is written on another stream), or none
  hipEvent_t index_after = nullptr;
  // an event recorded right after the match launch (the jobs in also_hash
  // are then hashed), or none
  hipEvent_t after_match = nullptr;
};
// the merge's last launches for any match kind: the group updates (from the
// links, successors and opener counts in a) and the representatives' index
hipError_t launch_merge_apply(const fastar_cache_t& c, const fastar_tensor_t& kn, const fastar_tensor_t& vn,
                              const int32_t* kb, const MergeArgs& a, int32_t* group_of_new,
                              int32_t* rep_offsets, int32_t* rep_perm, const MergeWs& ws,
                              fastar_diag_t* diag, hipStream_t s);

// tempcache_quant.hip ---------------------------------------------------------
// per-row symmetric b-bit codes of x's rows: codes [rows][dim] int8, norm2
// [rows] int32 (sum of squared codes)
hipError_t launch_scalar_codes(const fastar_tensor_t& x, int bits, int8_t* codes, int32_t* norm2,
                               hipStream_t s);
// the quantized match's workspace (beyond MergeWs's link / nextj / ocnt)
struct QuantWs {
  int8_t* codes;   // [H][tables][T][dim]
  int32_t* norm2;  // [H][tables][T]
  float* rn;       // [H][tables][T]   1 / sqrt(norm2) (0 for a zero code)
  float* bias;     // [H][tables][T]   0, or -inf for a token that is no candidate
  int32_t* ptgt;   // [H][F][T]     proposed candidate, or -1
  int32_t* pdot;   // [H][F][T]     exact code dot product with it
  float* pcos;     // [H][F][T]     float32 cosine estimate
  // codes etc. hold F + 1 tables, or 2F + 1 with query-driven matching (tables F + 1 .. 2F: queries)
};
size_t quant_workspace_bytes(int heads, int T, int F, int dim, bool query_driven);
QuantWs quant_carve(int heads, int T, int F, int dim, bool query_driven, void* ws);
// q_new: the new frames' queries (query-driven matching), or NULL
hipError_t launch_tempcache_merge_quant(const fastar_cache_t& c, const fastar_tensor_t& k_new,
                                        const fastar_tensor_t& v_new, const fastar_tensor_t* q_new,
                                        const int32_t* k_new_bucket, int n_frames, float tau, int bits,
                                        int32_t* group_of_new, int32_t* rep_offsets, int32_t* rep_perm,
                                        const MergeWs& ws, const QuantWs& qws, fastar_diag_t* diag,
                                        hipStream_t s);

hipError_t launch_tempcache_merge(const fastar_cache_t& c, const fastar_tensor_t& k_new,
                                  const fastar_tensor_t& v_new, const int32_t* k_new_bucket,
                                  int n_frames, float tau, int32_t* group_of_new,
                                  int32_t* rep_offsets, int32_t* rep_perm, const MergeWs& ws,
                                  fastar_diag_t* diag, hipStream_t s);

}  // namespace fastar

// extern "C" entry points of libfastar: host-side validation, workspace
// carving and kernel launches.  Nothing here allocates or synchronises.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

fastar_status_t fail(fastar_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

fastar_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return FASTAR_OK;
  return fail(FASTAR_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// checks common to every [H][N][d] tensor argument
fastar_status_t check_tensor(const fastar_tensor_t* t, const char* name) {
  if (!t) return fail(FASTAR_ERR_INVALID, "%s: null descriptor", name);
  if (t->dtype != FASTAR_F32 && t->dtype != FASTAR_BF16)
    return fail(FASTAR_ERR_UNSUPPORTED, "%s: dtype %d (want 0=f32 or 1=bf16)", name, t->dtype);
  if (t->dim != 64 && t->dim != 128)
    return fail(FASTAR_ERR_UNSUPPORTED, "%s: dim %d (want 64 or 128)", name, t->dim);
  if (t->heads < 0 || t->tokens < 0) return fail(FASTAR_ERR_INVALID, "%s: negative size", name);
  if ((int64_t)t->heads * t->tokens > 0) {
    if (!t->data) return fail(FASTAR_ERR_INVALID, "%s: null data", name);
    if (!aligned16(t->data)) return fail(FASTAR_ERR_INVALID, "%s: data not 16-byte aligned", name);
    if (t->stride_token < t->dim || t->stride_token % 8 != 0)
      return fail(FASTAR_ERR_INVALID, "%s: stride_token %lld must be >= dim and a multiple of 8",
                  name, (long long)t->stride_token);
    if (t->heads > 1 && (t->stride_head % 8 != 0 ||
                         t->stride_head < (t->tokens - 1) * t->stride_token + t->dim))
      return fail(FASTAR_ERR_INVALID, "%s: stride_head %lld overlaps tokens or is not a multiple of 8",
                  name, (long long)t->stride_head);
  }
  if ((int64_t)t->heads * t->tokens >= (int64_t)1 << 31)
    return fail(FASTAR_ERR_UNSUPPORTED, "%s: heads*tokens must be < 2^31", name);
  return FASTAR_OK;
}

fastar_status_t check_bits(int n_bits, int n_probes) {
  if (n_bits < 0 || n_bits > 15) return fail(FASTAR_ERR_UNSUPPORTED, "n_bits %d not in [0, 15]", n_bits);
  if (n_probes != 1 && n_probes != 2) return fail(FASTAR_ERR_UNSUPPORTED, "n_probes %d not 1 or 2", n_probes);
  if (n_probes == 2 && n_bits < 1) return fail(FASTAR_ERR_INVALID, "two probes need n_bits >= 1");
  return FASTAR_OK;
}

}  // namespace

extern "C" {

const char* fastar_status_string(int status) {
  switch (status) {
    case FASTAR_OK: return "ok";
    case FASTAR_ERR_INVALID: return "invalid argument";
    case FASTAR_ERR_UNSUPPORTED: return "unsupported argument";
    case FASTAR_ERR_WORKSPACE: return "workspace too small";
    case FASTAR_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* fastar_last_error(void) { return g_err; }

int fastar_version(void) { return 100; }

// ---------------------------------------------------------------------------
size_t fastar_hash_workspace(int heads, int64_t n, int n_bits, int n_probes) {
  (void)n_bits;
  (void)n_probes;
  if (heads < 0 || n < 0) return 0;
  // the bucket index's scratch (hashing itself needs none)
  return align_up(16 * (size_t)heads * (size_t)n);
}

fastar_status_t fastar_hash(const fastar_tensor_t* x, const void* planes, int n_bits, int n_probes,
                            int32_t* bucket, int32_t* offsets, int32_t* perm, void* ws,
                            size_t ws_bytes, fastar_diag_t* diag, hipStream_t stream) {
  fastar_status_t st = check_tensor(x, "x");
  if (st != FASTAR_OK) return st;
  if ((st = check_bits(n_bits, n_probes)) != FASTAR_OK) return st;
  const int64_t hn = (int64_t)x->heads * x->tokens;
  if ((offsets == nullptr && perm != nullptr) || (offsets != nullptr && perm == nullptr && hn > 0))
    return fail(FASTAR_ERR_INVALID, "offsets and perm must both be given or both be NULL");
  if (hn == 0) {
    if (offsets && x->heads > 0) {
      // an empty index: offsets all zero
      if (ws_bytes < fastar_hash_workspace(x->heads, 0, n_bits, n_probes))
        return fail(FASTAR_ERR_WORKSPACE, "workspace too small");
      return hip_status(fastar::launch_bucket_index(bucket, x->heads, 0, n_probes, n_bits, nullptr,
                                                    offsets, perm, (int32_t*)ws, stream),
                        "bucket_index");
    }
    return FASTAR_OK;
  }
  if (n_bits > 0 && (!planes || !aligned16(planes)))
    return fail(FASTAR_ERR_INVALID, "planes must be a non-null, 16-byte aligned pointer");
  if (!bucket) return fail(FASTAR_ERR_INVALID, "bucket is NULL");
  if (offsets && (!ws || ws_bytes < fastar_hash_workspace(x->heads, x->tokens, n_bits, n_probes)))
    return fail(FASTAR_ERR_WORKSPACE, "workspace: need %zu bytes, got %zu",
                fastar_hash_workspace(x->heads, x->tokens, n_bits, n_probes), ws_bytes);
  hipError_t e = fastar::launch_hash(*x, planes, n_bits, n_probes, bucket, diag, stream);
  if (e != hipSuccess) return hip_status(e, "hash");
  if (offsets)
    return hip_status(fastar::launch_bucket_index(bucket, x->heads, x->tokens, n_probes, n_bits,
                                                  nullptr, offsets, perm, (int32_t*)ws, stream),
                      "bucket_index");
  return FASTAR_OK;
}

// ---------------------------------------------------------------------------
fastar_status_t fastar_hash_multi(int count, const fastar_tensor_t* const* x, const int* n_probes,
                                  int32_t* const* bucket, const void* planes, int n_bits,
                                  fastar_diag_t* diag, hipStream_t stream) {
  if (count < 1 || count > fastar::kMaxHashJobs)
    return fail(FASTAR_ERR_INVALID, "count %d not in [1, %d]", count, fastar::kMaxHashJobs);
  if (!x || !n_probes || !bucket) return fail(FASTAR_ERR_INVALID, "x, n_probes and bucket must be arrays");
  fastar::HashJobs jobs;
  jobs.count = count;
  bool any = false;
  for (int i = 0; i < count; ++i) {
    fastar_status_t st = check_tensor(x[i], "x[i]");
    if (st != FASTAR_OK) return st;
    if ((st = check_bits(n_bits, n_probes[i])) != FASTAR_OK) return st;
    if (x[i]->dtype != x[0]->dtype || x[i]->dim != x[0]->dim)
      return fail(FASTAR_ERR_INVALID, "x[%d]: dtype and dim must match x[0]", i);
    const bool nonempty = (int64_t)x[i]->heads * x[i]->tokens > 0;
    if (nonempty && !bucket[i]) return fail(FASTAR_ERR_INVALID, "bucket[%d] is NULL", i);
    any = any || nonempty;
    jobs.j[i] = fastar::HashJob{x[i]->data, x[i]->stride_head, x[i]->stride_token, x[i]->tokens,
                                x[i]->heads, n_probes[i], bucket[i]};
  }
  if (!any) return FASTAR_OK;
  if (n_bits > 0 && (!planes || !aligned16(planes)))
    return fail(FASTAR_ERR_INVALID, "planes must be a non-null, 16-byte aligned pointer");
  return hip_status(fastar::launch_hash_multi(jobs, x[0]->dim, x[0]->dtype, planes, n_bits, diag, stream),
                    "hash_multi");
}

// ---------------------------------------------------------------------------
size_t fastar_bucket_index_workspace(int heads, int64_t n) {
  if (heads < 0 || n < 0) return 0;
  return align_up(16 * (size_t)heads * (size_t)n);
}

fastar_status_t fastar_bucket_index(const int32_t* bucket, int heads, int64_t n, int n_probes,
                                    int n_bits, const int32_t* n_valid, int32_t* offsets,
                                    int32_t* perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  fastar_status_t st = check_bits(n_bits, n_probes);
  if (st != FASTAR_OK) return st;
  if (heads < 0 || n < 0) return fail(FASTAR_ERR_INVALID, "negative size");
  if ((int64_t)heads * n >= (int64_t)1 << 31) return fail(FASTAR_ERR_UNSUPPORTED, "heads*n must be < 2^31");
  if (heads == 0) return FASTAR_OK;
  if (!offsets || (n > 0 && (!perm || !bucket))) return fail(FASTAR_ERR_INVALID, "null pointer");
  if (n > 0 && (!ws || ws_bytes < fastar_bucket_index_workspace(heads, n)))
    return fail(FASTAR_ERR_WORKSPACE, "workspace too small");
  return hip_status(fastar::launch_bucket_index(bucket, heads, n, n_probes, n_bits, n_valid, offsets,
                                                perm, (int32_t*)ws, stream),
                    "bucket_index");
}

// ---------------------------------------------------------------------------
size_t fastar_tempcache_workspace(const fastar_cache_t* c, int n_frames) {
  if (!c || n_frames < 0 || c->heads < 0 || c->tokens_per_frame < 0 || c->capacity < 0) return 0;
  if (c->n_bits < 0 || c->n_bits > 15) return 0;
  const size_t H = c->heads, T = c->tokens_per_frame, F = n_frames;
  const size_t nb = ((size_t)1 << c->n_bits) + 1;
  const size_t nblk = (F * T + 63) / 64;
  return align_up(4 * H * (F + 1) * nb) + 2 * align_up(4 * H * (F + 1) * T) + align_up(4 * H * T) +
         align_up(4 * H * F * T) + align_up(4 * H * (nblk + 1)) + align_up(4 * H * F * T) +
         align_up(16 * H * (size_t)c->capacity);
}

fastar_status_t fastar_tempcache_merge(const fastar_cache_t* c, const fastar_tensor_t* k_new,
                                       const fastar_tensor_t* v_new, const int32_t* k_new_bucket,
                                       int n_frames, float tau, int32_t* group_of_new,
                                       int32_t* rep_offsets, int32_t* rep_perm, void* ws,
                                       size_t ws_bytes, fastar_diag_t* diag, hipStream_t stream) {
  if (!c) return fail(FASTAR_ERR_INVALID, "cache is NULL");
  fastar_status_t st;
  if ((st = check_tensor(k_new, "k_new")) != FASTAR_OK) return st;
  if ((st = check_tensor(v_new, "v_new")) != FASTAR_OK) return st;
  if ((st = check_bits(c->n_bits, 1)) != FASTAR_OK) return st;
  if (c->dtype != k_new->dtype || c->dtype != v_new->dtype)
    return fail(FASTAR_ERR_INVALID, "cache, k_new and v_new must share one dtype");
  if (c->dim != k_new->dim || c->dim != v_new->dim)
    return fail(FASTAR_ERR_INVALID, "cache, k_new and v_new must share one dim");
  if (c->heads != k_new->heads || c->heads != v_new->heads)
    return fail(FASTAR_ERR_INVALID, "cache, k_new and v_new must share one head count");
  if (n_frames < 0) return fail(FASTAR_ERR_INVALID, "n_frames < 0");
  if (c->tokens_per_frame <= 0 || c->tokens_per_frame > 2048)
    return fail(FASTAR_ERR_UNSUPPORTED, "tokens_per_frame %d not in [1, 2048]", c->tokens_per_frame);
  if (k_new->tokens != (int64_t)n_frames * c->tokens_per_frame || v_new->tokens != k_new->tokens)
    return fail(FASTAR_ERR_INVALID, "k_new/v_new must hold n_frames * tokens_per_frame tokens");
  if (c->capacity < c->tokens_per_frame)
    return fail(FASTAR_ERR_INVALID, "capacity %d < tokens_per_frame", c->capacity);
  if ((int64_t)c->heads * c->capacity >= (int64_t)1 << 31)
    return fail(FASTAR_ERR_UNSUPPORTED, "heads*capacity must be < 2^31");
  if (!(tau == tau) || tau == INFINITY || tau == -INFINITY) return fail(FASTAR_ERR_INVALID, "tau must be finite");
  if ((rep_offsets == nullptr) != (rep_perm == nullptr))
    return fail(FASTAR_ERR_INVALID, "rep_offsets and rep_perm must both be given or both be NULL");
  if (c->heads == 0 || n_frames == 0) {
    if (rep_offsets && c->heads > 0) {
      if (!ws || ws_bytes < fastar_tempcache_workspace(c, n_frames))
        return fail(FASTAR_ERR_WORKSPACE, "workspace too small");
      const size_t off = fastar_tempcache_workspace(c, n_frames) -
                         align_up(16 * (size_t)c->heads * (size_t)c->capacity);
      return hip_status(fastar::launch_bucket_index(c->rep_bucket, c->heads, c->capacity, 1, c->n_bits,
                                                    c->n_groups, rep_offsets, rep_perm,
                                                    (int32_t*)((char*)ws + off), stream),
                        "bucket_index");
    }
    return FASTAR_OK;
  }
  if (!c->rep_k || !c->v_mean || !c->v_sum || !c->count || !c->log_count || !c->rep_bucket ||
      !c->n_groups || !c->frontier || !k_new_bucket)
    return fail(FASTAR_ERR_INVALID, "a cache buffer or k_new_bucket is NULL");
  if (!aligned16(c->rep_k) || !aligned16(c->v_mean) || !aligned16(c->v_sum))
    return fail(FASTAR_ERR_INVALID, "cache rows must be 16-byte aligned");
  if (!ws || ws_bytes < fastar_tempcache_workspace(c, n_frames))
    return fail(FASTAR_ERR_WORKSPACE, "workspace: need %zu bytes, got %zu",
                fastar_tempcache_workspace(c, n_frames), ws_bytes);
  const size_t H = c->heads, T = c->tokens_per_frame, F = n_frames;
  const size_t nb = ((size_t)1 << c->n_bits) + 1;
  char* w = (char*)ws;
  auto take = [&](size_t bytes) {
    char* p = w;
    w += align_up(bytes);
    return (int32_t*)p;
  };
  fastar::MergeWs mw;
  mw.off = take(4 * H * (F + 1) * nb);
  mw.tok = take(4 * H * (F + 1) * T);
  mw.tbk = take(4 * H * (F + 1) * T);
  mw.candg = take(4 * H * T);
  mw.link = take(4 * H * F * T);
  mw.ocnt = take(4 * H * ((F * T + 63) / 64 + 1));
  mw.nextj = take(4 * H * F * T);
  mw.index_ws = take(16 * H * (size_t)c->capacity);
  return hip_status(fastar::launch_tempcache_merge(*c, *k_new, *v_new, k_new_bucket, n_frames, tau,
                                                   group_of_new, rep_offsets, rep_perm, mw, diag,
                                                   stream),
                    "tempcache_merge");
}

// ---------------------------------------------------------------------------
fastar_status_t fastar_prune_prompt(const int32_t* q_bucket, int heads, int64_t n_q, int n_probes,
                                    const int32_t* p_bucket, int64_t n_prompt, int n_bits,
                                    uint8_t* keep, int32_t* kept_idx, int32_t* n_kept,
                                    hipStream_t stream) {
  fastar_status_t st = check_bits(n_bits, n_probes);
  if (st != FASTAR_OK) return st;
  if (heads < 0 || n_q < 0 || n_prompt < 0) return fail(FASTAR_ERR_INVALID, "negative size");
  if (heads == 0) return FASTAR_OK;
  if (!n_kept) return fail(FASTAR_ERR_INVALID, "n_kept is NULL");
  if (n_q > 0 && !q_bucket) return fail(FASTAR_ERR_INVALID, "q_bucket is NULL");
  if (n_prompt > 0 && (!p_bucket || !keep || !kept_idx))
    return fail(FASTAR_ERR_INVALID, "p_bucket, keep or kept_idx is NULL");
  if ((int64_t)heads * n_q * n_probes >= (int64_t)1 << 31 || (int64_t)heads * n_prompt >= (int64_t)1 << 31)
    return fail(FASTAR_ERR_UNSUPPORTED, "sizes must be < 2^31");
  return hip_status(fastar::launch_prune(q_bucket, heads, n_q, n_probes, p_bucket, n_prompt, n_bits,
                                         keep, kept_idx, n_kept, stream),
                    "prune_prompt");
}

// ---------------------------------------------------------------------------
fastar_status_t fastar_bucket_attention(const fastar_tensor_t* q, const int32_t* q_bucket,
                                        const int32_t* q_perm, int n_probes,
                                        const fastar_tensor_t* k, const fastar_tensor_t* v,
                                        const float* key_bias, const int32_t* k_offsets,
                                        const int32_t* k_perm, int n_bits,
                                        const int32_t* key_list, const int32_t* n_key_list,
                                        float scale, void* out, float* lse, hipStream_t stream) {
  fastar_status_t st;
  if ((st = check_tensor(q, "q")) != FASTAR_OK) return st;
  if ((st = check_tensor(k, "k")) != FASTAR_OK) return st;
  if ((st = check_tensor(v, "v")) != FASTAR_OK) return st;
  if (q->dtype != k->dtype || q->dtype != v->dtype) return fail(FASTAR_ERR_INVALID, "q, k, v dtypes differ");
  if (q->dim != k->dim || q->dim != v->dim) return fail(FASTAR_ERR_INVALID, "q, k, v dims differ");
  if (q->heads != k->heads || q->heads != v->heads) return fail(FASTAR_ERR_INVALID, "q, k, v head counts differ");
  if (k->tokens != v->tokens) return fail(FASTAR_ERR_INVALID, "k and v token counts differ");
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return fail(FASTAR_ERR_INVALID, "scale must be finite");
  int mode;
  if (k_offsets || k_perm) {
    if (!k_offsets || !k_perm) return fail(FASTAR_ERR_INVALID, "bucket mode needs k_offsets and k_perm");
    if (key_list || n_key_list) return fail(FASTAR_ERR_INVALID, "give either bucket segments or a key list");
    if ((st = check_bits(n_bits, n_probes)) != FASTAR_OK) return st;
    mode = 0;
  } else if (key_list || n_key_list) {
    if (!key_list || !n_key_list) return fail(FASTAR_ERR_INVALID, "list mode needs key_list and n_key_list");
    mode = 1;
  } else {
    mode = 2;
  }
  if ((int64_t)q->heads * q->tokens == 0) return FASTAR_OK;
  if (!out || !aligned16(out)) return fail(FASTAR_ERR_INVALID, "out must be a non-null 16-byte aligned pointer");
  if (mode == 0 && (!q_bucket || !q_perm)) return fail(FASTAR_ERR_INVALID, "bucket mode needs q_bucket and q_perm");
  if (q->dtype == FASTAR_BF16 && k->tokens > 0) {
    // the bf16 kernel addresses a head's k and v rows by 32-bit byte offsets
    const int64_t span_k = ((int64_t)(k->tokens - 1) * k->stride_token + k->dim) * 2;
    const int64_t span_v = ((int64_t)(v->tokens - 1) * v->stride_token + v->dim) * 2;
    if (span_k > 0xFFFFFFFFll || span_v > 0xFFFFFFFFll)
      return fail(FASTAR_ERR_UNSUPPORTED, "a head's k or v rows span more than 4 GiB");
  }
  fastar::AttnArgs a;
  a.q = q->data; a.q_sh = q->stride_head; a.q_st = q->stride_token; a.nq = q->tokens;
  a.q_bucket = q_bucket; a.q_perm = q_perm; a.n_probes = mode == 0 ? n_probes : 1;
  a.k = k->data; a.k_sh = k->stride_head; a.k_st = k->stride_token;
  a.v = v->data; a.v_sh = v->stride_head; a.v_st = v->stride_token; a.nk = k->tokens;
  a.key_bias = key_bias; a.k_offsets = k_offsets; a.k_perm = k_perm; a.n_bits = n_bits;
  a.key_list = key_list; a.n_key_list = n_key_list;
  a.scale = scale; a.out = out; a.lse = lse;
  a.heads = q->heads; a.dim = q->dim; a.dtype = q->dtype; a.mode = mode;
  return hip_status(fastar::launch_attention(a, stream), "bucket_attention");
}

}  // extern "C"

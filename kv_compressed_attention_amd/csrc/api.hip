// extern "C" entry points of libfastar: host-side validation, workspace
// carving and kernel launches.  Nothing here allocates; only
// fastar_cache_status synchronises.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kernels.h"

// The workspace of fastar_chunk_noalloc: one copy on every GPU the library
// runs on, 256-byte aligned like the workspace carve.  Host code never uses
// this name as an address: each device's address comes from
// hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[FASTAR_NOALLOC_SCRATCH_BYTES];

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
  if (n_probes < 1 || n_probes > FASTAR_MAX_PROBES)
    return fail(FASTAR_ERR_UNSUPPORTED, "n_probes %d not in [1, %d]", n_probes, FASTAR_MAX_PROBES);
  if (n_probes > n_bits + 1) return fail(FASTAR_ERR_INVALID, "%d probes need n_bits >= %d", n_probes, n_probes - 1);
  return FASTAR_OK;
}


// ---- argument checks shared by the single calls and fastar_chunk ----------

fastar_status_t hash_multi_check(int count, const fastar_tensor_t* const* x, const int* n_probes,
                                 int32_t* const* bucket, const void* planes, int n_bits,
                                 fastar::HashJobs* jobs, bool* any) {
  if (count < 1 || count > fastar::kMaxHashJobs)
    return fail(FASTAR_ERR_INVALID, "count %d not in [1, %d]", count, fastar::kMaxHashJobs);
  if (!x || !n_probes || !bucket) return fail(FASTAR_ERR_INVALID, "x, n_probes and bucket must be arrays");
  jobs->count = count;
  *any = false;
  for (int i = 0; i < count; ++i) {
    fastar_status_t st = check_tensor(x[i], "x[i]");
    if (st != FASTAR_OK) return st;
    if ((st = check_bits(n_bits, n_probes[i])) != FASTAR_OK) return st;
    if (x[i]->dtype != x[0]->dtype || x[i]->dim != x[0]->dim)
      return fail(FASTAR_ERR_INVALID, "x[%d]: dtype and dim must match x[0]", i);
    const bool nonempty = (int64_t)x[i]->heads * x[i]->tokens > 0;
    if (nonempty && !bucket[i]) return fail(FASTAR_ERR_INVALID, "bucket[%d] is NULL", i);
    *any = *any || nonempty;
    jobs->j[i] = fastar::HashJob{x[i]->data, x[i]->stride_head, x[i]->stride_token, x[i]->tokens,
                                 x[i]->heads, n_probes[i], bucket[i]};
  }
  if (*any && n_bits > 0 && (!planes || !aligned16(planes)))
    return fail(FASTAR_ERR_INVALID, "planes must be a non-null, 16-byte aligned pointer");
  // the bf16 launch numbers its 16-row tiles with 32-bit integers
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) tiles += (int64_t)x[i]->heads * ((x[i]->tokens + 15) / 16);
  if (tiles >= (int64_t)1 << 31)
    return fail(FASTAR_ERR_UNSUPPORTED, "more than 2^31 tiles of 16 rows in one call");
  return FASTAR_OK;
}

size_t merge_workspace(const fastar_cache_t* c, int n_frames) {
  if (!c || n_frames < 0 || c->heads < 0 || c->tokens_per_frame < 0 || c->capacity < 0) return 0;
  if (c->n_bits < 0 || c->n_bits > 15) return 0;
  const size_t H = c->heads, T = c->tokens_per_frame, F = n_frames;
  const size_t nb = ((size_t)1 << c->n_bits) + 1;
  const size_t nblk = (F * T + 63) / 64;
  return align_up(4 * H * (F + 1) * nb) + 2 * align_up(4 * H * (F + 1) * T) + align_up(4 * H * T) +
         align_up(4 * H * F * T) + align_up(4 * H * (nblk + 1)) + align_up(4 * H * F * T) +
         align_up(12 * H * F * T) + align_up(16 * H * F * ((T + 63) / 64)) +
         align_up(16 * H * (size_t)c->capacity);
}

// a merge's options, checked (NULL: the defaults)
struct MergeOpt {
  int match = FASTAR_MATCH_LSH, bits = 8, rep = FASTAR_REP_LAST;
  const fastar_tensor_t* q = nullptr;
};
fastar_status_t merge_opts(const fastar_merge_opts_t* o, MergeOpt* m) {
  *m = MergeOpt();
  if (!o) return FASTAR_OK;
  if (o->match != FASTAR_MATCH_LSH && o->match != FASTAR_MATCH_QUANT)
    return fail(FASTAR_ERR_UNSUPPORTED, "merge option match %d unknown", o->match);
  m->match = o->match;
  if (o->match == FASTAR_MATCH_QUANT && o->code_bits != 0) {
    if (o->code_bits < 2 || o->code_bits > 8)
      return fail(FASTAR_ERR_UNSUPPORTED, "code_bits %d not in [2, 8]", o->code_bits);
    m->bits = o->code_bits;
  }
  if (o->representative != FASTAR_REP_LAST && o->representative != FASTAR_REP_MEAN &&
      o->representative != FASTAR_REP_MEDOID)
    return fail(FASTAR_ERR_UNSUPPORTED, "representative %d unknown", o->representative);
  m->rep = o->representative;
  if (o->match_queries) {
    if (o->match != FASTAR_MATCH_QUANT)
      return fail(FASTAR_ERR_UNSUPPORTED, "query-driven matching needs FASTAR_MATCH_QUANT");
    m->q = o->match_queries;
  }
  return FASTAR_OK;
}

size_t merge_workspace_ex(const fastar_cache_t* c, int n_frames, const fastar_merge_opts_t* o) {
  MergeOpt m;
  if (merge_opts(o, &m) != FASTAR_OK) return 0;
  const size_t base = merge_workspace(c, n_frames);
  if (m.match != FASTAR_MATCH_QUANT || base == 0) return base;
  return base + fastar::quant_workspace_bytes(c->heads, c->tokens_per_frame, n_frames, c->dim, m.q != nullptr);
}

// the query tensor of query-driven matching against the new keys
fastar_status_t check_match_queries(const MergeOpt& m, const fastar_tensor_t* k_new) {
  if (!m.q) return FASTAR_OK;
  fastar_status_t st = check_tensor(m.q, "match_queries");
  if (st != FASTAR_OK) return st;
  if (m.q->dtype != k_new->dtype || m.q->dim != k_new->dim || m.q->heads != k_new->heads ||
      m.q->tokens != k_new->tokens)
    return fail(FASTAR_ERR_INVALID, "match_queries must have k_new's dtype, heads, tokens and dim");
  return FASTAR_OK;
}

// everything fastar_tempcache_merge checks for a call with n_frames > 0 and
// heads > 0 (ws: at least merge_workspace bytes)
fastar_status_t merge_check(const fastar_cache_t* c, const fastar_tensor_t* k_new,
                            const fastar_tensor_t* v_new, const int32_t* k_new_bucket, int n_frames,
                            float tau, const int32_t* rep_offsets, const int32_t* rep_perm) {
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
  if (c->heads == 0 || n_frames == 0) return FASTAR_OK;
  if (!c->rep_k || !c->v_mean || !c->v_sum || !c->count || !c->log_count || !c->rep_bucket ||
      !c->n_groups || !c->frontier || !c->status || !k_new_bucket)
    return fail(FASTAR_ERR_INVALID, "a cache buffer or k_new_bucket is NULL");
  if (!aligned16(c->rep_k) || !aligned16(c->v_mean) || !aligned16(c->v_sum))
    return fail(FASTAR_ERR_INVALID, "cache rows must be 16-byte aligned");
  return FASTAR_OK;
}

fastar::MergeWs merge_carve(const fastar_cache_t* c, int n_frames, void* ws) {
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
  mw.prop = take(12 * H * F * T);
  mw.mrange = take(16 * H * F * ((T + 63) / 64));
  mw.index_ws = take(16 * H * (size_t)c->capacity);
  return mw;
}

// the key sum that mean and medoid representatives keep
fastar_status_t check_rep(const fastar_cache_t* c, const MergeOpt& m) {
  if (m.rep == FASTAR_REP_LAST) return FASTAR_OK;
  if (!c->k_sum || !aligned16(c->k_sum))
    return fail(FASTAR_ERR_INVALID, "mean and medoid representatives need a 16-byte aligned cache->k_sum");
  return FASTAR_OK;
}

// frame f of a [H][n_frames * T][d] tensor
fastar_tensor_t frame_slice(const fastar_tensor_t& t, int T, int f) {
  fastar_tensor_t r = t;
  const size_t es = t.dtype == FASTAR_BF16 ? 2 : 4;
  r.data = (const char*)t.data + (size_t)f * T * (size_t)t.stride_token * es;
  r.tokens = T;
  return r;
}

// The merge's launches, in stream order.  With the last-key representative
// all frames go at once; mean and medoid representatives change what the
// next frame is matched against, so each frame is merged by its own launch
// sequence (workspace carved for one frame, rows strided as the whole call's;
// the hashing that rides on the match only with the first frame, the
// representatives' index and what rides on it only after the last).
fastar_status_t run_merge(const fastar_cache_t* c, const fastar_tensor_t* k_new, const fastar_tensor_t* v_new,
                          const int32_t* kb, int F, float tau, const MergeOpt& mo, int32_t* group_of_new,
                          int32_t* rep_offsets, int32_t* rep_perm, const fastar::MergeWs& mw, void* ws,
                          fastar_diag_t* diag, hipStream_t stream) {
  const int H = c->heads, T = c->tokens_per_frame;
  if (mo.rep == FASTAR_REP_LAST) {
    if (mo.match == FASTAR_MATCH_QUANT) {
      const fastar::QuantWs q =
          fastar::quant_carve(H, T, F, c->dim, mo.q != nullptr, (char*)ws + merge_workspace(c, F));
      return hip_status(fastar::launch_tempcache_merge_quant(*c, *k_new, *v_new, mo.q, kb, F, tau, mo.bits,
                                                             group_of_new, rep_offsets, rep_perm, mw, q, diag,
                                                             stream),
                        "tempcache_merge (quantized match)");
    }
    return hip_status(fastar::launch_tempcache_merge(*c, *k_new, *v_new, kb, F, tau, group_of_new, rep_offsets,
                                                     rep_perm, mw, diag, stream),
                      "tempcache_merge");
  }
  fastar::MergeWs one = merge_carve(c, 1, ws);
  one.rep = mo.rep;
  one.kb_stride = (int64_t)F * T;
  one.hash_planes = mw.hash_planes;
  one.hash_bits = mw.hash_bits;
  const fastar::QuantWs q1 =
      mo.match == FASTAR_MATCH_QUANT
          ? fastar::quant_carve(H, T, 1, c->dim, mo.q != nullptr, (char*)ws + merge_workspace(c, 1))
          : fastar::QuantWs{};
  for (int f = 0; f < F; ++f) {
    const bool last = f == F - 1;
    fastar::MergeWs wf = one;
    wf.also_hash = f == 0 ? mw.also_hash : nullptr;
    wf.also_index = last ? mw.also_index : nullptr;
    wf.index_after = last ? mw.index_after : nullptr;
    wf.after_match = f == 0 ? mw.after_match : nullptr;
    const fastar_tensor_t kf = frame_slice(*k_new, T, f), vf = frame_slice(*v_new, T, f);
    int32_t* gf = group_of_new ? group_of_new + (int64_t)f * T : nullptr;
    int32_t* ro = last ? rep_offsets : nullptr;
    int32_t* rp = last ? rep_perm : nullptr;
    fastar_status_t st;
    if (mo.match == FASTAR_MATCH_QUANT) {
      fastar_tensor_t qf;
      if (mo.q) qf = frame_slice(*mo.q, T, f);
      st = hip_status(fastar::launch_tempcache_merge_quant(*c, kf, vf, mo.q ? &qf : nullptr, kb + (int64_t)f * T, 1,
                                                           tau, mo.bits, gf, ro, rp, wf, q1, diag, stream),
                      "tempcache_merge (quantized match)");
    } else {
      st = hip_status(fastar::launch_tempcache_merge(*c, kf, vf, kb + (int64_t)f * T, 1, tau, gf, ro, rp, wf,
                                                     diag, stream),
                      "tempcache_merge");
    }
    if (st != FASTAR_OK) return st;
  }
  return FASTAR_OK;
}

fastar_status_t prune_check(const int32_t* q_bucket, int heads, int64_t n_q, int n_probes,
                            const int32_t* p_bucket, int64_t n_prompt, int n_bits,
                            const uint8_t* keep, const int32_t* kept_idx, const int32_t* n_kept) {
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
  return FASTAR_OK;
}

// checks a bucket-attention call and fills its launch arguments; *empty: no
// query rows (nothing to launch)
fastar_status_t attention_check(const fastar_tensor_t* q, const int32_t* q_bucket,
                                const int32_t* q_perm, int n_probes, const fastar_tensor_t* k,
                                const fastar_tensor_t* v, const float* key_bias,
                                const int32_t* k_offsets, const int32_t* k_perm, int n_bits,
                                const int32_t* key_list, const int32_t* n_key_list, float scale,
                                void* out, float* lse, fastar::AttnArgs* a, bool* empty) {
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
    mode = n_probes > 2 ? 3 : 0;  // more probes: the general (table, probe) mode
  } else if (key_list) {
    if (!n_key_list) return fail(FASTAR_ERR_INVALID, "list mode needs key_list and n_key_list");
    mode = 1;
  } else {
    mode = 2;  // dense: all keys, or with n_key_list a head's first n_key_list[h]
  }
  *empty = (int64_t)q->heads * q->tokens == 0;
  if (*empty) return FASTAR_OK;
  if (!out || !aligned16(out)) return fail(FASTAR_ERR_INVALID, "out must be a non-null 16-byte aligned pointer");
  if ((mode == 0 || mode == 3) && (!q_bucket || !q_perm))
    return fail(FASTAR_ERR_INVALID, "bucket mode needs q_bucket and q_perm");
  if (mode == 3 && (int64_t)q->heads * k->tokens >= (int64_t)1 << 31)
    return fail(FASTAR_ERR_UNSUPPORTED, "heads * keys must be < 2^31");
  if (q->dtype == FASTAR_BF16 && k->tokens > 0) {
    // the bf16 kernel addresses a head's k and v rows by 32-bit byte offsets
    const int64_t span_k = ((int64_t)(k->tokens - 1) * k->stride_token + k->dim) * 2;
    const int64_t span_v = ((int64_t)(v->tokens - 1) * v->stride_token + v->dim) * 2;
    if (span_k > 0xFFFFFFFFll || span_v > 0xFFFFFFFFll)
      return fail(FASTAR_ERR_UNSUPPORTED, "a head's k or v rows span more than 4 GiB");
  }
  a->q = q->data; a->q_sh = q->stride_head; a->q_st = q->stride_token; a->nq = q->tokens;
  a->q_bucket = q_bucket; a->q_perm = q_perm; a->n_probes = (mode == 0 || mode == 3) ? n_probes : 1;
  a->n_tables = 1; a->k_bucket = nullptr; a->n_attended = nullptr;
  a->k = k->data; a->k_sh = k->stride_head; a->k_st = k->stride_token;
  a->v = v->data; a->v_sh = v->stride_head; a->v_st = v->stride_token; a->nk = k->tokens;
  a->key_bias = key_bias; a->k_offsets = k_offsets; a->k_perm = k_perm; a->n_bits = n_bits;
  a->key_list = key_list; a->n_key_list = n_key_list;
  a->scale = scale; a->out = out; a->lse = lse;
  a->heads = q->heads; a->dim = q->dim; a->dtype = q->dtype; a->mode = mode;
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
    case FASTAR_ERR_CAPACITY: return "cache capacity exceeded";
    default: return "unknown status";
  }
}

const char* fastar_last_error(void) { return g_err; }

int fastar_version(void) { return 200; }

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
  fastar::HashJobs jobs;
  bool any;
  const fastar_status_t st = hash_multi_check(count, x, n_probes, bucket, planes, n_bits, &jobs, &any);
  if (st != FASTAR_OK || !any) return st;
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
  return merge_workspace(c, n_frames);
}

size_t fastar_tempcache_workspace_ex(const fastar_cache_t* c, int n_frames, const fastar_merge_opts_t* opts) {
  return merge_workspace_ex(c, n_frames, opts);
}

fastar_status_t fastar_tempcache_merge_ex(const fastar_cache_t* c, const fastar_tensor_t* k_new,
                                          const fastar_tensor_t* v_new, const int32_t* k_new_bucket,
                                          int n_frames, float tau, const fastar_merge_opts_t* opts,
                                          int32_t* group_of_new, int32_t* rep_offsets, int32_t* rep_perm,
                                          void* ws, size_t ws_bytes, fastar_diag_t* diag, hipStream_t stream) {
  MergeOpt mo;
  fastar_status_t st = merge_opts(opts, &mo);
  if (st != FASTAR_OK) return st;
  if ((st = merge_check(c, k_new, v_new, k_new_bucket, n_frames, tau, rep_offsets, rep_perm)) != FASTAR_OK)
    return st;
  if ((st = check_match_queries(mo, k_new)) != FASTAR_OK) return st;
  const size_t need = merge_workspace_ex(c, n_frames, opts);
  if (c->heads == 0 || n_frames == 0) {
    if (rep_offsets && c->heads > 0) {
      if (!ws || ws_bytes < need) return fail(FASTAR_ERR_WORKSPACE, "workspace too small");
      const size_t off = merge_workspace(c, n_frames) - align_up(16 * (size_t)c->heads * (size_t)c->capacity);
      return hip_status(fastar::launch_bucket_index(c->rep_bucket, c->heads, c->capacity, 1, c->n_bits,
                                                    c->n_groups, rep_offsets, rep_perm,
                                                    (int32_t*)((char*)ws + off), stream),
                        "bucket_index");
    }
    return FASTAR_OK;
  }
  if ((st = check_rep(c, mo)) != FASTAR_OK) return st;
  if (!ws || ws_bytes < need)
    return fail(FASTAR_ERR_WORKSPACE, "workspace: need %zu bytes, got %zu", need, ws_bytes);
  return run_merge(c, k_new, v_new, k_new_bucket, n_frames, tau, mo, group_of_new, rep_offsets, rep_perm,
                   merge_carve(c, n_frames, ws), ws, diag, stream);
}

fastar_status_t fastar_tempcache_merge(const fastar_cache_t* c, const fastar_tensor_t* k_new,
                                       const fastar_tensor_t* v_new, const int32_t* k_new_bucket,
                                       int n_frames, float tau, int32_t* group_of_new,
                                       int32_t* rep_offsets, int32_t* rep_perm, void* ws,
                                       size_t ws_bytes, fastar_diag_t* diag, hipStream_t stream) {
  return fastar_tempcache_merge_ex(c, k_new, v_new, k_new_bucket, n_frames, tau, nullptr, group_of_new,
                                   rep_offsets, rep_perm, ws, ws_bytes, diag, stream);
}

fastar_status_t fastar_scalar_codes(const fastar_tensor_t* x, int bits, int8_t* codes, int32_t* norm2,
                                    hipStream_t stream) {
  fastar_status_t st = check_tensor(x, "x");
  if (st != FASTAR_OK) return st;
  if (bits < 2 || bits > 8) return fail(FASTAR_ERR_UNSUPPORTED, "bits %d not in [2, 8]", bits);
  if ((int64_t)x->heads * x->tokens == 0) return FASTAR_OK;
  if (!codes || !norm2) return fail(FASTAR_ERR_INVALID, "codes and norm2 are required");
  if (((uintptr_t)codes & 7u) != 0) return fail(FASTAR_ERR_INVALID, "codes must be 8-byte aligned");
  return hip_status(fastar::launch_scalar_codes(*x, bits, codes, norm2, stream), "scalar_codes");
}

fastar_status_t fastar_cache_status(const fastar_cache_t* c, int clear, hipStream_t stream) {
  if (!c || !c->status) return fail(FASTAR_ERR_INVALID, "cache or its status word is NULL");
  int32_t word = 0;
  fastar_status_t st = hip_status(hipMemcpyAsync(&word, c->status, sizeof(word), hipMemcpyDeviceToHost, stream),
                                  "cache_status read");
  if (st == FASTAR_OK) st = hip_status(hipStreamSynchronize(stream), "cache_status sync");
  if (st != FASTAR_OK) return st;
  if (clear) {
    static const int32_t kZero = 0;
    st = hip_status(hipMemcpyAsync(c->status, &kZero, sizeof(kZero), hipMemcpyHostToDevice, stream),
                    "cache_status clear");
    if (st == FASTAR_OK) st = hip_status(hipStreamSynchronize(stream), "cache_status sync");
    if (st != FASTAR_OK) return st;
  }
  if (word & FASTAR_CACHE_OVERFLOW)
    return fail(FASTAR_ERR_CAPACITY, "a merge dropped groups: the cache's capacity was exceeded");
  return FASTAR_OK;
}

// ---------------------------------------------------------------------------
fastar_status_t fastar_prune_prompt(const int32_t* q_bucket, int heads, int64_t n_q, int n_probes,
                                    const int32_t* p_bucket, int64_t n_prompt, int n_bits,
                                    uint8_t* keep, int32_t* kept_idx, int32_t* n_kept,
                                    hipStream_t stream) {
  const fastar_status_t st =
      prune_check(q_bucket, heads, n_q, n_probes, p_bucket, n_prompt, n_bits, keep, kept_idx, n_kept);
  if (st != FASTAR_OK || heads == 0) return st;
  return hip_status(fastar::launch_prune(q_bucket, heads, n_q, n_probes, p_bucket, n_prompt, n_bits,
                                         keep, kept_idx, n_kept, stream),
                    "prune_prompt");
}

fastar_status_t fastar_prune_prompt_tables(const int32_t* q_bucket, int n_tables, int heads, int64_t n_q,
                                           int n_probes, const int32_t* p_bucket, int64_t n_prompt, int n_bits,
                                           uint8_t* keep, int32_t* kept_idx, int32_t* n_kept,
                                           hipStream_t stream) {
  if (n_tables < 1 || n_tables > FASTAR_MAX_TABLES)
    return fail(FASTAR_ERR_UNSUPPORTED, "n_tables %d not in [1, %d]", n_tables, FASTAR_MAX_TABLES);
  const fastar_status_t st =
      prune_check(q_bucket, heads, n_q, n_probes, p_bucket, n_prompt, n_bits, keep, kept_idx, n_kept);
  if (st != FASTAR_OK || heads == 0) return st;
  if ((int64_t)n_tables * heads * n_q * n_probes >= (int64_t)1 << 31 ||
      (int64_t)n_tables * heads * n_prompt >= (int64_t)1 << 31)
    return fail(FASTAR_ERR_UNSUPPORTED, "sizes times n_tables must be < 2^31");
  return hip_status(fastar::launch_prune(q_bucket, heads, n_q, n_probes, p_bucket, n_prompt, n_bits,
                                         keep, kept_idx, n_kept, stream, n_tables),
                    "prune_prompt_tables");
}

// ---------------------------------------------------------------------------
fastar_status_t fastar_bucket_attention(const fastar_tensor_t* q, const int32_t* q_bucket,
                                        const int32_t* q_perm, int n_probes,
                                        const fastar_tensor_t* k, const fastar_tensor_t* v,
                                        const float* key_bias, const int32_t* k_offsets,
                                        const int32_t* k_perm, int n_bits,
                                        const int32_t* key_list, const int32_t* n_key_list,
                                        float scale, void* out, float* lse, hipStream_t stream) {
  fastar::AttnArgs a;
  bool empty;
  const fastar_status_t st = attention_check(q, q_bucket, q_perm, n_probes, k, v, key_bias, k_offsets,
                                             k_perm, n_bits, key_list, n_key_list, scale, out, lse, &a,
                                             &empty);
  if (st != FASTAR_OK || empty) return st;
  return hip_status(fastar::launch_attention(a, stream), "bucket_attention");
}

fastar_status_t fastar_bucket_attention_tables(const fastar_tensor_t* q, int n_tables, const int32_t* q_bucket,
                                               const int32_t* q_perm, int n_probes, const fastar_tensor_t* k,
                                               const fastar_tensor_t* v, const float* key_bias,
                                               const int32_t* k_bucket, const int32_t* k_offsets,
                                               const int32_t* k_perm, int n_bits, float scale, void* out,
                                               float* lse, int32_t* n_attended, hipStream_t stream) {
  if (n_tables < 1 || n_tables > FASTAR_MAX_TABLES)
    return fail(FASTAR_ERR_UNSUPPORTED, "n_tables %d not in [1, %d]", n_tables, FASTAR_MAX_TABLES);
  if (n_probes < 1 || n_tables * n_probes > FASTAR_MAX_PROBES)
    return fail(FASTAR_ERR_UNSUPPORTED, "n_tables * n_probes must be in [1, %d]", FASTAR_MAX_PROBES);
  if (!k_offsets || !k_perm) return fail(FASTAR_ERR_INVALID, "k_offsets and k_perm are required");
  if (n_tables > 1 && !k_bucket) return fail(FASTAR_ERR_INVALID, "k_bucket is required with several tables");
  fastar::AttnArgs a;
  bool empty;
  fastar_status_t st = attention_check(q, q_bucket, q_perm, n_probes, k, v, key_bias, k_offsets, k_perm, n_bits,
                                       nullptr, nullptr, scale, out, lse, &a, &empty);
  if (st != FASTAR_OK || empty) return st;
  if ((int64_t)n_tables * q->heads * k->tokens >= (int64_t)1 << 31)
    return fail(FASTAR_ERR_UNSUPPORTED, "n_tables * heads * keys must be < 2^31");
  a.mode = 3;
  a.n_tables = n_tables;
  a.k_bucket = k_bucket;
  a.n_attended = n_attended;
  return hip_status(fastar::launch_attention(a, stream), "bucket_attention_tables");
}

// ---------------------------------------------------------------------------
fastar_status_t fastar_attention_recall(const float* lse_sparse, const float* lse_dense, int heads,
                                        int64_t n_q, const int32_t* q_bucket, int n_probes,
                                        const int32_t* k_offsets, int n_bits,
                                        const int32_t* n_retained, const int32_t* n_keys,
                                        float* recall, float* stats, hipStream_t stream) {
  if (heads < 0 || n_q < 0) return fail(FASTAR_ERR_INVALID, "negative size");
  if ((int64_t)heads * n_q >= (int64_t)1 << 31) return fail(FASTAR_ERR_UNSUPPORTED, "heads*n_q must be < 2^31");
  if (heads == 0) return FASTAR_OK;
  if (!stats || !n_keys) return fail(FASTAR_ERR_INVALID, "stats and n_keys are required");
  const bool bucket = k_offsets != nullptr;
  if (bucket) {
    fastar_status_t st = check_bits(n_bits, n_probes);
    if (st != FASTAR_OK) return st;
    if (n_q > 0 && !q_bucket) return fail(FASTAR_ERR_INVALID, "bucket mode needs q_bucket");
    if (n_retained) return fail(FASTAR_ERR_INVALID, "give either k_offsets or n_retained");
  } else if (!n_retained) {
    return fail(FASTAR_ERR_INVALID, "give k_offsets (bucket mode) or n_retained (list mode)");
  }
  if (n_q > 0 && (!lse_sparse || !lse_dense)) return fail(FASTAR_ERR_INVALID, "lse arrays are NULL");
  return hip_status(fastar::launch_recall(lse_sparse, lse_dense, heads, n_q, bucket ? q_bucket : nullptr,
                                          n_probes, k_offsets, n_bits, n_retained, n_keys, recall, stats,
                                          stream),
                    "attention_recall");
}

fastar_status_t fastar_attention_recall_counts(const float* lse_sparse, const float* lse_dense, int heads,
                                               int64_t n_q, const int32_t* n_attended, const int32_t* n_keys,
                                               float* recall, float* stats, hipStream_t stream) {
  if (heads < 0 || n_q < 0) return fail(FASTAR_ERR_INVALID, "negative size");
  if ((int64_t)heads * n_q >= (int64_t)1 << 31) return fail(FASTAR_ERR_UNSUPPORTED, "heads*n_q must be < 2^31");
  if (heads == 0) return FASTAR_OK;
  if (!stats || !n_keys) return fail(FASTAR_ERR_INVALID, "stats and n_keys are required");
  if (n_q > 0 && (!lse_sparse || !lse_dense || !n_attended))
    return fail(FASTAR_ERR_INVALID, "lse arrays and n_attended are required");
  return hip_status(fastar::launch_recall(lse_sparse, lse_dense, heads, n_q, nullptr, 1, nullptr, 0, nullptr,
                                          n_keys, recall, stats, stream, n_attended),
                    "attention_recall_counts");
}

}  // extern "C"

// ---------------------------------------------------------------------------
namespace {
// the cache's representatives and mean values as [H][capacity][dim] tensors
fastar_tensor_t cache_rows(const fastar_cache_t* c, void* data) {
  fastar_tensor_t t;
  t.data = data;
  t.dtype = c->dtype;
  t.heads = c->heads;
  t.tokens = c->capacity;
  t.dim = c->dim;
  t.reserved = 0;
  t.stride_head = (int64_t)c->capacity * c->dim;
  t.stride_token = c->dim;
  return t;
}
// The chunk's second branch: a stream of the library's per device (default
// priority, non-blocking) and the events that fork it from and join it to
// the caller's stream.  Created on the first chunk call of the device that
// is not under stream capture; a call that finds none runs on one stream.
struct AuxBranch {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, q_done = nullptr, done = nullptr;
};
constexpr int kAuxDevices = 64;
std::mutex g_aux_mutex;
AuxBranch g_aux[kAuxDevices];
bool g_aux_failed[kAuxDevices] = {};

bool aux_branch(hipStream_t stream, AuxBranch* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kAuxDevices) return false;
  std::lock_guard<std::mutex> lock(g_aux_mutex);
  AuxBranch& b = g_aux[dev];
  if (!b.s) {
    if (g_aux_failed[dev]) return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
    AuxBranch n;
    if (hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&n.q_done, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&n.done, hipEventDisableTiming) != hipSuccess) {
      g_aux_failed[dev] = true;  // (what was created stays: this is rare and once)
      return false;
    }
    b = n;
  }
  *out = b;
  return true;
}

size_t chunk_index_ws(const fastar_chunk_t* a) {
  // the queries' index in a launch of its own needs scratch
  if (fastar::direct_index_supported(a->q->tokens, a->n_probes, a->n_bits)) return 0;
  return align_up(16 * (size_t)a->q->heads * (size_t)a->q->tokens);
}
}  // namespace

extern "C" {

size_t fastar_chunk_workspace(const fastar_chunk_t* a) {
  if (!a || !a->cache || !a->q) return 0;
  return merge_workspace_ex(a->cache, a->n_frames, a->merge_opts) + chunk_index_ws(a);
}

fastar_status_t fastar_chunk(const fastar_chunk_t* a, void* ws, size_t ws_bytes, fastar_diag_t* diag,
                             hipStream_t stream) {
  if (!a) return fail(FASTAR_ERR_INVALID, "arguments are NULL");
  const fastar_cache_t* c = a->cache;
  if (!c || !a->q || !a->k_new || !a->v_new) return fail(FASTAR_ERR_INVALID, "cache, q, k_new and v_new are required");
  const bool prompt = a->prompt_k != nullptr;
  if (prompt != (a->prompt_v != nullptr)) return fail(FASTAR_ERR_INVALID, "prompt_k and prompt_v go together");
  if (a->q->heads != c->heads) return fail(FASTAR_ERR_INVALID, "q and the cache must share one head count");
  if (a->n_frames <= 0) return fail(FASTAR_ERR_INVALID, "n_frames must be > 0");
  if (!a->q_offsets || !a->q_perm || !a->rep_offsets || !a->rep_perm)
    return fail(FASTAR_ERR_INVALID, "q_offsets, q_perm, rep_offsets and rep_perm are required");
  fastar_status_t st;
  // 1. one hashing: queries, new keys, prompt keys
  const fastar_tensor_t* xs[3] = {a->q, a->k_new, a->prompt_k};
  const int probes[3] = {a->n_probes, 1, 1};
  int32_t* outs[3] = {a->q_bucket, a->k_bucket, a->p_bucket};
  fastar::HashJobs jobs;
  bool any;
  if ((st = hash_multi_check(prompt ? 3 : 2, xs, probes, outs, a->planes, a->n_bits, &jobs, &any)) != FASTAR_OK)
    return st;
  if (a->q->tokens > 0 && !a->q_bucket) return fail(FASTAR_ERR_INVALID, "q_bucket is NULL");
  // 2. the merge (and the queries' index)
  if (c->n_bits != a->n_bits) return fail(FASTAR_ERR_INVALID, "the cache's n_bits differs from n_bits");
  MergeOpt mo;
  if ((st = merge_opts(a->merge_opts, &mo)) != FASTAR_OK) return st;
  if ((st = check_match_queries(mo, a->k_new)) != FASTAR_OK) return st;
  if ((st = check_rep(c, mo)) != FASTAR_OK) return st;
  const int match = mo.match;
  if ((st = merge_check(c, a->k_new, a->v_new, a->k_bucket, a->n_frames, a->tau, a->rep_offsets,
                        a->rep_perm)) != FASTAR_OK)
    return st;
  if ((int64_t)a->q->heads * a->q->tokens * a->n_probes >= (int64_t)1 << 31)
    return fail(FASTAR_ERR_UNSUPPORTED, "heads*tokens*n_probes must be < 2^31");
  // 3. self-attention over the merged cache
  const fastar_tensor_t rk = cache_rows(c, c->rep_k), vm = cache_rows(c, c->v_mean);
  fastar::AttnArgs self, cross;
  bool self_empty, cross_empty = true;
  if ((st = attention_check(a->q, a->q_bucket, a->q_perm, a->n_probes, &rk, &vm, c->log_count,
                            a->rep_offsets, a->rep_perm, a->n_bits, nullptr, nullptr, a->scale, a->out,
                            a->lse, &self, &self_empty)) != FASTAR_OK)
    return st;
  // 4. AnnCA over the prompt
  if (prompt) {
    if (a->prompt_k->heads != c->heads) return fail(FASTAR_ERR_INVALID, "prompt and cache head counts differ");
    if ((st = prune_check(a->q_bucket, a->q->heads, a->q->tokens, a->n_probes, a->p_bucket,
                          a->prompt_k->tokens, a->n_bits, a->keep, a->kept_idx, a->n_kept)) != FASTAR_OK)
      return st;
    if ((st = attention_check(a->q, nullptr, nullptr, 1, a->prompt_k, a->prompt_v, nullptr, nullptr,
                              nullptr, a->n_bits, a->kept_idx, a->n_kept, a->scale, a->out_cross,
                              a->lse_cross, &cross, &cross_empty)) != FASTAR_OK)
      return st;
  }
  const size_t need = fastar_chunk_workspace(a);
  if (!ws || ws_bytes < need)
    return fail(FASTAR_ERR_WORKSPACE, "workspace: need %zu bytes, got %zu", need, ws_bytes);

  fastar::IndexJob qj{a->q_bucket, a->q->tokens, a->n_bits, a->n_probes, a->q_offsets, a->q_perm};
  // the queries' index rides along with the representatives' when both are
  // built by the single counting pass
  const bool fused = a->q->tokens > 0 &&
                     fastar::direct_index_supported(c->capacity, 1, c->n_bits, a->q->tokens, a->n_probes);
  fastar::MergeWs mw = merge_carve(c, a->n_frames, ws);
  if (fused) mw.also_index = &qj;
  // bf16 queries with the LSH match and at most two probes are hashed by
  // extra workgroups of the merge's match launch (only their index, after
  // the merge, and the attention need them)
  const bool ride = match == FASTAR_MATCH_LSH && a->q->dtype == FASTAR_BF16 && c->dtype == FASTAR_BF16 &&
                    a->q->dim == c->dim && a->n_probes <= 2 && c->heads > 0 &&
                    (int64_t)a->q->heads * a->q->tokens > 0;
  AuxBranch ab;
  if (c->heads > 0 && (int64_t)a->q->heads * a->q->tokens > 0 && (prompt || !ride) && aux_branch(stream, &ab)) {
    // Two branches.  The library's second stream prunes the prompt and runs
    // the cross-attention (neither touches the cache), and hashes the
    // queries when they do not ride on the match; the caller's stream hashes
    // the new keys (and with riding queries the prompt keys), merges them,
    // indexes the queries with the representatives, runs the
    // self-attention and joins the second branch.
    fastar::HashJobs side, mainj;
    side.count = mainj.count = 0;
    fastar::HashJobs qjobs;
    qjobs.count = 0;
    if (ride) {
      qjobs.count = 1;
      qjobs.j[0] = jobs.j[0];
      mw.also_hash = &qjobs;
      mw.hash_planes = a->planes;
      mw.hash_bits = a->n_bits;
      mw.after_match = ab.q_done;
      for (int i = 1; i < jobs.count; ++i) mainj.j[mainj.count++] = jobs.j[i];
    } else {
      side.j[side.count++] = jobs.j[0];
      if (prompt) side.j[side.count++] = jobs.j[2];
      mainj.j[mainj.count++] = jobs.j[1];
      mw.index_after = ab.q_done;
    }
    bool main_any = false;
    for (int i = 0; i < mainj.count; ++i) main_any = main_any || (int64_t)mainj.j[i].H * mainj.j[i].N > 0;
    if (main_any && (st = hip_status(fastar::launch_hash_multi(mainj, a->q->dim, a->q->dtype, a->planes, a->n_bits,
                                                               diag, stream),
                                     "hash")) != FASTAR_OK)
      return st;
    if (!ride) {
      if ((st = hip_status(hipEventRecord(ab.fork, stream), "hipEventRecord")) != FASTAR_OK) return st;
      if ((st = hip_status(hipStreamWaitEvent(ab.s, ab.fork, 0), "hipStreamWaitEvent")) != FASTAR_OK) return st;
      if ((st = hip_status(fastar::launch_hash_multi(side, a->q->dim, a->q->dtype, a->planes, a->n_bits, diag,
                                                     ab.s),
                           "hash")) != FASTAR_OK)
        return st;
      if ((st = hip_status(hipEventRecord(ab.q_done, ab.s), "hipEventRecord")) != FASTAR_OK) return st;
    }
    // the merge: with riding queries it records q_done right after its match
    // launch, and the second branch starts from there
    const bool side_first = !ride;
    if (side_first && prompt) {
      if ((st = hip_status(fastar::launch_prune(a->q_bucket, a->q->heads, a->q->tokens, a->n_probes, a->p_bucket,
                                                a->prompt_k->tokens, a->n_bits, a->keep, a->kept_idx, a->n_kept,
                                                ab.s),
                           "prune_prompt")) != FASTAR_OK)
        return st;
      if (!cross_empty &&
          (st = hip_status(fastar::launch_attention(cross, ab.s), "bucket_attention")) != FASTAR_OK)
        return st;
    }
    if (side_first && (st = hip_status(hipEventRecord(ab.done, ab.s), "hipEventRecord")) != FASTAR_OK) return st;
    if ((st = run_merge(c, a->k_new, a->v_new, a->k_bucket, a->n_frames, a->tau, mo, a->group_of_new,
                        a->rep_offsets, a->rep_perm, mw, ws, diag, stream)) != FASTAR_OK)
      return st;
    if (ride) {
      // the queries and prompt keys are hashed: prune and cross-attention
      if ((st = hip_status(hipStreamWaitEvent(ab.s, ab.q_done, 0), "hipStreamWaitEvent")) != FASTAR_OK) return st;
      if ((st = hip_status(fastar::launch_prune(a->q_bucket, a->q->heads, a->q->tokens, a->n_probes, a->p_bucket,
                                                a->prompt_k->tokens, a->n_bits, a->keep, a->kept_idx, a->n_kept,
                                                ab.s),
                           "prune_prompt")) != FASTAR_OK)
        return st;
      if (!cross_empty &&
          (st = hip_status(fastar::launch_attention(cross, ab.s), "bucket_attention")) != FASTAR_OK)
        return st;
      if ((st = hip_status(hipEventRecord(ab.done, ab.s), "hipEventRecord")) != FASTAR_OK) return st;
    }
    if (!fused) {
      if (!ride &&
          (st = hip_status(hipStreamWaitEvent(stream, ab.q_done, 0), "hipStreamWaitEvent")) != FASTAR_OK)
        return st;
      int32_t* iws = (int32_t*)((char*)ws + merge_workspace_ex(c, a->n_frames, a->merge_opts));
      if ((st = hip_status(fastar::launch_bucket_index(a->q_bucket, a->q->heads, a->q->tokens, a->n_probes,
                                                       a->n_bits, nullptr, a->q_offsets, a->q_perm, iws,
                                                       stream),
                           "bucket_index")) != FASTAR_OK)
        return st;
    }
    if (!self_empty &&
        (st = hip_status(fastar::launch_attention(self, stream), "bucket_attention")) != FASTAR_OK)
      return st;
    return hip_status(hipStreamWaitEvent(stream, ab.done, 0), "hipStreamWaitEvent");
  }

  // One stream (the second branch unavailable): launches in order.  bf16
  // queries with at most two probes are hashed by extra workgroups of the
  // merge's match launch (only their index, after the merge, and the
  // attention need them); the keys first, on their own.
  fastar::HashJobs qjobs;
  qjobs.count = 0;
  if (match == FASTAR_MATCH_LSH && a->q->dtype == FASTAR_BF16 && c->dtype == FASTAR_BF16 &&
      a->q->dim == c->dim && a->n_probes <= 2 && c->heads > 0 && (int64_t)a->q->heads * a->q->tokens > 0) {
    qjobs.count = 1;
    qjobs.j[0] = jobs.j[0];
    for (int i = 1; i < jobs.count; ++i) jobs.j[i - 1] = jobs.j[i];
    --jobs.count;
    mw.also_hash = &qjobs;
    mw.hash_planes = a->planes;
    mw.hash_bits = a->n_bits;
  }
  any = false;
  for (int i = 0; i < jobs.count; ++i) any = any || (int64_t)jobs.j[i].H * jobs.j[i].N > 0;
  if (any && (st = hip_status(fastar::launch_hash_multi(jobs, a->q->dim, a->q->dtype, a->planes, a->n_bits,
                                                       diag, stream), "hash")) != FASTAR_OK)
    return st;
  if ((st = run_merge(c, a->k_new, a->v_new, a->k_bucket, a->n_frames, a->tau, mo, a->group_of_new,
                      a->rep_offsets, a->rep_perm, mw, ws, diag, stream)) != FASTAR_OK)
    return st;
  if (!fused) {
    int32_t* iws = (int32_t*)((char*)ws + merge_workspace_ex(c, a->n_frames, a->merge_opts));
    if ((st = hip_status(fastar::launch_bucket_index(a->q_bucket, a->q->heads, a->q->tokens, a->n_probes,
                                                     a->n_bits, nullptr, a->q_offsets, a->q_perm, iws,
                                                     stream),
                         "bucket_index")) != FASTAR_OK)
      return st;
  }
  if (!self_empty &&
      (st = hip_status(fastar::launch_attention(self, stream), "bucket_attention")) != FASTAR_OK)
    return st;
  if (prompt) {
    if (c->heads > 0 &&
        (st = hip_status(fastar::launch_prune(a->q_bucket, a->q->heads, a->q->tokens, a->n_probes, a->p_bucket,
                                              a->prompt_k->tokens, a->n_bits, a->keep, a->kept_idx,
                                              a->n_kept, stream),
                         "prune_prompt")) != FASTAR_OK)
      return st;
    if (!cross_empty &&
        (st = hip_status(fastar::launch_attention(cross, stream), "bucket_attention")) != FASTAR_OK)
      return st;
  }
  return FASTAR_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

// the current device's scratch address, looked up once per device with that
// device current
fastar_status_t noalloc_scratch(void** ptr) {
  int dev = -1;
  fastar_status_t st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != FASTAR_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(FASTAR_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != FASTAR_OK) return st;
    if (!p) return fail(FASTAR_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return FASTAR_OK;
}
}  // namespace

extern "C" {

fastar_status_t fastar_chunk_noalloc(const fastar_chunk_t* a, fastar_diag_t* diag, hipStream_t stream) {
  if (!a || !a->cache || !a->q) return fail(FASTAR_ERR_INVALID, "arguments, cache and q are required");
  const size_t need = fastar_chunk_workspace(a);
  if (need > FASTAR_NOALLOC_SCRATCH_BYTES)
    return fail(FASTAR_ERR_WORKSPACE, "the call needs %zu bytes of workspace, more than the %zu bytes "
                "of the allocation-free scratch", need, (size_t)FASTAR_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const fastar_status_t st = noalloc_scratch(&ws);
  if (st != FASTAR_OK) return st;
  return fastar_chunk(a, ws, FASTAR_NOALLOC_SCRATCH_BYTES, diag, stream);
}

}  // extern "C"

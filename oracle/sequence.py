"""One layer's per-chunk call sequence (oracle).

Per chunk of new frames (paper.rainbus.top technical novelty: one hashing
serves TempCache, AnnCA and AnnSA; paperlayer.ai section 3: self-attention
keys are the current frames plus the cached earlier frames):

1. hash the chunk's queries (one or two probes) and the new frames' keys;
2. merge the new frames into the compressed cache, frame by frame (TempCache);
3. hash the prompt keys and prune the prompt against the queries' buckets
   (AnnCA);
4. self-attention of the queries over the whole compressed cache, restricted
   to their buckets, with the + ln m bias (AnnSA);
5. cross-attention of the queries over the kept prompt tokens.

Reading: merging happens every frame, in order, before attention; frames
before the measured chunk are merged the same way as set-up.

Variants:
* several LSH tables (paperlayer.ai section 2: hash-based retrieval probing
  several tables): table 0 is the hashing above; each further table hashes
  the queries and prompt keys with its own planes, and the representatives
  themselves (TempCache's match stays on table 0); AnnSA runs over the union
  of the tables' buckets and AnnCA keeps a prompt token any table keeps;
* the denoising warm-up (paper.rainbus.top limitations: the sparse attention
  is off in the first 30% of the denoising steps): the same merge, then dense
  self-attention over every group (with the + ln m bias) and dense
  cross-attention over the whole prompt.
"""

from __future__ import annotations

import numpy as np

from .simhash import simhash
from .index import bucket_index
from .tempcache import TempCacheOracle
from .tempcache_quant import TempCacheQuantOracle
from .annca import prune_prompt, cross_attention
from .attention import bucket_attention, dense_attention
from .multitable import bucket_attention_tables, prune_prompt_tables


def run_chunk(w, heads=None, attention=True, match="lsh", code_bits=8, query_driven=False,
              representative="last", extra_planes=None, sparse=True):
    """Run the sequence for workload-like object ``w`` on the given heads.

    ``w`` provides dtype, dim, n_bits, n_probes, tau, planes [b, d], q [H, N, d],
    and optionally k_frames/v_frames [H, F, T, d] with setup_frames, and
    prompt_k/prompt_v [H, Np, d].  ``match``: TempCache's LSH match ("lsh") or
    its quantized match ("quant", ``code_bits`` bits; ``query_driven``: the
    chunk's frames are matched by their queries, ``w.q`` being the chunk
    frames' tokens).  ``representative``: TempCache's group representative
    ("last", "mean" or "medoid").  ``extra_planes`` [L - 1, b, d]: the planes
    of further LSH tables.  ``sparse=False``: the warm-up step (dense
    attention).  Returns a dict of per-head result dicts.
    """
    heads = range(w.heads) if heads is None else heads
    scale = 1.0 / np.sqrt(w.dim)
    res = {}
    for h in heads:
        r = {}
        q = np.asarray(w.q[h], dtype=np.float64)
        r["q_ids"] = simhash(q, w.planes, w.n_probes)
        r["q_offsets"], r["q_perm"] = bucket_index(r["q_ids"], w.n_bits)
        if w.k_frames is not None:
            tc = (TempCacheQuantOracle(w.dim, w.dtype, code_bits, representative) if match == "quant"
                  else TempCacheOracle(w.dim, w.dtype, representative))
            F = w.k_frames.shape[1]
            groups = []
            setup_groups = []
            k_ids = []
            for f in range(F):
                kf = np.asarray(w.k_frames[h, f], dtype=np.float64)
                ids = simhash(kf, w.planes, 1)[:, 0]
                if f >= w.setup_frames:
                    k_ids.append(ids)
                if f == w.setup_frames:
                    r["n_groups_before"] = tc.n_groups
                if query_driven and f >= w.setup_frames:
                    T = w.k_frames.shape[2]
                    qf = np.asarray(w.q[h, (f - w.setup_frames) * T:(f - w.setup_frames + 1) * T],
                                    dtype=np.float64)
                    g = tc.merge_frame(kf, w.v_frames[h, f], ids, w.tau, match_vec=qf)
                else:
                    g = tc.merge_frame(kf, w.v_frames[h, f], ids, w.tau)
                (groups if f >= w.setup_frames else setup_groups).append(g)
            r["k_ids"] = np.concatenate(k_ids) if k_ids else np.zeros(0, np.int64)
            r["group_of_new"] = np.concatenate(groups) if groups else np.zeros(0, np.int64)
            r["setup_groups"] = (np.concatenate(setup_groups) if setup_groups
                                 else np.zeros(0, np.int64))
            r["cache"] = tc
            r["rep_offsets"], r["rep_perm"] = bucket_index(tc.rep_bucket, w.n_bits)
            if attention and not sparse:
                r["o_self"], r["lse_self"] = dense_attention(q, tc.rep_k, tc.v_mean, scale=scale,
                                                             bias=tc.log_count)
            elif attention and extra_planes is not None:
                r["q_ids_t"] = np.stack([r["q_ids"]] + [simhash(q, pl, w.n_probes) for pl in extra_planes])
                r["rep_ids_t"] = np.stack([tc.rep_bucket] + [simhash(tc.rep_k, pl, 1)[:, 0]
                                                             for pl in extra_planes])
                r["o_self"], r["lse_self"], r["n_attended"] = bucket_attention_tables(
                    q, r["q_ids_t"], tc.rep_k, tc.v_mean, r["rep_ids_t"], bias=tc.log_count, scale=scale)
            elif attention:
                r["o_self"], r["lse_self"] = bucket_attention(
                    q, r["q_ids"], tc.rep_k, tc.v_mean, tc.rep_bucket,
                    bias=tc.log_count, scale=scale)
        if w.prompt_k is not None:
            pk = np.asarray(w.prompt_k[h], dtype=np.float64)
            r["p_ids"] = simhash(pk, w.planes, 1)[:, 0]
            if not sparse:
                r["keep"], r["kept_idx"] = np.ones(len(pk), bool), np.arange(len(pk))
            elif extra_planes is not None:
                q_ids_t = np.stack([r["q_ids"]] + [simhash(q, pl, w.n_probes) for pl in extra_planes])
                p_ids_t = np.stack([r["p_ids"]] + [simhash(pk, pl, 1)[:, 0] for pl in extra_planes])
                r["keep"], r["kept_idx"] = prune_prompt_tables(q_ids_t, p_ids_t)
            else:
                r["keep"], r["kept_idx"] = prune_prompt(r["q_ids"], r["p_ids"])
            if attention:
                r["o_cross"], r["lse_cross"] = cross_attention(
                    q, pk, w.prompt_v[h], r["kept_idx"], scale)
        res[h] = r
    return res

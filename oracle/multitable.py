"""Multi-table LSH for AnnSA and AnnCA (oracle).

The pages name LSH as hash-based retrieval that probes buckets in several
tables (paperlayer.ai section 2 "Approximate nearest neighbor search"); the
method itself hashes queries and keys with one shared set of hyperplanes
(paper.rainbus.top, technical novelty).  Readings for L tables:
* table u has its own n_bits hyperplanes; every query, cache key and prompt
  key gets one bucket per table (simhash with that table's planes), queries
  n_probes per table (the multi-probe order of oracle.simhash);
* AnnSA: query q retains key j if, in any table u, j's table-u bucket is one
  of q's table-u probes; the attention runs over that union, each key once;
* AnnCA: a prompt token is kept if, in any table u, its table-u bucket is
  one of the table-u probes of any query.
With one table these are exactly the single-table definitions.
"""

from __future__ import annotations

import numpy as np

from .attention import _softmax_rows
from .simhash import simhash


def simhash_tables(x, planes, n_probes: int = 1) -> np.ndarray:
    """ids [L, N, n_probes] of the rows of x [N, d] for planes [L, n_bits, d]."""
    planes = np.asarray(planes, dtype=np.float64)
    return np.stack([simhash(x, planes[u], n_probes) for u in range(planes.shape[0])])


def retained_tables(q_ids, k_bucket) -> np.ndarray:
    """The retained mask [n, m]: q_ids [L, n, P], k_bucket [L, m]."""
    q_ids = np.asarray(q_ids, dtype=np.int64)
    k_bucket = np.asarray(k_bucket, dtype=np.int64)
    L, n, _ = q_ids.shape
    mask = np.zeros((n, k_bucket.shape[1]), dtype=bool)
    for u in range(L):
        mask |= (k_bucket[u][None, :, None] == q_ids[u][:, None, :]).any(axis=2)
    return mask


def bucket_attention_tables(q, q_ids, k, v, k_bucket, bias=None, scale=None):
    """AnnSA over the union of the tables' buckets: o [n, dv], lse [n] and the
    retained count [n] (|A(q)|, each key counted once)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    bias = np.zeros(k.shape[0]) if bias is None else np.asarray(bias, dtype=np.float64)
    mask = retained_tables(q_ids, k_bucket)
    o = np.zeros((q.shape[0], v.shape[1]))
    lse = np.full(q.shape[0], -np.inf)
    for r in range(q.shape[0]):
        keys = np.nonzero(mask[r])[0]
        if keys.size:
            logits = (q[r:r + 1] @ k[keys].T) * scale + bias[keys][None, :]
            o[r:r + 1], lse[r:r + 1] = _softmax_rows(logits, v[keys])
    return o, lse, mask.sum(axis=1)


def prune_prompt_tables(q_ids, p_ids):
    """keep [Np] bool, kept_idx ascending, for q_ids [L, n, P] and prompt
    buckets p_ids [L, Np]."""
    q_ids = np.asarray(q_ids, dtype=np.int64)
    p_ids = np.asarray(p_ids, dtype=np.int64)
    keep = np.zeros(p_ids.shape[1], dtype=bool)
    for u in range(q_ids.shape[0]):
        occupied = set(q_ids[u].reshape(-1).tolist())
        keep |= np.array([b in occupied for b in p_ids[u].tolist()], dtype=bool)
    return keep, np.nonzero(keep)[0].astype(np.int64)

"""Dense and bucket-restricted softmax attention (oracle), float64.

* Dense attention: o_q = sum_j softmax_j(q . k_j * s + bias_j) v_j over the
  whole key set (paperlayer.ai section 3, attention formulation; the cached
  keys are the current frame concatenated with earlier frames).
* AnnSA: each query attends only to keys whose bucket is one of the query's
  bucket(s) (paperlayer.ai section 5 "AnnSA"; gist.science technical summary,
  AnnSA; paper.rainbus.top method steps).
* With a TempCache-compressed cache the logit of group g is shifted by
  ln m_g and its value is the group mean (Lemma 5.1, paperlayer.ai
  appendix A), so the bias is an input here.

Readings: the logit scale s (1/sqrt(d) by default) multiplies q . k before the
bias is added; a query whose key set is empty gets o = 0 and lse = -inf.
"""

from __future__ import annotations

import numpy as np


def _softmax_rows(logits, values):
    """o = softmax(logits) @ values and lse, for logits [n, m], values [m, d]."""
    n = logits.shape[0]
    if logits.shape[1] == 0:
        return np.zeros((n, values.shape[1])), np.full(n, -np.inf)
    mx = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - mx)
    z = w.sum(axis=1, keepdims=True)
    o = (w @ values) / z
    lse = (mx + np.log(z))[:, 0]
    return o, lse


def dense_attention(q, k, v, scale=None, bias=None):
    """Dense softmax attention. q [n, d], k [m, d], v [m, dv], bias [m] or None."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    logits = (q @ k.T) * scale
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return _softmax_rows(logits, v)


def bucket_attention(q, q_ids, k, v, k_bucket, bias=None, scale=None):
    """AnnSA: query q attends to {j : k_bucket[j] in q_ids[q, :]}.

    q [n, d]; q_ids [n, P] bucket ids; k [m, d], v [m, dv]; k_bucket [m];
    bias [m] (ln of group counts for a compressed cache) or None.
    Returns o [n, dv], lse [n].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_ids = np.asarray(q_ids, dtype=np.int64).reshape(q.shape[0], -1)
    k_bucket = np.asarray(k_bucket, dtype=np.int64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    bias = np.zeros(k.shape[0]) if bias is None else np.asarray(bias, dtype=np.float64)
    o = np.zeros((q.shape[0], v.shape[1]))
    lse = np.full(q.shape[0], -np.inf)
    # queries with the same set of probe buckets share one key set
    sets = {}
    for r in range(q.shape[0]):
        sets.setdefault(tuple(sorted(set(q_ids[r].tolist()))), []).append(r)
    for probe_set, rows in sets.items():
        keys = np.nonzero(np.isin(k_bucket, probe_set))[0]
        rows = np.asarray(rows)
        logits = (q[rows] @ k[keys].T) * scale + bias[keys][None, :]
        o[rows], lse[rows] = _softmax_rows(logits, v[keys])
    return o, lse

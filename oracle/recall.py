"""Attention recall and density (oracle), float64.

The pages measure sparsity by attention recall: the dense-attention mass that
the retained entries keep (paperlayer.ai section 4 "Motivation", attention
sparsity; section 3 reports about 85% recall at 30% density; paper.rainbus.top,
figure 2, recall against density).  For a query q with retained key set A(q):

    recall(q)  = sum_{j in A(q)} p_j(q),  p(q) = softmax_j(s q.k_j + bias_j) over all keys
    density(q) = |A(q)| / (number of keys)

AnnSA retains the keys of q's bucket(s); AnnCA the kept prompt tokens; the
pages' reference curve retains the largest attention entries of each row
(top-k), which is the most mass any set of that size can keep.

Readings: the dense attention is taken over the same keys the sparse one
chooses from (for self-attention, the compressed cache with its + ln m bias,
so by Lemma 5.1 a group's mass is that of its merged raw keys); density counts
key-list entries (compressed groups), and a query with an empty retained set
has recall 0.
"""

from __future__ import annotations

import numpy as np


def _probs(q, k, scale=None, bias=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    logits = (q @ k.T) * scale
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], 0))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def attention_recall(q, k, retained, scale=None, bias=None):
    """recall [n], density [n] of the retained masks (bool [n, m]) of q [n, d]
    over keys k [m, d] (with an optional logit bias [m])."""
    p = _probs(q, k, scale, bias)
    retained = np.asarray(retained, dtype=bool)
    m = max(k.shape[0], 1)
    return (p * retained).sum(axis=1), retained.sum(axis=1) / m


def bucket_retained(q_ids, k_bucket):
    """AnnSA's retained mask: key j is retained for q if its bucket is one of
    q's probe buckets."""
    q_ids = np.asarray(q_ids, dtype=np.int64).reshape(len(q_ids), -1)
    kb = np.asarray(k_bucket, dtype=np.int64)
    return (kb[None, :, None] == q_ids[:, None, :]).any(axis=2)


def topk_recall(q, k, density, scale=None, bias=None):
    """The pages' reference: recall [n] when each row keeps its
    ceil(density * m) largest attention entries."""
    p = _probs(q, k, scale, bias)
    m = p.shape[1]
    keep = int(np.ceil(density * m - 1e-12))
    if keep <= 0:
        return np.zeros(p.shape[0])
    return np.sort(p, axis=1)[:, ::-1][:, :keep].sum(axis=1)

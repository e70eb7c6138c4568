"""Bucket-contiguous index (oracle).

Block-sparse attention over buckets needs, per head, the members of each
bucket stored contiguously (gist.science technical summary, AnnSA: attention
restricted to keys of the same bucket(s), run as a block-sparse operation).

Definition used here:
* one probe: members are sorted by bucket id, ties in ascending token order
  (a stable sort); offsets[B] is the number of members with bucket < B, so
  offsets has 2**n_bits + 1 entries and offsets[-1] = N;
* two probes: each query appears once, sorted by (first bucket, flipped bit,
  token), where the flipped bit is the position where its two bucket ids
  differ; offsets still count by first bucket.  Grouping by flipped bit keeps
  queries that share their second bucket together.
"""

from __future__ import annotations

import numpy as np


def _flip_bit(ids):
    x = (ids[:, 0] ^ ids[:, 1]).astype(np.int64)
    # position of the single set bit
    return np.log2(x).astype(np.int64)


def bucket_index(ids, n_bits: int):
    """offsets [2**n_bits + 1] (int64), perm [N] (int64) for ids [N, P]."""
    ids = np.asarray(ids, dtype=np.int64)
    if ids.ndim == 1:
        ids = ids[:, None]
    n, p = ids.shape
    first = ids[:, 0]
    if p == 2 and n:
        key = first * 16 + _flip_bit(ids)
    else:
        key = first
    perm = np.argsort(key, kind="stable")
    counts = np.bincount(first, minlength=1 << n_bits)
    offsets = np.zeros((1 << n_bits) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return offsets, perm.astype(np.int64)

"""Bucket-contiguous index (oracle).

Block-sparse attention over buckets needs, per head, the members of each
bucket stored contiguously (gist.science technical summary, AnnSA: attention
restricted to keys of the same bucket(s), run as a block-sparse operation).

Definition used here:
* members are sorted by bucket id (with several probes, by the smallest of
  the query's probe buckets), ties in ascending token order (a stable sort);
  each query appears once; offsets[B] is the number of members whose (smallest)
  bucket is < B, so offsets has 2**n_bits + 1 entries and offsets[-1] = N.

Reading: the pages only ask that a bucket's members be contiguous for the
block-sparse kernel; with several probes a query's keys come from all of its
buckets, and any grouping key is a valid index.  The smallest probe bucket
is taken: two queries probing the same pair {X, X ^ 2^j} share it whichever
of the two is their own bucket, so they sit side by side.
"""

from __future__ import annotations

import numpy as np


def bucket_index(ids, n_bits: int):
    """offsets [2**n_bits + 1] (int64), perm [N] (int64) for ids [N, P]."""
    ids = np.asarray(ids, dtype=np.int64)
    if ids.ndim == 1:
        ids = ids[:, None]
    key = ids.min(axis=1)
    perm = np.argsort(key, kind="stable")
    counts = np.bincount(key, minlength=1 << n_bits)
    offsets = np.zeros((1 << n_bits) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return offsets, perm.astype(np.int64)

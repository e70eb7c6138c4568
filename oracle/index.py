"""Bucket-contiguous index (oracle).

Block-sparse attention over buckets needs, per head, the members of each
bucket stored contiguously (gist.science technical summary, AnnSA: attention
restricted to keys of the same bucket(s), run as a block-sparse operation).

Definition used here:
* members are sorted by bucket id (with two probes, by the first probe's
  bucket), ties in ascending token order (a stable sort); each query appears
  once; offsets[B] is the number of members with (first) bucket < B, so
  offsets has 2**n_bits + 1 entries and offsets[-1] = N.

Reading: the pages only ask that a bucket's members be contiguous for the
block-sparse kernel; with two probes the query's keys come from both of its
buckets, and the index groups the queries by the first one.
"""

from __future__ import annotations

import numpy as np


def bucket_index(ids, n_bits: int):
    """offsets [2**n_bits + 1] (int64), perm [N] (int64) for ids [N, P]."""
    ids = np.asarray(ids, dtype=np.int64)
    if ids.ndim == 1:
        ids = ids[:, None]
    first = ids[:, 0]
    perm = np.argsort(first, kind="stable")
    counts = np.bincount(first, minlength=1 << n_bits)
    offsets = np.zeros((1 << n_bits) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return offsets, perm.astype(np.int64)

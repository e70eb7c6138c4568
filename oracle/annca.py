"""AnnCA: prompt-token pruning and cross-attention over the kept tokens (oracle).

The pages: queries of the current frame and prompt keys are hashed into one
shared space; a prompt token that shares no bucket with any current-frame
query is dropped for that frame, and cross-attention runs over the rest
(gist.science technical summary, AnnCA mechanism; paper.rainbus.top method
steps, AnnCA; paperlayer.ai section 5 "AnnCA").

Readings: pruning is per head; the occupied set is the union of every probe
bucket of every query; kept indices are ascending; nothing kept gives o = 0.
"""

from __future__ import annotations

import numpy as np

from .attention import dense_attention


def prune_prompt(q_ids, p_ids):
    """keep [Np] bool, kept_idx [n_kept] int64 for query ids [N, P], prompt ids [Np]."""
    q_ids = np.asarray(q_ids, dtype=np.int64)
    p_ids = np.asarray(p_ids, dtype=np.int64).reshape(-1)
    occupied = set(q_ids.reshape(-1).tolist())
    keep = np.array([b in occupied for b in p_ids.tolist()], dtype=bool)
    return keep, np.nonzero(keep)[0].astype(np.int64)


def cross_attention(q, pk, pv, kept_idx, scale=None):
    """Dense attention of q over the kept prompt keys only."""
    kept_idx = np.asarray(kept_idx, dtype=np.int64)
    return dense_attention(q, np.asarray(pk)[kept_idx], np.asarray(pv)[kept_idx], scale)

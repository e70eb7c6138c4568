"""SimHash bucketing (oracle).

Random-hyperplane LSH: a vector's bucket id is the sign pattern of its
projections on the hyperplane normals, so vectors at a small angle tend to
share a bucket (paperlayer.ai, section 2 "Approximate nearest neighbor
search" and section 5 "ANN Attention"; paper.rainbus.top, prerequisites,
"ANN": LSH maps vectors to buckets by random projection).  The same planes hash
queries, cache keys and prompt keys, so one hashing serves TempCache, AnnCA and
AnnSA (paper.rainbus.top, "technical novelty").

Readings where the pages are silent:
* bit j is 1 iff the exact real value of x . r_j is > 0 (exactly 0 gives 0),
  and bit 0 is the least significant bit of the id;
* with two probes ("one or more buckets" per query, paper.rainbus.top method
  steps, AnnSA), the second bucket is the Hamming-1 neighbour across the
  hyperplane nearest to x: flip bit j* = argmin_j |x . r_j| / |r_j|, ties to
  the smaller j;
* with P > 2 probes (multi-probe LSH, the bucket probing of paperlayer.ai
  section 2 "Approximate nearest neighbor search"), probe p >= 1 flips the
  bit of the p-th nearest hyperplane (the same distance, ascending, ties to
  the smaller j): the Hamming-1 neighbours in order of how close x lies to
  their boundary.  P <= n_bits + 1.
"""

from __future__ import annotations

import numpy as np

from .exact import exact_dot, exact_sqnorm

_U64 = 2.0 ** -53


def _exact_signs(x, planes, rows, cols, s):
    for r, c in zip(rows.tolist(), cols.tolist()):
        v = exact_dot(x[r], planes[c])
        s[r, c] = 1.0 if v > 0 else (-1.0 if v < 0 else 0.0)


def simhash(x, planes, n_probes: int = 1) -> np.ndarray:
    """Bucket ids [N, n_probes] (int64) of the rows of x [N, d].

    planes: [n_bits, d] hyperplane normals (rows), n_bits may be 0 (one bucket).
    """
    x = np.asarray(x, dtype=np.float64)
    planes = np.asarray(planes, dtype=np.float64).reshape(-1, x.shape[1])
    n, d = x.shape
    b = planes.shape[0]
    if n_probes < 1 or n_probes > b + 1:
        raise ValueError("n_probes must be in [1, n_bits + 1]")
    ids = np.zeros((n, n_probes), dtype=np.int64)
    if b == 0 or n == 0:
        return ids
    s = x @ planes.T                                   # float64 projections
    # |fl(s) - s| <= gamma_d * sum|x_i r_i|; the bound is inflated by 2 to
    # cover the rounding of the |x| |r| product itself.
    absdot = np.abs(x) @ np.abs(planes).T
    bound = 2.0 * (d + 2) * _U64 * absdot
    sign = np.sign(s)
    amb_r, amb_c = np.nonzero(np.abs(s) <= bound)
    _exact_signs(x, planes, amb_r, amb_c, sign)
    bits = (sign > 0).astype(np.int64)
    ids[:, 0] = (bits << np.arange(b, dtype=np.int64)).sum(axis=1)
    if n_probes == 1:
        return ids
    # distance of x to hyperplane j: |x . r_j| / |r_j|
    rn = np.sqrt(np.sum(planes * planes, axis=1))
    dist = np.abs(s) / rn
    err = bound / rn + dist * (2 * d + 8) * _U64
    lo, hi = dist - err, dist + err
    sqn = None
    k = n_probes - 1                                   # flipped bits wanted
    for r in range(n):
        order = np.argsort(dist[r], kind="stable")     # ascending, ties to the smaller j
        # planes that may be among the k nearest: any whose interval reaches
        # below the upper end of the k-th nearest's
        cand = np.nonzero(lo[r] <= hi[r, order[k - 1]])[0]
        first = order[:k]
        ivl = sorted(zip(lo[r, cand].tolist(), hi[r, cand].tolist()))
        disjoint = all(ivl[i][1] < ivl[i + 1][0] for i in range(len(ivl) - 1))
        if cand.size > k or not disjoint:
            if sqn is None:
                sqn = [exact_sqnorm(planes[j]) for j in range(b)]
            # order them by s_j^2 / |r_j|^2 exactly, ties to the smaller j
            keyed = []
            for j in cand.tolist():
                sj = exact_dot(x[r], planes[j])
                keyed.append((sj * sj / sqn[j], j))
            keyed.sort()
            first = [j for _, j in keyed[:k]]
        for p, j in enumerate(first):
            ids[r, p + 1] = ids[r, 0] ^ (1 << int(j))
    return ids

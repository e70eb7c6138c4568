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
  the smaller j.
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
    if n_probes not in (1, 2):
        raise ValueError("n_probes must be 1 or 2")
    if n_probes == 2 and b == 0:
        raise ValueError("a second probe needs at least one hyperplane")
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
    for r in range(n):
        j0 = int(np.argmin(dist[r]))
        cand = np.nonzero(lo[r] <= hi[r, j0])[0]
        if cand.size > 1:
            if sqn is None:
                sqn = [exact_sqnorm(planes[j]) for j in range(b)]
            # compare s_j^2 / |r_j|^2 exactly; ties go to the smaller j
            best, best_key = None, None
            for j in cand.tolist():
                sj = exact_dot(x[r], planes[j])
                key = sj * sj / sqn[j]
                if best_key is None or key < best_key:
                    best, best_key = j, key
            j0 = best
        ids[r, 1] = ids[r, 0] ^ (1 << j0)
    return ids

"""TempCache: temporal KV-cache compression (oracle), one attention head.

What the pages fix:
* each new key is matched top-1 to a temporally corresponding key with a
  lightweight ANN search (paperlayer.ai section 5 "TempCache"; the Chinese
  summary says the match is searched in the previous frame);
* corresponding keys form a group that keeps only its most recent key as
  representative ("last key"; paperlayer.ai appendix C, representative
  selection);
* a group of m_t positions is attended through one key with the group-mean
  value and logit shifted by + log m_t, which is exact when the keys are
  identical (Lemma 5.1, paperlayer.ai appendix A); in practice keys merge when
  their similarity passes a threshold (paperlayer.ai section 5, appendix C
  threshold ablation 0.9 -> 0.5).

Readings where the pages are silent:
* similarity is the cosine (cos of a zero vector is 0); the threshold test is
  cos >= tau with tau taken as its float32 value;
* candidates for new key j of frame f are the frame f-1 tokens whose bucket id
  equals j's; each of them is the current representative of its group;
* j proposes to its best candidate (largest cosine, ties to the smaller
  candidate index) if that cosine passes the threshold;
* one-to-one: a candidate proposed to by several new keys takes the one with
  the largest cosine (ties to the smaller j); all other new keys start new
  groups, numbered after the existing ones in ascending j;
* a merged group gets count + 1, value sum + v_j, representative key k_j and
  representative bucket b_j; the stored mean value is value sum / count
  rounded once to the storage dtype, the bias is ln(count);
* every decision in a frame uses the cache as it stood after frame f-1.

Representative variants (paperlayer.ai appendix C compares last-key,
mean-key and medoid-key representatives); readings:
* mean: the exact mean of the group's keys, rounded once to the storage
  dtype;
* medoid: kept online, since the members are not stored: after a merge the
  representative is whichever of the previous representative and the new key
  has the larger cosine with the group's key sum (exactly; ties keep the
  previous one);
* with either, a frame's candidates are the current representatives of the
  previous frame's groups, and a group's bucket is its newest key's bucket
  (the one the next frame's lookup uses).

Parity unpinned by the pages beyond Lemma 5.1: the selection rules above are
the definition; they are pinned by exact-duplicate and no-merge closed cases,
mass conservation and hand-worked tiny examples.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from .exact import exact_dot, exact_sqnorm, cos_compare, cos_at_least

_U64 = 2.0 ** -53


def round_fraction_to_storage(fr: Fraction, dtype: str) -> float:
    """The exact rational fr rounded once (to nearest, ties to even) to the
    storage dtype's precision (8 significant bits for bf16, 24 for f32)."""
    if fr == 0:
        return 0.0
    bits = 8 if dtype == "bf16" else 24
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # a = m 2^e with 1 <= m < 2: scale so that the integer part has `bits` bits
    scaled = a / (Fraction(2) ** (e - bits + 1))
    return sign * float(round(scaled)) * 2.0 ** (e - bits + 1)


def round_to_storage(x, dtype: str) -> np.ndarray:
    """Round float64 values once to the storage dtype (round to nearest even)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    m, e = np.frexp(x)                     # x = m 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)                 # 8 significant bits, ties to even
    return np.ldexp(r, e - 8)


class TempCacheOracle:
    """Compressed cache of one head, merged frame by frame."""

    def __init__(self, dim: int, dtype: str, representative: str = "last"):
        if representative not in ("last", "mean", "medoid"):
            raise ValueError(representative)
        self.dim = dim
        self.dtype = dtype
        self.representative = representative
        self.k_sum = []               # per group: exact key sum (Fractions), mean/medoid
        self.rep_k = np.zeros((0, dim))
        self.v_sum = np.zeros((0, dim))
        self.count = np.zeros(0, dtype=np.int64)
        self.rep_bucket = np.zeros(0, dtype=np.int64)
        self.frontier = None          # group id of each token of the last frame
        self.exact_evals = 0          # decisions float64 could not certify

    # -- derived quantities ------------------------------------------------
    @property
    def n_groups(self) -> int:
        return self.count.shape[0]

    @property
    def v_mean(self) -> np.ndarray:
        return round_to_storage(self.v_sum / self.count[:, None], self.dtype)

    @property
    def log_count(self) -> np.ndarray:
        return np.log(self.count.astype(np.float64))

    # -- one frame ---------------------------------------------------------
    def merge_frame(self, k, v, bucket, tau: float) -> np.ndarray:
        """Merge one frame (k, v [T, d], bucket [T]); return group of each token."""
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        bucket = np.asarray(bucket, dtype=np.int64)
        T, d = k.shape
        tau_q = Fraction(float(np.float32(tau)))
        target = np.full(T, -1, dtype=np.int64)       # proposed frame f-1 token
        tcos = np.zeros(T)                            # its cosine (float64)
        if self.frontier is not None:
            prev_k = self.rep_k[self.frontier]
            prev_b = self.rep_bucket[self.frontier]
            self._match(k, bucket, prev_k, prev_b, float(tau_q), tau_q, target, tcos)
            winner = self._resolve(k, prev_k, target, tcos)
        else:
            winner = {}
        group = np.empty(T, dtype=np.int64)
        merged = np.zeros(T, dtype=bool)
        for i, j in winner.items():
            merged[j] = True
            group[j] = self.frontier[i]
        fresh = np.nonzero(~merged)[0]                 # ascending j
        g0 = self.n_groups
        group[fresh] = g0 + np.arange(fresh.size)
        # state update from the frame f-1 snapshot
        mg = group[merged]
        mj = np.nonzero(merged)[0]
        self.count[mg] += 1
        self.v_sum[mg] += v[mj]
        if self.representative == "last":
            self.rep_k[mg] = k[mj]
        else:
            for g, j in zip(mg.tolist(), mj.tolist()):
                self._update_rep(g, k[j])
        self.rep_bucket[mg] = bucket[mj]
        if self.representative != "last":
            self.k_sum += [[Fraction(float(x)) for x in k[j]] for j in fresh.tolist()]
        self.rep_k = np.concatenate([self.rep_k, k[fresh]])
        self.v_sum = np.concatenate([self.v_sum, v[fresh]])
        self.count = np.concatenate([self.count, np.ones(fresh.size, dtype=np.int64)])
        self.rep_bucket = np.concatenate([self.rep_bucket, bucket[fresh]])
        self.frontier = group.copy()
        return group

    # -- representative of a group that key kj joins -------------------------
    def _update_rep(self, g, kj):
        s = self.k_sum[g]
        for i, x in enumerate(kj.tolist()):
            s[i] += Fraction(x)
        if self.representative == "mean":
            n = int(self.count[g])
            self.rep_k[g] = [round_fraction_to_storage(x / n, self.dtype) for x in s]
            return
        # medoid: the previous representative or kj, by cosine with the sum
        r = self.rep_k[g]
        dot = lambda a: sum((Fraction(float(u)) * w for u, w in zip(a, s)), Fraction(0))  # noqa: E731
        sq = lambda a: sum((Fraction(float(u)) ** 2 for u in a), Fraction(0))  # noqa: E731
        ss = sum((w * w for w in s), Fraction(0))
        if cos_compare(dot(kj), sq(kj) * ss, dot(r), sq(r) * ss) > 0:
            self.rep_k[g] = kj

    # -- step 1: each new key's best previous-frame candidate ---------------
    def _match(self, k, bucket, prev_k, prev_b, tau_f, tau_q, target, tcos):
        d = k.shape[1]
        err = (3 * d + 16) * _U64          # bound on |fl64(cos) - cos|
        nk = np.sqrt(np.sum(k * k, axis=1))
        npk = np.sqrt(np.sum(prev_k * prev_k, axis=1))
        for B in np.unique(bucket).tolist():
            J = np.nonzero(bucket == B)[0]
            I = np.nonzero(prev_b == B)[0]
            if I.size == 0:
                continue
            dots = k[J] @ prev_k[I].T
            den = nk[J][:, None] * npk[I][None, :]
            cos = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
            for a, j in enumerate(J.tolist()):
                row = cos[a]
                ib = int(np.argmax(row))              # first maximum = smallest i
                near = np.nonzero(row >= row[ib] - 2 * err)[0]
                if near.size > 1:
                    ib = self._exact_argmax(k[j], prev_k, I[near])
                    ib = int(np.nonzero(I == ib)[0][0])
                    self.exact_evals += 1
                c = row[ib]
                i = int(I[ib])
                if abs(c - tau_f) <= err:
                    self.exact_evals += 1
                    ok = cos_at_least(exact_dot(k[j], prev_k[i]),
                                      exact_sqnorm(k[j]) * exact_sqnorm(prev_k[i]), tau_q)
                else:
                    ok = c >= tau_f
                if ok:
                    target[j] = i
                    tcos[j] = c

    @staticmethod
    def _exact_argmax(kj, prev_k, cands):
        nj = exact_sqnorm(kj)
        best, bd, bn = None, None, None
        for i in sorted(cands.tolist()):
            di = exact_dot(kj, prev_k[i])
            ni = nj * exact_sqnorm(prev_k[i])
            if best is None or cos_compare(di, ni, bd, bn) > 0:
                best, bd, bn = i, di, ni
        return best

    # -- step 2: one-to-one, best proposer wins ------------------------------
    def _resolve(self, k, prev_k, target, tcos):
        d = k.shape[1]
        err = (3 * d + 16) * _U64
        winner = {}
        for i in np.unique(target[target >= 0]).tolist():
            P = np.nonzero(target == i)[0]            # ascending j
            c = tcos[P]
            jb = int(np.argmax(c))
            near = np.nonzero(c >= c[jb] - 2 * err)[0]
            if near.size > 1:
                self.exact_evals += 1
                ni = exact_sqnorm(prev_k[i])
                best, bd, bn = None, None, None
                for j in P[near].tolist():
                    dj = exact_dot(k[j], prev_k[i])
                    nn = exact_sqnorm(k[j]) * ni
                    if best is None or cos_compare(dj, nn, bd, bn) > 0:
                        best, bd, bn = j, dj, nn
                winner[i] = best
            else:
                winner[i] = int(P[jb])
        return winner

"""TempCache with quantized ANN matching ("Quant"), one attention head (oracle).

The pages offer two ANN searches for TempCache's top-1 match: LSH, and
quantized similarity search, both without offline preprocessing
(paperlayer.ai section 5 "ANN Attention"; gist.science technical summary,
TempCache mechanism: "LSH or quantisation"); the quantized variant is the
default, at 8 bits (paper.rainbus.top, reproducibility), and fewer bits trade
recall for speed (paperlayer.ai appendix C, quantization precision).

Readings where the pages are silent:
* codes: each key is quantized on its own row scale, symmetric, to
  b-bit signed integers: c_i = round_half_even(Q x_i / max_i |x_i|) with
  Q = 2^(b-1) - 1 (a zero row codes to zeros).  No codebook, nothing trained;
  the cosine of the decoded vectors equals the cosine of the integer codes,
  which is what the match compares, exactly;
* candidates: every token of the previous frame (no buckets: the quantized
  search replaces the hash-table lookup), i.e. the representatives of the
  frontier groups;
* query-driven correspondence (gist.science technical summary and
  paper.rainbus.top method steps: each current-frame token's QUERY finds its
  top-1 key in the previous frame): with ``match_vec`` the new side of the
  similarity is that token's query code instead of its key code; the token
  still joins the group with its key and value;
* everything else is TempCache's rule set unchanged (the LSH oracle's
  readings): the best candidate by similarity, ties to the smaller index;
  propose if similarity >= tau (tau as its float32 value); one-to-one, the
  largest similarity wins a candidate, ties to the smaller new index; last
  key, float32-free exact value sums, mean rounded once, ln m bias.  The
  representative's bucket still indexes the attention.

Parity unpinned by the pages beyond the closed cases (exact duplicates, tau
> 1, invariance to a positive rescaling of a key) and hand-worked codes.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from .exact import cos_compare, cos_at_least
from .tempcache import TempCacheOracle

_U64 = 2.0 ** -53


def scalar_codes(x, bits: int = 8) -> np.ndarray:
    """Per-row symmetric b-bit codes (int64) of x [N, d], rounded exactly."""
    if not 2 <= bits <= 8:
        raise ValueError("bits must be in [2, 8]")
    x = np.asarray(x, dtype=np.float64)
    q = (1 << (bits - 1)) - 1
    out = np.zeros(x.shape, dtype=np.int64)
    for r in range(x.shape[0]):
        m = float(np.max(np.abs(x[r]))) if x.shape[1] else 0.0
        if m == 0.0:
            continue
        fm = Fraction(m)
        out[r] = [round(Fraction(q) * Fraction(float(v)) / fm) for v in x[r]]  # round half to even
    return out


class TempCacheQuantOracle(TempCacheOracle):
    """TempCache whose top-1 match compares b-bit scalar codes of the keys
    against every previous-frame token."""

    def __init__(self, dim: int, dtype: str, bits: int = 8, representative: str = "last"):
        super().__init__(dim, dtype, representative)
        self.bits = bits
        self._match_vec = None

    def merge_frame(self, k, v, bucket, tau: float, match_vec=None) -> np.ndarray:
        """As TempCacheOracle.merge_frame; match_vec [T, d] (the tokens'
        queries): query-driven matching."""
        self._match_vec = None if match_vec is None else np.asarray(match_vec, dtype=np.float64)
        try:
            return super().merge_frame(k, v, bucket, tau)
        finally:
            self._match_vec = None

    def _match(self, k, bucket, prev_k, prev_b, tau_f, tau_q, target, tcos):
        ck = scalar_codes(k if self._match_vec is None else self._match_vec, self.bits)
        cp = scalar_codes(prev_k, self.bits)
        dots = ck @ cp.T                                  # exact (small integers)
        nk = (ck * ck).sum(axis=1)
        npv = (cp * cp).sum(axis=1)
        den = np.sqrt(nk[:, None].astype(np.float64) * npv[None, :].astype(np.float64))
        cos = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
        err = 4 * _U64                                    # |fl64(cos) - cos| / 1, generously
        self._codes = (ck, cp, dots, nk, npv)
        for j in range(k.shape[0]):
            row = cos[j]
            ib = int(np.argmax(row))                      # first maximum = smallest i
            near = np.nonzero(row >= row[ib] - 2 * err)[0]
            if near.size > 1:
                self.exact_evals += 1
                best = None
                for i in near.tolist():                   # ascending i
                    if best is None or cos_compare(int(dots[j, i]), int(nk[j]) * int(npv[i]),
                                                   int(dots[j, best]), int(nk[j]) * int(npv[best])) > 0:
                        best = i
                ib = best
            if abs(row[ib] - tau_f) <= err:
                self.exact_evals += 1
                ok = cos_at_least(Fraction(int(dots[j, ib])), Fraction(int(nk[j]) * int(npv[ib])), tau_q)
            else:
                ok = row[ib] >= tau_f
            if ok:
                target[j] = ib
                tcos[j] = row[ib]

    def _resolve(self, k, prev_k, target, tcos):
        ck, cp, dots, nk, npv = self._codes
        err = 4 * _U64
        winner = {}
        for i in np.unique(target[target >= 0]).tolist():
            P = np.nonzero(target == i)[0]                # ascending j
            c = tcos[P]
            jb = int(np.argmax(c))
            near = np.nonzero(c >= c[jb] - 2 * err)[0]
            if near.size > 1:
                self.exact_evals += 1
                best = None
                for j in P[near].tolist():
                    if best is None or cos_compare(int(dots[j, i]), int(nk[j]) * int(npv[i]),
                                                   int(dots[best, i]), int(nk[best]) * int(npv[i])) > 0:
                        best = j
                winner[i] = best
            else:
                winner[i] = int(P[jb])
        return winner

"""CPU oracle for the FAST-AR attention hot path -- TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never calls it and shares no code with it.

What it computes, step by step, in float64 on the dtype-rounded inputs, with
every integer decision that depends on a float comparison (a hash sign, an
arg-max, a threshold) settled on the exact real value of its operands:

* ``simhash``     -- random-hyperplane hashing of queries and keys into
                     bucket ids, optionally with more probes (paper page
                     "paperlayer.ai", section 5 Method, "ANN Attention";
                     paper.rainbus.top, prerequisites, ANN).
* ``index``       -- the bucket-contiguous index (stable counting sort) that
                     block-sparse attention consumes (gist.science technical
                     summary, AnnSA mechanism).
* ``tempcache``   -- TempCache: top-1 match of each new key against the
                     previous frame's keys in its bucket, threshold merge,
                     last key as representative, value mean and log-count
                     bias (paperlayer.ai section 5 "TempCache", appendix A,
                     Lemma 5.1; appendix C ablations).
* ``tempcache_quant`` -- TempCache's quantized-ANN variant: the top-1 match
                     compares b-bit scalar codes against every previous-frame
                     token (paperlayer.ai section 5 "ANN Attention", appendix
                     C quantization precision).
* ``annca``       -- AnnCA prompt pruning and cross-attention over the kept
                     prompt tokens (gist.science technical summary, AnnCA).
* ``attention``   -- dense softmax attention and AnnSA bucket-restricted
                     attention with the +log m bias (paperlayer.ai section 3
                     attention formulation, section 5 "AnnSA", appendix A).
* ``sequence``    -- one layer's per-chunk call sequence: hash, merge, prune,
                     self-attention, cross-attention.
* ``multitable``  -- several LSH tables (and more probes per table): AnnSA
                     over the union of the tables' buckets, AnnCA keeping a
                     prompt token that any table keeps (paperlayer.ai
                     section 2, approximate nearest neighbor search).
* ``recall``      -- attention recall (dense mass kept by the retained
                     entries) and density, and the top-k reference
                     (paperlayer.ai section 4, attention sparsity).

Pins (tests marked ``not gpu``) tie each function to something other than
itself: Lemma 5.1, dense attention in the one-bucket case, a library SDPA,
exact rational brute force on tiny inputs, closed forms and invariants.  The
thresholded TempCache selection rule beyond exact duplicates is not fixed by
the pages: its tie and conflict rules are readings, pinned only by hand-worked
examples and invariants.
"""

from .exact import exact_dot, exact_sqnorm, cos_compare, cos_at_least  # noqa: F401
from .simhash import simhash  # noqa: F401
from .index import bucket_index  # noqa: F401
from .tempcache import TempCacheOracle  # noqa: F401
from .tempcache_quant import TempCacheQuantOracle, scalar_codes  # noqa: F401
from .annca import prune_prompt, cross_attention  # noqa: F401
from .attention import dense_attention, bucket_attention  # noqa: F401
from .sequence import run_chunk  # noqa: F401
from .recall import attention_recall, bucket_retained, topk_recall  # noqa: F401
from .multitable import (simhash_tables, retained_tables, bucket_attention_tables,  # noqa: F401
                         prune_prompt_tables)

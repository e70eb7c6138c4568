"""FAST-AR attention hot path for AMD MI355X: Python binding of libfastar.

The compute runs in the HIP library ``libfastar.so`` (built in-tree by
``__graft_entry__.build()``); this package only marshals torch tensors
(device memory and streams) into its C ABI.  Importing the binding does not
load the library; the first call does, and fails loudly if it is missing.
"""

from .fastar import (  # noqa: F401
    FastarError,
    TempCache,
    fastar_attention_recall,
    fastar_attention_recall_counts,
    fastar_bucket_attention,
    fastar_bucket_attention_tables,
    fastar_bucket_index,
    fastar_hash,
    fastar_hash_multi,
    fastar_prune_prompt,
    fastar_prune_prompt_tables,
    fastar_scalar_codes,
    fastar_tempcache_merge,
    fastar_version,
    library,
    merge_opts,
    new_diag,
)

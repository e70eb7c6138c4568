"""ctypes binding of libfastar (include/fastar.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of libfastar.so.  torch supplies device memory and the stream.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfastar.so")

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


class FastarTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("tokens", ctypes.c_int64),
        ("dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("stride_head", ctypes.c_int64),
        ("stride_token", ctypes.c_int64),
    ]


class FastarCache(ctypes.Structure):
    _fields_ = [
        ("heads", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("tokens_per_frame", ctypes.c_int32),
        ("n_bits", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rep_k", ctypes.c_void_p),
        ("v_mean", ctypes.c_void_p),
        ("v_sum", ctypes.c_void_p),
        ("count", ctypes.c_void_p),
        ("log_count", ctypes.c_void_p),
        ("rep_bucket", ctypes.c_void_p),
        ("n_groups", ctypes.c_void_p),
        ("frontier", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("k_sum", ctypes.c_void_p),
    ]


class FastarMergeOpts(ctypes.Structure):
    _fields_ = [("match", ctypes.c_int32), ("code_bits", ctypes.c_int32),
                ("representative", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("match_queries", ctypes.c_void_p), ("reserved_ptr", ctypes.c_void_p)]


MATCH = {"lsh": 0, "quant": 1}
REPRESENTATIVE = {"last": 0, "mean": 1, "medoid": 2}


def merge_opts(match: str = "lsh", code_bits: int = 8, representative: str = "last",
               match_queries=None) -> FastarMergeOpts:
    """fastar_merge_opts_t for a TempCache variant: match "lsh" or "quant";
    representative "last", "mean" or "medoid"; match_queries (a [H, n, d]
    tensor of the new frames' queries): query-driven matching.  The returned
    struct keeps the query descriptor alive."""
    o = FastarMergeOpts(MATCH[match], code_bits, REPRESENTATIVE[representative], 0, None, None)
    if match_queries is not None:
        o._qdesc = _desc(match_queries)
        o._qtensor = match_queries
        o.match_queries = ctypes.addressof(o._qdesc)
    return o


class FastarChunk(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("n_probes", ctypes.c_int),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("n_frames", ctypes.c_int),
        ("prompt_k", ctypes.c_void_p), ("prompt_v", ctypes.c_void_p),
        ("planes", ctypes.c_void_p), ("n_bits", ctypes.c_int), ("tau", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("cache", ctypes.c_void_p),
        ("q_bucket", ctypes.c_void_p), ("q_offsets", ctypes.c_void_p), ("q_perm", ctypes.c_void_p),
        ("k_bucket", ctypes.c_void_p), ("group_of_new", ctypes.c_void_p),
        ("rep_offsets", ctypes.c_void_p), ("rep_perm", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("p_bucket", ctypes.c_void_p), ("keep", ctypes.c_void_p), ("kept_idx", ctypes.c_void_p),
        ("n_kept", ctypes.c_void_p), ("out_cross", ctypes.c_void_p), ("lse_cross", ctypes.c_void_p),
        ("merge_opts", ctypes.c_void_p),
    ]


class FastarError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libfastar status {status}: {message}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_TP = ctypes.POINTER(FastarTensor)
_CP = ctypes.POINTER(FastarCache)

_SIGNATURES = {
    "fastar_status_string": (ctypes.c_char_p, [_I]),
    "fastar_last_error": (ctypes.c_char_p, []),
    "fastar_version": (_I, []),
    "fastar_hash_workspace": (_SZ, [_I, _I64, _I, _I]),
    "fastar_hash": (_I, [_TP, _P, _I, _I, _P, _P, _P, _P, _SZ, _P, _P]),
    "fastar_hash_multi": (_I, [_I, _P, _P, _P, _P, _I, _P, _P]),
    "fastar_bucket_index_workspace": (_SZ, [_I, _I64]),
    "fastar_bucket_index": (_I, [_P, _I, _I64, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "fastar_tempcache_workspace": (_SZ, [_CP, _I]),
    "fastar_tempcache_workspace_ex": (_SZ, [_CP, _I, _P]),
    "fastar_tempcache_merge_ex": (_I, [_CP, _TP, _TP, _P, _I, _F, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "fastar_scalar_codes": (_I, [_TP, _I, _P, _P, _P]),
    "fastar_cache_status": (_I, [_CP, _I, _P]),
    "fastar_tempcache_merge": (_I, [_CP, _TP, _TP, _P, _I, _F, _P, _P, _P, _P, _SZ, _P, _P]),
    "fastar_prune_prompt": (_I, [_P, _I, _I64, _I, _P, _I64, _I, _P, _P, _P, _P]),
    "fastar_bucket_attention": (_I, [_TP, _P, _P, _I, _TP, _TP, _P, _P, _P, _I, _P, _P, _F, _P, _P, _P]),
    "fastar_attention_recall": (_I, [_P, _P, _I, _I64, _P, _I, _P, _I, _P, _P, _P, _P, _P]),
    "fastar_bucket_attention_tables": (_I, [_TP, _I, _P, _P, _I, _TP, _TP, _P, _P, _P, _P, _I, _F, _P, _P,
                                            _P, _P]),
    "fastar_prune_prompt_tables": (_I, [_P, _I, _I, _I64, _I, _P, _I64, _I, _P, _P, _P, _P]),
    "fastar_attention_recall_counts": (_I, [_P, _P, _I, _I64, _P, _P, _P, _P, _P]),
    "fastar_chunk_workspace": (_SZ, [_P]),
    "fastar_chunk": (_I, [_P, _P, _SZ, _P, _P]),
    "fastar_chunk_noalloc": (_I, [_P, _P, _P]),
}

# FASTAR_NOALLOC_SCRATCH_BYTES, FASTAR_MAX_PROBES, FASTAR_MAX_TABLES in include/fastar.h
NOALLOC_SCRATCH_BYTES = 48 << 20
MAX_PROBES = 8
MAX_TABLES = 4


def library():
    """Load libfastar.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        lib = library()
        raise FastarError(status, f"{lib.fastar_status_string(status).decode()}: "
                                  f"{lib.fastar_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("array arguments must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _desc(t: torch.Tensor) -> FastarTensor:
    if t.dim() != 3 or (t.numel() and t.stride(2) != 1):
        raise ValueError("expected a [heads, tokens, dim] tensor with a contiguous last dim")
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}")
    # an empty tensor's strides are not looked at
    sh, st = (t.stride(0), t.stride(1)) if t.numel() else (t.shape[1] * t.shape[2], t.shape[2])
    return FastarTensor(t.data_ptr(), _DTYPES[t.dtype], t.shape[0], t.shape[1], t.shape[2], 0, sh, st)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _i32(shape, device):
    return torch.empty(shape, dtype=torch.int32, device=device)


def _ws(nbytes: int, device, ws: Optional[torch.Tensor]):
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes < {nbytes}")
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def new_diag(device="cuda") -> torch.Tensor:
    """Zeroed fastar_diag_t counters (8 x int32) on the device."""
    return torch.zeros(8, dtype=torch.int32, device=device)


def fastar_version() -> int:
    return library().fastar_version()


def fastar_hash(x, planes, n_bits: int, n_probes: int = 1, with_index: bool = True,
                bucket=None, offsets=None, perm=None, ws=None, diag=None, stream=None):
    """Bucket ids [H, N, P] (+ offsets [H, 2^b+1], perm [H, N]) of x [H, N, d]."""
    lib = library()
    H, N, _ = x.shape
    if bucket is None:
        bucket = _i32((H, N, n_probes), x.device)
    if with_index:
        if offsets is None:
            offsets = _i32((H, (1 << n_bits) + 1), x.device)
        if perm is None:
            perm = _i32((H, N), x.device)
    else:
        offsets = perm = None
    nbytes = lib.fastar_hash_workspace(H, N, n_bits, n_probes)
    ws = _ws(nbytes, x.device, ws)
    d = _desc(x)
    _check(lib.fastar_hash(ctypes.byref(d), _ptr(planes), n_bits, n_probes, _ptr(bucket),
                           _ptr(offsets), _ptr(perm), _ptr(ws), ws.numel() * ws.element_size(),
                           _ptr(diag), _stream(stream)))
    return bucket, offsets, perm


def fastar_hash_multi(xs, planes, n_bits: int, n_probes, buckets=None, diag=None, stream=None):
    """Bucket ids [H_i, N_i, P_i] of each x_i [H_i, N_i, d] (one launch for bf16)."""
    lib = library()
    n = len(xs)
    if buckets is None:
        buckets = [_i32((x.shape[0], x.shape[1], p), x.device) for x, p in zip(xs, n_probes)]
    descs = [_desc(x) for x in xs]
    xp = (ctypes.c_void_p * n)(*[ctypes.addressof(d) for d in descs])
    npr = (ctypes.c_int * n)(*n_probes)
    bp = (ctypes.c_void_p * n)(*[b.data_ptr() for b in buckets])
    _check(lib.fastar_hash_multi(n, ctypes.cast(xp, _P), ctypes.cast(npr, _P), ctypes.cast(bp, _P),
                                 _ptr(planes), n_bits, _ptr(diag), _stream(stream)))
    return buckets


def fastar_bucket_index(bucket, n_bits: int, n_valid=None, offsets=None, perm=None, ws=None,
                        stream=None):
    """Index of precomputed ids bucket [H, n, P]."""
    lib = library()
    H, n, P = bucket.shape
    if offsets is None:
        offsets = _i32((H, (1 << n_bits) + 1), bucket.device)
    if perm is None:
        perm = _i32((H, n), bucket.device)
    ws = _ws(lib.fastar_bucket_index_workspace(H, n), bucket.device, ws)
    _check(lib.fastar_bucket_index(_ptr(bucket), H, n, P, n_bits, _ptr(n_valid), _ptr(offsets),
                                   _ptr(perm), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)))
    return offsets, perm


class TempCache:
    """Device buffers of one layer's compressed cache (fastar_cache_t)."""

    def __init__(self, heads, dim, capacity, tokens_per_frame, n_bits, dtype=torch.bfloat16,
                 device="cuda", key_sums: bool = False):
        """key_sums: also keep the float64 key sums that merges with the mean or
        medoid representative need."""
        self.heads, self.dim, self.capacity = heads, dim, capacity
        self.tokens_per_frame, self.n_bits, self.dtype = tokens_per_frame, n_bits, dtype
        z = dict(device=device)
        self.rep_k = torch.zeros(heads, capacity, dim, dtype=dtype, **z)
        self.v_mean = torch.zeros(heads, capacity, dim, dtype=dtype, **z)
        self.v_sum = torch.zeros(heads, capacity, dim, dtype=torch.float32, **z)
        self.count = torch.zeros(heads, capacity, dtype=torch.int32, **z)
        self.log_count = torch.zeros(heads, capacity, dtype=torch.float32, **z)
        self.rep_bucket = torch.zeros(heads, capacity, dtype=torch.int32, **z)
        self.n_groups = torch.zeros(heads, dtype=torch.int32, **z)
        self.frontier = torch.full((heads, tokens_per_frame), -1, dtype=torch.int32, **z)
        self.status = torch.zeros(1, dtype=torch.int32, **z)
        self.k_sum = (torch.zeros(heads, capacity, dim, dtype=torch.float64, **z) if key_sums
                      else None)

    def buffers(self):
        b = dict(rep_k=self.rep_k, v_mean=self.v_mean, v_sum=self.v_sum, count=self.count,
                 log_count=self.log_count, rep_bucket=self.rep_bucket,
                 n_groups=self.n_groups, frontier=self.frontier, status=self.status)
        if self.k_sum is not None:
            b["k_sum"] = self.k_sum
        return b

    def copy_from(self, other: "TempCache"):
        for name, t in self.buffers().items():
            t.copy_(getattr(other, name))

    _GROUP_ROWS = ("rep_k", "v_mean", "v_sum", "count", "log_count", "rep_bucket", "k_sum")

    def checkpoint(self) -> dict:
        """What later merges can change, saved for restore(): the rows of the
        last frame's groups (the only existing groups a merge extends: frame
        f's candidates are frame f - 1's groups, so every chain of later
        frames starts at one of them), the group count, the frontier and the
        status word.  Groups opened later lie past the saved count; a merge
        that opens them again rewrites every field of their rows.  Device
        copies only (stream-ordered)."""
        H, cap = self.heads, self.capacity
        heads = torch.arange(H, device=self.frontier.device)[:, None] * cap
        idx = (heads + self.frontier.clamp_min(0)).reshape(-1).long()
        rows = {}
        for name in self._GROUP_ROWS:
            t = getattr(self, name)
            if t is not None:
                rows[name] = t.view(H * cap, -1).index_select(0, idx)
        return {"idx": idx, "rows": rows, "n_groups": self.n_groups.clone(),
                "frontier": self.frontier.clone(), "status": self.status.clone()}

    def restore(self, ck: dict):
        """Undo the merges since checkpoint() returned ck."""
        H, cap = self.heads, self.capacity
        for name, saved in ck["rows"].items():
            getattr(self, name).view(H * cap, -1).index_copy_(0, ck["idx"], saved)
        self.n_groups.copy_(ck["n_groups"])
        self.frontier.copy_(ck["frontier"])
        self.status.copy_(ck["status"])

    def struct(self) -> FastarCache:
        return FastarCache(self.heads, self.dim, self.capacity, self.tokens_per_frame, self.n_bits,
                           _DTYPES[self.dtype], self.rep_k.data_ptr(), self.v_mean.data_ptr(),
                           self.v_sum.data_ptr(), self.count.data_ptr(),
                           self.log_count.data_ptr(), self.rep_bucket.data_ptr(),
                           self.n_groups.data_ptr(), self.frontier.data_ptr(),
                           self.status.data_ptr(),
                           None if self.k_sum is None else self.k_sum.data_ptr())

    def workspace_bytes(self, n_frames: int, opts: Optional[FastarMergeOpts] = None) -> int:
        c = self.struct()
        return library().fastar_tempcache_workspace_ex(ctypes.byref(c), n_frames,
                                                       None if opts is None else ctypes.byref(opts))

    def status_code(self, clear: bool = False, stream=None) -> int:
        """fastar_cache_status: 0 (ok) or 5 (FASTAR_ERR_CAPACITY: a merge since the
        last clear dropped groups).  Synchronises the stream."""
        c = self.struct()
        st = library().fastar_cache_status(ctypes.byref(c), int(clear), _stream(stream))
        if st not in (0, 5):
            _check(st)
        return st


def fastar_tempcache_merge(cache: TempCache, k_new, v_new, k_new_bucket, n_frames: int,
                           tau: float, group_of_new=None, with_index: bool = True,
                           rep_offsets=None, rep_perm=None, ws=None, diag=None, stream=None,
                           opts: Optional[FastarMergeOpts] = None):
    """Merge n_frames frames (k_new, v_new [H, n_frames*T, d]) into the cache
    (opts: the TempCache variant, merge_opts(); None: the defaults)."""
    lib = library()
    H = cache.heads
    dev = k_new.device
    if with_index:
        if rep_offsets is None:
            rep_offsets = _i32((H, (1 << cache.n_bits) + 1), dev)
        if rep_perm is None:
            rep_perm = _i32((H, cache.capacity), dev)
    else:
        rep_offsets = rep_perm = None
    c = cache.struct()
    o = None if opts is None else ctypes.byref(opts)
    ws = _ws(lib.fastar_tempcache_workspace_ex(ctypes.byref(c), n_frames, o), dev, ws)
    dk, dv = _desc(k_new), _desc(v_new)
    _check(lib.fastar_tempcache_merge_ex(ctypes.byref(c), ctypes.byref(dk), ctypes.byref(dv),
                                         _ptr(k_new_bucket), n_frames, float(tau), o, _ptr(group_of_new),
                                         _ptr(rep_offsets), _ptr(rep_perm), _ptr(ws),
                                         ws.numel() * ws.element_size(), _ptr(diag), _stream(stream)))
    return rep_offsets, rep_perm


def fastar_scalar_codes(x, bits: int = 8, codes=None, norm2=None, stream=None):
    """Per-row symmetric b-bit codes [H, N, d] (int8) and squared norms [H, N] of x."""
    lib = library()
    H, N, d = x.shape
    if codes is None:
        codes = torch.empty(H, N, d, dtype=torch.int8, device=x.device)
    if norm2 is None:
        norm2 = torch.empty(H, N, dtype=torch.int32, device=x.device)
    dx = _desc(x)
    _check(lib.fastar_scalar_codes(ctypes.byref(dx), bits, _ptr(codes), _ptr(norm2), _stream(stream)))
    return codes, norm2


def fastar_prune_prompt(q_bucket, p_bucket, n_bits: int, keep=None, kept_idx=None, n_kept=None,
                        stream=None):
    """AnnCA keep mask [H, Np] (uint8), kept indices [H, Np], counts [H]."""
    lib = library()
    H, nq, P = q_bucket.shape
    npr = p_bucket.shape[1]
    dev = q_bucket.device
    if keep is None:
        keep = torch.empty(H, npr, dtype=torch.uint8, device=dev)
    if kept_idx is None:
        kept_idx = _i32((H, npr), dev)
    if n_kept is None:
        n_kept = _i32((H,), dev)
    _check(lib.fastar_prune_prompt(_ptr(q_bucket), H, nq, P, _ptr(p_bucket), npr, n_bits,
                                   _ptr(keep), _ptr(kept_idx), _ptr(n_kept), _stream(stream)))
    return keep, kept_idx, n_kept


def fastar_bucket_attention(q, k, v, scale: Optional[float] = None, q_bucket=None, q_perm=None,
                            key_bias=None, k_offsets=None, k_perm=None, n_bits: int = 0,
                            key_list=None, n_key_list=None, out=None, lse=None,
                            want_lse: bool = True, stream=None):
    """Bucket (AnnSA), list (AnnCA) or dense attention; returns (out, lse)."""
    lib = library()
    H, nq, d = q.shape
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty(H, nq, d, dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(H, nq, dtype=torch.float32, device=q.device)
    n_probes = 1 if q_bucket is None else q_bucket.shape[2]
    dq, dk, dv = _desc(q), _desc(k), _desc(v)
    _check(lib.fastar_bucket_attention(ctypes.byref(dq), _ptr(q_bucket), _ptr(q_perm), n_probes,
                                       ctypes.byref(dk), ctypes.byref(dv), _ptr(key_bias),
                                       _ptr(k_offsets), _ptr(k_perm), n_bits, _ptr(key_list),
                                       _ptr(n_key_list), float(scale), _ptr(out), _ptr(lse),
                                       _stream(stream)))
    return out, lse


def fastar_bucket_attention_tables(q, k, v, q_bucket, q_perm, k_offsets, k_perm, n_bits: int,
                                   k_bucket=None, scale: Optional[float] = None, key_bias=None,
                                   out=None, lse=None, n_attended=None, want_lse: bool = True,
                                   want_count: bool = False, stream=None):
    """AnnSA over several LSH tables (q_bucket [L, H, nq, P], k_offsets
    [L, H, 2^b + 1], k_perm and k_bucket [L, H, nk]); returns (out, lse,
    n_attended)."""
    lib = library()
    H, nq, d = q.shape
    L, P = q_bucket.shape[0], q_bucket.shape[3]
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty(H, nq, d, dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(H, nq, dtype=torch.float32, device=q.device)
    if n_attended is None and want_count:
        n_attended = _i32((H, nq), q.device)
    dq, dk, dv = _desc(q), _desc(k), _desc(v)
    _check(lib.fastar_bucket_attention_tables(ctypes.byref(dq), L, _ptr(q_bucket), _ptr(q_perm), P,
                                              ctypes.byref(dk), ctypes.byref(dv), _ptr(key_bias),
                                              _ptr(k_bucket), _ptr(k_offsets), _ptr(k_perm), n_bits,
                                              float(scale), _ptr(out), _ptr(lse), _ptr(n_attended),
                                              _stream(stream)))
    return out, lse, n_attended


def fastar_prune_prompt_tables(q_bucket, p_bucket, n_bits: int, keep=None, kept_idx=None, n_kept=None,
                               stream=None):
    """AnnCA over several LSH tables: q_bucket [L, H, nq, P], p_bucket
    [L, H, Np]; returns keep [H, Np], kept indices [H, Np], counts [H]."""
    lib = library()
    L, H, nq, P = q_bucket.shape
    npr = p_bucket.shape[2]
    dev = q_bucket.device
    if keep is None:
        keep = torch.empty(H, npr, dtype=torch.uint8, device=dev)
    if kept_idx is None:
        kept_idx = _i32((H, npr), dev)
    if n_kept is None:
        n_kept = _i32((H,), dev)
    _check(lib.fastar_prune_prompt_tables(_ptr(q_bucket), L, H, nq, P, _ptr(p_bucket), npr, n_bits,
                                          _ptr(keep), _ptr(kept_idx), _ptr(n_kept), _stream(stream)))
    return keep, kept_idx, n_kept


def fastar_attention_recall_counts(lse_sparse, lse_dense, n_keys, n_attended, recall=None, stats=None,
                                   want_recall: bool = True, stream=None):
    """fastar_attention_recall with the retained counts given per query
    (n_attended [H, n_q])."""
    lib = library()
    H, nq = lse_sparse.shape
    dev = lse_sparse.device
    if recall is None and want_recall:
        recall = torch.empty(H, nq, dtype=torch.float32, device=dev)
    if stats is None:
        stats = torch.empty(H, 2, dtype=torch.float32, device=dev)
    _check(lib.fastar_attention_recall_counts(_ptr(lse_sparse), _ptr(lse_dense), H, nq, _ptr(n_attended),
                                              _ptr(n_keys), _ptr(recall), _ptr(stats), _stream(stream)))
    return recall, stats


def fastar_attention_recall(lse_sparse, lse_dense, n_keys, q_bucket=None, k_offsets=None,
                            n_bits: int = 0, n_retained=None, recall=None, stats=None,
                            want_recall: bool = True, stream=None):
    """Recall [H, n_q] (exp(lse_sparse - lse_dense)) and stats [H, 2] (mean
    recall, mean density) of a sparse attention against the dense one."""
    lib = library()
    H, nq = lse_sparse.shape
    dev = lse_sparse.device
    if recall is None and want_recall:
        recall = torch.empty(H, nq, dtype=torch.float32, device=dev)
    if stats is None:
        stats = torch.empty(H, 2, dtype=torch.float32, device=dev)
    P = 1 if q_bucket is None else q_bucket.shape[2]
    _check(lib.fastar_attention_recall(_ptr(lse_sparse), _ptr(lse_dense), H, nq, _ptr(q_bucket), P,
                                       _ptr(k_offsets), n_bits, _ptr(n_retained), _ptr(n_keys),
                                       _ptr(recall), _ptr(stats), _stream(stream)))
    return recall, stats


class ChunkCall:
    """fastar_chunk's argument block for fixed buffers: built once, so that a
    call (also under HIP graph capture) only passes pointers."""

    def __init__(self, q, n_probes, k_new, v_new, n_frames, planes, n_bits, tau, cache: TempCache,
                 q_bucket, q_offsets, q_perm, k_bucket, rep_offsets, rep_perm, out, lse=None,
                 group_of_new=None, scale=None, prompt_k=None, prompt_v=None, p_bucket=None,
                 keep=None, kept_idx=None, n_kept=None, out_cross=None, lse_cross=None,
                 opts: Optional[FastarMergeOpts] = None):
        d = q.shape[-1]
        self._keep = []  # everything the pointers below refer to

        def desc(t):
            if t is None:
                return None
            dd = _desc(t)
            self._keep.append(dd)
            return ctypes.addressof(dd)

        self.cache_struct = cache.struct()
        p = lambda t: None if t is None else _ptr(t).value
        self.args = FastarChunk(
            desc(q), n_probes, desc(k_new), desc(v_new), n_frames, desc(prompt_k), desc(prompt_v),
            p(planes), n_bits, tau, float(scale if scale is not None else d ** -0.5),
            ctypes.addressof(self.cache_struct),
            p(q_bucket), p(q_offsets), p(q_perm), p(k_bucket), p(group_of_new), p(rep_offsets),
            p(rep_perm), p(out), p(lse), p(p_bucket), p(keep), p(kept_idx), p(n_kept), p(out_cross),
            p(lse_cross), None if opts is None else ctypes.addressof(opts))
        self._keep.append(opts)
        self._keep += [q, k_new, v_new, prompt_k, prompt_v, planes, q_bucket, q_offsets, q_perm,
                       k_bucket, group_of_new, rep_offsets, rep_perm, out, lse, p_bucket, keep,
                       kept_idx, n_kept, out_cross, lse_cross]

    def workspace_bytes(self) -> int:
        return library().fastar_chunk_workspace(ctypes.byref(self.args))

    def __call__(self, ws, diag=None, stream=None):
        _check(library().fastar_chunk(ctypes.byref(self.args), _ptr(ws), ws.numel() * ws.element_size(),
                                      _ptr(diag), _stream(stream)))

    def noalloc(self, diag=None, stream=None):
        """fastar_chunk_noalloc: the same call with the library's scratch as
        workspace (nothing allocated, by torch or the library)."""
        _check(library().fastar_chunk_noalloc(ctypes.byref(self.args), _ptr(diag), _stream(stream)))

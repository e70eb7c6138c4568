"""Host-only checks of the C ABI: the library loads, exports every function
include/fastar.h declares, and rejects bad arguments before any launch
(so these run without a GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fastar.h")

fa = pytest.importorskip("kv_compressed_attention_amd")
from kv_compressed_attention_amd import fastar as fb  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fb.LIB_PATH):
        pytest.skip("libfastar.so not built (run __graft_entry__.build())")
    return fa.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fastar_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for op in ("fastar_hash", "fastar_tempcache_merge", "fastar_prune_prompt",
               "fastar_bucket_attention"):
        assert op in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fastar_[a-z_0-9]+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


def test_binding_covers_every_declared_symbol():
    assert set(fb._SIGNATURES) == set(declared_functions())


def test_struct_layouts_match_header(lib):
    assert ctypes.sizeof(fb.FastarTensor) == 48
    assert ctypes.sizeof(fb.FastarCache) == 24 + 10 * 8


def test_status_strings(lib):
    assert lib.fastar_status_string(0) == b"ok"
    assert lib.fastar_status_string(1) == b"invalid argument"
    assert lib.fastar_status_string(3) == b"workspace too small"
    assert lib.fastar_status_string(5) == b"cache capacity exceeded"
    assert lib.fastar_version() >= 200


def test_cache_status_rejects_missing_status_word(lib):
    # fastar_cache_status needs the cache and its device status word; the
    # merge needs the status word too (overflow is always reported)
    assert lib.fastar_cache_status(None, 0, None) == 1
    buf = 1 << 20
    c = fb.FastarCache(2, 128, 64, 16, 12, 1, *([buf] * 8), 0)
    assert lib.fastar_cache_status(ctypes.byref(c), 1, None) == 1
    k = _tensor(tokens=16)
    st = lib.fastar_tempcache_merge(ctypes.byref(c), ctypes.byref(k), ctypes.byref(k),
                                    ctypes.c_void_p(buf), 1, 0.9, None, None, None,
                                    ctypes.c_void_p(buf), 1 << 30, None, None)
    assert st == 1 and b"NULL" in lib.fastar_last_error()


def _tensor(dtype=1, heads=2, tokens=16, dim=128, data=1 << 20):
    return fb.FastarTensor(data, dtype, heads, tokens, dim, 0, tokens * dim, dim)


def test_hash_rejects_bad_arguments_without_launching(lib):
    buf = ctypes.c_void_p(1 << 20)
    cases = [
        (_tensor(dtype=7), 12, 1, 2),           # dtype
        (_tensor(dim=96), 12, 1, 2),            # head dim
        (_tensor(), 16, 1, 2),                  # n_bits > 15
        (_tensor(), 12, 9, 2),                  # n_probes > FASTAR_MAX_PROBES
        (_tensor(), 12, 0, 2),                  # n_probes < 1
        (_tensor(), 0, 2, 1),                   # two probes need a bit
        (_tensor(), 3, 5, 1),                   # five probes need four bits
        (_tensor(data=(1 << 20) + 2), 12, 1, 1),  # misaligned data
    ]
    for t, bits, probes, want in cases:
        st = lib.fastar_hash(ctypes.byref(t), buf, bits, probes, buf, None, None, buf,
                             1 << 30, None, None)
        assert st == want, (bits, probes, st, lib.fastar_last_error())
    # workspace too small (the index needs it)
    st = lib.fastar_hash(ctypes.byref(_tensor()), buf, 12, 1, buf, buf, buf, buf, 8, None, None)
    assert st == 3
    assert b"workspace" in lib.fastar_last_error()
    # offsets without perm
    st = lib.fastar_hash(ctypes.byref(_tensor()), buf, 12, 1, buf, buf, None, buf, 1 << 30, None, None)
    assert st == 1


def test_hash_multi_rejects_bad_arguments_without_launching(lib):
    buf = ctypes.c_void_p(1 << 20)

    def call(tensors, probes, bits=12, count=None):
        n = len(tensors)
        xp = (ctypes.c_void_p * n)(*[ctypes.addressof(t) for t in tensors])
        pr = (ctypes.c_int * n)(*probes)
        bp = (ctypes.c_void_p * n)(*([buf.value] * n))
        return lib.fastar_hash_multi(n if count is None else count, ctypes.cast(xp, ctypes.c_void_p),
                                     ctypes.cast(pr, ctypes.c_void_p), ctypes.cast(bp, ctypes.c_void_p),
                                     buf, bits, None, None)

    a, b = _tensor(), _tensor(tokens=32)
    assert call([a, b], [1, 1], count=0) == 1            # count < 1
    assert call([a, b, a, b, a], [1] * 5) == 1           # count > 4
    assert call([a, _tensor(dim=64)], [1, 1]) == 1       # dims differ
    assert call([a, _tensor(dtype=0)], [1, 1]) == 1      # dtypes differ
    assert call([a, b], [1, 9]) == 2                     # n_probes
    assert call([a, b], [1, 1], bits=16) == 2            # n_bits


def test_chunk_rejects_bad_arguments_without_launching(lib):
    """fastar_chunk checks every stage's arguments before its first launch:
    each of these calls fails on the host (no GPU here: a launch would fail
    with a HIP status instead)."""
    buf = 1 << 20
    q, k = _tensor(tokens=32), _tensor(tokens=3 * 16)
    cache = fb.FastarCache(2, 128, 64, 16, 12, 1, *([buf] * 9))

    def args(**kw):
        a = dict(q=ctypes.addressof(q), n_probes=1, k_new=ctypes.addressof(k), v_new=ctypes.addressof(k),
                 n_frames=3, planes=buf, n_bits=12, tau=0.9, scale=0.1, cache=ctypes.addressof(cache),
                 q_bucket=buf, q_offsets=buf, q_perm=buf, k_bucket=buf, rep_offsets=buf, rep_perm=buf,
                 out=buf)
        a.update(kw)
        return fb.FastarChunk(**a)

    def call(a, ws_bytes=1 << 30):
        return lib.fastar_chunk(ctypes.byref(a), ctypes.c_void_p(buf), ws_bytes, None, None)

    assert lib.fastar_chunk(None, None, 0, None, None) == 1
    assert call(args(cache=None)) == 1                       # no cache
    assert call(args(n_frames=2)) == 1                       # k_new holds 3 frames
    assert call(args(n_probes=9)) == 2                       # probes
    assert call(args(n_bits=10)) == 1                        # differs from the cache's
    assert call(args(tau=float("inf"))) == 1                 # tau
    assert call(args(scale=float("nan"))) == 1               # scale
    assert call(args(q_perm=None)) == 1                      # the queries' index is required
    assert call(args(prompt_k=ctypes.addressof(k))) == 1     # prompt_k without prompt_v
    qh = _tensor(heads=3, tokens=32)
    assert call(args(q=ctypes.addressof(qh))) == 1           # head counts differ
    assert call(args(), ws_bytes=16) == 3                    # workspace
    assert b"workspace" in lib.fastar_last_error()
    assert lib.fastar_chunk_workspace(ctypes.byref(args())) >= lib.fastar_tempcache_workspace(
        ctypes.byref(cache), 3)


def test_attention_rejects_bad_arguments_without_launching(lib):
    buf = ctypes.c_void_p(1 << 20)
    q, k = _tensor(), _tensor(tokens=32)
    kf = _tensor(dtype=0, tokens=32)
    # mixed dtypes
    st = lib.fastar_bucket_attention(ctypes.byref(q), None, None, 1, ctypes.byref(kf),
                                     ctypes.byref(kf), None, None, None, 0, None, None, 0.1,
                                     buf, None, None)
    assert st == 1
    # bucket mode missing k_perm
    st = lib.fastar_bucket_attention(ctypes.byref(q), buf, buf, 1, ctypes.byref(k), ctypes.byref(k),
                                     None, buf, None, 4, None, None, 0.1, buf, None, None)
    assert st == 1
    # non-finite scale
    st = lib.fastar_bucket_attention(ctypes.byref(q), None, None, 1, ctypes.byref(k), ctypes.byref(k),
                                     None, None, None, 0, None, None, float("nan"), buf, None, None)
    assert st == 1
    # token counts of k and v differ
    st = lib.fastar_bucket_attention(ctypes.byref(q), None, None, 1, ctypes.byref(k), ctypes.byref(q),
                                     None, None, None, 0, None, None, 0.1, buf, None, None)
    assert st == 1


def test_merge_and_prune_reject_bad_arguments(lib):
    buf = 1 << 20
    c = fb.FastarCache(2, 128, 64, 16, 12, 1, *([buf] * 9))
    k = _tensor(tokens=32)
    # k_new must hold n_frames * tokens_per_frame tokens
    st = lib.fastar_tempcache_merge(ctypes.byref(c), ctypes.byref(k), ctypes.byref(k), ctypes.c_void_p(buf),
                                    3, 0.9, None, None, None, ctypes.c_void_p(buf), 1 << 30, None, None)
    assert st == 1
    # tau must be finite
    st = lib.fastar_tempcache_merge(ctypes.byref(c), ctypes.byref(k), ctypes.byref(k), ctypes.c_void_p(buf),
                                    2, float("inf"), None, None, None, ctypes.c_void_p(buf), 1 << 30, None, None)
    assert st == 1
    # capacity below one frame
    c2 = fb.FastarCache(2, 128, 8, 16, 12, 1, *([buf] * 9))
    st = lib.fastar_tempcache_merge(ctypes.byref(c2), ctypes.byref(k), ctypes.byref(k), ctypes.c_void_p(buf),
                                    2, 0.9, None, None, None, ctypes.c_void_p(buf), 1 << 30, None, None)
    assert st == 1
    # dtype mismatch between cache and keys
    kf = _tensor(dtype=0, tokens=32)
    st = lib.fastar_tempcache_merge(ctypes.byref(c), ctypes.byref(kf), ctypes.byref(kf), ctypes.c_void_p(buf),
                                    2, 0.9, None, None, None, ctypes.c_void_p(buf), 1 << 30, None, None)
    assert st == 1
    # prune: bits out of range, probes out of range
    p = ctypes.c_void_p(buf)
    assert lib.fastar_prune_prompt(p, 2, 10, 1, p, 5, 16, p, p, p, None) == 2
    assert lib.fastar_prune_prompt(p, 2, 10, 0, p, 5, 8, p, p, p, None) == 2
    assert lib.fastar_prune_prompt(p, 2, 10, 1, p, 5, 8, p, p, None, None) == 1


def test_workspace_queries_scale_with_size(lib):
    a = lib.fastar_hash_workspace(12, 4680, 12, 1)
    b = lib.fastar_hash_workspace(24, 8192, 14, 2)
    assert 0 < a < b
    assert lib.fastar_bucket_index_workspace(12, 1000) >= 16 * 12 * 1000
    c = fb.FastarCache(12, 128, 20000, 1560, 12, 1, *([0] * 9))
    assert lib.fastar_tempcache_workspace(ctypes.byref(c), 3) >= 16 * 12 * 20000


def test_noalloc_chunk_rejects_oversized_workspace_without_launching(lib):
    # a chunk whose workspace exceeds the allocation-free scratch is refused
    # on the host, before any HIP call
    buf = 1 << 20
    H, T, cap = 24, 2048, 1 << 20
    c = fb.FastarCache(H, 128, cap, T, 14, 1, *([buf] * 9))
    q = fb.FastarTensor(buf, 1, H, 8192, 128, 0, 8192 * 128, 128)
    k = fb.FastarTensor(buf, 1, H, 4 * T, 128, 0, 4 * T * 128, 128)
    a = fb.FastarChunk(ctypes.addressof(q), 2, ctypes.addressof(k), ctypes.addressof(k), 4, None,
                       None, buf, 14, 0.999, 0.088, ctypes.addressof(c), *([buf] * 9))
    need = lib.fastar_chunk_workspace(ctypes.byref(a))
    assert need > fb.NOALLOC_SCRATCH_BYTES
    assert lib.fastar_chunk_noalloc(ctypes.byref(a), None, None) == 3
    assert b"scratch" in lib.fastar_last_error()


def test_noalloc_scratch_size_matches_header():
    m = re.search(r"#define FASTAR_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == fb.NOALLOC_SCRATCH_BYTES


def test_recall_rejects_bad_arguments_without_launching(lib):
    buf = ctypes.c_void_p(1 << 20)
    # stats and n_keys are required; exactly one of k_offsets / n_retained
    assert lib.fastar_attention_recall(buf, buf, 2, 10, buf, 1, buf, 4, None, buf, None, None, None) == 1
    assert lib.fastar_attention_recall(buf, buf, 2, 10, buf, 1, buf, 4, buf, buf, None, buf, None) == 1
    assert lib.fastar_attention_recall(buf, buf, 2, 10, None, 1, None, 4, None, buf, None, buf, None) == 1
    assert lib.fastar_attention_recall(buf, buf, 2, 10, buf, 9, buf, 4, None, buf, None, buf, None) == 2
    assert lib.fastar_attention_recall(None, buf, 2, 10, None, 1, None, 0, buf, buf, None, buf, None) == 1
    assert lib.fastar_attention_recall(None, None, 0, 10, None, 1, None, 0, None, None, None, None, None) == 0


def test_merge_options_rejected_without_launching(lib):
    buf = 1 << 20
    c = fb.FastarCache(2, 128, 64, 16, 12, 1, *([buf] * 9))
    k = _tensor(tokens=16)
    for match, bits, want in [(7, 8, 2), (1, 9, 2), (1, 1, 2)]:
        o = fb.FastarMergeOpts(match, bits)
        st = lib.fastar_tempcache_merge_ex(ctypes.byref(c), ctypes.byref(k), ctypes.byref(k),
                                           ctypes.c_void_p(buf), 1, 0.9, ctypes.byref(o), None, None,
                                           None, ctypes.c_void_p(buf), 1 << 30, None, None)
        assert st == want, (match, bits)
    # an unknown representative; mean and medoid without (or with a
    # misaligned) key-sum buffer
    for rep, k_sum, want in [(3, None, 2), (1, None, 1), (2, None, 1), (1, buf + 8, 1)]:
        c.k_sum = k_sum
        o = fb.FastarMergeOpts(0, 8, rep)
        st = lib.fastar_tempcache_merge_ex(ctypes.byref(c), ctypes.byref(k), ctypes.byref(k),
                                           ctypes.c_void_p(buf), 1, 0.9, ctypes.byref(o), None, None,
                                           None, ctypes.c_void_p(buf), 1 << 30, None, None)
        assert st == want, (rep, k_sum)
    c.k_sum = None
    assert lib.fastar_tempcache_workspace_ex(ctypes.byref(c), 1, ctypes.byref(fb.FastarMergeOpts(1, 8))) > \
        lib.fastar_tempcache_workspace(ctypes.byref(c), 1)
    assert lib.fastar_scalar_codes(ctypes.byref(k), 1, ctypes.c_void_p(buf), ctypes.c_void_p(buf), None) == 2
    assert lib.fastar_scalar_codes(ctypes.byref(k), 8, None, ctypes.c_void_p(buf), None) == 1


def test_tables_calls_reject_bad_arguments_without_launching(lib):
    buf = ctypes.c_void_p(1 << 20)
    q, k = _tensor(), _tensor(tokens=32)

    def attn(n_tables, probes, k_bucket=buf, bits=6):
        return lib.fastar_bucket_attention_tables(ctypes.byref(q), n_tables, buf, buf, probes, ctypes.byref(k),
                                                  ctypes.byref(k), None, k_bucket, buf, buf, bits, 0.1, buf,
                                                  None, None, None)
    assert attn(0, 1) == 2 and attn(5, 1) == 2           # tables outside [1, FASTAR_MAX_TABLES]
    assert attn(3, 3) == 2                               # 9 (table, probe) entries
    assert attn(2, 2, k_bucket=None) == 1                # several tables need the keys' buckets
    assert attn(1, 4, bits=2) == 1                       # four probes need three bits

    def prune(n_tables, probes=1):
        return lib.fastar_prune_prompt_tables(buf, n_tables, 2, 16, probes, buf, 32, 6, buf, buf, buf, None)
    assert prune(0) == 2 and prune(5) == 2 and prune(2, 9) == 2
    assert lib.fastar_attention_recall_counts(buf, buf, 2, 16, None, buf, None, buf, None) == 1
    assert lib.fastar_attention_recall_counts(buf, buf, 2, 16, buf, None, None, buf, None) == 1

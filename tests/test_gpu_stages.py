"""Stage-isolated GPU parity: each libfastar call against the CPU oracle on the
same seeded inputs.  Integers bit-exact; floats within max-abs 2e-2 (bf16)
or 1e-5 (fp32)."""

import numpy as np
import pytest
import torch

import oracle
from synth import gaussian, round_to_dtype

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_compressed_attention_amd as m
    m.library()
    return m


def dev_tensor(a, dtype):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device="cuda").to(TDT[dtype])


def i32(a):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.int32, device="cuda")


def near_plane_rows(n, d, planes, seed, dtype):
    """Rows projected onto a random hyperplane, so that x . r_j is ~0 before rounding."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    j = rng.integers(0, planes.shape[0], n)
    r = planes[j].astype(np.float64)
    x = x - (np.sum(x * r, axis=1) / np.sum(r * r, axis=1))[:, None] * r
    return round_to_dtype(x, dtype)


# ---------------------------------------------------------------------------
# hash + index
# ---------------------------------------------------------------------------
HASH_CASES = [
    # dtype, heads, n, d, bits, probes
    ("bf16", 3, 1000, 128, 12, 1),
    ("bf16", 2, 777, 128, 14, 2),
    ("bf16", 2, 333, 64, 6, 1),
    ("bf16", 1, 17, 128, 15, 2),
    ("bf16", 2, 250, 128, 0, 1),
    ("bf16", 1, 1, 64, 3, 2),
    ("f32", 1, 256, 64, 6, 1),
    ("f32", 2, 301, 128, 10, 2),
]


@pytest.mark.parametrize("dtype,H,n,d,b,P", HASH_CASES)
def test_hash_and_index_match_oracle(fa, dtype, H, n, d, b, P):
    seed = 1000 + n + b
    planes = gaussian((b, d), seed, dtype) if b else np.zeros((1, d), np.float32)
    x = gaussian((H, n, d), seed + 1, dtype)
    # a third of the rows sit on a hyperplane to exercise the fallback paths
    if b:
        for h in range(H):
            x[h, ::3] = near_plane_rows(x[h, ::3].shape[0], d, planes, seed + 2 + h, dtype)
    x[:, 0] = 0.0  # the zero vector: bucket 0, probe flips plane 0
    if b:
        # x . r_j = r_j1 r_j0 - r_j0 r_j1 + r_j3 r_j2 - r_j2 r_j3 = 0 exactly, with
        # nonzero terms: only exact arithmetic can tell that bit j is 0
        for i in range(1, n, 7):
            jj = i % b
            x[:, i] = 0.0
            x[:, i, 0], x[:, i, 1] = planes[jj, 1], -planes[jj, 0]
            x[:, i, 2], x[:, i, 3] = planes[jj, 3], -planes[jj, 2]
    diag = fa.new_diag()
    ids, off, perm = fa.fastar_hash(dev_tensor(x, dtype), dev_tensor(planes, dtype), b, P, diag=diag)
    torch.cuda.synchronize()
    ids, off, perm = ids.cpu().numpy(), off.cpu().numpy(), perm.cpu().numpy()
    for h in range(H):
        ref = oracle.simhash(x[h], planes[:b], P)
        assert np.array_equal(ids[h], ref), f"head {h}: {np.sum(ids[h] != ref)} ids differ"
        r_off, r_perm = oracle.bucket_index(ref, b)
        assert np.array_equal(off[h], r_off)
        assert np.array_equal(perm[h], r_perm)
    dg = diag.cpu().numpy()
    assert dg[3] == 0, f"unresolved decisions: {dg}"
    if b and n > 1:
        # (row 0 is the zero row, which needs no float64 pass)
        assert dg[0] > 0, "near-plane rows should have taken the float64 path"
    if b and n > 1:
        assert dg[1] > 0, "exactly orthogonal rows should have needed exact signs"


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_hash_two_probe_ties_and_near_ties(fa, dtype, d):
    """Second probes of rows whose two nearest hyperplanes lie at exactly the
    same distance (planes 2 = s e0 and 5 = s e1, rows with x0 = x1 = 2^-6: the
    smaller index wins, decided in integer arithmetic) or 2^-25 apart
    relatively (planes 7 = s e2 and 8 = s (e3 + 2^-12 e4), rows with x2 = x3
    = 2^-6: plane 8 is nearer, below float32's bound and decided in float64):
    ids equal the oracle's and no decision is left unresolved."""
    print(f"hash ties {dtype} d{d}", flush=True)
    b, n = 10, 600
    planes = gaussian((b, d), 112, dtype)
    s = 0.75
    for j in (2, 5, 7, 8):
        planes[j] = 0.0
    planes[2, 0] = planes[5, 1] = planes[7, 2] = planes[8, 3] = s
    planes[8, 4] = s * 2.0 ** -12
    x = gaussian((1, n, d), 113, dtype)
    a = 2.0 ** -6
    x[0, 0::2, 0] = x[0, 0::2, 1] = a          # exact ties
    x[0, 0::2, 2] = x[0, 0::2, 3] = 1.0
    x[0, 1::2, 2] = x[0, 1::2, 3] = a          # near ties
    x[0, 1::2, 4] = 0.0
    x[0, 1::2, 0] = x[0, 1::2, 1] = 1.0
    for P in (2, 3):
        diag = fa.new_diag()
        ids, _, _ = fa.fastar_hash(dev_tensor(x, dtype), dev_tensor(planes, dtype), b, P, diag=diag)
        torch.cuda.synchronize()
        ref = oracle.simhash(x[0], planes, P)
        got = ids.cpu().numpy()[0]
        assert np.array_equal(got, ref), f"P={P}: {np.sum(np.any(got != ref, axis=1))} rows differ"
        dg = diag.cpu().numpy()
        assert dg[3] == 0 and dg[0] > 0, dg.tolist()


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_hash_multi_matches_oracle(fa, dtype, d):
    """Queries (two probes), keys and prompt keys of different head and row
    counts in one call: each tensor's ids equal the oracle's, and an empty
    tensor in the list is skipped."""
    b = 12
    planes = gaussian((b, d), 41, dtype)
    shapes = [(3, 1000, 2), (3, 2300, 1), (2, 77, 1), (3, 0, 1)]
    xs = []
    for i, (H, n, _) in enumerate(shapes):
        x = gaussian((H, n, d), 50 + i, dtype)
        if n:
            for h in range(H):
                x[h, ::4] = near_plane_rows(x[h, ::4].shape[0], d, planes, 60 + 7 * i + h, dtype)
        xs.append(x)
    diag = fa.new_diag()
    outs = fa.fastar_hash_multi([dev_tensor(x, dtype) for x in xs], dev_tensor(planes, dtype), b,
                                [P for _, _, P in shapes], diag=diag)
    torch.cuda.synchronize()
    for x, (H, n, P), ids in zip(xs, shapes, outs):
        ids = ids.cpu().numpy()
        assert ids.shape == (H, n, P)
        for h in range(H):
            assert np.array_equal(ids[h], oracle.simhash(x[h], planes, P)), (H, n, P, h)
    dg = diag.cpu().numpy()
    assert dg[3] == 0 and dg[0] > 0


def test_hash_is_deterministic(fa):
    x = dev_tensor(gaussian((4, 3000, 128), 7, "bf16"), "bf16")
    planes = dev_tensor(gaussian((14, 128), 8, "bf16"), "bf16")
    a = fa.fastar_hash(x, planes, 14, 2)
    b = fa.fastar_hash(x, planes, 14, 2)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_hash_strided_input(fa):
    base = gaussian((2, 300, 256), 9, "bf16")
    x = dev_tensor(base, "bf16")[:, :, 64:192]          # token stride 256, dim 128
    planes = gaussian((12, 128), 10, "bf16")
    ids, _, _ = fa.fastar_hash(x, dev_tensor(planes, "bf16"), 12, 1, with_index=False)
    for h in range(2):
        assert np.array_equal(ids[h].cpu().numpy(), oracle.simhash(base[h, :, 64:192], planes, 1))


@pytest.mark.parametrize("n,b,P", [(5000, 12, 1), (4096, 14, 2), (100, 3, 1), (0, 4, 1), (65535, 12, 1),
                                   (3100, 3, 1), (12289, 9, 1), (1537, 12, 1),
                                   # the counting pass by bucket ranges at 13-15 bits, two
                                   # probes, and 32-bit counters past 65535 items
                                   (8192, 14, 2), (32768, 14, 1), (1000, 14, 1), (1, 14, 2),
                                   (20000, 13, 2), (70000, 13, 1), (93600, 12, 1), (66000, 3, 1),
                                   (5000, 15, 1), (70000, 14, 1), (65535, 15, 2), (70000, 15, 1),
                                   (40, 13, 1),
                                   # range mode: every wave's slice in registers (two tiles,
                                   # 1024 ids) and one id past it
                                   (16384, 14, 1), (16385, 14, 2),
                                   # the radix fallback
                                   (3000, 2, 2)])
def test_bucket_index_of_given_ids(fa, n, b, P):
    rng = np.random.default_rng(n + b)
    H = 3
    first = rng.integers(0, 1 << b, (H, n))
    if P == 2:
        j = rng.integers(0, b, (H, n))
        ids = np.stack([first, first ^ (1 << j)], axis=2)
    else:
        ids = first[:, :, None]
    n_valid = np.array([n, n // 2, 0], dtype=np.int32)
    off, perm = fa.fastar_bucket_index(i32(ids), b, n_valid=i32(n_valid))
    torch.cuda.synchronize()
    off, perm = off.cpu().numpy(), perm.cpu().numpy()
    for h in range(H):
        nv = n_valid[h]
        r_off, r_perm = oracle.bucket_index(ids[h, :nv], b)
        assert np.array_equal(off[h], r_off)
        assert np.array_equal(perm[h, :nv], r_perm)


@pytest.mark.parametrize("n,b", [(70000, 12), (65535, 14), (9000, 13), (66000, 15)])
def test_bucket_index_one_full_bucket(fa, n, b):
    # every item in one bucket: its count reaches n (past 16 bits for 70000)
    H = 2
    ids = np.full((H, n, 1), 5, dtype=np.int64)
    ids[1, ::2, 0] = 7
    off, perm = fa.fastar_bucket_index(i32(ids), b)
    torch.cuda.synchronize()
    off, perm = off.cpu().numpy(), perm.cpu().numpy()
    for h in range(H):
        r_off, r_perm = oracle.bucket_index(ids[h], b)
        assert np.array_equal(off[h], r_off)
        assert np.array_equal(perm[h], r_perm)


# ---------------------------------------------------------------------------
# prune
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("b,P,nq,npr", [(10, 1, 4680, 512), (14, 2, 3000, 512), (6, 1, 256, 64),
                                         (4, 1, 10, 2500), (8, 2, 0, 300)])
def test_prune_matches_oracle(fa, b, P, nq, npr):
    rng = np.random.default_rng(b * 100 + nq)
    H = 3
    q_ids = rng.integers(0, 1 << b, (H, nq, P))
    p_ids = rng.integers(0, 1 << b, (H, npr))
    keep, kept, n_kept = fa.fastar_prune_prompt(i32(q_ids), i32(p_ids), b)
    torch.cuda.synchronize()
    keep, kept, n_kept = keep.cpu().numpy(), kept.cpu().numpy(), n_kept.cpu().numpy()
    for h in range(H):
        r_keep, r_kept = oracle.prune_prompt(q_ids[h], p_ids[h])
        assert np.array_equal(keep[h].astype(bool), r_keep)
        assert n_kept[h] == r_kept.size
        assert np.array_equal(kept[h, :n_kept[h]], r_kept)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _attn_case(dtype, H, nq, nk, d, b, P, seed, bias=True):
    rng = np.random.default_rng(seed)
    q = gaussian((H, nq, d), seed + 1, dtype)
    k = gaussian((H, nk, d), seed + 2, dtype)
    v = gaussian((H, nk, d), seed + 3, dtype)
    first = rng.integers(0, 1 << b, (H, nq))
    if P == 2:
        j = rng.integers(0, b, (H, nq))
        q_ids = np.stack([first, first ^ (1 << j)], axis=2)
    else:
        q_ids = first[:, :, None]
    k_ids = rng.integers(0, 1 << b, (H, nk))
    kb = np.log(rng.integers(1, 6, (H, nk)).astype(np.float64)).astype(np.float32) if bias else None
    return q, k, v, q_ids, k_ids, kb


ATTN_CASES = [
    # dtype, H, nq, nk, d, bits, probes
    ("bf16", 2, 1000, 3000, 128, 4, 1),     # many 32-key chunks per bucket, ragged tails
    ("bf16", 2, 777, 2000, 128, 6, 2),
    ("bf16", 1, 300, 5000, 64, 2, 1),
    ("bf16", 3, 100, 90, 128, 8, 1),        # many empty buckets
    ("bf16", 1, 50, 1, 128, 1, 2),
    ("bf16", 2, 900, 1800, 64, 7, 2),        # d = 64 with two probes
    ("f32", 1, 256, 500, 64, 6, 1),
    ("f32", 2, 200, 400, 128, 5, 2),
]


@pytest.mark.parametrize("dtype,H,nq,nk,d,b,P", ATTN_CASES)
def test_bucket_attention_matches_oracle(fa, dtype, H, nq, nk, d, b, P):
    q, k, v, q_ids, k_ids, kb = _attn_case(dtype, H, nq, nk, d, b, P, seed=nq + nk + b)
    tq = dev_tensor(q, dtype)
    q_off, q_perm = fa.fastar_bucket_index(i32(q_ids), b)
    k_off, k_perm = fa.fastar_bucket_index(i32(k_ids[:, :, None]), b)
    out, lse = fa.fastar_bucket_attention(tq, dev_tensor(k, dtype), dev_tensor(v, dtype),
                                          q_bucket=i32(q_ids), q_perm=q_perm,
                                          key_bias=torch.tensor(kb, device="cuda"),
                                          k_offsets=k_off, k_perm=k_perm, n_bits=b)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for h in range(H):
        o_ref, lse_ref = oracle.bucket_attention(q[h], q_ids[h], k[h], v[h], k_ids[h], bias=kb[h])
        err = np.max(np.abs(out[h] - o_ref))
        assert err <= TOL[dtype], f"head {h}: max|err| {err}"
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse[h]), fin)
        assert np.all(lse[h][~fin] == -np.inf)
        assert np.max(np.abs(lse[h][fin] - lse_ref[fin]), initial=0) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_bucket_attention_equal_probes_count_keys_once(fa, dtype, d):
    # caller-supplied ids with both probes equal name one key set: its keys
    # count once (the oracle takes the set of probe buckets)
    H, nq, nk, b = 2, 300, 800, 4
    q, k, v, q_ids, k_ids, kb = _attn_case(dtype, H, nq, nk, d, b, 2, seed=91)
    q_ids[:, ::3, 1] = q_ids[:, ::3, 0]
    q_off, q_perm = fa.fastar_bucket_index(i32(q_ids), b)
    k_off, k_perm = fa.fastar_bucket_index(i32(k_ids[:, :, None]), b)
    out, lse = fa.fastar_bucket_attention(dev_tensor(q, dtype), dev_tensor(k, dtype),
                                          dev_tensor(v, dtype), q_bucket=i32(q_ids), q_perm=q_perm,
                                          key_bias=torch.tensor(kb, device="cuda"),
                                          k_offsets=k_off, k_perm=k_perm, n_bits=b)
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    for h in range(H):
        o_ref, lse_ref = oracle.bucket_attention(q[h], q_ids[h], k[h], v[h], k_ids[h], bias=kb[h])
        assert np.max(np.abs(out[h] - o_ref)) <= TOL[dtype]
        fin = np.isfinite(lse_ref)
        assert np.max(np.abs(lse[h][fin] - lse_ref[fin]), initial=0) <= TOL[dtype]


@pytest.mark.parametrize("P", [1, 2])
def test_bucket_attention_any_row_order(fa, P):
    # q_perm in a random order instead of the index's bucket order: a
    # workgroup then meets a bucket in several runs of rows; every row must
    # still see exactly its own bucket's keys
    H, nq, nk, d, b = 2, 700, 1500, 128, 5
    q, k, v, q_ids, k_ids, kb = _attn_case("bf16", H, nq, nk, d, b, P, seed=77)
    rng = np.random.default_rng(78)
    perm = np.stack([rng.permutation(nq) for _ in range(H)]).astype(np.int32)
    k_off, k_perm = fa.fastar_bucket_index(i32(k_ids[:, :, None]), b)
    out, lse = fa.fastar_bucket_attention(dev_tensor(q, "bf16"), dev_tensor(k, "bf16"),
                                          dev_tensor(v, "bf16"), q_bucket=i32(q_ids),
                                          q_perm=i32(perm), key_bias=torch.tensor(kb, device="cuda"),
                                          k_offsets=k_off, k_perm=k_perm, n_bits=b)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    for h in range(H):
        o_ref, _ = oracle.bucket_attention(q[h], q_ids[h], k[h], v[h], k_ids[h], bias=kb[h])
        assert np.max(np.abs(out[h] - o_ref)) <= TOL["bf16"], f"head {h}"


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_list_and_dense_modes_match_oracle(fa, dtype, d):
    H, nq, nk = 2, 333, 512
    q = gaussian((H, nq, d), 21, dtype)
    k = gaussian((H, nk, d), 22, dtype)
    v = gaussian((H, nk, d), 23, dtype)
    rng = np.random.default_rng(24)
    keep = rng.random((H, nk)) < 0.12
    keep[1] = False                                   # head 1 keeps nothing
    kept = np.zeros((H, nk), np.int64)
    n_kept = keep.sum(axis=1)
    for h in range(H):
        kept[h, :n_kept[h]] = np.nonzero(keep[h])[0]
    tq, tk, tv = dev_tensor(q, dtype), dev_tensor(k, dtype), dev_tensor(v, dtype)
    o_list, l_list = fa.fastar_bucket_attention(tq, tk, tv, key_list=i32(kept), n_key_list=i32(n_kept))
    o_dense, _ = fa.fastar_bucket_attention(tq, tk, tv)
    torch.cuda.synchronize()
    for h in range(H):
        r_list, _ = oracle.cross_attention(q[h], k[h], v[h], kept[h, :n_kept[h]])
        r_dense, _ = oracle.dense_attention(q[h], k[h], v[h])
        assert np.max(np.abs(o_list[h].float().cpu().numpy() - r_list)) <= TOL[dtype]
        assert np.max(np.abs(o_dense[h].float().cpu().numpy() - r_dense)) <= TOL[dtype]
    assert torch.all(o_list[1] == 0) and torch.all(torch.isinf(l_list[1]))


@pytest.mark.parametrize("d", [128, 64])
def test_list_mode_long_lists_bias_and_lse(fa, d):
    """bf16 list mode against the oracle's dense attention over the listed keys
    (with their + ln m biases), outputs and lse: lists shorter than, equal to
    and longer than the 256 keys a workgroup keeps resident (the longer ones
    pass through in windows), in any order and with a repeated key (it counts
    twice, as in the list), over rows that end inside a step."""
    print(f"list d{d}", flush=True)
    H, nq, nk = 4, 600, 700
    q = gaussian((H, nq, d), 91, "bf16")
    k = gaussian((H, nk, d), 92, "bf16")
    v = gaussian((H, nk, d), 93, "bf16")
    rng = np.random.default_rng(94)
    kb = np.log(rng.integers(1, 6, (H, nk)).astype(np.float64)).astype(np.float32)
    lens = [300, 256, 257, 61]
    lists = np.zeros((H, nk), np.int64)
    for h, n in enumerate(lens):
        lists[h, :n] = rng.permutation(nk)[:n]
    lists[3, 5] = lists[3, 9]  # a repeated key
    out, lse = fa.fastar_bucket_attention(dev_tensor(q, "bf16"), dev_tensor(k, "bf16"), dev_tensor(v, "bf16"),
                                          key_bias=torch.tensor(kb, device="cuda"), key_list=i32(lists),
                                          n_key_list=i32(np.array(lens)))
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    for h, n in enumerate(lens):
        idx = lists[h, :n]
        o_ref, lse_ref = oracle.dense_attention(q[h], k[h][idx], v[h][idx], bias=kb[h][idx])
        assert np.max(np.abs(out[h] - o_ref)) <= TOL["bf16"], f"head {h}"
        assert np.max(np.abs(lse[h] - lse_ref)) <= TOL["bf16"], f"head {h}"


def test_attention_lemma_duplicates_on_gpu(fa):
    # Lemma 5.1 on the GPU: attention over the merged representatives with
    # the bf16 group means and + ln m equals the oracle's dense attention
    # over the raw duplicated keys (float64), within the bf16 tolerance; so
    # does the GPU's dense attention over the raw keys
    rng = np.random.default_rng(31)
    g, d = 200, 128
    reps = gaussian((1, g, d), 32, "bf16")
    m = rng.integers(1, 5, g)
    keys = np.repeat(reps, m, axis=1)
    vals = gaussian((1, keys.shape[1], d), 33, "bf16")
    owner = np.repeat(np.arange(g), m)
    means = round_to_dtype(np.stack([vals[0, owner == t].mean(axis=0) for t in range(g)])[None], "bf16")
    q = gaussian((1, 256, d), 34, "bf16")
    o_raw, _ = fa.fastar_bucket_attention(dev_tensor(q, "bf16"), dev_tensor(keys, "bf16"),
                                          dev_tensor(vals, "bf16"))
    o_m, _ = fa.fastar_bucket_attention(dev_tensor(q, "bf16"), dev_tensor(reps, "bf16"),
                                        dev_tensor(means, "bf16"),
                                        key_bias=torch.tensor(np.log(m)[None].astype(np.float32), device="cuda"))
    torch.cuda.synchronize()
    ref, _ = oracle.dense_attention(q[0], keys[0], vals[0])
    assert np.max(np.abs(o_m[0].float().cpu().numpy() - ref)) <= TOL["bf16"]
    assert np.max(np.abs(o_raw[0].float().cpu().numpy() - ref)) <= TOL["bf16"]
    # without the bias the identity fails by far more than the tolerance
    o_nb, _ = fa.fastar_bucket_attention(dev_tensor(q, "bf16"), dev_tensor(reps, "bf16"),
                                         dev_tensor(means, "bf16"))
    torch.cuda.synchronize()
    assert np.max(np.abs(o_nb[0].float().cpu().numpy() - ref)) > 5 * TOL["bf16"]


# ---------------------------------------------------------------------------
# TempCache merge
# ---------------------------------------------------------------------------
def _frames(H, F, T, d, seed, dtype, carry=0.75, noise=0.02):
    rng = np.random.default_rng(seed)
    k = np.empty((H, F, T, d))
    k[:, 0] = rng.standard_normal((H, T, d))
    for f in range(1, F):
        keep = rng.random((H, T)) < carry
        k[:, f] = np.where(keep[..., None], k[:, f - 1] + noise * rng.standard_normal((H, T, d)),
                           rng.standard_normal((H, T, d)))
    v = rng.standard_normal((H, F, T, d))
    return round_to_dtype(k, dtype), round_to_dtype(v, dtype)


MERGE_CASES = [
    # dtype, H, F, T, d, bits, tau, frames per call
    ("f32", 1, 4, 256, 64, 6, 0.9, 1),
    ("bf16", 2, 5, 300, 128, 8, 0.999, 2),
    ("bf16", 2, 4, 200, 128, 0, 0.99, 4),
    ("bf16", 1, 3, 700, 64, 10, 0.5, 3),
    # 14 bits: the match workgroups find their own ranges
    ("bf16", 2, 3, 300, 64, 14, 0.9, 3),
]


@pytest.mark.parametrize("dtype,H,F,T,d,b,tau,fpc", MERGE_CASES)
def test_tempcache_merge_matches_oracle(fa, dtype, H, F, T, d, b, tau, fpc):
    k, v = _frames(H, F, T, d, seed=F * T + b, dtype=dtype)
    planes = gaussian((max(b, 1), d), 40 + b, dtype)
    cap = F * T
    cache = fa.TempCache(H, d, cap, T, b, TDT[dtype], "cuda")
    diag = fa.new_diag()
    tplanes = dev_tensor(planes, dtype)
    refs = [oracle.TempCacheOracle(d, dtype) for _ in range(H)]
    for f0 in range(0, F, fpc):
        f1 = min(F, f0 + fpc)
        kk = np.ascontiguousarray(k[:, f0:f1].reshape(H, -1, d))
        vv = np.ascontiguousarray(v[:, f0:f1].reshape(H, -1, d))
        tk = dev_tensor(kk, dtype)
        ids, _, _ = fa.fastar_hash(tk, tplanes, b, 1, with_index=False)
        gon = torch.empty(H, kk.shape[1], dtype=torch.int32, device="cuda")
        rep_off, rep_perm = fa.fastar_tempcache_merge(cache, tk, dev_tensor(vv, dtype),
                                                      ids[:, :, 0].contiguous(), f1 - f0, tau,
                                                      group_of_new=gon, diag=diag)
        torch.cuda.synchronize()
        gon = gon.cpu().numpy()
        for h in range(H):
            ref_groups = []
            for f in range(f0, f1):
                kid = oracle.simhash(k[h, f], planes[:b], 1)[:, 0]
                ref_groups.append(refs[h].merge_frame(k[h, f], v[h, f], kid, tau))
            assert np.array_equal(gon[h], np.concatenate(ref_groups)), f"frames {f0}-{f1} head {h}"
    for h in range(H):
        r = refs[h]
        G = r.n_groups
        assert int(cache.n_groups[h]) == G
        assert np.array_equal(cache.count[h, :G].cpu().numpy(), r.count)
        assert np.array_equal(cache.rep_bucket[h, :G].cpu().numpy(), r.rep_bucket)
        assert np.array_equal(cache.rep_k[h, :G].float().cpu().numpy(), r.rep_k)
        assert np.array_equal(cache.frontier[h].cpu().numpy(), r.frontier)
        assert np.max(np.abs(cache.v_mean[h, :G].float().cpu().numpy() - r.v_mean)) <= TOL[dtype]
        assert np.max(np.abs(cache.log_count[h, :G].cpu().numpy() - r.log_count)) <= 1e-5
        r_off, r_perm = oracle.bucket_index(r.rep_bucket, b)
        assert np.array_equal(rep_off[h].cpu().numpy(), r_off)
        assert np.array_equal(rep_perm[h, :G].cpu().numpy(), r_perm)
    assert diag[3].item() == 0 and diag[4].item() == 0, diag.tolist()


@pytest.mark.parametrize("fpc", [1, 3])
def test_tempcache_overflow_sets_status_word(fa, fpc):
    # no merges (tau > 1) into a cache of 2.5 frames: merging 3 frames (one
    # call each, or all in one call) overflows.  The status word reports it
    # with no diag buffer; groups up to the capacity are numbered as usual
    # and the rest are dropped (-1); clearing resets the word.
    H, T, d = 2, 64, 64
    F = 3
    k, v = _frames(H, F, T, d, seed=7, dtype="bf16")
    cap = 2 * T + T // 2
    cache = fa.TempCache(H, d, cap, T, 4, torch.bfloat16, "cuda")
    planes = dev_tensor(gaussian((4, d), 8, "bf16"), "bf16")
    assert cache.status_code() == 0
    groups = []
    for f0 in range(0, F, fpc):
        kk = np.ascontiguousarray(k[:, f0:f0 + fpc].reshape(H, -1, d))
        vv = np.ascontiguousarray(v[:, f0:f0 + fpc].reshape(H, -1, d))
        tk = dev_tensor(kk, "bf16")
        ids, _, _ = fa.fastar_hash(tk, planes, 4, 1, with_index=False)
        gon = torch.empty(H, kk.shape[1], dtype=torch.int32, device="cuda")
        fa.fastar_tempcache_merge(cache, tk, dev_tensor(vv, "bf16"), ids[:, :, 0].contiguous(),
                                  kk.shape[1] // T, 1.5, group_of_new=gon)
        groups.append(gon)
        if f0 + fpc <= 2:
            assert cache.status_code() == 0, "no overflow within the capacity"
    assert cache.status_code() == 5
    assert cache.status_code(clear=True) == 5
    assert cache.status_code() == 0
    g = torch.cat(groups, 1).cpu().numpy()
    for h in range(H):
        assert np.array_equal(g[h, :cap], np.arange(cap))
        assert np.all(g[h, cap:] == -1)
        assert int(cache.n_groups[h]) == cap


def test_tempcache_capacity_overflow_is_reported(fa):
    # no merges (tau > 1): the second frame does not fit a one-frame cache
    H, T, d = 1, 64, 64
    k, v = _frames(H, 2, T, d, seed=5, dtype="f32")
    cache = fa.TempCache(H, d, T + 10, T, 4, torch.float32, "cuda")
    diag = fa.new_diag()
    planes = dev_tensor(gaussian((4, d), 6), "f32")
    gon = torch.empty(H, T, dtype=torch.int32, device="cuda")
    for f in range(2):
        tk = dev_tensor(np.ascontiguousarray(k[:, f]), "f32")
        ids, _, _ = fa.fastar_hash(tk, planes, 4, 1, with_index=False)
        fa.fastar_tempcache_merge(cache, tk, dev_tensor(np.ascontiguousarray(v[:, f]), "f32"),
                                  ids[:, :, 0].contiguous(), 1, 1.5, group_of_new=gon, diag=diag)
    torch.cuda.synchronize()
    assert int(cache.n_groups[0]) == T + 10
    assert diag[4].item() == T - 10
    g = gon[0].cpu().numpy()
    assert np.array_equal(g[:10], T + np.arange(10)) and np.all(g[10:] == -1)


def test_dense_one_bucket_full_size_sampled(fa):
    # the one-bucket measurement's size and launch (12 heads, 4680 queries,
    # 23,400 keys, d = 128, bf16, dense mode): sampled rows against the oracle
    H, nq, nk, d = 12, 4680, 23400, 128
    q, k, v = gaussian((H, nq, d), 501, "bf16"), gaussian((H, nk, d), 502, "bf16"), \
        gaussian((H, nk, d), 503, "bf16")
    out, lse = fa.fastar_bucket_attention(dev_tensor(q, "bf16"), dev_tensor(k, "bf16"),
                                          dev_tensor(v, "bf16"))
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    rows = np.array([0, 1, 63, 64, 2047, 4095, 4616, 4679])
    for h in (0, 5, 11):
        o_ref, lse_ref = oracle.dense_attention(q[h][rows], k[h], v[h])
        assert np.max(np.abs(out[h][rows] - o_ref)) <= TOL["bf16"], f"head {h}"
        assert np.max(np.abs(lse[h][rows] - lse_ref)) <= TOL["bf16"], f"head {h}"

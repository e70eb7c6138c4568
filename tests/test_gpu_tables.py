"""Multi-probe SimHash and multi-table LSH on the GPU against the oracle:
hash ids and indexes bit for bit, AnnSA over the union of the tables'
buckets element by element (and its retained counts exactly), AnnCA's
multi-table prune bit for bit, recall from per-query counts."""

import numpy as np
import pytest
import torch

import oracle
from synth import gaussian

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


HASH_CASES = [
    # dtype, heads, n, d, bits, probes
    ("bf16", 2, 1000, 128, 10, 3),
    ("bf16", 1, 777, 64, 7, 8),      # every Hamming-1 neighbour
    ("bf16", 2, 500, 128, 14, 5),
    ("f32", 1, 300, 64, 7, 8),
    ("f32", 2, 257, 128, 12, 4),
]


@pytest.mark.parametrize("dtype,H,n,d,b,P", HASH_CASES)
def test_multi_probe_hash_matches_oracle(fa, dtype, H, n, d, b, P):
    print(f"hash {dtype} H{H} n{n} d{d} b{b} P{P}", flush=True)
    seed = 4000 + n + b + P
    planes = gaussian((b, d), seed, dtype)
    x = gaussian((H, n, d), seed + 1, dtype)
    x[:, 0] = 0.0               # every distance 0: the flips go to bits 0, 1, ...
    # rows at the same distance from planes 0 and 1 (equal projections on
    # unit-norm-equal planes are rare; here x is built on two equal axes)
    if d >= 4:
        for i in range(5, n, 11):
            x[:, i] = 0.0
            x[:, i, 0] = x[:, i, 1] = 1.0
    eq_planes = planes.copy()
    eq_planes[0] = 0.0
    eq_planes[1] = 0.0
    eq_planes[0, 0] = eq_planes[1, 1] = 1.0
    for pl in (planes, eq_planes):
        diag = fa.new_diag()
        ids, off, perm = fa.fastar_hash(dev_tensor(x, dtype), dev_tensor(pl, dtype), b, P, diag=diag)
        torch.cuda.synchronize()
        ids, off, perm = ids.cpu().numpy(), off.cpu().numpy(), perm.cpu().numpy()
        for h in range(H):
            ref = oracle.simhash(x[h], pl, P)
            assert np.array_equal(ids[h], ref), f"head {h}: {np.sum(np.any(ids[h] != ref, axis=1))} rows differ"
            r_off, r_perm = oracle.bucket_index(ref, b)
            assert np.array_equal(off[h], r_off) and np.array_equal(perm[h], r_perm)
        # exact ties of two distances are decided exactly, not left unresolved
        assert diag.cpu().numpy()[3] == 0, diag.tolist()


def _tables_case(dtype, L, H, nq, nk, d, b, P, seed):
    planes = gaussian((L, b, d), seed, dtype)
    q = gaussian((H, nq, d), seed + 1, dtype)
    k = gaussian((H, nk, d), seed + 2, dtype)
    v = gaussian((H, nk, d), seed + 3, dtype)
    rng = np.random.default_rng(seed + 4)
    kb = np.log(rng.integers(1, 6, (H, nk)).astype(np.float64)).astype(np.float32)
    q_ids = np.stack([np.stack([oracle.simhash(q[h], planes[u], P) for h in range(H)]) for u in range(L)])
    k_ids = np.stack([np.stack([oracle.simhash(k[h], planes[u], 1)[:, 0] for h in range(H)])
                      for u in range(L)])
    return planes, q, k, v, kb, q_ids, k_ids


def _gpu_tables(fa, dtype, planes, q, k, v, kb, P, b, hash_on_gpu=True):
    """Hash, index and attend on the GPU, table by table; returns out, lse,
    counts and the ids."""
    L = planes.shape[0]
    H, nq, d = q.shape
    tq, tk, tv = dev_tensor(q, dtype), dev_tensor(k, dtype), dev_tensor(v, dtype)
    q_ids, k_ids, k_off, k_perm = [], [], [], []
    for u in range(L):
        tp = dev_tensor(planes[u], dtype)
        qi, _, _ = fa.fastar_hash(tq, tp, b, P, with_index=False)
        ki, ko, kp = fa.fastar_hash(tk, tp, b, 1)
        q_ids.append(qi)
        k_ids.append(ki[:, :, 0])
        k_off.append(ko)
        k_perm.append(kp)
    q_ids = torch.stack(q_ids).contiguous()
    k_ids, k_off, k_perm = (torch.stack(t).contiguous() for t in (k_ids, k_off, k_perm))
    _, q_perm = fa.fastar_bucket_index(q_ids[0], b)
    out, lse, cnt = fa.fastar_bucket_attention_tables(
        tq, tk, tv, q_ids, q_perm, k_off, k_perm, b, k_bucket=k_ids,
        key_bias=torch.tensor(kb, device="cuda"), want_count=True)
    torch.cuda.synchronize()
    return out, lse, cnt, q_ids, k_ids


TABLE_CASES = [
    # dtype, tables, H, nq, nk, d, bits, probes per table
    ("bf16", 2, 2, 1000, 3000, 128, 6, 1),
    ("bf16", 2, 2, 777, 2000, 128, 7, 2),
    ("bf16", 3, 1, 600, 2500, 64, 5, 2),
    ("bf16", 4, 2, 500, 1500, 128, 8, 2),     # 8 entries per row
    ("bf16", 1, 2, 900, 2000, 128, 6, 4),     # one table, four probes
    ("bf16", 1, 1, 400, 1000, 64, 5, 6),
    ("bf16", 2, 1, 64, 40, 128, 9, 3),         # many empty buckets, tiny key set
    ("f32", 2, 1, 256, 700, 64, 5, 2),
    ("f32", 1, 2, 200, 500, 128, 6, 5),
]


@pytest.mark.parametrize("dtype,L,H,nq,nk,d,b,P", TABLE_CASES)
def test_tables_attention_matches_oracle(fa, dtype, L, H, nq, nk, d, b, P):
    print(f"tables {dtype} L{L} H{H} nq{nq} nk{nk} d{d} b{b} P{P}", flush=True)
    planes, q, k, v, kb, q_ids, k_ids = _tables_case(dtype, L, H, nq, nk, d, b, P, seed=nq + nk + L * 10 + P)
    out, lse, cnt, gq, gk = _gpu_tables(fa, dtype, planes, q, k, v, kb, P, b)
    assert np.array_equal(gq.cpu().numpy(), q_ids) and np.array_equal(gk.cpu().numpy(), k_ids)
    out, lse, cnt = out.float().cpu().numpy(), lse.cpu().numpy(), cnt.cpu().numpy()
    for h in range(H):
        o_ref, lse_ref, n_ref = oracle.bucket_attention_tables(q[h], q_ids[:, h], k[h], v[h], k_ids[:, h],
                                                               bias=kb[h])
        assert np.array_equal(cnt[h], n_ref), f"head {h}: {np.sum(cnt[h] != n_ref)} counts differ"
        err = np.max(np.abs(out[h] - o_ref))
        assert err <= TOL[dtype], f"head {h}: max|err| {err}"
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse[h]), fin)
        assert np.max(np.abs(lse[h][fin] - lse_ref[fin]), initial=0) <= TOL[dtype]


def test_single_table_many_probes_through_plain_call(fa):
    # fastar_bucket_attention takes more than two probes of one table
    H, nq, nk, d, b, P = 2, 800, 2400, 128, 7, 5
    planes, q, k, v, kb, q_ids, k_ids = _tables_case("bf16", 1, H, nq, nk, d, b, P, seed=3131)
    q_off, q_perm = fa.fastar_bucket_index(i32(q_ids[0]), b)
    k_off, k_perm = fa.fastar_bucket_index(i32(k_ids[0][:, :, None]), b)
    out, lse = fa.fastar_bucket_attention(dev_tensor(q, "bf16"), dev_tensor(k, "bf16"), dev_tensor(v, "bf16"),
                                          q_bucket=i32(q_ids[0]), q_perm=q_perm,
                                          key_bias=torch.tensor(kb, device="cuda"), k_offsets=k_off,
                                          k_perm=k_perm, n_bits=b)
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    for h in range(H):
        o_ref, lse_ref = oracle.bucket_attention(q[h], q_ids[0, h], k[h], v[h], k_ids[0, h], bias=kb[h])
        assert np.max(np.abs(out[h] - o_ref)) <= TOL["bf16"]
        fin = np.isfinite(lse_ref)
        assert np.max(np.abs(lse[h][fin] - lse_ref[fin]), initial=0) <= TOL["bf16"]


def test_tables_attention_any_row_order_and_shared_buckets(fa):
    # rows visited in a random order, and tables whose planes coincide (every
    # key retained by table 0 is also retained by table 1: counted once)
    H, nq, nk, d, b, P = 2, 700, 1600, 128, 5, 2
    planes, q, k, v, kb, q_ids, k_ids = _tables_case("bf16", 2, H, nq, nk, d, b, P, seed=777)
    planes[1] = planes[0]
    q_ids[1], k_ids[1] = q_ids[0], k_ids[0]
    tq, tk, tv = dev_tensor(q, "bf16"), dev_tensor(k, "bf16"), dev_tensor(v, "bf16")
    offs, perms = [], []
    for u in range(2):
        o, p = fa.fastar_bucket_index(i32(k_ids[u][:, :, None]), b)
        offs.append(o)
        perms.append(p)
    rng = np.random.default_rng(778)
    q_perm = i32(np.stack([rng.permutation(nq) for _ in range(H)]))
    out, lse, cnt = fa.fastar_bucket_attention_tables(
        tq, tk, tv, i32(q_ids), q_perm, torch.stack(offs).contiguous(), torch.stack(perms).contiguous(), b,
        k_bucket=i32(k_ids), key_bias=torch.tensor(kb, device="cuda"), want_count=True)
    torch.cuda.synchronize()
    out, cnt = out.float().cpu().numpy(), cnt.cpu().numpy()
    for h in range(H):
        o_ref, _, n_ref = oracle.bucket_attention_tables(q[h], q_ids[:, h], k[h], v[h], k_ids[:, h], bias=kb[h])
        o1, _ = oracle.bucket_attention(q[h], q_ids[0, h], k[h], v[h], k_ids[0, h], bias=kb[h])
        assert np.allclose(o_ref, o1, atol=1e-12)
        assert np.array_equal(cnt[h], n_ref)
        assert np.max(np.abs(out[h] - o_ref)) <= TOL["bf16"]


@pytest.mark.parametrize("L,P,b", [(2, 2, 6), (3, 1, 9), (4, 2, 15), (1, 5, 8)])
def test_tables_prune_matches_oracle(fa, L, P, b):
    H, nq, npr, d = 3, 500, 3000, 128
    planes = gaussian((L, b, d), 90 + L + b, "bf16")
    q = gaussian((H, nq, d), 91, "bf16")
    pk = gaussian((H, npr, d), 92, "bf16")
    q_ids = np.stack([np.stack([oracle.simhash(q[h], planes[u], P) for h in range(H)]) for u in range(L)])
    p_ids = np.stack([np.stack([oracle.simhash(pk[h], planes[u], 1)[:, 0] for h in range(H)])
                      for u in range(L)])
    keep, kept_idx, n_kept = fa.fastar_prune_prompt_tables(i32(q_ids), i32(p_ids), b)
    torch.cuda.synchronize()
    keep, kept_idx, n_kept = keep.cpu().numpy(), kept_idx.cpu().numpy(), n_kept.cpu().numpy()
    for h in range(H):
        k_ref, i_ref = oracle.prune_prompt_tables(q_ids[:, h], p_ids[:, h])
        assert np.array_equal(keep[h].astype(bool), k_ref)
        assert n_kept[h] == i_ref.size and np.array_equal(kept_idx[h, :i_ref.size], i_ref)


def test_tables_recall_from_counts(fa):
    H, nq, nk, d, b, P, L = 2, 600, 2000, 128, 5, 2, 2
    planes, q, k, v, kb, q_ids, k_ids = _tables_case("bf16", L, H, nq, nk, d, b, P, seed=4242)
    out, lse, cnt, _, _ = _gpu_tables(fa, "bf16", planes, q, k, v, kb, P, b)
    _, lse_d = fa.fastar_bucket_attention(dev_tensor(q, "bf16"), dev_tensor(k, "bf16"), dev_tensor(v, "bf16"),
                                          key_bias=torch.tensor(kb, device="cuda"))
    n_keys = torch.full((H,), nk, dtype=torch.int32, device="cuda")
    recall, stats = fa.fastar_attention_recall_counts(lse, lse_d, n_keys, cnt)
    torch.cuda.synchronize()
    recall, stats = recall.cpu().numpy(), stats.cpu().numpy()
    for h in range(H):
        mask = oracle.retained_tables(q_ids[:, h], k_ids[:, h])
        r_ref, d_ref = oracle.attention_recall(q[h], k[h], mask, bias=kb[h])
        # recall = exp(lse_s - lse_d): the two lse errors (each <= TOL) give
        # a relative error <= exp(2 TOL) - 1
        assert np.max(np.abs(recall[h] - r_ref) / np.maximum(r_ref, 1e-30)) <= np.exp(2 * TOL["bf16"]) - 1
        assert abs(stats[h, 1] - d_ref.mean()) <= 1e-6
        assert abs(stats[h, 0] - r_ref.mean()) <= (np.exp(2 * TOL["bf16"]) - 1) * r_ref.mean()

"""Pins of the oracle's multi-probe SimHash and multi-table LSH (no GPU).

Each test states what fixes the expected value: a hand-worked example, an
order-free property (the full Hamming-1 ball), the inclusion-exclusion
identity of softmax normalisers over a union, brute force by loops, torch
SDPA in float64 with the retained mask, or the closed-form collision rate of
random-hyperplane hashing over several tables.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (simhash, simhash_tables, retained_tables, bucket_attention_tables, prune_prompt,
                    prune_prompt_tables, bucket_attention)
from synth import gaussian


def test_probe_order_by_hand():
    # x = (3, 1, 2) against the unit axes: distances 3, 1, 2, so the flips go
    # to bits 1, 2, 0; the id is 0b111 = 7
    ids = simhash(np.array([[3.0, 1.0, 2.0]]), np.eye(3), 4)
    assert ids.tolist() == [[7, 7 ^ 2, 7 ^ 4, 7 ^ 1]]
    # scaling a plane changes no distance (|x.r| / |r|)
    ids = simhash(np.array([[3.0, 1.0, 2.0]]), np.diag([10.0, 0.5, 3.0]), 4)
    assert ids.tolist() == [[7, 5, 3, 6]]
    # a negative projection clears its bit and still counts by magnitude
    ids = simhash(np.array([[3.0, -1.0, 2.0]]), np.eye(3), 3)
    assert ids.tolist() == [[5, 7, 1]]


def test_probe_order_exact_ties_go_to_smaller_bit():
    ids = simhash(np.array([[1.0, 1.0, 1.0, 1.0]]), np.eye(4), 5)
    assert ids.tolist() == [[15, 14, 13, 11, 7]]


def test_all_probes_are_the_hamming_ball():
    # with n_bits + 1 probes the probe set is the id and all its Hamming-1
    # neighbours, whatever the order
    x = gaussian((200, 64), 11, "bf16")
    planes = gaussian((7, 64), 12, "bf16")
    ids = simhash(x, planes, 8)
    for row in ids.tolist():
        assert sorted(row[1:]) == sorted(row[0] ^ (1 << j) for j in range(7))


def test_probe_prefix_property():
    # the first P' probes do not depend on how many are asked for
    x = gaussian((300, 128), 13, "bf16")
    planes = gaussian((10, 128), 14, "bf16")
    full = simhash(x, planes, 6)
    for p in range(1, 6):
        assert np.array_equal(simhash(x, planes, p), full[:, :p])


def test_third_probe_below_float64_resolution():
    # distances 1 (plane 0), 1 / sqrt(1 + 2^-60) (plane 1) and
    # (1 + 2^-29) / sqrt(1 + 2^-58) (plane 2): float64 sees planes 0 and 1 at
    # the same distance, exactly plane 1 is nearer; plane 2 is farthest
    e = 2.0 ** -30
    planes = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, e, 0.0], [0.0, 0.0, 0.0, 1.0]])
    planes[2, 1] = 2 * e                      # |r2|^2 = 1 + 4 e^2
    x = np.array([[1.0, 1.0, 0.0, 1.0]])      # x.r0 = 1, x.r1 = 1, x.r2 = 1 + 2e
    assert np.sqrt(1.0 + e * e) == 1.0
    ids = simhash(x, planes, 4)
    assert ids.tolist() == [[7, 7 ^ 2, 7 ^ 1, 7 ^ 4]]


def test_n_probes_bounds():
    with pytest.raises(ValueError):
        simhash(np.ones((1, 4)), np.eye(4)[:2], 4)
    assert simhash(np.ones((2, 4)), np.zeros((0, 4)), 1).tolist() == [[0], [0]]


def _tables_case(seed, n=40, m=90, d=32, L=2, b=3, P=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((m, d))
    v = rng.standard_normal((m, d))
    bias = np.log(rng.integers(1, 5, m).astype(np.float64))
    planes = rng.standard_normal((L, b, d))
    q_ids = simhash_tables(q, planes, P)
    k_ids = simhash_tables(k, planes, 1)[:, :, 0]
    return q, k, v, bias, q_ids, k_ids, b


def test_one_table_is_the_single_table_definition():
    q, k, v, bias, q_ids, k_ids, _ = _tables_case(1, L=1)
    o, lse, n = bucket_attention_tables(q, q_ids, k, v, k_ids, bias)
    o1, lse1 = bucket_attention(q, q_ids[0], k, v, k_ids[0], bias)
    assert np.allclose(o, o1, rtol=0, atol=1e-12) and np.allclose(lse, lse1, rtol=0, atol=1e-12)


def test_union_by_inclusion_exclusion():
    # Z(S1 u S2) = Z(S1) + Z(S2) - Z(S1 n S2), and the same for Z o; the
    # intersection is single-table attention over pair buckets (b1, b2)
    q, k, v, bias, q_ids, k_ids, b = _tables_case(2, L=2, b=3, P=2)
    o, lse, cnt = bucket_attention_tables(q, q_ids, k, v, k_ids, bias)
    o1, l1 = bucket_attention(q, q_ids[0], k, v, k_ids[0], bias)
    o2, l2 = bucket_attention(q, q_ids[1], k, v, k_ids[1], bias)
    pair_q = (q_ids[0][:, :, None] * (1 << b) + q_ids[1][:, None, :]).reshape(len(q), -1)
    pair_k = k_ids[0] * (1 << b) + k_ids[1]
    o12, l12 = bucket_attention(q, pair_q, k, v, pair_k, bias)
    z1, z2, z12 = np.exp(l1), np.exp(l2), np.exp(l12)
    z = z1 + z2 - z12
    assert np.allclose(np.exp(lse), z, rtol=1e-12, atol=0)
    num = o1 * z1[:, None] + o2 * z2[:, None] - o12 * z12[:, None]
    assert np.allclose(o * z[:, None], num, rtol=1e-10, atol=1e-12)
    # the retained count likewise
    n1 = np.array([np.isin(k_ids[0], r).sum() for r in q_ids[0]])
    n2 = np.array([np.isin(k_ids[1], r).sum() for r in q_ids[1]])
    n12 = np.array([np.isin(pair_k, r).sum() for r in pair_q])
    assert np.array_equal(cnt, n1 + n2 - n12)


def test_union_attention_is_masked_sdpa_and_brute_force():
    q, k, v, bias, q_ids, k_ids, _ = _tables_case(3, n=12, m=30, L=3, b=2, P=3)
    o, lse, cnt = bucket_attention_tables(q, q_ids, k, v, k_ids, bias)
    s = 1.0 / math.sqrt(q.shape[1])
    for r in range(len(q)):
        keep = [j for j in range(len(k))
                if any(k_ids[u, j] in q_ids[u, r].tolist() for u in range(q_ids.shape[0]))]
        assert cnt[r] == len(keep)
        if not keep:
            assert np.all(o[r] == 0) and lse[r] == -np.inf
            continue
        logits = [float(q[r] @ k[j]) * s + bias[j] for j in keep]
        mx = max(logits)
        w = [math.exp(t - mx) for t in logits]
        ref = sum(wi * v[j] for wi, j in zip(w, keep)) / sum(w)
        assert np.allclose(o[r], ref, rtol=1e-12, atol=1e-12)
        assert abs(lse[r] - (mx + math.log(sum(w)))) < 1e-12
    # and torch's SDPA with the retained mask
    mask = retained_tables(q_ids, k_ids)
    rows = mask.any(axis=1)
    am = torch.where(torch.tensor(mask[rows]), torch.tensor(bias)[None, :], torch.tensor(-math.inf))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q[rows])[None, None], torch.tensor(k)[None, None], torch.tensor(v)[None, None],
        attn_mask=am[None, None].to(torch.float64))[0, 0].numpy()
    assert np.allclose(o[rows], ref, rtol=1e-10, atol=1e-12)


def test_prune_tables():
    q_ids = np.array([[[1, 2], [3, 1]], [[0, 0], [5, 4]]])        # [L=2, n=2, P=2]
    p_ids = np.array([[1, 2, 7, 0, 3], [6, 6, 4, 0, 1]])           # [L=2, Np=5]
    keep, idx = prune_prompt_tables(q_ids, p_ids)
    # token 0: bucket 1 in table 0; 1: bucket 2; 2: table 1 bucket 4;
    # 3: table 1 bucket 0; 4: table 0 bucket 3
    assert keep.tolist() == [True, True, True, True, True]
    p_ids[1, 2] = 6
    keep, idx = prune_prompt_tables(q_ids, p_ids)
    assert keep.tolist() == [True, True, False, True, True] and idx.tolist() == [0, 1, 3, 4]
    k1, i1 = prune_prompt(q_ids[0], p_ids[0])
    k2, i2 = prune_prompt_tables(q_ids[:1], p_ids[:1])
    assert np.array_equal(k1, k2) and np.array_equal(i1, i2)


def test_multi_table_collision_rate():
    # two unit vectors at angle theta share a b-bit bucket in a table with
    # probability (1 - theta / pi)^b (Charikar), so in at least one of L
    # independent tables with probability 1 - (1 - (1 - theta / pi)^b)^L
    rng = np.random.default_rng(21)
    d, b, L, trials = 16, 4, 3, 4000
    theta = 1.0
    u = np.zeros(d)
    u[0] = 1.0
    w = np.zeros(d)
    w[0], w[1] = math.cos(theta), math.sin(theta)
    hits = 0
    for _ in range(trials):
        planes = rng.standard_normal((L, b, d))
        iu = simhash_tables(u[None], planes)[:, 0, 0]
        iw = simhash_tables(w[None], planes)[:, 0, 0]
        hits += bool(np.any(iu == iw))
    p = 1 - (1 - (1 - theta / math.pi) ** b) ** L
    sd = math.sqrt(p * (1 - p) / trials)
    assert abs(hits / trials - p) < 5 * sd


def test_sequence_with_repeated_tables_is_the_single_table_sequence():
    # further tables with table 0's planes retain exactly table 0's keys
    from dataclasses import replace
    from oracle import run_chunk
    from synth import make_workload
    w = make_workload(0)
    one = run_chunk(w)[0]
    rep = run_chunk(w, extra_planes=np.stack([w.planes, w.planes]))[0]
    assert np.array_equal(rep["group_of_new"], one["group_of_new"])
    assert np.allclose(rep["o_self"], one["o_self"], rtol=0, atol=1e-12)
    assert np.array_equal(rep["kept_idx"], one["kept_idx"])
    # and a second table that retains more can only add keys
    w2 = replace(w, n_probes=1)
    other = np.random.default_rng(5).standard_normal(w.planes.shape)
    more = run_chunk(w2, extra_planes=other[None])[0]
    single = np.array([np.isin(one["cache"].rep_bucket, row).sum() for row in one["q_ids"]])
    assert np.all(more["n_attended"] >= single)
    assert set(one["kept_idx"].tolist()) <= set(more["kept_idx"].tolist())


def test_sequence_dense_warmup_is_the_one_bucket_sequence():
    # with no hyperplanes every key shares the one bucket: sparse = dense
    from dataclasses import replace
    from oracle import run_chunk
    from synth import make_workload
    w = make_workload(0)
    w0 = replace(w, n_bits=0, planes=w.planes[:0])
    sparse = run_chunk(w0)[0]
    dense = run_chunk(w, sparse=False)[0]
    dense0 = run_chunk(w0, sparse=False)[0]
    assert np.allclose(sparse["o_self"], dense0["o_self"], rtol=0, atol=1e-12)
    assert np.allclose(sparse["o_cross"], dense0["o_cross"], rtol=0, atol=1e-12)
    # the warm-up keeps the sparse run's merge (the cache does not depend on
    # whether attention is sparse), and attends to every group and prompt token
    ref = run_chunk(w)[0]
    assert np.array_equal(dense["group_of_new"], ref["group_of_new"])
    assert dense["kept_idx"].size == w.prompt_k.shape[1]

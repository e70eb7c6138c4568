"""Pins of the CPU oracle to facts other than itself (no GPU needed).

Each test states what fixes the expected value: the pages' Lemma 5.1, a
library routine (torch SDPA in float64), a closed form, an invariant, or a
tiny example worked by hand from the stated rules.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (
    simhash, bucket_index, TempCacheOracle, prune_prompt, cross_attention,
    dense_attention, bucket_attention, exact_dot,
)
from oracle.tempcache import round_to_storage
from synth import gaussian, round_to_dtype


def sdpa64(q, k, v, mask=None, bias=None, scale=None):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    qt = torch.tensor(q, dtype=torch.float64)[None, None]
    kt = torch.tensor(k, dtype=torch.float64)[None, None]
    vt = torch.tensor(v, dtype=torch.float64)[None, None]
    am = None
    if mask is not None or bias is not None:
        am = torch.zeros(q.shape[0], k.shape[0], dtype=torch.float64)
        if bias is not None:
            am = am + torch.tensor(bias, dtype=torch.float64)[None, :]
        if mask is not None:
            am = am.masked_fill(~torch.tensor(mask), float("-inf"))
        am = am[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)
    return o[0, 0].numpy()


# --------------------------------------------------------------------------
# SimHash
# --------------------------------------------------------------------------

def test_hash_quadrants_by_hand():
    planes = np.array([[1.0, 0.0], [0.0, 1.0]])
    x = np.array([[1, 2], [-1, 2], [1, -2], [-1, -2], [0, 1], [1, 0], [0, 0]], float)
    ids = simhash(x, planes)[:, 0]
    # bit j = [x . r_j > 0], bit 0 least significant; exact zero gives 0
    assert ids.tolist() == [3, 2, 1, 0, 2, 1, 0]


def test_hash_zero_vector_is_bucket_zero():
    planes = gaussian((12, 128), 1, "bf16")
    assert simhash(np.zeros((3, 128)), planes, 2)[:, 0].tolist() == [0, 0, 0]
    # all distances 0: the tie goes to plane 0
    assert simhash(np.zeros((1, 128)), planes, 2)[0, 1] == 1


def test_hash_exact_sign_beyond_float64():
    # x . r = 1 + 2^-60 - 1 = 2^-60 > 0, which float64 rounds to 0
    x = np.array([[1.0, 2.0 ** -60, -1.0]])
    r = np.array([[1.0, 1.0, 1.0]])
    assert float(exact_dot(x[0], r[0])) == 2.0 ** -60
    assert simhash(x, r)[0, 0] == 1
    assert simhash(-x, r)[0, 0] == 0


def test_second_probe_uses_normalised_distance():
    # distances to the planes are |x.r_j|/|r_j| = 0.8 and 1.0 -> flip bit 0
    # (the raw projections 3.2 and 1.0 would flip bit 1)
    planes = np.array([[4.0, 0.0], [0.0, 1.0]])
    ids = simhash(np.array([[0.8, 1.0]]), planes, 2)
    assert ids.tolist() == [[3, 2]]
    # equal distances: the smaller plane index is flipped
    ids = simhash(np.array([[1.0, 1.0]]), np.eye(2), 2)
    assert ids.tolist() == [[3, 2]]


def test_second_probe_exact_near_tie():
    # distances 1 and 1 + 2^-40: float64 error bounds overlap only with the
    # exact path active when the gap is below its window; the gap here is
    # resolvable in float64 but exercises the candidate window
    planes = np.array([[1.0, 0.0], [0.0, 1.0]])
    ids = simhash(np.array([[1.0 + 2.0 ** -40, 1.0]]), planes, 2)
    assert ids.tolist() == [[3, 1]]


def test_hash_plane_permutation_permutes_bits():
    x = gaussian((500, 64), 2, "bf16")
    planes = gaussian((9, 64), 3, "bf16")
    perm = np.random.default_rng(4).permutation(9)
    a = simhash(x, planes)[:, 0]
    b = simhash(x, planes[perm])[:, 0]
    bits_a = (a[:, None] >> np.arange(9)) & 1
    bits_b = (b[:, None] >> np.arange(9)) & 1
    assert np.array_equal(bits_b, bits_a[:, perm])


def test_hash_negation_complements_bits():
    x = gaussian((300, 128), 5, "bf16")
    planes = gaussian((12, 128), 6, "bf16")
    a = simhash(x, planes)[:, 0]
    b = simhash(-x, planes)[:, 0]
    assert np.array_equal(a ^ b, np.full_like(a, (1 << 12) - 1))


def test_hash_collision_probability_charikar():
    # P[bit agrees] = 1 - theta/pi for Gaussian hyperplanes (Charikar 2002)
    rng = np.random.default_rng(7)
    d = 32
    u = rng.standard_normal(d)
    w = rng.standard_normal(d)
    w -= (w @ u) / (u @ u) * u
    theta = 1.0
    v = np.cos(theta) * u / np.linalg.norm(u) + np.sin(theta) * w / np.linalg.norm(w)
    planes = rng.standard_normal((12, d))
    trials = 2000
    agree = 0
    for t in range(trials):
        p = rng.standard_normal((12, d))
        ids = simhash(np.stack([u, v]), p)[:, 0]
        agree += 12 - bin(int(ids[0] ^ ids[1])).count("1")
    rate = agree / (12 * trials)
    expect = 1 - theta / math.pi
    sd = math.sqrt(expect * (1 - expect) / (12 * trials))
    assert abs(rate - expect) < 5 * sd
    del planes


def test_hash_no_planes_single_bucket():
    ids = simhash(gaussian((10, 64), 8), np.zeros((0, 64)))
    assert ids[:, 0].tolist() == [0] * 10


# --------------------------------------------------------------------------
# Bucket index
# --------------------------------------------------------------------------

def test_index_by_hand_one_probe():
    off, perm = bucket_index(np.array([3, 1, 3, 0, 1]), 2)
    assert perm.tolist() == [3, 1, 4, 0, 2]
    assert off.tolist() == [0, 1, 3, 3, 5]


def test_index_by_hand_two_probes():
    # several probes: each query once, stably by its smallest probe bucket
    # (keys 0, 1, 0, 0 and 2)
    ids = np.array([[1, 0], [1, 3], [1, 0], [0, 2], [3, 2]])
    off, perm = bucket_index(ids, 2)
    assert perm.tolist() == [0, 2, 3, 1, 4]
    assert off.tolist() == [0, 3, 4, 5, 5]
    # with three probes the smallest of all three
    off, perm = bucket_index(np.array([[3, 2, 1], [2, 3, 0], [1, 0, 3]]), 2)
    assert perm.tolist() == [1, 2, 0] and off.tolist() == [0, 2, 3, 3, 3]


def test_index_invariants():
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 1 << 7, 5000)
    off, perm = bucket_index(ids, 7)
    assert sorted(perm.tolist()) == list(range(5000))          # a permutation
    k = ids[perm]
    assert np.all(np.diff(k) >= 0)                               # sorted by bucket
    same = np.diff(k) == 0
    assert np.all(np.diff(perm)[same] > 0)                      # stable
    assert np.array_equal(np.diff(off), np.bincount(ids, minlength=128))
    assert off[-1] == 5000 and off[0] == 0


# --------------------------------------------------------------------------
# Attention (Lemma 5.1, dense equivalence)
# --------------------------------------------------------------------------

def _dup_cache(rng, g, d, dv, max_m):
    reps = rng.standard_normal((g, d))
    m = rng.integers(1, max_m + 1, g)
    keys = np.repeat(reps, m, axis=0)
    vals = rng.standard_normal((keys.shape[0], dv))
    owner = np.repeat(np.arange(g), m)
    means = np.stack([vals[owner == t].mean(axis=0) for t in range(g)])
    return reps, m, keys, vals, means


def test_lemma_5_1_merge_is_exact():
    rng = np.random.default_rng(10)
    reps, m, keys, vals, means = _dup_cache(rng, 40, 64, 64, 5)
    q = rng.standard_normal((30, 64))
    o_full, lse_full = dense_attention(q, keys, vals)
    o_merged, lse_merged = dense_attention(q, reps, means, bias=np.log(m))
    assert np.max(np.abs(o_full - o_merged)) < 1e-12
    assert np.max(np.abs(lse_full - lse_merged)) < 1e-12
    # without the + log m shift the identity fails
    o_nobias, _ = dense_attention(q, reps, means)
    assert np.max(np.abs(o_full - o_nobias)) > 1e-3


def test_lemma_no_duplicates_is_standard_attention():
    rng = np.random.default_rng(11)
    q, k, v = rng.standard_normal((8, 32)), rng.standard_normal((20, 32)), rng.standard_normal((20, 32))
    o1, _ = dense_attention(q, k, v, bias=np.log(np.ones(20)))
    assert np.max(np.abs(o1 - sdpa64(q, k, v))) < 1e-12


def test_dense_attention_matches_torch_sdpa():
    rng = np.random.default_rng(12)
    q, k, v = rng.standard_normal((16, 128)), rng.standard_normal((70, 128)), rng.standard_normal((70, 128))
    bias = rng.standard_normal(70)
    o, _ = dense_attention(q, k, v, bias=bias)
    assert np.max(np.abs(o - sdpa64(q, k, v, bias=bias))) < 1e-12


def test_one_bucket_equals_dense():
    rng = np.random.default_rng(13)
    q, k, v = rng.standard_normal((16, 64)), rng.standard_normal((50, 64)), rng.standard_normal((50, 64))
    o, lse = bucket_attention(q, np.zeros((16, 1), int), k, v, np.zeros(50, int))
    assert np.max(np.abs(o - sdpa64(q, k, v))) < 1e-12


@pytest.mark.parametrize("probes", [1, 2])
def test_bucket_attention_is_masked_sdpa(probes):
    rng = np.random.default_rng(14 + probes)
    n, m, d = 40, 300, 64
    q, k, v = rng.standard_normal((n, d)), rng.standard_normal((m, d)), rng.standard_normal((m, d))
    q_ids = rng.integers(0, 8, (n, probes))
    k_b = rng.integers(0, 8, m)
    bias = np.log(rng.integers(1, 4, m).astype(float))
    o, lse = bucket_attention(q, q_ids, k, v, k_b, bias=bias)
    mask = (k_b[None, :] == q_ids[:, :1])
    if probes == 2:
        mask |= (k_b[None, :] == q_ids[:, 1:2])
    assert mask.any(axis=1).all()
    ref = sdpa64(q, k, v, mask=mask, bias=bias)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_empty_key_set_gives_zero():
    q = np.ones((2, 4))
    o, lse = bucket_attention(q, np.array([[1], [2]]), np.ones((3, 4)), np.ones((3, 4)), np.array([0, 0, 2]))
    assert np.all(o[0] == 0) and lse[0] == -np.inf
    assert np.allclose(o[1], 1.0)


def test_single_key_and_equal_logits_closed_forms():
    v = np.array([[1.0, -2.0], [3.0, 4.0]])
    o, lse = dense_attention(np.array([[1.0, 0.0]]), np.array([[0.5, 0.5]]), v[:1])
    assert np.array_equal(o, v[:1])
    o, lse = dense_attention(np.array([[1.0, 0.0]]), np.array([[0.0, 1.0], [0.0, -1.0]]), v)
    assert np.allclose(o, v.mean(axis=0), atol=0, rtol=1e-15)
    assert abs(lse[0] - math.log(2.0)) < 1e-15


def test_uniform_duplication_leaves_output_unchanged():
    rng = np.random.default_rng(15)
    q, k, v = rng.standard_normal((6, 32)), rng.standard_normal((25, 32)), rng.standard_normal((25, 32))
    o1, _ = dense_attention(q, k, v)
    o2, _ = dense_attention(q, k, v, bias=np.full(25, math.log(2.0)))
    assert np.max(np.abs(o1 - o2)) < 1e-13


# --------------------------------------------------------------------------
# TempCache
# --------------------------------------------------------------------------

def _run_frames(frames_k, frames_v, planes, tau, dtype="f32"):
    tc = TempCacheOracle(frames_k.shape[-1], dtype)
    groups = []
    for f in range(frames_k.shape[0]):
        ids = simhash(frames_k[f], planes)[:, 0]
        groups.append(tc.merge_frame(frames_k[f], frames_v[f], ids, tau))
    return tc, groups


@pytest.mark.parametrize("tau", [0.5, 0.9, 1.0])
def test_exact_duplicate_frames_merge_one_to_one(tau):
    T, d, F = 64, 32, 5
    k0 = gaussian((T, d), 20, "bf16")
    ks = np.stack([k0] * F)
    vs = gaussian((F, T, d), 21, "bf16")
    tc, groups = _run_frames(ks, vs, gaussian((5, d), 22, "bf16"), tau, "bf16")
    assert tc.n_groups == T
    for g in groups:
        assert g.tolist() == list(range(T))
    assert np.all(tc.count == F)
    assert np.array_equal(tc.v_sum, vs.astype(np.float64).sum(axis=0))
    assert np.max(np.abs(tc.v_mean - vs.mean(axis=0))) <= 2.0 ** -8 * np.max(np.abs(vs))


def test_threshold_above_one_merges_nothing():
    T, d, F = 32, 16, 3
    k0 = gaussian((T, d), 23)
    tc, groups = _run_frames(np.stack([k0] * F), gaussian((F, T, d), 24), gaussian((3, d), 25), 1.5)
    assert tc.n_groups == F * T
    assert np.concatenate(groups).tolist() == list(range(F * T))
    assert np.all(tc.count == 1)


def test_duplicates_then_attention_is_lemma_exact():
    # TempCache over exact duplicates composed with the biased attention must
    # reproduce dense attention over the raw, uncompressed cache (Lemma 5.1)
    T, d, F = 48, 32, 4
    k0 = gaussian((T, d), 26, "bf16")
    ks = np.stack([k0] * F)
    vs = gaussian((F, T, d), 27, "bf16")
    tc, _ = _run_frames(ks, vs, np.zeros((0, d)), 0.9)
    q = gaussian((20, d), 28)
    o_raw, _ = dense_attention(q, ks.reshape(-1, d), vs.reshape(-1, d))
    o_tc, _ = bucket_attention(q, np.zeros((20, 1), int), tc.rep_k, tc.v_sum / tc.count[:, None],
                               tc.rep_bucket, bias=tc.log_count)
    assert np.max(np.abs(o_raw - o_tc)) < 1e-12


def test_mass_conservation_random_frames():
    T, d, F = 128, 32, 6
    rng = np.random.default_rng(29)
    k = np.empty((F, T, d))
    k[0] = rng.standard_normal((T, d))
    for f in range(1, F):
        keep = rng.random(T) < 0.7
        k[f] = np.where(keep[:, None], k[f - 1] + 0.02 * rng.standard_normal((T, d)),
                        rng.standard_normal((T, d)))
    k = round_to_dtype(k, "bf16")
    v = gaussian((F, T, d), 30, "bf16")
    tc, groups = _run_frames(k, v, gaussian((4, d), 31, "bf16"), 0.99, "bf16")
    assert tc.count.sum() == F * T
    assert np.array_equal(tc.v_sum.sum(axis=0), v.astype(np.float64).reshape(-1, d).sum(axis=0))
    # every group's members: count equals the number of tokens mapped to it
    allg = np.concatenate(groups)
    assert np.array_equal(np.bincount(allg, minlength=tc.n_groups), tc.count)
    # merged groups keep the last key as representative
    last = {}
    for f in range(F):
        for j, g in enumerate(groups[f].tolist()):
            last[g] = (f, j)
    for g, (f, j) in last.items():
        assert np.array_equal(tc.rep_k[g], k[f, j])
    # within a frame no two tokens share a group (one-to-one)
    for g in groups:
        assert len(set(g.tolist())) == T
    assert 0 < tc.n_groups < F * T


def test_conflict_goes_to_highest_cosine_by_hand():
    # frame 0: k0=(1,0) k1=(0,1); frame 1: j0=(1,.1) j1=(1,.01) j2=(0,1)
    # j0 and j1 both pick k0; j1 has the larger cosine and wins; j0 opens
    # group 2; j2 extends group 1.
    tc = TempCacheOracle(2, "f32")
    tc.merge_frame(np.array([[1.0, 0.0], [0.0, 1.0]]), np.array([[1.0, 1.0], [2.0, 2.0]]),
                   np.zeros(2, int), 0.9)
    g = tc.merge_frame(np.array([[1.0, 0.1], [1.0, 0.01], [0.0, 1.0]]),
                       np.array([[3.0, 3.0], [5.0, 5.0], [4.0, 4.0]]), np.zeros(3, int), 0.9)
    assert g.tolist() == [2, 0, 1]
    assert tc.count.tolist() == [2, 2, 1]
    assert tc.rep_k[0].tolist() == [1.0, 0.01]
    assert tc.v_mean.tolist() == [[3.0, 3.0], [3.0, 3.0], [3.0, 3.0]]


def test_ties_go_to_smaller_indices_by_hand():
    # frame 0 has two identical keys; both new keys tie on both candidates:
    # each picks candidate 0, and the smaller new index wins the conflict.
    tc = TempCacheOracle(2, "f32")
    tc.merge_frame(np.array([[1.0, 0.0], [1.0, 0.0]]), np.ones((2, 2)), np.zeros(2, int), 0.9)
    g = tc.merge_frame(np.array([[1.0, 0.0], [3.0, 0.0]]), np.ones((2, 2)), np.zeros(2, int), 0.9)
    assert g.tolist() == [0, 2]
    assert tc.n_groups == 3
    # group 1 was not extended, so its frame-0 key is no longer a candidate;
    # frame-1 candidates are groups 0 and 2, both at cos 1: again both new
    # keys pick candidate 0, j=0 wins and j=1 opens group 3
    g = tc.merge_frame(np.array([[1.0, 0.0], [1.0, 0.0]]), np.ones((2, 2)), np.zeros(2, int), 0.9)
    assert g.tolist() == [0, 3]
    assert tc.count.tolist() == [3, 1, 1, 1]


def test_threshold_is_inclusive_and_uses_float32_tau():
    # cos((1,0,0,0,0), (3,2,1,1,1)) = 3/4 exactly
    a = np.array([[1.0, 0, 0, 0, 0]])
    b = np.array([[3.0, 2, 1, 1, 1]])
    for tau, merges in [(0.75, True), (0.7500001, False), (0.7499999, True)]:
        tc = TempCacheOracle(5, "f32")
        tc.merge_frame(a, np.ones((1, 5)), np.zeros(1, int), tau)
        g = tc.merge_frame(b, np.ones((1, 5)), np.zeros(1, int), tau)
        assert (g[0] == 0) == merges, tau


def test_different_buckets_never_merge():
    tc = TempCacheOracle(2, "f32")
    tc.merge_frame(np.array([[1.0, 0.0]]), np.ones((1, 2)), np.array([1]), 0.5)
    g = tc.merge_frame(np.array([[1.0, 0.0]]), np.ones((1, 2)), np.array([2]), 0.5)
    assert g.tolist() == [1]


def test_round_to_storage_bf16_ties_to_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -(1.0 + 2.0 ** -8)])
    assert round_to_storage(x, "bf16").tolist() == [1.0, 1.0 + 2.0 ** -6, 1.0, -1.0]


# --------------------------------------------------------------------------
# AnnCA
# --------------------------------------------------------------------------

def test_prune_by_hand():
    keep, kept = prune_prompt(np.array([[1, 5], [3, 1]]), np.array([0, 1, 2, 3, 4, 5, 1]))
    assert keep.tolist() == [False, True, False, True, False, True, True]
    assert kept.tolist() == [1, 3, 5, 6]


def test_prune_single_bucket_keeps_all_and_equals_dense():
    rng = np.random.default_rng(32)
    q, pk, pv = rng.standard_normal((10, 64)), rng.standard_normal((40, 64)), rng.standard_normal((40, 64))
    planes = np.zeros((0, 64))
    keep, kept = prune_prompt(simhash(q, planes), simhash(pk, planes)[:, 0])
    assert keep.all()
    o, _ = cross_attention(q, pk, pv, kept)
    assert np.max(np.abs(o - sdpa64(q, pk, pv))) < 1e-12


def test_cross_attention_nothing_kept_is_zero():
    o, lse = cross_attention(np.ones((3, 4)), np.ones((5, 4)), np.ones((5, 4)), np.zeros(0, int))
    assert np.all(o == 0) and np.all(lse == -np.inf)


# --------------------------------------------------------------------------
# The per-chunk sequence (oracle.run_chunk)
# --------------------------------------------------------------------------

def _seq_workload(k_frames, v_frames, q, setup_frames, tau, n_bits=0, planes=None,
                  prompt_k=None, prompt_v=None, n_probes=1, dtype="f32"):
    """A Workload holding given arrays (k/v frames [H, F, T, d], q [H, N, d])."""
    from synth import Workload
    H, _, _, d = k_frames.shape
    if planes is None:
        planes = np.zeros((n_bits, d), np.float32)
    return Workload(-1, "pin", dtype, H, d, n_bits, n_probes, tau, planes, q, k_frames,
                    v_frames, setup_frames=setup_frames, prompt_k=prompt_k, prompt_v=prompt_v)


def test_sequence_no_merge_one_bucket_is_dense_over_raw_frames():
    # tau > 1 merges nothing and b = 0 puts every key in one bucket: the
    # self-attention of the chunk is dense attention over every raw key of
    # every frame, the chunk's own frames included (the merge runs before the
    # attention), with no bias
    H, F, T, d = 1, 4, 40, 64
    k = gaussian((H, F, T, d), 201)
    v = gaussian((H, F, T, d), 202)
    q = gaussian((H, 30, d), 203)
    r = oracle_run_chunk(_seq_workload(k, v, q, setup_frames=2, tau=1.5))[0]
    assert r["cache"].n_groups == F * T
    ref = sdpa64(q[0], k[0].reshape(-1, d), v[0].reshape(-1, d))
    assert np.max(np.abs(r["o_self"] - ref)) < 1e-12
    # the lse is the log of the softmax normaliser over the same keys
    logits = (q[0].astype(np.float64) @ k[0].reshape(-1, d).T.astype(np.float64)) / math.sqrt(d)
    lse = np.log(np.exp(logits - logits.max(1, keepdims=True)).sum(1)) + logits.max(1)
    assert np.max(np.abs(r["lse_self"] - lse)) < 1e-12


def test_sequence_exact_duplicates_is_lemma_exact_over_raw_cache():
    # Frames whose carried tokens are exact copies of the previous frame's
    # (the rest fresh): groups of unequal size m form, and with b = 0 the
    # chunk's self-attention over the compressed cache (mean values, + ln m)
    # equals dense attention over the raw, uncompressed frames (Lemma 5.1,
    # paperlayer.ai appendix A).  Unequal m makes the bias matter, so a
    # dropped bias, attention before the chunk's merge, or an unrounded
    # mean of the wrong frames fails.
    H, F, T, d = 1, 5, 48, 64
    rng = np.random.default_rng(204)
    k = np.empty((H, F, T, d), np.float32)
    k[:, 0] = gaussian((H, T, d), 205)
    for f in range(1, F):
        carry = rng.random((H, T)) < 0.6
        fresh = gaussian((H, T, d), 206 + f)
        k[:, f] = np.where(carry[..., None], k[:, f - 1], fresh)
    v = gaussian((H, F, T, d), 211)
    q = gaussian((H, 25, d), 212)
    for tau in (0.5, 0.999, 1.0):
        r = oracle_run_chunk(_seq_workload(k, v, q, setup_frames=3, tau=tau))[0]
        tc = r["cache"]
        assert tc.count.max() > 1 and tc.count.min() == 1       # unequal group sizes
        assert tc.count.sum() == F * T
        ref = sdpa64(q[0], k[0].reshape(-1, d), v[0].reshape(-1, d))
        # only the float32 rounding of the stored means separates the two
        assert np.max(np.abs(r["o_self"] - ref)) < 1e-6
    # dropping the bias breaks the identity
    o_nobias, _ = bucket_attention(q[0], r["q_ids"], tc.rep_k, tc.v_mean, tc.rep_bucket)
    assert np.max(np.abs(o_nobias - ref)) > 1e-3


def test_sequence_unpruned_prompt_is_dense_cross_attention():
    # b = 0: every prompt key shares the queries' one bucket, so AnnCA keeps
    # all of them and the cross-attention is dense attention over the prompt
    H, T, d = 1, 16, 64
    k = gaussian((H, 2, T, d), 220)
    v = gaussian((H, 2, T, d), 221)
    q = gaussian((H, 20, d), 222)
    pk, pv = gaussian((H, 33, d), 223), gaussian((H, 33, d), 224)
    r = oracle_run_chunk(_seq_workload(k, v, q, 1, 0.9, prompt_k=pk, prompt_v=pv))[0]
    assert r["keep"].all() and r["kept_idx"].tolist() == list(range(33))
    assert np.max(np.abs(r["o_cross"] - sdpa64(q[0], pk[0], pv[0]))) < 1e-12


def test_sequence_buckets_restrict_attention_to_probe_sets():
    # with hashing on, the sequence's self-attention equals masked SDPA over
    # the compressed cache, the mask being "representative bucket is one of
    # the query's probe buckets" (two probes), computed from the sequence's
    # own ids: a wrong probe's ids or an unmasked key fails
    H, F, T, d = 1, 3, 64, 64
    k = gaussian((H, F, T, d), 230)
    v = gaussian((H, F, T, d), 231)
    q = gaussian((H, 50, d), 232)
    planes = gaussian((3, d), 233)
    r = oracle_run_chunk(_seq_workload(k, v, q, 1, 1.5, n_bits=3, planes=planes, n_probes=2))[0]
    tc = r["cache"]
    ids = simhash(q[0], planes, 2)
    assert np.array_equal(r["q_ids"], ids)
    mask = (tc.rep_bucket[None, :] == ids[:, :1]) | (tc.rep_bucket[None, :] == ids[:, 1:2])
    rows = mask.any(axis=1)
    ref = sdpa64(q[0][rows], tc.rep_k, tc.v_mean, mask=mask[rows], bias=tc.log_count)
    assert np.max(np.abs(r["o_self"][rows] - ref)) < 1e-12
    assert np.all(r["o_self"][~rows] == 0)


def oracle_run_chunk(w):
    from oracle import run_chunk
    return run_chunk(w)


# --------------------------------------------------------------------------
# Decisions whose true gap float64 cannot resolve
# --------------------------------------------------------------------------

def test_tempcache_argmax_below_float64_resolution():
    # key a = (1, 0); candidates b0 = (1, 3 e), b1 = (1, e) with e = 2^-30:
    # cos(a, b_i) = 1 / sqrt(1 + (c e)^2), which float64 rounds to exactly 1
    # for both, but b1 is strictly closer.  The smaller-index tie rule would
    # pick b0; the exact comparison picks b1.
    e = 2.0 ** -30
    tc = TempCacheOracle(2, "f32")
    tc.merge_frame(np.array([[1.0, 3 * e], [1.0, e]]), np.ones((2, 2)), np.zeros(2, int), 0.5)
    cos_f64 = [np.float64(1.0) / np.sqrt(1.0 + (c * e) ** 2) for c in (3, 1)]
    assert cos_f64[0] == cos_f64[1] == 1.0
    g = tc.merge_frame(np.array([[1.0, 0.0]]), np.ones((1, 2)), np.zeros(1, int), 0.5)
    assert g.tolist() == [1]
    assert tc.exact_evals > 0


def test_tempcache_conflict_below_float64_resolution():
    # two new keys propose to one candidate (1, 0); their cosines 1 / sqrt(1
    # + (c e)^2) are both 1.0 in float64, the second is strictly larger and
    # wins the candidate; the first opens a new group
    e = 2.0 ** -30
    tc = TempCacheOracle(2, "f32")
    tc.merge_frame(np.array([[1.0, 0.0]]), np.ones((1, 2)), np.zeros(1, int), 0.5)
    g = tc.merge_frame(np.array([[1.0, 3 * e], [1.0, e]]), np.ones((2, 2)), np.zeros(2, int), 0.5)
    assert g.tolist() == [1, 0]


def test_tempcache_threshold_below_float64_resolution():
    # cos(a, b) = 1 / sqrt(1 + e^2) with e = 2^-30 is 1.0 in float64 but is
    # strictly below tau = 1: no merge.  With b = a exactly it merges.
    e = 2.0 ** -30
    tc = TempCacheOracle(2, "f32")
    tc.merge_frame(np.array([[1.0, e]]), np.ones((1, 2)), np.zeros(1, int), 1.0)
    g = tc.merge_frame(np.array([[1.0, 0.0]]), np.ones((1, 2)), np.zeros(1, int), 1.0)
    assert g.tolist() == [1]
    g = tc.merge_frame(np.array([[1.0, 0.0]]), np.ones((1, 2)), np.zeros(1, int), 1.0)
    assert g.tolist() == [1]


def test_second_probe_below_float64_resolution():
    # planes r0 = (1, 0, 0), r1 = (0, 1, e) with e = 2^-30 and x = (1, 1, 0):
    # both projections are 1, so the distances are 1 / |r_j|; |r1| =
    # sqrt(1 + e^2) is 1.0 in float64, but x is strictly nearer plane 1.  The
    # smaller-index tie rule would flip bit 0; the exact comparison flips bit 1.
    e = 2.0 ** -30
    planes = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, e]])
    assert np.sqrt(1.0 + e * e) == 1.0
    ids = simhash(np.array([[1.0, 1.0, 0.0]]), planes, 2)
    assert ids.tolist() == [[3, 1]]


def test_stored_mean_is_rounded_once_to_bf16_by_hand():
    # two identical keys merge; values 1 and 1 + 2^-7 average to 1 + 2^-8,
    # halfway between the bf16 neighbours 1 and 1 + 2^-7: ties to even give
    # 1.  Values 1 + 2^-7 and 1 + 2^-6 average to 1 + 3 2^-8, halfway
    # between 1 + 2^-7 (odd) and 1 + 2^-6 (even): 1 + 2^-6.
    for (v0, v1), mean in [((1.0, 1.0 + 2.0 ** -7), 1.0),
                           ((1.0 + 2.0 ** -7, 1.0 + 2.0 ** -6), 1.0 + 2.0 ** -6)]:
        tc = TempCacheOracle(2, "bf16")
        tc.merge_frame(np.array([[1.0, 0.0]]), np.array([[v0, v0]]), np.zeros(1, int), 0.9)
        tc.merge_frame(np.array([[1.0, 0.0]]), np.array([[v1, v1]]), np.zeros(1, int), 0.9)
        assert tc.count.tolist() == [2]
        assert tc.v_mean.tolist() == [[mean, mean]]
        assert tc.v_sum.tolist() == [[v0 + v1, v0 + v1]]


def test_sequence_bookkeeping_invariants():
    # the set-up frames' and the chunk's groups together account for every
    # token exactly once: per-group member counts equal the stored counts,
    # the chunk's ids and groups cover exactly its frames, and the group
    # count before the chunk is what the set-up frames opened
    from synth import make_workload
    w = make_workload(0)
    r = oracle_run_chunk(w)[0]
    tc = r["cache"]
    T = w.tokens_per_frame
    assert r["k_ids"].shape == (w.chunk_frames * T,)
    assert r["group_of_new"].shape == (w.chunk_frames * T,)
    assert r["setup_groups"].shape == (w.setup_frames * T,)
    allg = np.concatenate([r["setup_groups"], r["group_of_new"]])
    assert np.array_equal(np.bincount(allg, minlength=tc.n_groups), tc.count)
    assert r["n_groups_before"] == r["setup_groups"].max() + 1
    assert r["group_of_new"].max() == tc.n_groups - 1
    # chunk keys' ids are the hash of the chunk's own frames (not a set-up frame)
    k_last = w.k_frames[0, -1].astype(np.float64)
    assert np.array_equal(r["k_ids"][-T:], simhash(k_last, w.planes, 1)[:, 0])


# --------------------------------------------------------------------------
# Attention recall and density
# --------------------------------------------------------------------------

def test_recall_by_hand():
    # two keys with logits 0 and ln 3 (scale 1): p = (1/4, 3/4)
    from oracle import attention_recall
    q = np.array([[1.0]])
    k = np.array([[0.0], [math.log(3.0)]])
    rec, den = attention_recall(q, k, np.array([[False, True]]), scale=1.0)
    assert abs(rec[0] - 0.75) < 1e-15 and den[0] == 0.5
    rec, den = attention_recall(q, k, np.array([[True, False]]), scale=1.0)
    assert abs(rec[0] - 0.25) < 1e-15
    # a bias of ln 3 on key 0 evens them out
    rec, _ = attention_recall(q, k, np.array([[True, False]]), scale=1.0, bias=np.array([math.log(3.0), 0]))
    assert abs(rec[0] - 0.5) < 1e-15


def test_recall_one_bucket_is_one():
    # b = 0: every key shares the query's bucket, nothing is dropped
    from oracle import attention_recall, bucket_retained
    rng = np.random.default_rng(40)
    q, k = rng.standard_normal((20, 32)), rng.standard_normal((70, 32))
    ids = simhash(q, np.zeros((0, 32)))
    mask = bucket_retained(ids, simhash(k, np.zeros((0, 32)))[:, 0])
    rec, den = attention_recall(q, k, mask)
    assert np.allclose(rec, 1.0, atol=1e-14, rtol=0) and np.all(den == 1.0)


def test_recall_is_lse_difference_and_topk_bounds_it():
    # recall = exp(lse over the retained keys - lse over all keys) (the
    # softmax normalisers), and the top-k reference at the same count keeps
    # at least as much mass as any retained set of that size
    from oracle import attention_recall, bucket_retained, topk_recall
    rng = np.random.default_rng(41)
    q, k = rng.standard_normal((30, 64)), rng.standard_normal((200, 64))
    bias = np.log(rng.integers(1, 4, 200).astype(float))
    planes = rng.standard_normal((3, 64))
    q_ids, k_b = simhash(q, planes, 2), simhash(k, planes)[:, 0]
    mask = bucket_retained(q_ids, k_b)
    rec, den = attention_recall(q, k, mask, bias=bias)
    _, lse_all = dense_attention(q, k, np.zeros((200, 1)), bias=bias)
    _, lse_a = bucket_attention(q, q_ids, k, np.zeros((200, 1)), k_b, bias=bias)
    assert np.max(np.abs(rec - np.exp(lse_a - lse_all))) < 1e-12
    for i in range(30):
        top = topk_recall(q[i:i + 1], k, den[i], bias=bias)[0]
        assert top >= rec[i] - 1e-12
    # the reference curve: 0 at density 0, 1 at density 1, nondecreasing
    curve = [topk_recall(q, k, r, bias=bias).mean() for r in (0.0, 0.1, 0.3, 0.5, 1.0)]
    assert curve[0] == 0.0 and abs(curve[-1] - 1.0) < 1e-12
    assert all(a <= b + 1e-15 for a, b in zip(curve, curve[1:]))


# --------------------------------------------------------------------------
# TempCache with quantized matching
# --------------------------------------------------------------------------

def test_scalar_codes_by_hand():
    from oracle import scalar_codes
    x = np.array([[1.0, -0.5, 0.25, 0.0], [2.0, 1.0, -3.0, 0.5], [0.0, 0.0, 0.0, 0.0]])
    # 8 bits, Q = 127, row scale max|x|: -63.5 ties to the even -64; 84.67 -> 85
    assert scalar_codes(x, 8).tolist() == [[127, -64, 32, 0], [85, 42, -127, 21], [0, 0, 0, 0]]
    # 2 bits, Q = 1: -0.5 ties to the even 0
    assert scalar_codes(x, 2).tolist() == [[1, 0, 0, 0], [1, 0, -1, 0], [0, 0, 0, 0]]
    # a positive power-of-two rescaling is exact and leaves the codes unchanged
    assert np.array_equal(scalar_codes(x * 8.0, 5), scalar_codes(x, 5))


@pytest.mark.parametrize("tau", [0.5, 1.0])
def test_quant_exact_duplicates_merge_one_to_one(tau):
    from oracle import TempCacheQuantOracle
    T, d, F = 40, 32, 4
    k0 = gaussian((T, d), 240, "bf16")
    vs = gaussian((F, T, d), 241, "bf16")
    tc = TempCacheQuantOracle(d, "bf16", 8)
    for f in range(F):
        g = tc.merge_frame(k0, vs[f], np.zeros(T, int), tau)
        assert g.tolist() == list(range(T))
    assert np.all(tc.count == F)
    assert np.array_equal(tc.v_sum, vs.astype(np.float64).sum(axis=0))


def test_quant_threshold_above_one_merges_nothing():
    from oracle import TempCacheQuantOracle
    T, d = 20, 16
    k0 = gaussian((T, d), 242)
    tc = TempCacheQuantOracle(d, "f32", 8)
    for f in range(3):
        g = tc.merge_frame(k0, np.ones((T, d)), np.zeros(T, int), 1.5)
    assert tc.n_groups == 3 * T and g.tolist() == list(range(2 * T, 3 * T))


def test_quant_matches_across_buckets_and_by_codes_by_hand():
    # the quantized search sees every previous-frame token, whatever its
    # bucket: key (1, 0.3) of bucket 7 finds (1, 0.29) of bucket 2.  At 2
    # bits both code to (1, 0) (0.3 and 0.29 round to 0), cos 1; at 8 bits
    # the codes (127, 38) and (127, 37) differ but pass tau = 0.999.
    from oracle import TempCacheQuantOracle
    for bits in (2, 8):
        tc = TempCacheQuantOracle(2, "f32", bits)
        tc.merge_frame(np.array([[0.0, 1.0], [1.0, 0.29]]), np.ones((2, 2)), np.array([5, 2]), 0.999)
        g = tc.merge_frame(np.array([[1.0, 0.3]]), np.ones((1, 2)), np.array([7]), 0.999)
        assert g.tolist() == [1] and tc.rep_bucket.tolist() == [5, 7]
    # at 2 bits two different new keys code alike and tie on the candidate:
    # the smaller index wins, the other opens a group
    tc = TempCacheQuantOracle(2, "f32", 2)
    tc.merge_frame(np.array([[1.0, 0.0]]), np.ones((1, 2)), np.zeros(1, int), 1.0)
    g = tc.merge_frame(np.array([[1.0, 0.3], [1.0, 0.1]]), np.ones((2, 2)), np.zeros(2, int), 1.0)
    assert g.tolist() == [0, 1]
    # at 8 bits the second (closer) key wins instead
    tc = TempCacheQuantOracle(2, "f32", 8)
    tc.merge_frame(np.array([[1.0, 0.0]]), np.ones((1, 2)), np.zeros(1, int), 0.9)
    g = tc.merge_frame(np.array([[1.0, 0.3], [1.0, 0.1]]), np.ones((2, 2)), np.zeros(2, int), 0.9)
    assert g.tolist() == [1, 0]


def test_quant_rescaled_keys_give_the_same_groups_and_conserve_mass():
    from oracle import TempCacheQuantOracle
    T, d, F = 64, 32, 5
    rng = np.random.default_rng(243)
    k = np.empty((F, T, d))
    k[0] = rng.standard_normal((T, d))
    for f in range(1, F):
        keep = rng.random(T) < 0.7
        k[f] = np.where(keep[:, None], k[f - 1] + 0.02 * rng.standard_normal((T, d)), rng.standard_normal((T, d)))
    k = round_to_dtype(k, "bf16")
    v = gaussian((F, T, d), 244, "bf16")
    scale = 2.0 ** rng.integers(-3, 4, (F, T, 1))            # exact in bf16
    a, b = TempCacheQuantOracle(d, "bf16", 8), TempCacheQuantOracle(d, "bf16", 8)
    ga = [a.merge_frame(k[f], v[f], np.zeros(T, int), 0.99) for f in range(F)]
    gb = [b.merge_frame(k[f] * scale[f], v[f], np.zeros(T, int), 0.99) for f in range(F)]
    assert all(np.array_equal(x, y) for x, y in zip(ga, gb))
    assert a.count.sum() == F * T and 0 < a.n_groups < F * T
    assert np.array_equal(a.v_sum.sum(axis=0), v.astype(np.float64).reshape(-1, d).sum(axis=0))
    assert np.array_equal(np.bincount(np.concatenate(ga), minlength=a.n_groups), a.count)
    for g in ga:
        assert len(set(g.tolist())) == T


def test_quant_query_driven_by_hand():
    # the new token's query (0, 1) finds the previous key (0.1, 1) although its
    # own key (1, 0) would have matched the other previous key (1, 0.05): the
    # token joins group 0 with its key and value
    from oracle import TempCacheQuantOracle
    prev = np.array([[0.1, 1.0], [1.0, 0.05]])
    for qd, want in [(True, [0]), (False, [1])]:
        tc = TempCacheQuantOracle(2, "f32", 8)
        tc.merge_frame(prev, np.ones((2, 2)), np.zeros(2, int), 0.99)
        g = tc.merge_frame(np.array([[1.0, 0.0]]), np.array([[3.0, 3.0]]), np.zeros(1, int), 0.99,
                           match_vec=np.array([[0.0, 1.0]]) if qd else None)
        assert g.tolist() == want
        assert tc.rep_k[want[0]].tolist() == [1.0, 0.0] and tc.count[want[0]] == 2
    # a query equal to its key gives the key-driven result
    rng = np.random.default_rng(250)
    k = round_to_dtype(rng.standard_normal((3, 30, 16)), "bf16")
    a, b = TempCacheQuantOracle(16, "bf16"), TempCacheQuantOracle(16, "bf16")
    for f in range(3):
        ga = a.merge_frame(k[f], np.ones((30, 16)), np.zeros(30, int), 0.3)
        gb = b.merge_frame(k[f], np.ones((30, 16)), np.zeros(30, int), 0.3, match_vec=k[f])
        assert np.array_equal(ga, gb)


# --------------------------------------------------------------------------
# Representative variants
# --------------------------------------------------------------------------

def test_round_fraction_to_storage_by_hand():
    from fractions import Fraction
    from oracle.tempcache import round_fraction_to_storage as rf
    assert rf(Fraction(1), "bf16") == 1.0
    assert rf(Fraction(1) + Fraction(1, 512), "bf16") == 1.0                 # tie to even
    assert rf(Fraction(1) + Fraction(3, 512), "bf16") == 1.0 + 2.0 ** -7     # tie to even (up)
    assert rf(Fraction(1, 3), "bf16") == 171 / 512    # 1.0101010|1010.. x 2^-2 rounds up to 1.0101011
    assert rf(Fraction(1, 3), "f32") == float(np.float32(1.0) / np.float32(3.0))
    assert rf(Fraction(-5, 2), "bf16") == -2.5
    # a mean of three keys rounded once: (1 + 1 + 1 + 2^-7) / 3 sits just above 1
    assert rf((Fraction(3) + Fraction(1, 128)) / 3, "bf16") == 1.0


def test_mean_and_medoid_representatives_by_hand():
    # keys (1, 1) then (3, 1) merge (cos 0.894 >= 0.5); sum (4, 2).  Mean: (2, 1).
    # Medoid: cos((1,1), (4,2)) = 0.949 < cos((3,1), (4,2)) = 0.990: the new key.
    for rep, want in [("mean", [[2.0, 1.0]]), ("medoid", [[3.0, 1.0]]), ("last", [[3.0, 1.0]])]:
        tc = TempCacheOracle(2, "f32", rep)
        tc.merge_frame(np.array([[1.0, 1.0]]), np.ones((1, 2)), np.zeros(1, int), 0.5)
        g = tc.merge_frame(np.array([[3.0, 1.0]]), np.ones((1, 2)), np.zeros(1, int), 0.5)
        assert g.tolist() == [0] and tc.rep_k.tolist() == want, rep
    # medoid over four frames: (1,0); (1,.5): sum (2,.5), cos .970 < .976, moves;
    # (1,-.5): sum (3,0), cos .894 = .894 exactly, a tie keeps (1,.5); (1,0):
    # sum (4,0), cos .894 < 1, moves.  The candidate each frame is matched
    # against is the current representative (cos .6 and .894 pass 0.5).
    tc = TempCacheOracle(2, "f32", "medoid")
    steps = [([1.0, 0.0], [1.0, 0.0]), ([1.0, 0.5], [1.0, 0.5]), ([1.0, -0.5], [1.0, 0.5]),
             ([1.0, 0.0], [1.0, 0.0])]
    for key, rep in steps:
        g = tc.merge_frame(np.array([key]), np.ones((1, 2)), np.zeros(1, int), 0.5)
        assert g.tolist() == [0] and tc.rep_k.tolist() == [rep], (key, rep)
    # the mean after the same four keys: (4, 0) / 4
    tc = TempCacheOracle(2, "f32", "mean")
    for key, _ in steps:
        tc.merge_frame(np.array([key]), np.ones((1, 2)), np.zeros(1, int), 0.5)
    assert tc.rep_k.tolist() == [[1.0, 0.0]] and tc.count.tolist() == [4]


def test_representatives_on_exact_duplicates_agree():
    # exact duplicates: every representative rule gives the same key, and the
    # groups are the same
    T, d, F = 30, 16, 4
    k0 = gaussian((T, d), 260, "bf16")
    vs = gaussian((F, T, d), 261, "bf16")
    outs = []
    for rep in ("last", "mean", "medoid"):
        tc = TempCacheOracle(d, "bf16", rep)
        gs = [tc.merge_frame(k0, vs[f], np.zeros(T, int), 0.9) for f in range(F)]
        outs.append((tc.rep_k.copy(), np.concatenate(gs)))
    for rk, g in outs[1:]:
        assert np.array_equal(rk, outs[0][0]) and np.array_equal(g, outs[0][1])

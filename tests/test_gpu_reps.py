"""TempCache's mean-key and medoid-key representatives on the GPU against the
oracle: groups, counts, buckets, representatives and key sums bit for bit,
value means within the dtype tolerance, for both match kinds and with several
frames per call (merged one frame at a time)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import gaussian, make_workload, round_to_dtype

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


def _frames(H, F, T, d, seed, dtype, carry=0.75, noise=0.02, dup=False):
    # a frame carries most of the previous frame's keys over, with noise
    rng = np.random.default_rng(seed)
    k = np.empty((H, F, T, d))
    k[:, 0] = rng.standard_normal((H, T, d))
    for f in range(1, F):
        keep = rng.random((H, T)) < carry
        nxt = k[:, f - 1] if dup else k[:, f - 1] + noise * rng.standard_normal((H, T, d))
        k[:, f] = np.where(keep[..., None], nxt, rng.standard_normal((H, T, d)))
    v = rng.standard_normal((H, F, T, d))
    return round_to_dtype(k, dtype), round_to_dtype(v, dtype)


def _exact_sums(ref):
    return np.array([[float(x) for x in row] for row in ref.k_sum])


def _check_cache(cache, ref, h, dtype, b, rep_off=None, rep_perm=None):
    G = ref.n_groups
    assert int(cache.n_groups[h]) == G
    assert np.array_equal(cache.count[h, :G].cpu().numpy(), ref.count)
    assert np.array_equal(cache.rep_bucket[h, :G].cpu().numpy(), ref.rep_bucket)
    got = cache.rep_k[h, :G].float().cpu().numpy()
    bad = np.nonzero(np.any(got != ref.rep_k, axis=1))[0]
    assert bad.size == 0, f"head {h}: representatives of groups {bad[:8].tolist()} differ"
    assert np.array_equal(cache.frontier[h].cpu().numpy(), ref.frontier)
    # the float64 key sums are exact here (every sum fits float64)
    assert np.array_equal(cache.k_sum[h, :G].cpu().numpy(), _exact_sums(ref))
    assert np.max(np.abs(cache.v_mean[h, :G].float().cpu().numpy() - ref.v_mean)) <= TOL[dtype]
    if rep_off is not None:
        r_off, r_perm = oracle.bucket_index(ref.rep_bucket, b)
        assert np.array_equal(rep_off[h].cpu().numpy(), r_off)
        assert np.array_equal(rep_perm[h, :G].cpu().numpy(), r_perm)


REP_CASES = [
    # dtype, representative, match, H, F, T, d, hash bits, tau, frames per call, duplicates
    ("bf16", "mean", "lsh", 2, 4, 256, 128, 6, 0.9, 2, False),
    ("f32", "mean", "lsh", 1, 4, 200, 64, 4, 0.8, 4, False),
    ("bf16", "medoid", "lsh", 2, 4, 256, 128, 6, 0.9, 3, False),
    ("f32", "medoid", "lsh", 1, 3, 150, 64, 3, 0.5, 1, False),
    ("bf16", "mean", "quant", 1, 3, 200, 128, 5, 0.99, 3, False),
    ("bf16", "medoid", "quant", 2, 3, 300, 64, 4, 0.95, 2, False),
    ("bf16", "medoid", "lsh", 1, 4, 128, 128, 4, 1.0, 4, True),   # identical keys: ties keep
    ("bf16", "mean", "lsh", 1, 4, 128, 64, 4, 1.0, 2, True),      # mean of identical keys: the key
]


@pytest.mark.parametrize("dtype,rep,match,H,F,T,d,b,tau,fpc,dup", REP_CASES)
def test_rep_merge_matches_oracle(fa, dtype, rep, match, H, F, T, d, b, tau, fpc, dup):
    print(f"representative {rep} match {match} {dtype} H{H} F{F} T{T} d{d} b{b} tau{tau} fpc{fpc}", flush=True)
    k, v = _frames(H, F, T, d, seed=7 * F + T + d + b, dtype=dtype, dup=dup)
    planes = gaussian((max(b, 1), d), 60 + b, dtype)
    tplanes = dev_tensor(planes, dtype)
    cache = fa.TempCache(H, d, F * T, T, b, TDT[dtype], "cuda", key_sums=True)
    opts = fa.merge_opts(match, 8, rep)
    diag = fa.new_diag()
    if match == "quant":
        refs = [oracle.TempCacheQuantOracle(d, dtype, 8, rep) for _ in range(H)]
    else:
        refs = [oracle.TempCacheOracle(d, dtype, rep) for _ in range(H)]
    for f0 in range(0, F, fpc):
        f1 = min(F, f0 + fpc)
        kk = np.ascontiguousarray(k[:, f0:f1].reshape(H, -1, d))
        vv = np.ascontiguousarray(v[:, f0:f1].reshape(H, -1, d))
        tk = dev_tensor(kk, dtype)
        ids, _, _ = fa.fastar_hash(tk, tplanes, b, 1, with_index=False)
        gon = torch.empty(H, kk.shape[1], dtype=torch.int32, device="cuda")
        rep_off, rep_perm = fa.fastar_tempcache_merge(cache, tk, dev_tensor(vv, dtype),
                                                      ids[:, :, 0].contiguous(), f1 - f0, tau,
                                                      group_of_new=gon, diag=diag, opts=opts)
        torch.cuda.synchronize()
        gon = gon.cpu().numpy()
        for h in range(H):
            want = np.concatenate([
                refs[h].merge_frame(k[h, f], v[h, f], oracle.simhash(k[h, f], planes[:b], 1)[:, 0], tau)
                for f in range(f0, f1)])
            assert np.array_equal(gon[h], want), f"frames {f0}-{f1} head {h}: {np.sum(gon[h] != want)} differ"
    for h in range(H):
        _check_cache(cache, refs[h], h, dtype, b, rep_off, rep_perm)
    merged = sum(int((r.count > 1).sum()) for r in refs)
    assert merged > 0, "the case should merge"
    assert int(diag[3]) == 0 and int(diag[4]) == 0, diag.tolist()
    if rep == "mean" and dup:
        for h in range(H):
            # a group of identical keys has that key as its mean
            G = refs[h].n_groups
            sums = _exact_sums(refs[h])
            assert np.array_equal(cache.rep_k[h, :G].float().cpu().numpy(),
                                  sums / refs[h].count[:, None])


def test_rep_query_driven_matches_oracle(fa):
    # medoid representatives with the quantized match driven by the queries
    H, F, T, d, b, tau = 2, 3, 256, 128, 5, 0.99
    k, v = _frames(H, F, T, d, seed=501, dtype="bf16")
    rng = np.random.default_rng(502)
    qv = round_to_dtype(k + 0.05 * rng.standard_normal(k.shape), "bf16")
    planes = gaussian((b, d), 503, "bf16")
    cache = fa.TempCache(H, d, F * T, T, b, torch.bfloat16, "cuda", key_sums=True)
    refs = [oracle.TempCacheQuantOracle(d, "bf16", 8, "medoid") for _ in range(H)]
    diag = fa.new_diag()
    kk = dev_tensor(np.ascontiguousarray(k.reshape(H, -1, d)), "bf16")
    qq = dev_tensor(np.ascontiguousarray(qv.reshape(H, -1, d)), "bf16")
    vv = dev_tensor(np.ascontiguousarray(v.reshape(H, -1, d)), "bf16")
    ids, _, _ = fa.fastar_hash(kk, dev_tensor(planes, "bf16"), b, 1, with_index=False)
    gon = torch.empty(H, F * T, dtype=torch.int32, device="cuda")
    opts = fa.merge_opts("quant", 8, "medoid", match_queries=qq)
    rep_off, rep_perm = fa.fastar_tempcache_merge(cache, kk, vv, ids[:, :, 0].contiguous(), F, tau,
                                                  group_of_new=gon, diag=diag, opts=opts)
    torch.cuda.synchronize()
    for h in range(H):
        want = np.concatenate([
            refs[h].merge_frame(k[h, f], v[h, f], oracle.simhash(k[h, f], planes, 1)[:, 0], tau,
                                match_vec=qv[h, f]) for f in range(F)])
        assert np.array_equal(gon[h].cpu().numpy(), want), f"head {h}"
        _check_cache(cache, refs[h], h, "bf16", b, rep_off, rep_perm)
    assert int(diag[3]) == 0, diag.tolist()


def test_mean_rounding_midpoints(fa):
    # groups whose mean falls exactly on a bf16 rounding midpoint: keys 1 and
    # 1 + 2^-7 (mean 1 + 2^-8: to the even 1), 1 and 1 + 3 2^-7 (mean
    # 1 + 3 2^-8: up to the even 1 + 2^-6), 1 and 1 + 5 2^-7 (mean
    # 1 + 5 2^-8: down to 1 + 2^-6); token j alone in bucket j
    H, T, d, b = 1, 64, 64, 6
    base = np.ones((T, d))
    second = base.copy()
    second[:, 0::3] += 2.0 ** -7
    second[:, 1::3] += 3 * 2.0 ** -7
    second[:, 2::3] += 5 * 2.0 ** -7
    k = np.stack([base, second])[None]          # [H, F=2, T, d]
    v = np.zeros_like(k)
    cache = fa.TempCache(H, d, 2 * T, T, b, torch.bfloat16, "cuda", key_sums=True)
    opts = fa.merge_opts("lsh", 8, "mean")
    kk = dev_tensor(k.reshape(H, -1, d), "bf16")
    ids = torch.arange(T, dtype=torch.int32, device="cuda").repeat(2)[None].contiguous()
    diag = fa.new_diag()
    fa.fastar_tempcache_merge(cache, kk, dev_tensor(v.reshape(H, -1, d), "bf16"), ids, 2, 0.5,
                              diag=diag, opts=opts)
    torch.cuda.synchronize()
    ref = oracle.TempCacheOracle(d, "bf16", "mean")
    for f in range(2):
        ref.merge_frame(k[0, f], v[0, f], np.arange(T), 0.5)
    G = ref.n_groups
    assert G == T and np.all(ref.count == 2)
    got = cache.rep_k[0, :G].float().cpu().numpy()
    assert np.array_equal(got, ref.rep_k)
    # the ties themselves
    assert np.all(got[:, 0::3] == 1.0)
    assert np.all(got[:, 1::3] == 1.0 + 2.0 ** -6) and np.all(got[:, 2::3] == 1.0 + 2.0 ** -6)
    assert Fraction(float(ref.rep_k[0, 2])) == Fraction(1) + Fraction(1, 64)
    assert int(diag[3]) == 0


@pytest.mark.parametrize("rep", ["mean", "medoid"])
def test_rep_chunk_matches_oracle(fa, rep):
    """The whole chunk (layer workload) with mean or medoid representatives:
    groups, cache and self-attention against the oracle on sampled heads."""
    from kv_compressed_attention_amd.layer import FastARLayer

    w = make_workload(1)
    H, F, T, d = w.k_frames.shape
    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries, w.chunk_frames,
                        dtype=TDT[w.dtype], device="cuda", representative=rep)
    layer.set_planes(dev_tensor(w.planes, w.dtype))
    for f in range(w.setup_frames):
        layer.merge(dev_tensor(w.k_frames[:, f], w.dtype), dev_tensor(w.v_frames[:, f], w.dtype), 1,
                    with_index=False)
    q = dev_tensor(w.q, w.dtype)
    k_new, v_new = (dev_tensor(a, w.dtype) for a in w.frames(w.setup_frames, F))
    layer.step(q, k_new, v_new)
    torch.cuda.synchronize()
    heads = [0, H - 1]
    ref = oracle.run_chunk(w, heads=heads, representative=rep)
    c = layer.cache
    for h in heads:
        r = ref[h]
        assert np.array_equal(layer.group_of_new[h].cpu().numpy(), r["group_of_new"]), f"head {h} groups"
        _check_cache(c, r["cache"], h, w.dtype, w.n_bits)
        err = np.max(np.abs(layer.o_self[h].float().cpu().numpy() - r["o_self"]))
        assert err <= TOL[w.dtype], f"head {h} self-attention max|err| {err}"
    assert int(layer.diag[3]) == 0 and c.status_code() == 0

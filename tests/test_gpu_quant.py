"""TempCache's quantized match (FASTAR_MATCH_QUANT) on the GPU against the
oracle: the scalar codes, the groups and the cache bit for bit, value means
within the dtype tolerance."""

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


@pytest.mark.parametrize("dtype,d,bits", [("bf16", 128, 8), ("bf16", 64, 4), ("f32", 128, 8), ("f32", 64, 2)])
def test_scalar_codes_match_oracle(fa, dtype, d, bits):
    H, n = 2, 700
    x = gaussian((H, n, d), 300 + d + bits, dtype)
    # rows whose quotients are exact half-integers (ties to even) and their
    # neighbours: max 127, elements k + 1/2 (representable in bf16)
    q = (1 << (bits - 1)) - 1
    for r in range(0, n, 9):
        row = np.zeros(d)
        row[0] = q
        row[1:] = (np.arange(1, d) % q) + 0.5
        if r % 2:
            row[1:] = np.nextafter(row[1:].astype(np.float32), np.float32(np.inf)) if dtype == "f32" else row[1:] + 2.0 ** -3
        x[0, r] = round_to_dtype(row, dtype)
    x[1, 5] = 0.0
    codes, norm2 = fa.fastar_scalar_codes(dev_tensor(x, dtype), bits)
    torch.cuda.synchronize()
    for h in range(H):
        ref = oracle.scalar_codes(x[h], bits)
        assert np.array_equal(codes[h].cpu().numpy().astype(np.int64), ref), f"head {h}"
        assert np.array_equal(norm2[h].cpu().numpy(), (ref * ref).sum(axis=1))


def _frames(H, F, T, d, seed, dtype, carry=0.75, noise=0.02, dup=False):
    rng = np.random.default_rng(seed)
    k = np.empty((H, F, T, d))
    k[:, 0] = rng.standard_normal((H, T, d))
    for f in range(1, F):
        keep = rng.random((H, T)) < carry
        nxt = k[:, f - 1] if dup else k[:, f - 1] + noise * rng.standard_normal((H, T, d))
        k[:, f] = np.where(keep[..., None], nxt, rng.standard_normal((H, T, d)))
    v = rng.standard_normal((H, F, T, d))
    return round_to_dtype(k, dtype), round_to_dtype(v, dtype)


QUANT_CASES = [
    # dtype, H, F, T, d, hash bits, tau, frames per call, code bits, exact-duplicate carry
    ("f32", 1, 4, 256, 64, 6, 0.9, 1, 8, False),
    ("bf16", 2, 5, 300, 128, 8, 0.999, 2, 8, False),
    ("bf16", 2, 4, 200, 128, 0, 0.99, 4, 4, False),
    ("bf16", 1, 3, 700, 64, 10, 0.5, 3, 2, False),
    ("bf16", 2, 3, 2048, 128, 14, 0.999, 3, 8, False),
    ("bf16", 2, 4, 333, 128, 5, 1.0, 2, 8, True),     # exact duplicates: cosine 1, ties
    ("f32", 1, 3, 150, 128, 3, -0.5, 1, 6, False),   # negative threshold: everything proposes
]


@pytest.mark.parametrize("dtype,H,F,T,d,b,tau,fpc,bits,dup", QUANT_CASES)
def test_quant_merge_matches_oracle(fa, dtype, H, F, T, d, b, tau, fpc, bits, dup):
    k, v = _frames(H, F, T, d, seed=F * T + b + bits, dtype=dtype, dup=dup)
    planes = gaussian((max(b, 1), d), 80 + b, dtype)
    cache = fa.TempCache(H, d, F * T, T, b, TDT[dtype], "cuda")
    opts = fa.merge_opts("quant", bits)
    diag = fa.new_diag()
    tplanes = dev_tensor(planes, dtype)
    refs = [oracle.TempCacheQuantOracle(d, dtype, bits) for _ in range(H)]
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
            ref_groups = []
            for f in range(f0, f1):
                kid = oracle.simhash(k[h, f], planes[:b], 1)[:, 0]
                ref_groups.append(refs[h].merge_frame(k[h, f], v[h, f], kid, tau))
            want = np.concatenate(ref_groups)
            assert np.array_equal(gon[h], want), f"frames {f0}-{f1} head {h}: {np.sum(gon[h] != want)} differ"
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
    if dup:
        assert diag[2].item() > 0, "exact ties should have taken the exact path"


@pytest.mark.parametrize("index", [1, 4])
def test_quant_chunk_matches_oracle(fa, index):
    """The whole chunk with the quantized match (the layer workload and the
    wide two-probe workload): groups, cache and self-attention against the
    oracle's sequence on sampled heads."""
    from kv_compressed_attention_amd.layer import FastARLayer

    w = make_workload(index)
    H, F, T, d = w.k_frames.shape
    npr = 0 if w.prompt_k is None else w.prompt_k.shape[1]
    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries, w.chunk_frames,
                        n_prompt=npr, dtype=TDT[w.dtype], device="cuda", match="quant", code_bits=8)
    layer.set_planes(dev_tensor(w.planes, w.dtype))
    for f in range(w.setup_frames):
        layer.merge(dev_tensor(w.k_frames[:, f], w.dtype), dev_tensor(w.v_frames[:, f], w.dtype), 1,
                    with_index=False)
    q = dev_tensor(w.q, w.dtype)
    k_new, v_new = (dev_tensor(a, w.dtype) for a in w.frames(w.setup_frames, F))
    pk = dev_tensor(w.prompt_k, w.dtype) if npr else None
    pv = dev_tensor(w.prompt_v, w.dtype) if npr else None
    layer.step(q, k_new, v_new, pk, pv)
    torch.cuda.synchronize()
    heads = [0, H - 1]
    ref = oracle.run_chunk(w, heads=heads, match="quant", code_bits=8)
    c = layer.cache
    for h in heads:
        r = ref[h]
        tc = r["cache"]
        G = tc.n_groups
        assert np.array_equal(layer.group_of_new[h].cpu().numpy(), r["group_of_new"]), f"head {h} groups"
        assert int(c.n_groups[h]) == G
        assert np.array_equal(c.count[h, :G].cpu().numpy(), tc.count)
        err = np.max(np.abs(layer.o_self[h].float().cpu().numpy() - r["o_self"]))
        assert err <= TOL[w.dtype], f"head {h} self-attention max|err| {err}"
    assert int(layer.diag[3]) == 0 and c.status_code() == 0


def test_quant_chunk_equals_calls_one_by_one(fa):
    from kv_compressed_attention_amd.layer import FastARLayer

    w = make_workload(1)
    H, F, T, d = w.k_frames.shape
    layers = []
    for _ in range(2):
        layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries, w.chunk_frames,
                            dtype=torch.bfloat16, device="cuda", match="quant")
        layer.set_planes(dev_tensor(w.planes, "bf16"))
        layers.append(layer)
    for f in range(w.setup_frames):
        layers[0].merge(dev_tensor(w.k_frames[:, f], "bf16"), dev_tensor(w.v_frames[:, f], "bf16"), 1,
                        with_index=False)
    layers[1].cache.copy_from(layers[0].cache)
    q = dev_tensor(w.q, "bf16")
    k_new, v_new = (dev_tensor(a, "bf16") for a in w.frames(w.setup_frames, F))
    layers[0].step(q, k_new, v_new, concurrent=False)
    layers[1].step(q, k_new, v_new, concurrent="chunk")
    torch.cuda.synchronize()
    for n in ("q_ids", "q_off", "q_perm", "k_ids", "group_of_new", "rep_off", "o_self", "lse_self"):
        assert torch.equal(getattr(layers[0], n), getattr(layers[1], n)), n
    for n, t in layers[0].cache.buffers().items():
        assert torch.equal(t, layers[1].cache.buffers()[n]), n


def test_quant_query_driven_merge_matches_oracle(fa):
    # each new token matched by its query (a noisy copy of its key, so that
    # the query and key sometimes pick different candidates)
    H, F, T, d, b, tau, bits = 2, 4, 400, 128, 6, 0.99, 8
    k, v = _frames(H, F, T, d, seed=91, dtype="bf16")
    rng = np.random.default_rng(92)
    qv = round_to_dtype(k + 0.05 * rng.standard_normal(k.shape), "bf16")
    planes = gaussian((b, d), 93, "bf16")
    cache = fa.TempCache(H, d, F * T, T, b, torch.bfloat16, "cuda")
    refs = [oracle.TempCacheQuantOracle(d, "bf16", bits) for _ in range(H)]
    for f0, f1 in [(0, 1), (1, 3), (3, 4)]:
        kk = dev_tensor(np.ascontiguousarray(k[:, f0:f1].reshape(H, -1, d)), "bf16")
        qq = dev_tensor(np.ascontiguousarray(qv[:, f0:f1].reshape(H, -1, d)), "bf16")
        vv = dev_tensor(np.ascontiguousarray(v[:, f0:f1].reshape(H, -1, d)), "bf16")
        ids, _, _ = fa.fastar_hash(kk, dev_tensor(planes, "bf16"), b, 1, with_index=False)
        gon = torch.empty(H, kk.shape[1], dtype=torch.int32, device="cuda")
        opts = fa.merge_opts("quant", bits, match_queries=qq)
        fa.fastar_tempcache_merge(cache, kk, vv, ids[:, :, 0].contiguous(), f1 - f0, tau,
                                  group_of_new=gon, opts=opts)
        torch.cuda.synchronize()
        for h in range(H):
            want = np.concatenate([refs[h].merge_frame(k[h, f], v[h, f], oracle.simhash(k[h, f], planes, 1)[:, 0],
                                                       tau, match_vec=qv[h, f]) for f in range(f0, f1)])
            assert np.array_equal(gon[h].cpu().numpy(), want), f"frames {f0}-{f1} head {h}"
    for h in range(H):
        G = refs[h].n_groups
        assert int(cache.n_groups[h]) == G
        assert np.array_equal(cache.rep_k[h, :G].float().cpu().numpy(), refs[h].rep_k)


def test_quant_query_driven_chunk_matches_oracle(fa):
    from kv_compressed_attention_amd.layer import FastARLayer

    w = make_workload(1)
    H, F, T, d = w.k_frames.shape
    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries, w.chunk_frames,
                        dtype=torch.bfloat16, device="cuda", match="quant", query_driven=True)
    layer.set_planes(dev_tensor(w.planes, "bf16"))
    for f in range(w.setup_frames):
        layer.merge(dev_tensor(w.k_frames[:, f], "bf16"), dev_tensor(w.v_frames[:, f], "bf16"), 1,
                    with_index=False)
    q = dev_tensor(w.q, "bf16")
    k_new, v_new = (dev_tensor(a, "bf16") for a in w.frames(w.setup_frames, F))
    layer.step(q, k_new, v_new)
    torch.cuda.synchronize()
    ref = oracle.run_chunk(w, heads=[3], match="quant", query_driven=True)
    r = ref[3]
    assert np.array_equal(layer.group_of_new[3].cpu().numpy(), r["group_of_new"])
    assert int(layer.cache.n_groups[3]) == r["cache"].n_groups
    err = np.max(np.abs(layer.o_self[3].float().cpu().numpy() - r["o_self"]))
    assert err <= TOL["bf16"]

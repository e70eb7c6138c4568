"""The layer's multi-table chunk, its dense (warm-up) chunk and the denoising
driver on the GPU against the oracle's sequence."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from synth import make_workload, round_to_dtype

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


def _layer(w, **kw):
    from kv_compressed_attention_amd.layer import FastARLayer
    H, F, T, d = w.k_frames.shape
    npr = 0 if w.prompt_k is None else w.prompt_k.shape[1]
    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries, w.chunk_frames,
                        n_prompt=npr, dtype=TDT[w.dtype], device="cuda", **kw)
    return layer


def _setup(layer, w):
    for f in range(w.setup_frames):
        layer.merge(dev_tensor(w.k_frames[:, f], w.dtype), dev_tensor(w.v_frames[:, f], w.dtype), 1,
                    with_index=False)


def _inputs(w):
    H, F = w.k_frames.shape[:2]
    k_new, v_new = (dev_tensor(a, w.dtype) for a in w.frames(w.setup_frames, F))
    pk = dev_tensor(w.prompt_k, w.dtype) if w.prompt_k is not None else None
    pv = dev_tensor(w.prompt_v, w.dtype) if w.prompt_v is not None else None
    return dev_tensor(w.q, w.dtype), k_new, v_new, pk, pv


def _check(layer, ref, heads, dtype, cross=True, counts=False, kept=True):
    c = layer.cache
    for h in heads:
        r = ref[h]
        tc = r["cache"]
        G = tc.n_groups
        assert np.array_equal(layer.group_of_new[h].cpu().numpy(), r["group_of_new"]), f"head {h} groups"
        assert int(c.n_groups[h]) == G
        err = np.max(np.abs(layer.o_self[h].float().cpu().numpy() - r["o_self"]))
        assert err <= TOL[dtype], f"head {h} self-attention max|err| {err}"
        fin = np.isfinite(r["lse_self"])
        lse = layer.lse_self[h].cpu().numpy()
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.max(np.abs(lse[fin] - r["lse_self"][fin]), initial=0) <= TOL[dtype]
        if counts:
            assert np.array_equal(layer.n_attended[h].cpu().numpy(), r["n_attended"])
        if cross and "o_cross" in r:
            n = r["kept_idx"].size
            if kept:
                assert int(layer.n_kept[h]) == n
                assert np.array_equal(layer.kept_idx[h, :n].cpu().numpy(), r["kept_idx"])
            err = np.max(np.abs(layer.o_cross[h].float().cpu().numpy() - r["o_cross"]))
            assert err <= TOL[dtype], f"head {h} cross-attention max|err| {err}"


@pytest.mark.parametrize("index,L", [(0, 2), (0, 3), (1, 2)])
def test_tables_chunk_matches_oracle(fa, index, L):
    print(f"tables chunk workload {index} L{L}", flush=True)
    w = make_workload(index)
    H = w.heads
    extra = round_to_dtype(np.random.default_rng(700 + L).standard_normal((L - 1,) + w.planes.shape), w.dtype)
    layer = _layer(w, n_tables=L)
    layer.set_planes(dev_tensor(np.concatenate([w.planes[None], extra]), w.dtype))
    _setup(layer, w)
    layer.step(*_inputs(w))
    torch.cuda.synchronize()
    heads = [0] if H == 1 else [0, H - 1]
    ref = oracle.run_chunk(w, heads=heads, extra_planes=extra)
    _check(layer, ref, heads, w.dtype, counts=True)
    assert int(layer.diag[3]) == 0 and layer.cache.status_code() == 0


@pytest.mark.parametrize("index", [0, 1])
def test_dense_chunk_matches_oracle(fa, index):
    w = make_workload(index)
    layer = _layer(w)
    layer.set_planes(dev_tensor(w.planes, w.dtype))
    _setup(layer, w)
    layer.step_dense(*_inputs(w))
    torch.cuda.synchronize()
    heads = [0] if w.heads == 1 else [0, w.heads - 1]
    ref = oracle.run_chunk(w, heads=heads, sparse=False)
    _check(layer, ref, heads, w.dtype, kept=False)


def test_denoising_driver_matches_oracle(fa):
    """Five denoising steps of one chunk (two dense, three sparse), each with
    its own inputs, against the oracle's sequence from the same pre-chunk
    cache; afterwards the cache holds the last step's merge."""
    from kv_compressed_attention_amd.denoise import DenoisingDriver
    w = make_workload(0)
    H, F, T, d = w.k_frames.shape
    S = 5
    rng = np.random.default_rng(808)
    steps = []
    for s in range(S):
        k = w.k_frames.copy()
        v = w.v_frames.copy()
        k[:, w.setup_frames:] += 0.1 * rng.standard_normal(k[:, w.setup_frames:].shape)
        v[:, w.setup_frames:] = rng.standard_normal(v[:, w.setup_frames:].shape)
        q = w.q + 0.1 * rng.standard_normal(w.q.shape)
        steps.append(replace(w, q=round_to_dtype(q, w.dtype), k_frames=round_to_dtype(k, w.dtype),
                             v_frames=round_to_dtype(v, w.dtype)))
    layer = _layer(w)
    layer.set_planes(dev_tensor(w.planes, w.dtype))
    _setup(layer, w)
    inputs = [_inputs(ws) for ws in steps]
    got = []

    def on_step(s, dense):
        torch.cuda.synchronize()
        got.append((dense, layer.group_of_new[0].cpu().numpy(), layer.o_self[0].float().cpu().numpy(),
                    layer.o_cross[0].float().cpu().numpy()))
    flags = DenoisingDriver(layer, S, warmup=0.3).run(lambda s: inputs[s], on_step)
    torch.cuda.synchronize()
    assert flags == [True, True, False, False, False]
    for s in range(S):
        ref = oracle.run_chunk(steps[s], heads=[0], sparse=not flags[s])[0]
        dense, groups, o_self, o_cross = got[s]
        assert dense == flags[s]
        assert np.array_equal(groups, ref["group_of_new"]), f"step {s}"
        assert np.max(np.abs(o_self - ref["o_self"])) <= TOL[w.dtype], f"step {s}"
        assert np.max(np.abs(o_cross - ref["o_cross"])) <= TOL[w.dtype], f"step {s}"
    # the chunk entered the cache once: the last step's merge
    tc = oracle.run_chunk(steps[-1], heads=[0], attention=False)[0]["cache"]
    G = tc.n_groups
    assert int(layer.cache.n_groups[0]) == G
    assert np.array_equal(layer.cache.count[0, :G].cpu().numpy(), tc.count)
    assert np.array_equal(layer.cache.rep_k[0, :G].float().cpu().numpy(), tc.rep_k)


@pytest.mark.parametrize("rep", ["last", "medoid"])
def test_cache_checkpoint_restore(fa, rep):
    """restore() undoes the merges since checkpoint(): the next merge then
    gives what it gives on a full copy of the checkpointed cache."""
    w = make_workload(1)
    H, F, T, d = w.k_frames.shape
    layer = _layer(w, representative=rep)
    layer.set_planes(dev_tensor(w.planes, w.dtype))
    _setup(layer, w)
    c = layer.cache
    copy = fa.TempCache(H, d, F * T, T, w.n_bits, TDT[w.dtype], "cuda", key_sums=rep != "last")
    copy.copy_from(c)
    ck = c.checkpoint()
    rng = np.random.default_rng(31)
    k_new, v_new = w.frames(w.setup_frames, F)
    other_k = round_to_dtype(k_new + 0.2 * rng.standard_normal(k_new.shape), w.dtype)
    layer.merge(dev_tensor(other_k, w.dtype), dev_tensor(v_new, w.dtype), w.chunk_frames)
    c.restore(ck)
    layer.merge(dev_tensor(k_new, w.dtype), dev_tensor(v_new, w.dtype), w.chunk_frames)
    g1 = layer.group_of_new.clone()
    layer.cache = copy
    layer.merge(dev_tensor(k_new, w.dtype), dev_tensor(v_new, w.dtype), w.chunk_frames)
    torch.cuda.synchronize()
    assert torch.equal(g1, layer.group_of_new)
    for h in range(H):
        G = int(copy.n_groups[h])
        assert int(c.n_groups[h]) == G
        for name in ("rep_k", "v_mean", "v_sum", "count", "log_count", "rep_bucket") + (
                ("k_sum",) if rep != "last" else ()):
            assert torch.equal(getattr(c, name)[h, :G], getattr(copy, name)[h, :G]), name
    assert torch.equal(c.frontier, copy.frontier)

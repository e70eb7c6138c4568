"""End-to-end GPU parity on the five synthetic workloads, at full size.

The GPU runs the whole per-layer sequence for every head, in the same launch
configuration bench.py times (the set-up frames merged one frame per call,
then the measured chunk in one call).  The oracle recomputes a sample of heads
in full; integer results (bucket ids, indexes, TempCache groups, prune masks)
must match bit for bit, float outputs within max-abs 2e-2 (bf16) / 1e-5 (fp32).
"""

import time

import numpy as np
import pytest
import torch

import oracle
from synth import make_workload

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}
# heads the oracle recomputes (all for the small workloads)
SAMPLE = {0: [0], 1: [0, 5, 11], 2: [0, 6, 11], 3: [0, 7], 4: [0, 13, 23]}


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_compressed_attention_amd as m
    m.library()
    return m


def _up(a, dtype):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device="cuda").to(TDT[dtype])


def run_gpu(w):
    """The GPU sequence; returns host copies of every intermediate."""
    from kv_compressed_attention_amd.layer import FastARLayer
    import kv_compressed_attention_amd as fa

    H, nq, d = w.q.shape
    out = {}
    q = _up(w.q, w.dtype)
    if w.k_frames is None:
        # cross-attention only
        planes = _up(w.planes, w.dtype)
        ids, off, perm = fa.fastar_hash(q, planes, w.n_bits, w.n_probes)
        pk = _up(w.prompt_k, w.dtype)
        p_ids, _, _ = fa.fastar_hash(pk, planes, w.n_bits, 1, with_index=False)
        keep, kept, n_kept = fa.fastar_prune_prompt(ids, p_ids[:, :, 0].contiguous(), w.n_bits)
        o, lse = fa.fastar_bucket_attention(q, pk, _up(w.prompt_v, w.dtype), key_list=kept,
                                            n_key_list=n_kept)
        torch.cuda.synchronize()
        out.update(q_ids=ids, q_offsets=off, q_perm=perm, p_ids=p_ids[:, :, 0], keep=keep,
                   kept=kept, n_kept=n_kept, o_cross=o, lse_cross=lse)
        return {k: v.cpu() for k, v in out.items()}
    _, F, T, _ = w.k_frames.shape
    npr = 0 if w.prompt_k is None else w.prompt_k.shape[1]
    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, nq, w.chunk_frames,
                        n_prompt=npr, dtype=TDT[w.dtype], device="cuda")
    layer.set_planes(_up(w.planes, w.dtype))
    setup_groups = []
    for f in range(w.setup_frames):
        g = torch.empty(H, T, dtype=torch.int32, device="cuda")
        layer.merge(_up(w.k_frames[:, f], w.dtype), _up(w.v_frames[:, f], w.dtype), 1,
                    with_index=False, group_of_new=g)
        setup_groups.append(g)
    out["n_groups_before"] = layer.cache.n_groups.clone()
    k_new, v_new = (_up(a, w.dtype) for a in w.frames(w.setup_frames, F))
    pk = pv = None
    if npr:
        pk, pv = _up(w.prompt_k, w.dtype), _up(w.prompt_v, w.dtype)
    layer.step(q, k_new, v_new, pk, pv)
    torch.cuda.synchronize()
    c = layer.cache
    out.update(q_ids=layer.q_ids, q_offsets=layer.q_off, q_perm=layer.q_perm,
               k_ids=layer.k_ids[:, :, 0], group_of_new=layer.group_of_new,
               setup_groups=torch.stack(setup_groups, 1) if setup_groups else None,
               n_groups=c.n_groups, count=c.count, rep_bucket=c.rep_bucket, rep_k=c.rep_k,
               v_mean=c.v_mean, log_count=c.log_count, rep_off=layer.rep_off,
               rep_perm=layer.rep_perm, o_self=layer.o_self, lse_self=layer.lse_self,
               diag=layer.diag)
    if npr:
        out.update(p_ids=layer.p_ids[:, :, 0], keep=layer.keep, kept=layer.kept_idx,
                   n_kept=layer.n_kept, o_cross=layer.o_cross, lse_cross=layer.lse_cross)
    return {k: (None if v is None else v.cpu()) for k, v in out.items()}


def check_head(w, g, r, h, setup_groups_ref):
    tol = TOL[w.dtype]
    i = lambda t: t[h].numpy().astype(np.int64)  # noqa: E731
    assert np.array_equal(i(g["q_ids"]), r["q_ids"]), "query bucket ids"
    assert np.array_equal(i(g["q_offsets"]), r["q_offsets"]), "query index offsets"
    assert np.array_equal(i(g["q_perm"]), r["q_perm"]), "query index perm"
    if w.k_frames is not None:
        tc = r["cache"]
        G = tc.n_groups
        assert np.array_equal(i(g["k_ids"]), r["k_ids"]), "new key bucket ids"
        if w.setup_frames:
            assert np.array_equal(g["setup_groups"][h].numpy().reshape(-1), setup_groups_ref), \
                "set-up frame groups"
        assert int(g["n_groups_before"][h]) == r["n_groups_before"]
        assert np.array_equal(i(g["group_of_new"]), r["group_of_new"]), "chunk groups"
        assert int(g["n_groups"][h]) == G, "group count"
        assert np.array_equal(i(g["count"])[:G], tc.count), "group sizes"
        assert np.array_equal(i(g["rep_bucket"])[:G], tc.rep_bucket), "representative buckets"
        assert np.array_equal(g["rep_k"][h, :G].float().numpy(), tc.rep_k), "representative keys"
        assert np.max(np.abs(g["v_mean"][h, :G].float().numpy() - tc.v_mean)) <= tol
        assert np.max(np.abs(g["log_count"][h, :G].numpy() - tc.log_count)) <= 1e-5
        assert np.array_equal(i(g["rep_off"]), r["rep_offsets"]), "representative index offsets"
        assert np.array_equal(i(g["rep_perm"])[:G], r["rep_perm"]), "representative index perm"
        err = np.max(np.abs(g["o_self"][h].float().numpy() - r["o_self"]))
        assert err <= tol, f"self-attention max|err| {err}"
        check_lse(g["lse_self"][h].numpy(), r["lse_self"], tol, "self-attention lse")
    if w.prompt_k is not None:
        assert np.array_equal(i(g["p_ids"]), r["p_ids"]), "prompt bucket ids"
        assert np.array_equal(g["keep"][h].numpy().astype(bool), r["keep"]), "prune mask"
        nk = int(g["n_kept"][h])
        assert nk == r["kept_idx"].size
        assert np.array_equal(i(g["kept"])[:nk], r["kept_idx"]), "kept prompt indices"
        err = np.max(np.abs(g["o_cross"][h].float().numpy() - r["o_cross"]))
        assert err <= tol, f"cross-attention max|err| {err}"
        check_lse(g["lse_cross"][h].numpy(), r["lse_cross"], tol, "cross-attention lse")


def check_lse(got, ref, tol, what):
    """Element-wise: the same rows are empty (-inf), the rest within tol."""
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: empty rows differ"
    assert np.all(got[~fin] == -np.inf), f"{what}: empty rows must be -inf"
    err = np.max(np.abs(got[fin] - ref[fin]), initial=0.0)
    assert err <= tol, f"{what} max|err| {err}"


def check_all_heads_integers(w, g):
    """Hash ids (and the prune mask) of every head, not just the sampled
    ones: the oracle's hashing and pruning are cheap."""
    for h in range(w.heads):
        q_ids = oracle.simhash(w.q[h], w.planes, w.n_probes)
        assert np.array_equal(g["q_ids"][h].numpy(), q_ids), f"query ids, head {h}"
        if w.k_frames is not None:
            kf = w.k_frames[h, w.setup_frames:].reshape(-1, w.dim)
            assert np.array_equal(g["k_ids"][h].numpy(), oracle.simhash(kf, w.planes, 1)[:, 0]), \
                f"new key ids, head {h}"
        if w.prompt_k is not None:
            p_ids = oracle.simhash(w.prompt_k[h], w.planes, 1)[:, 0]
            assert np.array_equal(g["p_ids"][h].numpy(), p_ids), f"prompt ids, head {h}"
            keep, kept = oracle.prune_prompt(q_ids, p_ids)
            assert np.array_equal(g["keep"][h].numpy().astype(bool), keep), f"prune mask, head {h}"


@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])
def test_workload_end_to_end(fa, index):
    t0 = time.time()
    w = make_workload(index)
    t1 = time.time()
    g = run_gpu(w)
    t2 = time.time()
    ref = oracle.run_chunk(w, heads=SAMPLE[index])
    t3 = time.time()
    for h in SAMPLE[index]:
        check_head(w, g, ref[h], h, ref[h].get("setup_groups"))
    check_all_heads_integers(w, g)
    if "diag" in g:
        d = g["diag"].numpy()
        assert d[3] == 0, f"unresolved decisions {d}"
        assert d[4] == 0, f"capacity overflow {d}"
    print(f"workload {index} {w.name}: generate {t1 - t0:.1f}s gpu {t2 - t1:.1f}s "
          f"oracle {t3 - t2:.1f}s check {time.time() - t3:.1f}s", flush=True)

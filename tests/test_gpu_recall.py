"""Attention recall and density on the GPU against the oracle.

recall(q) = exp(lse_sparse(q) - lse_dense(q)) from two attention launches
(the sparse one and the dense one over the same keys and bias), density from
the retained set's size (paperlayer.ai section 4, attention sparsity).  Each
lse is within the attention tolerance TOL of the oracle's, so a recall is
within exp(2 TOL) - 1 of the oracle's (recall <= 1); densities are exact
ratios, compared to 1e-6.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import gaussian, make_workload

pytestmark = pytest.mark.gpu
TOL = {"bf16": 2e-2, "f32": 1e-5}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}
SAMPLE = {0: [0], 1: [0, 7], 4: [0, 17]}


def rtol(dtype):
    return float(np.expm1(2 * TOL[dtype]))


def _up(a, dtype):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device="cuda").to(TDT[dtype])


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_compressed_attention_amd as m
    m.library()
    return m


def test_dense_over_first_n_keys_matches_oracle(fa):
    # dense mode with n_key_list alone: head h attends to its first n[h] keys
    H, nq, nk, d = 3, 200, 700, 128
    q, k, v = (gaussian((H, n, d), 60 + i, "bf16") for i, n in enumerate((nq, nk, nk)))
    bias = np.log(np.random.default_rng(63).integers(1, 5, (H, nk)).astype(np.float64)).astype(np.float32)
    n = np.array([700, 333, 0], dtype=np.int32)
    out, lse = fa.fastar_bucket_attention(_up(q, "bf16"), _up(k, "bf16"), _up(v, "bf16"),
                                          key_bias=torch.tensor(bias, device="cuda"),
                                          n_key_list=torch.tensor(n, device="cuda"))
    torch.cuda.synchronize()
    for h in range(H):
        o_ref, lse_ref = oracle.dense_attention(q[h], k[h, :n[h]], v[h, :n[h]], bias=bias[h, :n[h]])
        assert np.max(np.abs(out[h].float().cpu().numpy() - o_ref)) <= TOL["bf16"]
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse[h].cpu().numpy()), fin)
        assert np.max(np.abs(lse[h].cpu().numpy()[fin] - lse_ref[fin]), initial=0) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,P", [("bf16", 2), ("bf16", 1), ("f32", 2)])
def test_bucket_recall_matches_oracle(fa, dtype, P):
    H, nq, nk, d, b = 2, 500, 900, 64 if dtype == "f32" else 128, 4
    rng = np.random.default_rng(70 + P)
    q, k, v = (gaussian((H, n, d), 71 + i, dtype) for i, n in enumerate((nq, nk, nk)))
    first = rng.integers(0, 1 << b, (H, nq))
    q_ids = np.stack([first, first ^ (1 << rng.integers(0, b, (H, nq)))], 2) if P == 2 else first[:, :, None]
    k_ids = rng.integers(0, 1 << b, (H, nk))
    bias = np.log(rng.integers(1, 5, (H, nk)).astype(np.float64)).astype(np.float32)
    i32 = lambda a: torch.tensor(np.ascontiguousarray(a), dtype=torch.int32, device="cuda")  # noqa: E731
    tq, tk, tv, tb = _up(q, dtype), _up(k, dtype), _up(v, dtype), torch.tensor(bias, device="cuda")
    q_off, q_perm = fa.fastar_bucket_index(i32(q_ids), b)
    k_off, k_perm = fa.fastar_bucket_index(i32(k_ids[:, :, None]), b)
    _, lse_s = fa.fastar_bucket_attention(tq, tk, tv, q_bucket=i32(q_ids), q_perm=q_perm, key_bias=tb,
                                          k_offsets=k_off, k_perm=k_perm, n_bits=b)
    _, lse_d = fa.fastar_bucket_attention(tq, tk, tv, key_bias=tb)
    n_keys = torch.full((H,), nk, dtype=torch.int32, device="cuda")
    rec, stats = fa.fastar_attention_recall(lse_s, lse_d, n_keys, q_bucket=i32(q_ids), k_offsets=k_off,
                                            n_bits=b)
    torch.cuda.synchronize()
    rec, stats = rec.cpu().numpy(), stats.cpu().numpy()
    for h in range(H):
        r_ref, d_ref = oracle.attention_recall(q[h], k[h], oracle.bucket_retained(q_ids[h], k_ids[h]),
                                               bias=bias[h])
        assert np.max(np.abs(rec[h] - r_ref)) <= rtol(dtype)
        assert abs(stats[h, 0] - r_ref.mean()) <= rtol(dtype)
        assert abs(stats[h, 1] - d_ref.mean()) <= 1e-6


@pytest.mark.parametrize("index", [0, 1, 4])
def test_workload_recall_matches_oracle(fa, index):
    """The chunk's AnnSA (over the compressed cache, + ln m) and AnnCA (over
    the kept prompt) recall and density against the oracle's sequence."""
    from kv_compressed_attention_amd.layer import FastARLayer

    w = make_workload(index)
    H, F, T, d = w.k_frames.shape
    npr = 0 if w.prompt_k is None else w.prompt_k.shape[1]
    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries, w.chunk_frames,
                        n_prompt=npr, dtype=TDT[w.dtype], device="cuda")
    layer.set_planes(_up(w.planes, w.dtype))
    for f in range(w.setup_frames):
        layer.merge(_up(w.k_frames[:, f], w.dtype), _up(w.v_frames[:, f], w.dtype), 1, with_index=False)
    q = _up(w.q, w.dtype)
    k_new, v_new = (_up(a, w.dtype) for a in w.frames(w.setup_frames, F))
    pk = _up(w.prompt_k, w.dtype) if npr else None
    pv = _up(w.prompt_v, w.dtype) if npr else None
    layer.step(q, k_new, v_new, pk, pv)
    c = layer.cache
    _, lse_d = fa.fastar_bucket_attention(q, c.rep_k, c.v_mean, key_bias=c.log_count, n_key_list=c.n_groups)
    rec, stats = fa.fastar_attention_recall(layer.lse_self, lse_d, c.n_groups, q_bucket=layer.q_ids,
                                            k_offsets=layer.rep_off, n_bits=w.n_bits)
    if npr:
        _, lse_cd = fa.fastar_bucket_attention(q, pk, pv)
        n_all = torch.full((H,), npr, dtype=torch.int32, device="cuda")
        crec, cstats = fa.fastar_attention_recall(layer.lse_cross, lse_cd, n_all, n_retained=layer.n_kept)
    torch.cuda.synchronize()
    ref = oracle.run_chunk(w, heads=SAMPLE[index], attention=False)
    for h in SAMPLE[index]:
        r = ref[h]
        tc = r["cache"]
        qh = w.q[h].astype(np.float64)
        r_ref, d_ref = oracle.attention_recall(qh, tc.rep_k, oracle.bucket_retained(r["q_ids"], tc.rep_bucket),
                                               bias=tc.log_count)
        assert np.max(np.abs(rec[h].cpu().numpy() - r_ref)) <= rtol(w.dtype), f"head {h} AnnSA recall"
        assert abs(float(stats[h, 1]) - d_ref.mean()) <= 1e-6, f"head {h} AnnSA density"
        if npr:
            keep = np.broadcast_to(r["keep"][None, :], (w.n_queries, npr))
            cr_ref, cd_ref = oracle.attention_recall(qh, w.prompt_k[h], keep)
            assert np.max(np.abs(crec[h].cpu().numpy() - cr_ref)) <= rtol(w.dtype), f"head {h} AnnCA recall"
            assert abs(float(cstats[h, 1]) - cd_ref.mean()) <= 1e-6, f"head {h} AnnCA density"

"""fastar_chunk against the same calls made one by one.

The chunk entry point puts work that does not depend on a launch into extra
workgroups of it: bf16 queries are hashed by the merge's match launch, and
their one-probe index is built by the launch that indexes the
representatives.  Its outputs must equal, bit for bit, those of
fastar_hash_multi, fastar_bucket_index, fastar_tempcache_merge,
fastar_bucket_attention and (with a prompt) fastar_prune_prompt plus the
list-mode attention, called in order on the same inputs: every kernel on the
path is deterministic.  Workload 0 (fp32, prompt, one probe: every hashing in
the hash launch) and 4 (bf16, prompt, two probes: the queries' index in a
launch of its own) cover the other paths and the AnnCA tail; workload 1 is
the layer workload itself.
"""

import numpy as np
import pytest
import torch

from synth import make_workload

pytestmark = pytest.mark.gpu
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _up(a, dtype):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device="cuda").to(TDT[dtype])


def _outputs(layer, prompt):
    c = layer.cache
    names = dict(q_ids=layer.q_ids, q_off=layer.q_off, q_perm=layer.q_perm, k_ids=layer.k_ids,
                 group_of_new=layer.group_of_new, rep_off=layer.rep_off, o_self=layer.o_self,
                 lse_self=layer.lse_self)
    if prompt:
        names.update(p_ids=layer.p_ids, keep=layer.keep, n_kept=layer.n_kept, o_cross=layer.o_cross,
                     lse_cross=layer.lse_cross)
    names.update({"cache_" + n: t for n, t in c.buffers().items()})
    out = {n: t.clone() for n, t in names.items()}
    G = c.n_groups.tolist()
    out["rep_perm"] = [layer.rep_perm[h, :g].clone() for h, g in enumerate(G)]
    if prompt:
        K = layer.n_kept.tolist()
        out["kept_idx"] = [layer.kept_idx[h, :k].clone() for h, k in enumerate(K)]
    return out


@pytest.mark.parametrize("index", [0, 1, 4])
def test_chunk_matches_calls_one_by_one(index):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_compressed_attention_amd.layer import FastARLayer

    w = make_workload(index)
    H, F, T, d = w.k_frames.shape
    prompt = w.prompt_k is not None
    np_ = w.prompt_k.shape[1] if prompt else 0
    layers = []
    for _ in range(2):
        layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries,
                            w.chunk_frames, n_prompt=np_, dtype=TDT[w.dtype], device="cuda")
        layer.set_planes(_up(w.planes, w.dtype))
        layers.append(layer)
    for f in range(w.setup_frames):
        kf, vf = _up(w.k_frames[:, f], w.dtype), _up(w.v_frames[:, f], w.dtype)
        layers[0].merge(kf, vf, 1, with_index=False)
    layers[1].cache.copy_from(layers[0].cache)
    q = _up(w.q, w.dtype)
    k_new, v_new = (_up(a, w.dtype) for a in w.frames(w.setup_frames, F))
    pk = _up(w.prompt_k, w.dtype) if prompt else None
    pv = _up(w.prompt_v, w.dtype) if prompt else None
    layers[0].step(q, k_new, v_new, pk, pv, concurrent=False)
    layers[1].step(q, k_new, v_new, pk, pv, concurrent="chunk")
    torch.cuda.synchronize()
    a, b = _outputs(layers[0], prompt), _outputs(layers[1], prompt)
    for n in a:
        if isinstance(a[n], list):
            assert all(torch.equal(x, y) for x, y in zip(a[n], b[n])), n
        else:
            assert torch.equal(a[n], b[n]), n
    assert int(layers[1].diag[3]) == 0

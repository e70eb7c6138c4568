"""The layer's chunk captured into HIP graphs and replayed.

Every replay must reproduce the eager step bit for bit (every kernel on the
path is deterministic: counters that race only count, and every ordered
result is ranked).  Replays alternate with eager work and synchronisations,
and each one is checked on its own.
"""

import numpy as np
import pytest
import torch

from synth import make_workload

pytestmark = pytest.mark.gpu
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _up(a, dtype):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device="cuda").to(TDT[dtype])


def _outputs(layer):
    c = layer.cache
    names = dict(q_ids=layer.q_ids, q_off=layer.q_off, q_perm=layer.q_perm, k_ids=layer.k_ids,
                 group_of_new=layer.group_of_new, rep_off=layer.rep_off,
                 rep_perm=layer.rep_perm, o_self=layer.o_self, lse_self=layer.lse_self)
    names.update({"cache_" + n: t for n, t in c.buffers().items()})
    out = {n: t.clone() for n, t in names.items()}
    # the index fills only each head's first n_groups entries of rep_perm
    G = c.n_groups.tolist()
    out["rep_perm"] = [out["rep_perm"][h, :g] for h, g in enumerate(G)]
    return out


def _same(a, b):
    if isinstance(a, list):
        return len(a) == len(b) and all(torch.equal(x, y) for x, y in zip(a, b))
    return torch.equal(a, b)


@pytest.mark.parametrize("concurrent", ["chunk", True, False])
@pytest.mark.parametrize("index", [0, 1])
def test_graph_replay_matches_eager(index, concurrent):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_compressed_attention_amd.layer import FastARLayer

    w = make_workload(index)
    H, F, T, d = w.k_frames.shape
    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries,
                        w.chunk_frames, dtype=TDT[w.dtype], device="cuda")
    layer.set_planes(_up(w.planes, w.dtype))
    for f in range(w.setup_frames):
        layer.merge(_up(w.k_frames[:, f], w.dtype), _up(w.v_frames[:, f], w.dtype), 1,
                    with_index=False)
    q = _up(w.q, w.dtype)
    k_new, v_new = (_up(a, w.dtype) for a in w.frames(w.setup_frames, F))
    torch.cuda.synchronize()
    snap = {n: t.clone() for n, t in layer.cache.buffers().items()}

    def restore():
        for n, t in layer.cache.buffers().items():
            t.copy_(snap[n])

    layer.step(q, k_new, v_new, concurrent=concurrent)
    torch.cuda.synchronize()
    ref = _outputs(layer)
    restore()
    graph = layer.capture(q, k_new, v_new, concurrent=concurrent)
    for rep in range(4):
        # eager work between replays: restore the cache, scribble over the
        # outputs, then sync
        restore()
        for t in (layer.o_self, layer.lse_self, layer.q_perm, layer.rep_perm):
            t.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(layer)
        for n, t in ref.items():
            assert _same(got[n], t), f"replay {rep}: {n} differs from the eager step"
        if rep == 1:
            # an eager step in between gives the same result too
            restore()
            layer.step(q, k_new, v_new, concurrent=False if concurrent is not False else "chunk")
            torch.cuda.synchronize()
            for n, t in _outputs(layer).items():
                assert _same(t, ref[n]), f"eager step after replays: {n}"

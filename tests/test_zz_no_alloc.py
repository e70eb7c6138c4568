"""fastar_chunk_noalloc (the allocation-free chunk call, whose workspace is
the library's own per-GPU scratch) against fastar_chunk with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller
input, every output and the merged cache bit for bit equal (the same kernels
run on the same inputs)."""

import numpy as np
import pytest
import torch

from synth import make_workload

pytestmark = pytest.mark.gpu
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _up(a, dtype):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device="cuda").to(TDT[dtype])


def _pair(w):
    """Two layers on the same pre-chunk cache, and the chunk's inputs."""
    from kv_compressed_attention_amd.layer import FastARLayer

    H, F, T, d = w.k_frames.shape
    npr = 0 if w.prompt_k is None else w.prompt_k.shape[1]
    layers = []
    for _ in range(2):
        layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries,
                            w.chunk_frames, n_prompt=npr, dtype=TDT[w.dtype], device="cuda")
        layer.set_planes(_up(w.planes, w.dtype))
        layers.append(layer)
    for f in range(w.setup_frames):
        layers[0].merge(_up(w.k_frames[:, f], w.dtype), _up(w.v_frames[:, f], w.dtype), 1,
                        with_index=False)
    layers[1].cache.copy_from(layers[0].cache)
    q = _up(w.q, w.dtype)
    k, v = (_up(a, w.dtype) for a in w.frames(w.setup_frames, F))
    pk = _up(w.prompt_k, w.dtype) if npr else None
    pv = _up(w.prompt_v, w.dtype) if npr else None
    return layers, (q, k, v, pk, pv)


def _outputs(layer, prompt):
    c = layer.cache
    out = dict(q_ids=layer.q_ids, q_off=layer.q_off, q_perm=layer.q_perm, k_ids=layer.k_ids,
               group_of_new=layer.group_of_new, rep_off=layer.rep_off, o_self=layer.o_self,
               lse_self=layer.lse_self, diag=layer.diag)
    if prompt:
        out.update(p_ids=layer.p_ids, keep=layer.keep, n_kept=layer.n_kept,
                   o_cross=layer.o_cross, lse_cross=layer.lse_cross)
    out.update({"cache_" + n: t for n, t in c.buffers().items()})
    out = {n: t.clone() for n, t in out.items()}
    G = c.n_groups.tolist()
    out["rep_perm"] = [layer.rep_perm[h, :g].clone() for h, g in enumerate(G)]
    if prompt:
        out["kept_idx"] = [layer.kept_idx[h, :k].clone() for h, k in enumerate(layer.n_kept.tolist())]
    return out


@pytest.mark.parametrize("first,second", [(4, 0), (1, 0)])
def test_noalloc_chunk_matches_chunk(first, second):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_compressed_attention_amd.fastar as fb

    for index in (first, second):            # two calls in a row, the second smaller
        w = make_workload(index)
        (ref, got), (q, k, v, pk, pv) = _pair(w)
        prompt = pk is not None
        call_ref = ref._chunk_call(q, k, v, pk, pv, ref.cache)
        call_got = got._chunk_call(q, k, v, pk, pv, got.cache)
        assert call_got.workspace_bytes() <= fb.NOALLOC_SCRATCH_BYTES
        # the counters compare this call only (the set-up merges ran on ref)
        ref.diag.zero_()
        got.diag.zero_()
        call_ref(ref.ws, diag=ref.diag)
        call_got.noalloc(diag=got.diag)
        torch.cuda.synchronize()
        a, b = _outputs(ref, prompt), _outputs(got, prompt)
        for n in a:
            if isinstance(a[n], list):
                assert all(torch.equal(x, y) for x, y in zip(a[n], b[n])), (index, n)
            else:
                assert torch.equal(a[n], b[n]), (index, n)
        assert int(got.diag[3]) == 0 and got.cache.status_code() == 0

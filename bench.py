"""Benchmark of one attention layer's FAST-AR hot path on one MI355X.

A step is one chunk of the per-layer sequence on the layer workload (12 heads,
d=128, 4680 queries = 3 frames x 1560 tokens, a 6-frame KV cache, 12 hash
bits, one probe, bf16): hash the queries and build their bucket index, hash
the chunk's 3 new frames of keys, TempCache-merge them frame by frame into the
compressed cache of the first 3 frames and index the representatives, then
AnnSA bucket attention of the queries over the compressed cache with the
+ ln m bias.  The merge works in place, so each of the K timed steps merges
into a resident copy of the pre-chunk cache of its own (made before the timed
region); after the run the K merged caches are checked to be identical.

A step is one fastar_chunk call, six launches on one stream: the new keys
hashed; the merge's index, match (whose extra workgroups hash the queries)
and apply launches; the representatives' index (whose extra workgroups build
the queries' index); the attention.  --order picks the older call-by-call
orders, on one stream or with the query side on a second one.  The steps are captured
into HIP graphs, --graph-steps of them (each on its own cache) per graph, as
a model captures the chunks of its layers together, and replayed (--eager
launches from Python instead, with per-call event times in "stages_ms").
The attention kernel's duration for the roofline comes from two HIP events
around K launches of it right after the timed region, captured into one
graph and replayed on the stream the events are recorded on (so host
enqueue time stays out of it).

Prints one JSON line.  --gpus N with N > 1 is refused: the library has no
multi-GPU path (heads are independent, so a multi-GPU layer would shard them
with no collective).
"""

from __future__ import annotations

import argparse
import copy
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attention query tokens/s per layer; achieved TFLOP/s vs bf16 MFMA peak"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--graph-steps", type=int, default=10,
                   help="steps captured per HIP graph (each on its own cache, in order, as the "
                        "chunks of a model's layers are captured together)")
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", type=int, default=1, help="synthetic workload index (1, 3 or 4)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true",
                   help="skip the one-bucket (dense, MFMA-bound) attention measurement")
    p.add_argument("--order", choices=["chunk", "serial", "2stream", "split"], default="chunk",
                   help="chunk: one fastar_chunk call per step (default); serial: every call on "
                        "one stream; 2stream: the query index (and AnnCA) on a second stream; "
                        "split: the query hashing on the second stream as well")
    p.add_argument("--eager", action="store_true",
                   help="launch every kernel from Python each step instead of replaying the "
                        "captured HIP graphs (per-stage event times, host-launch bound)")
    return p.parse_args()


def attention_work(q_ids, rep_off, n_bits, H, nq, d, P):
    """Algorithmic bytes and flops of one self-attention launch.

    Bytes: Q and O rows (bf16), lse (fp32), the query's ids and index entry,
    and once per (head, bucket occupied by some query probe) that bucket's
    representative keys and mean values (bf16), bias (fp32) and index entry.
    Flops: 4 d per attended (query, key) pair.
    """
    nb = 1 << n_bits
    seg = np.diff(rep_off, axis=1)                       # keys per bucket [H, nb]
    pairs = 0
    kv_keys = 0
    for h in range(H):
        occ = np.zeros(nb, dtype=bool)
        occ[q_ids[h].reshape(-1)] = True
        kv_keys += int(seg[h][occ].sum())
        pairs += int(seg[h][q_ids[h]].sum())
    qo = H * nq * (2 * d * 2 + 4 + 4 * P + 4)
    kv = kv_keys * (2 * d * 2 + 4 + 4)
    return qo + kv, 4 * d * pairs, pairs


def cpu_baseline(w, min_seconds=10.0, max_reps=20):
    """Time the oracle on the whole chunk (all heads), repeated to >= min_seconds.

    The set-up merges that build the pre-chunk cache are not timed.
    Returns (seconds per chunk, repetitions).
    """
    import oracle
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        setup = []
        for h in range(w.heads):
            tc = oracle.TempCacheOracle(w.dim, w.dtype)
            for f in range(w.setup_frames):
                kf = w.k_frames[h, f].astype(np.float64)
                tc.merge_frame(kf, w.v_frames[h, f], oracle.simhash(kf, w.planes, 1)[:, 0], w.tau)
            setup.append(tc)
        total, reps = 0.0, 0
        while reps < max_reps and (total < min_seconds or reps == 0):
            states = [copy.deepcopy(tc) for tc in setup]
            t0 = time.perf_counter()
            for h in range(w.heads):
                tc = states[h]
                q = w.q[h].astype(np.float64)
                q_ids = oracle.simhash(q, w.planes, w.n_probes)
                oracle.bucket_index(q_ids, w.n_bits)
                for f in range(w.setup_frames, w.n_frames):
                    kf = w.k_frames[h, f].astype(np.float64)
                    tc.merge_frame(kf, w.v_frames[h, f], oracle.simhash(kf, w.planes, 1)[:, 0],
                                   w.tau)
                oracle.bucket_index(tc.rep_bucket, w.n_bits)
                oracle.bucket_attention(q, q_ids, tc.rep_k, tc.v_mean, tc.rep_bucket,
                                        bias=tc.log_count)
            total += time.perf_counter() - t0
            reps += 1
    return total / reps, reps


def dense_one_bucket(dev, reps: int = 5):
    """The attention kernel with all keys in one bucket (dense mode) at the
    rollout size: 12 heads, 4680 queries, 23,400 keys, d = 128, bf16, seeded
    normal inputs.  Every query meets every key, so the kernel is bound by
    its MFMA work and its fraction of the bf16 peak measures MFMA quality.
    reps launches in one HIP graph, replayed between two events."""
    import kv_compressed_attention_amd as fa
    from synth import gaussian

    H, nq, nk, d = 12, 4680, 23400, 128

    def up(a):
        return torch.tensor(a, dtype=torch.float32, device=dev).to(torch.bfloat16)

    q, k, v = up(gaussian((H, nq, d), 501, "bf16")), up(gaussian((H, nk, d), 502, "bf16")), \
        up(gaussian((H, nk, d), 503, "bf16"))
    out = torch.empty(H, nq, d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(H, nq, dtype=torch.float32, device=dev)
    fa.fastar_bucket_attention(q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fa.fastar_bucket_attention(q, k, v, out=out, lse=lse)
    graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    tflops = 4.0 * d * nq * nk * H / (ms * 1e-3) / 1e12
    return {"workload": f"one_bucket_bf16_h{H}_d{d}_q{nq}_k{nk}", "bound": "mfma", "launch_ms": ms,
            "tflops": tflops, "frac_bf16_mfma_peak": tflops / PEAK_BF16_TFLOPS}


def recorded_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter passes, if
    they were taken on this workload with the current attention sources
    (else None)."""
    import glob
    import hashlib
    import re

    src = b"".join(open(os.path.join(ROOT, "kv_compressed_attention_amd", "csrc", f), "rb").read()
                   for f in ("attention.hip", "common.h"))
    digest = hashlib.sha256(src).hexdigest()[:16]
    for path in glob.glob(os.path.join(ROOT, "profiles", "attn_bf16_*.md")):
        m = re.search(r"traffic_bytes_per_launch=(\d+) source_sha256=([0-9a-f]+) workload=(\S+)",
                      open(path).read())
        if m and m.group(2) == digest and m.group(3) == workload:
            return int(m.group(1))
    return None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: libfastar has no multi-GPU path (heads are "
              "independent and would shard across GPUs with no collective)", file=sys.stderr)
        sys.exit(2)
    import kv_compressed_attention_amd as fa
    from kv_compressed_attention_amd.layer import FastARLayer
    from synth import make_workload

    dev = torch.device("cuda:0")
    w = make_workload(args.workload)
    H, F, T, d = w.k_frames.shape
    nq = w.n_queries
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a):
        return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device=dev).to(tdt)

    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, nq, w.chunk_frames,
                        dtype=tdt, device=dev)
    layer.set_planes(up(w.planes))
    q = up(w.q)
    for f in range(w.setup_frames):
        layer.merge(up(w.k_frames[:, f]), up(w.v_frames[:, f]), 1, with_index=False)
    k_new, v_new = (up(a) for a in w.frames(w.setup_frames, F))
    torch.cuda.synchronize()
    # the merge is in place: every timed step gets a resident copy of the
    # pre-chunk cache of its own, so the K steps are identical work and the
    # timed region holds only the hot path
    pristine = layer.cache
    caches = []
    for _ in range(args.steps):
        c = fa.TempCache(H, d, F * T, T, w.n_bits, tdt, dev)
        c.copy_from(pristine)
        caches.append(c)
    scratch = fa.TempCache(H, d, F * T, T, w.n_bits, tdt, dev)

    # a plain 64 MiB device copy before the timed region: the calibration
    # kernel for the FETCH_SIZE / WRITE_SIZE counter passes
    cal_src = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    del cal_src, cal_dst

    timing = {}
    concurrent = {"chunk": "chunk", "serial": False, "2stream": True, "split": "split"}[args.order]

    def warm_step():
        scratch.copy_from(pristine)
        layer.step(q, k_new, v_new, cache=scratch, concurrent=concurrent)

    for _ in range(args.warmup):
        warm_step()
    torch.cuda.synchronize()
    if args.eager:
        def step(i):
            layer.step(q, k_new, v_new, cache=caches[i], concurrent=concurrent, timing=timing)
    else:
        G = max(1, args.graph_steps)
        graphs = [layer.capture(q, k_new, v_new, concurrent=concurrent, caches=caches[i:i + G])
                  for i in range(0, args.steps, G)]
        warm = layer.capture(q, k_new, v_new, cache=scratch, concurrent=concurrent)
        for _ in range(args.warmup):
            scratch.copy_from(pristine)
            warm.replay()
        torch.cuda.synchronize()

        def step(i):
            # one graph launch runs steps i .. i + G - 1
            if i % G == 0:
                graphs[i // G].replay()
    # timed region: exactly K steps (eager: with HIP events around the
    # stages, each recorded on the stream its stage is enqueued on)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    t_enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {s: float(np.mean([a.elapsed_time(b) for a, b in v])) for s, v in timing.items()}
    if "attention" not in stage_ms:
        # the attention kernel's average launch duration: K launches on the
        # inputs and buffers of the last timed step, captured in one HIP graph
        # and replayed between two events on the stream they run on (host
        # enqueue time, which a per-launch event pair can include, stays out)
        torch.cuda.synchronize()
        g_attn = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_attn):
            for _ in range(args.steps):
                layer.self_attention(q, None, caches[-1])
        g_attn.replay()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        g_attn.replay()
        ev1.record()
        torch.cuda.synchronize()
        stage_ms["attention"] = ev0.elapsed_time(ev1) / args.steps
    check_steps_agree(layer, caches)

    ms = wall * 1e3 / args.steps
    q_ids = layer.q_ids.cpu().numpy()
    rep_off = layer.rep_off.cpu().numpy()
    nbytes, flops, pairs = attention_work(q_ids, rep_off, w.n_bits, H, nq, d, w.n_probes)
    t_att = stage_ms["attention"] * 1e-3
    achieved_gbs = nbytes / t_att / 1e9
    tflops = flops / t_att / 1e12
    ai = flops / nbytes
    out = {
        "metric": METRIC,
        "value": nq / (ms * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "heads": H, "head_dim": d, "queries": nq,
                   "cache_frames": F, "tokens_per_frame": T, "new_frames": w.chunk_frames,
                   "n_bits": w.n_bits, "n_probes": w.n_probes, "tau": w.tau},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / PEAK_HBM_GBS, "traffic": recorded_traffic(w.name),
                     "kernel": "attn_bf16_kernel (fastar_bucket_attention, bucket mode)",
                     "bytes_per_launch": nbytes, "launch_ms": stage_ms["attention"]},
        "attention": {"tflops": tflops, "frac_bf16_mfma_peak": tflops / PEAK_BF16_TFLOPS,
                      "arith_intensity_flop_per_byte": ai,
                      "roofline_tflops": min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3),
                      "attended_pairs": pairs,
                      "query_tokens_per_s": nq / t_att,
                      "compressed_keys_per_head": ngb_after(layer, caches[-1])},
        "launch": ("eager" if args.eager else f"hip_graph{max(1, args.graph_steps)}") + "_" + args.order,
        "stages_ms": stage_ms,
        "host_enqueue_ms_per_step": t_enq * 1e3 / args.steps,
        "diag": layer.diag.tolist(),
    }
    if not args.no_dense:
        out["dense_one_bucket"] = dense_one_bucket(dev)
    if not args.no_cpu_baseline:
        per_step, reps = cpu_baseline(w)
        out["cpu_baseline"] = {"value": nq / per_step, "unit": "query tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the whole chunk, all {H} heads (hash queries, hash and "
                                         f"merge {w.chunk_frames} frames, index, bucket "
                                         f"attention; cache restore not needed), {reps} "
                                         f"repetitions of {per_step:.2f} s, one thread"}
    print(json.dumps(out))


def ngb_after(layer, cache):
    return int(cache.n_groups.max().item())


def check_steps_agree(layer, caches):
    """Every timed step did the same work: the caches it merged into agree."""
    ref = caches[0]
    for c in caches[1:]:
        for n, t in c.buffers().items():
            if not torch.equal(t, ref.buffers()[n]):
                raise RuntimeError(f"timed steps disagree on the merged cache ({n})")


if __name__ == "__main__":
    main()

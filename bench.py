"""Benchmark of one attention layer's FAST-AR hot path on one MI355X.

Default workload: the wide world-model shape (24 heads, d = 128, a chunk of
4 frames x 2048 tokens = 8192 queries, a 16-frame KV cache, 14 hash bits,
two probes per query, a 512-token prompt, bf16).  A step is one chunk of the
whole per-layer sequence, one fastar_chunk call: hash the queries, the 4 new
frames' keys and the prompt keys; TempCache-merge the new frames into the
compressed cache of the first 12 frames and index the representatives;
index the queries; AnnSA bucket self-attention with the + ln m bias; AnnCA
prune of the prompt and cross-attention over the kept prompt tokens.

Cold and hot.  The merge works in place, so every timed step merges into a
resident copy of the pre-chunk cache of its own (made before the timed
region; afterwards the K merged caches are checked to be identical, so every
step did the same work).  In the cold run (the headline) every step also has
its own copy of the queries, new frames and prompt: one step touches more
bytes than the 256 MB Infinity Cache holds, so each step starts on inputs no
recent step has read.  The hot run shares one copy of the inputs between the
steps.  Steps are captured into HIP graphs, --graph-steps per graph, and
replayed; the timed region brackets exactly K steps with synchronisation.

Kernel durations.  Each stage of the chunk is also captured on its own, K
launches on the K steps' buffers in one HIP graph, and replayed between two
HIP events on the stream it runs on; duration = elapsed / K.  Algorithmic
bytes per launch (from the actual bucket occupancy and merge outcome) over
that duration give each kernel's fraction of the HBM peak; the roofline
object is the stage with the largest duration.

Also reported: the oracle on the host's cores (one thread, then one process
per core over heads; taken before the GPU is first used), the other
workloads (the layer, AnnCA and rollout shapes; --no-extra skips them), the
one-bucket (dense, MFMA-bound) attention, and the pages' own end-to-end
figures for context.  Prints one JSON line.  --gpus N with N > 1 is refused:
the library has no multi-GPU path (heads are independent, so a multi-GPU
layer would shard them with no collective).
"""

from __future__ import annotations

import argparse
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
FLUSH_BYTES = 512 << 20   # > the 256 MB Infinity Cache

# The pages' end-to-end figures (another system, other hardware): context only
PAGES = {
    "end_to_end_speedup_vs_dense_flashattention3":
        "up to 5-10x (paperlayer.ai summary, abstract and introduction; the introduction "
        "states a single H100; precision not stated)",
    "dense_flashattention3_3000_frames":
        "about 11 minutes, memory growing throughout (paper.rainbus.top, motivation; "
        "hardware not stated there)",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--graph-steps", type=int, default=10,
                   help="steps captured per HIP graph (each on its own buffers, in order, as "
                        "the chunks of a model's layers are captured together)")
    p.add_argument("--workload", type=int, default=4,
                   help="synthetic workload of the headline (1, 3 or 4; 4 = wide)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true",
                   help="skip the one-bucket (dense, MFMA-bound) attention measurement")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the layer, AnnCA and rollout workloads")
    p.add_argument("--no-hot", action="store_true", help="skip the hot (shared inputs) run")
    p.add_argument("--cpu-sample-heads", type=int, default=0,
                   help="heads of the one-thread oracle sample (0: enough for about 10 s)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------
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
        ids = q_ids[h].reshape(nq, -1)
        # keys of the distinct probe buckets of each query
        same = ids[:, 1:] == ids[:, :1] if ids.shape[1] > 1 else np.zeros((nq, 0), bool)
        pairs += int(seg[h][ids[:, 0]].sum())
        if ids.shape[1] > 1:
            pairs += int(seg[h][ids[:, 1]][~same[:, 0]].sum())
    qo = H * nq * (2 * d * 2 + 4 + 4 * P + 4)
    kv = kv_keys * (2 * d * 2 + 4 + 4)
    return qo + kv, 4 * d * pairs, pairs


def cross_work(n_kept, H, nq, npr, d):
    """Bytes and flops of the cross-attention over the kept prompt tokens
    (Q, O and lse per query; the kept keys' K and V rows and list entries
    once per head) and of the prune (query ids, prompt ids, mask, list)."""
    kept = int(np.sum(n_kept))
    att_bytes = H * nq * (2 * d * 2 + 4) + kept * (2 * d * 2 + 4)
    flops = 4 * d * nq * kept
    return att_bytes, flops


def merge_work(n_before, n_after, group_of_new, H, F, T, d, s=2):
    """Algorithmic bytes of one merge call of F frames (all heads), from its
    outcome: the new frames' keys and values read; the previous frame's
    keys (the candidates of frame 0) read once; per group the call touches
    (every frontier group a chunk token extends, and every new group) its
    float32 value sum read (if it existed) and written, its mean value and
    key written, its count, ln count and bucket; each token's bucket read and
    group written, and the frontier written."""
    total = 0
    for h in range(H):
        g = group_of_new[h]
        ext = np.unique(g[(g >= 0) & (g < n_before[h])]).size
        new = int(n_after[h] - n_before[h])
        total += F * T * (2 * d * s + 8) + T * d * s + T * 4
        total += ext * (2 * 4 * d + 2 * d * s + 12) + new * (4 * d + 2 * d * s + 12)
    return total


def hash_work(rows, d, P, s=2):
    return rows * (d * s + 4 * P)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host's cores (before the GPU is touched)
# ---------------------------------------------------------------------------
_CPU_W = None


def _oracle_chunk_head(h):
    """The chunk's sequence for head h: set-up merges untimed, then hash,
    merge, index, self-attention, prune and cross-attention timed.
    Returns seconds."""
    import oracle
    from threadpoolctl import threadpool_limits

    w = _CPU_W
    with threadpool_limits(limits=1):
        tc = oracle.TempCacheOracle(w.dim, w.dtype)
        for f in range(w.setup_frames):
            kf = w.k_frames[h, f].astype(np.float64)
            tc.merge_frame(kf, w.v_frames[h, f], oracle.simhash(kf, w.planes, 1)[:, 0], w.tau)
        t0 = time.perf_counter()
        q = w.q[h].astype(np.float64)
        q_ids = oracle.simhash(q, w.planes, w.n_probes)
        oracle.bucket_index(q_ids, w.n_bits)
        for f in range(w.setup_frames, w.n_frames):
            kf = w.k_frames[h, f].astype(np.float64)
            tc.merge_frame(kf, w.v_frames[h, f], oracle.simhash(kf, w.planes, 1)[:, 0], w.tau)
        oracle.bucket_index(tc.rep_bucket, w.n_bits)
        oracle.bucket_attention(q, q_ids, tc.rep_k, tc.v_mean, tc.rep_bucket, bias=tc.log_count)
        if w.prompt_k is not None:
            pk = w.prompt_k[h].astype(np.float64)
            p_ids = oracle.simhash(pk, w.planes, 1)[:, 0]
            _, kept = oracle.prune_prompt(q_ids, p_ids)
            oracle.cross_attention(q, pk, w.prompt_v[h], kept)
        return time.perf_counter() - t0


def cpu_baseline(w, sample_heads=0):
    """Oracle time per chunk (all heads), one thread and all cores.

    One thread: `sample_heads` heads in this process (default: as many as
    take about 10 s, at least one), scaled to all heads.  All cores: one
    process per core (fork, at most 16: the host share of one GPU), each
    running one head; the slowest head's time, scaled by heads / processes.
    """
    import multiprocessing as mp

    global _CPU_W
    _CPU_W = w
    H = w.heads
    t1 = [_oracle_chunk_head(0)]
    n1 = sample_heads or max(1, min(H, int(10.0 / max(t1[0], 1e-3))))
    for h in range(1, n1):
        t1.append(_oracle_chunk_head(h))
    one = float(np.mean(t1)) * H
    host = os.cpu_count() or 1
    procs = max(1, min(host, 16, H))
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        tp = pool.map(_oracle_chunk_head, list(range(procs)))
    allc = max(tp) * H / procs
    return {"one_thread_s_per_chunk": one, "one_thread_heads": n1,
            "all_cores_s_per_chunk": allc, "processes": procs, "host_cpus": host}


# ---------------------------------------------------------------------------
# GPU helpers
# ---------------------------------------------------------------------------
def graph_time(fns, before=None, reps=1):
    """Capture the callables fns (in order) into one HIP graph, replay it once
    (warm-up), then time `reps` replays between two events on the current
    stream; returns ms per callable.  before(): untimed work before each
    replay (e.g. restoring in-place state)."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    if before:
        before()
    g.replay()
    torch.cuda.synchronize()
    total = 0.0
    for _ in range(reps):
        if before:
            before()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
    del g
    return total / reps / len(fns)


class Setup:
    """A workload's layer, its pre-chunk cache, and per-step copies."""

    def __init__(self, w, dev, steps, rotate, match="lsh"):
        import kv_compressed_attention_amd as fa
        from kv_compressed_attention_amd.layer import FastARLayer

        self.w, self.dev = w, dev
        H, F, T, d = w.k_frames.shape
        self.H, self.F, self.T, self.d = H, F, T, d
        self.tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        npr = 0 if w.prompt_k is None else w.prompt_k.shape[1]
        self.npr = npr
        self.layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries,
                                 w.chunk_frames, n_prompt=npr, dtype=self.tdt, device=dev, match=match)
        self.layer.set_planes(self.up(w.planes))
        for f in range(w.setup_frames):
            self.layer.merge(self.up(w.k_frames[:, f]), self.up(w.v_frames[:, f]), 1,
                             with_index=False)
        q = self.up(w.q)
        k_new, v_new = (self.up(a) for a in w.frames(w.setup_frames, F))
        pk = self.up(w.prompt_k) if npr else None
        pv = self.up(w.prompt_v) if npr else None
        torch.cuda.synchronize()
        self.pristine = self.layer.cache
        self.caches = []
        for _ in range(steps):
            c = fa.TempCache(H, d, F * T, T, w.n_bits, self.tdt, dev)
            c.copy_from(self.pristine)
            self.caches.append(c)
        self.scratch = fa.TempCache(H, d, F * T, T, w.n_bits, self.tdt, dev)

        def clone(t):
            return None if t is None else t.clone()
        n_in = steps if rotate else 1
        self.inputs = [(q, k_new, v_new, pk, pv)] + [
            tuple(clone(t) for t in (q, k_new, v_new, pk, pv)) for _ in range(n_in - 1)]
        torch.cuda.synchronize()

    def up(self, a):
        return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32,
                            device=self.dev).to(self.tdt)

    def inp(self, i):
        return self.inputs[i % len(self.inputs)]

    def restore(self):
        for c in self.caches:
            c.copy_from(self.pristine)

    def step(self, i, cache=None):
        q, k, v, pk, pv = self.inp(i)
        self.layer.step(q, k, v, pk, pv, cache=self.caches[i] if cache is None else cache)

    def check_steps_agree(self):
        """Every timed step did the same work: the caches it merged into agree."""
        ref = self.caches[0]
        for c in self.caches[1:]:
            for n, t in c.buffers().items():
                if not torch.equal(t, ref.buffers()[n]):
                    raise RuntimeError(f"timed steps disagree on the merged cache ({n})")


def timed_steps(st, steps, warmup, graph_steps):
    """Warm up, capture the K steps into graphs of graph_steps, then the timed
    region: exactly K steps (graph replays) bracketed by synchronisation.
    Returns wall seconds of the timed region."""
    for i in range(warmup):
        st.scratch.copy_from(st.pristine)
        st.step(i, cache=st.scratch)
    torch.cuda.synchronize()
    G = max(1, graph_steps)
    graphs = []
    for i0 in range(0, steps, G):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(i0, min(steps, i0 + G)):
                st.step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    # the captures merged nothing; the caches are still pristine
    t0 = time.perf_counter()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st.check_steps_agree()
    del graphs
    return wall


def stage_times(st, steps):
    """Each stage of the chunk on its own (cold: step i's buffers), K
    launches per graph; ms per launch, plus the algorithmic work."""
    import kv_compressed_attention_amd.fastar as fb

    L, w = st.layer, st.w
    H, d = st.H, st.d
    idx = list(range(steps))
    out = {}

    def run(name, make, before=None):
        out[name] = graph_time([make(i) for i in idx], before=before)

    run("hash_keys_prompt", lambda i: (lambda: fb.fastar_hash_multi(
        [st.inp(i)[1]] + ([st.inp(i)[3]] if st.npr else []), L.planes, w.n_bits,
        [1] + ([1] if st.npr else []), buckets=[L.k_ids] + ([L.p_ids] if st.npr else []),
        diag=L.diag)))
    run("hash_queries", lambda i: (lambda: fb.fastar_hash_multi(
        [st.inp(i)[0]], L.planes, w.n_bits, [w.n_probes], buckets=[L.q_ids], diag=L.diag)))
    run("index_queries", lambda i: (lambda: fb.fastar_bucket_index(
        L.q_ids, w.n_bits, offsets=L.q_off, perm=L.q_perm, ws=L.ws_q)))
    # the merge is in place: the caches are restored before each replay
    run("merge", lambda i: (lambda: fb.fastar_tempcache_merge(
        st.caches[i], st.inp(i)[1], st.inp(i)[2], L.k_ids.view(H, -1), w.chunk_frames, w.tau,
        group_of_new=L.group_of_new, rep_offsets=L.rep_off, rep_perm=L.rep_perm, ws=L.ws,
        diag=L.diag, opts=L.opts)), before=st.restore)
    n_before = st.pristine.n_groups.cpu().numpy()
    n_after = st.caches[-1].n_groups.cpu().numpy()
    gon = L.group_of_new.cpu().numpy()
    run("attention_self", lambda i: (lambda: fb.fastar_bucket_attention(
        st.inp(i)[0], st.caches[i].rep_k, st.caches[i].v_mean, q_bucket=L.q_ids, q_perm=L.q_perm,
        key_bias=st.caches[i].log_count, k_offsets=L.rep_off, k_perm=L.rep_perm,
        n_bits=w.n_bits, out=L.o_self, lse=L.lse_self)))
    if st.npr:
        run("prune", lambda i: (lambda: fb.fastar_prune_prompt(
            L.q_ids, L.p_ids.view(H, -1), w.n_bits, keep=L.keep, kept_idx=L.kept_idx,
            n_kept=L.n_kept)))
        run("attention_cross", lambda i: (lambda: fb.fastar_bucket_attention(
            st.inp(i)[0], st.inp(i)[3], st.inp(i)[4], key_list=L.kept_idx, n_key_list=L.n_kept,
            out=L.o_cross, lse=L.lse_cross)))
    torch.cuda.synchronize()

    nq, P, T, Fc = w.n_queries, w.n_probes, st.T, w.chunk_frames
    q_ids = L.q_ids.cpu().numpy()
    rep_off = L.rep_off.cpu().numpy()
    a_bytes, a_flops, pairs = attention_work(q_ids, rep_off, w.n_bits, H, nq, d, P)
    kern = {}

    def put(name, nbytes, flops=None, kernel=""):
        ms = out[name]
        gbs = nbytes / (ms * 1e-3) / 1e9
        e = {"kernel": kernel, "launch_ms": ms, "bytes_per_launch": int(nbytes), "achieved_gbs": gbs,
             "frac_hbm": gbs / PEAK_HBM_GBS}
        if flops is not None:
            e["tflops"] = flops / (ms * 1e-3) / 1e12
        kern[name] = e

    put("attention_self", a_bytes, a_flops, "attn_bf16_kernel<128, P, 0> (bucket mode)")
    put("hash_keys_prompt", hash_work(H * (Fc * T + st.npr), d, 1), None, "hash_bf16_kernel<128>")
    put("hash_queries", hash_work(H * nq, d, P), None, "hash_bf16_kernel<128>")
    put("index_queries", H * nq * (4 * P + 4) + H * ((1 << w.n_bits) + 1) * 4, None,
        "bucket index of the queries")
    m_bytes = merge_work(n_before, n_after, gon, H, Fc, T, d)
    m_bytes += int(n_after.sum()) * 8 + H * ((1 << w.n_bits) + 1) * 4   # the representatives' index
    put("merge", m_bytes, None, "tc_index + tc_match + tc_apply + representatives' index")
    extra = {"attended_pairs": pairs, "compressed_keys_per_head_max": int(n_after.max()),
             "compressed_keys_per_head_mean": float(n_after.mean())}
    if st.npr:
        n_kept = L.n_kept.cpu().numpy()
        c_bytes, c_flops = cross_work(n_kept, H, nq, st.npr, d)
        put("attention_cross", c_bytes, c_flops, "attn_bf16_kernel<128, 1, 1> (key-list mode)")
        put("prune", H * nq * 4 * P + H * st.npr * (4 + 1 + 4) + H * 4, None, "prune")
        extra["prompt_kept_per_head_mean"] = float(n_kept.mean())
        extra["prompt_prune_ratio"] = 1.0 - float(n_kept.mean()) / st.npr
    return kern, extra


def recall_stats(st, i=0):
    """AnnSA's (and with a prompt AnnCA's) attention recall and density on
    step i's merged cache: recall(q) = exp(lse_sparse - lse_dense), the dense
    attention over the same keys and bias, both from the attention kernel
    (the pages' measure of sparsity: the dense mass the retained entries
    keep).  Means over queries and heads."""
    import kv_compressed_attention_amd.fastar as fb

    L, w, c = st.layer, st.w, st.caches[i]
    q = st.inp(i)[0]
    _, lse_s = fb.fastar_bucket_attention(q, c.rep_k, c.v_mean, q_bucket=L.q_ids, q_perm=L.q_perm,
                                          key_bias=c.log_count, k_offsets=L.rep_off, k_perm=L.rep_perm,
                                          n_bits=w.n_bits)
    _, lse_d = fb.fastar_bucket_attention(q, c.rep_k, c.v_mean, key_bias=c.log_count,
                                          n_key_list=c.n_groups)
    _, stats = fb.fastar_attention_recall(lse_s, lse_d, c.n_groups, q_bucket=L.q_ids, k_offsets=L.rep_off,
                                          n_bits=w.n_bits, want_recall=False)
    s = stats.cpu().numpy()
    out = {"annsa": {"recall": float(s[:, 0].mean()), "density": float(s[:, 1].mean()),
                     "over": "the compressed cache with its + ln m bias"}}
    if st.npr:
        pk, pv = st.inp(i)[3], st.inp(i)[4]
        _, lse_cs = fb.fastar_bucket_attention(q, pk, pv, key_list=L.kept_idx, n_key_list=L.n_kept)
        _, lse_cd = fb.fastar_bucket_attention(q, pk, pv)
        n_all = torch.full((st.H,), st.npr, dtype=torch.int32, device=q.device)
        _, cs = fb.fastar_attention_recall(lse_cs, lse_cd, n_all, n_retained=L.n_kept, want_recall=False)
        cs = cs.cpu().numpy()
        out["annca"] = {"recall": float(cs[:, 0].mean()), "density": float(cs[:, 1].mean()),
                        "over": "the prompt"}
    return out


def flushed_chunk_ms(st, flush, i):
    """One eager chunk on step i's buffers after a 512 MB write (the
    Infinity Cache flushed, and the GPU busy while the host enqueues), timed
    between two events."""
    flush.zero_()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    st.step(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def dense_one_bucket(dev, reps: int = 5):
    """The attention kernel with all keys in one bucket (dense mode) at the
    rollout size: 12 heads, 4680 queries, 23,400 keys, d = 128, bf16, seeded
    normal inputs.  Every query meets every key, so the kernel is bound by
    its MFMA work and its fraction of the bf16 peak measures MFMA quality."""
    import kv_compressed_attention_amd as fa
    from synth import gaussian

    H, nq, nk, d = 12, 4680, 23400, 128

    def up(a):
        return torch.tensor(a, dtype=torch.float32, device=dev).to(torch.bfloat16)

    q, k, v = up(gaussian((H, nq, d), 501, "bf16")), up(gaussian((H, nk, d), 502, "bf16")), \
        up(gaussian((H, nk, d), 503, "bf16"))
    out = torch.empty(H, nq, d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(H, nq, dtype=torch.float32, device=dev)
    ms = graph_time([lambda: fa.fastar_bucket_attention(q, k, v, out=out, lse=lse)] * reps)
    tflops = 4.0 * d * nq * nk * H / (ms * 1e-3) / 1e12
    return {"workload": f"one_bucket_bf16_h{H}_d{d}_q{nq}_k{nk}", "bound": "mfma", "launch_ms": ms,
            "tflops": tflops, "frac_bf16_mfma_peak": tflops / PEAK_BF16_TFLOPS}


def recorded_traffic(workload: str, kernel_file: str):
    """HBM bytes per launch of the roofline kernel from the committed counter
    passes, if they were taken on this workload with the current sources of
    that kernel (else None)."""
    import glob
    import hashlib
    import re

    src = b"".join(open(os.path.join(ROOT, "kv_compressed_attention_amd", "csrc", f), "rb").read()
                   for f in (kernel_file, "common.h"))
    digest = hashlib.sha256(src).hexdigest()[:16]
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        for m in re.finditer(r"traffic_bytes_per_launch=(\d+) source_sha256=([0-9a-f]+) workload=(\S+)",
                             open(path).read()):
            if m.group(2) == digest and m.group(3) == workload:
                return int(m.group(1))
    return None


KERNEL_FILES = {"attention_self": "attention.hip", "attention_cross": "attention.hip",
                "hash_keys_prompt": "hash.hip", "hash_queries": "hash.hip",
                "merge": "tempcache.hip", "index_queries": "index.hip", "prune": "prune.hip"}


def measure_workload(w, dev, steps, warmup, graph_steps, hot=True, match="lsh"):
    """Cold (rotated inputs) and, optionally, hot chunk steps plus per-stage
    kernel times of workload w (TempCache's match: "lsh" or "quant")."""
    st = Setup(w, dev, steps, rotate=True, match=match)
    res = {"cold_s": timed_steps(st, steps, warmup, graph_steps)}
    if hot:
        st_hot_inputs = st.inputs
        st.inputs = st.inputs[:1]
        st.restore()
        res["hot_s"] = timed_steps(st, steps, warmup, graph_steps)
        st.inputs = st_hot_inputs
    st.restore()
    res["kernels"], res["extra"] = stage_times(st, steps)
    res["recall"] = recall_stats(st)
    ng = st.caches[0].n_groups.cpu().numpy()
    res["cache_density"] = float(ng.mean()) / (w.n_frames * st.T)
    res["diag"] = st.layer.diag.tolist()
    res["setup"] = st
    return res


def rollout(w, dev, flush):
    """The rollout workload as a stream of chunks from an empty cache: every
    3 frames one fastar_chunk (queries: the workload's 4680, the chunk
    sequence's shape), each timed cold (after a 512 MB write) between two
    events; per chunk the time, the compressed keys per head, the density
    (compressed keys / raw keys so far) and the compressed cache's bytes."""
    from kv_compressed_attention_amd.layer import FastARLayer

    H, F, T, d = w.k_frames.shape
    tdt = torch.bfloat16
    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries, 3,
                        dtype=tdt, device=dev)

    def up(a):
        return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device=dev).to(tdt)
    layer.set_planes(up(w.planes))
    q = up(w.q)
    chunks = [tuple(up(a) for a in w.frames(3 * c, 3 * c + 3)) for c in range(F // 3)]
    # the calls' argument blocks are built before the timed calls
    for k, v in chunks:
        layer._chunk_call(q, k, v, None, None, layer.cache)
    torch.cuda.synchronize()
    group_bytes = 2 * d * 2 + 4 * d + 4 + 4 + 4      # key, mean, float32 sum, count, ln m, bucket
    out = []
    for c, (k, v) in enumerate(chunks):
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.step(q, k, v)
        e1.record()
        torch.cuda.synchronize()
        ng = layer.cache.n_groups.cpu().numpy()
        out.append({"chunk": c, "frames": 3 * c + 3, "ms": e0.elapsed_time(e1),
                    "keys_per_head": float(ng.mean()),
                    "density": float(ng.mean()) / (3 * (c + 1) * T),
                    "cache_mb": float(ng.sum()) * group_bytes / 1e6})
    if layer.cache.status_code() != 0:
        raise RuntimeError("rollout cache overflowed")
    import kv_compressed_attention_amd.fastar as fb
    c = layer.cache
    _, lse_d = fb.fastar_bucket_attention(q, c.rep_k, c.v_mean, key_bias=c.log_count, n_key_list=c.n_groups)
    _, stats = fb.fastar_attention_recall(layer.lse_self, lse_d, c.n_groups, q_bucket=layer.q_ids,
                                          k_offsets=layer.rep_off, n_bits=w.n_bits, want_recall=False)
    s = stats.cpu().numpy()
    out[-1]["annsa_recall"] = float(s[:, 0].mean())
    out[-1]["annsa_density"] = float(s[:, 1].mean())
    return out


def tau_sweep(w, dev, taus, match="lsh", representative="last"):
    """TempCache's threshold swept on workload w (paperlayer.ai appendix C,
    tau 0.9 -> 0.5): per tau the chunk time (cold, after a 512 MB write), the
    compressed cache's density (groups / raw keys), AnnSA's recall, and the
    merging's error: dense attention over the compressed cache (+ ln m, all
    groups) against dense attention over the raw frames, as the mean relative
    L2 error of the outputs and of the normalisers' ratio (exp(lse_comp -
    lse_raw), 1 when the merged groups keep every raw key's mass).
    representative: the groups' representative key (last, mean or medoid)."""
    import kv_compressed_attention_amd.fastar as fb
    from kv_compressed_attention_amd.layer import FastARLayer

    H, F, T, d = w.k_frames.shape
    tdt = torch.bfloat16

    def up(a):
        return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device=dev).to(tdt)
    q = up(w.q)
    raw_k = up(w.k_frames.reshape(H, F * T, d))
    raw_v = up(w.v_frames.reshape(H, F * T, d))
    o_raw, lse_raw = fb.fastar_bucket_attention(q, raw_k, raw_v)
    k_new, v_new = (up(a) for a in w.frames(w.setup_frames, F))
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    out = []
    for tau in taus:
        layer = FastARLayer(H, d, w.n_bits, w.n_probes, tau, T, F * T, w.n_queries, w.chunk_frames,
                            dtype=tdt, device=dev, match=match, representative=representative)
        layer.set_planes(up(w.planes))
        for f in range(w.setup_frames):
            layer.merge(up(w.k_frames[:, f]), up(w.v_frames[:, f]), 1, with_index=False)
        layer._chunk_call(q, k_new, v_new, None, None, layer.cache)
        torch.cuda.synchronize()
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.step(q, k_new, v_new)
        e1.record()
        torch.cuda.synchronize()
        c = layer.cache
        o_c, lse_c = fb.fastar_bucket_attention(q, c.rep_k, c.v_mean, key_bias=c.log_count,
                                                n_key_list=c.n_groups)
        _, rs = fb.fastar_attention_recall(layer.lse_self, lse_c, c.n_groups, q_bucket=layer.q_ids,
                                           k_offsets=layer.rep_off, n_bits=w.n_bits, want_recall=False)
        rel = ((o_c.float() - o_raw.float()).norm(dim=2) / o_raw.float().norm(dim=2).clamp_min(1e-30))
        ng = c.n_groups.cpu().numpy()
        out.append({"tau": tau, "chunk_ms": e0.elapsed_time(e1),
                    "cache_density": float(ng.mean()) / (F * T),
                    "annsa_recall": float(rs[:, 0].mean().item()),
                    "merge_rel_l2_error": float(rel.mean().item()),
                    "mass_ratio": float(torch.exp(lse_c - lse_raw).mean().item())})
        del layer
    return out


def lsh_tables_sweep(w, dev, configs, reps=5):
    """Several LSH tables and more probes per table for AnnSA and AnnCA
    (paperlayer.ai section 2: LSH probes buckets in several tables) on
    workload w: per (tables, probes per table) the chunk time (cold: a 512 MB
    write before each of reps chunks, each merging into its own copy of the
    pre-chunk cache; median), the self-attention launch alone (hot, median of
    reps), and AnnSA's mean recall and density against dense attention over
    the compressed cache.  Table 0 is the workload's planes; further tables
    draw their own."""
    from dataclasses import replace
    import kv_compressed_attention_amd.fastar as fb
    from kv_compressed_attention_amd.layer import FastARLayer

    H, F, T, d = w.k_frames.shape
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    npr = 0 if w.prompt_k is None else w.prompt_k.shape[1]

    def up(a):
        return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device=dev).to(tdt)
    q = up(w.q)
    k_new, v_new = (up(a) for a in w.frames(w.setup_frames, F))
    pk = up(w.prompt_k) if npr else None
    pv = up(w.prompt_v) if npr else None
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    out = []
    for L, P in configs:
        if P > w.n_bits + 1:
            continue
        extra = np.random.default_rng(900 + L).standard_normal((max(L - 1, 0), w.n_bits, d))
        planes = np.concatenate([w.planes[None], extra]) if L > 1 else w.planes[None]
        layer = FastARLayer(H, d, w.n_bits, P, w.tau, T, F * T, w.n_queries, w.chunk_frames, n_prompt=npr,
                            dtype=tdt, device=dev, n_tables=L)
        layer.set_planes(up(planes))
        for f in range(w.setup_frames):
            layer.merge(up(w.k_frames[:, f]), up(w.v_frames[:, f]), 1, with_index=False)
        pristine = layer.cache
        work = fb.TempCache(H, d, F * T, T, w.n_bits, tdt, dev)
        work.copy_from(pristine)
        layer.step(q, k_new, v_new, pk, pv, cache=work)   # first use: set-up outside the timing
        ms = []
        for _ in range(reps):
            work.copy_from(pristine)
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            layer.step(q, k_new, v_new, pk, pv, cache=work)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        c = work
        if L > 1:
            def attn():
                fb.fastar_bucket_attention_tables(
                    q, c.rep_k, c.v_mean, layer.q_ids_t, layer.q_perm, layer.rep_off_t, layer.rep_perm_t,
                    w.n_bits, k_bucket=layer.rep_ids_t, key_bias=c.log_count, out=layer.o_self,
                    lse=layer.lse_self, n_attended=layer.n_attended)
        else:
            def attn():
                fb.fastar_bucket_attention(q, c.rep_k, c.v_mean, q_bucket=layer.q_ids, q_perm=layer.q_perm,
                                           key_bias=c.log_count, k_offsets=layer.rep_off,
                                           k_perm=layer.rep_perm, n_bits=w.n_bits, out=layer.o_self,
                                           lse=layer.lse_self)
        at = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            attn()
            e1.record()
            torch.cuda.synchronize()
            at.append(e0.elapsed_time(e1))
        _, lse_d = fb.fastar_bucket_attention(q, c.rep_k, c.v_mean, key_bias=c.log_count, n_key_list=c.n_groups)
        if L > 1:
            _, st = fb.fastar_attention_recall_counts(layer.lse_self, lse_d, c.n_groups, layer.n_attended,
                                                      want_recall=False)
        else:
            _, st = fb.fastar_attention_recall(layer.lse_self, lse_d, c.n_groups, q_bucket=layer.q_ids,
                                               k_offsets=layer.rep_off, n_bits=w.n_bits, want_recall=False)
        st = st.cpu().numpy()
        row = {"tables": L, "probes_per_table": P, "chunk_ms": float(np.median(ms)),
               "attention_ms": float(np.median(at)), "annsa_recall": float(st[:, 0].mean()),
               "annsa_density": float(st[:, 1].mean())}
        if npr:
            row["annca_kept_frac"] = float(layer.n_kept.float().mean().item()) / npr
        out.append(row)
        del layer, work
        torch.cuda.empty_cache()
    return out


def denoise_loop(w, dev, n_steps=10, warmup=0.3, reps=3):
    """One chunk's denoising loop around the layer (paper.rainbus.top,
    limitations: the sparse attention is off in the first 30% of the steps):
    the loop's time with that warm-up, with every step sparse and with every
    step dense (the same merge per step, dense attention over every group and
    the whole prompt).  Hot inputs (each step reuses the chunk's tensors);
    median over reps loops."""
    from kv_compressed_attention_amd.denoise import DenoisingDriver, warmup_steps
    from kv_compressed_attention_amd.layer import FastARLayer

    H, F, T, d = w.k_frames.shape
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    npr = 0 if w.prompt_k is None else w.prompt_k.shape[1]

    def up(a):
        return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device=dev).to(tdt)
    q = up(w.q)
    k_new, v_new = (up(a) for a in w.frames(w.setup_frames, F))
    pk = up(w.prompt_k) if npr else None
    pv = up(w.prompt_v) if npr else None
    layer = FastARLayer(H, d, w.n_bits, w.n_probes, w.tau, T, F * T, w.n_queries, w.chunk_frames,
                        n_prompt=npr, dtype=tdt, device=dev)
    layer.set_planes(up(w.planes))
    for f in range(w.setup_frames):
        layer.merge(up(w.k_frames[:, f]), up(w.v_frames[:, f]), 1, with_index=False)
    import kv_compressed_attention_amd.fastar as fb
    start = fb.TempCache(H, d, F * T, T, w.n_bits, tdt, dev)
    start.copy_from(layer.cache)
    res = {"steps": n_steps, "warmup": warmup, "dense_steps": warmup_steps(n_steps, warmup)}
    for name, frac in (("warmup", warmup), ("all_sparse", 0.0), ("all_dense", 1.0)):
        drv = DenoisingDriver(layer, n_steps, frac)
        times = []
        for r in range(reps + 1):
            layer.cache.copy_from(start)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            drv.run(lambda s: (q, k_new, v_new, pk, pv))
            e1.record()
            torch.cuda.synchronize()
            if r:
                times.append(e0.elapsed_time(e1))
        res[name + "_ms"] = float(np.median(times))
    res["speedup_vs_all_dense"] = res["all_dense_ms"] / res["warmup_ms"]
    res["speedup_all_sparse_vs_all_dense"] = res["all_dense_ms"] / res["all_sparse_ms"]
    return res


def annca(w, dev, steps):
    """The AnnCA workload: hash the queries and the prompt, prune, and
    cross-attention over the kept prompt keys; per-call times (cold: one
    copy of the inputs per step) and the prune ratio."""
    import kv_compressed_attention_amd.fastar as fb

    H, nq, d = w.q.shape
    npr = w.prompt_k.shape[1]
    tdt = torch.bfloat16

    def up(a):
        return torch.tensor(np.ascontiguousarray(a), dtype=torch.float32, device=dev).to(tdt)
    planes = up(w.planes)
    ins = [(up(w.q), up(w.prompt_k), up(w.prompt_v))]
    ins += [tuple(t.clone() for t in ins[0]) for _ in range(steps - 1)]
    i32 = dict(dtype=torch.int32, device=dev)
    q_ids, p_ids = torch.empty(H, nq, 1, **i32), torch.empty(H, npr, 1, **i32)
    keep = torch.empty(H, npr, dtype=torch.uint8, device=dev)
    kept, n_kept = torch.empty(H, npr, **i32), torch.empty(H, **i32)
    o, lse = torch.empty(H, nq, d, dtype=tdt, device=dev), torch.empty(H, nq, device=dev)

    def hash_(i):
        return lambda: fb.fastar_hash_multi([ins[i][0], ins[i][1]], planes, w.n_bits, [1, 1],
                                            buckets=[q_ids, p_ids])

    def prune(i):
        return lambda: fb.fastar_prune_prompt(q_ids, p_ids.view(H, -1), w.n_bits, keep=keep,
                                              kept_idx=kept, n_kept=n_kept)

    def cross(i):
        return lambda: fb.fastar_bucket_attention(ins[i][0], ins[i][1], ins[i][2], key_list=kept,
                                                  n_key_list=n_kept, out=o, lse=lse)
    t_hash = graph_time([hash_(i) for i in range(steps)])
    t_prune = graph_time([prune(i) for i in range(steps)])
    t_cross = graph_time([cross(i) for i in range(steps)])
    t_all = graph_time([f for i in range(steps) for f in (hash_(i), prune(i), cross(i))]) * 3
    _, lse_d = fb.fastar_bucket_attention(ins[0][0], ins[0][1], ins[0][2])
    _, rstats = fb.fastar_attention_recall(lse, lse_d, torch.full((H,), npr, dtype=torch.int32, device=dev),
                                           n_retained=n_kept, want_recall=False)
    rs = rstats.cpu().numpy()
    nk = n_kept.cpu().numpy()
    c_bytes, c_flops = cross_work(nk, H, nq, npr, d)
    return {"workload": w.name, "prompt_tokens": npr, "kept_per_head_mean": float(nk.mean()),
            "kept_per_head_min": int(nk.min()), "kept_per_head_max": int(nk.max()),
            "prune_ratio": 1.0 - float(nk.mean()) / npr,
            "annca_recall": float(rs[:, 0].mean()), "annca_density": float(rs[:, 1].mean()),
            "ms": {"hash_queries_prompt": t_hash, "prune": t_prune, "attention_cross": t_cross,
                   "all": t_all},
            "query_tokens_per_s": nq / (t_all * 1e-3),
            "cross_attention_gbs": c_bytes / (t_cross * 1e-3) / 1e9,
            "cross_attention_tflops": c_flops / (t_cross * 1e-3) / 1e12}


def summarize(w, res, steps):
    nq = w.n_queries
    cold_ms = res["cold_s"] * 1e3 / steps
    d = {"ms_per_step": cold_ms, "query_tokens_per_s": nq / (cold_ms * 1e-3)}
    if "hot_s" in res:
        hot_ms = res["hot_s"] * 1e3 / steps
        d["hot"] = {"ms_per_step": hot_ms, "query_tokens_per_s": nq / (hot_ms * 1e-3)}
    d["kernels_ms"] = {k: v["launch_ms"] for k, v in res["kernels"].items()}
    d["recall"] = res["recall"]
    d["cache_density"] = res["cache_density"]
    a = res["kernels"]["attention_self"]
    d["attention_frac_hbm"] = a["frac_hbm"]
    return d


def progress(msg: str) -> None:
    """One line per finished stage on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench {time.monotonic() - _T0:7.1f} s] {msg}", file=sys.stderr, flush=True)


_T0 = time.monotonic()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: libfastar has no multi-GPU path (heads are "
              "independent and would shard across GPUs with no collective)", file=sys.stderr)
        sys.exit(2)
    from synth import make_workload

    w = make_workload(args.workload)
    # the oracle first: its worker processes are forked before this process
    # touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_sample_heads)
        progress("cpu baseline")

    import kv_compressed_attention_amd as fa
    dev = torch.device("cuda:0")
    fa.library()
    # a plain 64 MiB device copy before the timed region: the calibration
    # kernel for the FETCH_SIZE / WRITE_SIZE counter passes
    cal_src = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    del cal_src, cal_dst

    res = measure_workload(w, dev, args.steps, args.warmup, args.graph_steps, hot=not args.no_hot)
    progress(f"{w.name}: timed steps and stages")
    H, F, T, d = w.k_frames.shape
    nq = w.n_queries
    ms = res["cold_s"] * 1e3 / args.steps
    kern = res["kernels"]
    # the roofline kernel: the single launch of largest duration (the merge
    # stage is four launches and is reported beside it in "kernels")
    dom = max((k for k in kern if k != "merge"), key=lambda k: kern[k]["launch_ms"])
    a = kern["attention_self"]
    t_att = a["launch_ms"] * 1e-3
    a_bytes = a["bytes_per_launch"]
    flops = a["tflops"] * 1e12 * t_att
    ai = flops / a_bytes
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
                   "n_bits": w.n_bits, "n_probes": w.n_probes, "tau": w.tau,
                   "prompt_tokens": 0 if w.prompt_k is None else int(w.prompt_k.shape[1]),
                   "inputs": "cold: every step on its own copy of the inputs and cache"},
        "roofline": {"bound": "hbm", "achieved": kern[dom]["achieved_gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": kern[dom]["frac_hbm"],
                     "traffic": recorded_traffic(w.name + ":" + dom, KERNEL_FILES[dom]),
                     "kernel": f"{dom}: {kern[dom]['kernel']}",
                     "bytes_per_launch": kern[dom]["bytes_per_launch"],
                     "launch_ms": kern[dom]["launch_ms"]},
        "kernels": kern,
        "attention": {"tflops": a["tflops"], "frac_bf16_mfma_peak": a["tflops"] / PEAK_BF16_TFLOPS,
                      "arith_intensity_flop_per_byte": ai,
                      "roofline_tflops": min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3),
                      "frac_of_roofline": a["tflops"] / min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3),
                      "query_tokens_per_s": nq / t_att, **res["extra"]},
        "launch": f"hip_graph{max(1, args.graph_steps)}_chunk",
        "recall": res["recall"],
        "cache_density": res["cache_density"],
        "diag": res["diag"],
        "pages": PAGES,
    }
    if "hot_s" in res:
        hms = res["hot_s"] * 1e3 / args.steps
        out["hot"] = {"ms_per_step": hms, "value": nq / (hms * 1e-3),
                      "inputs": "one copy of the inputs shared by every step (each still merges "
                                "into its own cache)"}
    st = res.pop("setup")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flushed = []
    for i in range(min(5, args.steps)):
        st.caches[i].copy_from(st.pristine)
        flushed.append(flushed_chunk_ms(st, flush, i))
    out["flushed_chunk_ms"] = float(np.median(flushed))
    del st, res
    torch.cuda.empty_cache()

    if not args.no_extra:
        # TempCache's quantized match (8-bit codes, every previous-frame token a
        # candidate) on the same workload
        rq = measure_workload(w, dev, args.steps, args.warmup, args.graph_steps, hot=False, match="quant")
        rq.pop("setup")
        out["tempcache_quant8"] = summarize(w, rq, args.steps)
        progress("quantized match")
        del rq
        torch.cuda.empty_cache()
        extra = {}
        if args.workload != 1:
            w1 = make_workload(1)
            r1 = measure_workload(w1, dev, args.steps, args.warmup, args.graph_steps,
                                  hot=not args.no_hot)
            r1.pop("setup")
            extra[w1.name] = summarize(w1, r1, args.steps)
            progress(w1.name)
            del r1
            torch.cuda.empty_cache()
        w1 = make_workload(1)
        extra["tau_sweep"] = {"workload": w1.name, "lsh": tau_sweep(w1, dev, [0.999, 0.99, 0.95, 0.9, 0.7, 0.5]),
                              "quant8": tau_sweep(w1, dev, [0.999, 0.99, 0.9, 0.5], match="quant")}
        # the group representative (paperlayer.ai appendix C: last, mean and
        # medoid keys) at two thresholds
        extra["representatives"] = {"workload": w1.name, **{
            rep: tau_sweep(w1, dev, [0.9, 0.7], representative=rep) for rep in ("last", "mean", "medoid")}}
        progress("tau sweep and representatives")
        extra["annca"] = annca(make_workload(2), dev, args.steps)
        progress("annca")
        # several LSH tables and more probes (AnnSA recall / density / time)
        extra["lsh_tables"] = {
            "workload": w1.name,
            "configs": lsh_tables_sweep(w1, dev, [(1, 1), (1, 2), (1, 4), (2, 1), (2, 2), (4, 1), (4, 2)])}
        if args.workload != 1:
            extra["lsh_tables_" + w.name] = lsh_tables_sweep(w, dev, [(1, 2), (2, 2), (1, 4)])
        progress("lsh tables")
        # the denoising loop with the 30% dense warm-up
        extra["denoise"] = {"workload": w.name, **denoise_loop(w, dev)}
        progress("denoising loop")
        w3 = make_workload(3)
        roll = rollout(w3, dev, flush)
        progress("rollout")
        extra["rollout"] = {"workload": w3.name, "chunks": roll,
                            "first_last_ms": [roll[0]["ms"], roll[-1]["ms"]],
                            "last_chunk_density": roll[-1]["density"],
                            "last_chunk_annsa": {"recall": roll[-1]["annsa_recall"],
                                                 "density": roll[-1]["annsa_density"]}}
        del w3
        torch.cuda.empty_cache()
        out["extra_workloads"] = extra
    if not args.no_dense:
        out["dense_one_bucket"] = dense_one_bucket(dev)
        progress("one-bucket attention")
    if cpu is not None:
        out["cpu_baseline"] = {
            "value": nq / cpu["all_cores_s_per_chunk"], "unit": "query tokens/s",
            "cores": cpu["processes"], "kind": "oracle",
            "sample": (f"the whole chunk (hash, merge {w.chunk_frames} frames, index, bucket "
                       f"self-attention, prune, cross-attention) of {cpu['processes']} heads, "
                       f"one process per head and core, scaled to all {H} heads; set-up "
                       f"merges untimed"),
            "host_cpus": cpu["host_cpus"],
            "one_thread": {"value": nq / cpu["one_thread_s_per_chunk"], "cores": 1,
                           "sample": f"{cpu['one_thread_heads']} head(s) in one thread, "
                                     f"scaled to all {H} heads"},
        }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

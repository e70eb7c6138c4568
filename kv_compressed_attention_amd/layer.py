"""One attention layer's per-chunk sequence over libfastar, with preallocated
buffers so that repeated steps do no allocation.

Order (one hashing serves all three modules; the self-attention keys are the
compressed cache including the chunk's own frames):
  1. hash the chunk's queries (1 or 2 probes), new keys and prompt keys, in
     one launch;
  2. build the queries' bucket index;
  3. TempCache-merge the new frames, frame by frame, and index the
     representatives by bucket;
  4. prune the prompt keys against the queries' buckets (AnnCA);
  5. AnnSA bucket attention over the cache with the + ln m bias;
  6. cross-attention over the kept prompt tokens.
Every step is a libfastar call; this class only owns the torch buffers and
the ordering.  By default one fastar_chunk call runs the whole sequence on
the caller's stream (bf16 queries hashed by extra workgroups of the merge's
match launch, their index by extra workgroups of the launch that indexes the
representatives).  The other orders issue the calls one by one: on one
stream, or with the query side (2, then 4 and 6), which does not touch the
cache, on a second stream of default priority; all streams join before step
returns.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import fastar as fb


class FastARLayer:
    def __init__(self, heads: int, dim: int, n_bits: int, n_probes: int, tau: float,
                 tokens_per_frame: int, capacity: int, n_queries: int, chunk_frames: int,
                 n_prompt: int = 0, dtype=torch.bfloat16, device="cuda", match: str = "lsh",
                 code_bits: int = 8, query_driven: bool = False, representative: str = "last",
                 n_tables: int = 1):
        self.heads, self.dim, self.n_bits, self.n_probes = heads, dim, n_bits, n_probes
        self.tau, self.T, self.capacity = tau, tokens_per_frame, capacity
        self.nq, self.chunk_frames, self.n_prompt = n_queries, chunk_frames, n_prompt
        self.dtype, self.device = dtype, torch.device(device)
        # the TempCache variant (None: the library's defaults)
        self.opts = (None if match == "lsh" and representative == "last"
                     else fb.merge_opts(match, code_bits, representative))
        self.representative = representative
        # query-driven matching of a chunk's frames (by the chunk's queries,
        # which are then the new frames' tokens); set-up merges stay key-driven
        self.match, self.code_bits, self.query_driven = match, code_bits, query_driven
        H, dev = heads, self.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.cache = fb.TempCache(H, dim, capacity, tokens_per_frame, n_bits, dtype, dev,
                                  key_sums=representative != "last")
        # several LSH tables: planes [n_tables, n_bits, dim]; table 0's also
        # drive TempCache's match and the fused chunk
        self.n_tables = n_tables
        self.planes_t = torch.zeros(n_tables, max(n_bits, 1), dim, dtype=dtype, device=dev)
        self.planes = self.planes_t[0]
        nk = chunk_frames * tokens_per_frame
        lib = fb.library()
        size_opts = self.opts
        if query_driven:
            # the workspace of query-driven matching (only the presence of the
            # query tensor matters for its size)
            self._qd_desc = fb.FastarTensor(0, fb._DTYPES[dtype], H, nk, dim, 0, nk * dim, dim)
            size_opts = fb.merge_opts(match, code_bits, representative)
            size_opts.match_queries = ctypes.addressof(self._qd_desc)
        ws_bytes = max(lib.fastar_hash_workspace(H, n_queries, n_bits, n_probes),
                       lib.fastar_hash_workspace(H, nk, n_bits, 1),
                       lib.fastar_hash_workspace(H, n_prompt, n_bits, 1),
                       # fastar_chunk: the merge's, then (at most) the queries' index scratch
                       self.cache.workspace_bytes(chunk_frames, size_opts) +
                       lib.fastar_hash_workspace(H, n_queries, n_bits, n_probes),
                       self.cache.workspace_bytes(1, self.opts),
                       # several tables: the representatives' index per table
                       lib.fastar_hash_workspace(H, capacity, n_bits, 1))
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        # the query-side stream has a workspace of its own
        ws_q = max(lib.fastar_hash_workspace(H, n_queries, n_bits, n_probes),
                   lib.fastar_hash_workspace(H, n_prompt, n_bits, 1))
        self.ws_q = torch.empty(ws_q, dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream(device=dev)
        self.q_ids = torch.empty(H, n_queries, n_probes, **i32)
        self.q_off = torch.empty(H, (1 << n_bits) + 1, **i32)
        self.q_perm = torch.empty(H, n_queries, **i32)
        self.k_ids = torch.empty(H, nk, 1, **i32)
        self.group_of_new = torch.empty(H, nk, **i32)
        self.rep_off = torch.empty(H, (1 << n_bits) + 1, **i32)
        self.rep_perm = torch.empty(H, capacity, **i32)
        self.o_self = torch.empty(H, n_queries, dim, dtype=dtype, device=dev)
        self.lse_self = torch.empty(H, n_queries, dtype=torch.float32, device=dev)
        if n_prompt:
            self.p_ids = torch.empty(H, n_prompt, 1, **i32)
            self.keep = torch.empty(H, n_prompt, dtype=torch.uint8, device=dev)
            self.kept_idx = torch.empty(H, n_prompt, **i32)
            self.n_kept = torch.empty(H, **i32)
            self.o_cross = torch.empty(H, n_queries, dim, dtype=dtype, device=dev)
            self.lse_cross = torch.empty(H, n_queries, dtype=torch.float32, device=dev)
        if n_tables > 1:
            L = n_tables
            self.q_ids_t = torch.empty(L, H, n_queries, n_probes, **i32)
            self.rep_ids_t = torch.empty(L, H, capacity, **i32)
            self.rep_off_t = torch.empty(L, H, (1 << n_bits) + 1, **i32)
            self.rep_perm_t = torch.empty(L, H, capacity, **i32)
            self.n_attended = torch.empty(H, n_queries, **i32)
            if n_prompt:
                self.p_ids_t = torch.empty(L, H, n_prompt, 1, **i32)
        self.diag = fb.new_diag(dev)
        self._calls = {}

    def set_planes(self, planes: torch.Tensor):
        """planes [n_bits, dim] (one table) or [n_tables, n_bits, dim]."""
        if self.n_bits:
            self.planes_t.copy_(planes.view(self.n_tables, self.n_bits, self.dim))

    # -- building blocks ----------------------------------------------------
    def hash_keys(self, k: torch.Tensor, out: Optional[torch.Tensor] = None):
        """One-probe bucket ids [H, n, 1] of keys k [H, n, d]."""
        H, n, _ = k.shape
        if out is None:
            out = torch.empty(H, n, 1, dtype=torch.int32, device=self.device)
        fb.fastar_hash(k, self.planes, self.n_bits, 1, with_index=False, bucket=out, ws=self.ws,
                       diag=self.diag)
        return out

    def merge(self, k: torch.Tensor, v: torch.Tensor, n_frames: int, with_index: bool = True,
              group_of_new: Optional[torch.Tensor] = None):
        """Hash and merge n_frames new frames k, v [H, n_frames*T, d] (set-up path)."""
        ids = self.hash_keys(k)
        return fb.fastar_tempcache_merge(
            self.cache, k, v, ids.view(self.heads, -1), n_frames, self.tau,
            group_of_new=group_of_new, with_index=with_index, rep_offsets=self.rep_off,
            rep_perm=self.rep_perm, ws=self.ws, diag=self.diag, opts=self.opts)

    # -- one chunk ----------------------------------------------------------
    def _ev(self, timing):
        e = torch.cuda.Event(enable_timing=timing is not None)
        e.record()
        return e

    def _timed(self, timing, name, fn):
        if timing is None:
            return fn()
        a = self._ev(timing)
        r = fn()
        timing.setdefault(name, []).append((a, self._ev(timing)))
        return r

    def _hash_all(self, q, k_new, prompt_k, timing):
        xs, probes, outs = [q, k_new], [self.n_probes, 1], [self.q_ids, self.k_ids]
        if prompt_k is not None:
            xs.append(prompt_k)
            probes.append(1)
            outs.append(self.p_ids)
        self._timed(timing, "hash", lambda: fb.fastar_hash_multi(
            xs, self.planes, self.n_bits, probes, buckets=outs, diag=self.diag))

    def _query_index(self, timing):
        self._timed(timing, "index_q", lambda: fb.fastar_bucket_index(
            self.q_ids, self.n_bits, offsets=self.q_off, perm=self.q_perm, ws=self.ws_q))

    def _query_hash(self, q, timing):
        self._timed(timing, "hash_q", lambda: fb.fastar_hash(
            q, self.planes, self.n_bits, self.n_probes, bucket=self.q_ids, offsets=self.q_off,
            perm=self.q_perm, ws=self.ws_q, diag=self.diag))

    def _cross(self, q, prompt_k, prompt_v, timing, hashed=False):
        def run():
            if not hashed:
                fb.fastar_hash(prompt_k, self.planes, self.n_bits, 1, with_index=False,
                               bucket=self.p_ids, ws=self.ws_q, diag=self.diag)
            fb.fastar_prune_prompt(self.q_ids, self.p_ids.view(self.heads, -1), self.n_bits,
                                   keep=self.keep, kept_idx=self.kept_idx, n_kept=self.n_kept)
            fb.fastar_bucket_attention(q, prompt_k, prompt_v, key_list=self.kept_idx,
                                       n_key_list=self.n_kept, out=self.o_cross,
                                       lse=self.lse_cross)
        self._timed(timing, "cross", run)

    def _merge(self, cache, k_new, v_new, timing, q=None):
        opts = self.opts
        if self.query_driven:
            opts = fb.merge_opts(self.match, self.code_bits, self.representative, match_queries=q)
        self._timed(timing, "merge", lambda: fb.fastar_tempcache_merge(
            cache, k_new, v_new, self.k_ids.view(self.heads, -1), self.chunk_frames, self.tau,
            group_of_new=self.group_of_new, rep_offsets=self.rep_off, rep_perm=self.rep_perm,
            ws=self.ws, diag=self.diag, opts=opts))

    def self_attention(self, q, timing=None, cache=None):
        c = self.cache if cache is None else cache
        self._timed(timing, "attention", lambda: fb.fastar_bucket_attention(
            q, c.rep_k, c.v_mean, q_bucket=self.q_ids, q_perm=self.q_perm, key_bias=c.log_count,
            k_offsets=self.rep_off, k_perm=self.rep_perm, n_bits=self.n_bits, out=self.o_self,
            lse=self.lse_self))

    def _chunk_call(self, q, k_new, v_new, prompt_k, prompt_v, cache):
        key = tuple(0 if t is None else t.data_ptr() for t in (q, k_new, v_new, prompt_k, prompt_v)) + (
            id(cache),)
        call = self._calls.get(key)
        if call is None:
            extra = {}
            if prompt_k is not None:
                extra = dict(prompt_k=prompt_k, prompt_v=prompt_v, p_bucket=self.p_ids, keep=self.keep,
                             kept_idx=self.kept_idx, n_kept=self.n_kept, out_cross=self.o_cross,
                             lse_cross=self.lse_cross)
            opts = self.opts
            if self.query_driven:
                opts = fb.merge_opts(self.match, self.code_bits, self.representative, match_queries=q)
            call = fb.ChunkCall(q, self.n_probes, k_new, v_new, self.chunk_frames, self.planes,
                                self.n_bits, self.tau, cache, self.q_ids, self.q_off, self.q_perm,
                                self.k_ids, self.rep_off, self.rep_perm, self.o_self,
                                lse=self.lse_self, group_of_new=self.group_of_new, opts=opts,
                                **extra)
            self._calls[key] = call
        return call

    def step(self, q, k_new, v_new, prompt_k=None, prompt_v=None, cache=None, concurrent="chunk",
             timing=None):
        """One chunk, merged into ``cache`` (default: the layer's own).

        ``concurrent``: "chunk" (default) one fastar_chunk call; False every
        call queued on the caller's stream in order; True the query side on
        the second stream, forked after everything already queued on the
        caller's stream and joined before the self-attention; "split" the
        query hashing on the second stream as well.
        ``timing`` (optional dict) receives (start, end) event pairs per
        stage, recorded on the stream each stage runs on."""
        cache = self.cache if cache is None else cache
        if self.n_tables > 1:
            self._step_tables(q, k_new, v_new, prompt_k, prompt_v, cache, timing)
            return
        if concurrent == "chunk":
            call = self._chunk_call(q, k_new, v_new, prompt_k, prompt_v, cache)
            self._timed(timing, "chunk", lambda: call(self.ws, diag=self.diag))
            return
        if concurrent == "split":
            # the query side as its own branch from the start: its hashing
            # and index on the second stream, queued first; the keys' hashing
            # and the merge on this one
            main = torch.cuda.current_stream(self.device)
            start = self._ev(None)
            with torch.cuda.stream(self.side):
                self.side.wait_event(start)
                self._timed(timing, "hash_q", lambda: fb.fastar_hash_multi(
                    [q] + ([prompt_k] if prompt_k is not None else []), self.planes, self.n_bits,
                    [self.n_probes] + ([1] if prompt_k is not None else []),
                    buckets=[self.q_ids] + ([self.p_ids] if prompt_k is not None else []),
                    diag=self.diag))
                self._query_index(timing)
                q_done = self._ev(None)
                if prompt_k is not None:
                    self._cross(q, prompt_k, prompt_v, timing, hashed=True)
                side_done = self._ev(None)
            self._timed(timing, "hash_k", lambda: fb.fastar_hash_multi(
                [k_new], self.planes, self.n_bits, [1], buckets=[self.k_ids], diag=self.diag))
            self._merge(cache, k_new, v_new, timing, q)
            main.wait_event(q_done)
            self.self_attention(q, timing, cache)
            main.wait_event(side_done)
            return
        self._hash_all(q, k_new, prompt_k, timing)
        if not concurrent:
            self._query_index(timing)
            self._merge(cache, k_new, v_new, timing, q)
            self.self_attention(q, timing, cache)
            if prompt_k is not None:
                self._cross(q, prompt_k, prompt_v, timing, hashed=True)
            return
        main = torch.cuda.current_stream(self.device)
        hashed = self._ev(None)
        with torch.cuda.stream(self.side):
            self.side.wait_event(hashed)
            self._query_index(timing)
            q_done = self._ev(None)
            if prompt_k is not None:
                self._cross(q, prompt_k, prompt_v, timing, hashed=True)
            side_done = self._ev(None)
        self._merge(cache, k_new, v_new, timing, q)
        main.wait_event(q_done)
        self.self_attention(q, timing, cache)
        main.wait_event(side_done)

    def _step_tables(self, q, k_new, v_new, prompt_k, prompt_v, cache, timing):
        """One chunk with several LSH tables, call by call on the caller's
        stream: the chunk's queries and prompt keys hashed with every table's
        planes, the new keys with table 0's (TempCache's match); the merge and
        table 0's index of the representatives; tables 1.. hash the
        representatives themselves and index them (the groups in use); AnnSA
        over the union of the tables' buckets; AnnCA keeps a prompt token any
        table keeps."""
        L, H = self.n_tables, self.heads

        def hashes():
            for u in range(L):
                xs, probes, outs = [q], [self.n_probes], [self.q_ids_t[u]]
                if u == 0:
                    xs.append(k_new)
                    probes.append(1)
                    outs.append(self.k_ids)
                if prompt_k is not None:
                    xs.append(prompt_k)
                    probes.append(1)
                    outs.append(self.p_ids_t[u])
                fb.fastar_hash_multi(xs, self.planes_t[u], self.n_bits, probes, buckets=outs,
                                     diag=self.diag)
            fb.fastar_bucket_index(self.q_ids_t[0], self.n_bits, offsets=self.q_off, perm=self.q_perm,
                                   ws=self.ws_q)
        self._timed(timing, "hash", hashes)
        self._merge(cache, k_new, v_new, timing, q)

        def rep_index():
            self.rep_ids_t[0].copy_(cache.rep_bucket)
            self.rep_off_t[0].copy_(self.rep_off)
            self.rep_perm_t[0].copy_(self.rep_perm)
            for u in range(1, L):
                fb.fastar_hash(cache.rep_k, self.planes_t[u], self.n_bits, 1, with_index=False,
                               bucket=self.rep_ids_t[u].view(H, -1, 1), diag=self.diag)
                fb.fastar_bucket_index(self.rep_ids_t[u].view(H, -1, 1), self.n_bits,
                                       n_valid=cache.n_groups, offsets=self.rep_off_t[u],
                                       perm=self.rep_perm_t[u], ws=self.ws)
        self._timed(timing, "rep_index", rep_index)
        self._timed(timing, "attention", lambda: fb.fastar_bucket_attention_tables(
            q, cache.rep_k, cache.v_mean, self.q_ids_t, self.q_perm, self.rep_off_t, self.rep_perm_t,
            self.n_bits, k_bucket=self.rep_ids_t, key_bias=cache.log_count, out=self.o_self,
            lse=self.lse_self, n_attended=self.n_attended))
        if prompt_k is not None:
            def cross():
                fb.fastar_prune_prompt_tables(self.q_ids_t, self.p_ids_t.view(L, H, -1), self.n_bits,
                                              keep=self.keep, kept_idx=self.kept_idx, n_kept=self.n_kept)
                fb.fastar_bucket_attention(q, prompt_k, prompt_v, key_list=self.kept_idx,
                                           n_key_list=self.n_kept, out=self.o_cross, lse=self.lse_cross)
            self._timed(timing, "cross", cross)

    def step_dense(self, q, k_new, v_new, prompt_k=None, prompt_v=None, cache=None, timing=None):
        """One chunk with the sparse attention switched off (the denoising
        warm-up): the same merge, then dense self-attention over every group of
        the compressed cache (with the + ln m bias) and dense cross-attention
        over the whole prompt."""
        cache = self.cache if cache is None else cache
        self._timed(timing, "hash_k", lambda: fb.fastar_hash(
            k_new, self.planes, self.n_bits, 1, with_index=False, bucket=self.k_ids, diag=self.diag))
        self._merge(cache, k_new, v_new, timing, q)
        self._timed(timing, "attention", lambda: fb.fastar_bucket_attention(
            q, cache.rep_k, cache.v_mean, key_bias=cache.log_count, n_key_list=cache.n_groups,
            out=self.o_self, lse=self.lse_self))
        if prompt_k is not None:
            self._timed(timing, "cross", lambda: fb.fastar_bucket_attention(
                q, prompt_k, prompt_v, out=self.o_cross, lse=self.lse_cross))

    def capture(self, q, k_new, v_new, prompt_k=None, prompt_v=None, cache=None,
                concurrent="chunk", caches=None):
        """Capture one chunk on these buffers into a HIP graph, replayed with
        ``.replay()`` on the current stream: one graph launch instead of one
        launch per kernel.  With ``caches``, one chunk per cache in order (as
        a model captures the chunks of its layers together), one launch for
        all of them.

        Call after at least one eager ``step`` (first use of torch's streams
        and events does one-time set-up, which capture does not allow).  Every
        replay reads and writes the same addresses."""
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in (caches if caches is not None else [cache]):
                self.step(q, k_new, v_new, prompt_k, prompt_v, cache=c, concurrent=concurrent)
        torch.cuda.synchronize(self.device)
        return g

"""Seeded, synthetic stand-ins for the video-latent tensors the method runs on.

The pages measure on real model features (Rolling-Forcing, LongVie2) which are
not available here.  These recipes reproduce the structure the pages describe
instead: keys that repeat across frames with small drift (the temporal
redundancy TempCache exploits), queries and keys that cluster semantically
(what AnnSA exploits), and long prompts of which only a few tokens lie near the
current frame's queries (what AnnCA exploits).

Every array is drawn in float64, cast to float32 and then rounded to the
storage dtype with round-to-nearest-even, so the values handed to the oracle
(as float64) and to the GPU (as bf16 or fp32) are the same real numbers.

Five workloads, indexed 0..4:

0  tiny fp32: 1 head, d=64, 4 frames x 256 tokens, 256 queries, 64 prompt keys,
   6 hash bits, threshold 0.9, one probe.
1  one layer, bf16: 12 heads, d=128, 6 frames x 1560 tokens, queries are the
   3 newest frames (4680), 12 bits, threshold 0.999, one probe.
2  cross-attention, bf16: 12 heads, d=128, 4680 queries around 16 centroids,
   512 prompt keys (48 near the centroids), 10 bits.
3  long rollout, bf16: the workload-1 process run for 60 frames; the last
   3-frame chunk is the measured one.
4  wide, bf16: 24 heads, d=128, 16 frames x 2048 tokens from 128 drifting
   clusters, 4 newest frames as queries (8192), 14 bits, two probes,
   512 prompt keys.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

CONFIG_NAMES = (
    "tiny_f32_h1_d64_q256_cache4x256",
    "layer_bf16_h12_d128_q4680_cache6x1560",
    "annca_bf16_h12_d128_q4680_prompt512",
    "rollout_bf16_h12_d128_q4680_cache60x1560",
    "wide_bf16_h24_d128_q8192_cache16x2048_p2",
)


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round to the storage dtype; return float32 holding the exact values.

    bf16 uses round-to-nearest-even on the float32 bit pattern.
    """
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    if dtype == "f32":
        return x32
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-exact")
    return (u >> 16).astype(np.uint16)


def gaussian(shape, seed, dtype: str = "f32", scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) draws rounded to dtype (float32 container)."""
    rng = np.random.default_rng(seed)
    return round_to_dtype(scale * rng.standard_normal(shape), dtype)


@dataclass
class Workload:
    index: int
    name: str
    dtype: str                 # "f32" or "bf16"
    heads: int
    dim: int
    n_bits: int
    n_probes: int
    tau: float
    planes: np.ndarray         # [n_bits, dim]
    q: np.ndarray              # [H, Nq, dim]
    k_frames: Optional[np.ndarray] = None   # [H, F, T, dim]
    v_frames: Optional[np.ndarray] = None   # [H, F, T, dim]
    setup_frames: int = 0      # frames merged before the measured chunk
    prompt_k: Optional[np.ndarray] = None   # [H, Np, dim]
    prompt_v: Optional[np.ndarray] = None   # [H, Np, dim]
    notes: dict = field(default_factory=dict)

    @property
    def n_frames(self) -> int:
        return 0 if self.k_frames is None else self.k_frames.shape[1]

    @property
    def tokens_per_frame(self) -> int:
        return 0 if self.k_frames is None else self.k_frames.shape[2]

    @property
    def chunk_frames(self) -> int:
        return self.n_frames - self.setup_frames

    @property
    def n_queries(self) -> int:
        return self.q.shape[1]

    def frames(self, f0: int, f1: int):
        """Keys and values of frames [f0, f1) as [H, (f1-f0)*T, dim]."""
        H, _, T, d = self.k_frames.shape
        k = self.k_frames[:, f0:f1].reshape(H, (f1 - f0) * T, d)
        v = self.v_frames[:, f0:f1].reshape(H, (f1 - f0) * T, d)
        return k, v


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _near_prompt_keys(rng, anchors, per_anchor, d):
    """Keys at cosine c ~ U[0.8, 1] from each anchor direction, norm sqrt(d)."""
    H, A, _ = anchors.shape
    u = _unit(anchors)[:, :, None, :].repeat(per_anchor, axis=2)       # [H,A,m,d]
    w = rng.standard_normal((H, A, per_anchor, d))
    w = w - np.sum(w * u, axis=-1, keepdims=True) * u                   # orthogonal part
    w = _unit(w)
    c = rng.uniform(0.8, 1.0, (H, A, per_anchor, 1))
    k = np.sqrt(d) * (c * u + np.sqrt(1.0 - c * c) * w)
    return k.reshape(H, A * per_anchor, d)


def _prompt(rng, anchors, n_near_per_anchor, n_random, d):
    H = anchors.shape[0]
    near = _near_prompt_keys(rng, anchors, n_near_per_anchor, d)
    rand = rng.standard_normal((H, n_random, d))
    k = np.concatenate([near, rand], axis=1)
    order = np.stack([rng.permutation(k.shape[1]) for _ in range(H)])
    k = np.take_along_axis(k, order[:, :, None], axis=1)
    v = rng.standard_normal(k.shape)
    return k, v


def _cluster_video(rng, H, F, T, d, n_centers, carry, sigma_fresh, sigma_drift,
                   center_drift, q_frames):
    """Cluster-structured keys with frame-to-frame carry-over.

    Returns keys [H,F,T,d], values [H,F,T,d] and queries for the last
    q_frames frames [H, q_frames*T, d].
    """
    centers = rng.standard_normal((H, n_centers, d))
    hidx = np.arange(H)[:, None]
    labels = rng.integers(0, n_centers, (H, T))
    k = np.empty((H, F, T, d), dtype=np.float32)
    k_prev = centers[hidx, labels] + sigma_fresh * rng.standard_normal((H, T, d))
    k[:, 0] = k_prev
    qs = []
    for f in range(F):
        if f > 0:
            if center_drift > 0:
                centers = centers + center_drift * rng.standard_normal(centers.shape)
            carried = rng.random((H, T)) < carry
            new_labels = rng.integers(0, n_centers, (H, T))
            labels = np.where(carried, labels, new_labels)
            fresh = centers[hidx, labels] + sigma_fresh * rng.standard_normal((H, T, d))
            drift = k_prev + sigma_drift * rng.standard_normal((H, T, d))
            k_prev = np.where(carried[:, :, None], drift, fresh)
            k[:, f] = k_prev
        if f >= F - q_frames:
            qs.append(centers[hidx, labels] + sigma_fresh * rng.standard_normal((H, T, d)))
    v = rng.standard_normal((H, F, T, d))
    q = np.concatenate(qs, axis=1)
    return k, v, q


def make_workload(index: int) -> Workload:
    """Build workload `index` (0..4) deterministically."""
    planes_rng = np.random.default_rng(index)
    rng = np.random.default_rng(100 + index)
    if index == 0:
        H, d, T, F, b = 1, 64, 256, 4, 6
        planes = planes_rng.standard_normal((b, d))
        k = np.empty((H, F, T, d))
        k[:, 0] = rng.standard_normal((H, T, d))
        for f in range(1, F):
            keep = rng.random((H, T)) < 0.75
            noisy = k[:, f - 1] + 0.05 * rng.standard_normal((H, T, d))
            fresh = rng.standard_normal((H, T, d))
            k[:, f] = np.where(keep[:, :, None], noisy, fresh)
        v = rng.standard_normal((H, F, T, d))
        q = rng.standard_normal((H, 256, d))
        pk = rng.standard_normal((H, 64, d))
        pv = rng.standard_normal((H, 64, d))
        dt = "f32"
        return Workload(index, CONFIG_NAMES[index], dt, H, d, b, 1, 0.9,
                        round_to_dtype(planes, dt), round_to_dtype(q, dt),
                        round_to_dtype(k, dt), round_to_dtype(v, dt), setup_frames=3,
                        prompt_k=round_to_dtype(pk, dt), prompt_v=round_to_dtype(pv, dt))
    if index in (1, 3):
        H, d, T, b = 12, 128, 1560, 12
        F = 6 if index == 1 else 60
        planes = planes_rng.standard_normal((b, d))
        k, v, q = _cluster_video(rng, H, F, T, d, n_centers=64, carry=0.8,
                                 sigma_fresh=0.1, sigma_drift=0.02, center_drift=0.0,
                                 q_frames=3)
        dt = "bf16"
        return Workload(index, CONFIG_NAMES[index], dt, H, d, b, 1, 0.999,
                        round_to_dtype(planes, dt), round_to_dtype(q, dt),
                        round_to_dtype(k, dt), round_to_dtype(v, dt), setup_frames=F - 3)
    if index == 2:
        H, d, b, nq = 12, 128, 10, 4680
        planes = planes_rng.standard_normal((b, d))
        cents = rng.standard_normal((H, 16, d))
        labels = rng.integers(0, 16, (H, nq))
        q = cents[np.arange(H)[:, None], labels] + 0.1 * rng.standard_normal((H, nq, d))
        pk, pv = _prompt(rng, cents, 3, 464, d)
        dt = "bf16"
        return Workload(index, CONFIG_NAMES[index], dt, H, d, b, 1, 0.999,
                        round_to_dtype(planes, dt), round_to_dtype(q, dt),
                        prompt_k=round_to_dtype(pk, dt), prompt_v=round_to_dtype(pv, dt))
    if index == 4:
        H, d, T, F, b = 24, 128, 2048, 16, 14
        planes = planes_rng.standard_normal((b, d))
        k, v, q = _cluster_video(rng, H, F, T, d, n_centers=128, carry=0.8,
                                 sigma_fresh=0.1, sigma_drift=0.02, center_drift=0.02,
                                 q_frames=4)
        # the near prompt keys sit around the directions of 16 randomly chosen
        # queries, i.e. near 16 of the clusters the current chunk occupies
        pick = np.stack([rng.choice(q.shape[1], 16, replace=False) for _ in range(H)])
        anchors = q[np.arange(H)[:, None], pick]
        pk, pv = _prompt(rng, anchors, 3, 464, d)
        dt = "bf16"
        return Workload(index, CONFIG_NAMES[index], dt, H, d, b, 2, 0.999,
                        round_to_dtype(planes, dt), round_to_dtype(q, dt),
                        round_to_dtype(k, dt), round_to_dtype(v, dt), setup_frames=F - 4,
                        prompt_k=round_to_dtype(pk, dt), prompt_v=round_to_dtype(pv, dt))
    raise ValueError(f"workload index must be 0..4, got {index}")

"""The denoising loop of one chunk around a FastARLayer, with the sparse
attention switched off during a warm-up.

The pages report that the sparse attention is disabled for the first 30% of
the denoising steps, so that early generation runs full attention
(paper.rainbus.top, limitations).  Readings:
* step s (0-based) of n_steps is a warm-up step iff s < warmup * n_steps, so
  ceil(warmup * n_steps) steps are dense;
* a warm-up step runs the same TempCache merge and dense attention (self over
  every group of the compressed cache with the + ln m bias, cross over the
  whole prompt); the other steps run the sparse chunk (AnnSA, AnnCA);
* every step attends from the cache as it stood before the chunk (the chunk's
  frames change from step to step); after the last step its merged state is
  kept: the chunk's frames enter the cache once, as generated.
All compute is libfastar's; this module only orders calls and restores the
cache between steps.
"""

from __future__ import annotations

from fractions import Fraction
from typing import Callable, List, Optional



def is_warmup_step(step: int, n_steps: int, warmup: float = 0.3) -> bool:
    """Whether denoising step ``step`` of ``n_steps`` runs dense attention."""
    if not 0.0 <= warmup <= 1.0:
        raise ValueError("warmup must be in [0, 1]")
    if not 0 <= step < n_steps:
        raise ValueError("step out of range")
    # exactly, on the rational values (no rounding of warmup * n_steps)
    return Fraction(step) < Fraction(warmup) * n_steps


def warmup_steps(n_steps: int, warmup: float = 0.3) -> int:
    """The number of dense steps: ceil(warmup * n_steps)."""
    return sum(is_warmup_step(s, n_steps, warmup) for s in range(n_steps))


class DenoisingDriver:
    """Runs one chunk's n_steps denoising steps on ``layer``.

    ``run(inputs, on_step)``: inputs(s) gives step s's (q, k_new, v_new,
    prompt_k, prompt_v) (prompt may be None); on_step(s, dense), if given, is
    called after each step is queued (the layer's o_self, lse_self, o_cross
    hold that step's results until the next step runs).  The layer's cache
    is the cache before the chunk and, when run returns, the cache after it:
    each step merges into it, and the next step first undoes that merge
    (TempCache.checkpoint / restore: only the last frame's groups and the
    counts are restored, not the whole cache).
    """

    def __init__(self, layer, n_steps: int, warmup: float = 0.3):
        if n_steps < 1:
            raise ValueError("n_steps must be >= 1")
        self.layer, self.n_steps, self.warmup = layer, n_steps, warmup
        self.dense = [is_warmup_step(s, n_steps, warmup) for s in range(n_steps)]

    def run(self, inputs: Callable[[int], tuple], on_step: Optional[Callable[[int, bool], None]] = None,
            timing: Optional[dict] = None) -> List[bool]:
        layer = self.layer
        cache = layer.cache
        ck = cache.checkpoint()
        for s in range(self.n_steps):
            q, k_new, v_new, prompt_k, prompt_v = inputs(s)
            if s:
                cache.restore(ck)
            if self.dense[s]:
                layer.step_dense(q, k_new, v_new, prompt_k, prompt_v, cache=cache, timing=timing)
            else:
                layer.step(q, k_new, v_new, prompt_k, prompt_v, cache=cache, timing=timing)
            if on_step is not None:
                on_step(s, self.dense[s])
        # the last step's merge is the chunk's: it stays
        return list(self.dense)


__all__ = ["DenoisingDriver", "is_warmup_step", "warmup_steps"]

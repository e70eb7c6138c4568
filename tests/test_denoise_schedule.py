"""The denoising warm-up schedule (host logic, no GPU): the first 30% of a
chunk's denoising steps run dense attention (paper.rainbus.top,
limitations); step s is a warm-up step iff s < 0.3 n."""

import pytest

from kv_compressed_attention_amd.denoise import is_warmup_step, warmup_steps


@pytest.mark.parametrize("n,dense", [(50, 15), (10, 3), (4, 2), (1, 1), (3, 1), (7, 3), (100, 30)])
def test_warmup_counts(n, dense):
    assert warmup_steps(n) == dense
    # the dense steps come first
    flags = [is_warmup_step(s, n) for s in range(n)]
    assert flags == [True] * dense + [False] * (n - dense)


def test_warmup_bounds():
    assert warmup_steps(20, 0.0) == 0 and warmup_steps(20, 1.0) == 20
    with pytest.raises(ValueError):
        is_warmup_step(0, 10, 1.5)
    with pytest.raises(ValueError):
        is_warmup_step(10, 10)

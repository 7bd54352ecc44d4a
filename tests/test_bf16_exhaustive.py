"""The oracle's float32 -> bfloat16 rounding against torch's conversion on every float32 pattern.

bfloat16 keeps the top 16 bits of a float32; the oracle rounds to nearest, ties to even, with
NaN kept quiet. torch's CPU conversion is the library routine this is pinned to: all 2^32 bit
patterns are compared (finite values bit for bit, NaN as NaN, infinities unchanged), in 256
chunks of 2^24 spread over worker processes (about a minute on 8 cores).
"""

import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest

CHUNK = 1 << 24


def _check_chunk(c: int) -> int:
    """Number of disagreeing patterns in chunk c (patterns c * 2^24 .. (c + 1) * 2^24 - 1)."""
    import torch

    from oracle import decoder as ref

    torch.set_num_threads(1)
    pats = (np.arange(CHUNK, dtype=np.uint64) + np.uint64(c * CHUNK)).astype(np.uint32)
    x = pats.view(np.float32)
    ours = ref.round_f32_to_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    finite = np.isfinite(x)
    bad = int(np.count_nonzero(ours[finite].view(np.uint32) != want[finite].view(np.uint32)))
    nan = np.isnan(x)
    bad += int(np.count_nonzero(~np.isnan(ours[nan])))
    inf = np.isinf(x)
    bad += int(np.count_nonzero(ours[inf] != x[inf]))
    return bad


@pytest.mark.slow
def test_bf16_rounding_matches_torch_on_every_pattern():
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ProcessPoolExecutor(workers) as ex:
        bad = list(ex.map(_check_chunk, range((1 << 32) // CHUNK)))
    assert sum(bad) == 0, [(c, n) for c, n in enumerate(bad) if n]

"""Decoding of step-trace buffers (host logic only)."""

import numpy as np

from bandwidth_bound_transformer_amd import trace


def test_intervals_of_a_synthetic_trace():
    L, nwg = 2, 3
    st = trace.stride(L)
    buf = np.zeros(nwg * st, np.uint64)
    for w in range(nwg):
        t = 1000 + 10 * w
        row = buf[w * st : (w + 1) * st]
        row[0] = t
        row[1] = t + 100  # setup: 1 us
        tick = t + 100
        for l in range(L):
            for e in range(len(trace.LAYER_EVENTS)):
                if w == 1 and e in (4, 5):
                    continue  # this workgroup had no attention unit
                tick += 50 * (e + 1)
                row[2 + 16 * l + e] = tick
        for e in range(4):
            tick += 7
            row[2 + 16 * L + e] = tick
    parts, total = trace.intervals(buf, L, nwg)
    assert np.allclose(parts["QKV rows streamed"], 1.5)  # 150 ticks
    assert np.isnan(parts["RoPE, KV append, chunk streamed"][1]).all()
    # the boundary after a skipped one measures from the last reached one
    assert np.allclose(parts["chunk partials published"][1], 50 * 7 * 0.01)
    assert np.allclose(parts["argmax done"], 0.07)
    assert total.shape == (nwg,) and np.all(total > 0)
    text = trace.summary(buf, L, nwg)
    assert "x gathered" in text and "sum of medians" in text

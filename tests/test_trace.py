"""Decoding of step-trace buffers (host logic only)."""

import numpy as np

from bandwidth_bound_transformer_amd import trace

EV = len(trace.LAYER_EVENTS)


def _synthetic(L, nwg, skip_wg=1, skip=(4, 5)):
    """Workgroup w starts at 1000 + 10 w; boundary e of every layer comes 50 (e + 1) ticks after
    the previous reached one; workgroup `skip_wg` never reaches the boundaries in `skip`."""
    st = trace.stride(L)
    buf = np.zeros(nwg * st, np.uint64)
    for w in range(nwg):
        t = 1000 + 10 * w
        row = buf[w * st : (w + 1) * st]
        row[0] = t
        row[1] = t + 100  # setup: 1 us
        tick = t + 100
        for l in range(L):
            for e in range(EV - 1):  # the last slot of a layer is not stamped
                if w == skip_wg and e in skip:
                    continue  # this workgroup had no attention unit
                tick += 50 * (e + 1)
                row[2 + EV * l + e] = tick
        for e in range(4):
            tick += 7
            row[2 + EV * L + e] = tick
    return buf


def test_layout_matches_kernel():
    assert EV == 24 and trace.stride(3) == 2 + 24 * 3 + 4


def test_intervals_of_a_synthetic_trace():
    L, nwg = 2, 3
    buf = _synthetic(L, nwg)
    parts, total = trace.intervals(buf, L, nwg)
    assert np.allclose(parts[trace.LAYER_EVENTS[2]], 1.5)  # 150 ticks
    assert np.isnan(parts[trace.LAYER_EVENTS[5]][1]).all()
    # the boundary after skipped ones measures from the last reached one (boundary 3)
    assert np.allclose(parts[trace.LAYER_EVENTS[6]][1], 50 * 7 * 0.01)
    assert np.allclose(parts["argmax done"], 0.07)
    assert total.shape == (nwg,) and np.all(total > 0)
    text = trace.summary(buf, L, nwg)
    assert "x gathered" in text and "sum of medians" in text


def test_critical_path_follows_the_last_workgroup():
    L, nwg = 2, 3
    buf = _synthetic(L, nwg, skip_wg=-1)
    text = trace.critical_path(buf, L, nwg)
    # every boundary is 50 (e + 1) ticks after the previous one in every workgroup
    for e in (0, 3, 10):
        line = next(x for x in text.splitlines() if x.strip().startswith(trace.LAYER_EVENTS[e]))
        assert f"+{0.5 * (e + 1):7.2f} us" in line


def test_chrome_trace_export():
    """Every reached boundary becomes one complete event on its workgroup's track; events of a
    track tile its timeline without gaps or overlaps, and the whole is valid JSON."""
    import json

    L, nwg = 2, 3
    buf = _synthetic(L, nwg)
    doc = trace.to_chrome_trace(buf, L, nwg)
    json.loads(json.dumps(doc))
    ev = [e for e in doc["traceEvents"] if e["ph"] == "X"]
    st = trace.stride(L)
    reached = (buf.reshape(nwg, st)[:, 1:] > 0).sum()
    assert len(ev) == reached
    for w in range(nwg):
        mine = sorted((e for e in ev if e["tid"] == w), key=lambda e: e["ts"])
        assert mine[0]["name"] == "setup" and np.isclose(mine[0]["dur"], 1.0)
        assert np.isclose(mine[0]["ts"], 0.1 * w)  # workgroup w starts 10 w ticks after the first
        for a, b in zip(mine, mine[1:]):
            assert np.isclose(a["ts"] + a["dur"], b["ts"])
    # the skipped boundaries of workgroup 1 leave no events
    names1 = {e["name"] for e in ev if e["tid"] == 1}
    assert f"L0 {trace.LAYER_EVENTS[4]}" not in names1 and f"L0 {trace.LAYER_EVENTS[6]}" in names1

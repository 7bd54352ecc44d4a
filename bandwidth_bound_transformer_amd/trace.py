"""Decode the per-workgroup phase timestamps written by a traced kd_step.

Layout (see kd_trace in include/kd.h): per workgroup, slot 0 = step start, slot 1 = setup
done, then 24 phase boundaries per layer (23 used), then 4 final ones. The timestamps come from the
GPU's 100 MHz constant clock (10 ns ticks). A boundary a workgroup did not reach (e.g. no
attention unit assigned) holds 0 and is skipped.
"""

from __future__ import annotations

import warnings

import numpy as np

TICK_US = 0.01
LAYER_EVENTS = (
    "x gathered",
    "RMSNorm",
    "QKV rows streamed",
    "QKV reduced, published",
    "q/k/v gathered (first unit)",
    "RoPE",
    "K/V rounded, appended",
    "chunk streamed",
    "waves joined",
    "chunk partials published",
    "attention units done",
    "merge partials gathered",
    "head merges done",
    "o gathered",
    "O rows streamed",
    "O reduced, residual, published",
    "x' gathered",
    "RMSNorm (FFN)",
    "gate/up rows streamed",
    "SiLU*up",
    "down slice streamed, published",
    "down partials gathered",
    "x rows summed, published",
    "(unused)",
)
FINAL_EVENTS = ("x gathered, final norm", "LM head streamed", "argmax partial published", "argmax done")


def stride(n_layers: int) -> int:
    return 2 + len(LAYER_EVENTS) * n_layers + len(FINAL_EVENTS)


def intervals(buf: np.ndarray, n_layers: int, n_wg: int):
    """Per workgroup, the time (us) spent before each reached boundary; dict name -> [n_wg, n_layers] or [n_wg]."""
    st = stride(n_layers)
    t = np.asarray(buf, np.int64)[: n_wg * st].reshape(n_wg, st)
    layer = t[:, 2 : 2 + len(LAYER_EVENTS) * n_layers].reshape(n_wg, n_layers, len(LAYER_EVENTS))
    final = t[:, 2 + len(LAYER_EVENTS) * n_layers :]
    # walk the boundaries in order, keeping the last reached stamp
    seq = np.concatenate([t[:, 1:2], layer.reshape(n_wg, -1), final], axis=1)
    prev = seq[:, 0].copy()
    deltas = np.zeros(seq.shape, np.float64)
    for j in range(1, seq.shape[1]):
        reached = seq[:, j] > 0
        deltas[:, j] = np.where(reached, (seq[:, j] - prev) * TICK_US, np.nan)
        prev = np.where(reached, seq[:, j], prev)
    lay = deltas[:, 1 : 1 + n_layers * len(LAYER_EVENTS)].reshape(n_wg, n_layers, len(LAYER_EVENTS))
    fin = deltas[:, 1 + n_layers * len(LAYER_EVENTS) :]
    out = {name: lay[:, :, i] for i, name in enumerate(LAYER_EVENTS)}
    out.update({name: fin[:, i] for i, name in enumerate(FINAL_EVENTS)})
    total = (np.max(np.where(seq > 0, seq, 0), axis=1) - t[:, 0]) * TICK_US
    return out, total


def summary(buf: np.ndarray, n_layers: int, n_wg: int) -> str:
    """Median (over workgroups) time per step spent before each boundary, summed over layers."""
    parts, total = intervals(buf, n_layers, n_wg)
    lines = [f"step span per workgroup: median {np.median(total):.1f} us, max {np.max(total):.1f} us"]
    acc = 0.0
    for name, v in parts.items():
        per_step = np.nansum(v, axis=1) if v.ndim == 2 else np.nan_to_num(v)
        med = float(np.median(per_step))
        acc += med
        per_layer = float(np.nanmedian(v)) if v.ndim == 2 and np.isfinite(v).any() else float("nan")
        lines.append(f"  {name:38s} {med:9.1f} us/step" + (f"   ({per_layer:6.2f} us/layer median)" if v.ndim == 2 else ""))
    lines.append(f"  {'sum of medians':38s} {acc:9.1f} us/step")
    return "\n".join(lines)


def critical_path(buf: np.ndarray, n_layers: int, n_wg: int) -> str:
    """When the last workgroup reached each boundary, as the median over layers of the time since
    the last workgroup reached the previous boundary (the step's critical path, event by event)."""
    st = stride(n_layers)
    t = np.asarray(buf, np.int64)[: n_wg * st].reshape(n_wg, st).astype(np.float64)
    t[t == 0] = np.nan
    ev = len(LAYER_EVENTS)
    lay = t[:, 2 : 2 + ev * n_layers].reshape(n_wg, n_layers, ev)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)  # boundaries no workgroup reached
        last = np.nanmax(lay, axis=0)  # [layer, event]
        first = np.nanmin(lay, axis=0)
    lines = ["critical path per layer (median over layers; last WG to reach each boundary):"]
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        prev_end = np.nanmax(last, axis=1)  # latest boundary any workgroup reached in each layer
    prev = np.concatenate([[np.nanmax(t[:, 1])], prev_end[:-1]])
    acc = 0.0
    for e in range(ev):
        if np.all(np.isnan(last[:, e])):
            continue
        d = (last[:, e] - prev) * TICK_US
        spread = (last[:, e] - first[:, e]) * TICK_US
        med = float(np.nanmedian(d))
        acc += med
        lines.append(f"  {LAYER_EVENTS[e]:34s} +{med:7.2f} us   (first..last WG spread {float(np.nanmedian(spread)):6.2f} us)")
        prev = np.where(np.isnan(last[:, e]), prev, last[:, e])
    lines.append(f"  {'layer total':34s} {acc:8.2f} us")
    return "\n".join(lines)


def to_chrome_trace(buf: np.ndarray, n_layers: int, n_wg: int) -> dict:
    """The step as Chrome trace-event JSON (loadable in Perfetto or chrome://tracing).

    One track per workgroup (tid = workgroup index); every reached boundary closes a complete
    event ("ph": "X") named after it, which spans the time since the workgroup's previous reached
    boundary. Timestamps are microseconds from the earliest step start.
    """
    st = stride(n_layers)
    t = np.asarray(buf, np.int64)[: n_wg * st].reshape(n_wg, st)
    names = ["setup"]
    for l in range(n_layers):
        names += [f"L{l} {e}" for e in LAYER_EVENTS]
    names += list(FINAL_EVENTS)
    started = t[:, 0] > 0
    t0 = int(t[started, 0].min()) if started.any() else 0
    events = []
    for w in range(n_wg):
        if t[w, 0] <= 0:
            continue
        prev = int(t[w, 0])
        for j in range(1, st):
            cur = int(t[w, j])
            if cur <= 0:
                continue
            events.append({"name": names[j - 1], "ph": "X", "pid": 0, "tid": w,
                           "ts": (prev - t0) * TICK_US, "dur": (cur - prev) * TICK_US})
            prev = cur
    meta = [{"name": "thread_name", "ph": "M", "pid": 0, "tid": w, "args": {"name": f"workgroup {w}"}}
            for w in range(n_wg) if t[w, 0] > 0]
    return {"traceEvents": meta + events, "displayTimeUnit": "ns"}

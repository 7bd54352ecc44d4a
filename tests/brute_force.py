"""Scalar brute-force decoder for micro shapes: an independent check of the oracle.

Written with plain Python floats and loops, straight from the textbook
definitions of each operation. It does not import the oracle and shares no
helper with it. Its bf16 rounding picks the nearer of the two neighbouring
bf16 values, where the oracle adds a rounding bias to the bit pattern. Only
for shapes of a few dozen values per dimension.
"""

from __future__ import annotations

import math
import struct


def _f32(x: float) -> float:
    """Nearest float32 to x (struct rounds to nearest, ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _bits32(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def _from_bits32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def bf16_nearest(x: float) -> float:
    """Round a float32 value to bf16: choose the closer neighbour, ties to the even pattern."""
    b = _bits32(x)
    lo_bits = b & 0xFFFF0000
    lo = _from_bits32(lo_bits)
    if lo == x:
        return x
    hi_bits = lo_bits + 0x10000  # next bf16 away from zero (same sign)
    hi = _from_bits32(hi_bits)
    dlo, dhi = abs(x - lo), abs(hi - x)
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if (lo_bits >> 16) % 2 == 0 else hi


def bf16_value(bits: int) -> float:
    return _from_bits32(int(bits) << 16)


def _fp8_rows(t):
    """An E4M3 matrix (codes and per-row scales) -> nested list of Python floats. The codes are
    decoded by torch's float8_e4m3fn type, not by a formula of this file or of the oracle."""
    import torch

    vals = torch.from_numpy(t.codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).tolist()
    return [[v * float(s) for v in row] for row, s in zip(vals, t.scale.tolist())]


def _int8_rows(t):
    """An int8 matrix (codes and per-row scales) -> nested list of Python floats: each code is read
    as a Python int from the signed bytes, then times its row's scale."""
    return [[int(v) * float(s) for v in row] for row, s in zip(t.codes.tolist(), t.scale.tolist())]


def _tolist(t, dtype):
    """Stored tensor -> nested list of Python floats."""
    if hasattr(t, "codes"):
        return _int8_rows(t) if t.codes.dtype.kind == "i" else _fp8_rows(t)
    if dtype in ("bf16", "fp8", "int8"):
        conv = bf16_value
    else:
        conv = float
    if hasattr(t, "ndim") and t.ndim == 2:
        return [[conv(v) for v in row] for row in t.tolist()]
    return [conv(v) for v in t.tolist()]


def matvec(w, x):
    return [sum(w[r][c] * x[c] for c in range(len(x))) for r in range(len(w))]


def decode(shape, weights, feeds, prefill=None):
    """Run (token, position) pairs of one session; return the logits of each.

    ``prefill`` optionally maps (layer, kv_head) -> (keys, values) lists of
    stored vectors for positions 0..n-1.
    """
    m = shape
    dt = weights["dtype"]
    E = _tolist(weights["embed"], dt)
    LM = _tolist(weights["lm_head"], dt)
    gf = _tolist(weights["final_norm"], dt)
    layers = [{k: _tolist(v, dt) for k, v in lw.items()} for lw in weights["layers"]]
    hd, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    grp = hq // hkv
    half = hd // 2

    def store(val):
        v32 = _f32(val)
        return bf16_nearest(v32) if m.kv_dtype == "bf16" else v32

    def norm(x, g):
        ms = sum(v * v for v in x) / len(x)
        inv = 1.0 / math.sqrt(ms + m.norm_eps)
        return [x[i] * inv * g[i] for i in range(len(x))]

    def rotate(vec, pos):
        out = list(vec)
        for i in range(half):
            ang = pos * (m.rope_base ** (-(2.0 * i) / hd))
            c, s = math.cos(ang), math.sin(ang)
            a, b = vec[i], vec[i + half]
            out[i] = a * c - b * s
            out[i + half] = a * s + b * c
        return out

    K = [[dict() for _ in range(hkv)] for _ in range(m.n_layers)]
    V = [[dict() for _ in range(hkv)] for _ in range(m.n_layers)]
    if prefill:
        for (l, g), (ks, vs) in prefill.items():
            for j, (kv, vv) in enumerate(zip(ks, vs)):
                K[l][g][j] = list(kv)
                V[l][g][j] = list(vv)

    results = []
    for token, pos in feeds:
        x = list(E[token])
        for l, lw in enumerate(layers):
            h = norm(x, lw["attn_norm"])
            q = matvec(lw["wq"], h)
            k = matvec(lw["wk"], h)
            v = matvec(lw["wv"], h)
            for g in range(hkv):
                kg = rotate(k[g * hd:(g + 1) * hd], pos)
                K[l][g][pos] = [store(t) for t in kg]
                V[l][g][pos] = [store(t) for t in v[g * hd:(g + 1) * hd]]
            o = []
            for hh in range(hq):
                g = hh // grp
                qh = rotate(q[hh * hd:(hh + 1) * hd], pos)
                scores = []
                for j in range(pos + 1):
                    kj = K[l][g][j]
                    scores.append(sum(qh[i] * kj[i] for i in range(hd)) / math.sqrt(hd))
                mx = max(scores)
                ex = [math.exp(s - mx) for s in scores]
                tot = sum(ex)
                for i in range(hd):
                    o.append(sum(ex[j] / tot * V[l][g][j][i] for j in range(pos + 1)))
            att = matvec(lw["wo"], o)
            x = [x[i] + att[i] for i in range(len(x))]
            h2 = norm(x, lw["ffn_norm"])
            gate = matvec(lw["w_gate"], h2)
            up = matvec(lw["w_up"], h2)
            act = [gate[i] / (1.0 + math.exp(-gate[i])) * up[i] for i in range(len(gate))]
            down = matvec(lw["w_down"], act)
            x = [x[i] + down[i] for i in range(len(x))]
        hf = norm(x, gf)
        results.append(matvec(LM, hf))
    return results

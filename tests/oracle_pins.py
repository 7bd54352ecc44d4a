"""Pins that tie the reference decoder to facts outside itself.

Each ``pin_*`` function takes the decoder module as an argument, so the same
checks run against the real oracle (all must pass) and against copies with
planted mistakes (at least one must fail; see test_oracle_mutants.py).

What each pin rests on:

* a brute-force scalar decoder written independently (tests/brute_force.py);
* invariants: incremental KV-cache decoding equals recomputing the full
  sequence; softmax rows sum to 1; RoPE preserves norms and its dot products
  depend only on the position difference;
* closed forms: a single cached position returns its V; identical keys give
  the mean of V; two keys with score gap a give weights sigmoid(a); RoPE of a
  unit vector; RMS of an RMSNorm output; silu at special points; zero
  attention and FFN outputs leave the embedding untouched;
* library routines: torch's float32 -> bfloat16 conversion, numpy's argmax
  and scipy's logistic function; torch's float8_e4m3fn type for the value of
  every FP8 E4M3 code, and the brute force fed the weights torch decodes for
  an fp8 model; for an int8 model, the brute force fed each code as a Python
  integer (every value -128..127 occurs) times its row's scale.
"""

from __future__ import annotations

import numpy as np

import workloads
from workloads import ModelShape

from . import brute_force

MICRO_GQA = ModelShape(2, 16, 4, 2, 8, 24, 40, rope_base=10000.0, weight_dtype="bf16", kv_dtype="bf16")
MICRO_MHA_F32 = ModelShape(1, 12, 3, 3, 4, 20, 33, rope_base=500.0, weight_dtype="f32", kv_dtype="f32")
MICRO_FP8 = ModelShape(2, 16, 4, 2, 8, 24, 40, rope_base=10000.0, weight_dtype="fp8", kv_dtype="bf16")
MICRO_INT8 = ModelShape(2, 16, 4, 2, 8, 24, 40, rope_base=10000.0, weight_dtype="int8", kv_dtype="bf16")
FP8_MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def micro_weights(shape: ModelShape, seed: int = 7) -> dict:
    """Seeded weights with random (not unit) norm gains, so each gain matters."""
    w = workloads.make_weights(shape, seed=seed, workers=1)
    rng = np.random.default_rng(seed + 1000)

    def gain(n):
        g = rng.uniform(0.5, 1.5, n).astype(np.float32)
        return workloads.bf16_bits_from_f32(g) if shape.weight_dtype == "bf16" else g

    for lw in w["layers"]:
        lw["attn_norm"] = gain(shape.d_model)
        lw["ffn_norm"] = gain(shape.d_model)
    w["final_norm"] = gain(shape.d_model)
    # larger matrices than the 0.02 default so that every term is visible
    for lw in w["layers"]:
        for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            vals = rng.standard_normal(lw[name].shape).astype(np.float32) * np.float32(0.4)
            lw[name] = workloads.bf16_bits_from_f32(vals) if shape.weight_dtype == "bf16" else vals
    return w


def micro_fp8_weights(seed: int = 41) -> dict:
    """An fp8 micro model whose codes cover every finite E4M3 value (both signs, the subnormals,
    448) and whose row scales differ from row to row, so a code misread or a scale applied to the
    wrong row or column shows."""
    w = micro_weights(MICRO_GQA, seed=seed)
    w["dtype"] = "fp8"
    rng = np.random.default_rng(seed + 2000)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)

    def fp8(shape):
        codes = rng.choice(finite, size=shape).astype(np.uint8)
        codes.reshape(-1)[: finite.size] = finite[: min(finite.size, codes.size)]
        scale = (rng.uniform(0.25, 2.0, shape[0]) * (0.4 / 448.0)).astype(np.float32)
        return workloads.Fp8Matrix(codes, scale)

    for lw in w["layers"]:
        for name in FP8_MATRICES:
            lw[name] = fp8(lw[name].shape)
    w["lm_head"] = fp8(w["lm_head"].shape)
    return w


def micro_int8_weights(seed: int = 43) -> dict:
    """An int8 micro model whose codes cover every value -128..127 and whose row scales differ
    from row to row, so a code read without its sign, or a scale applied to the wrong row or
    column, shows."""
    w = micro_weights(MICRO_GQA, seed=seed)
    w["dtype"] = "int8"
    rng = np.random.default_rng(seed + 2000)
    every = np.arange(-128, 128, dtype=np.int16).astype(np.int8)

    def int8(shape):
        codes = rng.integers(-128, 128, size=shape).astype(np.int8)
        codes.reshape(-1)[: every.size] = every[: min(every.size, codes.size)]
        scale = (rng.uniform(0.25, 2.0, shape[0]) * (0.4 / 127.0)).astype(np.float32)
        return workloads.Int8Matrix(codes, scale)

    for lw in w["layers"]:
        for name in FP8_MATRICES:
            lw[name] = int8(lw[name].shape)
    w["lm_head"] = int8(w["lm_head"].shape)
    return w


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------- #
def pin_brute_force(mod):
    """Whole decoder on micro shapes equals the scalar brute-force decoder."""
    for shape, feeds in (
        (MICRO_GQA, [(3, 0), (17, 1), (39, 2), (0, 3), (22, 4), (5, 5)]),
        (MICRO_MHA_F32, [(1, 0), (32, 1), (7, 2), (7, 3)]),
    ):
        w = micro_weights(shape)
        o = mod.Oracle(shape, w, batch=1, max_seq=8)
        ref = brute_force.decode(shape, w, feeds)
        for (tok, pos), r in zip(feeds, ref):
            got = o.step_one(0, tok, pos)
            assert _rel(got, r) < 1e-9, (shape, pos, _rel(got, r))


def pin_brute_force_prefilled(mod):
    """Steps that start from a pre-filled cache equal the brute force fed the same cache."""
    shape = MICRO_GQA
    w = micro_weights(shape, seed=11)
    rng = np.random.default_rng(5)
    n0 = 5
    o = mod.Oracle(shape, w, batch=1, max_seq=n0 + 3)
    pre = {}
    for l in range(shape.n_layers):
        for g in range(shape.n_kv_heads):
            ks = workloads.f32_from_bf16_bits(workloads.bf16_bits_from_f32(rng.standard_normal((n0, shape.head_dim)).astype(np.float32)))
            vs = workloads.f32_from_bf16_bits(workloads.bf16_bits_from_f32(rng.standard_normal((n0, shape.head_dim)).astype(np.float32)))
            o.load_kv(0, l, g, ks, vs)
            pre[(l, g)] = (ks.astype(np.float64).tolist(), vs.astype(np.float64).tolist())
    feeds = [(9, n0), (30, n0 + 1), (2, n0 + 2)]
    ref = brute_force.decode(shape, w, feeds, prefill=pre)
    for (tok, pos), r in zip(feeds, ref):
        assert _rel(o.step_one(0, tok, pos), r) < 1e-9


def pin_incremental_equals_full(mod):
    """KV-cache decoding, token by token, equals causal recomputation of the whole sequence."""
    for shape in (MICRO_GQA, MICRO_MHA_F32, ModelShape(2, 32, 4, 1, 8, 40, 50, rope_base=10000.0)):
        w = micro_weights(shape, seed=3)
        seq = np.random.default_rng(1).integers(0, shape.vocab, 9)
        o = mod.Oracle(shape, w, batch=1, max_seq=len(seq))
        inc = np.stack([o.step_one(0, int(t), p) for p, t in enumerate(seq)])
        full = mod.forward_full(shape, w, seq)
        assert _rel(inc, full) < 1e-9


def pin_softmax(mod):
    rng = np.random.default_rng(2)
    s = rng.standard_normal((7, 13)) * 10
    p = mod.softmax(s)
    assert np.allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p > 0)
    assert np.allclose(mod.softmax(s + 123.0), p, rtol=1e-12, atol=0)
    # a row with one dominant entry
    big = np.zeros(5)
    big[3] = 800.0
    assert abs(mod.softmax(big)[3] - 1.0) < 1e-15


def pin_rope(mod):
    hd, base = 16, 10000.0
    half = hd // 2
    for pos in (0, 1, 7, 1000, 32767):
        cos, sin = mod.rope_cos_sin(pos, hd, base)
        for i in range(half):
            theta = base ** (-2.0 * i / hd)
            # unit vector e_i turns towards e_{i+half}; e_{i+half} turns towards -e_i
            e = np.zeros(hd)
            e[i] = 1.0
            r = mod.apply_rope(e, cos, sin)
            want = np.zeros(hd)
            want[i] = np.cos(pos * theta)
            want[i + half] = np.sin(pos * theta)
            assert np.allclose(r, want, rtol=0, atol=1e-12), (pos, i)
            e2 = np.zeros(hd)
            e2[i + half] = 1.0
            r2 = mod.apply_rope(e2, cos, sin)
            want2 = np.zeros(hd)
            want2[i] = -np.sin(pos * theta)
            want2[i + half] = np.cos(pos * theta)
            assert np.allclose(r2, want2, rtol=0, atol=1e-12), (pos, i)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, hd))
    c0, s0 = mod.rope_cos_sin(0, hd, base)
    assert np.array_equal(mod.apply_rope(x, c0, s0), x)
    for pos in (3, 99, 4096):
        c, s = mod.rope_cos_sin(pos, hd, base)
        assert np.allclose(np.linalg.norm(mod.apply_rope(x, c, s), axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)

    def dot(m, n):
        cm, sm = mod.rope_cos_sin(m, hd, base)
        cn, sn = mod.rope_cos_sin(n, hd, base)
        return mod.apply_rope(q, cm, sm) @ mod.apply_rope(k, cn, sn)

    assert abs(dot(10, 4) - dot(106, 100)) < 1e-10
    assert abs(dot(3, 3) - q @ k) < 1e-12


def pin_attention(mod):
    rng = np.random.default_rng(8)
    hd = 8
    # one cached position: the output is that position's V, whatever q is
    q = rng.standard_normal((2, hd)) * 50
    k = rng.standard_normal((1, 1, hd))
    v = rng.standard_normal((1, 1, hd))
    out = mod.attend(q, k, v)
    assert np.allclose(out, np.broadcast_to(v[0, 0], (2, hd)), rtol=0, atol=1e-15)
    # identical keys: uniform weights, output = mean of V
    kk = np.broadcast_to(rng.standard_normal(hd), (1, 6, hd)).copy()
    vv = rng.standard_normal((1, 6, hd))
    out = mod.attend(rng.standard_normal((1, hd)), kk, vv)
    assert np.allclose(out[0], vv[0].mean(0), rtol=1e-12, atol=1e-14)
    # two keys whose scaled scores differ by a: weight sigmoid(a) on the first
    a = 1.3
    qv = np.zeros((1, hd))
    qv[0, 0] = 1.0
    k2 = np.zeros((1, 2, hd))
    k2[0, 0, 0] = a * np.sqrt(hd)
    v2 = rng.standard_normal((1, 2, hd))
    w0 = 1.0 / (1.0 + np.exp(-a))
    assert np.allclose(mod.attend(qv, k2, v2)[0], w0 * v2[0, 0] + (1 - w0) * v2[0, 1], rtol=1e-12)


def pin_gqa(mod):
    """Grouped-query attention equals multi-head attention with each kv head repeated G times."""
    rng = np.random.default_rng(9)
    hq, hkv, n, hd = 6, 2, 5, 4
    q = rng.standard_normal((hq, hd))
    k = rng.standard_normal((hkv, n, hd))
    v = rng.standard_normal((hkv, n, hd))
    g = hq // hkv
    k_rep = np.repeat(k, g, axis=0)
    v_rep = np.repeat(v, g, axis=0)
    assert np.allclose(mod.attend(q, k, v), mod.attend(q, k_rep, v_rep), rtol=1e-13)
    # and MHA per head is a plain softmax-weighted sum
    for h in range(hq):
        s = k_rep[h] @ q[h] / np.sqrt(hd)
        w = np.exp(s - s.max())
        w /= w.sum()
        assert np.allclose(mod.attend(q, k_rep, v_rep)[h], w @ v_rep[h], rtol=1e-13)


def pin_rmsnorm(mod):
    rng = np.random.default_rng(10)
    eps = 1e-5
    for scale in (1e-3, 1.0, 40.0):
        x = rng.standard_normal(64) * scale
        y = mod.rms_norm(x, np.ones(64), eps)
        ms = np.mean(x * x)
        assert abs(np.sqrt(np.mean(y * y)) - 1.0 / np.sqrt(1.0 + eps / ms)) < 1e-12
    x = rng.standard_normal(32)
    g = rng.uniform(0.5, 2.0, 32)
    # scale invariance: rms_norm(c x) with eps*c^2 equals rms_norm(x) with eps
    assert np.allclose(mod.rms_norm(7.0 * x, g, eps * 49.0), mod.rms_norm(x, g, eps), rtol=1e-13)
    # the gain multiplies each normalised component
    assert np.allclose(mod.rms_norm(x, g, eps), mod.rms_norm(x, np.ones(32), eps) * g, rtol=1e-14)


def pin_silu(mod):
    from scipy.special import expit

    assert mod.silu(np.array([0.0]))[0] == 0.0
    y = np.linspace(-30, 30, 121)
    assert np.allclose(mod.silu(y), y * expit(y), rtol=1e-13, atol=1e-300)
    assert abs(mod.silu(np.array([50.0]))[0] - 50.0) < 1e-15
    assert abs(mod.silu(np.array([-50.0]))[0]) < 1e-18
    # odd-even identity: silu(y) - silu(-y) = y
    assert np.allclose(mod.silu(y) - mod.silu(-y), y, rtol=0, atol=1e-12)


def pin_argmax(mod):
    l = np.array([[0.5, 2.0, -1.0, 2.0, 1.0], [3.0, 3.0, 3.0, 3.0, 3.0]])
    assert mod.greedy_token(l).tolist() == [1, 0]
    # values equal after rounding to float32 tie; the lower index wins
    tiny = np.array([[1.0, 1.0 + 1e-12, 0.0]])
    assert mod.greedy_token(tiny).tolist() == [0]
    rng = np.random.default_rng(12)
    r = rng.standard_normal((20, 1000))
    assert np.array_equal(mod.greedy_token(r), np.argmax(r.astype(np.float32), axis=-1))


def pin_bf16(mod, n_random: int = 1 << 20):
    """Round-to-nearest-even float32 -> bf16 agrees with torch on edge and random patterns."""
    import torch

    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    pats = (hi[:, None] | lows[None, :]).reshape(-1)
    rng = np.random.default_rng(13)
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, n_random, dtype=np.uint64).astype(np.uint32)])
    x = pats.view(np.float32)
    finite = np.isfinite(x)
    ours = mod.round_f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.all(np.isnan(ours[np.isnan(x)]))
    inf = np.isinf(x)
    assert np.array_equal(ours[inf], x[inf])


def pin_identity_layers(mod):
    """With W_o = 0 and W_down = 0 every layer passes x through: logits depend on the token only."""
    shape = MICRO_GQA
    w = micro_weights(shape, seed=21)
    for lw in w["layers"]:
        lw["wo"] = np.zeros_like(lw["wo"])
        lw["w_down"] = np.zeros_like(lw["w_down"])
    dt = w["dtype"]
    emb = workloads.f32_from_bf16_bits(w["embed"]).astype(np.float64)
    lm = workloads.f32_from_bf16_bits(w["lm_head"]).astype(np.float64)
    gf = workloads.f32_from_bf16_bits(w["final_norm"]).astype(np.float64)
    assert dt == "bf16"
    o = mod.Oracle(shape, w, batch=1, max_seq=6)
    for pos, tok in enumerate([4, 9, 4, 31, 0]):
        got = o.step_one(0, tok, pos)
        x = emb[tok]
        want = lm @ (x / np.sqrt(np.mean(x * x) + shape.norm_eps) * gf)
        assert _rel(got, want) < 1e-12


def pin_sessions_independent(mod):
    """Sessions stepped together are independent: a multi-session step of sessions in a scrambled
    order, at ragged positions with distinct tokens, gives each session bit for bit what a
    one-session oracle fed the same history gives, and what the brute force gives."""
    shape = MICRO_GQA
    w = micro_weights(shape, seed=31)
    # per session: its own token history (session s has its own length and ids)
    hist = {0: [5, 11, 2, 37], 1: [23, 8], 2: [1, 14, 39, 6, 20, 9]}
    multi = mod.Oracle(shape, w, batch=3, max_seq=8)
    single = {s: mod.Oracle(shape, w, batch=1, max_seq=8) for s in hist}
    brute = {s: brute_force.decode(shape, w, [(t, p) for p, t in enumerate(seq)]) for s, seq in hist.items()}
    got = {s: [] for s in hist}
    # ticks: each names the sessions stepped together, in the order passed
    ticks = [[2, 0, 1], [0, 2], [2, 1, 0], [0, 2], [2], [2]]
    pos = {s: 0 for s in hist}
    for tick in ticks:
        toks = [hist[s][pos[s]] for s in tick]
        ps = [pos[s] for s in tick]
        out = multi.step_sessions(tick, toks, ps)
        for i, s in enumerate(tick):
            got[s].append(out[i])
            pos[s] += 1
    for s, seq in hist.items():
        assert pos[s] == len(seq)
        want = [single[s].step_one(0, t, p) for p, t in enumerate(seq)]
        for p in range(len(seq)):
            assert np.array_equal(np.asarray(got[s][p]).view(np.uint64), np.asarray(want[p]).view(np.uint64)), (s, p)
            assert _rel(got[s][p], brute[s][p]) < 1e-9, (s, p)
        # the cache rows of the session hold exactly its own history
        n = len(seq)
        assert np.array_equal(multi.k_cache[s, :, :, :n], single[s].k_cache[0, :, :, :n])
        assert np.array_equal(multi.v_cache[s, :, :, :n], single[s].v_cache[0, :, :, :n])
        assert not np.any(multi.k_cache[s, :, :, n:])


def pin_fp8(mod):
    """FP8 E4M3 weights: every code's value equals torch's float8_e4m3fn value, and an fp8 micro
    model steps exactly as the brute force fed the weights torch decodes (codes times row scales)."""
    import torch

    codes = np.arange(256, dtype=np.uint8)
    ours = mod.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    w = micro_fp8_weights()
    o = mod.Oracle(MICRO_FP8, w, batch=1, max_seq=8)
    feeds = [(3, 0), (17, 1), (39, 2), (0, 3), (22, 4)]
    want = brute_force.decode(MICRO_FP8, w, feeds)
    for (tok, pos), r in zip(feeds, want):
        got = o.step_one(0, tok, pos)
        assert _rel(got, r) < 1e-9, (pos, _rel(got, r))


def pin_int8(mod):
    """int8 weights: an int8 micro model steps exactly as the brute force fed each code as a
    Python integer times its row's scale."""
    w = micro_int8_weights()
    o = mod.Oracle(MICRO_INT8, w, batch=1, max_seq=8)
    feeds = [(3, 0), (17, 1), (39, 2), (0, 3), (22, 4)]
    want = brute_force.decode(MICRO_INT8, w, feeds)
    for (tok, pos), r in zip(feeds, want):
        got = o.step_one(0, tok, pos)
        assert _rel(got, r) < 1e-9, (pos, _rel(got, r))


ALL_PINS = [
    pin_brute_force,
    pin_brute_force_prefilled,
    pin_incremental_equals_full,
    pin_softmax,
    pin_rope,
    pin_attention,
    pin_gqa,
    pin_rmsnorm,
    pin_silu,
    pin_argmax,
    pin_bf16,
    pin_identity_layers,
    pin_sessions_independent,
    pin_fp8,
    pin_int8,
]

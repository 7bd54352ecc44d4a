"""Reference decoder on the CPU (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The HIP library never calls it, and it
shares no code with the library: no kernels, headers, helpers or tables.
Only the seeded input generators in ``workloads/`` serve both.

What it computes
----------------
One step of a pre-norm decoder with grouped-query attention, rotary position
embeddings and a SwiGLU feed-forward block, followed by a greedy argmax.

The pages explain *why* this step is bound by memory bandwidth. Producing one
token reads every weight plus the whole KV cache ("Kog 3000 tok/s real-time
inference", section "three-layer strategy for memory-bandwidth
optimisation"). The single-request engine runs the whole step without
returning to the host ("Real-time LLM inference on standard data-centre GPUs
(3,000 tokens/s single request)", section "technical principles"). The pages
print no equations for the individual operations, so each function below
states the textbook definition it implements. The readings of points the
pages leave open are:

* RoPE rotates the pair (i, i + hd/2) ("rotate-half") by the angle
  p * base**(-2i/hd), with p counted from 0 at the first prompt token.
* q head h reads kv head floor(h / G), where G = Hq / Hkv.
* Attention is causal and includes the current token. Scores are scaled by
  1/sqrt(hd). There are no biases and no window.
* RMSNorm puts eps inside the square root and multiplies by the gain after
  normalising. The norm gains are part of the weights.
* silu(y) = y / (1 + exp(-y)); the FFN output is W_down (silu(W_gate h) * (W_up h)).
* Embedding and LM head are separate tensors.

Precision. Activations are float64. Weights are the exact values of the
stored bf16 or float32 numbers. Two points mirror what the kernel stores or
decides:

* The KV cache holds the kernel's storage type: each K (after RoPE) and V
  value is rounded to float32, then to bf16 for a bf16 cache.
* The next token is the argmax of the logits rounded to float32, lowest
  index on ties. The kernel takes that decision in float32.

FP8 weights. Lowering the precision of the parameters cuts the bytes every
token reads ("17k tokens/sec" page, best practice 2 and FAQ 3, which names
FP8). An fp8 model stores each projection matrix and the LM head as OCP FP8
E4M3 codes with one float32 scale per output row; its embedding and norm gains
are bf16. The oracle is fed those codes and scales and computes with the
weights they stand for, code value times row scale, exactly in float64.

INT8 weights (the same page, best practice 2, names INT8): the projection
matrices and the LM head are int8 codes (two's complement) with one float32
scale per output row; the weight is the code times its row's scale, exactly in
float64. Everything else is as for fp8 models.
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------- #
# number formats
# --------------------------------------------------------------------------- #
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the pattern is the top half of a float32."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16, ties to even; return float32 values.

    A bf16 keeps the sign, the 8 exponent bits and the top 7 fraction bits of
    a float32. Rounding adds half of the dropped range, plus one when the kept
    part is odd, so that exact halves go to the even neighbour. A carry
    simply moves into the exponent. NaN stays a quiet NaN.
    """
    x = np.asarray(x, np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    keep_odd = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + keep_odd) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value after storing ``x`` in a cache of ``dtype`` ("f32" or "bf16"); returned as float64."""
    f32 = np.asarray(x, np.float64).astype(np.float32)
    if dtype == "bf16":
        f32 = round_f32_to_bf16(f32)
    elif dtype != "f32":
        raise ValueError(f"unknown storage dtype {dtype!r}")
    return f32.astype(np.float64)


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 bit patterns: sign, 4 exponent bits (bias 7), 3 fraction bits.

    Exponent field 0 holds the subnormals f/8 * 2**-6; every other field e holds
    (1 + f/8) * 2**(e - 7). There are no infinities; S.1111.111 is NaN.
    """
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, f / 8.0 * 2.0**-6, (1.0 + f / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, out)


# the value of every code, from the definition above (large matrices index it rather than
# evaluating the definition element by element)
_E4M3_VALUES = fp8_e4m3_to_f64(np.arange(256, dtype=np.uint8))


def weight_f64(w, dtype: str) -> np.ndarray:
    """float64 values of a stored weight tensor.

    bf16 bit patterns or float32 arrays; for fp8 (int8) models, an object with ``codes`` (E4M3
    bit patterns, or int8 values, [rows, cols]) and ``scale`` (float32 [rows]) for each projection
    matrix, whose value is the code's value times its row's scale, and bf16 patterns for the rest.
    """
    if dtype == "fp8" and hasattr(w, "codes"):
        return _E4M3_VALUES[np.asarray(w.codes, np.uint8)] * np.asarray(w.scale, np.float32).astype(np.float64)[:, None]
    if dtype == "int8" and hasattr(w, "codes"):
        return np.asarray(w.codes, np.int8).astype(np.float64) * np.asarray(w.scale, np.float32).astype(np.float64)[:, None]
    if dtype in ("bf16", "fp8", "int8"):
        return bf16_to_f64(w)
    if dtype == "f32":
        return np.asarray(w, np.float32).astype(np.float64)
    raise ValueError(f"unknown weight dtype {dtype!r}")


# --------------------------------------------------------------------------- #
# the operations of one layer
# --------------------------------------------------------------------------- #
def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps), times the gain; over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def rope_cos_sin(position: int, head_dim: int, base: float):
    """cos and sin of position * base**(-2i/head_dim) for i < head_dim/2, in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * i / head_dim)
    angle = np.float64(position) * theta
    return np.cos(angle), np.sin(angle)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate each pair (x_i, x_{i+hd/2}) of the last axis by the angle whose cos/sin are given."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum exp(s - max s) over the last axis."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def silu(y: np.ndarray) -> np.ndarray:
    """y * sigmoid(y) = y / (1 + exp(-y))."""
    return y / (1.0 + np.exp(-y))


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Attention of one query position over n cached positions.

    q: [Hq, hd]; k, v: [Hkv, n, hd].  q head h uses kv head h // (Hq/Hkv).
    Returns [Hq, hd]: for each head, softmax(q . K_j / sqrt(hd)) weighted sum of V_j.
    """
    hq, hd = q.shape
    group = hq // k.shape[0]
    out = np.empty_like(q)
    for h in range(hq):
        g = h // group
        w = softmax(k[g] @ q[h] / np.sqrt(hd))
        out[h] = w @ v[g]
    return out


def greedy_token(logits: np.ndarray) -> np.ndarray:
    """Lowest index of the maximum of the logits rounded to float32, per row."""
    l32 = np.asarray(logits, np.float64).astype(np.float32)
    if np.isnan(l32).any():
        raise ValueError("NaN in logits")
    return np.argmax(l32, axis=-1).astype(np.int32)


# --------------------------------------------------------------------------- #
# the decoder
# --------------------------------------------------------------------------- #
class Oracle:
    """Incremental decoder over a per-session KV cache.

    ``weights`` is the dict made by ``workloads.make_weights`` (bf16 bit
    patterns or float32 arrays).  Each session b owns a K and a V cache of
    ``max_seq`` positions per layer and kv head, holding values as stored
    (rounded to the cache type).
    """

    def __init__(self, shape, weights: dict, batch: int = 1, max_seq: int = 0):
        if shape.n_q_heads % shape.n_kv_heads:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        if shape.head_dim % 2:
            raise ValueError("head_dim must be even")
        self.shape = shape
        self.w = weights
        self.wdt = weights["dtype"]
        self.batch = batch
        self.max_seq = max_seq
        m = shape
        # cached values are exact in float32 (they are float32 or bf16 numbers)
        self.k_cache = np.zeros((batch, m.n_layers, m.n_kv_heads, max_seq, m.head_dim), np.float32)
        self.v_cache = np.zeros_like(self.k_cache)
        # For a small model, the float64 value of each stored matrix is made once instead of at
        # every use (the same values; large models convert per use to bound host memory). The
        # dict holds the stored arrays' ids, which stay unique while self.w keeps them alive.
        self._f64 = {}
        stored = [lw[k] for lw in weights["layers"] for k in lw] + [weights["final_norm"], weights["lm_head"]]
        if sum(a.size for a in stored) * 8 <= (1 << 30):
            self._f64 = {id(a): weight_f64(a, self.wdt) for a in stored}

    def mat(self, t: np.ndarray) -> np.ndarray:
        cached = self._f64.get(id(t))
        return cached if cached is not None else weight_f64(t, self.wdt)

    def load_kv(self, session: int, layer: int, kv_head: int, keys: np.ndarray, values: np.ndarray) -> None:
        """Put pre-filled cache contents (already in storage precision) at positions 0..n-1."""
        n = keys.shape[0]
        if n > self.max_seq:
            raise ValueError("pre-filled length exceeds max_seq")
        self.k_cache[session, layer, kv_head, :n] = keys
        self.v_cache[session, layer, kv_head, :n] = values

    def _store(self, x: np.ndarray) -> np.ndarray:
        return to_storage(x, self.shape.kv_dtype).astype(np.float32)

    def step_sessions(self, sessions, tokens, positions) -> np.ndarray:
        """Feed ``tokens[i]`` of session ``sessions[i]`` at ``positions[i]``; return logits [n, V] (float64).

        Sessions are independent: each goes through exactly the operations of a step of its own.
        The loop is layer-major only so that a layer's weights are converted to float64 once per
        call rather than once per session.
        """
        m, w = self.shape, self.w
        hd, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
        for token, position in zip(tokens, positions):
            if not 0 <= token < m.vocab:
                raise ValueError(f"token {token} out of range")
            if not 0 <= position < self.max_seq:
                raise ValueError(f"position {position} out of range")
        rope = [rope_cos_sin(int(p), hd, m.rope_base) for p in positions]
        xs = [self.mat(w["embed"][int(t)]) for t in tokens]
        for l, lw in enumerate(w["layers"]):
            W = {k: self.mat(lw[k]) for k in lw}
            for i, session in enumerate(sessions):
                position = int(positions[i])
                cos, sin = rope[i]
                x = xs[i]
                h = rms_norm(x, W["attn_norm"], m.norm_eps)
                q = (W["wq"] @ h).reshape(hq, hd)
                k = (W["wk"] @ h).reshape(hkv, hd)
                v = (W["wv"] @ h).reshape(hkv, hd)
                q = apply_rope(q, cos, sin)
                k = apply_rope(k, cos, sin)
                self.k_cache[session, l, :, position] = self._store(k)
                self.v_cache[session, l, :, position] = self._store(v)
                kc = self.k_cache[session, l, :, : position + 1].astype(np.float64)
                vc = self.v_cache[session, l, :, : position + 1].astype(np.float64)
                o = attend(q, kc, vc).reshape(hq * hd)
                x = x + W["wo"] @ o
                h2 = rms_norm(x, W["ffn_norm"], m.norm_eps)
                a = silu(W["w_gate"] @ h2) * (W["w_up"] @ h2)
                xs[i] = x + W["w_down"] @ a
            del W
        g_final = self.mat(w["final_norm"])
        lm = self.mat(w["lm_head"])
        return np.stack([lm @ rms_norm(x, g_final, m.norm_eps) for x in xs])

    def step_one(self, session: int, token: int, position: int) -> np.ndarray:
        """Feed one token of one session at ``position``; return its logits [V] (float64)."""
        return self.step_sessions([session], [token], [position])[0]

    def step(self, tokens, positions) -> np.ndarray:
        """One step of every session: ``tokens[b]`` at ``positions[b]``; logits [B, V]."""
        return self.step_sessions(range(self.batch), [int(t) for t in tokens], [int(p) for p in positions])

    def generate(self, prompt, n_tokens: int, session: int = 0):
        """Feed ``prompt`` from position 0, then greedily generate ``n_tokens`` tokens.

        Returns (generated ids, logits of every step that produced one).
        """
        logits = None
        for p, t in enumerate(prompt):
            logits = self.step_one(session, int(t), p)
        out, all_logits = [], []
        pos = len(prompt)
        for i in range(n_tokens):
            nxt = int(greedy_token(logits[None])[0])
            out.append(nxt)
            all_logits.append(logits)
            if i + 1 < n_tokens:
                logits = self.step_one(session, nxt, pos)
                pos += 1
        return np.array(out, np.int32), np.stack(all_logits)


def forward_full(shape, weights: dict, tokens) -> np.ndarray:
    """Logits at every position of ``tokens`` (positions 0..T-1), with no cache.

    The whole sequence goes through each layer at once, with a causal mask.
    K and V are rounded to the cache type, as the incremental path stores
    them.
    """
    m, w = shape, weights
    wdt = w["dtype"]
    mat = lambda t: weight_f64(t, wdt)  # noqa: E731
    tokens = np.asarray(tokens)
    n = len(tokens)
    hd, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    group = hq // hkv
    cs = [rope_cos_sin(p, hd, m.rope_base) for p in range(n)]
    cos = np.stack([c for c, _ in cs])[:, None, :]
    sin = np.stack([s for _, s in cs])[:, None, :]
    causal = np.tril(np.ones((n, n), bool))
    x = mat(w["embed"][tokens])
    for lw in w["layers"]:
        h = rms_norm(x, mat(lw["attn_norm"]), m.norm_eps)
        q = apply_rope((h @ mat(lw["wq"]).T).reshape(n, hq, hd), cos, sin)
        k = apply_rope((h @ mat(lw["wk"]).T).reshape(n, hkv, hd), cos, sin)
        v = (h @ mat(lw["wv"]).T).reshape(n, hkv, hd)
        k = to_storage(k, m.kv_dtype)
        v = to_storage(v, m.kv_dtype)
        o = np.empty((n, hq, hd))
        for hh in range(hq):
            g = hh // group
            s = (q[:, hh, :] @ k[:, g, :].T) / np.sqrt(hd)
            s = np.where(causal, s, -np.inf)
            o[:, hh, :] = softmax(s) @ v[:, g, :]
        x = x + o.reshape(n, hq * hd) @ mat(lw["wo"]).T
        h2 = rms_norm(x, mat(lw["ffn_norm"]), m.norm_eps)
        a = silu(h2 @ mat(lw["w_gate"]).T) * (h2 @ mat(lw["w_up"]).T)
        x = x + a @ mat(lw["w_down"]).T
    hf = rms_norm(x, mat(w["final_norm"]), m.norm_eps)
    return hf @ mat(w["lm_head"]).T

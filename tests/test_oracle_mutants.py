"""Plant plausible mistakes in a copy of the reference decoder and check that the pins catch each.

Every mutant rewrites one spot of ``oracle/decoder.py`` in memory (the file
is never touched), loads the copy as a separate module and runs the pins.
At least one pin has to fail.  This shows that the pins would notice such a
slip in the oracle itself.
"""

import os
import types

import pytest

from . import oracle_pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "decoder.py")

MUTANTS = {
    "rope_interleaved_pairs": (
        "a, b = x[..., :half], x[..., half:]\n    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)",
        "a, b = x[..., 0::2], x[..., 1::2]\n    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)",
    ),
    "rope_sign_flip": ("[a * cos - b * sin, a * sin + b * cos]", "[a * cos + b * sin, -a * sin + b * cos]"),
    "rope_wrong_frequency": ("-2.0 * i / head_dim", "-1.0 * i / head_dim"),
    "attention_no_scale": ("k[g] @ q[h] / np.sqrt(hd)", "k[g] @ q[h]"),
    "gqa_modulo_map": ("g = h // group", "g = h % k.shape[0]"),
    "causal_excludes_current": (
        "kc = self.k_cache[session, l, :, : position + 1]",
        "kc = self.k_cache[session, l, :, : position]",
    ),
    "attention_residual_dropped": ('x = x + W["wo"] @ o', 'x = W["wo"] @ o'),
    "ffn_residual_dropped": ('xs[i] = x + W["w_down"] @ a', 'xs[i] = W["w_down"] @ a'),
    "silu_on_up_branch": (
        'a = silu(W["w_gate"] @ h2) * (W["w_up"] @ h2)',
        'a = (W["w_gate"] @ h2) * silu(W["w_up"] @ h2)',
    ),
    "rmsnorm_eps_outside_sqrt": ("x / np.sqrt(ms + eps) * gain", "x / (np.sqrt(ms) + eps) * gain"),
    "rmsnorm_sum_not_mean": ("ms = np.mean(x * x, axis=-1, keepdims=True)", "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    "k_cached_before_rope": (
        "                k = apply_rope(k, cos, sin)\n                self.k_cache[session, l, :, position] = self._store(k)",
        "                self.k_cache[session, l, :, position] = self._store(k)\n                k = apply_rope(k, cos, sin)",
    ),
    "ffn_uses_attention_gain": ('h2 = rms_norm(x, W["ffn_norm"]', 'h2 = rms_norm(x, W["attn_norm"]'),
    "final_norm_skipped": (
        "return np.stack([lm @ rms_norm(x, g_final, m.norm_eps) for x in xs])",
        "return np.stack([lm @ x for x in xs])",
    ),
    "lm_head_tied_to_embedding": ('lm = self.mat(w["lm_head"])', 'lm = self.mat(w["embed"])'),
    "wk_wv_swapped": (
        'k = (W["wk"] @ h).reshape(hkv, hd)\n                v = (W["wv"] @ h)',
        'k = (W["wv"] @ h).reshape(hkv, hd)\n                v = (W["wk"] @ h)',
    ),
    "wo_transposed": ('x = x + W["wo"] @ o', 'x = x + W["wo"].T @ o'),
    "argmax_ties_to_last": (
        "return np.argmax(l32, axis=-1).astype(np.int32)",
        "return (l32.shape[-1] - 1 - np.argmax(l32[..., ::-1], axis=-1)).astype(np.int32)",
    ),
    "bf16_truncates": ("rounded = ((bits + 0x7FFF + keep_odd) >> 16) << 16", "rounded = (bits >> 16) << 16"),
    "bf16_ties_away": ("rounded = ((bits + 0x7FFF + keep_odd) >> 16) << 16", "rounded = ((bits + 0x8000) >> 16) << 16"),
    "kv_not_rounded_to_cache_type": ('if dtype == "bf16":\n        f32 = round_f32_to_bf16(f32)', "if False:\n        pass"),
    "softmax_no_max_shift": ("e = np.exp(s - m)", "e = np.exp(s)"),
    "rope_position_off_by_one": ("angle = np.float64(position) * theta", "angle = np.float64(position + 1) * theta"),
    # multi-session steps: every session must use its own angles, residual stream and cache rows
    "sessions_share_first_rope": ("cos, sin = rope[i]", "cos, sin = rope[0]"),
    "sessions_share_one_x": ("x = xs[i]", "x = xs[0]"),
    "k_cache_indexed_by_call_slot": (
        "self.k_cache[session, l, :, position] = self._store(k)",
        "self.k_cache[i, l, :, position] = self._store(k)",
    ),
    "v_cache_read_by_call_slot": (
        "vc = self.v_cache[session, l, :, : position + 1]",
        "vc = self.v_cache[i, l, :, : position + 1]",
    ),
    # fp8 weights: exponent bias, subnormals, the sign, and which axis the scales run along
    "fp8_bias_8": ("np.exp2((e - 7).astype(np.float64))", "np.exp2((e - 8).astype(np.float64))"),
    "fp8_subnormals_as_normals": ("np.where(e == 0, f / 8.0 * 2.0**-6,", "np.where(e < 0, f / 8.0 * 2.0**-6,"),
    "fp8_sign_ignored": ("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = np.where(c & 0x00, -1.0, 1.0)"),
    "fp8_scale_per_column": (
        "_E4M3_VALUES[np.asarray(w.codes, np.uint8)] * np.asarray(w.scale, np.float32).astype(np.float64)[:, None]",
        "_E4M3_VALUES[np.asarray(w.codes, np.uint8)] * "
        "np.resize(np.asarray(w.scale, np.float32).astype(np.float64), w.codes.shape[1])[None, :]",
    ),
    # int8 weights: the codes' sign, and which axis the scales run along
    "int8_read_unsigned": (
        "np.asarray(w.codes, np.int8).astype(np.float64)",
        "np.asarray(w.codes, np.int8).view(np.uint8).astype(np.float64)",
    ),
    "int8_scale_per_column": (
        "np.asarray(w.codes, np.int8).astype(np.float64) * np.asarray(w.scale, np.float32).astype(np.float64)[:, None]",
        "np.asarray(w.codes, np.int8).astype(np.float64) * "
        "np.resize(np.asarray(w.scale, np.float32).astype(np.float64), w.codes.shape[1])[None, :]",
    ),
}

# cheapest pins first: a mutant stops at its first failing pin
PIN_ORDER = [
    oracle_pins.pin_softmax,
    oracle_pins.pin_rope,
    oracle_pins.pin_attention,
    oracle_pins.pin_gqa,
    oracle_pins.pin_rmsnorm,
    oracle_pins.pin_argmax,
    oracle_pins.pin_identity_layers,
    oracle_pins.pin_brute_force,
    oracle_pins.pin_brute_force_prefilled,
    oracle_pins.pin_incremental_equals_full,
    oracle_pins.pin_silu,
    oracle_pins.pin_sessions_independent,
    oracle_pins.pin_fp8,
    oracle_pins.pin_int8,
    lambda mod: oracle_pins.pin_bf16(mod, n_random=1 << 14),
]


def _load_mutant(name: str) -> types.ModuleType:
    src = open(SRC_PATH, encoding="utf-8").read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutant {name}: pattern must occur exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(name)
    for pin in PIN_ORDER:
        try:
            with __import__("warnings").catch_warnings():
                __import__("warnings").simplefilter("ignore")
                pin(mod)
        except Exception:
            return
    pytest.fail(f"no pin caught mutant {name}")

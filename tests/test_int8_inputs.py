"""The int8 input generator: per-row absmax quantisation of the seeded bf16 weights to int8.

The codes and scales are inputs: both the HIP library and the oracle receive them unchanged.
These checks hold the generator to its definition: codes within -127..127, every dequantised
weight within half a code step (half the row's scale) of the weight it stands for, each row's
largest magnitude at code +-127, halves rounded to the even code, and the int8 workloads keep
the bf16 workloads' other tensors.
"""

import numpy as np

import workloads
from workloads import ModelShape


def test_quantised_rows_within_half_step():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((64, 512)) * rng.uniform(0.001, 1.0, (64, 1))).astype(np.float32)
    w[5] = 0.0  # an all-zero row keeps a finite scale and zero codes
    q = workloads.quantize_rows_int8(w)
    assert q.codes.dtype == np.int8 and q.scale.dtype == np.float32
    c = q.codes.astype(np.int64)
    assert np.all(np.abs(c) <= 127)
    s = q.scale.astype(np.float64)[:, None]
    # w / scale is rounded in float32 first: allow one float32 ulp of it beyond the half step
    assert np.all(np.abs(c * s - w.astype(np.float64)) <= s * (0.5 + 2.0**-16))
    nz = np.max(np.abs(w), axis=1) > 0
    assert np.all(np.max(np.abs(c[nz]), axis=1) == 127)
    assert np.all(q.codes[5] == 0) and q.scale[5] == 1.0


def test_halves_round_to_even():
    # scale 1 (the row's largest magnitude is 127), so the codes are the values rounded
    w = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.49, -126.5]], np.float32)
    q = workloads.quantize_rows_int8(w)
    assert q.scale[0] == 1.0
    assert q.codes[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 3, -126]


def test_int8_workload_quantises_the_bf16_model():
    shape = ModelShape(2, 64, 4, 2, 16, 96, 50, weight_dtype="int8", kv_dtype="bf16")
    w8 = workloads.make_weights(shape, seed=3, workers=1)
    wb = workloads.make_weights(ModelShape(2, 64, 4, 2, 16, 96, 50), seed=3, workers=1)
    assert w8["dtype"] == "int8"
    assert np.array_equal(w8["embed"], wb["embed"])
    assert np.array_equal(w8["final_norm"], wb["final_norm"])
    for l8, lb in zip(w8["layers"], wb["layers"]):
        assert np.array_equal(l8["attn_norm"], lb["attn_norm"]) and np.array_equal(l8["ffn_norm"], lb["ffn_norm"])
        for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            q = l8[name]
            assert isinstance(q, workloads.Int8Matrix) and q.shape == lb[name].shape
            ref = workloads.quantize_rows_int8(workloads.f32_from_bf16_bits(lb[name]))
            assert np.array_equal(q.codes, ref.codes) and np.array_equal(q.scale, ref.scale)
    assert isinstance(w8["lm_head"], workloads.Int8Matrix)


def test_int8_step_bytes_match_fp8():
    """An int8 step reads what an fp8 step reads: one byte per matrix element, four per row."""
    from bandwidth_bound_transformer_amd import roofline

    m8 = workloads.get("8b_int8").model
    mf = workloads.get("8b_fp8").model
    assert m8.quantised and m8.weight_bytes == 1 and m8.embed_bytes == 2
    assert m8.streamed_weight_bytes() == mf.streamed_weight_bytes()
    assert roofline.step_bytes(m8, 1, 1100) == roofline.step_bytes(mf, 1, 1100)

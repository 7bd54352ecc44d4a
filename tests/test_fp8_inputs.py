"""The fp8 input generator: per-row E4M3 quantisation of the seeded bf16 weights.

The quantised codes and scales are inputs: both the HIP library and the oracle receive them
unchanged. These checks hold the generator to the E4M3 grid: every dequantised weight lies
within half a step of that grid of the weight it stands for, the largest magnitude of each row
maps to 448 exactly, and the fp8 workloads keep the bf16 workloads' other tensors.
"""

import numpy as np
import torch

import workloads
from workloads import ModelShape


def _e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_quantised_rows_within_half_step():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 512)) * rng.uniform(0.001, 1.0, (64, 1))).astype(np.float32)
    w[3] = 0.0  # an all-zero row keeps a finite scale and zero codes
    q = workloads.quantize_rows_e4m3(w)
    assert q.codes.dtype == np.uint8 and q.scale.dtype == np.float32
    v = _e4m3(q.codes)  # values on the E4M3 grid, before the row scale
    assert np.all(np.isfinite(v)) and np.max(np.abs(v)) <= 448.0
    x = w.astype(np.float64) / q.scale.astype(np.float64)[:, None]
    # half a step of the grid at x: normals (|x| >= 2**-6) have steps of 2**(floor(log2|x|) - 3),
    # subnormals 2**-9
    ex = np.floor(np.log2(np.maximum(np.abs(x), 2.0**-6)))
    half = 2.0 ** (ex - 4)
    assert np.all(np.abs(v - x) <= half * (1 + 1e-12))
    nz = np.max(np.abs(w), axis=1) > 0
    assert np.all(np.max(np.abs(v[nz]), axis=1) == 448.0)
    assert np.all(q.codes[3] == 0) and q.scale[3] == 1.0


def test_fp8_workload_quantises_the_bf16_model():
    shape = ModelShape(2, 64, 4, 2, 16, 96, 50, weight_dtype="fp8", kv_dtype="bf16")
    w8 = workloads.make_weights(shape, seed=3, workers=1)
    wb = workloads.make_weights(ModelShape(2, 64, 4, 2, 16, 96, 50), seed=3, workers=1)
    assert w8["dtype"] == "fp8"
    assert np.array_equal(w8["embed"], wb["embed"])
    assert np.array_equal(w8["final_norm"], wb["final_norm"])
    for l8, lb in zip(w8["layers"], wb["layers"]):
        assert np.array_equal(l8["attn_norm"], lb["attn_norm"]) and np.array_equal(l8["ffn_norm"], lb["ffn_norm"])
        for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            q = l8[name]
            assert isinstance(q, workloads.Fp8Matrix) and q.shape == lb[name].shape
            ref = workloads.quantize_rows_e4m3(workloads.f32_from_bf16_bits(lb[name]))
            assert np.array_equal(q.codes, ref.codes) and np.array_equal(q.scale, ref.scale)
    assert isinstance(w8["lm_head"], workloads.Fp8Matrix)


def test_fp8_step_bytes():
    """An fp8 step reads one byte per matrix element plus four per matrix row, and bf16 gains."""
    from bandwidth_bound_transformer_amd import roofline

    m = workloads.get("8b_fp8").model
    mb = workloads.get("8b").model
    d, L, V = m.d_model, m.n_layers, m.vocab
    matrix_elems = L * (m.q_dim * d + 2 * m.kv_dim * d + d * m.q_dim + 3 * m.ffn_dim * d) + V * d
    rows = L * (m.q_dim + 2 * m.kv_dim + d + 2 * m.ffn_dim + d) + V
    assert m.streamed_weight_bytes() == matrix_elems + 4 * rows + 2 * (2 * L + 1) * d
    b8 = roofline.step_bytes(m, 1, 1100)
    bb = roofline.step_bytes(mb, 1, 1100)
    assert b8.kv_read == bb.kv_read and b8.embedding == bb.embedding
    assert 0.49 < b8.weights / bb.weights < 0.51

"""Roofline accounting: the pages' table, and the byte counts of the workloads."""

import json
import os

import pytest

import workloads
from bandwidth_bound_transformer_amd import roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_roofline_table.json")


def test_reproduces_page_roofline_table():
    page = json.load(open(GOLDEN))
    bytes_per_token = page["model_params"] * page["bytes_per_param"]
    for row in page["rows"]:
        bound = roofline.tokens_per_s_bound(row["aggregate_bandwidth_TBps"] * 1e12, bytes_per_token)
        # the page prints bounds rounded to the nearest hundred
        assert abs(bound - row["printed_bound_tok_s"]) <= 50, (row, bound)
        assert row["printed_achieved_tok_s"] < bound


def test_streamed_parameter_counts():
    # Llama-3-8B shape: 8,030,261,248 parameters in total
    assert workloads.get("8b").model.total_params() == 8_030_261_248
    assert roofline.streamed_params(workloads.get("2b").model) == 1_646_897_152
    assert roofline.streamed_params(workloads.get("8b").model) == 7_504_924_672


@pytest.mark.parametrize(
    "name,mean_mb,bound_tok_s",
    [("2b", 3334.9, 2399), ("8b", 15161.6, 527.7), ("2b_long", 5042.2, 1587)],
)
def test_workload_bytes(name, mean_mb, bound_tok_s):
    wl = workloads.get(name)
    b = roofline.mean_step_bytes(wl)
    assert abs(b / 1e6 - mean_mb) < 0.2
    assert abs(roofline.tokens_per_s_bound(roofline.MI355X_HBM_BYTES_PER_S, b, wl.batch) - bound_tok_s) / bound_tok_s < 1e-3


def test_decode_positions():
    assert roofline.decode_positions(workloads.get("2b")) == range(512, 1023)
    assert roofline.decode_positions(workloads.get("2b_long")) == range(32768, 32896)
    assert roofline.decode_positions(workloads.get("11b_x56")) == range(4096, 4296)


def test_prefill_flops_counts_each_product_once():
    """prefill_flops against a count made position by position for a small shape: the seven
    matrices of every layer times each position, q.k and p.v over 0..p for each q head, and the LM
    head once."""
    from bandwidth_bound_transformer_amd import roofline
    from workloads import ModelShape

    m = ModelShape(3, 64, 4, 2, 16, 96, 50)
    P = 7
    count = 0
    for p in range(P):
        for _ in range(m.n_layers):
            count += 2 * (m.q_dim * m.d_model + 2 * m.kv_dim * m.d_model + m.d_model * m.q_dim + 3 * m.ffn_dim * m.d_model)
            count += m.n_q_heads * (p + 1) * m.head_dim * 2 * 2  # scores and weighted sums
    count += 2 * m.vocab * m.d_model
    assert roofline.prefill_flops(m, P) == count

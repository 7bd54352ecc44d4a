"""Seeded input generators: determinism, shapes and storage formats."""

import numpy as np
import torch

import workloads
from workloads import ModelShape, Workload


def test_presets_shapes():
    tiny = workloads.get("tiny")
    assert (tiny.model.n_layers, tiny.model.d_model, tiny.model.vocab) == (2, 256, 1024)
    assert tiny.model.weight_dtype == "f32" and tiny.max_seq == 96
    m8 = workloads.get("8b").model
    assert (m8.q_dim, m8.kv_dim, m8.group, m8.rope_base) == (4096, 1024, 4, 500000.0)
    assert workloads.get("11b_x56").batch == 56
    assert workloads.get("2b").decode_steps == 511 and workloads.get("2b_long").decode_steps == 128


def test_weights_deterministic_and_shaped():
    shape = ModelShape(2, 64, 4, 2, 16, 96, 77)
    a = workloads.make_weights(shape, seed=5, workers=2)
    b = workloads.make_weights(shape, seed=5, workers=1)
    c = workloads.make_weights(shape, seed=6, workers=1)
    assert a["embed"].dtype == np.uint16 and a["embed"].shape == (77, 64)
    assert a["layers"][1]["w_down"].shape == (64, 96)
    for x, y in [(a["embed"], b["embed"]), (a["lm_head"], b["lm_head"]), (a["layers"][1]["wq"], b["layers"][1]["wq"])]:
        assert np.array_equal(x, y)
    assert not np.array_equal(a["lm_head"], c["lm_head"])
    assert np.all(workloads.f32_from_bf16_bits(a["layers"][0]["attn_norm"]) == 1.0)
    vals = workloads.f32_from_bf16_bits(a["layers"][0]["w_gate"])
    assert abs(vals.std() - 0.02) < 0.002 and abs(vals.mean()) < 0.002


def test_chunking_is_part_of_the_recipe():
    # a tensor larger than one chunk is made of independently seeded row runs
    shape = ModelShape(1, 4096, 32, 8, 128, 64, 2048)
    w = workloads.make_weights(shape, seed=0, workers=4)
    rows_per_chunk = (1 << 22) // 4096
    first = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, 0, 0]))).standard_normal((rows_per_chunk, 4096), dtype=np.float32) * np.float32(0.02)
    assert np.array_equal(w["embed"][:rows_per_chunk], workloads.bf16_bits_from_f32(first))


def test_generator_bf16_matches_torch():
    x = np.random.default_rng(0).standard_normal(1 << 16).astype(np.float32) * 0.02
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.bf16_bits_from_f32(x), ref)


def test_prompts_and_first_tokens():
    wl = workloads.get("2b")
    p = workloads.make_prompt(wl, 0)
    assert p.shape == (512,) and p.dtype == np.int32 and p.min() >= 0 and p.max() < 32000
    assert np.array_equal(p, workloads.make_prompt(wl, 0))
    assert not np.array_equal(p, workloads.make_prompt(wl, 1))
    ft = workloads.make_first_tokens(workloads.get("11b_x56"))
    assert ft.shape == (56,) and len(set(ft.tolist())) > 40


def test_kv_prefill_layout():
    wl = Workload("t", ModelShape(2, 32, 4, 2, 8, 40, 50), batch=3, prefill_len=6, gen_tokens=2)
    out = np.zeros((2, 2, 3, 2, wl.max_seq, 8), np.uint16)
    workloads.fill_kv_prefill(wl, out, sessions=[0, 2], workers=2)
    assert np.array_equal(out[1, 0, 2, 1, :6], workloads.kv_prefill_block(wl, 1, 0, 2, 1))
    assert np.all(out[:, :, 1] == 0) and np.all(out[..., 6:, :] == 0)
    v = workloads.f32_from_bf16_bits(workloads.kv_prefill_block(wl, 0, 1, 0, 0))
    assert v.shape == (6, 8)

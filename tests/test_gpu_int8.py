"""Parity of the batch-1 step with int8 weights (through the C ABI) with the CPU oracle.

The projection matrices and the LM head are int8 codes with one float32 scale per row; the
embedding, gains and cache are bf16 ("17k tokens/sec" page, best practice 2, which names INT8).
Both sides receive the same codes and scales: the oracle computes with code times row scale in
float64, the kernel converts each code to float exactly, accumulates in float32 and scales each
row's total. The tolerance is the bf16 one, 2e-2 of the largest reference logit, and every greedy
token must match except at a tie-flip (see gpu_harness.compare_sequence).
"""

import dataclasses

import numpy as np
import pytest

import workloads
from oracle import decoder as ref
from workloads import ModelShape

from . import gpu_harness as gh
from .test_gpu_parity import _check_steps_from_cache, _oracle_from_gpu_cache

pytestmark = pytest.mark.gpu

TOL = 2e-2
# two layers at the smallest dimensions the one-byte kernel takes: d_model and q_dim 1024 (one
# packet per row), G = 4, ffn 2048 (one 8-column unit per workgroup), vocab 4096
SMALL_INT8 = ModelShape(2, 1024, 8, 2, 128, 2048, 4096, rope_base=10000.0, weight_dtype="int8", kv_dtype="bf16")
MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


@pytest.fixture(scope="module")
def torch():
    import torch as t

    assert t.cuda.is_available()
    return t


@pytest.fixture(scope="module")
def kdm():
    from bandwidth_bound_transformer_amd import kd

    kd.library()
    return kd


def _every_code_weights(seed: int) -> dict:
    """The small model with codes drawn uniformly from all of -128..127 (so -128, which the
    quantiser never writes, and every byte position of every 32-bit word occur) and per-row
    scales around 0.02 / 74, which keeps the weights' spread near the bf16 model's."""
    w = workloads.make_weights(SMALL_INT8, seed=seed)
    rng = np.random.default_rng(seed + 100)

    def codes(shape):
        return workloads.Int8Matrix(rng.integers(-128, 128, size=shape).astype(np.int8),
                                    (rng.uniform(0.5, 1.5, shape[0]) * (0.02 / 74.0)).astype(np.float32))

    for lw in w["layers"]:
        for name in MATRICES:
            lw[name] = codes(lw[name].shape)
    w["lm_head"] = codes(w["lm_head"].shape)
    return w


def _run_and_compare(torch, kdm, shape, w, prompt, n_gen, max_seq, tag):
    dec = kdm.Decoder(shape, w, max_seq=max_seq)
    toks, logits = gh.run_prompt(dec, prompt, n_gen, torch)
    assert dec.status() == 0
    print(f"{tag}: GPU run done; oracle ...", flush=True)
    seq = list(prompt) + [int(t) for t in toks[len(prompt) - 1 : -1]]
    want = ref.forward_full(shape, w, seq)
    worst, flips, defects = gh.compare_sequence(toks, logits, want, TOL)
    print(f"{tag}: max rel logit err {worst:.3e} over {len(seq)} steps, tie-flips {flips}")
    assert worst <= TOL
    assert not defects and flips <= 2
    return dec


def test_int8_small_model_every_code(torch, kdm):
    """The small int8 model with every code value over its whole run: 24-token prompt, 40
    greedy tokens."""
    w = _every_code_weights(9)
    prompt = np.random.default_rng(10).integers(0, SMALL_INT8.vocab, 24).astype(np.int32)
    dec = _run_and_compare(torch, kdm, SMALL_INT8, w, prompt, 40, 64, "int8 small")
    dec.close()


def test_2b_int8_generation(torch, kdm):
    """2B decoder with int8 weights (the quantised bf16 model) at its real shape: a 256-token
    prompt and 64 greedy tokens, every step against the oracle's full-sequence recomputation on
    the GPU's tokens."""
    wl = workloads.get("2b_int8")
    w = workloads.make_weights(wl.model, seed=wl.weight_seed)
    print("2b_int8: weights ready", flush=True)
    prompt = workloads.make_prompt(wl, 0)[:256]
    dec = _run_and_compare(torch, kdm, wl.model, w, prompt, 64, wl.max_seq, "2b_int8")
    dec.close()


def test_8b_int8_sampled_steps(torch, kdm):
    """Llama-3-8B shape with int8 weights at the benchmark's positions: the 1024-token prompt and
    the decode run on the GPU; positions 1023-1024 and the last two, 1277-1278, against the oracle
    started from the GPU's cache."""
    wl = workloads.get("8b_int8")
    m = wl.model
    w = workloads.make_weights(m, seed=wl.weight_seed)
    print("8b_int8: weights ready", flush=True)
    dec = kdm.Decoder(m, w, max_seq=wl.max_seq)
    prompt = workloads.make_prompt(wl, 0)
    P = len(prompt)
    prompt_d = torch.as_tensor(np.asarray(prompt, np.int32), device=dec.device)
    dec.positions.zero_()
    for p in range(P - 1):
        dec.tokens.copy_(prompt_d[p : p + 1])
        dec.step(write_logits=False)
    torch.cuda.synchronize()
    assert dec.status() == 0 and int(dec.positions.item()) == P - 1
    o = _oracle_from_gpu_cache(m, w, dec, P - 1, P + 2)
    dec.tokens.fill_(int(prompt[P - 1]))
    _check_steps_from_cache(dec, o, int(prompt[P - 1]), P - 1, 2, "8b_int8")
    del o
    last = wl.max_seq - 2
    while int(dec.positions.item()) < last:
        dec.step(write_logits=False)
    torch.cuda.synchronize()
    assert dec.status() == 0 and int(dec.positions.item()) == last
    o = _oracle_from_gpu_cache(m, w, dec, last, wl.max_seq)
    _check_steps_from_cache(dec, o, int(dec.tokens.item()), last, 2, "8b_int8 last")
    dec.close()


def test_int8_rejects_unsupported_configs(kdm):
    """int8 weights need a bf16 cache: at batch 1, in lockstep sessions and for a prefill engine."""
    w = workloads.make_weights(SMALL_INT8, seed=9)
    f32_cache = dataclasses.replace(SMALL_INT8, kv_dtype="f32")
    for shape, batch, chunk in ((f32_cache, 1, 0), (f32_cache, 4, 0), (f32_cache, 1, 64)):
        cfg = kdm.make_config(shape, batch, 64, prefill_chunk=chunk)
        with pytest.raises(kdm.KDError) as e:
            kdm.kd_init(cfg, w)
        assert e.value.code == kdm.KD_ERR_UNSUPPORTED

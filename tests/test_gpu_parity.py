"""Parity of the HIP decode step (through the C ABI) with the CPU oracle, on an MI355X.

Every input is seeded and synthetic (``workloads``); every expected value comes from
``oracle``. Tolerance: the largest logit error over the largest reference logit must stay
within 2e-2 for bf16 weights with fp32 arithmetic. The greedy token of every step must equal
the oracle's argmax (in float32), except at an exact tie-flip (see gpu_harness.compare_sequence).
The fp32 tiny decoder is held to a much tighter bound, 1e-4, because there the only error
sources are fp32 rounding and the hardware exp and sqrt.
"""

import numpy as np
import pytest

import workloads
from oracle import decoder as ref

from . import gpu_harness as gh

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-4


@pytest.fixture(scope="module")
def torch():
    import torch as t

    assert t.cuda.is_available()
    return t


@pytest.fixture(scope="module")
def kdm():
    from bandwidth_bound_transformer_amd import kd

    kd.library()  # fails loudly if the HIP library is missing
    return kd


@pytest.fixture(scope="module")
def tiny():
    wl = workloads.get("tiny")
    return wl, workloads.make_weights(wl.model, seed=wl.weight_seed)


def _decoder(kdm, wl, w, max_seq=None):
    return kdm.Decoder(wl.model, w, max_seq=max_seq or wl.max_seq)


def test_tiny_generation_and_cache(torch, kdm, tiny):
    """The tiny workload end to end: 32-token prompt, 64 greedy tokens, KV cache contents."""
    wl, w = tiny
    dec = _decoder(kdm, wl, w)
    prompt = workloads.make_prompt(wl, 0)
    toks, logits = gh.run_prompt(dec, prompt, wl.gen_tokens, torch)
    assert dec.status() == 0
    o = ref.Oracle(wl.model, w, batch=1, max_seq=wl.max_seq)
    feed = list(prompt) + [int(t) for t in toks[len(prompt) - 1 : -1]]
    want = np.stack([o.step_one(0, int(t), p) for p, t in enumerate(feed)])
    worst, flips, defects = gh.compare_sequence(toks, logits, want, F32_TOL)
    print(f"tiny: max rel logit err {worst:.3e}, tie-flips {flips}")
    assert worst <= F32_TOL
    assert not defects and flips == 0
    # the cache holds K (after RoPE) and V of every fed position, as the oracle stored them
    kv = dec.kv_view().float().cpu().numpy()
    n = len(feed)
    k_err = np.max(np.abs(kv[:, 0, 0, :, :n] - o.k_cache[0][:, :, :n]))
    v_err = np.max(np.abs(kv[:, 1, 0, :, :n] - o.v_cache[0][:, :, :n]))
    assert k_err < 1e-4 * max(1.0, np.max(np.abs(o.k_cache))) and v_err < 1e-4 * max(1.0, np.max(np.abs(o.v_cache)))
    # positions advanced once per step
    assert int(dec.positions.item()) == n
    dec.close()


def test_tiny_first_position_and_null_logits(torch, kdm, tiny):
    """Position 0 (a single cached key) and a step that skips the logits write give the same token."""
    wl, w = tiny
    dec = _decoder(kdm, wl, w)
    dec.tokens.fill_(7)
    dec.positions.zero_()
    dec.step(write_logits=True)
    t_with = int(dec.tokens.item())
    l0 = dec.logits[0].cpu().numpy()
    want = ref.Oracle(wl.model, w, 1, wl.max_seq).step_one(0, 7, 0)
    assert gh.inf_rel_err(l0, want) <= F32_TOL
    dec.kv.zero_()
    dec.tokens.fill_(7)
    dec.positions.zero_()
    dec.logits.fill_(123.0)
    dec.step(write_logits=False)
    torch.cuda.synchronize()
    assert int(dec.tokens.item()) == t_with
    assert bool(torch.all(dec.logits == 123.0))
    dec.close()


def test_tiny_bitwise_deterministic(torch, kdm, tiny):
    """Two runs of the same inputs give identical bits (fixed reduction orders, no float atomics)."""
    wl, w = tiny
    runs = []
    for _ in range(2):
        dec = _decoder(kdm, wl, w)
        toks, logits = gh.run_prompt(dec, workloads.make_prompt(wl, 0)[:8], 24, torch)
        runs.append((toks, logits, dec.kv_view().float().cpu().numpy()))
        dec.close()
    assert np.array_equal(runs[0][0], runs[1][0])
    assert np.array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))
    assert np.array_equal(runs[0][2], runs[1][2])


def test_input_errors_set_status_and_write_nothing(torch, kdm, tiny):
    wl, w = tiny
    dec = _decoder(kdm, wl, w)
    for token, pos, bit in ((wl.model.vocab, 0, kdm.KD_STATUS_TOKEN_RANGE), (-1, 0, kdm.KD_STATUS_TOKEN_RANGE),
                            (5, wl.max_seq, kdm.KD_STATUS_POS_OVERFLOW), (5, -3, kdm.KD_STATUS_POS_OVERFLOW)):
        dec.tokens.fill_(token)
        dec.positions.fill_(pos)
        dec.logits.fill_(-7.0)
        before = dec.kv.clone()
        dec.step()
        assert dec.status(clear=True) == bit
        assert int(dec.tokens.item()) == token and int(dec.positions.item()) == pos
        assert bool(torch.all(dec.logits == -7.0)) and bool(torch.equal(before, dec.kv))
    # the handle keeps working afterwards
    dec.tokens.fill_(3)
    dec.positions.zero_()
    dec.step()
    assert dec.status() == 0
    dec.close()


def test_2b_prompt512_generation(torch, kdm):
    """2B-class decoder at its real shape and full extent: the 512-token prompt, then all 512
    greedy tokens; every step's logits and token against the oracle's full-sequence recomputation
    on the GPU's token sequence (teacher-forced), tie-flips counted."""
    wl = workloads.get("2b")
    w = workloads.make_weights(wl.model, seed=wl.weight_seed)
    print("2b: weights ready", flush=True)
    dec = _decoder(kdm, wl, w)
    prompt = workloads.make_prompt(wl, 0)
    n_gen = wl.gen_tokens
    toks, logits = gh.run_prompt(dec, prompt, n_gen, torch)
    assert dec.status() == 0
    print("2b: GPU run done; oracle ...", flush=True)
    seq = list(prompt) + [int(t) for t in toks[len(prompt) - 1 : -1]]
    want = ref.forward_full(wl.model, w, seq)
    worst, flips, defects = gh.compare_sequence(toks, logits, want, BF16_TOL)
    print(f"2b: max rel logit err {worst:.3e} over {len(seq)} steps, tie-flips {flips}")
    assert worst <= BF16_TOL
    assert not defects and flips <= 2
    assert int(dec.positions.item()) == wl.prompt_len + wl.gen_tokens - 1
    dec.close()


def test_8b_short_prompt(torch, kdm):
    """Llama-3-8B shape at its real dimensions and launch configuration, 48-token prompt + 6 tokens."""
    wl = workloads.get("8b")
    w = workloads.make_weights(wl.model, seed=wl.weight_seed)
    print("8b: weights ready", flush=True)
    dec = _decoder(kdm, wl, w)
    prompt = workloads.make_prompt(wl, 0)[:48]
    toks, logits = gh.run_prompt(dec, prompt, 6, torch)
    assert dec.status() == 0
    print("8b: GPU run done; oracle ...", flush=True)
    seq = list(prompt) + [int(t) for t in toks[len(prompt) - 1 : -1]]
    want = ref.forward_full(wl.model, w, seq)
    worst, flips, defects = gh.compare_sequence(toks, logits, want, BF16_TOL)
    print(f"8b: max rel logit err {worst:.3e} over {len(seq)} steps, tie-flips {flips}")
    assert worst <= BF16_TOL
    assert not defects
    dec.close()


def _oracle_from_gpu_cache(m, w, dec, n, max_seq):
    """An oracle whose cache holds the GPU's cache contents at positions 0..n-1."""
    o = ref.Oracle(m, w, batch=1, max_seq=max_seq)
    kv = dec.kv_view()
    for l in range(m.n_layers):
        c = kv[l, :, 0, :, :n].float().cpu().numpy()  # [K/V][kv head][position][dim]
        for g in range(m.n_kv_heads):
            o.load_kv(0, l, g, c[0, g], c[1, g])
    return o


def _check_steps_from_cache(dec, o, tok, first_pos, n, tag):
    """Step GPU and oracle n times from the same cache and token; logits, token, appended K/V."""
    for i in range(n):
        dec.step()
        gl = dec.logits[0].cpu().numpy()
        want = o.step_one(0, tok, first_pos + i)
        err = gh.inf_rel_err(gl, want)
        print(f"{tag}: position {first_pos + i}: rel logit err {err:.3e}", flush=True)
        assert err <= BF16_TOL
        g_tok = int(dec.tokens.item())
        if g_tok != int(ref.greedy_token(want[None])[0]):
            assert gh.top2_margin(want) <= 2 * np.max(np.abs(gl - want))
        tok = g_tok
    assert dec.status() == 0
    return tok


def test_8b_full_prompt_sampled_steps(torch, kdm):
    """Llama-3-8B shape at the benchmark's positions and full extent: the 1024-token prompt and all
    255 decode steps run on the GPU. The steps at positions 1023 and 1024 (the first of the decode)
    and at 1277 and 1278 (its last two) are checked against the oracle, which starts from the GPU's
    cache before each pair (sampled outputs at full size; the prompt path itself is checked from
    position 0 by the 2B and short 8B tests). The K/V appended at those positions must match what
    the oracle stored."""
    wl = workloads.get("8b")
    m = wl.model
    w = workloads.make_weights(m, seed=wl.weight_seed)
    print("8b full: weights ready", flush=True)
    dec = _decoder(kdm, wl, w)
    prompt = workloads.make_prompt(wl, 0)
    P = len(prompt)
    prompt_d = torch.as_tensor(np.asarray(prompt, np.int32), device=dec.device)
    dec.positions.zero_()
    for p in range(P - 1):
        dec.tokens.copy_(prompt_d[p : p + 1])
        dec.step()
    torch.cuda.synchronize()
    assert dec.status() == 0 and int(dec.positions.item()) == P - 1
    print(f"8b full: GPU prompt 0..{P - 2} done", flush=True)
    o = _oracle_from_gpu_cache(m, w, dec, P - 1, P + 2)
    dec.tokens.fill_(int(prompt[P - 1]))
    tok = _check_steps_from_cache(dec, o, int(prompt[P - 1]), P - 1, 2, "8b full")
    kv = dec.kv_view()
    for l in (0, m.n_layers - 1):
        got = kv[l, :, 0, :, P - 1 : P + 1].float().cpu().numpy()
        for s, ref_cache in ((0, o.k_cache), (1, o.v_cache)):
            exp = ref_cache[0, l, :, P - 1 : P + 1]
            assert np.max(np.abs(got[s] - exp)) <= 2e-2 * np.max(np.abs(exp))
    del o
    # the rest of the decode on the GPU, up to the last two positions
    last = wl.max_seq - 2  # 1277: the decode's steps run at positions 1023 .. 1278
    while int(dec.positions.item()) < last:
        dec.step(write_logits=False)
    torch.cuda.synchronize()
    assert dec.status() == 0 and int(dec.positions.item()) == last
    tok = int(dec.tokens.item())
    print(f"8b full: GPU decode to position {last - 1} done", flush=True)
    o = _oracle_from_gpu_cache(m, w, dec, last, wl.max_seq)
    _check_steps_from_cache(dec, o, tok, last, 2, "8b full")
    assert int(dec.positions.item()) == wl.max_seq
    dec.close()


def test_2b_long_context_prefilled(torch, kdm):
    """2B decoder with the KV cache pre-filled to 32768 positions, over the workload's full extent:
    the first two of its 128 steps from the seeded first token, then (after the GPU has run the
    rest) its last two, each pair against the oracle."""
    wl = workloads.get("2b_long")
    m = wl.model
    w = workloads.make_weights(m, seed=wl.weight_seed)
    dec = _decoder(kdm, wl, w)
    kv_host = np.zeros((m.n_layers, 2, 1, m.n_kv_heads, dec.s_alloc, m.head_dim), np.uint16)
    workloads.fill_kv_prefill(wl, kv_host)
    dec.kv.view(torch.int16).copy_(torch.from_numpy(kv_host.view(np.int16).reshape(-1)))
    o = ref.Oracle(m, w, batch=1, max_seq=wl.max_seq)
    for l in range(m.n_layers):
        for g in range(m.n_kv_heads):
            o.load_kv(0, l, g, workloads.f32_from_bf16_bits(kv_host[l, 0, 0, g, : wl.prefill_len]),
                      workloads.f32_from_bf16_bits(kv_host[l, 1, 0, g, : wl.prefill_len]))
    del kv_host
    print("2b_long: cache pre-filled on both sides", flush=True)
    first = int(workloads.make_first_tokens(wl)[0])
    dec.tokens.fill_(first)
    dec.positions.fill_(wl.prefill_len)
    tok = first
    for i in range(2):
        dec.step()
        gl = dec.logits[0].cpu().numpy()
        want = o.step_one(0, tok, wl.prefill_len + i)
        err = gh.inf_rel_err(gl, want)
        print(f"2b_long step {i}: rel logit err {err:.3e}", flush=True)
        assert err <= BF16_TOL
        g_tok = int(dec.tokens.item())
        if g_tok != int(ref.greedy_token(want[None])[0]):
            assert gh.top2_margin(want) <= 2 * np.max(np.abs(gl - want))
        tok = g_tok
    assert dec.status() == 0
    # the new positions were appended to the cache as the oracle stored them
    kv = dec.kv_view()
    for l in (0, m.n_layers - 1):
        got = kv[l, 0, 0, :, wl.prefill_len : wl.prefill_len + 2].float().cpu().numpy()
        assert np.max(np.abs(got - o.k_cache[0, l, :, wl.prefill_len : wl.prefill_len + 2])) <= 2e-2 * np.max(np.abs(got))
    del o
    # the rest of the workload's 128 steps on the GPU; its last two against the oracle started
    # from the GPU's cache (positions 0 .. 32893)
    last = wl.max_seq - 2
    while int(dec.positions.item()) < last:
        dec.step(write_logits=False)
    torch.cuda.synchronize()
    assert dec.status() == 0 and int(dec.positions.item()) == last
    print(f"2b_long: GPU at position {last}", flush=True)
    o = _oracle_from_gpu_cache(m, w, dec, last, wl.max_seq)
    _check_steps_from_cache(dec, o, int(dec.tokens.item()), last, 2, "2b_long last")
    assert int(dec.positions.item()) == wl.max_seq
    dec.close()

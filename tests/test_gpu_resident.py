"""Resident multi-step decoding (kd_generate) and the failure paths of a call, on an MI355X.

* kd_generate runs n greedy steps in one persistent launch (batch 1) or n ticks back to back
  (lockstep sessions); its tokens, logits and KV cache must equal, bit for bit, n kd_step calls
  from the same state, and the greedy sequence must match the oracle's.
* The cancel word and the wait limit force a call to give up from the host side: every
  workgroup leaves through the same exit as after a failed wait, the status bit is set, the
  outputs stay as the contract says, and the next call runs normally (the abort is scoped to
  the call that gave up).

Every input is seeded and synthetic (``workloads``); every expected value comes from the HIP
library's own kd_step (bitwise comparisons) or from ``oracle``.
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


def _feed_prompt(dec, prompt, torch):
    pd = torch.as_tensor(np.asarray(prompt, np.int32), device=dec.device)
    dec.positions.zero_()
    for p in range(len(prompt)):
        dec.tokens.copy_(pd[p : p + 1])
        dec.step(write_logits=False)
    torch.cuda.synchronize()


def _generate_vs_steps(torch, kdm, wl, w, prompt_len, n, tag):
    """Prompt by kd_step on two decoders, then n steps: kd_generate on one, kd_step on the other."""
    prompt = workloads.make_prompt(wl, 0)[:prompt_len]
    m = wl.model
    a = kdm.Decoder(m, w, max_seq=wl.max_seq)
    b = kdm.Decoder(m, w, max_seq=wl.max_seq)
    for dec in (a, b):
        _feed_prompt(dec, prompt, torch)
    out = torch.full((n,), -1, dtype=torch.int32, device=a.device)
    lg = torch.zeros(n, m.vocab, dtype=torch.float32, device=a.device)
    prog = torch.zeros(1, dtype=torch.int32, device=a.device)
    a.generate(n, out_tokens=out, logits=lg, progress=prog)
    steps_tok, steps_lg = [], []
    for _ in range(n):
        b.step()
        steps_tok.append(b.tokens.clone())
        steps_lg.append(b.logits[0].clone())
    torch.cuda.synchronize()
    assert a.status() == 0 and b.status() == 0
    assert int(prog.item()) == n
    gen_tok = out.cpu().numpy()
    ref_tok = torch.cat(steps_tok).cpu().numpy()
    print(f"{tag}: generate {n} steps, first tokens {gen_tok[:8].tolist()}", flush=True)
    assert np.array_equal(gen_tok, ref_tok)
    assert np.array_equal(lg.cpu().numpy().view(np.uint32), torch.stack(steps_lg).cpu().numpy().view(np.uint32))
    assert int(a.tokens.item()) == int(b.tokens.item()) and int(a.positions.item()) == prompt_len + n
    assert int(b.positions.item()) == prompt_len + n
    assert bool(torch.equal(a.kv, b.kv))
    a.close()
    b.close()
    return prompt, gen_tok, lg.cpu().numpy()


def test_generate_equals_steps_tiny(torch, kdm, tiny):
    """40 resident steps after an 8-token prompt: bitwise the same as 40 kd_step calls, and the
    greedy sequence the oracle produces from the same prompt."""
    wl, w = tiny
    prompt, toks, logits = _generate_vs_steps(torch, kdm, wl, w, 8, 40, "tiny")
    # the oracle after the same prompt: resident step i is fed the token chosen before it, at
    # position len(prompt) + i
    o = ref.Oracle(wl.model, w, batch=1, max_seq=wl.max_seq)
    for p, t in enumerate(prompt):
        last = o.step_one(0, int(t), p)
    tok = int(ref.greedy_token(last[None])[0])
    worst = 0.0
    for i in range(len(toks)):
        want_i = o.step_one(0, tok, len(prompt) + i)
        worst = max(worst, gh.inf_rel_err(logits[i], want_i))
        assert int(toks[i]) == int(ref.greedy_token(want_i[None])[0]), i
        tok = int(toks[i])
    print(f"tiny generate: max rel logit err {worst:.3e}")
    assert worst <= F32_TOL


def test_generate_equals_steps_2b(torch, kdm):
    """The 2B decoder at its real shape: 64 resident steps after a 128-token prompt, bitwise equal
    to 64 kd_step calls (the K/V each step appends is read back by later steps of the same
    launch on other compute units)."""
    wl = workloads.get("2b")
    w = workloads.make_weights(wl.model, seed=wl.weight_seed)
    print("2b generate: weights ready", flush=True)
    _generate_vs_steps(torch, kdm, wl, w, 128, 64, "2b")


@pytest.mark.parametrize("name", ["2b_fp8", "2b_int8"])
def test_generate_equals_steps_one_byte_weights(torch, kdm, name):
    """The resident loop of the one-byte kernels (E4M3 and int8 codes with row scales): 48 steps
    after a 128-token prompt, bitwise equal to 48 kd_step calls."""
    wl = workloads.get(name)
    w = workloads.make_weights(wl.model, seed=wl.weight_seed)
    print(f"{name} generate: weights ready", flush=True)
    _generate_vs_steps(torch, kdm, wl, w, 128, 48, name)


def test_generate_stops_at_cache_end(torch, kdm, tiny):
    """Asking for more steps than the cache holds runs the steps that fit, then stops with
    KD_STATUS_POS_OVERFLOW."""
    wl, w = tiny
    dec = kdm.Decoder(wl.model, w, max_seq=wl.max_seq)
    dec.tokens.fill_(5)
    dec.positions.fill_(wl.max_seq - 3)
    out = torch.full((8,), -1, dtype=torch.int32, device=dec.device)
    prog = torch.zeros(1, dtype=torch.int32, device=dec.device)
    dec.generate(8, out_tokens=out, progress=prog)
    assert dec.status(clear=True) == kdm.KD_STATUS_POS_OVERFLOW
    assert int(prog.item()) == 3 and int(dec.positions.item()) == wl.max_seq
    o = out.cpu().numpy()
    assert np.all(o[:3] >= 0) and np.all(o[3:] == -1)
    dec.close()


def test_generate_lockstep_equals_ticks(torch, kdm):
    """Lockstep sessions: kd_generate's n ticks equal n kd_step ticks bit for bit, with the
    per-tick tokens recorded [tick][session]."""
    from workloads.presets import ModelShape, Workload

    shape = ModelShape(2, 512, 4, 2, 128, 512, 1024, rope_base=500000.0)
    B, n = 17, 6
    wl = Workload("gen_b17", shape, batch=B, prefill_len=40, gen_tokens=n, weight_seed=31, kv_seed=32,
                  first_token_seed=33)
    w = workloads.make_weights(shape, seed=wl.weight_seed)
    decs = [kdm.Decoder(shape, w, max_seq=wl.max_seq, batch=B) for _ in range(2)]
    first = torch.from_numpy(workloads.make_first_tokens(wl))
    for dec in decs:
        dec.tokens.copy_(first)
        dec.positions.fill_(wl.prefill_len)
    out = torch.full((n, B), -1, dtype=torch.int32, device=decs[0].device)
    lg = torch.zeros(n, B, shape.vocab, dtype=torch.float32, device=decs[0].device)
    prog = torch.zeros(1, dtype=torch.int32, device=decs[0].device)
    decs[0].generate(n, out_tokens=out, logits=lg, progress=prog)
    toks, lgs = [], []
    for _ in range(n):
        decs[1].step()
        toks.append(decs[1].tokens.clone())
        lgs.append(decs[1].logits.clone())
    torch.cuda.synchronize()
    assert decs[0].status() == 0 and decs[1].status() == 0 and int(prog.item()) == n
    assert np.array_equal(out.cpu().numpy(), torch.stack(toks).cpu().numpy())
    assert np.array_equal(lg.cpu().numpy().view(np.uint32), torch.stack(lgs).cpu().numpy().view(np.uint32))
    assert bool(torch.equal(decs[0].kv, decs[1].kv))
    for dec in decs:
        dec.close()


def test_cancel_word_abandons_calls(torch, kdm, tiny):
    """With the cancel word set, kd_step and kd_generate leave at once through the drain path:
    KD_STATUS_CANCELLED, tokens, positions, logits and cache untouched, no progress. Cleared, the
    next step matches the oracle."""
    wl, w = tiny
    dec = kdm.Decoder(wl.model, w, max_seq=wl.max_seq)
    prompt = workloads.make_prompt(wl, 0)[:5]
    _feed_prompt(dec, prompt[:-1], torch)
    dec.tokens.fill_(int(prompt[-1]))
    dec.logits.fill_(-3.0)
    before = dec.kv.clone()
    dec.control(kdm.KD_CTRL_CANCEL, 1)
    dec.step()
    assert dec.status(clear=True) == kdm.KD_STATUS_CANCELLED
    prog = torch.zeros(1, dtype=torch.int32, device=dec.device)
    out = torch.full((4,), -1, dtype=torch.int32, device=dec.device)
    dec.generate(4, out_tokens=out, progress=prog)
    assert dec.status(clear=True) == kdm.KD_STATUS_CANCELLED
    assert int(prog.item()) == 0 and bool(torch.all(out == -1))
    assert int(dec.tokens.item()) == int(prompt[-1]) and int(dec.positions.item()) == len(prompt) - 1
    assert bool(torch.all(dec.logits == -3.0)) and bool(torch.equal(before, dec.kv))
    dec.control(kdm.KD_CTRL_CANCEL, 0)
    dec.step()
    assert dec.status() == 0
    o = ref.Oracle(wl.model, w, batch=1, max_seq=wl.max_seq)
    for p, t in enumerate(prompt):
        want = o.step_one(0, int(t), p)
    assert gh.inf_rel_err(dec.logits[0].cpu().numpy(), want) <= F32_TOL
    assert int(dec.tokens.item()) == int(ref.greedy_token(want[None])[0])
    dec.close()


def test_cancel_word_skips_lockstep_tick(torch, kdm):
    """The lockstep path honours the cancel word too: the tick writes nothing."""
    from workloads.presets import ModelShape

    shape = ModelShape(2, 512, 4, 2, 128, 512, 1024, rope_base=500000.0)
    w = workloads.make_weights(shape, seed=41)
    dec = kdm.Decoder(shape, w, max_seq=64, batch=3)
    dec.tokens.fill_(9)
    dec.positions.fill_(0)
    dec.logits.fill_(-3.0)
    dec.control(kdm.KD_CTRL_CANCEL, 1)
    dec.step()
    assert dec.status(clear=True) == kdm.KD_STATUS_CANCELLED
    assert bool(torch.all(dec.positions == 0)) and bool(torch.all(dec.logits == -3.0))
    dec.control(kdm.KD_CTRL_CANCEL, 0)
    dec.step()
    assert dec.status() == 0 and bool(torch.all(dec.positions == 1))
    dec.close()


@pytest.mark.parametrize("name", ["tiny", "2b"])
def test_wait_limit_gives_up_then_recovers(torch, kdm, name):
    """A wait limit of 0 makes the first wait that is not satisfied at once give up: the call ends
    with KD_STATUS_SYNC_TIMEOUT and writes no token or position. With the limit restored, the next
    call runs normally (the abort is scoped to the call that gave up) and matches the oracle."""
    wl = workloads.get(name)
    w = workloads.make_weights(wl.model, seed=wl.weight_seed)
    tol = F32_TOL if wl.model.weight_dtype == "f32" else BF16_TOL
    dec = kdm.Decoder(wl.model, w, max_seq=wl.max_seq)
    prompt = workloads.make_prompt(wl, 0)[:3]
    _feed_prompt(dec, prompt[:-1], torch)
    dec.tokens.fill_(int(prompt[-1]))
    dec.control(kdm.KD_CTRL_WAIT_LIMIT_US, 0)
    dec.step()
    bits = dec.status(clear=True)
    print(f"{name}: status after a step with wait limit 0: {bits:#x}", flush=True)
    assert bits == kdm.KD_STATUS_SYNC_TIMEOUT
    assert int(dec.tokens.item()) == int(prompt[-1]) and int(dec.positions.item()) == len(prompt) - 1
    dec.control(kdm.KD_CTRL_WAIT_LIMIT_US, 2_000_000)
    o = ref.Oracle(wl.model, w, batch=1, max_seq=wl.max_seq)
    for p, t in enumerate(prompt[:-1]):
        o.step_one(0, int(t), p)
    tok = int(prompt[-1])
    for i in range(2):  # the retried step, then one more, each against the oracle fed the same token
        dec.step()
        want = o.step_one(0, tok, len(prompt) - 1 + i)
        gl = dec.logits[0].cpu().numpy()
        assert gh.inf_rel_err(gl, want) <= tol, i
        g_tok = int(dec.tokens.item())
        if g_tok != int(ref.greedy_token(want[None])[0]):
            assert gh.top2_margin(want) <= 2 * np.max(np.abs(gl - want))
        tok = g_tok
    assert dec.status() == 0 and int(dec.positions.item()) == len(prompt) + 1
    dec.close()

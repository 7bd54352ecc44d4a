"""Edge cases of both paths against the CPU oracle: ragged per-session positions, the smallest and
largest session counts, every query-group size the lockstep path takes, and the last cache slot.

Every input is seeded and synthetic (``workloads``); every expected value comes from ``oracle``.
Tolerances: 2e-2 of the largest reference logit for bf16 weights, 1e-4 for the fp32 tiny
decoder; a greedy token may differ from the oracle's only at a tie-flip (top-2 margin within
twice the step's measured logit error), and the oracle is teacher-forced with the GPU's tokens.
"""

import numpy as np
import pytest

import workloads
from oracle import decoder as ref
from workloads.presets import ModelShape, Workload

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


def _check(gl, g_tok, want, tol, tag):
    err = gh.inf_rel_err(gl, want)
    assert err <= tol, (tag, err)
    ref_tok = int(ref.greedy_token(want[None])[0])
    if int(g_tok) != ref_tok:
        abs_err = float(np.max(np.abs(np.asarray(gl, np.float64) - want)))
        assert gh.top2_margin(want) <= 2 * abs_err, (tag, int(g_tok), ref_tok, gh.top2_margin(want), abs_err)
        return err, 1
    return err, 0


# (sessions, q heads, kv heads, d_model): the smallest batch with plain multi-head attention, an
# odd batch (a partly filled 16-row MFMA tile) with two query heads per kv head, the largest batch
# with four, and a d_model of 256, whose gate/up GEMM runs unsplit and so writes SiLU(gate) * up
# itself. Every GEMM of these shapes meets the lockstep path's tile and split constraints.
RAGGED_CASES = [(2, 2, 2, 512), (17, 4, 2, 512), (64, 8, 2, 512), (17, 2, 1, 256)]


@pytest.mark.parametrize("B,hq,hkv,d", RAGGED_CASES)
def test_lockstep_ragged_positions(torch, kdm, B, hq, hkv, d):
    """Sessions at different positions in one tick: from position 0 (a single cached key) through
    both sides of the 512-position attention chunk boundaries, to the last slot of the cache on
    the final tick. Logits, tokens and positions of every session, every tick."""
    ticks = 5
    shape = ModelShape(2, d, hq, hkv, 128, 512, 1024, rope_base=500000.0)
    start = np.array([(b * 389) % 1090 for b in range(B)], np.int64)
    start[0] = 0
    start[-1] = 1090  # reaches max_seq - 1 on the last tick
    start[B // 2] = 511  # crosses a chunk boundary
    prefill = int(start.max())
    wl = Workload(f"ragged_b{B}", shape, batch=B, prefill_len=prefill, gen_tokens=ticks, weight_seed=21, kv_seed=22,
                  first_token_seed=23)
    assert wl.max_seq == prefill + ticks
    w = workloads.make_weights(shape, seed=wl.weight_seed)
    dec = kdm.Decoder(shape, w, max_seq=wl.max_seq, batch=B)
    info = kdm.kd_get_info(dec.handle)
    assert info["workgroups"] == 0  # the lockstep path
    if d == 256:  # one K chunk pair: gate/up unsplit, SiLU fused into it (9 launches per layer)
        assert info["split_k"][2] == 1 and info["kernels_per_step"] == 2 + 9 * shape.n_layers + 2
    o = ref.Oracle(shape, w, batch=B, max_seq=wl.max_seq)
    kv = dec.kv_view().view(torch.int16)
    for l in range(shape.n_layers):
        for g in range(hkv):
            for b in range(B):
                n = int(start[b])
                kb = workloads.kv_prefill_block(wl, l, 0, b, g)[:n]
                vb = workloads.kv_prefill_block(wl, l, 1, b, g)[:n]
                kv[l, 0, b, g, :n] = torch.from_numpy(kb.view(np.int16))
                kv[l, 1, b, g, :n] = torch.from_numpy(vb.view(np.int16))
                o.load_kv(b, l, g, workloads.f32_from_bf16_bits(kb), workloads.f32_from_bf16_bits(vb))
    tok = workloads.make_first_tokens(wl).astype(np.int64)
    dec.tokens.copy_(torch.from_numpy(tok.astype(np.int32)))
    dec.positions.copy_(torch.from_numpy(start.astype(np.int32)))
    worst, flips = 0.0, 0
    for t in range(ticks):
        dec.step()
        gl = dec.logits.cpu().numpy()
        g_tok = dec.tokens.cpu().numpy()
        want = o.step(tok, start + t)
        for b in range(B):
            err, f = _check(gl[b], g_tok[b], want[b], BF16_TOL, (t, b, int(start[b] + t)))
            worst = max(worst, err)
            flips += f
        tok = g_tok.astype(np.int64)
    print(f"ragged B={B} G={hq // hkv} d={d}: max rel logit err {worst:.3e}, tie-flips {flips}", flush=True)
    assert flips <= 1
    assert dec.status() == 0
    assert np.array_equal(dec.positions.cpu().numpy(), start + ticks)
    # the next tick would write past the cache of the last session: refused, nothing written
    dec.logits.fill_(-7.0)
    before = dec.kv.clone()
    dec.step()
    assert dec.status(clear=True) == kdm.KD_STATUS_POS_OVERFLOW
    assert bool(torch.all(dec.logits == -7.0)) and bool(torch.equal(before, dec.kv))
    dec.close()


def test_batch1_last_cache_slot(torch, kdm):
    """Batch 1 (the persistent kernel) with a cache of exactly prompt + generated positions: the
    last step writes the cache's final slot; the step after it is refused."""
    wl = workloads.get("tiny").with_(prompt_len=9, gen_tokens=4)
    m = wl.model
    w = workloads.make_weights(m, seed=wl.weight_seed)
    dec = kdm.Decoder(m, w, max_seq=wl.max_seq)
    prompt = workloads.make_prompt(wl, 0)[: wl.prompt_len]
    # every step that fills the cache produces logits: the prompt, then the generated tokens
    toks, logits = gh.run_prompt(dec, prompt, wl.max_seq - wl.prompt_len + 1, torch)
    o = ref.Oracle(m, w, batch=1, max_seq=wl.max_seq)
    worst, flips = 0.0, 0
    fed = list(prompt) + [int(t) for t in toks[wl.prompt_len - 1 : -1]]
    assert len(fed) == wl.max_seq
    for p, t in enumerate(fed):
        want = o.step_one(0, int(t), p)
        err, f = _check(logits[p], toks[p], want, F32_TOL, p)
        worst = max(worst, err)
        flips += f
    assert flips == 0
    assert int(dec.positions.item()) == wl.max_seq and dec.status() == 0
    # the K the kernel appended at the last slot matches the oracle's
    kv = dec.kv_view()
    k_last = kv[:, 0, 0, :, wl.max_seq - 1].float().cpu().numpy()  # [L][hkv][hd]
    assert np.max(np.abs(k_last - o.k_cache[0, :, :, wl.max_seq - 1])) <= 1e-5 * max(1.0, np.max(np.abs(k_last)))
    before = dec.kv.clone()
    dec.step()
    assert dec.status(clear=True) == kdm.KD_STATUS_POS_OVERFLOW
    assert bool(torch.equal(before, dec.kv))
    dec.close()


def _tiny_run(kdm, wl, w, n_steps, torch, stream=None, trace=False, other=None):
    """Steps of the tiny decoder from position 0 on `stream`; with `other` (a second decoder), the
    two handles step alternately. Returns the logits of every step (and the trace buffer)."""
    m = wl.model
    dec = kdm.Decoder(m, w, max_seq=wl.max_seq)
    buf = None
    if trace:
        info = kdm.kd_get_info(dec.handle)
        stride = kdm.kd_trace(dec.handle, None, 0)
        buf = torch.zeros(stride * info["workgroups"], dtype=torch.int64, device=dec.device)
        kdm.kd_trace(dec.handle, buf, buf.numel())
    prompt = workloads.make_prompt(wl, 0)
    out = []
    # every fill, step and copy goes on one stream (the current one inside the block)
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
        for p in range(n_steps):
            dec.tokens.fill_(int(prompt[p]))
            dec.positions.fill_(p)
            dec.step()
            if other is not None:
                other.tokens.fill_(int(prompt[-1 - p]))
                other.positions.fill_(p)
                other.step()
            out.append(dec.logits.clone())
    torch.cuda.synchronize()
    assert dec.status() == 0
    logits = torch.stack(out).cpu().numpy()
    raw = buf.cpu().numpy() if buf is not None else None
    if trace:
        kdm.kd_trace(dec.handle, None, 0)
    dec.close()
    return logits, raw


def test_trace_stream_and_second_handle_leave_results_bitwise_equal(torch, kdm):
    """Tracing a step, launching on a non-default stream, and stepping a second handle in between
    change no bit of the logits; the trace holds one increasing run of timestamps per workgroup."""
    from bandwidth_bound_transformer_amd import trace as tr

    wl = workloads.get("tiny")
    m = wl.model
    w = workloads.make_weights(m, seed=wl.weight_seed)
    w2 = workloads.make_weights(m, seed=wl.weight_seed + 100)
    n = 6
    base, _ = _tiny_run(kdm, wl, w, n, torch)
    traced, raw = _tiny_run(kdm, wl, w, n, torch, trace=True)
    assert np.array_equal(base.view(np.uint32), traced.view(np.uint32))
    side = torch.cuda.Stream()  # default priority
    on_side, _ = _tiny_run(kdm, wl, w, n, torch, stream=side)
    assert np.array_equal(base.view(np.uint32), on_side.view(np.uint32))
    other = kdm.Decoder(m, w2, max_seq=wl.max_seq)
    mixed, _ = _tiny_run(kdm, wl, w, n, torch, other=other)
    assert other.status() == 0
    other.close()
    assert np.array_equal(base.view(np.uint32), mixed.view(np.uint32))
    # the traced buffer holds the last step: every workgroup stamped its start, setup and final
    # phases, and the stamps it reached never go backwards
    nwg = 256
    st = tr.stride(m.n_layers)
    t = raw[: nwg * st].reshape(nwg, st)
    assert np.all(t[:, 0] > 0) and np.all(t[:, 1] >= t[:, 0])
    for row in t:
        reached = row[row > 0]
        assert np.all(np.diff(reached) >= 0)
    parts, total = tr.intervals(raw, m.n_layers, nwg)
    assert np.all(total > 0) and np.all(total < 1e5)  # microseconds
    # the oracle agrees with the untraced run
    o = ref.Oracle(m, w, batch=1, max_seq=wl.max_seq)
    prompt = workloads.make_prompt(wl, 0)
    for p in range(n):
        want = o.step_one(0, int(prompt[p]), p)
        assert gh.inf_rel_err(base[p, 0], want) <= F32_TOL, p


def _snapshot(dec):
    """Session state is the caller's buffers: cache, positions and tokens (device copies)."""
    return dec.kv.clone(), dec.positions.clone(), dec.tokens.clone()


def _restore(dec, snap):
    kv, pos, tok = snap
    dec.kv.copy_(kv)
    dec.positions.copy_(pos)
    dec.tokens.copy_(tok)


@pytest.mark.parametrize("kind", ["batch1", "lockstep"])
def test_checkpoint_resume_is_bitwise_exact(torch, kdm, kind):
    """Decoding N + M steps on one handle equals decoding N, snapshotting the caller-owned state,
    destroying the handle, restoring into a new one and decoding M: the same bits of logits,
    tokens, positions and cache."""
    if kind == "batch1":
        wl = workloads.get("tiny").with_(prompt_len=12, gen_tokens=12)
        B = 1
    else:
        shape = ModelShape(2, 512, 4, 2, 128, 512, 1024, rope_base=500000.0)
        wl = Workload("resume_x17", shape, batch=17, prefill_len=40, gen_tokens=12, weight_seed=31, kv_seed=32,
                      first_token_seed=33)
        B = 17
    m = wl.model
    w = workloads.make_weights(m, seed=wl.weight_seed)
    N, M = 7, 5

    def start(dec):
        if wl.prefill_len > 0:
            kv = dec.kv_view().view(torch.int16)
            for l in range(m.n_layers):
                for s in range(2):
                    for b in range(B):
                        for g in range(m.n_kv_heads):
                            blk = workloads.kv_prefill_block(wl, l, s, b, g)
                            kv[l, s, b, g, : wl.prefill_len] = torch.from_numpy(blk.view(np.int16))
            dec.tokens.copy_(torch.from_numpy(workloads.make_first_tokens(wl)))
            dec.positions.fill_(wl.prefill_len)
        else:
            # the prompt's first token at position 0; every later step feeds back the greedy token
            dec.tokens.fill_(int(workloads.make_prompt(wl, 0)[0]))
            dec.positions.zero_()

    def run(dec, n):
        out = []
        for _ in range(n):
            dec.step()
            out.append(torch.cat([dec.logits.flatten(), dec.tokens.float(), dec.positions.float()]))
        torch.cuda.synchronize()
        return torch.stack(out).cpu().numpy()

    a = kdm.Decoder(m, w, max_seq=wl.max_seq, batch=B)
    start(a)
    whole = run(a, N + M)
    kv_whole = a.kv.clone()
    assert a.status() == 0
    a.close()

    b = kdm.Decoder(m, w, max_seq=wl.max_seq, batch=B)
    start(b)
    first = run(b, N)
    snap = _snapshot(b)
    b.close()
    c = kdm.Decoder(m, w, max_seq=wl.max_seq, batch=B)
    _restore(c, snap)
    second = run(c, M)
    assert c.status() == 0
    assert np.array_equal(np.concatenate([first, second]).view(np.uint32), whole.view(np.uint32))
    assert bool(torch.equal(c.kv, kv_whole))
    c.close()

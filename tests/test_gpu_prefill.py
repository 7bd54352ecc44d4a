"""kd_prefill: a prompt run as small-M GEMMs on the matrix cores, chunk by chunk (through the C ABI).

A prompt's positions become the rows of the lockstep kernels, all appending to and attending over
one session's cache ("Kog 3000 tok/s real-time inference", section "deployable parameters and
monitoring checklist": time to first token). What must hold:

* the cache it fills equals the cache that one-token steps fill, to bf16 rounding: the matrix
  cores take the activations as bf16 hi/lo pairs (about 16 significant bits), so a stored K or V
  value may land on a neighbouring bf16 value (within two bf16 steps of the largest entry of its
  vector; over the 2B's 26 layers about a fifth of the stored values differ by such a step);
* the logits of the last prompt position, and of the decode steps after it, match the oracle's
  full-sequence recomputation within 2e-2 of the largest logit, with the same greedy tokens
  (tie-flips aside, see gpu_harness.compare_sequence);
* chunks that end mid-prompt, prompts that continue an earlier context, and every chunk size
  give the same results.
"""

import numpy as np
import pytest

import workloads
from oracle import decoder as ref
from workloads import ModelShape

from . import gpu_harness as gh
from .test_gpu_parity import _oracle_from_gpu_cache

pytestmark = pytest.mark.gpu

TOL = 2e-2
# small enough for the oracle, and a shape both the batch-1 kernel and the lockstep kernels take
SMALL = ModelShape(2, 512, 4, 2, 128, 2048, 2048, rope_base=10000.0)
# plain multi-head attention (one q head per kv head): the prefill attention's G = 1 instantiation
SMALL_MHA = ModelShape(2, 512, 4, 4, 128, 2048, 2048, rope_base=10000.0)


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


def _stepwise(dec, prompt, torch):
    """Feed the prompt one kd_step per token from position 0 (the reference path on the GPU)."""
    p_d = torch.as_tensor(np.asarray(prompt, np.int32), device=dec.device)
    dec.positions.zero_()
    for p in range(len(prompt)):
        dec.tokens.copy_(p_d[p : p + 1])
        dec.step()
    torch.cuda.synchronize()


def _cache_close(a, b, n, tag):
    """Caches [L][2][1][Hkv][S][hd] over positions 0..n-1: each stored K or V vector (one layer, slot,
    head and position) within two bf16 steps of its largest entry. The matrix cores' error is
    relative to the size of the dot product's terms, so a value near zero can move by more than
    one step of its own; bounded by the vector it sits in, it cannot."""
    x = a[:, :, :, :, :n].float().cpu().numpy()
    y = b[:, :, :, :, :n].float().cpu().numpy()
    diff = np.abs(x - y)
    vec_max = np.max(np.abs(y), axis=-1, keepdims=True)
    frac = float(np.mean(diff > 0))
    ratio = float(np.max(diff / vec_max))
    print(f"{tag}: cache max |diff| {np.max(diff):.3e}, largest |diff| / vector max {ratio:.3e}, values that differ {frac:.2%}")
    assert ratio <= 2.0**-6


@pytest.mark.parametrize("chunk,mha", [(128, False), (64, False), (16, False), (128, True)])
def test_prefill_small_ragged_and_continued(torch, kdm, chunk, mha):
    """100 prompt tokens (a last chunk that ends mid-chunk), then 30 more from position 100, then a
    decode step: cache, tokens and logits against one-token steps and the oracle (two q heads per kv
    head, or one)."""
    SHAPE = SMALL_MHA if mha else SMALL
    w = workloads.make_weights(SHAPE, seed=4)
    rng = np.random.default_rng(12)
    prompt = rng.integers(0, SHAPE.vocab, 130).astype(np.int32)
    pre = kdm.Decoder(SHAPE, w, max_seq=160, prefill_chunk=chunk)
    step = kdm.Decoder(SHAPE, w, max_seq=160)
    assert kdm.kd_get_info(pre.handle)["kernels_per_step"] == chunk  # info[5]: the prefill chunk
    p_d = torch.as_tensor(prompt, device=pre.device)
    pre.positions.zero_()
    pre.prefill(p_d[:100])
    torch.cuda.synchronize()
    assert pre.status() == 0
    assert int(pre.positions.item()) == 100
    want = ref.forward_full(SHAPE, w, prompt[:100])[-1]
    err = gh.inf_rel_err(pre.logits[0].cpu().numpy(), want)
    print(f"prefill chunk {chunk}: last-position rel logit err {err:.3e}")
    assert err <= TOL
    assert int(pre.tokens.item()) == int(ref.greedy_token(want[None])[0]) or gh.top2_margin(want) <= 2 * err * np.max(np.abs(want))
    _stepwise(step, prompt[:100], torch)
    _cache_close(pre.kv_view(), step.kv_view(), 100, f"chunk {chunk}, positions 0..99")
    # continue the same session from position 100
    pre.prefill(p_d[100:130])
    torch.cuda.synchronize()
    assert pre.status() == 0 and int(pre.positions.item()) == 130
    want = ref.forward_full(SHAPE, w, prompt[:130])
    err = gh.inf_rel_err(pre.logits[0].cpu().numpy(), want[-1])
    assert err <= TOL
    nxt = int(pre.tokens.item())
    # a decode step from the prefilled cache
    pre.step()
    got = pre.logits[0].cpu().numpy()
    want2 = ref.forward_full(SHAPE, w, list(prompt[:130]) + [nxt])[-1]
    err2 = gh.inf_rel_err(got, want2)
    print(f"prefill chunk {chunk}: continued prefill err {err:.3e}, next decode step err {err2:.3e}")
    assert err2 <= TOL
    assert pre.status() == 0 and int(pre.positions.item()) == 131
    pre.close()
    step.close()


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_prefill_one_byte_weights(torch, kdm, dtype):
    """An fp8 or int8 model: the prefill engine computes with its weights decoded to bf16 (code times
    row scale, rounded once), the decode steps with the codes themselves. 100 prompt tokens in
    passes of 64: the last position's logits against the oracle fed the same codes and scales, the
    cache against one-token steps of the one-byte kernel, then a decode step from that cache."""
    shape = ModelShape(2, 1024, 8, 2, 128, 2048, 4096, rope_base=10000.0, weight_dtype=dtype, kv_dtype="bf16")
    w = workloads.make_weights(shape, seed=6)
    prompt = np.random.default_rng(13).integers(0, shape.vocab, 100).astype(np.int32)
    pre = kdm.Decoder(shape, w, max_seq=128, prefill_chunk=64)
    step = kdm.Decoder(shape, w, max_seq=128)
    p_d = torch.as_tensor(prompt, device=pre.device)
    pre.positions.zero_()
    pre.prefill(p_d)
    torch.cuda.synchronize()
    assert pre.status() == 0 and int(pre.positions.item()) == 100
    want = ref.forward_full(shape, w, prompt)[-1]
    err = gh.inf_rel_err(pre.logits[0].cpu().numpy(), want)
    assert err <= TOL
    assert int(pre.tokens.item()) == int(ref.greedy_token(want[None])[0]) or gh.top2_margin(want) <= 2 * err * np.max(np.abs(want))
    _stepwise(step, prompt, torch)
    _cache_close(pre.kv_view(), step.kv_view(), 100, f"{dtype} prefill, positions 0..99")
    nxt = int(pre.tokens.item())
    pre.step()
    want2 = ref.forward_full(shape, w, list(prompt) + [nxt])[-1]
    err2 = gh.inf_rel_err(pre.logits[0].cpu().numpy(), want2)
    print(f"{dtype} prefill: last-position rel logit err {err:.3e}, next decode step {err2:.3e}")
    assert err2 <= TOL and pre.status() == 0 and int(pre.positions.item()) == 101
    pre.close()
    step.close()


def test_prefill_chunk_boundary_and_single_position(torch, kdm):
    """256 prompt tokens in two full passes of 128 (ending on a 256-position attention chunk), then one
    more token alone at position 256 (a pass of one row that opens the next chunk): logits against
    the oracle, and the one-row pass against a one-token step from the same cache."""
    w = workloads.make_weights(SMALL, seed=6)
    rng = np.random.default_rng(13)
    prompt = rng.integers(0, SMALL.vocab, 257).astype(np.int32)
    pre = kdm.Decoder(SMALL, w, max_seq=300, prefill_chunk=128)
    p_d = torch.as_tensor(prompt, device=pre.device)
    pre.positions.zero_()
    pre.prefill(p_d[:256])
    torch.cuda.synchronize()
    assert pre.status() == 0 and int(pre.positions.item()) == 256
    want = ref.forward_full(SMALL, w, prompt[:257])
    err = gh.inf_rel_err(pre.logits[0].cpu().numpy(), want[255])
    assert err <= TOL, err
    step = kdm.Decoder(SMALL, w, max_seq=300)
    step.kv_view().copy_(pre.kv_view())
    step.positions.fill_(256)
    step.tokens.fill_(int(prompt[256]))
    step.step()
    pre.prefill(p_d[256:257])
    torch.cuda.synchronize()
    assert pre.status() == 0 and int(pre.positions.item()) == 257
    got = pre.logits[0].cpu().numpy()
    err1 = gh.inf_rel_err(got, want[256])
    err2 = gh.inf_rel_err(got, step.logits[0].cpu().numpy())
    print(f"prefill at a chunk boundary: rel logit err {err:.3e}; one-row pass {err1:.3e} (oracle), {err2:.3e} (one-token step)")
    assert err1 <= TOL and err2 <= TOL
    pre.close()
    step.close()


def test_2b_prefill_then_decode(torch, kdm):
    """The 2B decoder's 512-token prompt through kd_prefill (8 chunks of 64), against the cache one-token
    steps fill, then 8 greedy decode steps from it, every logit against the oracle."""
    wl = workloads.get("2b")
    w = workloads.make_weights(wl.model, seed=wl.weight_seed)
    prompt = workloads.make_prompt(wl, 0)
    pre = kdm.Decoder(wl.model, w, max_seq=wl.max_seq, prefill_chunk=64)
    pre.positions.zero_()
    pre.prefill(torch.as_tensor(prompt, device=pre.device))
    toks = [int(pre.tokens.item())]
    logits = [pre.logits[0].cpu().numpy()]
    for _ in range(7):
        pre.step()
        toks.append(int(pre.tokens.item()))
        logits.append(pre.logits[0].cpu().numpy())
    torch.cuda.synchronize()
    assert pre.status() == 0
    step = kdm.Decoder(wl.model, w, max_seq=wl.max_seq)
    _stepwise(step, prompt, torch)
    _cache_close(pre.kv_view(), step.kv_view(), len(prompt), "2b prompt")
    step.close()
    print("2b prefill: GPU done; oracle ...", flush=True)
    seq = list(prompt) + toks[:-1]
    want = ref.forward_full(wl.model, w, seq)[len(prompt) - 1 :]
    worst, flips, defects = gh.compare_sequence(np.array(toks), np.stack(logits), want, TOL)
    print(f"2b prefill + 8 steps: max rel logit err {worst:.3e}, tie-flips {flips}")
    assert worst <= TOL and not defects and flips <= 1
    pre.close()


def test_8b_prefill_1024(torch, kdm):
    """The Llama-3-8B shape's 1024-token prompt through kd_prefill (8 chunks of 128, the eight-tile
    GEMMs): its cache against the one one-token steps fill, and the last position's logits against the
    oracle run from that cache."""
    wl = workloads.get("8b")
    m = wl.model
    w = workloads.make_weights(m, seed=wl.weight_seed)
    prompt = workloads.make_prompt(wl, 0)
    P = len(prompt)
    pre = kdm.Decoder(m, w, max_seq=wl.max_seq, prefill_chunk=128)
    pre.positions.zero_()
    pre.prefill(torch.as_tensor(prompt, device=pre.device))
    torch.cuda.synchronize()
    assert pre.status() == 0 and int(pre.positions.item()) == P
    got = pre.logits[0].cpu().numpy()
    tok = int(pre.tokens.item())
    step = kdm.Decoder(m, w, max_seq=wl.max_seq)
    _stepwise(step, prompt[: P - 1], torch)
    print("8b prefill: GPU done; oracle ...", flush=True)
    o = _oracle_from_gpu_cache(m, w, step, P - 1, P + 1)
    want = o.step_one(0, int(prompt[P - 1]), P - 1)
    err = gh.inf_rel_err(got, want)
    print(f"8b prefill: last-position rel logit err {err:.3e}")
    assert err <= TOL
    assert tok == int(ref.greedy_token(want[None])[0]) or gh.top2_margin(want) <= 2 * np.max(np.abs(got - want))
    step.tokens.fill_(int(prompt[P - 1]))
    step.step()
    torch.cuda.synchronize()
    _cache_close(pre.kv_view(), step.kv_view(), P, "8b prompt")
    pre.close()
    step.close()


def test_prefill_refusals(torch, kdm):
    """kd_prefill needs a handle made with prefill_chunk, bf16 weights, and at least one token."""
    w = workloads.make_weights(SMALL, seed=4)
    plain = kdm.Decoder(SMALL, w, max_seq=64)
    p_d = torch.zeros(4, dtype=torch.int32, device=plain.device)
    with pytest.raises(kdm.KDError) as e:
        plain.prefill(p_d)
    assert e.value.code == kdm.KD_ERR_UNSUPPORTED
    plain.close()
    pre = kdm.Decoder(SMALL, w, max_seq=64, prefill_chunk=64)
    with pytest.raises(kdm.KDError) as e:
        kdm.kd_prefill(pre.handle, p_d, 0, pre.tokens, pre.positions, pre.kv)
    assert e.value.code == kdm.KD_ERR_INVALID_ARG
    pre.close()
    for bad in (1, 129, -1):  # a pass holds 2..128 positions
        with pytest.raises(kdm.KDError) as e:
            kdm.kd_init(kdm.make_config(SMALL, 1, 64, prefill_chunk=bad), w)
        assert e.value.code == kdm.KD_ERR_INVALID_ARG

"""kd_step_noalloc: the batch-1 step with the library's static scratch instead of the handle's
exchange memory. Its outputs must equal kd_step's bit for bit (same kernel, same inputs), on calls
in a row whose models need less and less of the shared array.

Inputs are seeded and synthetic (``workloads``); the expected values come from kd_step on a
second handle with the same weights and state.
"""

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


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


def _pair(kdm, torch, wl, w, prompt_len):
    """Two decoders with the same weights, both stepped through the same prompt by kd_step."""
    decs = [kdm.Decoder(wl.model, w, max_seq=wl.max_seq) for _ in range(2)]
    prompt = torch.as_tensor(np.asarray(workloads.make_prompt(wl, 0)[:prompt_len], np.int32), device=decs[0].device)
    for dec in decs:
        dec.positions.zero_()
        for p in range(prompt_len):
            dec.tokens.copy_(prompt[p : p + 1])
            dec.step(write_logits=False)
    torch.cuda.synchronize()
    return decs


def _compare(kdm, torch, a, b, steps, tag):
    """a steps with kd_step, b with kd_step_noalloc, each fed its own greedy tokens."""
    for i in range(steps):
        a.step()
        kdm.kd_step_noalloc(b.handle, b.tokens, b.positions, b.kv, b.logits, torch.cuda.current_stream(b.device))
        torch.cuda.synchronize()
        assert a.status() == 0 and b.status() == 0, (tag, i)
        assert int(a.tokens.item()) == int(b.tokens.item()), (tag, i)
        assert int(a.positions.item()) == int(b.positions.item()), (tag, i)
        la, lb = a.logits.cpu().numpy(), b.logits.cpu().numpy()
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), (tag, i)
    assert bool(torch.equal(a.kv, b.kv)), tag
    print(f"{tag}: {steps} kd_step_noalloc calls equal kd_step bit for bit", flush=True)


def test_noalloc_matches_step_large_then_small(torch, kdm):
    """The 2B shape (8.1 MiB of exchange words), then the tiny one (1 MiB) in the same array,
    then the 2B again: every call equals kd_step on a twin handle."""
    big = workloads.get("2b")
    w_big = workloads.make_weights(big.model, seed=big.weight_seed)
    a, b = _pair(kdm, torch, big, w_big, 16)
    _compare(kdm, torch, a, b, 3, "2b")
    small = workloads.get("tiny")
    w_small = workloads.make_weights(small.model, seed=small.weight_seed)
    c, d = _pair(kdm, torch, small, w_small, 6)
    _compare(kdm, torch, c, d, 3, "tiny")
    _compare(kdm, torch, a, b, 2, "2b again")
    for dec in (a, b, c, d):
        dec.close()

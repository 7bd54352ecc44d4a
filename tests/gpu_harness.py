"""Drive the HIP library through its C ABI and compare what it produces with the oracle.

Helpers for the GPU tests, the smoke check and the benchmark's parity
sampling.  Inputs come from ``workloads`` only; expected values come from
``oracle`` only.
"""

from __future__ import annotations

import numpy as np

from oracle import decoder as ref


def inf_rel_err(got, want) -> float:
    """max_i |got_i - want_i| / max_i |want_i|: error relative to the largest reference logit."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))


def top2_margin(logits) -> float:
    l32 = np.sort(np.asarray(logits, np.float64).astype(np.float32))
    return float(l32[-1] - l32[-2])


def run_prompt(dec, prompt, n_gen: int, torch):
    """Feed ``prompt`` from position 0, then generate greedily; return (tokens, logits per step).

    Logits are returned for every step that produced a token: the last prompt step and the
    n_gen - 1 decode steps after it, plus the prompt steps before (all on the device until the end).
    """
    dev = dec.device
    prompt_d = torch.as_tensor(np.asarray(prompt, np.int32), device=dev)
    dec.positions.zero_()
    out_logits = []
    out_tokens = []
    for p in range(len(prompt)):
        dec.tokens.copy_(prompt_d[p : p + 1])
        dec.step()
        out_logits.append(dec.logits[0].clone())
        out_tokens.append(dec.tokens.clone())
    for _ in range(n_gen - 1):
        dec.step()
        out_logits.append(dec.logits[0].clone())
        out_tokens.append(dec.tokens.clone())
    torch.cuda.synchronize(dev)
    logits = torch.stack(out_logits).cpu().numpy()
    toks = torch.cat(out_tokens).cpu().numpy()
    return toks, logits


def compare_sequence(gpu_tokens, gpu_logits, ref_logits, tol: float):
    """Check logits step by step and the greedy choice of every step.

    A step whose GPU token differs from the oracle's argmax counts as a tie-flip when the
    oracle's top-2 margin is within twice that step's measured logit error; otherwise it is a
    defect. Returns (max relative error, number of tie-flips, list of defects).
    """
    worst = 0.0
    flips = 0
    defects = []
    for i, (g_tok, gl, rl) in enumerate(zip(gpu_tokens, gpu_logits, ref_logits)):
        err = inf_rel_err(gl, rl)
        worst = max(worst, err)
        want = int(ref.greedy_token(rl[None])[0])
        if int(g_tok) != want:
            abs_err = float(np.max(np.abs(np.asarray(gl, np.float64) - rl)))
            if top2_margin(rl) <= 2.0 * abs_err:
                flips += 1
            else:
                defects.append((i, int(g_tok), want, top2_margin(rl), abs_err))
    return worst, flips, defects

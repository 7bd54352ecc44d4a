"""More edge cases of both paths against the CPU oracle, on an MI355X.

* Every batch-1 kernel variant the library builds (bf16 or f32 weights, head_dim 64 or 128) at
  query-group sizes 2 and 3; the lockstep path refuses group size 3 (its q width could not be
  256 times a power of two).
* Planted exact argmax ties: duplicated LM-head rows whose equal logits land in different
  workgroups (and in one workgroup), on both paths; the lowest index must win, as in the oracle.
* A NaN LM-head row: the status bit is set and the argmax skips the NaN, on both paths.
* Bitwise determinism of the batch-1 exchange over 500 decode steps of the 2B decoder.

Every input is seeded and synthetic (``workloads``); every expected value comes from ``oracle``
(or, for determinism, from a second run of the library itself).
"""

import numpy as np
import pytest

import workloads
from oracle import decoder as ref
from workloads.presets import ModelShape

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


# (name, shape): each batch-1 kernel variant (weight/cache type x head_dim) at G = 2 or 3
VARIANTS = [
    ("bf16_hd64_g2", ModelShape(2, 512, 8, 4, 64, 2048, 1024, rope_base=10000.0, weight_dtype="bf16", kv_dtype="bf16")),
    ("bf16_hd128_g3", ModelShape(2, 1024, 12, 4, 128, 2048, 2048, rope_base=500000.0, weight_dtype="bf16", kv_dtype="bf16")),
    ("f32_hd128_g3", ModelShape(2, 512, 12, 4, 128, 1024, 1024, rope_base=10000.0, weight_dtype="f32", kv_dtype="f32")),
    ("f32_hd64_g2", ModelShape(2, 256, 8, 4, 64, 1024, 1024, rope_base=10000.0, weight_dtype="f32", kv_dtype="f32")),
]


@pytest.mark.parametrize("name,shape", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_batch1_kernel_variants(torch, kdm, name, shape):
    """A 40-token prompt and 8 greedy tokens through each batch-1 kernel variant; every step's
    logits and token against the oracle (teacher-forced with the GPU's tokens)."""
    w = workloads.make_weights(shape, seed=51)
    max_seq = 48
    dec = kdm.Decoder(shape, w, max_seq=max_seq)
    assert kdm.kd_get_info(dec.handle)["workgroups"] > 0  # the persistent kernel
    prompt = np.random.default_rng(52).integers(0, shape.vocab, 40).astype(np.int32)
    toks, logits = gh.run_prompt(dec, prompt, 8, torch)
    assert dec.status() == 0
    seq = list(prompt) + [int(t) for t in toks[len(prompt) - 1 : -1]]
    want = ref.forward_full(shape, w, seq)
    tol = F32_TOL if shape.weight_dtype == "f32" else BF16_TOL
    worst, flips, defects = gh.compare_sequence(toks, logits, want, tol)
    print(f"{name}: max rel logit err {worst:.3e} over {len(seq)} steps, tie-flips {flips}", flush=True)
    assert worst <= tol and not defects and flips == 0
    dec.close()


def test_lockstep_refuses_group_of_three(kdm):
    shape = ModelShape(2, 512, 6, 2, 128, 512, 1024, weight_dtype="bf16", kv_dtype="bf16")
    w = workloads.make_weights(shape, seed=53)
    with pytest.raises(kdm.KDError) as e:
        kdm.Decoder(shape, w, max_seq=32, batch=4)
    assert e.value.code == kdm.KD_ERR_UNSUPPORTED


def _plant(w, rows, sign, dtype, seed):
    """LM head: the rows in `rows` all equal sign * v, every other row equals -sign * v, so every
    logit is exactly +c or -c: either the planted rows tie at the maximum or all the others do."""
    v = (np.random.default_rng(seed).standard_normal(w["lm_head"].shape[1]) * 0.5).astype(np.float32)
    v = v * np.float32(sign)
    if dtype == "bf16":
        vb = workloads.bf16_bits_from_f32(v)
        lm = np.broadcast_to(vb ^ np.uint16(0x8000), w["lm_head"].shape).copy()
        lm[list(rows)] = vb
    else:
        lm = np.broadcast_to(-v, w["lm_head"].shape).copy()
        lm[list(rows)] = v
    out = dict(w)
    out["lm_head"] = lm
    return out


# planted rows of the tiny decoder's LM head (4 rows per workgroup): far apart, neighbouring
# workgroups, one workgroup, and a three-way tie
TIE_ROWS = [(5, 1000), (0, 4), (300, 301), (3, 515, 1023)]


@pytest.mark.parametrize("rows", TIE_ROWS, ids=[str(r) for r in TIE_ROWS])
def test_batch1_planted_argmax_ties(torch, kdm, rows):
    wl = workloads.get("tiny")
    base = workloads.make_weights(wl.model, seed=wl.weight_seed)
    for sign in (1, -1):
        w = _plant(base, rows, sign, "f32", seed=61)
        dec = kdm.Decoder(wl.model, w, max_seq=8)
        dec.tokens.fill_(17)
        dec.positions.zero_()
        dec.step()
        gl = dec.logits[0].cpu().numpy()
        g_tok = int(dec.tokens.item())
        assert dec.status() == 0
        want = ref.Oracle(wl.model, w, 1, 8).step_one(0, 17, 0)
        exp = int(ref.greedy_token(want[None])[0])
        # the planted logits are bitwise equal on the GPU, so this is an exact tie
        assert len({gl[r].tobytes() for r in rows}) == 1
        top = np.flatnonzero(gl == gl.max())
        print(f"rows {rows} sign {sign}: {len(top)} tied maxima, GPU {g_tok}, oracle {exp}", flush=True)
        assert len(top) >= 2 and g_tok == int(top[0]) == exp
        dec.close()


def test_lockstep_planted_argmax_ties(torch, kdm):
    """Three sessions, LM-head rows tied across GEMM workgroups (128 columns each)."""
    shape = ModelShape(2, 512, 4, 2, 128, 512, 1024, rope_base=500000.0)
    base = workloads.make_weights(shape, seed=55)
    rows = (7, 700, 1023)
    for sign in (1, -1):
        w = _plant(base, rows, sign, "bf16", seed=62)
        dec = kdm.Decoder(shape, w, max_seq=8, batch=3)
        toks = np.array([17, 230, 999], np.int32)
        dec.tokens.copy_(torch.from_numpy(toks))
        dec.positions.zero_()
        dec.step()
        gl = dec.logits.cpu().numpy()
        g_tok = dec.tokens.cpu().numpy()
        assert dec.status() == 0
        want = ref.Oracle(shape, w, batch=3, max_seq=8).step([int(t) for t in toks], [0, 0, 0])
        for b in range(3):
            assert len({gl[b, r].tobytes() for r in rows}) == 1
            top = np.flatnonzero(gl[b] == gl[b].max())
            exp = int(ref.greedy_token(want[b][None])[0])
            assert len(top) >= 2 and int(g_tok[b]) == int(top[0]) == exp, (sign, b)
        dec.close()


def _nan_row(w, row, dtype):
    out = dict(w)
    lm = w["lm_head"].copy()
    lm[row] = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    out["lm_head"] = lm
    zero = w["lm_head"].copy()
    zero[row] = 0
    ref_w = dict(w)
    ref_w["lm_head"] = zero
    return out, ref_w


def _expect_skipping(want, row):
    l32 = np.asarray(want, np.float64).astype(np.float32).copy()
    l32[row] = -np.inf
    return int(np.argmax(l32))


def test_batch1_nan_logit_sets_status(torch, kdm):
    wl = workloads.get("tiny")
    base = workloads.make_weights(wl.model, seed=wl.weight_seed)
    row = 613
    w, ref_w = _nan_row(base, row, "f32")
    dec = kdm.Decoder(wl.model, w, max_seq=8)
    dec.tokens.fill_(17)
    dec.positions.zero_()
    dec.step()
    gl = dec.logits[0].cpu().numpy()
    assert dec.status(clear=True) == kdm.KD_STATUS_NAN
    assert np.isnan(gl[row]) and np.isfinite(np.delete(gl, row)).all()
    want = ref.Oracle(wl.model, ref_w, 1, 8).step_one(0, 17, 0)
    assert gh.inf_rel_err(np.delete(gl, row), np.delete(want, row)) <= F32_TOL
    assert int(dec.tokens.item()) == _expect_skipping(want, row)
    assert int(dec.positions.item()) == 1
    dec.close()


def test_lockstep_nan_logit_sets_status(torch, kdm):
    shape = ModelShape(2, 512, 4, 2, 128, 512, 1024, rope_base=500000.0)
    base = workloads.make_weights(shape, seed=56)
    row = 77
    w, ref_w = _nan_row(base, row, "bf16")
    dec = kdm.Decoder(shape, w, max_seq=8, batch=2)
    toks = np.array([5, 600], np.int32)
    dec.tokens.copy_(torch.from_numpy(toks))
    dec.positions.zero_()
    dec.step()
    gl = dec.logits.cpu().numpy()
    g_tok = dec.tokens.cpu().numpy()
    assert dec.status(clear=True) == kdm.KD_STATUS_NAN
    want = ref.Oracle(shape, ref_w, batch=2, max_seq=8).step([5, 600], [0, 0])
    for b in range(2):
        assert np.isnan(gl[b, row])
        assert gh.inf_rel_err(np.delete(gl[b], row), np.delete(want[b], row)) <= BF16_TOL
        exp = _expect_skipping(want[b], row)
        if int(g_tok[b]) != exp:
            rest = np.delete(np.asarray(want[b], np.float64), row)
            assert gh.top2_margin(rest) <= 2 * np.max(np.abs(np.delete(gl[b], row) - rest))
    dec.close()


def test_2b_500_steps_bitwise_deterministic(torch, kdm):
    """The lock-free exchange at full size: two runs of 500 decode steps of the 2B decoder from the
    same 16-token prompt give the same tokens, logits and final cache, bit for bit."""
    wl = workloads.get("2b")
    w = workloads.make_weights(wl.model, seed=wl.weight_seed)
    print("2b determinism: weights ready", flush=True)
    prompt = torch.as_tensor(np.asarray(workloads.make_prompt(wl, 0)[:16], np.int32), device="cuda:0")
    runs = []
    for r in range(2):
        dec = kdm.Decoder(wl.model, w, max_seq=wl.max_seq)
        dec.positions.zero_()
        for p in range(len(prompt)):
            dec.tokens.copy_(prompt[p : p + 1])
            dec.step(write_logits=False)
        toks = torch.empty(500, dtype=torch.int32, device=dec.device)
        lg = torch.empty(500, wl.model.vocab, dtype=torch.float32, device=dec.device)
        for i in range(500):
            dec.step()
            toks[i : i + 1].copy_(dec.tokens)
            lg[i].copy_(dec.logits[0])
        torch.cuda.synchronize()
        assert dec.status() == 0
        runs.append((toks.cpu().numpy(), lg.cpu().numpy().view(np.uint32), dec.kv.view(torch.int16).cpu().numpy()))
        dec.close()
    (t0, l0, k0), (t1, l1, k1) = runs
    same_tok = t0 == t1
    first = int(np.argmin(same_tok)) if not same_tok.all() else -1
    assert first == -1, f"tokens differ first at step {first}"
    rows_equal = np.all(l0 == l1, axis=1)
    assert rows_equal.all(), f"logits differ first at step {int(np.argmin(rows_equal))}"
    assert np.array_equal(k0, k1)
    print(f"2b determinism: 500 steps bitwise equal, last token {int(t0[-1])}", flush=True)

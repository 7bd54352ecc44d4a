"""Seeded generators for weights, prompts, first tokens and pre-filled KV values.

Recipe (stated once, used by every consumer):

* Weight tensors are numbered in a fixed order: 0 = embed; for layer l the
  nine tensors attn_norm, wq, wk, wv, wo, ffn_norm, w_gate, w_up, w_down get
  indices 1 + 9*l + (0..8); then final_norm and lm_head.  Norm gains are 1.0.
  Every matrix is 0.02 * N(0,1), drawn in float32 by numpy's PCG64 seeded with
  SeedSequence([seed, tensor_index, chunk_index]), where a chunk is a run of
  whole rows holding at most 2**22 values.  bf16 workloads round those float32
  draws to bf16 (round-to-nearest-even) and hand out the raw 16-bit patterns.
* Prompt ids for session b: uniform integers in [0, vocab) from
  SeedSequence([prompt_seed, b]).  First tokens of pre-filled workloads use
  SeedSequence([first_token_seed, b]) the same way.
* fp8 workloads draw exactly the bf16 workload's weights, then quantise each
  projection matrix and the LM head row by row: a row's scale is its largest
  magnitude divided by 448 (the largest finite E4M3 value), and its codes are
  the OCP FP8 E4M3 values nearest to weight / scale (torch's float8_e4m3fn
  conversion).  The embedding and the norm gains stay bf16.
* int8 workloads quantise the same bf16 weights row by row to int8: a row's
  scale is its largest magnitude divided by 127, and its codes are weight /
  scale (in float32) rounded to nearest, ties to even, within -127..127.
* Pre-filled KV values: for layer l, slot s (0 = K after RoPE, 1 = V), session
  b and kv head g, an array [prefill_len, head_dim] of N(0,1) float32 draws
  from SeedSequence([kv_seed, l, s, b, g]), rounded to bf16 for bf16 caches.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .presets import LAYER_TENSOR_NAMES, TENSORS_PER_LAYER, ModelShape, Workload

_CHUNK_VALUES = 1 << 22
_INIT_STD = np.float32(0.02)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); return uint16 bit patterns."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


E4M3_MAX = 448.0  # largest finite OCP FP8 E4M3 value


@dataclass(frozen=True)
class Fp8Matrix:
    """A matrix stored as OCP FP8 E4M3 codes with one float32 scale per row.

    The value of element (r, c) is (E4M3 value of codes[r, c]) * scale[r]."""

    codes: np.ndarray  # uint8 [rows, cols]
    scale: np.ndarray  # float32 [rows]

    @property
    def shape(self) -> tuple:
        return self.codes.shape

    @property
    def size(self) -> int:
        return self.codes.size

    @property
    def nbytes(self) -> int:
        return self.codes.nbytes + self.scale.nbytes


def quantize_rows_e4m3(w: np.ndarray) -> Fp8Matrix:
    """Per-row absmax quantisation of a float32 matrix to E4M3 codes and float32 scales."""
    import torch

    w = np.ascontiguousarray(w, np.float32)
    amax = np.max(np.abs(w), axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = np.clip(w / scale[:, None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return Fp8Matrix(codes, scale)


INT8_MAX = 127  # largest int8 code a row scale maps to (codes stay symmetric: -127..127)


@dataclass(frozen=True)
class Int8Matrix:
    """A matrix stored as int8 codes with one float32 scale per row.

    The value of element (r, c) is codes[r, c] * scale[r]."""

    codes: np.ndarray  # int8 [rows, cols]
    scale: np.ndarray  # float32 [rows]

    @property
    def shape(self) -> tuple:
        return self.codes.shape

    @property
    def size(self) -> int:
        return self.codes.size

    @property
    def nbytes(self) -> int:
        return self.codes.nbytes + self.scale.nbytes


def quantize_rows_int8(w: np.ndarray) -> Int8Matrix:
    """Per-row absmax quantisation of a float32 matrix to int8 codes and float32 scales: scale =
    max |row| / 127 (1 for an all-zero row), code = w / scale (float32) rounded to nearest, ties to
    even, clipped to -127..127."""
    import torch  # the same float32 arithmetic as numpy's, on all host threads

    t = torch.from_numpy(np.ascontiguousarray(w, np.float32))
    amax = t.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / float(INT8_MAX), torch.ones_like(amax))
    codes = torch.round(t / scale[:, None]).clamp_(-INT8_MAX, INT8_MAX).to(torch.int8)  # ties to even
    return Int8Matrix(codes.numpy().copy(), scale.numpy().copy())


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _fill_matrix(out: np.ndarray, seed: int, tensor_index: int, as_bf16: bool, pool: ThreadPoolExecutor) -> None:
    rows, cols = out.shape
    rows_per_chunk = max(1, _CHUNK_VALUES // cols)

    def work(c: int) -> None:
        r0 = c * rows_per_chunk
        r1 = min(rows, r0 + rows_per_chunk)
        vals = _rng(seed, tensor_index, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        vals *= _INIT_STD
        out[r0:r1] = bf16_bits_from_f32(vals) if as_bf16 else vals

    n_chunks = (rows + rows_per_chunk - 1) // rows_per_chunk
    list(pool.map(work, range(n_chunks)))


def make_weights(shape: ModelShape, seed: int = 0, workers: int | None = None) -> dict:
    """Generate all weights of ``shape`` in the canonical row-major layout.

    Returns a dict: ``embed`` [V, d], ``layers`` (list of dicts with the nine
    per-layer tensors), ``final_norm`` [d], ``lm_head`` [V, d] and ``dtype``.
    bf16 tensors are uint16 bit patterns; f32 tensors are float32. For fp8
    (int8) models the seven matrices of each layer and the LM head are
    ``Fp8Matrix`` (``Int8Matrix``) objects, quantised from the bf16 model's
    weights, and the embedding and gains are bf16.
    """
    fp8 = shape.weight_dtype == "fp8"
    int8 = shape.weight_dtype == "int8"
    as_bf16 = shape.weight_dtype in ("bf16", "fp8", "int8")
    store = np.uint16 if as_bf16 else np.float32
    one = bf16_bits_from_f32(np.ones(1, np.float32))[0] if as_bf16 else np.float32(1.0)
    w = {"dtype": shape.weight_dtype, "layers": []}
    with ThreadPoolExecutor(max_workers=workers or _workers()) as pool:
        def matrix(name: str, index: int, quantise: bool = True):
            arr = np.empty(shape.tensor_shape(name), dtype=store)
            _fill_matrix(arr, seed, index, as_bf16, pool)
            if fp8 and quantise:
                return quantize_rows_e4m3(f32_from_bf16_bits(arr))
            if int8 and quantise:
                return quantize_rows_int8(f32_from_bf16_bits(arr))
            return arr

        def gain(name: str) -> np.ndarray:
            return np.full(shape.tensor_shape(name), one, dtype=store)

        w["embed"] = matrix("embed", 0, quantise=False)
        for l in range(shape.n_layers):
            base = 1 + TENSORS_PER_LAYER * l
            layer = {}
            for j, name in enumerate(LAYER_TENSOR_NAMES):
                layer[name] = gain(name) if name.endswith("norm") else matrix(name, base + j)
            w["layers"].append(layer)
        w["final_norm"] = gain("final_norm")
        w["lm_head"] = matrix("lm_head", 1 + TENSORS_PER_LAYER * shape.n_layers + 1)
    return w


def make_prompt(wl: Workload, session: int = 0) -> np.ndarray:
    """Prompt ids of one session: ``prompt_len`` uniform ids in [0, vocab)."""
    return _rng(wl.prompt_seed, session).integers(0, wl.model.vocab, wl.prompt_len, dtype=np.int64).astype(np.int32)


def make_first_tokens(wl: Workload) -> np.ndarray:
    """Seeded first input token of every session (pre-filled workloads)."""
    return np.array(
        [_rng(wl.first_token_seed, b).integers(0, wl.model.vocab, 1, dtype=np.int64)[0] for b in range(wl.batch)],
        dtype=np.int32,
    )


def kv_prefill_block(wl: Workload, layer: int, slot: int, session: int, kv_head: int) -> np.ndarray:
    """Pre-filled values of one (layer, K/V slot, session, kv head): [prefill_len, head_dim].

    float32 for f32 caches, uint16 bf16 bit patterns for bf16 caches.
    """
    m = wl.model
    vals = _rng(wl.kv_seed, layer, slot, session, kv_head).standard_normal((wl.prefill_len, m.head_dim), dtype=np.float32)
    return bf16_bits_from_f32(vals) if m.kv_dtype == "bf16" else vals


def fill_kv_prefill(wl: Workload, out: np.ndarray, sessions=None, workers: int | None = None) -> None:
    """Write pre-filled values into ``out`` laid out [L][2][B][Hkv][S][hd].

    ``out`` must have the storage dtype (uint16 for bf16, float32 for f32) and
    at least ``prefill_len`` positions; only ``sessions`` (default: all) are written.
    """
    m = wl.model
    sessions = range(wl.batch) if sessions is None else sessions
    jobs = [(l, s, b, g) for l in range(m.n_layers) for s in range(2) for b in sessions for g in range(m.n_kv_heads)]

    def work(job):
        l, s, b, g = job
        out[l, s, b, g, : wl.prefill_len] = kv_prefill_block(wl, l, s, b, g)

    with ThreadPoolExecutor(max_workers=workers or _workers()) as pool:
        list(pool.map(work, jobs))


def fill_kv_prefill_device(wl: Workload, kv_storage_view, torch, sessions=None, log=None) -> None:
    """Write the pre-filled values of ``sessions`` (default: all) into a device cache.

    ``kv_storage_view`` is the caller's cache viewed [L][2][B][Hkv][S][hd] with the storage's
    bit patterns (torch.int16 for bf16, torch.float32 for f32). One layer at a time: the blocks
    are generated on host threads, then copied in one transfer.
    """
    m = wl.model
    sessions = list(range(wl.batch)) if sessions is None else list(sessions)
    storage = np.uint16 if m.kv_dtype == "bf16" else np.float32
    host = np.zeros((2, len(sessions), m.n_kv_heads, wl.prefill_len, m.head_dim), storage)
    jobs = [(s, i, g) for s in range(2) for i in range(len(sessions)) for g in range(m.n_kv_heads)]
    with ThreadPoolExecutor(max_workers=_workers()) as pool:
        for l in range(m.n_layers):
            def work(job, l=l):
                s, i, g = job
                host[s, i, g] = kv_prefill_block(wl, l, s, sessions[i], g)

            list(pool.map(work, jobs))
            src = torch.from_numpy(host.view(np.int16) if m.kv_dtype == "bf16" else host)
            if sessions == list(range(wl.batch)):
                kv_storage_view[l, :, :, :, : wl.prefill_len] = src
            else:
                for i, b in enumerate(sessions):
                    kv_storage_view[l, :, b, :, : wl.prefill_len] = src[:, i]
            if log and ((l + 1) % 8 == 0 or l + 1 == m.n_layers):
                log(f"pre-filled cache: {l + 1}/{m.n_layers} layers")

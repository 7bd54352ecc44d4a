"""Algorithmic HBM bytes of one decode step, and the bandwidth roofline they imply.

Producing one token reads every weight and the whole KV cache once ("Kog 3000
tok/s real-time inference", section "three-layer strategy for memory-bandwidth
optimisation").  The pages turn that into a tokens/s bound: aggregate HBM
bandwidth divided by the bytes a token must read ("Real-time LLM inference on
standard data-centre GPUs (3,000 tokens/s single request)", performance-benchmark
table: 33.6 TB/s over 2B fp16 parameters gives 8,400 tokens/s).

The count below is what the method itself must move per step, not what an
implementation happens to move:

* every layer weight, the final norm and the LM head, once per step (once per
  tick for all B sessions together); for fp8 and int8 models, one byte per matrix
  element plus a float32 scale per matrix row, and bf16 norm gains;
* one embedding row per session;
* per session, the KV cache over positions 0..p (K and V, every layer and kv head);
* per session, the K and V written at position p;
* the fp32 logits, when they are written out.
"""

from __future__ import annotations

from dataclasses import dataclass

MI355X_HBM_BYTES_PER_S = 8.0e12


@dataclass(frozen=True)
class StepBytes:
    weights: int
    embedding: int
    kv_read: int
    kv_write: int
    logits: int

    @property
    def total(self) -> int:
        return self.weights + self.embedding + self.kv_read + self.kv_write + self.logits


def streamed_params(shape) -> int:
    """Parameters read once per step: all layers, the final norm and the LM head."""
    return shape.n_layers * shape.layer_params() + shape.d_model + shape.vocab * shape.d_model


def step_bytes(shape, batch: int, position: int, write_logits: bool = True) -> StepBytes:
    """Bytes of one step in which every session attends over positions 0..position."""
    kv_per_pos = shape.n_layers * 2 * shape.n_kv_heads * shape.head_dim * shape.kv_bytes
    return StepBytes(
        weights=shape.streamed_weight_bytes(),
        embedding=batch * shape.d_model * shape.embed_bytes,
        kv_read=batch * (position + 1) * kv_per_pos,
        kv_write=batch * kv_per_pos,
        logits=batch * shape.vocab * 4 if write_logits else 0,
    )


def decode_positions(workload) -> range:
    """Positions of the decode-phase steps (steps whose input is a generated or seeded token)."""
    start = workload.prefill_len if workload.prefill_len > 0 else workload.prompt_len
    return range(start, start + workload.decode_steps)


def mean_step_bytes(workload, write_logits: bool = True) -> float:
    """Average algorithmic bytes per decode step of ``workload``."""
    pos = decode_positions(workload)
    tot = sum(step_bytes(workload.model, workload.batch, p, write_logits).total for p in pos)
    return tot / max(len(pos), 1)


def step_flops(shape, batch: int, position: int) -> int:
    """Multiply-add work of one step, counted as 2 flops per multiply-add."""
    per_token = 2 * (streamed_params(shape) - shape.d_model * (2 * shape.n_layers + 1))
    attn = 2 * 2 * shape.n_layers * shape.n_q_heads * shape.head_dim * (position + 1)
    return batch * (per_token + attn)


MI355X_BF16_DENSE_FLOPS = 2.5e15  # matrix cores, dense bf16


def prefill_flops(shape, prompt_len: int) -> int:
    """Multiply-add work (2 flops each) of running a prompt of ``prompt_len`` positions from an
    empty cache to its first token: every projection for every position, attention of position p
    over 0..p (scores and weighted sums), and the LM head for the last position only."""
    d, L = shape.d_model, shape.n_layers
    matrix_params = shape.layer_params() - 2 * d  # the seven matrices of a layer
    proj = 2 * prompt_len * L * matrix_params
    attended = prompt_len * (prompt_len + 1) // 2  # sum over p of (p + 1)
    attn = 2 * 2 * L * shape.n_q_heads * shape.head_dim * attended
    return proj + attn + 2 * shape.vocab * d


def tokens_per_s_bound(bandwidth_bytes_per_s: float, bytes_per_step: float, batch: int = 1) -> float:
    """Roofline tokens/s: ``batch`` tokens per step, each step limited by streaming its bytes."""
    return batch * bandwidth_bytes_per_s / bytes_per_step

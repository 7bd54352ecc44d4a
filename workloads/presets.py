"""Model shapes and workload presets.

The presets are the decode workloads this library is measured on:

* ``tiny``    -- 2 layers, d_model 256, 4 heads x 64 (MHA), SwiGLU 1024,
                 vocab 1024, fp32 weights; 32-token prompt, 64 greedy tokens.
* ``2b``      -- 26 layers, d_model 2048, 16 q / 4 kv heads x 128, SwiGLU 8192,
                 vocab 32000 untied, bf16; 512-token prompt, 512 greedy tokens.
                 Stands in for the Kog engine's 2B fp16 preview model ("Real-time
                 LLM inference on standard data-centre GPUs (3,000 tokens/s single
                 request)", section "performance benchmark").
* ``8b``      -- Llama-3-8B shape (32 layers, d_model 4096, 32 q / 8 kv heads,
                 SwiGLU 14336, vocab 128256, RoPE base 500000), bf16;
                 1024-token prompt, 256 greedy tokens ("Kog 3000 tok/s real-time
                 inference", section "three-layer strategy", which reports
                 Llama-3 8B decode).
* ``2b_long`` -- the 2B decoder with a KV cache pre-filled to 32768 positions
                 with N(0,1) bf16 values; 128 greedy tokens (the KV read grows
                 with context: "17k tokens/sec" page, FAQ on long context).
* ``2b_fp8``, ``8b_fp8`` -- the 2B and 8B decoders with their projection matrices
                 and LM head quantised to FP8 E4M3, one float32 scale per output
                 row; embedding, norm gains and KV cache stay bf16 ("17k
                 tokens/sec" page, best practice 2 and FAQ 3: lower-precision
                 parameters cut the bytes each token reads).
* ``11b_x56_fp8``, ``11b_x56_int8`` -- the 56-session workload with E4M3 or
                 int8 projection matrices and LM head (lockstep sessions stream
                 the codes).
* ``2b_int8``, ``8b_int8`` -- the same with int8 codes: one float32 scale per
                 output row (its largest magnitude over 127), codes rounded to
                 nearest, ties to even (best practice 2 of the same page names
                 INT8).
* ``11b_x56`` -- 40 layers, d_model 4096, 32 q / 8 kv heads, SwiGLU 16384,
                 vocab 128256, bf16; 56 sessions stepped in lockstep, each with
                 its own KV cache pre-filled to 4096 positions; 200 ticks
                 ("Why is real-time AI inference 56x more expensive?", sections
                 "advance all active sessions in lockstep" and "measured data:
                 from 1 to 56").

Readings where the pages and the preset list are silent (recorded with the
rest of the design notes): RMSNorm eps is 1e-5 everywhere; RoPE base is
10000 for the tiny and 2B shapes and 500000 for the Llama-3-shaped 8B and
11B; norm gains are 1.0; embedding and LM head are untied.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

LAYER_TENSOR_NAMES = (
    "attn_norm",
    "wq",
    "wk",
    "wv",
    "wo",
    "ffn_norm",
    "w_gate",
    "w_up",
    "w_down",
)
TENSORS_PER_LAYER = len(LAYER_TENSOR_NAMES)


@dataclass(frozen=True)
class ModelShape:
    """Shape of a pre-norm decoder with grouped-query attention and SwiGLU."""

    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rope_base: float = 10000.0
    norm_eps: float = 1e-5
    weight_dtype: str = "bf16"  # "bf16", "f32", "fp8" or "int8" (E4M3 or int8 projection matrices, bf16 embedding and gains)
    kv_dtype: str = "bf16"  # "bf16" or "f32"

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def weight_bytes(self) -> int:
        """Bytes of one element of a projection matrix (or of any weight, for bf16 and f32)."""
        return {"bf16": 2, "f32": 4, "fp8": 1, "int8": 1}[self.weight_dtype]

    @property
    def quantised(self) -> bool:
        """Projection matrices and LM head as one-byte codes with a float32 scale per row."""
        return self.weight_dtype in ("fp8", "int8")

    @property
    def embed_bytes(self) -> int:
        """Bytes of one element of the embedding and the norm gains (bf16 for fp8 and int8 models)."""
        return 4 if self.weight_dtype == "f32" else 2

    @property
    def matrix_rows_per_layer(self) -> int:
        """Output rows of a layer's seven matrices (one scale each in fp8 and int8 models)."""
        return self.q_dim + 2 * self.kv_dim + self.d_model + 2 * self.ffn_dim + self.d_model

    @property
    def kv_bytes(self) -> int:
        return 2 if self.kv_dtype == "bf16" else 4

    def tensor_shape(self, name: str) -> tuple:
        d, q, kv, f, v = self.d_model, self.q_dim, self.kv_dim, self.ffn_dim, self.vocab
        return {
            "embed": (v, d),
            "attn_norm": (d,),
            "wq": (q, d),
            "wk": (kv, d),
            "wv": (kv, d),
            "wo": (d, q),
            "ffn_norm": (d,),
            "w_gate": (f, d),
            "w_up": (f, d),
            "w_down": (d, f),
            "final_norm": (d,),
            "lm_head": (v, d),
        }[name]

    def layer_params(self) -> int:
        d, q, kv, f = self.d_model, self.q_dim, self.kv_dim, self.ffn_dim
        return 2 * d + q * d + 2 * kv * d + d * q + 3 * f * d

    def total_params(self) -> int:
        return 2 * self.vocab * self.d_model + self.n_layers * self.layer_params() + self.d_model

    def streamed_weight_bytes(self) -> int:
        """Bytes of everything a step reads once: every layer, the final norm and the LM head.

        fp8 and int8 models store each projection matrix as one byte per element plus one float32
        scale per output row, and their norm gains in bf16."""
        d, V, L = self.d_model, self.vocab, self.n_layers
        if not self.quantised:
            return (L * self.layer_params() + d + V * d) * self.weight_bytes
        matrices = L * (self.layer_params() - 2 * d) + V * d
        scales = 4 * (L * self.matrix_rows_per_layer + V)
        gains = 2 * (2 * L * d + d)
        return matrices + scales + gains


@dataclass(frozen=True)
class Workload:
    """One decode workload: a model shape plus how the run is fed.

    ``prompt_len`` prompt tokens are fed one per step from position 0, then
    ``gen_tokens`` tokens are generated greedily (the first comes out of the
    last prompt step).  When ``prefill_len`` > 0 there is no prompt: the KV
    cache already holds ``prefill_len`` positions and every one of the
    ``gen_tokens`` steps starts from a seeded first token.
    """

    name: str
    model: ModelShape
    batch: int = 1
    prompt_len: int = 0
    prefill_len: int = 0
    gen_tokens: int = 0
    weight_seed: int = 0
    prompt_seed: int = 1
    kv_seed: int = 2
    first_token_seed: int = 3
    description: str = field(default="", compare=False)

    @property
    def max_seq(self) -> int:
        return self.prompt_len + self.prefill_len + self.gen_tokens

    @property
    def decode_steps(self) -> int:
        """Steps whose input is a generated (or seeded first) token."""
        if self.prefill_len > 0:
            return self.gen_tokens
        return max(self.gen_tokens - 1, 0)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


_TINY = ModelShape(2, 256, 4, 4, 64, 1024, 1024, rope_base=10000.0, weight_dtype="f32", kv_dtype="f32")
_2B = ModelShape(26, 2048, 16, 4, 128, 8192, 32000, rope_base=10000.0)
_8B = ModelShape(32, 4096, 32, 8, 128, 14336, 128256, rope_base=500000.0)
_11B = ModelShape(40, 4096, 32, 8, 128, 16384, 128256, rope_base=500000.0)
_2B_FP8 = replace(_2B, weight_dtype="fp8")
_8B_FP8 = replace(_8B, weight_dtype="fp8")
_2B_INT8 = replace(_2B, weight_dtype="int8")
_8B_INT8 = replace(_8B, weight_dtype="int8")
_11B_FP8 = replace(_11B, weight_dtype="fp8")
_11B_INT8 = replace(_11B, weight_dtype="int8")

PRESETS = {
    "tiny": Workload("tiny", _TINY, batch=1, prompt_len=32, gen_tokens=64,
                     description="tiny decoder, batch 1, fp32"),
    "2b": Workload("2b", _2B, batch=1, prompt_len=512, gen_tokens=512,
                   description="2B-class dense decoder, batch 1, bf16"),
    "8b": Workload("8b", _8B, batch=1, prompt_len=1024, gen_tokens=256,
                   description="Llama-3-8B-shaped decoder, batch 1, bf16"),
    "2b_long": Workload("2b_long", _2B, batch=1, prefill_len=32768, gen_tokens=128,
                        description="2B decoder, KV pre-filled to 32768 positions"),
    "11b_x56": Workload("11b_x56", _11B, batch=56, prefill_len=4096, gen_tokens=200,
                        description="11B decoder, 56 lockstep sessions, KV at 4096"),
    "11b_x56_fp8": Workload("11b_x56_fp8", _11B_FP8, batch=56, prefill_len=4096, gen_tokens=200,
                            description="11B decoder, 56 lockstep sessions, KV at 4096, E4M3 weights with per-row scales"),
    "11b_x56_int8": Workload("11b_x56_int8", _11B_INT8, batch=56, prefill_len=4096, gen_tokens=200,
                             description="11B decoder, 56 lockstep sessions, KV at 4096, int8 weights with per-row scales"),
    "2b_fp8": Workload("2b_fp8", _2B_FP8, batch=1, prompt_len=512, gen_tokens=512,
                       description="2B decoder, batch 1, E4M3 weights with per-row scales"),
    "8b_fp8": Workload("8b_fp8", _8B_FP8, batch=1, prompt_len=1024, gen_tokens=256,
                       description="Llama-3-8B-shaped decoder, batch 1, E4M3 weights with per-row scales"),
    "2b_int8": Workload("2b_int8", _2B_INT8, batch=1, prompt_len=512, gen_tokens=512,
                        description="2B decoder, batch 1, int8 weights with per-row scales"),
    "8b_int8": Workload("8b_int8", _8B_INT8, batch=1, prompt_len=1024, gen_tokens=256,
                        description="Llama-3-8B-shaped decoder, batch 1, int8 weights with per-row scales"),
}


def get(name: str) -> Workload:
    try:
        return PRESETS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(PRESETS)}") from None

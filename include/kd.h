/*
 * kd.h -- C ABI of the bandwidth-bound decode library (libkd.so) for AMD MI355X (gfx950).
 *
 * One call of kd_step runs one decode step of a pre-norm decoder. The step
 * covers token embedding, then per layer RMSNorm, fused QKV projection, RoPE,
 * KV-cache append, grouped-query attention over the cache, output projection,
 * RMSNorm and the SwiGLU feed-forward block, then the final norm, the LM head
 * and a greedy argmax. All of it runs as one persistent kernel launch with no
 * host round trip between operations.
 *
 * Why this shape:
 *  - Batch-1 decode is bound by memory bandwidth. Every generated token reads
 *    every weight and the whole KV cache, so the weight layout is packed for
 *    aligned, coalesced streaming ("Kog 3000 tok/s real-time inference:
 *    memory-bandwidth optimisation and request-level concurrency trade-offs",
 *    section "three-layer strategy for memory-bandwidth optimisation").
 *  - A single persistent kernel removes kernel-boundary and launch overhead
 *    ("Real-time LLM inference on standard data-centre GPUs (3,000 tokens/s
 *    single request)", section "technical principles").
 *  - Per step the host only feeds the input tokens and takes the output. The
 *    schedule and all memory are fixed before the first call, and nothing is
 *    allocated per step ("Why is real-time AI inference 56x more expensive?
 *    Continuous inference and resident kernels", sections "keep the work
 *    resident on the GPU" and "decide everything ahead of time").
 *
 * Conventions
 *  - Every function returns KD_OK (0) or a negative KD_ERR_* code. The
 *    library never prints, never aborts and never throws across this ABI.
 *  - Pointers documented as "host" are CPU memory. Pointers documented as
 *    "device" are memory of the GPU that was current at kd_init.
 *  - Calls on one handle must not overlap. kd_step launches on the caller's
 *    stream; steps of one handle must be issued on a single stream (or be
 *    otherwise ordered), because the handle owns the step's scratch memory.
 */
#ifndef KD_H_
#define KD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define KD_OK 0
#define KD_ERR_INVALID_ARG (-1) /* NULL pointer, inconsistent or out-of-range configuration value */
#define KD_ERR_UNSUPPORTED (-2) /* valid but not implemented here (e.g. head_dim not 64/128, non-gfx950 GPU) */
#define KD_ERR_NO_DEVICE (-3)   /* no HIP device visible */
#define KD_ERR_OOM (-4)         /* device memory allocation failed */
#define KD_ERR_HIP (-5)         /* a HIP runtime call failed */
#define KD_ERR_LAUNCH (-6)      /* the kernel launch was rejected by the HIP runtime */
#define KD_ERR_SCRATCH (-7)     /* kd_step_noalloc: the handle needs more than its 16 MiB static scratch */

/* ---- sticky device status bits (kd_device_status) ------------------------ */
#define KD_STATUS_TOKEN_RANGE 0x1u  /* an input token was outside [0, vocab): that call wrote nothing */
#define KD_STATUS_POS_OVERFLOW 0x2u /* a position was outside [0, max_seq): the call wrote nothing for it
                                       (kd_generate: it stopped at the step that would overflow) */
#define KD_STATUS_SYNC_TIMEOUT 0x4u /* batch 1: a wait for another workgroup ran past the wait limit; that
                                       call was abandoned (later calls run normally) */
#define KD_STATUS_NAN 0x8u          /* a NaN reached the logits; the argmax skipped it */
#define KD_STATUS_CANCELLED 0x10u   /* the cancel word was set (kd_control): the call was abandoned */

/* ---- kd_control operations ---------------------------------------------- */
#define KD_CTRL_CANCEL 1        /* value != 0 sets the handle's cancel word, 0 clears it */
#define KD_CTRL_WAIT_LIMIT_US 2 /* batch 1: longest wait for another workgroup, in microseconds
                                   (0 .. 60e6; default 2e6) */

/* ---- number formats ---------------------------------------------------------- */
#define KD_DTYPE_F32 0  /* IEEE binary32 */
#define KD_DTYPE_BF16 1 /* bfloat16: the top 16 bits of a binary32 */
/* OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 fraction bits; no infinities; S.1111.111 is
   NaN), weight_dtype only: the projection matrices and the LM head are E4M3 codes with one float32
   scale per output row, and the embedding, the norm gains and the cache are bf16. Cutting the
   bytes of the parameters cuts what every token reads ("17k tokens/sec" page, best practice 2 on
   model quantisation, and its FAQ question 3, which names FP8). */
#define KD_DTYPE_FP8_E4M3 2
/* int8 (two's complement, -128..127), weight_dtype only, laid out like KD_DTYPE_FP8_E4M3: the
   projection matrices and the LM head are int8 codes with one float32 scale per output row (the
   weight is code times scale), and the embedding, the norm gains and the cache are bf16 ("17k
   tokens/sec" page, best practice 2, which names INT8 as the lower precision for the parameters). */
#define KD_DTYPE_INT8 3

/*
 * Model and run configuration, fixed at kd_init.
 *   d_model      = n_q_heads * head_dim is not required, but q_dim = n_q_heads*head_dim
 *                  and d_model must both be multiples of 512 (bf16) / 256 (f32) elements,
 *                  and d_model a multiple of 64.
 *   n_q_heads    must be a multiple of n_kv_heads; G = n_q_heads / n_kv_heads <= 4.
 *   head_dim     64 or 128.
 *   ffn_dim      must be a multiple of 8 (bf16) or 4 (f32) elements.
 *   max_seq      capacity of the KV cache in positions (steps may use positions 0..max_seq-1).
 *   batch        sessions stepped together in lockstep. batch == 1 runs the single persistent
 *                kernel. 2 <= batch <= 64 runs the lockstep-sessions path: the projections become
 *                small-M GEMMs on the matrix cores (with fp8 or int8 weights the GEMMs stream the
 *                one-byte codes, decode them to bf16 in registers and scale each output column by
 *                its row's scale). That path needs bf16, fp8 or int8 weights, a bf16 cache,
 *                head_dim 128, G of 1, 2 or 4, d_model one of 256, 512, 1024, 2048 or 4096, n_q_heads*head_dim
 *                and ffn_dim each split into 2, 4, 7, 8, 14, 16, 28 or 32 runs of 128 after halving
 *                (e.g. 256 times a power of two, or 14336), and d_model, 2*ffn_dim,
 *                (n_q_heads+2*n_kv_heads)*head_dim and vocab multiples of 128.
 *   norm_eps     RMSNorm epsilon (inside the square root).
 *   rope_base    RoPE base: pair (i, i + head_dim/2) turns by position * rope_base^(-2i/head_dim).
 *   prefill_chunk batch 1 only: 0, or 2..128 to set up kd_prefill, which runs a prompt in chunks of
 *                this many positions as small-M GEMMs on the matrix cores (the shape must meet the
 *                lockstep path's conditions above; the
 *                library then holds a second copy of the weights, in bf16 in the matrix cores'
 *                tile layout: for fp8 and int8 models each code times its row's scale, rounded to
 *                bf16 once, so the prefill's results may differ from one-token steps by that rounding).
 *   weight_dtype KD_DTYPE_BF16 or KD_DTYPE_F32, with kv_dtype the same; or KD_DTYPE_FP8_E4M3 or
 *                KD_DTYPE_INT8 with kv_dtype KD_DTYPE_BF16 (at batch 1: head_dim 128, d_model and q_dim multiples
 *                of 1024, ffn_dim a multiple of 8 with ffn_dim/8 >= the GPU's compute units).
 */
typedef struct kd_config {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn_dim;
  int32_t vocab;
  int32_t max_seq;
  int32_t batch;
  float norm_eps;
  float rope_base;
  int32_t weight_dtype;
  int32_t kv_dtype;
  int32_t prefill_chunk;
} kd_config;

/* Host pointers to one layer's tensors, row-major, in weight_dtype (bf16 = uint16 patterns). With
 * KD_DTYPE_FP8_E4M3 (or KD_DTYPE_INT8) the seven matrices are one-byte E4M3 (or int8) codes, the
 * gains bf16, and the s_* arrays hold the float32 scale of each output row of the matching matrix:
 * the weight at (r, c) is the code's value times row r's scale. For other weight types the s_*
 * pointers are ignored. */
typedef struct kd_layer_weights {
  const void* attn_norm; /* [d_model] */
  const void* wq;        /* [n_q_heads*head_dim, d_model] */
  const void* wk;        /* [n_kv_heads*head_dim, d_model] */
  const void* wv;        /* [n_kv_heads*head_dim, d_model] */
  const void* wo;        /* [d_model, n_q_heads*head_dim] */
  const void* ffn_norm;  /* [d_model] */
  const void* w_gate;    /* [ffn_dim, d_model] */
  const void* w_up;      /* [ffn_dim, d_model] */
  const void* w_down;    /* [d_model, ffn_dim] */
  const float* s_wq;     /* [n_q_heads*head_dim]  fp8 and int8 only: row scales */
  const float* s_wk;     /* [n_kv_heads*head_dim] */
  const float* s_wv;     /* [n_kv_heads*head_dim] */
  const float* s_wo;     /* [d_model] */
  const float* s_gate;   /* [ffn_dim] */
  const float* s_up;     /* [ffn_dim] */
  const float* s_down;   /* [d_model] */
} kd_layer_weights;

/* Host pointers to all weights.  layers points to n_layers entries. */
typedef struct kd_weights {
  const void* embed;              /* [vocab, d_model] */
  const kd_layer_weights* layers; /* [n_layers] */
  const void* final_norm;         /* [d_model] */
  const void* lm_head;            /* [vocab, d_model] (separate from embed) */
  const float* s_lm_head;         /* [vocab] fp8 and int8 only: row scales of lm_head */
} kd_weights;

typedef struct kd_handle kd_handle;

/*
 * Validate cfg, pack the weights into library-owned device memory on the
 * current HIP device, and allocate every buffer a step needs. The schedule and
 * every address are fixed here, before the first step, so no step plans or
 * allocates anything ("Why is real-time AI inference 56x more expensive?",
 * section "decide everything ahead of time").
 *   cfg  host, read only: the model and run configuration (see kd_config).
 *   w    host, read only: canonical row-major weights in cfg->weight_dtype. They
 *        may be freed as soon as kd_init returns.
 *   out  host: receives the handle, which the library owns until kd_destroy.
 * Synchronous. Returns KD_OK, or KD_ERR_INVALID_ARG (NULL pointer, inconsistent
 * cfg), KD_ERR_UNSUPPORTED (a shape or GPU this library does not handle),
 * KD_ERR_NO_DEVICE, KD_ERR_OOM or KD_ERR_HIP; on error *out stays NULL and no
 * device memory is kept.
 */
int kd_init(const kd_config* cfg, const kd_weights* w, kd_handle** out);

/*
 * Layout of the caller-owned KV cache for cfg. A session's cache is allocated
 * once for its whole length and stays in place for the session: it is read at
 * every step and cannot be freed or moved out between steps ("17k tokens/sec"
 * page, best practice 3 on pre-allocated contiguous KV memory; "Why is real-time
 * AI inference 56x more expensive?", section "why it is so expensive").
 * The cache is one device buffer of kv_dtype values indexed
 * [layer][slot][session][kv_head][position][dim]: slot 0 holds K after RoPE,
 * slot 1 holds V.
 *   cfg      host, read only.
 *   bytes    host: receives the buffer size in bytes.
 *   strides  host array of 6: receives the element strides of the six indices (dim stride
 *            is 1); the position extent is max_seq + 7 rounded up to a multiple of 16.
 * Host-only computation, no device needed. Returns KD_OK or KD_ERR_INVALID_ARG.
 */
int kd_kv_layout(const kd_config* cfg, size_t* bytes, size_t strides[6]);

/*
 * Enqueue one decode step on `stream` (a hipStream_t; NULL = the null stream) and return.
 * The whole step runs on the GPU with no host round trip between operations: per step the
 * host only hands over the input and takes the output ("Why is real-time AI inference 56x
 * more expensive?", section "keep the work resident on the GPU"; "Real-time LLM inference
 * on standard data-centre GPUs (3,000 tokens/s single request)", section "technical
 * principles": one resident kernel, no launch or kernel-boundary gaps).
 *   tokens    device int32[batch], in/out: read as this step's input ids, overwritten with the
 *             greedy next ids (lowest index on ties).
 *   positions device int32[batch], in/out: read as the position p of each input token (the
 *             step attends over cached positions 0..p and writes K,V at p), then incremented.
 *   kv        device buffer laid out as kd_kv_layout reports; read and written.
 *   logits    device float[batch, vocab] written with this step's logits, or NULL to skip.
 * All four are caller-owned. No allocation, no synchronisation and no host<->device copy
 * happen here. Returns KD_OK, KD_ERR_INVALID_ARG (NULL handle or buffer), KD_ERR_HIP or
 * KD_ERR_LAUNCH. Device-detected errors set sticky status bits (kd_device_status):
 * invalid input leaves every output unchanged; a timed-out or cancelled step stops where it
 * was (tokens and positions unchanged, logits possibly in part). Each call is its own: the
 * next one runs normally.
 * Batch 1 launches one workgroup per compute unit and relies on all of them being resident
 * together (each needs most of a CU's local memory, so on an otherwise idle GPU they are).
 * If another kernel holds compute units, the waits between workgroups end at the wait limit
 * (KD_CTRL_WAIT_LIMIT_US) with KD_STATUS_SYNC_TIMEOUT instead of hanging.
 */
int kd_step(kd_handle* h, int32_t* tokens, int32_t* positions, void* kv, float* logits, void* stream);

/*
 * kd_step for callers that cannot allocate device memory at the time of the call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation). Same arguments,
 * results, ownership and errors as kd_step at batch 1, bit for bit; it allocates nothing and
 * calls no allocating routine. The step's exchange memory (the words workgroups pass between
 * phases, and the abort word) is not the handle's but one static device array of 16 MiB per GPU,
 * set up by kd_init and held until the process ends. The caller still passes inputs and outputs.
 *   Returns KD_ERR_UNSUPPORTED for batch > 1, and KD_ERR_SCRATCH (before launching anything) when
 *   the model's exchange memory exceeds 16 MiB. On a 256-CU MI355X every shape kd_init accepts
 *   fits (at most 12.3 MiB, at d_model 4096 with 4 q heads per kv head; the 2B and Llama-3-8B
 *   shapes need 8.1 and 12.2 MiB); the check guards GPUs with more compute units.
 * Every call on one GPU shares that GPU's array, so calls that overlap on one GPU race, also
 * from different handles: issue them in order (one stream, or synchronised). Nothing in the array
 * needs clearing between calls: every call tags its words with tags no earlier call on that GPU
 * used (the array is cleared, by a kernel on the stream, only when the tags start over).
 */
int kd_step_noalloc(kd_handle* h, int32_t* tokens, int32_t* positions, void* kv, float* logits, void* stream);

/*
 * Run a prompt through the decoder on the matrix cores (batch 1, a handle made with
 * prefill_chunk > 0) and return: the step before decoding, and what sets the time to the first
 * token ("Kog 3000 tok/s real-time inference", section "deployable parameters and monitoring
 * checklist", which tracks time to first token beside the time between tokens). The n prompt
 * tokens go in at positions p .. p+n-1, where p = positions[0] on the device (0 for a fresh
 * session, or the end of an earlier context), in chunks of prefill_chunk positions. Each chunk
 * is one pass of the lockstep kernels with its positions as the rows of the small-M GEMMs; each
 * row appends its K and V and attends over positions 0 .. its own, as one-token steps would.
 *   prompt    device int32[n], read only.
 *   tokens    device int32[1]: receives the greedy token after the last prompt position.
 *   positions device int32[1], in/out: read as p, then set to p + n.
 *   kv        the caller's cache (kd_kv_layout), read and written.
 *   logits    device float[vocab] receiving the logits of the last prompt position, or NULL.
 * Enqueued on `stream`; no allocation, no synchronisation. Returns KD_OK, KD_ERR_INVALID_ARG
 * (NULL pointer, n < 1), KD_ERR_UNSUPPORTED (no prefill set up at kd_init) or KD_ERR_LAUNCH.
 * A chunk whose tokens or positions are out of range sets the status bits and writes nothing
 * (its positions stay unfilled); the outputs are written only when the last chunk ran.
 */
int kd_prefill(kd_handle* h, const int32_t* prompt, int32_t n, int32_t* tokens, int32_t* positions, void* kv,
               float* logits, void* stream);

/*
 * Run n_steps greedy decode steps as one persistent launch (batch 1) and return: each step is
 * fed the token the step before chose, on the device, and the workgroups stay resident from
 * one step to the next; the host only takes the output ("Why is real-time AI inference 56x
 * more expensive?", section "keep the work resident on the GPU": the program stays on the
 * GPU and its threads do not exit between ticks). For batch > 1 the n_steps ticks' kernel
 * sequences are enqueued back to back on the stream, with the same device-side feedback.
 *   tokens, positions, kv  as for kd_step; after the call they hold the last step's next
 *             tokens and positions + n_steps.
 *   out_tokens device int32[n_steps][batch], or NULL: the greedy token of every step.
 *   logits    device float[n_steps][batch][vocab], or NULL: the logits of every step.
 *   progress  device (or host-pinned, device-visible) uint32, or NULL: set to the number of
 *             completed steps after each step, written through to memory after that step's
 *             outputs, so the host can poll it while the call runs.
 * Same errors and ownership as kd_step, plus KD_ERR_INVALID_ARG for n_steps < 1. A step
 * whose position would reach max_seq is not run (KD_STATUS_POS_OVERFLOW); a timed-out or
 * cancelled step ends the call (the outputs of earlier steps stay).
 */
int kd_generate(kd_handle* h, int32_t n_steps, int32_t* tokens, int32_t* positions, void* kv, int32_t* out_tokens,
                float* logits, uint32_t* progress, void* stream);

/*
 * Read (and optionally clear) the sticky KD_STATUS_* bits. Synchronises with the device.
 * A late or abandoned step must be visible to the caller, not hidden in an average
 * ("Why is real-time AI inference 56x more expensive?", section "why it is so expensive":
 * tokens/s and mean latency can look fine while one session stutters).
 *   bits   host: receives the bits.   clear  nonzero: reset them to 0 afterwards.
 * Returns KD_OK, KD_ERR_INVALID_ARG or KD_ERR_HIP. The caller's current device is kept.
 */
int kd_device_status(kd_handle* h, uint32_t* bits, int clear);

/*
 * Host controls of a handle (no passage of the pages defines these; they are this library's
 * failure handling).
 *   KD_CTRL_CANCEL         value != 0 sets the cancel word: a call that starts while it is set,
 *                          or that is waiting on another workgroup when it is set, stops with
 *                          KD_STATUS_CANCELLED. value 0 clears it. Synchronous; may be called
 *                          while a call runs on another stream (it uses a stream of its own).
 *   KD_CTRL_WAIT_LIMIT_US  batch 1: longest wait for another workgroup before the call gives up
 *                          with KD_STATUS_SYNC_TIMEOUT; applies to later calls.
 * Returns KD_OK, KD_ERR_INVALID_ARG (unknown op, value out of range) or KD_ERR_HIP.
 */
int kd_control(kd_handle* h, int32_t op, int64_t value);

/* Free everything the library owns. NULL is accepted. Caller buffers are never touched.
 * Synchronises with the device. (No passage of the pages defines teardown.) */
void kd_destroy(kd_handle* h);

/* Static description of a status code. (No passage of the pages defines it.) */
const char* kd_strerror(int code);

/*
 * Step tracing, for measurement (batch 1 and at most 40 layers; KD_ERR_UNSUPPORTED otherwise).
 * With dev_buf non-NULL, every later kd_step records 64-bit timestamps of the GPU's 100 MHz
 * constant clock at its phase boundaries (held in LDS during the step, written out at its end,
 * so recording them does not delay the step's memory waits): workgroup w uses
 * dev_buf[w * stride .. (w + 1) * stride).  Slot 0 is the step start, slot 1 the end of setup,
 * slots 2 + 24*l + e (e < 24) the phase boundaries of layer l, and the last 4 slots the final
 * norm, LM head and argmax.  dev_buf is device memory of at least stride * workgroups words,
 * owned by the caller; NULL turns tracing off.  *stride (optional) receives the stride.
 * Returns KD_ERR_INVALID_ARG if the buffer is too small.
 */
int kd_trace(kd_handle* h, uint64_t* dev_buf, int64_t words, int64_t* stride);

/*
 * Measurement aid (no passage of the pages defines it): enqueue one plain read of `bytes` bytes
 * of device memory at buf (16-byte aligned, a multiple of 16 bytes) on `stream`, with 16-byte
 * non-temporal loads over the whole GPU, and return. Timed by the caller, it gives the
 * sustained read rate of this GPU's HBM that the decode kernels are compared with.
 * Returns KD_OK, KD_ERR_INVALID_ARG or KD_ERR_LAUNCH.
 */
int kd_stream_read(const void* buf, size_t bytes, void* stream);

/*
 * Facts about an initialised handle (for measurement and tests).
 *   info[0] workgroups in the persistent grid      info[1] threads per workgroup
 *   info[2] packed weight bytes on the device      info[3] LDS bytes per workgroup
 *   info[4] ring depth (1 KB packets per compute wave)
 *   info[5] prefill chunk (positions per kd_prefill pass; 0: kd_prefill not set up)
 * For batch > 1: info[0] = 0 (no persistent grid), info[1] threads per GEMM workgroup,
 *   info[2] weight bytes on the device, info[5] kernels one kd_step enqueues,
 *   info[6] split-K factors of the QKV / O / gate-up / down GEMMs (one byte each, low first),
 *   info[7] attention chunk length in positions.
 */
int kd_get_info(kd_handle* h, int64_t info[8]);

#ifdef __cplusplus
}
#endif
#endif /* KD_H_ */

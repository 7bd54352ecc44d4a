// kd_batch_host.h -- host side of the B > 1 (lockstep sessions) path behind kd_init / kd_step.
//
// Everything is fixed at init: weight layout, split-K factors, attention chunking and every
// buffer ("Why is real-time AI inference 56x more expensive?", section "decide everything ahead
// of time"). A tick then only enqueues the fixed kernel sequence of kd_batch.h on the caller's
// stream: no allocation, no synchronisation, no host-side decision that depends on device data.
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "kd.h"
#include "kd_batch.h"

namespace kd {
namespace bt {

// One projection: W[N][K] (bf16 in the tile layout of tile_pack_kernel, or one-byte codes in that of
// tile_pack_q8_kernel) times the activation block, split over KS K-ranges.
struct Gemm {
  int N = 0, K = 0, KS = 1;
};

struct BatchState {
  int B = 0, L = 0, d = 0, hq = 0, hkv = 0, hd = 0, F = 0, V = 0, S = 0, max_seq = 0;
  int nqkv = 0, qdim = 0, lda = 0;  // lda: row stride of the hi/lo activation blocks
  int CH = 0, NCmax = 0;            // attention chunk length and most chunks per (session, kv head)
  int MT = 4;                       // 16-row tiles of the activation blocks: 4 (B <= 64) or 8 (B <= 128, prefill)
  float eps = 0.f;
  Gemm g_qkv, g_o, g_gu, g_d, g_lm;
  size_t layer_elems = 0;           // per-layer weight elements: qkv, o, gate/up (interleaved), down
  uint16_t* w = nullptr;            // L layers, then the LM head (bf16 tiles)
  int q = 0;                        // session weights: 0 bf16 (w), 1 E4M3 or 2 int8 codes (w8, wscale)
  uint8_t* w8 = nullptr;            // one-byte tiles, at the same element offsets as w
  float* wscale = nullptr;          // row scales in packed row order: per layer qkv, o, gate/up, down; then the LM head
  size_t srows = 0;                 // scale rows per layer
  uint16_t* embed = nullptr;        // [V][d]
  uint16_t* norms = nullptr;        // [L][2][d] then [d]
  float2* rope = nullptr;           // [S][hd/2]
  float* X = nullptr;               // [B][d] residual stream
  uint16_t* Ahi = nullptr;          // [64][lda] activation block, hi halves (rows >= B stay zero)
  uint16_t* Alo = nullptr;          // [64][lda] lo halves
  uint16_t* A2hi = nullptr;         // [64][lda] input of the down projection when gate/up writes SiLU*up itself
  uint16_t* A2lo = nullptr;
  float* P = nullptr;               // split-K partial sums [KS][B][N]
  float* Qs = nullptr;              // [B][hq * hd] rotated, scaled queries
  float* part = nullptr;            // attention chunk partials [B][hq][NCmax][hd + 2]
  float* logits = nullptr;          // [B][V] when the caller passes none
  int32_t* rows_tok = nullptr;      // prefill: the chunk's tokens, then its greedy tokens [B]
  int32_t* rows_pos = nullptr;      // prefill: the chunk's positions [B]
  size_t w_qkv = 0, w_o = 0, w_gu = 0, w_d = 0, w_lm = 0;  // element offsets inside a layer / the blob
};

// Split-K factor of a GEMM: the power of two whose estimated time is least, over K ranges of
// 2, 4, 7, 8, 14, 16, 28 or 32 chunks of 128 K (the unrolled kernel variants; 7, 14 and 28 take
// K = 14336, the Llama-3-8B FFN width). The estimate: the weight
// stream at about 6.5 TB/s, or, when there are too few workgroups for that, rounds of one
// workgroup per CU each paying a fixed start-up latency and streaming at a single CU's rate;
// plus writing and reading back the fp32 partial sums. Returns -1 if no split is valid.
inline bool chunks_ok(int nch) {
  return nch == 2 || nch == 4 || nch == 7 || nch == 8 || nch == 14 || nch == 16 || nch == 28 || nch == 32;
}
inline int pick_ks(int N, int K, int B, int nwg) {
  const double bw = 6.5e12, bw_cu = 50e9, start = 3e-6;
  const int nch_all = K / kKC;
  int best = -1;
  double best_t = 1e30;
  for (int ks = 1; ks <= nch_all && nch_all % ks == 0; ks *= 2) {
    const int nch = nch_all / ks;
    if (!chunks_ok(nch)) continue;
    const int64_t units = (int64_t)(N / kNB) * ks;
    const double rounds = (double)((units + nwg - 1) / nwg);
    const double per_unit = start + nch * (double)kNB * kKC * 2.0 / bw_cu;
    const double t = std::max(2.0 * N * K / bw, rounds * per_unit) + 2.0 * ks * B * (double)N * 4.0 / bw;
    if (t < best_t) {
      best_t = t;
      best = ks;
    }
  }
  return best;
}
typedef void (*GemmFn)(const uint16_t*, int, int, const uint16_t*, const uint16_t*, int, float*, int, int, const uint32_t*,
                       uint16_t*, uint16_t*, const float*);
template <bool SILU, int MT, int Q>
inline GemmFn gemm_for_mt(int nch) {
  switch (nch) {
    case 2: return gemm_kernel<2, SILU, MT, Q>;
    case 4: return gemm_kernel<4, SILU, MT, Q>;
    case 7: return gemm_kernel<7, SILU, MT, Q>;
    case 8: return gemm_kernel<8, SILU, MT, Q>;
    case 14: return gemm_kernel<14, SILU, MT, Q>;
    case 16: return gemm_kernel<16, SILU, MT, Q>;
    case 28: return gemm_kernel<28, SILU, MT, Q>;
    case 32: return gemm_kernel<32, SILU, MT, Q>;
    default: return nullptr;
  }
}
// mt: 16-row tiles of the activation block (4 for up to 64 rows, 8 for up to 128); q: weight
// format (0 bf16, 1 E4M3, 2 int8; one-byte formats with 4 tiles only)
template <bool SILU>
inline GemmFn gemm_for(int nch, int mt, int q) {
  if (mt == 8) return q == 0 ? gemm_for_mt<SILU, 8, 0>(nch) : nullptr;
  return q == 0 ? gemm_for_mt<SILU, 4, 0>(nch) : q == 1 ? gemm_for_mt<SILU, 4, 1>(nch) : gemm_for_mt<SILU, 4, 2>(nch);
}
// gate/up without a K split writes SiLU(gate) * up itself (no silu_kernel launch)
inline bool fused_silu(const BatchState& st) { return st.g_gu.KS == 1; }

typedef void (*AttFn)(const float*, const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, int, int, int, float*,
                      const uint32_t*);
// G = 3 cannot occur: n_q_heads * 128 would be a multiple of 3, never 256 times a power of two.
template <int CHUNK>
inline AttFn att_for_g(int G) {
  switch (G) {
    case 1: return attention_kernel<1, CHUNK>;
    case 2: return attention_kernel<2, CHUNK>;
    case 4: return attention_kernel<4, CHUNK>;
    default: return nullptr;
  }
}
inline AttFn att_for(int G, int chunk) { return chunk == 2 * kChunk ? att_for_g<2 * kChunk>(G) : att_for_g<kChunk>(G); }
typedef void (*PrefillAttFn)(const float*, const uint16_t*, int64_t, int64_t, const int32_t*, int, int, int, float*,
                             const uint32_t*);
inline PrefillAttFn prefill_att_for(int G) {
  switch (G) {
    case 1: return prefill_attention_kernel<1>;
    case 2: return prefill_attention_kernel<2>;
    case 4: return prefill_attention_kernel<4>;
    default: return nullptr;
  }
}

// max_rows: kM for session handles, kMPrefill for the prefill engine. Weights may be bf16, or fp8
// or int8 codes with row scales: session handles stream the codes, the prefill engine keeps its
// own copy decoded to bf16.
inline int batch_check(const kd_config* c, int max_rows = kM) {
  if (c->batch < 2 || c->batch > max_rows) return KD_ERR_UNSUPPORTED;
  const bool q8 = c->weight_dtype == KD_DTYPE_FP8_E4M3 || c->weight_dtype == KD_DTYPE_INT8;
  if ((c->weight_dtype != KD_DTYPE_BF16 && !q8) || c->kv_dtype != KD_DTYPE_BF16) return KD_ERR_UNSUPPORTED;
  if (c->head_dim != 128) return KD_ERR_UNSUPPORTED;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return KD_ERR_UNSUPPORTED;
  const int64_t qdim = (int64_t)c->n_q_heads * c->head_dim, nqkv = qdim + 2LL * c->n_kv_heads * c->head_dim;
  // every GEMM's K must split into ranges of 2, 4, 7, 8, 14, 16, 28 or 32 chunks of 128
  for (int64_t K : {(int64_t)c->d_model, qdim, (int64_t)c->ffn_dim}) {
    if (K % kKC) return KD_ERR_UNSUPPORTED;
    int64_t nch = K / kKC;
    while (nch > 32 && nch % 2 == 0) nch /= 2;
    if (!chunks_ok((int)nch)) return KD_ERR_UNSUPPORTED;
  }
  if (!chunks_ok(c->d_model / kKC)) return KD_ERR_UNSUPPORTED;  // the LM head runs unsplit; d <= 4096
  if (nqkv % kNB || c->d_model % kNB || c->vocab % kNB || (2LL * c->ffn_dim) % kNB) return KD_ERR_UNSUPPORTED;
  return KD_OK;
}

inline void batch_free(BatchState& st) {
  void* ptrs[] = {st.w,  st.embed, st.norms, st.rope, st.X,      st.Ahi,      st.Alo,      st.A2hi,
                  st.A2lo, st.P,   st.Qs,    st.part, st.logits, st.rows_tok, st.rows_pos, st.w8, st.wscale};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  st = BatchState{};
}

#define KD_BT_TRY(expr)             \
  do {                              \
    if ((expr) != hipSuccess) {     \
      batch_free(st);               \
      return KD_ERR_HIP;            \
    }                               \
  } while (0)
#define KD_BT_ALLOC(ptr, bytes)                                        \
  do {                                                                 \
    if (hipMalloc(&(ptr), (bytes)) != hipSuccess) {                    \
      batch_free(st);                                                  \
      return KD_ERR_OOM;                                               \
    }                                                                  \
  } while (0)

// sessions: a lockstep-sessions handle (each row a session); false for the prefill engine, whose
// rows are positions of one session.
inline int batch_init(const kd_config* c, const kd_weights* w, int nwg, bool sessions, BatchState& st) {
  st = BatchState{};
  st.B = c->batch; st.MT = c->batch > kM ? 8 : 4; st.L = c->n_layers; st.d = c->d_model; st.hq = c->n_q_heads; st.hkv = c->n_kv_heads;
  st.hd = c->head_dim; st.F = c->ffn_dim; st.V = c->vocab; st.max_seq = c->max_seq; st.eps = c->norm_eps;
  st.S = (int)((((int64_t)c->max_seq + 7 + 15) / 16) * 16);
  st.qdim = st.hq * st.hd;
  st.nqkv = st.qdim + 2 * st.hkv * st.hd;
  st.lda = std::max({st.d, st.qdim, st.F});
  st.g_qkv = {st.nqkv, st.d, pick_ks(st.nqkv, st.d, st.B, nwg)};
  st.g_o = {st.d, st.qdim, pick_ks(st.d, st.qdim, st.B, nwg)};
  st.g_gu = {2 * st.F, st.d, pick_ks(2 * st.F, st.d, st.B, nwg)};
  st.g_d = {st.d, st.F, pick_ks(st.d, st.F, st.B, nwg)};
  for (const Gemm* g : {&st.g_qkv, &st.g_o, &st.g_gu, &st.g_d})
    if (g->KS < 1) return KD_ERR_UNSUPPORTED;
  st.g_lm = {st.V, st.d, 1};  // written straight into the logits: no split
  // attention: chunks of 512 positions, or 1024 for session batches whose sessions and kv heads
  // alone give a workgroup per compute unit (the merge then has half the chunks to combine); the
  // prefill engine's chunks of 256 positions serve every row of a pass at once
  st.CH = !sessions ? kChunkPrefill : (int64_t)st.B * st.hkv >= nwg ? 2 * kChunk : kChunk;
  st.NCmax = (st.max_seq + st.CH - 1) / st.CH;

  const size_t d = st.d;
  st.w_qkv = 0;
  st.w_o = st.w_qkv + (size_t)st.nqkv * d;
  st.w_gu = st.w_o + d * st.qdim;
  st.w_d = st.w_gu + 2 * (size_t)st.F * d;
  st.layer_elems = st.w_d + d * st.F;
  st.w_lm = (size_t)st.L * st.layer_elems;
  const size_t blob = st.w_lm + (size_t)st.V * d;
  size_t p_elems = 0;
  for (const Gemm* g : {&st.g_qkv, &st.g_o, &st.g_gu, &st.g_d})
    p_elems = std::max(p_elems, (size_t)g->KS * st.B * g->N);

  // session handles of fp8 and int8 models stream the codes (one byte per weight) and scale each
  // output column; the prefill engine keeps a bf16 copy
  const bool q8w = c->weight_dtype != KD_DTYPE_BF16;
  st.q = sessions && q8w ? (c->weight_dtype == KD_DTYPE_INT8 ? 2 : 1) : 0;
  st.srows = (size_t)st.nqkv + d + 2 * (size_t)st.F + d;
  if (st.q) {
    KD_BT_ALLOC(st.w8, blob);
    KD_BT_ALLOC(st.wscale, ((size_t)st.L * st.srows + st.V) * 4);
  } else {
    KD_BT_ALLOC(st.w, blob * 2);
  }
  KD_BT_ALLOC(st.embed, (size_t)st.V * d * 2);
  KD_BT_ALLOC(st.norms, (size_t)(2 * st.L + 1) * d * 2);
  KD_BT_ALLOC(st.rope, (size_t)st.S * (st.hd / 2) * sizeof(float2));
  KD_BT_ALLOC(st.X, (size_t)st.B * d * 4);
  const size_t rows = (size_t)16 * st.MT;
  KD_BT_ALLOC(st.Ahi, rows * st.lda * 2);
  KD_BT_ALLOC(st.Alo, rows * st.lda * 2);
  KD_BT_ALLOC(st.A2hi, rows * st.lda * 2);
  KD_BT_ALLOC(st.A2lo, rows * st.lda * 2);
  KD_BT_ALLOC(st.P, p_elems * 4);
  KD_BT_ALLOC(st.Qs, (size_t)st.B * st.qdim * 4);
  KD_BT_ALLOC(st.part, (size_t)st.B * st.hq * st.NCmax * (st.hd + 2) * 4);
  KD_BT_ALLOC(st.logits, (size_t)st.B * st.V * 4);
  KD_BT_ALLOC(st.rows_tok, (size_t)st.B * 4);
  KD_BT_ALLOC(st.rows_pos, (size_t)st.B * 4);
  KD_BT_TRY(hipMemset(st.Ahi, 0, rows * st.lda * 2));  // padding rows stay zero for good
  KD_BT_TRY(hipMemset(st.Alo, 0, rows * st.lda * 2));
  KD_BT_TRY(hipMemset(st.A2hi, 0, rows * st.lda * 2));
  KD_BT_TRY(hipMemset(st.A2lo, 0, rows * st.lda * 2));

  // Every matrix goes row-major into a staging buffer, then tile_pack_kernel (tile_pack_q8_kernel
  // for the codes a session handle streams) writes it into the blob in the tile layout the GEMM
  // streams. For the prefill engine of an fp8 or int8 model the codes and row scales land first,
  // and dequant_rows_kernel writes code x scale into the staging buffer as bf16.
  const int int8 = c->weight_dtype == KD_DTYPE_INT8;
  const size_t row = d * 2;
  uint16_t* stage = nullptr;
  uint8_t* qcodes = nullptr;
  float* qscale = nullptr;
  {
    size_t most = std::max({(size_t)st.nqkv * d, d * st.qdim, 2 * (size_t)st.F * d, (size_t)st.V * d});
    size_t most_rows = std::max({(size_t)st.nqkv, d, (size_t)st.F, (size_t)st.V});
    if ((!st.q && hipMalloc(&stage, most * 2) != hipSuccess) ||
        (q8w && (hipMalloc(&qcodes, most) != hipSuccess || hipMalloc(&qscale, most_rows * 4) != hipSuccess))) {
      if (stage) (void)hipFree(stage);
      if (qcodes) (void)hipFree(qcodes);
      batch_free(st);
      return KD_ERR_OOM;
    }
  }
#define KD_BT_STAGE_TRY(expr)   \
  do {                          \
    if ((expr) != hipSuccess) { \
      (void)hipFree(stage);     \
      if (qcodes) (void)hipFree(qcodes); \
      if (qscale) (void)hipFree(qscale); \
      batch_free(st);           \
      return KD_ERR_HIP;        \
    }                           \
  } while (0)
  // codes[rows][cols] and their row scales (host) -> bf16 rows of dst, row r at
  // (r / bin) * bout + boff + r % bin (the gate/up interleave; bin = rows keeps the order)
  auto put_q8 = [&](uint16_t* dst, const void* codes, const float* scales, int rows, int cols, int bin, int bout,
                    int boff) {
    hipError_t e = hipMemcpy(qcodes, codes, (size_t)rows * cols, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(qscale, scales, (size_t)rows * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)rows * cols;
    hipLaunchKernelGGL(dequant_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, 0, (const uint8_t*)qcodes,
                       (const float*)qscale, rows, cols, int8, bin, bout, boff, dst);
    return hipGetLastError();
  };
  auto pack = [&](uint16_t* dst, int N, int K) {
    const int64_t pieces = (int64_t)N * K / 8;
    hipLaunchKernelGGL(tile_pack_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, 0, (const uint16_t*)stage,
                       dst, N, K);
    return hipDeviceSynchronize();  // the next copy reuses the staging buffer
  };
  // session handles of one-byte models: codes row-major into qcodes, then tile_pack_q8_kernel; the
  // row scales gathered on the host in packed row order
  std::vector<float> hs(st.q ? (size_t)st.L * st.srows + st.V : 0);
  auto pack_q8 = [&](size_t e, int N, int K) {
    const int64_t pieces = (int64_t)N * K / 16;
    hipLaunchKernelGGL(tile_pack_q8_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, 0, (const uint8_t*)qcodes,
                       st.w8 + e, N, K);
    return hipDeviceSynchronize();  // the next copy reuses the staging buffer
  };
  // rows [0, rows) of a host matrix [rows][cols] (bf16 patterns, or codes with row scales) into
  // rows (r / bin) * bout + boff + r % bin of the staged matrix whose row 0 is row r0 of the packed
  // one (bin = rows: in order)
  auto stage_rows = [&](size_t r0, const void* host, const float* hscale, int rows, int cols, int bin, int bout,
                        int boff, size_t srow0) -> hipError_t {
    const size_t nblk = (size_t)rows / bin, eb = st.q ? 1 : 2;  // bytes per staged element
    if (!q8w || st.q) {
      uint8_t* dst = (st.q ? (uint8_t*)qcodes + r0 * cols : (uint8_t*)(stage + r0 * cols)) + (size_t)boff * cols * eb;
      const hipError_t e = bin == rows ? hipMemcpy(dst, host, (size_t)rows * cols * eb, hipMemcpyHostToDevice)
                                       : hipMemcpy2D(dst, (size_t)bout * cols * eb, host, (size_t)bin * cols * eb,
                                                     (size_t)bin * cols * eb, nblk, hipMemcpyHostToDevice);
      if (e != hipSuccess || !st.q) return e;
      for (int r = 0; r < rows; ++r) hs[srow0 + r0 + (size_t)(r / bin) * bout + boff + r % bin] = hscale[r];
      return hipSuccess;
    }
    return put_q8(stage + r0 * cols, host, hscale, rows, cols, bin, bout, boff);  // prefill engine: decoded to bf16
  };
  auto finish = [&](size_t e, int N, int K) { return st.q ? pack_q8(e, N, K) : pack(st.w + e, N, K); };
  for (int l = 0; l < st.L; ++l) {
    const kd_layer_weights& lw = w->layers[l];
    const size_t lay = (size_t)l * st.layer_elems, srl = (size_t)l * st.srows;
    const int kvdim = st.hkv * st.hd;
    KD_BT_STAGE_TRY(stage_rows(0, lw.wq, lw.s_wq, st.qdim, st.d, st.qdim, st.qdim, 0, srl));
    KD_BT_STAGE_TRY(stage_rows(st.qdim, lw.wk, lw.s_wk, kvdim, st.d, kvdim, kvdim, 0, srl));
    KD_BT_STAGE_TRY(stage_rows((size_t)st.qdim + kvdim, lw.wv, lw.s_wv, kvdim, st.d, kvdim, kvdim, 0, srl));
    KD_BT_STAGE_TRY(finish(lay + st.w_qkv, st.nqkv, st.d));
    KD_BT_STAGE_TRY(stage_rows(0, lw.wo, lw.s_wo, st.d, st.qdim, st.d, st.d, 0, srl + st.nqkv));
    KD_BT_STAGE_TRY(finish(lay + st.w_o, st.d, st.qdim));
    // gate/up interleaved in blocks of 32 rows: rows [64j, 64j+32) = gate rows [32j, 32j+32),
    // rows [64j+32, 64j+64) = the matching up rows, so every GEMM tile holds whole pairs
    KD_BT_STAGE_TRY(stage_rows(0, lw.w_gate, lw.s_gate, st.F, st.d, 32, 64, 0, srl + st.nqkv + d));
    KD_BT_STAGE_TRY(stage_rows(0, lw.w_up, lw.s_up, st.F, st.d, 32, 64, 32, srl + st.nqkv + d));
    KD_BT_STAGE_TRY(finish(lay + st.w_gu, 2 * st.F, st.d));
    KD_BT_STAGE_TRY(stage_rows(0, lw.w_down, lw.s_down, st.d, st.F, st.d, st.d, 0, srl + st.nqkv + d + 2 * (size_t)st.F));
    KD_BT_STAGE_TRY(finish(lay + st.w_d, st.d, st.F));
    KD_BT_STAGE_TRY(hipMemcpy(st.norms + (size_t)(2 * l) * d, lw.attn_norm, row, hipMemcpyHostToDevice));
    KD_BT_STAGE_TRY(hipMemcpy(st.norms + (size_t)(2 * l + 1) * d, lw.ffn_norm, row, hipMemcpyHostToDevice));
  }
  KD_BT_STAGE_TRY(stage_rows(0, w->lm_head, w->s_lm_head, st.V, st.d, st.V, st.V, 0, (size_t)st.L * st.srows));
  KD_BT_STAGE_TRY(finish(st.w_lm, st.V, st.d));
  if (st.q) KD_BT_STAGE_TRY(hipMemcpy(st.wscale, hs.data(), hs.size() * sizeof(float), hipMemcpyHostToDevice));
#undef KD_BT_STAGE_TRY
  (void)hipFree(stage);
  if (qcodes) (void)hipFree(qcodes);
  if (qscale) (void)hipFree(qscale);
  KD_BT_TRY(hipMemcpy(st.norms + (size_t)(2 * st.L) * d, w->final_norm, row, hipMemcpyHostToDevice));
  KD_BT_TRY(hipMemcpy(st.embed, w->embed, (size_t)st.V * row, hipMemcpyHostToDevice));
  {
    // RoPE: pair (i, i + hd/2) turns by position * base^(-2i/hd); angles, cos and sin in float64
    const int half = st.hd / 2;
    std::vector<double> theta(half);
    for (int i = 0; i < half; ++i) theta[i] = std::pow((double)c->rope_base, -2.0 * (double)i / (double)st.hd);
    std::vector<float2> tab((size_t)st.S * half);
    for (int64_t pos = 0; pos < st.S; ++pos)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)pos * theta[i];
        tab[(size_t)pos * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
      }
    KD_BT_TRY(hipMemcpy(st.rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice));
  }
  KD_BT_TRY(hipDeviceSynchronize());
  return KD_OK;
}

// Kernels one tick enqueues: check, embed+norm, 10 per layer, LM head, argmax.
inline int batch_kernels_per_tick(const BatchState& st) { return 2 + (fused_silu(st) ? 9 : 10) * st.L + 2; }

// Where a tick's rows keep their K and V: element strides of the cache's layer, K/V slot, row
// (session) and kv head. Lockstep sessions each have their own slab; the rows of a prefill chunk
// all share one session's, with row stride 0.
struct KvStrides {
  int64_t layer, slot, row, head;
};
inline KvStrides session_strides(const BatchState& st) {
  const int64_t head = (int64_t)st.S * st.hd, row = st.hkv * head, slot = st.B * row;
  return {2 * slot, slot, row, head};
}

// Enqueue one tick of nb <= B rows. flags: [0] sticky status bits, [2] this tick's skip flag, [3]
// the cancel word. lm: run the LM head and the argmax (which writes tokens and advances
// positions). out (optional) receives the tick's tokens; progress (optional) is set to
// progress_value after it.
inline int batch_tick(const BatchState& st, int nb, int32_t* tokens, int32_t* positions, void* kvp, KvStrides kvs,
                      float* logits, bool lm, hipStream_t s, uint32_t* flags, int32_t* out, uint32_t* progress,
                      uint32_t progress_value) {
  uint32_t* status = flags;
  const uint32_t* skip = flags + 2;
  uint16_t* kv = (uint16_t*)kvp;
  float* lg = logits ? logits : st.logits;
  // weights at element offset e (bf16 tiles, or one-byte tiles at the same offsets) and the row
  // scales from packed row r (one-byte weights only)
  auto wp = [&](size_t e) { return st.q ? (const uint16_t*)(st.w8 + e) : (const uint16_t*)(st.w + e); };
  auto sp = [&](size_t r) { return st.q ? (const float*)(st.wscale + r) : (const float*)nullptr; };
  auto gemm = [&](size_t we, size_t sr, const Gemm& g, float* out) {
    hipLaunchKernelGGL(gemm_for<false>(g.K / (g.KS * kKC), st.MT, st.q), dim3((g.N / kNB) * g.KS), dim3(gemm_threads(st.MT)), 0, s,
                       wp(we), g.N, g.K, (const uint16_t*)st.Ahi, (const uint16_t*)st.Alo, st.lda, out, g.KS, nb, skip,
                       (uint16_t*)nullptr, (uint16_t*)nullptr, sp(sr));
  };
  auto norm = [&](int mode, const Gemm* g, int gain_index) {
    hipLaunchKernelGGL(residual_norm_kernel, dim3(nb), dim3(1024), 0, s, mode, (const uint16_t*)st.embed,
                       (const int32_t*)tokens, (const float*)st.P, g ? g->KS : 0, st.X,
                       (const uint16_t*)(st.norms + (size_t)gain_index * st.d), st.d, st.eps, st.Ahi, st.Alo, st.lda,
                       nb, skip);
  };
  hipLaunchKernelGGL(check_kernel, dim3(1), dim3(1), 0, s, (const int32_t*)tokens, (const int32_t*)positions, nb, st.V,
                     st.max_seq, status, flags + 2, (const uint32_t*)(flags + 3));
  norm(0, nullptr, 0);
  for (int l = 0; l < st.L; ++l) {
    const size_t lay = (size_t)l * st.layer_elems, srl = (size_t)l * st.srows;  // this layer's weights and scales
    uint16_t* kvl = kv + (int64_t)l * kvs.layer;
    gemm(lay + st.w_qkv, srl, st.g_qkv, st.P);
    hipLaunchKernelGGL(qkv_epilogue_kernel, dim3(st.hq + 2 * st.hkv, nb), dim3(st.hd), 0, s, (const float*)st.P,
                       st.g_qkv.KS, st.nqkv, st.hq, st.hkv, st.hd, (const float2*)st.rope, (const int32_t*)positions,
                       st.Qs, kvl, kvs.slot, kvs.row, kvs.head, nb, skip);
    if (kvs.row == 0) {
      // prefill: the rows are consecutive positions of one session; a chunk of its cache serves all
      const int G = st.hq / st.hkv, rows_per_wg = 64 / G;
      hipLaunchKernelGGL(prefill_att_for(G), dim3(st.NCmax, st.hkv, (nb + rows_per_wg - 1) / rows_per_wg), dim3(256), 0,
                         s, (const float*)st.Qs, (const uint16_t*)kvl, kvs.slot, kvs.head, (const int32_t*)positions, nb,
                         st.hq, st.NCmax, st.part, skip);
    } else {
      hipLaunchKernelGGL(att_for(st.hq / st.hkv, st.CH), dim3(st.NCmax, st.hkv, nb), dim3(kAttThreads), 0, s, (const float*)st.Qs,
                         (const uint16_t*)kvl, kvs.slot, kvs.row, kvs.head, (const int32_t*)positions, st.hq, st.hkv,
                         st.NCmax, st.part, skip);
    }
    hipLaunchKernelGGL(merge_kernel, dim3(st.hq, nb), dim3(st.hd), 0, s, (const float*)st.part,
                       (const int32_t*)positions, st.hq, st.hd, st.CH, st.NCmax, st.Ahi, st.Alo, st.lda, skip);
    gemm(lay + st.w_o, srl + st.nqkv, st.g_o, st.P);
    norm(1, &st.g_o, 2 * l + 1);
    if (fused_silu(st)) {
      // gate/up writes SiLU(gate) * up into the second activation block, which the down
      // projection reads (the first is still being read while gate/up runs)
      const Gemm& g = st.g_gu;
      hipLaunchKernelGGL(gemm_for<true>(g.K / kKC, st.MT, st.q), dim3(g.N / kNB), dim3(gemm_threads(st.MT)), 0, s, wp(lay + st.w_gu),
                         g.N, g.K, (const uint16_t*)st.Ahi, (const uint16_t*)st.Alo, st.lda, st.P, 1, nb, skip, st.A2hi,
                         st.A2lo, sp(srl + st.nqkv + st.d));
      const Gemm& gd = st.g_d;
      hipLaunchKernelGGL(gemm_for<false>(gd.K / (gd.KS * kKC), st.MT, st.q), dim3((gd.N / kNB) * gd.KS), dim3(gemm_threads(st.MT)), 0,
                         s, wp(lay + st.w_d), gd.N, gd.K, (const uint16_t*)st.A2hi, (const uint16_t*)st.A2lo, st.lda, st.P,
                         gd.KS, nb, skip, (uint16_t*)nullptr, (uint16_t*)nullptr, sp(srl + st.nqkv + st.d + 2 * (size_t)st.F));
    } else {
      gemm(lay + st.w_gu, srl + st.nqkv + st.d, st.g_gu, st.P);
      hipLaunchKernelGGL(silu_kernel, dim3(st.F / 256, nb), dim3(256), 0, s, (const float*)st.P, st.g_gu.KS, st.F, st.Ahi,
                         st.Alo, st.lda, nb, skip);
      gemm(lay + st.w_d, srl + st.nqkv + st.d + 2 * (size_t)st.F, st.g_d, st.P);
    }
    norm(1, &st.g_d, l + 1 < st.L ? 2 * (l + 1) : 2 * st.L);
  }
  if (lm) {
    gemm(st.w_lm, (size_t)st.L * st.srows, st.g_lm, lg);
    hipLaunchKernelGGL(argmax_kernel, dim3(nb), dim3(1024), 0, s, (const float*)lg, st.V, tokens, positions, status, skip,
                       out);
  }
  if (progress) hipLaunchKernelGGL(progress_kernel, dim3(1), dim3(1), 0, s, progress, progress_value, skip);
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

// One tick of all B lockstep sessions.
inline int batch_step(const BatchState& st, int32_t* tokens, int32_t* positions, void* kvp, float* logits,
                      hipStream_t s, uint32_t* flags, int32_t* out, uint32_t* progress, uint32_t progress_value) {
  return batch_tick(st, st.B, tokens, positions, kvp, session_strides(st), logits, true, s, flags, out, progress,
                    progress_value);
}

// Prefill of one session (batch-1 cache layout): the n prompt tokens at positions *positions ..
// *positions + n - 1, in chunks of up to B positions, each chunk one tick whose rows are its
// positions. Every row appends its K and V to the session's cache and attends over positions 0 ..
// its own, so the chunks must run in order. Only the last chunk runs the LM head; its last row's
// greedy token, next position and logits go to tokens[0], positions[0] and logits.
inline int batch_prefill(const BatchState& st, const int32_t* prompt, int n, int32_t* tokens, int32_t* positions,
                         void* kvp, float* logits, hipStream_t s, uint32_t* flags) {
  const int64_t head = (int64_t)st.S * st.hd, slot = st.hkv * head;
  const KvStrides one{2 * slot, slot, 0, head};
  for (int first = 0; first < n; first += st.B) {
    const int nb = std::min(st.B, n - first);
    const bool last = first + nb == n;
    hipLaunchKernelGGL(prefill_rows_kernel, dim3(1), dim3(kMPrefill), 0, s, prompt, first, nb, (const int32_t*)positions,
                       st.rows_tok, st.rows_pos);
    const int rc = batch_tick(st, nb, st.rows_tok, st.rows_pos, kvp, one, nullptr, last, s, flags, nullptr, nullptr, 0);
    if (rc != KD_OK) return rc;
    if (last)
      hipLaunchKernelGGL(prefill_finish_kernel, dim3(64), dim3(256), 0, s, (const int32_t*)st.rows_tok,
                         (const int32_t*)st.rows_pos, nb - 1, (const float*)st.logits, st.V, tokens, positions, logits,
                         (const uint32_t*)(flags + 2));
  }
  return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

#undef KD_BT_TRY
#undef KD_BT_ALLOC

}  // namespace bt
}  // namespace kd

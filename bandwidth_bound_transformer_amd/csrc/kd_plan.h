// kd_plan.h -- static work plan of one decode step, shared by the host packer and the kernel.
//
// The whole schedule of a step is fixed before the first call: which workgroup
// streams which weight rows, which KV positions each wave reads and where every
// intermediate vector lives ("Why is real-time AI inference 56x more expensive?",
// section "decide everything ahead of time"). Only the attention split depends
// on the current position, and that is integer arithmetic every workgroup repeats.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define KD_HD __host__ __device__ __forceinline__
#else
#define KD_HD inline
#endif

namespace kd {

constexpr int kThreads = 512;      // 8 waves of 64 lanes per workgroup
constexpr int kWaves = 8;          // every wave streams packets and joins every exchange (wave_lo assumes 8)
constexpr int kPacketBytes = 1024; // one 16-byte load by each of 64 lanes
constexpr int kMaxDim = 4096;      // largest d_model and n_q_heads*head_dim held in LDS
constexpr int kMaxGroup = 4;       // largest q heads per kv head
constexpr int kMaxHeadDim = 128;
constexpr int kChunkMin = 32;      // fewest cached positions per attention unit
constexpr int kMaxUnits = 4;       // attention units one workgroup may hold in one step
constexpr int kMergeWords = 4096;  // largest gather of one merge unit
constexpr int kRowPart = 96;       // row partial sums kept per wave
constexpr int kScorePos = 96;      // attention scores kept per wave (positions)
constexpr int kStageWords = 4096;  // staging area for gathers that are not the activation

// Tag kinds of the vectors exchanged between workgroups (an exchange word carries value|tag).
enum Kind : int { kQKV = 0, kATTP = 1, kO = 2, kXP = 3, kDP = 4, kX = 5, kLM = 6 };

// Start of part i when n items are cut into `parts` contiguous parts.
KD_HD int64_t part_lo(int64_t n, int64_t parts, int64_t i) { return n * i / parts; }
// Items of a tile handed to waves 0 .. v-1. Waves v and v + 4 share a SIMD, and the older one
// (v < 4) wins issue arbitration and streams faster, so waves 0-3 get the larger share.
// Measured: shares 29:21 make both halves finish together (2B +6%, 8B +2% over equal shares).
#ifndef KD_WSKEW
#define KD_WSKEW 4
#endif
constexpr int kWaveWeightHi = 25 + KD_WSKEW, kWaveWeightLo = 25 - KD_WSKEW;
static_assert(kWaves == 8 && kWaveWeightLo > 0, "wave_lo splits over 8 waves with positive weights");
KD_HD int64_t wave_lo(int64_t n, int v) {
  const int64_t hi = v < 4 ? v : 4, lo = v > 4 ? v - 4 : 0;
  return n * (hi * kWaveWeightHi + lo * kWaveWeightLo) / (4 * (kWaveWeightHi + kWaveWeightLo));
}
// Part that holds item i (inverse of part_lo), for n > 0.
KD_HD int64_t part_of(int64_t n, int64_t parts, int64_t i) { return (parts * i + parts - 1) / n; }

KD_HD int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Dims {
  int32_t L, d, hq, hkv, hd, F, V, S, nwg;  // S: KV positions allocated per (layer, slot, session, head)
  int32_t wbytes, kvbytes;                 // matrix elements: 1 (fp8), 2 (bf16) or 4 (f32); cache: 2 or 4
  int32_t G, qdim, kvdim, nqkv;            // nqkv = qdim + 2*kvdim rows of the fused QKV matrix
  int32_t vpl;                             // weight values per 16-byte lane load
  int32_t kv_vpl;                          // KV values per 16-byte lane load
  int32_t lpp, ppp;                        // lanes per KV position, KV positions per packet
  int32_t cd, cq;                          // packets per weight row for K = d and K = qdim
  int64_t off_qkv, off_o, off_gu, off_d, layer_elems, off_lm;  // element offsets in the packed blob
  int64_t blob_elems;
};

// fp8 row scales (floats): per layer the QKV rows, the O rows, the gate/up rows in packed order and
// the down rows; then the LM head's rows.
struct ScaleLayout {
  int64_t o, gu, d, layer, lm, total;
};
KD_HD ScaleLayout scale_layout(const Dims& m) {
  ScaleLayout s{};
  s.o = m.nqkv;
  s.gu = s.o + m.d;
  s.d = s.gu + (int64_t)2 * m.F;
  s.layer = s.d + m.d;
  s.lm = (int64_t)m.L * s.layer;
  s.total = s.lm + m.V;
  return s;
}

KD_HD Dims make_dims(int L, int d, int hq, int hkv, int hd, int F, int V, int max_seq, int nwg, int wbytes, int kvbytes) {
  Dims m{};
  m.L = L; m.d = d; m.hq = hq; m.hkv = hkv; m.hd = hd; m.F = F; m.V = V; m.nwg = nwg;
  // the last packet of an attention chunk may cover up to 7 positions past the current one
  m.S = (int32_t)(ceil_div((int64_t)max_seq + 7, 16) * 16);
  m.wbytes = wbytes; m.kvbytes = kvbytes;
  m.G = hq / hkv; m.qdim = hq * hd; m.kvdim = hkv * hd; m.nqkv = m.qdim + 2 * m.kvdim;
  m.vpl = 16 / wbytes; m.kv_vpl = 16 / kvbytes;
  m.lpp = hd / m.kv_vpl; m.ppp = 64 / m.lpp;
  m.cd = d * wbytes / kPacketBytes; m.cq = m.qdim * wbytes / kPacketBytes;
  m.off_qkv = 0;
  m.off_o = m.off_qkv + (int64_t)m.nqkv * d;
  m.off_gu = m.off_o + (int64_t)d * m.qdim;
  m.off_d = m.off_gu + (int64_t)2 * F * d;
  m.layer_elems = m.off_d + (int64_t)d * F;
  m.off_lm = (int64_t)L * m.layer_elems;
  m.blob_elems = m.off_lm + (int64_t)V * d;
  return m;
}

// Element bytes of the embedding and the norm gains: bf16 when the matrices are fp8.
KD_HD int32_t embed_bytes(const Dims& m) { return m.wbytes == 1 ? 2 : m.wbytes; }
// FFN columns per slice unit (a workgroup owns whole units). fp8 keeps 8-column units: a down
// packet then holds two 64-row halves of 8 columns each, so a down block is 128 rows.
KD_HD int32_t ffn_unit(const Dims& m) { return m.wbytes == 1 ? 8 : m.vpl; }
KD_HD int32_t down_block_rows(const Dims& m) { return m.wbytes == 1 ? 128 : 64; }

// FFN columns owned by workgroup w: [ffn_lo(w), ffn_lo(w+1)), whole units of ffn_unit columns.
KD_HD int64_t ffn_lo(const Dims& m, int64_t w) { return (int64_t)ffn_unit(m) * part_lo(m.F / ffn_unit(m), m.nwg, w); }

// Element offset of workgroup w's down-projection packets inside a layer's down block.
KD_HD int64_t down_wg_off(const Dims& m, int64_t w) { return (int64_t)m.d * ffn_lo(m, w); }

// Attention split of one step at position p (P = p+1 positions attended, 0..p).
//   NC chunks of CH positions per kv head -> units = NC * hkv, unit u = (head u / NC, chunk u % NC).
//   The cached positions 0..p-1 are streamed; position p comes from this step's QKV and is
//   added by the unit holding the last chunk.
//   Merge units: q head h, dim slice s of MS dims -> nmerge = hq * (hd / MS).
struct AttPlan {
  int32_t P, CH, NC, units, MS, nmerge;
};

// Chunks per kv head that one round of units (one per workgroup) covers.
KD_HD int64_t chunk_round(const Dims& m) {
  const int64_t r = m.nwg / m.hkv;
  return r < 1 ? 1 : r;
}

KD_HD AttPlan att_plan(const Dims& m, int32_t p) {
  AttPlan a{};
  a.P = p + 1;
  const int64_t cap = chunk_round(m);
  int64_t nc = ceil_div(a.P, kChunkMin);
  if (nc > cap) nc = cap;
  int64_t ch = 0;
  while (true) {
    ch = ceil_div(ceil_div(a.P, nc), m.ppp) * m.ppp;
    // a wave keeps the scores of its share of the chunk in LDS: add rounds of units until it fits
    if (ceil_div(ceil_div(ch, m.ppp), kWaves) * m.ppp <= kScorePos || nc >= cap * kMaxUnits) break;
    nc += cap;
  }
  a.CH = (int32_t)ch;
  a.NC = (int32_t)ceil_div(a.P, ch);
  a.units = a.NC * m.hkv;
  // merge slices: the most merge units that still fit one workgroup each, slices of >= 2 dims
  int32_t ms = m.hd;
  while (ms > 2 && ((int64_t)m.hq * (m.hd / (ms / 2)) <= m.nwg || (int64_t)a.NC * (ms + 2) > kMergeWords)) ms /= 2;
  a.MS = ms;
  a.nmerge = m.hq * (m.hd / ms);
  return a;
}

// Most chunks any step can use (sizes the partial buffer).
KD_HD int32_t max_chunks(const Dims& m) { return (int32_t)(chunk_round(m) * kMaxUnits); }

// Word offsets of the exchange buffers (64-bit words) for one session.
struct LLLayout {
  int64_t qkv, attp, o, xp, dp, x, lm, total;
};

KD_HD LLLayout ll_layout(const Dims& m) {
  LLLayout l{};
  int64_t at = 0;
  auto take = [&](int64_t n) { int64_t r = at; at += (n + 1) / 2 * 2; return r; };
  l.qkv = take(m.nqkv);
  l.attp = take((int64_t)m.hq * max_chunks(m) * (m.hd + 2));
  l.o = take(m.qdim);
  l.xp = take(m.d);
  l.dp = take((int64_t)m.nwg * m.d);  // [producer workgroup][d]: each producer's partial is contiguous
  l.x = take(m.d);
  l.lm = take((int64_t)m.nwg * 2);
  l.total = at;
  return l;
}

// Step trace: per workgroup, slots 0-1 (start, setup done), kTraceLayerEvents phase
// boundaries per layer, then 4 for the final norm, LM head and argmax.
constexpr int kTraceLayerEvents = 24;
KD_HD int64_t trace_stride(int L) { return 2 + (int64_t)kTraceLayerEvents * L + 4; }
constexpr int kTraceMaxLayers = 40;  // step tracing covers models of up to this many layers
constexpr int kTraceMaxSlots = 2 + kTraceLayerEvents * kTraceMaxLayers + 4;

// Tags one step uses: 8 per layer plus 8 for the LM head. A call of n steps takes the n * stride
// tags from its base; the host never hands out a range that wraps past zero (tag 0 is what a
// cleared word holds, so it never names a live vector).
KD_HD uint32_t tag_stride(const Dims& m) { return (uint32_t)(8 * (m.L + 1)); }
// Tag of vector `kind` of layer `layer` (layer == L for the LM head) in the step whose tags start at `base`.
KD_HD uint32_t ll_tag(uint32_t base, int layer, int kind) { return base + (uint32_t)(8 * layer + kind); }

}  // namespace kd

// kd_device.h -- the persistent decode-step kernel for gfx950.
//
// One launch runs a whole decode step: embedding, every layer, LM head and argmax.
//
// Grid. One workgroup per compute unit. Every workgroup stays resident for the
// whole step, as in the single-kernel runtime of the Kog engine ("Real-time LLM
// inference on standard data-centre GPUs (3,000 tokens/s single request)",
// section "technical principles"). A workgroup has 8 waves:
//
//  * Waves 1..7 are compute waves. Each streams a fixed, precomputed sequence
//    of 1 KB packets: its share of every weight tile of the step, plus its
//    share of the KV positions its workgroup attends over. Packets arrive
//    through a private ring in LDS, filled by LDS-DMA loads
//    (global_load_lds_dwordx4, non-temporal). The loads run RING packets
//    ahead of the consumer, straight across phase boundaries. Weights do not
//    depend on activations, so HBM keeps streaming while the workgroup waits
//    for the previous phase's results. This is the single-GPU form of "keep
//    computing and synchronise later" ("Kog 3000 tok/s real-time inference",
//    section "KCCL").
//  * Wave 0 is the control wave. It never has weight loads in flight, so its
//    waits are short. It collects the vectors other workgroups produced, runs
//    RMSNorm, RoPE and softmax merges, reduces the compute waves' partial
//    sums, and publishes this workgroup's results.
//
// Exchange between workgroups. Vectors travel as "LL words": 64-bit words with
// a float in the low half and a tag in the high half. They are written with
// device-scope relaxed atomic stores and read with device-scope loads (sc1).
// A tag names the step, layer and vector kind, so a reader spins until every
// word it needs carries the expected tag. One round trip therefore does both
// the synchronisation and the data transfer, with no grid-wide barrier and no
// L2 writeback or invalidate. Each word is one naturally aligned 64-bit
// atomic, so a reader never accepts a stale or torn value.
//
// Layer dataflow (WG = workgroup; every WG does each step for its own slice):
//   x --gather--> RMSNorm --> QKV rows (row-split)      --> LL qkv
//   q,k,v --gather--> RoPE, KV append, attention over one chunk of positions --> LL partials
//   partials --gather--> merge (log-sum-exp) of one head slice --> LL o
//   o --gather--> O rows + residual (row-split)        --> LL x'
//   x' --gather--> RMSNorm --> gate/up rows of this WG's FFN slice --> SiLU*up stays in LDS
//   local FFN slice --> down projection of that slice for all d rows --> LL partial sums
//   partial sums for this WG's rows --gather--> sum + residual --> LL x
#pragma once
#include <hip/hip_runtime.h>

#include "kd_plan.h"

namespace kd {

struct Params {
  const uint8_t* blob;   // packed layer weights and LM head, weight dtype
  const uint8_t* embed;  // [V][d], weight dtype
  const uint8_t* norms;  // [L][2][d] attention/FFN gains, then final gain [d], weight dtype
  uint64_t* ll;          // exchange words
  LLLayout lo;
  uint8_t* kv;           // caller's cache [L][2][B][hkv][S][hd]
  int32_t* tokens;
  int32_t* positions;
  float* logits;
  uint32_t* status;
  uint32_t* abortf;
  uint64_t* trace;  // per-workgroup phase timestamps (100 MHz clock), or null
  uint32_t seq;
  int32_t max_seq;
  float eps;
  float rope_base;
  Dims m;
};

constexpr uint32_t kStatusTokenRange = 0x1u, kStatusPosOverflow = 0x2u, kStatusTimeout = 0x4u, kStatusNaN = 0x8u;
constexpr uint64_t kSpinTicks = 200000000ull;  // 2 s of the 100 MHz realtime counter

// ----------------------------------------------------------------------------------------------
// small helpers
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 64 lanes x 16 bytes from per-lane global addresses into LDS [lds_addr, lds_addr + 1 KB).
// Non-temporal: weights and KV are read once per step.  Waits for this wave's earlier LDS reads
// first, so a slot is never refilled while a read of it is still in flight.
__device__ __forceinline__ void dma_packet(const void* lane_addr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(lane_addr)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// device-scope (sc1) 16-byte load of two LL words, bounds-checked by the buffer descriptor
__device__ __forceinline__ uint4 ll_load2(__amdgpu_buffer_rsrc_t r, int64_t word) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(word * 8), 0, 16));
}

__device__ __forceinline__ void ll_store(uint64_t* ll, int64_t word, float v, uint32_t tag) {
  uint32_t bits = __float_as_uint(v);
  if ((bits & 0x7fffffffu) > 0x7f800000u) bits = 0x7fc00000u;
  __hip_atomic_store(ll + word, ((uint64_t)tag << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ll_store_bits(uint64_t* ll, int64_t word, uint32_t bits, uint32_t tag) {
  __hip_atomic_store(ll + word, ((uint64_t)tag << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t ld_flag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int WB>
__device__ __forceinline__ float load_w(const uint8_t* base, int64_t i) {
  if constexpr (WB == 2) return __uint_as_float((uint32_t)((const uint16_t*)base)[i] << 16);
  else return ((const float*)base)[i];
}

// ----------------------------------------------------------------------------------------------
// 32-bit plan arithmetic for the device (every count here fits in 31 bits)
// ----------------------------------------------------------------------------------------------
__device__ __forceinline__ int p_lo(int n, int parts, int i) { return (int)(((uint32_t)n * (uint32_t)i) / (uint32_t)parts); }
__device__ __forceinline__ int p_of(int n, int parts, int i) { return (int)(((uint32_t)parts * (uint32_t)i + (uint32_t)parts - 1u) / (uint32_t)n); }
__device__ __forceinline__ int c_div(int a, int b) { return (a + b - 1) / b; }
__device__ __forceinline__ int ffn_lo32(const Dims& m, int w) { return m.vpl * p_lo(m.F / m.vpl, m.nwg, w); }

// ----------------------------------------------------------------------------------------------
// shared memory
// ----------------------------------------------------------------------------------------------
constexpr int kMaxUnits = 16;  // attention units one workgroup handles in one step

// One contiguous run of packets in a compute wave's sequence. `base` is the address of packet 0
// at layer 0; kind says how it moves with the layer.
enum SegKind : int32_t { kSegWeight = 0, kSegKV = 1, kSegOnce = 2 };
struct SegEntry {
  const uint8_t* base;
  int32_t lo, hi;
  int32_t kind, pad;
};

// Per-layer order of a compute wave's segments: QKV, (K, V) of each attention unit, O, gate/up, down.
__device__ __forceinline__ int seg_o(int nunits) { return 1 + 2 * nunits; }

enum Tile : int { kTileQKV = 0, kTileO = 1, kTileGU = 2, kTileD = 3, kTileLM = 4, kTiles = 5 };

template <int RING>
struct Smem {
  uint4 ring[kComputeWaves][RING][64];
  float x[kMaxDim];    // residual stream x (or x') of the current layer
  float act[kMaxDim];  // input of the current projection (normalised x, o, or the FFN slice)
  union {
    float part_r[kComputeWaves][kSegR];      // per-wave row sums
    float part_c[kComputeWaves][kSegC][64];  // per-wave 64-row block sums (down projection)
    struct {
      float q[kMaxGroup][kMaxHeadDim];       // rotated queries of this unit's kv head, times 1/sqrt(hd)
      float kp[kMaxHeadDim];                 // K and V of the current position, as stored
      float vp[kMaxHeadDim];
      float scores[kComputeWaves][kScorePos][kMaxGroup];
      float acc[kComputeWaves][kMaxGroup][kMaxHeadDim];
      float ml[kComputeWaves][kMaxGroup][2];
    } att;
    float stage[kMergeWords + 64];
  } u;
  SegEntry segs[kComputeWaves][4 + 2 * kMaxUnits];
  SegEntry lm_seg[kComputeWaves];
  int32_t split[kTiles][kComputeWaves + 1];  // wave boundaries of each tile (packets)
  int32_t first[kTiles][kComputeWaves];      // first row / block of each wave's share
  float rope_c[kMaxHeadDim / 2];
  float rope_s[kMaxHeadDim / 2];
  int abort_flag;
};

// ----------------------------------------------------------------------------------------------
// step-level facts every wave derives from the inputs
// ----------------------------------------------------------------------------------------------
struct StepInfo {
  int32_t p;       // position of the input token
  AttPlan ap;
  int32_t nunits;  // attention units of this workgroup
};

// Attention unit k of workgroup w: kv head g, chunk c, cached positions [j0, j1).
struct Unit {
  int32_t g, c, j0, j1, last;
};
__device__ __forceinline__ Unit unit_of(const StepInfo& si, int w, int k, int nwg) {
  Unit u{};
  const int32_t id = w + k * nwg;
  u.g = id / si.ap.NC;
  u.c = id - u.g * si.ap.NC;
  u.j0 = u.c * si.ap.CH;
  const int32_t end = min((u.c + 1) * si.ap.CH, si.ap.P);
  u.last = end == si.ap.P;
  u.j1 = min(end, si.p);  // the current position comes from this step's QKV, not from the cache
  if (u.j1 < u.j0) u.j1 = u.j0;
  return u;
}

// Packets of each tile of workgroup w, and how many packets a row (or 64-row block) spans.
__device__ __forceinline__ void tile_shape(const Dims& m, int w, int tile, int& T, int& C) {
  if (tile == kTileQKV) { C = m.cd; T = (p_lo(m.nqkv, m.nwg, w + 1) - p_lo(m.nqkv, m.nwg, w)) * C; }
  else if (tile == kTileO) { C = m.cq; T = (p_lo(m.d, m.nwg, w + 1) - p_lo(m.d, m.nwg, w)) * C; }
  else if (tile == kTileGU) { C = m.cd; T = 2 * (ffn_lo32(m, w + 1) - ffn_lo32(m, w)) * C; }
  else if (tile == kTileD) { C = (ffn_lo32(m, w + 1) - ffn_lo32(m, w)) / m.vpl; T = (m.d / 64) * C; }
  else { C = m.cd; T = (p_lo(m.V, m.nwg, w + 1) - p_lo(m.V, m.nwg, w)) * C; }
}

// Fill compute wave v's segment table (done by the wave itself).
template <int RING>
__device__ __forceinline__ void build_segments(const Params& P, const StepInfo& si, int w, int v, Smem<RING>& sm) {
  const Dims& m = P.m;
  if (lane_id() != 0) return;
  auto put = [&](SegEntry& e, const uint8_t* base, int T, int kind) {
    e.base = base;
    e.lo = p_lo(T, kComputeWaves, v);
    e.hi = p_lo(T, kComputeWaves, v + 1);
    e.kind = kind;
  };
  SegEntry* t = sm.segs[v];
  int T, C;
  tile_shape(m, w, kTileQKV, T, C);
  put(t[0], P.blob + (m.off_qkv + (int64_t)p_lo(m.nqkv, m.nwg, w) * m.d) * m.wbytes, T, kSegWeight);
  for (int k = 0; k < si.nunits; ++k) {
    const Unit u = unit_of(si, w, k, m.nwg);
    const int n = u.j1 > u.j0 ? c_div(u.j1 - u.j0, m.ppp) : 0;
    const int64_t kbase = (((int64_t)0 * 2 + 0) * m.hkv + u.g) * m.S + u.j0;
    const int64_t vbase = (((int64_t)0 * 2 + 1) * m.hkv + u.g) * m.S + u.j0;
    put(t[1 + 2 * k], P.kv + kbase * m.hd * m.kvbytes, n, kSegKV);
    put(t[2 + 2 * k], P.kv + vbase * m.hd * m.kvbytes, n, kSegKV);
  }
  const int o = seg_o(si.nunits);
  tile_shape(m, w, kTileO, T, C);
  put(t[o], P.blob + (m.off_o + (int64_t)p_lo(m.d, m.nwg, w) * m.qdim) * m.wbytes, T, kSegWeight);
  tile_shape(m, w, kTileGU, T, C);
  put(t[o + 1], P.blob + (m.off_gu + (int64_t)2 * ffn_lo32(m, w) * m.d) * m.wbytes, T, kSegWeight);
  tile_shape(m, w, kTileD, T, C);
  put(t[o + 2], P.blob + (m.off_d + (int64_t)m.d * ffn_lo32(m, w)) * m.wbytes, T, kSegWeight);
  tile_shape(m, w, kTileLM, T, C);
  put(sm.lm_seg[v], P.blob + (m.off_lm + (int64_t)p_lo(m.V, m.nwg, w) * m.d) * m.wbytes, T, kSegOnce);
}

// Walks this wave's packet sequence ahead of the consumer and issues the loads.
struct Issuer {
  const SegEntry* tab;
  const SegEntry* lm;
  int nseg, L;
  int64_t wstride, kvstride;
  int layer, e;  // layer == L: the LM head; layer > L: past the end
  const uint8_t* base;
  int32_t idx, hi;
  const uint8_t* last;

  __device__ __forceinline__ void next_entry() {
    if (layer < L) {
      if (++e == nseg) { e = 0; ++layer; }
    } else {
      ++layer;
    }
  }
  __device__ __forceinline__ void load() {
    while (layer <= L) {
      const SegEntry s = layer < L ? tab[e] : *lm;
      if (s.hi > s.lo) {
        base = s.base + (s.kind == kSegWeight ? layer * wstride : (s.kind == kSegKV ? layer * kvstride : 0));
        idx = s.lo;
        hi = s.hi;
        return;
      }
      next_entry();
    }
  }
  // Issue the next packet of the sequence into an LDS slot; past the end, reload the last one.
  __device__ __forceinline__ void issue(uint32_t slot_addr) {
    const uint8_t* a = last;
    if (layer <= L) {
      a = base + (int64_t)idx * kPacketBytes;
      last = a;
      if (++idx == hi) { next_entry(); load(); }
    }
    dma_packet(a + lane_id() * 16, slot_addr);
  }
};

// Consumer side of the ring: take the next packet (waiting for its load), then give the slot back.
template <int RING>
struct Ring {
  const uint4* slots;  // this wave's RING x 64 x 16 bytes
  uint32_t slot_lds;   // LDS address of slot 0
  uint32_t cnt;
  Issuer is;
  __device__ __forceinline__ uint4 take() const {
    wait_vm<RING - 1>();
    return slots[(cnt % RING) * 64 + lane_id()];
  }
  __device__ __forceinline__ void give() {
    is.issue(slot_lds + (cnt % RING) * kPacketBytes);
    ++cnt;
  }
};

// ----------------------------------------------------------------------------------------------
// packet arithmetic
// ----------------------------------------------------------------------------------------------
// One 16-byte lane load of weights times the matching activation values (8 bf16 or 4 f32).
template <int WB>
__device__ __forceinline__ float dot16(const uint4 w, const float* a) {
  if constexpr (WB == 2) {
    const float4 a0 = *(const float4*)a, a1 = *(const float4*)(a + 4);
    float s = bf16_lo(w.x) * a0.x;
    s = fmaf(bf16_hi(w.x), a0.y, s);
    s = fmaf(bf16_lo(w.y), a0.z, s);
    s = fmaf(bf16_hi(w.y), a0.w, s);
    s = fmaf(bf16_lo(w.z), a1.x, s);
    s = fmaf(bf16_hi(w.z), a1.y, s);
    s = fmaf(bf16_lo(w.w), a1.z, s);
    s = fmaf(bf16_hi(w.w), a1.w, s);
    return s;
  } else {
    const float4 a0 = *(const float4*)a;
    float s = __uint_as_float(w.x) * a0.x;
    s = fmaf(__uint_as_float(w.y), a0.y, s);
    s = fmaf(__uint_as_float(w.z), a0.z, s);
    s = fmaf(__uint_as_float(w.w), a0.w, s);
    return s;
  }
}

template <int KB>
__device__ __forceinline__ void unpack16(const uint4 w, float* out) {
  if constexpr (KB == 2) {
    out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z); out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
  } else {
    out[0] = __uint_as_float(w.x); out[1] = __uint_as_float(w.y); out[2] = __uint_as_float(w.z); out[3] = __uint_as_float(w.w);
  }
}

// Row-split matrix-vector product: packets are row chunks of 64*vpl values; act is the input vector.
// A row's lane sums are reduced across the wave when the row (or this wave's share of it) ends.
template <int RING, int WB>
__device__ __forceinline__ void consume_rows(Ring<RING>& rg, const SegEntry& s, int C, const float* act, float* part) {
  constexpr int VPL = 16 / WB;
  const int lane = lane_id();
  int r = s.lo / C;
  const int r_first = r;
  int c = s.lo - r * C;
  float acc = 0.f;
  for (int i = s.lo; i < s.hi; ++i) {
    const uint4 wv = rg.take();
    acc += dot16<WB>(wv, act + c * (64 * VPL) + lane * VPL);
    rg.give();
    if (++c == C || i + 1 == s.hi) {
      const float t = wave_sum(acc);
      if (lane == 0) part[r - r_first] = t;
      acc = 0.f;
      c = 0;
      ++r;
    }
  }
}

// Column-block product of the down projection: packets hold 64 rows x vpl columns of this
// workgroup's FFN slice; every lane owns one row, and all lanes read the same slice values.
template <int RING, int WB>
__device__ __forceinline__ void consume_cols(Ring<RING>& rg, const SegEntry& s, int g, const float* a, float* part /* [kSegC][64] */) {
  constexpr int VPL = 16 / WB;
  const int lane = lane_id();
  int b = s.lo / g;
  const int b_first = b;
  int j = s.lo - b * g;
  float acc = 0.f;
  for (int i = s.lo; i < s.hi; ++i) {
    const uint4 wv = rg.take();
    acc += dot16<WB>(wv, a + j * VPL);
    rg.give();
    if (++j == g || i + 1 == s.hi) {
      part[(b - b_first) * 64 + lane] = acc;
      acc = 0.f;
      j = 0;
      ++b;
    }
  }
}

// Scores, then the exp-weighted V sum, of one attention unit over this wave's share of the
// unit's cached positions. lpp lanes hold one position; each lane holds kv_vpl of its dims.
template <int RING, int KB, int HD>
__device__ __forceinline__ void consume_attention(Ring<RING>& rg, const SegEntry& sk, const Unit& u, int G, Smem<RING>& sm,
                                                  int v) {
  constexpr int KVPL = 16 / KB;
  constexpr int LPP = HD / KVPL;
  constexpr int PPP = 64 / LPP;
  const int lane = lane_id();
  const int q_in = lane / LPP;  // position inside a packet
  const int dim0 = (lane % LPP) * KVPL;
  float qv[kMaxGroup][KVPL];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
    for (int e = 0; e < KVPL; ++e) qv[h][e] = h < G ? sm.u.att.q[h][dim0 + e] : 0.f;
  float mh[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) mh[h] = -INFINITY;
  // pass 1: scores (q already carries 1/sqrt(hd))
  for (int i = sk.lo; i < sk.hi; ++i) {
    const uint4 kw = rg.take();
    float kf[KVPL];
    unpack16<KB>(kw, kf);
    rg.give();
    const int pos = u.j0 + i * PPP + q_in;
    const bool valid = pos < u.j1;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < G) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < KVPL; ++e) s = fmaf(qv[h][e], kf[e], s);
#pragma unroll
        for (int o = LPP / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
        if (valid) {
          mh[h] = fmaxf(mh[h], s);
          if (lane % LPP == 0) sm.u.att.scores[v][(i - sk.lo) * PPP + q_in][h] = s;
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
    for (int o = 32; o >= LPP; o >>= 1) mh[h] = fmaxf(mh[h], __shfl_xor(mh[h], o));
  // pass 2: V weighted by exp(score - wave max)
  float acc[kMaxGroup][KVPL];
  float lsum[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < KVPL; ++e) acc[h][e] = 0.f;
  }
  for (int i = sk.lo; i < sk.hi; ++i) {
    const uint4 vw = rg.take();
    float vf[KVPL];
    unpack16<KB>(vw, vf);
    rg.give();
    const int pos = u.j0 + i * PPP + q_in;
    if (pos < u.j1) {
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < G) {
          const float e = __expf(sm.u.att.scores[v][(i - sk.lo) * PPP + q_in][h] - mh[h]);
          lsum[h] += e;
#pragma unroll
          for (int k = 0; k < KVPL; ++k) acc[h][k] = fmaf(e, vf[k], acc[h][k]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
#pragma unroll
    for (int o = 32; o >= LPP; o >>= 1) {
      lsum[h] += __shfl_xor(lsum[h], o);
#pragma unroll
      for (int k = 0; k < KVPL; ++k) acc[h][k] += __shfl_xor(acc[h][k], o);
    }
  }
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < G) {
      if (lane < LPP) {
#pragma unroll
        for (int k = 0; k < KVPL; ++k) sm.u.att.acc[v][h][dim0 + k] = acc[h][k];
      }
      if (lane == 0) {
        sm.u.att.ml[v][h][0] = mh[h];
        sm.u.att.ml[v][h][1] = lsum[h];
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
// control wave: exchange, normalisation, reductions
// ----------------------------------------------------------------------------------------------
template <int RING>
struct Ctl {
  const Params& P;
  __amdgpu_buffer_rsrc_t llr;
  Smem<RING>& sm;

  __device__ __forceinline__ bool failed() const { return sm.abort_flag != 0; }

  __device__ __forceinline__ void fail(uint32_t bit) {
    if (lane_id() == 0) {
      __hip_atomic_fetch_or(P.status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(P.abortf, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sm.abort_flag = 1;
  }

  // Collect npieces 16-byte pieces (two LL words each) at word offsets off(k), wait until both
  // words of every piece carry `tag`, then hand the two floats of piece k to sink(k, a, b).
  template <class Off, class Sink>
  __device__ __forceinline__ void gather(uint32_t tag, int npieces, Off off, Sink sink) {
    constexpr int NB = 8;
    const int lane = lane_id();
    for (int base = 0; base < npieces; base += 64 * NB) {
      if (failed()) return;
      uint4 val[NB];
      uint64_t t0 = 0;
      bool started = false;
      while (true) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int k = base + lane + 64 * i;
          if (k < npieces) val[i] = ll_load2(llr, off(k));
        }
        bool ok = true;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int k = base + lane + 64 * i;
          if (k < npieces) ok = ok && val[i].y == tag && val[i].w == tag;
        }
        if (__all(ok)) break;
        if (!started) { t0 = now_ticks(); started = true; }
        if (now_ticks() - t0 > kSpinTicks) { fail(kStatusTimeout); return; }
        if (ld_flag(P.abortf)) { sm.abort_flag = 1; return; }
        __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int k = base + lane + 64 * i;
        if (k < npieces) sink(k, __uint_as_float(val[i].x), __uint_as_float(val[i].z));
      }
    }
  }

  // Gather n consecutive LL words (n even) starting at word `at` into dst[0..n).
  __device__ __forceinline__ void gather_vec(uint32_t tag, int64_t at, int n, float* dst) {
    gather(tag, n / 2, [&](int k) { return at + 2 * (int64_t)k; },
           [&](int k, float a, float b) {
             dst[2 * k] = a;
             dst[2 * k + 1] = b;
           });
  }

  template <int WB>
  __device__ __forceinline__ void rmsnorm(const float* x, const uint8_t* gain, float* out, int d) {
    const int lane = lane_id();
    float ss = 0.f;
    for (int i = lane; i < d; i += 64) ss = fmaf(x[i], x[i], ss);
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + P.eps);
    for (int i = lane; i < d; i += 64) out[i] = x[i] * r * load_w<WB>(gain, i);
  }

  // Boundaries of every tile's wave shares, for the reductions below.
  __device__ __forceinline__ void build_splits(int w) {
    const int lane = lane_id();
    if (lane < kTiles) {
      int T, C;
      tile_shape(P.m, w, lane, T, C);
      for (int v = 0; v <= kComputeWaves; ++v) sm.split[lane][v] = p_lo(T, kComputeWaves, v);
      for (int v = 0; v < kComputeWaves; ++v) sm.first[lane][v] = C > 0 ? sm.split[lane][v] / C : 0;
    }
  }

  // Total of row r (C packets per row) of a tile over the compute waves that touched it.
  __device__ __forceinline__ float row_total(int tile, int C, int r) const {
    const int a = r * C, b = a + C;
    float s = 0.f;
    for (int v = 0; v < kComputeWaves; ++v) {
      const int lo = sm.split[tile][v], hi = sm.split[tile][v + 1];
      if (lo < hi && lo < b && hi > a) s += sm.u.part_r[v][r - sm.first[tile][v]];
    }
    return s;
  }
  __device__ __forceinline__ float block_total(int g, int blk, int lane) const {
    const int a = blk * g, b = a + g;
    float s = 0.f;
    for (int v = 0; v < kComputeWaves; ++v) {
      const int lo = sm.split[kTileD][v], hi = sm.split[kTileD][v + 1];
      if (lo < hi && lo < b && hi > a) s += sm.u.part_c[v][blk - sm.first[kTileD][v]][lane];
    }
    return s;
  }
};

// ----------------------------------------------------------------------------------------------
// the kernel
// ----------------------------------------------------------------------------------------------
// Workgroup barrier that waits for this wave's LDS traffic only. Compute waves keep their
// LDS-DMA loads in flight across it; that is the point of the ring.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Timestamp slot of phase-boundary `ev` (layer < L) or of the final phases (layer == L).
__device__ __forceinline__ int trace_slot(int L, int layer, int ev) { return 2 + kTraceLayerEvents * layer + ev; }

// Phase protocol. Every phase runs as: control prepares the input in LDS; barrier B; compute
// waves stream their packets into per-wave partial sums; barrier A; control reduces and
// publishes. A failed wait sets the LDS abort flag before the next barrier B. All waves read the
// flag right after B and leave together, so the barrier sequences of the waves always match.
template <int RING, int WB, int KB, int HD>
__global__ __launch_bounds__(kThreads, 1) void decode_step_kernel(const Params P_arg) {
  __shared__ Smem<RING> sm;
  // work on a private copy: references into the kernel-argument segment would force a stack copy
  const Params P = P_arg;
  const Dims m = P.m;
  const int w = (int)blockIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();

  // inputs of this step; every wave of every workgroup takes the same decision
  StepInfo si{};
  const int32_t token = P.tokens[0];
  si.p = P.positions[0];
  if (token < 0 || token >= m.V || si.p < 0 || si.p >= P.max_seq) {
    if (w == 0 && threadIdx.x == 0) {
      uint32_t bit = (token < 0 || token >= m.V) ? kStatusTokenRange : 0u;
      if (si.p < 0 || si.p >= P.max_seq) bit |= kStatusPosOverflow;
      __hip_atomic_fetch_or(P.status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  si.ap = att_plan(m, si.p);
  si.nunits = w < si.ap.units ? c_div(si.ap.units - w, m.nwg) : 0;
  const int mfirst = m.nwg - 1 - w;
  const int nmerge_here = mfirst < si.ap.nmerge ? c_div(si.ap.nmerge - mfirst, m.nwg) : 0;
  const int oseg = seg_o(si.nunits);

  if (threadIdx.x == 0) sm.abort_flag = 0;

  if (wave > 0) {
    // ============================ compute waves ============================
    const int v = wave - 1;
    build_segments(P, si, w, v, sm);
    const SegEntry* tab = sm.segs[v];
    Ring<RING> rg;
    rg.slots = &sm.ring[v][0][0];
    rg.slot_lds = lds_addr_of(&sm.ring[v][0][0]);
    rg.cnt = 0;
    rg.is.tab = tab;
    rg.is.lm = &sm.lm_seg[v];
    rg.is.nseg = oseg + 3;
    rg.is.L = m.L;
    rg.is.wstride = m.layer_elems * m.wbytes;
    rg.is.kvstride = (int64_t)2 * m.hkv * m.S * m.hd * m.kvbytes;
    rg.is.layer = 0;
    rg.is.e = 0;
    rg.is.last = P.blob;
    rg.is.load();
    for (int s = 0; s < RING; ++s) rg.is.issue(rg.slot_lds + s * kPacketBytes);

    int gD, T_unused;
    tile_shape(m, w, kTileD, T_unused, gD);
    for (int layer = 0; layer < m.L; ++layer) {
      wg_barrier();
      if (sm.abort_flag) goto drain;
      consume_rows<RING, WB>(rg, tab[0], m.cd, sm.act, sm.u.part_r[v]);
      wg_barrier();
      for (int k = 0; k < si.nunits; ++k) {
        wg_barrier();
        if (sm.abort_flag) goto drain;
        const Unit u = unit_of(si, w, k, m.nwg);
        consume_attention<RING, KB, HD>(rg, tab[1 + 2 * k], u, m.G, sm, v);
        wg_barrier();
      }
      wg_barrier();
      if (sm.abort_flag) goto drain;
      consume_rows<RING, WB>(rg, tab[oseg], m.cq, sm.act, sm.u.part_r[v]);
      wg_barrier();
      wg_barrier();
      if (sm.abort_flag) goto drain;
      consume_rows<RING, WB>(rg, tab[oseg + 1], m.cd, sm.act, sm.u.part_r[v]);
      wg_barrier();
      wg_barrier();
      if (sm.abort_flag) goto drain;
      consume_cols<RING, WB>(rg, tab[oseg + 2], gD, sm.act, &sm.u.part_c[v][0][0]);
      wg_barrier();
    }
    wg_barrier();
    if (sm.abort_flag) goto drain;
    consume_rows<RING, WB>(rg, sm.lm_seg[v], m.cd, sm.act, sm.u.part_r[v]);
    wg_barrier();
  drain:
    wait_vm<0>();
    return;
  }

  // ============================ control wave ============================
  Ctl<RING> ctl{P, __builtin_amdgcn_make_buffer_rsrc(P.ll, (short)0, (int)(P.lo.total * 8), 0x00020000), sm};
  ctl.build_splits(w);
  const int rows_d0 = p_lo(m.d, m.nwg, w);
  const int nrow_d = p_lo(m.d, m.nwg, w + 1) - rows_d0;
  const int nf = ffn_lo32(m, w + 1) - ffn_lo32(m, w);
  const int r_qkv0 = p_lo(m.nqkv, m.nwg, w), n_qkv = p_lo(m.nqkv, m.nwg, w + 1) - r_qkv0;
  const int r_lm0 = p_lo(m.V, m.nwg, w), n_lm = p_lo(m.V, m.nwg, w + 1) - r_lm0;
  const int gD = nf / m.vpl;
  const int mc = max_chunks(m);

  uint64_t* const tr = P.trace ? P.trace + (int64_t)w * trace_stride(m.L) : nullptr;
  auto stamp = [&](int slot) {
    if (tr && lane == 0) tr[slot] = now_ticks();
  };
  stamp(0);
  // RoPE angles of this step's position, in float64 then rounded to float32
  for (int i = lane; i < m.hd / 2; i += 64) {
    const double theta = pow((double)P.rope_base, -2.0 * (double)i / (double)m.hd);
    const double ang = (double)si.p * theta;
    sm.rope_c[i] = (float)cos(ang);
    sm.rope_s[i] = (float)sin(ang);
  }
  // embedding row of the input token
  for (int i = lane; i < m.d; i += 64) sm.x[i] = load_w<WB>(P.embed, (int64_t)token * m.d + i);

  const float inv_sqrt_hd = 1.0f / sqrtf((float)m.hd);
  stamp(1);
  for (int layer = 0; layer < m.L; ++layer) {
    const uint8_t* g_attn = P.norms + ((int64_t)layer * 2 + 0) * m.d * m.wbytes;
    const uint8_t* g_ffn = P.norms + ((int64_t)layer * 2 + 1) * m.d * m.wbytes;
    // ---- QKV rows ----
    if (layer > 0) ctl.gather_vec(ll_tag(m, P.seq, layer - 1, kX), P.lo.x, m.d, sm.x);
    if (!ctl.failed()) ctl.template rmsnorm<WB>(sm.x, g_attn, sm.act, m.d);
    stamp(trace_slot(m.L, layer, 0));
    wg_barrier();
    if (sm.abort_flag) return;
    wg_barrier();
    stamp(trace_slot(m.L, layer, 1));
    {
      const uint32_t tag = ll_tag(m, P.seq, layer, kQKV);
      for (int r = lane; r < n_qkv; r += 64) ll_store(P.ll, P.lo.qkv + r_qkv0 + r, ctl.row_total(kTileQKV, m.cd, r), tag);
    }
    stamp(trace_slot(m.L, layer, 2));
    // ---- attention units: one chunk of positions of one kv head each ----
    for (int k = 0; k < si.nunits; ++k) {
      const Unit u = unit_of(si, w, k, m.nwg);
      const int G = m.G;
      const int64_t qoff = P.lo.qkv + (int64_t)u.g * G * m.hd;
      const int64_t koff = P.lo.qkv + m.qdim + (int64_t)u.g * m.hd;
      const int64_t voff = P.lo.qkv + m.qdim + m.kvdim + (int64_t)u.g * m.hd;
      const int nq = G * m.hd / 2, nk = m.hd / 2;
      ctl.gather(
          ll_tag(m, P.seq, layer, kQKV), nq + 2 * nk,
          [&](int k2) -> int64_t {
            return k2 < nq ? qoff + 2 * k2 : (k2 < nq + nk ? koff + 2 * (k2 - nq) : voff + 2 * (k2 - nq - nk));
          },
          [&](int k2, float a, float b) {
            if (k2 < nq) {
              const int h = (2 * k2) / m.hd, e = (2 * k2) - h * m.hd;
              sm.u.att.q[h][e] = a;
              sm.u.att.q[h][e + 1] = b;
            } else if (k2 < nq + nk) {
              sm.u.att.kp[2 * (k2 - nq)] = a;
              sm.u.att.kp[2 * (k2 - nq) + 1] = b;
            } else {
              sm.u.att.vp[2 * (k2 - nq - nk)] = a;
              sm.u.att.vp[2 * (k2 - nq - nk) + 1] = b;
            }
          });
      if (!ctl.failed()) {
        // RoPE on q (and the 1/sqrt(hd) score scale) and on k; K and V rounded to the cache type
        const int half = m.hd / 2;
        for (int i = lane; i < half; i += 64) {
          const float c = sm.rope_c[i], s = sm.rope_s[i];
          for (int h = 0; h < G; ++h) {
            const float a = sm.u.att.q[h][i], b = sm.u.att.q[h][i + half];
            sm.u.att.q[h][i] = (a * c - b * s) * inv_sqrt_hd;
            sm.u.att.q[h][i + half] = (a * s + b * c) * inv_sqrt_hd;
          }
          const float a = sm.u.att.kp[i], b = sm.u.att.kp[i + half];
          sm.u.att.kp[i] = a * c - b * s;
          sm.u.att.kp[i + half] = a * s + b * c;
        }
        const int64_t kh = (((int64_t)layer * 2 + 0) * m.hkv + u.g) * m.S + si.p;
        const int64_t vh = (((int64_t)layer * 2 + 1) * m.hkv + u.g) * m.S + si.p;
        for (int i = lane; i < m.hd; i += 64) {
          float kk = sm.u.att.kp[i], vv = sm.u.att.vp[i];
          if constexpr (KB == 2) {
            const uint32_t kb = bf16_rne_bits(kk), vb = bf16_rne_bits(vv);
            kk = __uint_as_float(kb << 16);
            vv = __uint_as_float(vb << 16);
            if (u.last) {
              ((uint16_t*)P.kv)[kh * m.hd + i] = (uint16_t)kb;
              ((uint16_t*)P.kv)[vh * m.hd + i] = (uint16_t)vb;
            }
          } else {
            if (u.last) {
              ((float*)P.kv)[kh * m.hd + i] = kk;
              ((float*)P.kv)[vh * m.hd + i] = vv;
            }
          }
          sm.u.att.kp[i] = kk;
          sm.u.att.vp[i] = vv;
        }
      }
      if (k == 0) stamp(trace_slot(m.L, layer, 3));
      wg_barrier();
      if (sm.abort_flag) return;
      wg_barrier();
      if (k == 0) stamp(trace_slot(m.L, layer, 4));
      // merge the compute waves' partial softmax sums, plus the current position in the last chunk
      if (!ctl.failed()) {
        const uint32_t tag = ll_tag(m, P.seq, layer, kATTP);
        for (int h = 0; h < G; ++h) {
          float sp = -INFINITY;
          if (u.last) {
            float t = 0.f;
            for (int i = lane; i < m.hd; i += 64) t = fmaf(sm.u.att.q[h][i], sm.u.att.kp[i], t);
            sp = wave_sum(t);
          }
          float M = sp;
#pragma unroll
          for (int vv = 0; vv < kComputeWaves; ++vv)
            if (sm.u.att.ml[vv][h][1] > 0.f) M = fmaxf(M, sm.u.att.ml[vv][h][0]);
          float Lsum = 0.f;
#pragma unroll
          for (int vv = 0; vv < kComputeWaves; ++vv) {
            const float lv = sm.u.att.ml[vv][h][1];
            if (lv > 0.f) Lsum = fmaf(__expf(sm.u.att.ml[vv][h][0] - M), lv, Lsum);
          }
          const float sp_w = u.last ? __expf(sp - M) : 0.f;
          Lsum += sp_w;
          const int hq = u.g * G + h;
          const int64_t at = P.lo.attp + ((int64_t)hq * mc + u.c) * (m.hd + 2);
          for (int i = lane; i < m.hd; i += 64) {
            float a = sp_w * sm.u.att.vp[i];
#pragma unroll
            for (int vv = 0; vv < kComputeWaves; ++vv) {
              const float lv = sm.u.att.ml[vv][h][1];
              if (lv > 0.f) a = fmaf(__expf(sm.u.att.ml[vv][h][0] - M), sm.u.att.acc[vv][h][i], a);
            }
            ll_store(P.ll, at + 2 + i, a, tag);
          }
          if (lane == 0) {
            ll_store(P.ll, at, M, tag);
            ll_store(P.ll, at + 1, Lsum, tag);
          }
        }
      }
    }
    stamp(trace_slot(m.L, layer, 5));
    // ---- merge units: one slice of one head's output, over all chunks ----
    for (int k = 0; k < nmerge_here && !ctl.failed(); ++k) {
      const int mu = mfirst + k * m.nwg;
      const int NC = si.ap.NC, MS = si.ap.MS;
      const int per_head = m.hd / MS;
      const int hq = mu / per_head, sl = mu - hq * per_head;
      const int ppc = 1 + MS / 2;  // pieces per chunk: (m, l), then the slice
      const int64_t head_at = P.lo.attp + (int64_t)hq * mc * (m.hd + 2);
      float* st = sm.u.stage;  // [NC][2 + MS]
      ctl.gather(
          ll_tag(m, P.seq, layer, kATTP), NC * ppc,
          [&](int k2) -> int64_t {
            const int c = k2 / ppc, t = k2 - c * ppc;
            const int64_t cb = head_at + (int64_t)c * (m.hd + 2);
            return t == 0 ? cb : cb + 2 + (int64_t)sl * MS + 2 * (t - 1);
          },
          [&](int k2, float a, float b) {
            const int c = k2 / ppc, t = k2 - c * ppc;
            st[c * (2 + MS) + 2 * t] = a;
            st[c * (2 + MS) + 2 * t + 1] = b;
          });
      if (ctl.failed()) break;
      float M = -INFINITY;
      for (int c = lane; c < NC; c += 64) M = fmaxf(M, st[c * (2 + MS)]);
      M = wave_max(M);
      // chunk weights exp(m_c - M), stored over the m_c slots
      float Ls = 0.f;
      for (int c = lane; c < NC; c += 64) {
        const float sc = __expf(st[c * (2 + MS)] - M);
        Ls = fmaf(sc, st[c * (2 + MS) + 1], Ls);
        st[c * (2 + MS)] = sc;
      }
      Ls = wave_sum(Ls);
      const float invL = 1.0f / Ls;
      const uint32_t tag = ll_tag(m, P.seq, layer, kO);
      for (int i = lane; i < MS; i += 64) {
        float a = 0.f;
        for (int c = 0; c < NC; ++c) a = fmaf(st[c * (2 + MS)], st[c * (2 + MS) + 2 + i], a);
        ll_store(P.ll, P.lo.o + (int64_t)hq * m.hd + (int64_t)sl * MS + i, a * invL, tag);
      }
    }
    stamp(trace_slot(m.L, layer, 6));
    // ---- output projection rows + residual ----
    ctl.gather_vec(ll_tag(m, P.seq, layer, kO), P.lo.o, m.qdim, sm.act);
    stamp(trace_slot(m.L, layer, 7));
    wg_barrier();
    if (sm.abort_flag) return;
    wg_barrier();
    stamp(trace_slot(m.L, layer, 8));
    {
      const uint32_t tag = ll_tag(m, P.seq, layer, kXP);
      for (int r = lane; r < nrow_d; r += 64)
        ll_store(P.ll, P.lo.xp + rows_d0 + r, sm.x[rows_d0 + r] + ctl.row_total(kTileO, m.cq, r), tag);
    }
    stamp(trace_slot(m.L, layer, 9));
    // ---- gate/up rows of this workgroup's FFN slice ----
    ctl.gather_vec(ll_tag(m, P.seq, layer, kXP), P.lo.xp, m.d, sm.x);
    if (!ctl.failed()) ctl.template rmsnorm<WB>(sm.x, g_ffn, sm.act, m.d);
    stamp(trace_slot(m.L, layer, 10));
    wg_barrier();
    if (sm.abort_flag) return;
    wg_barrier();
    stamp(trace_slot(m.L, layer, 11));
    for (int i = lane; i < nf; i += 64) {
      const float gt = ctl.row_total(kTileGU, m.cd, i);
      const float up = ctl.row_total(kTileGU, m.cd, nf + i);
      sm.act[i] = gt / (1.0f + __expf(-gt)) * up;
    }
    stamp(trace_slot(m.L, layer, 12));
    // ---- down projection of the slice, for all d rows ----
    wg_barrier();
    if (sm.abort_flag) return;
    wg_barrier();
    stamp(trace_slot(m.L, layer, 13));
    {
      const uint32_t tag = ll_tag(m, P.seq, layer, kDP);
      for (int b = 0; b < m.d / 64; ++b) {
        const int i = b * 64 + lane;
        const float val = gD > 0 ? ctl.block_total(gD, b, lane) : 0.f;
        const int o = p_of(m.d, m.nwg, i);
        const int olo = p_lo(m.d, m.nwg, o), ohi = p_lo(m.d, m.nwg, o + 1);
        ll_store(P.ll, P.lo.dp + (int64_t)olo * m.nwg + (int64_t)w * (ohi - olo) + (i - olo), val, tag);
      }
    }
    stamp(trace_slot(m.L, layer, 14));
    // ---- sum every slice's contribution to this workgroup's rows; residual add ----
    {
      float* st = sm.act;  // [nwg][nrow_d]
      ctl.gather_vec(ll_tag(m, P.seq, layer, kDP), P.lo.dp + (int64_t)rows_d0 * m.nwg, m.nwg * nrow_d, st);
      if (!ctl.failed() && nrow_d > 0) {
        // lane = (row, group of producers); fixed summation order, so results are reproducible
        const int groups = 64 / nrow_d;
        const int r = lane % nrow_d, grp = lane / nrow_d;
        float s = 0.f;
        if (grp < groups)
          for (int pr = grp; pr < m.nwg; pr += groups) s += st[pr * nrow_d + r];
        float tot = 0.f;
        for (int q2 = 0; q2 < groups; ++q2) tot += __shfl(s, q2 * nrow_d + r);
        if (lane < nrow_d) ll_store(P.ll, P.lo.x + rows_d0 + lane, sm.x[rows_d0 + lane] + tot, ll_tag(m, P.seq, layer, kX));
      }
    }
    stamp(trace_slot(m.L, layer, 15));
  }

  // ---- final norm, LM head rows, argmax ----
  ctl.gather_vec(ll_tag(m, P.seq, m.L - 1, kX), P.lo.x, m.d, sm.x);
  if (!ctl.failed()) ctl.template rmsnorm<WB>(sm.x, P.norms + (int64_t)m.L * 2 * m.d * m.wbytes, sm.act, m.d);
  stamp(trace_slot(m.L, m.L, 0));
  wg_barrier();
  if (sm.abort_flag) return;
  wg_barrier();
  stamp(trace_slot(m.L, m.L, 1));
  {
    float best = -INFINITY;
    int32_t besti = 0x7fffffff;
    bool nan = false;
    for (int r = lane; r < n_lm; r += 64) {
      const float val = ctl.row_total(kTileLM, m.cd, r);
      if (P.logits) P.logits[r_lm0 + r] = val;
      if (val != val) { nan = true; continue; }
      if (val > best || (val == best && r_lm0 + r < besti)) { best = val; besti = r_lm0 + r; }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float ob = __shfl_xor(best, o);
      const int32_t oi = __shfl_xor(besti, o);
      if (ob > best || (ob == best && oi < besti)) { best = ob; besti = oi; }
    }
    if (__any(nan) && lane == 0) __hip_atomic_fetch_or(P.status, kStatusNaN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) {
      const uint32_t tag = ll_tag(m, P.seq, m.L, kLM);
      ll_store_bits(P.ll, P.lo.lm + 2 * w, __float_as_uint(best), tag);
      ll_store_bits(P.ll, P.lo.lm + 2 * w + 1, (uint32_t)besti, tag);
    }
  }
  stamp(trace_slot(m.L, m.L, 2));
  if (w == 0) {
    float best = -INFINITY;
    int32_t besti = 0x7fffffff;
    ctl.gather(ll_tag(m, P.seq, m.L, kLM), m.nwg, [&](int k) -> int64_t { return P.lo.lm + 2 * (int64_t)k; },
               [&](int k, float a, float b) {
                 const int32_t idx = (int32_t)__float_as_uint(b);
                 if (a > best || (a == best && idx < besti)) { best = a; besti = idx; }
               });
    if (ctl.failed() || ld_flag(P.abortf)) return;
    for (int o = 32; o > 0; o >>= 1) {
      const float ob = __shfl_xor(best, o);
      const int32_t oi = __shfl_xor(besti, o);
      if (ob > best || (ob == best && oi < besti)) { best = ob; besti = oi; }
    }
    if (lane == 0) {
      P.tokens[0] = besti == 0x7fffffff ? 0 : besti;
      P.positions[0] = si.p + 1;
    }
    stamp(trace_slot(m.L, m.L, 3));
  }
}

}  // namespace kd

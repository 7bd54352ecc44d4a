// kd_device.h -- the persistent decode-step kernel for gfx950.
//
// One launch runs a whole decode step: embedding, every layer, LM head and argmax.
//
// Grid. One workgroup per compute unit, resident for the whole step, as in the
// single-kernel runtime of the Kog engine ("Real-time LLM inference on standard
// data-centre GPUs (3,000 tokens/s single request)", section "technical
// principles"). A workgroup has 8 waves, and all of them do the same kind of work:
//
//  * Streaming. Each wave walks a fixed sequence of 1 KB packets: its share of
//    every weight tile of the step, plus its share of the KV positions of its
//    workgroup's attention units. Packets arrive through a private ring in LDS,
//    filled by LDS-DMA loads (global_load_lds_dwordx4, non-temporal). The loads
//    run up to RING packets ahead, straight across phase boundaries. Weights do
//    not depend on activations, so HBM keeps streaming while the workgroup
//    waits for the previous phase's results. This is the single-GPU form of
//    "keep computing and synchronise later" ("Kog 3000 tok/s real-time
//    inference", section "KCCL").
//  * Exchange. Between phases every wave helps gather the vector the next
//    phase needs. All 512 lanes poll at once, so one round of 16-byte loads
//    covers up to 4096 values.
//
// Exchange between workgroups. Vectors travel as "exchange words": 64-bit words
// with a float in the low half and a tag in the high half. They are written with
// device-scope relaxed atomic stores and read with device-scope 16-byte loads.
// A tag names the step, layer and vector kind, so a reader spins until every
// word it needs carries the expected tag. One round trip therefore does both the
// synchronisation and the data transfer, with no grid-wide barrier and no L2
// writeback or invalidate. Each word is one naturally aligned 64-bit store, so a
// reader never accepts a stale or torn value. Every producer writes its part of
// a vector as one contiguous run.
//
// Layer dataflow (WG = workgroup; every WG does each step for its own slice):
//   x --gather--> RMSNorm --> QKV rows (row split)           --> qkv words
//   q,k,v of one kv head --gather--> RoPE, KV append, attention over a chunk of positions
//                                                            --> partial (max, sum, acc) words
//   partials of one head slice --gather--> log-sum-exp merge --> o words
//   o --gather--> O rows + residual (row split)              --> x' words
//   x' --gather--> RMSNorm --> gate/up rows of this WG's FFN slice; SiLU(gate)*up stays in LDS
//   FFN slice --> down projection of the slice for all d rows --> partial words (per producer)
//   partials of this WG's rows --gather--> fixed-order sum + residual --> x words
#pragma once
#include <hip/hip_runtime.h>

#include "kd_plan.h"

namespace kd {

struct Params {
  const uint8_t* blob;   // packed layer weights and LM head, weight dtype
  const uint8_t* embed;  // [V][d], bf16 (fp8, int8 and bf16 models) or f32
  const uint8_t* norms;  // [L][2][d] attention/FFN gains, then final gain [d], embedding dtype
  const float* scales;   // fp8 or int8 weights: row scales laid out as scale_layout() says (else null)
  const float2* rope;    // [S][hd/2] (cos, sin) of position * theta_i
  uint64_t* ll;          // exchange words
  LLLayout lo;
  uint8_t* kv;           // caller's cache [L][2][B][hkv][S][hd]
  int32_t* tokens;
  int32_t* positions;
  float* logits;
  uint32_t* flags;           // [0] sticky status bits, [3] cancel word (nonzero: abandon the call)
  uint32_t* abortf;          // tag base of the last call a workgroup gave up on
  uint64_t* trace;           // per-workgroup phase timestamps (100 MHz clock), or null
  int32_t* out_tokens;       // multi-step launches: [n_steps] greedy token of every step, or null
  uint32_t* progress;        // multi-step launches: steps completed (system-scope store after each), or null
  uint32_t spin_us;          // longest wait for another workgroup, in microseconds
  uint32_t tag0;             // tag base of step 0; step s uses tag0 + s * tag_stride
  int32_t n_steps;           // multi-step launches: decode steps, each fed the previous step's token
  int32_t max_seq;
  float eps;
  Dims m;
};

constexpr int kFlagStatus = 0, kFlagCancel = 3;  // words of Params::flags
constexpr uint32_t kStatusTokenRange = 0x1u, kStatusPosOverflow = 0x2u, kStatusTimeout = 0x4u, kStatusNaN = 0x8u,
                   kStatusCancelled = 0x10u;
constexpr int kMaxRowsD = 64;                  // most d rows one workgroup owns
constexpr int kMaxSlice = 128;                 // most FFN columns one workgroup owns

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

// Cross-lane moves without LDS: DPP within 16-lane rows, and gfx950's permlane swaps across rows.
// (ds_bpermute-based shuffles would queue behind the LDS-DMA writes of the weight stream.)
constexpr int kDppQuad1 = 0xB1;       // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuad2 = 0x4E;       // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within each 16 lanes
constexpr int kDppRor8 = 0x128;       // lane i <- (i + 8) mod 16 within each 16 lanes: lane ^ 8

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
// {a, b} = this lane's value and that of lane ^ 16 (or ^ 32), in an order that depends on the lane
struct LanePair {
  uint32_t a, b;
};
__device__ __forceinline__ LanePair swap16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return {r[0], r[1]};
}
__device__ __forceinline__ LanePair swap32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return {r[0], r[1]};
}

// Sums over groups of 8 / 16 lanes (every lane of a group ends with the bitwise-same value), and
// butterfly steps that add lane ^ 8, ^ 16, ^ 32. Every step adds two identical operand values in
// both partner lanes, so all lanes of a group always hold the same bits.
__device__ __forceinline__ float sum_rows8(float v) {
  v += dpp_f<kDppQuad1>(v);
  v += dpp_f<kDppQuad2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v;
}
__device__ __forceinline__ float sum_rows16(float v) {
  const float t = sum_rows8(v);
  return t + dpp_f<kDppMirror>(t);
}
__device__ __forceinline__ float xsum8(float v) { return v + dpp_f<kDppRor8>(v); }
__device__ __forceinline__ float xsum16(float v) {
  const LanePair p = swap16(__float_as_uint(v));
  return __uint_as_float(p.a) + __uint_as_float(p.b);
}
__device__ __forceinline__ float xsum32(float v) {
  const LanePair p = swap32(__float_as_uint(v));
  return __uint_as_float(p.a) + __uint_as_float(p.b);
}
__device__ __forceinline__ float xmax8(float v) { return fmaxf(v, dpp_f<kDppRor8>(v)); }
__device__ __forceinline__ float xmax16(float v) {
  const LanePair p = swap16(__float_as_uint(v));
  return fmaxf(__uint_as_float(p.a), __uint_as_float(p.b));
}
__device__ __forceinline__ float xmax32(float v) {
  const LanePair p = swap32(__float_as_uint(v));
  return fmaxf(__uint_as_float(p.a), __uint_as_float(p.b));
}

__device__ __forceinline__ float wave_sum(float v) { return xsum32(xsum16(sum_rows16(v))); }
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuad1>(v));
  v = fmaxf(v, dpp_f<kDppQuad2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return xmax32(xmax16(v));
}

// Sum over the N lanes that hold one KV position (N = 8, 16 or 32 consecutive lanes).
template <int N>
__device__ __forceinline__ float sum_lanes(float v) {
  if constexpr (N == 8) return sum_rows8(v);
  else if constexpr (N == 16) return sum_rows16(v);
  else return xsum16(sum_rows16(v));
}
// Sum over the positions of a packet: lanes with the same index modulo N (N = 8, 16 or 32).
template <int N>
__device__ __forceinline__ float sum_positions(float v) {
  v = xsum32(v);
  if constexpr (N <= 16) v = xsum16(v);
  if constexpr (N <= 8) v = xsum8(v);
  return v;
}
template <int N>
__device__ __forceinline__ float max_positions(float v) {
  v = xmax32(v);
  if constexpr (N <= 16) v = xmax16(v);
  if constexpr (N <= 8) v = xmax8(v);
  return v;
}

// (value, index) maximum over the wave, ties to the lower index; every lane ends with the result.
__device__ __forceinline__ bool better(float b, int32_t ib, float a, int32_t ia) { return b > a || (b == a && ib < ia); }
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& best, int32_t& besti) {
  const float ob = dpp_f<CTRL>(best);
  const int32_t oi = dpp_i<CTRL>(besti);
  if (better(ob, oi, best, besti)) { best = ob; besti = oi; }
}
__device__ __forceinline__ void argmax_swap(LanePair vb, LanePair vi, float& best, int32_t& besti) {
  const float a = __uint_as_float(vb.a), b = __uint_as_float(vb.b);
  const int32_t ia = (int32_t)vi.a, ib = (int32_t)vi.b;
  if (better(b, ib, a, ia)) { best = b; besti = ib; } else { best = a; besti = ia; }
}
__device__ __forceinline__ void wave_argmax(float& best, int32_t& besti) {
  argmax_step<kDppQuad1>(best, besti);
  argmax_step<kDppQuad2>(best, besti);
  argmax_step<kDppHalfMirror>(best, besti);
  argmax_step<kDppMirror>(best, besti);
  argmax_swap(swap16(__float_as_uint(best)), swap16((uint32_t)besti), best, besti);
  argmax_swap(swap32(__float_as_uint(best)), swap32((uint32_t)besti), best, besti);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that waits for LDS traffic only. Each wave's LDS-DMA loads stay in flight
// across it; that is the point of the ring.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 64 lanes x 16 bytes from per-lane global addresses into LDS [lds_addr, lds_addr + 1 KB).
// Non-temporal: weights and KV are read once per step. Waits for this wave's earlier LDS reads
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

// The same load with device-scope coherence (sc1): it sees values another workgroup of the same
// launch stored with device-scope stores, where the plain load could hit a stale line of this
// compute unit's L2. Used for K/V positions appended earlier in the same launch.
__device__ __forceinline__ void dma_packet_coherent(const void* lane_addr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off sc1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(lane_addr)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// device-scope (sc1) 16-byte load of two exchange words, bounds-checked by the buffer descriptor
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
__device__ __forceinline__ int c_div(int a, int b) { return (a + b - 1) / b; }
// FFN columns per slice unit and rows per down block, fixed by the matrix element size (the values
// ffn_unit() and down_block_rows() give, as compile-time constants of each kernel)
template <int WB> constexpr int kFu = WB == 1 ? 8 : 16 / WB;
template <int WB> constexpr int kDbr = WB == 1 ? 128 : 64;
template <int WB>
__device__ __forceinline__ int ffn_lo32(const Dims& m, int w) { return kFu<WB> * p_lo(m.F / kFu<WB>, m.nwg, w); }
// d rows are owned in pairs, so every workgroup's run of exchange words starts 16-byte aligned
__device__ __forceinline__ int drow_lo(const Dims& m, int w) { return 2 * p_lo(m.d / 2, m.nwg, w); }

// ----------------------------------------------------------------------------------------------
// the packet sequence of each wave
// ----------------------------------------------------------------------------------------------
// One contiguous run of packets. `base` is the address of packet 0 at layer 0; kind says how it
// moves with the layer.
enum SegKind : int32_t { kSegWeight = 0, kSegKV = 1, kSegOnce = 2 };
struct SegEntry {
  const uint8_t* base;
  int32_t lo, hi;
  int32_t kind;
  int32_t coh;  // packets from this index on are loaded with device-scope coherence
};
constexpr int32_t kNoCoherent = 0x7fffffff;

// A segment entry read from LDS, marked wave-uniform (every lane reads the same entry), so that the
// loop bounds and packet addresses derived from it stay in scalar registers.
__device__ __forceinline__ SegEntry uniform(const SegEntry& e) {
  SegEntry u;
  const uint64_t b = (uint64_t)(uintptr_t)e.base;
  const uint32_t lo32 = __builtin_amdgcn_readfirstlane((uint32_t)b), hi32 = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  u.base = (const uint8_t*)(uintptr_t)(((uint64_t)hi32 << 32) | lo32);
  u.lo = __builtin_amdgcn_readfirstlane(e.lo);
  u.hi = __builtin_amdgcn_readfirstlane(e.hi);
  u.kind = __builtin_amdgcn_readfirstlane(e.kind);
  u.coh = __builtin_amdgcn_readfirstlane(e.coh);
  return u;
}

// Per-layer order of a wave's segments: QKV, (K, V) of each attention unit, O, gate/up, down.
__device__ __forceinline__ int seg_o(int nunits) { return 1 + 2 * nunits; }

enum Tile : int { kTileQKV = 0, kTileO = 1, kTileGU = 2, kTileD = 3, kTileLM = 4, kTiles = 5 };

template <int RING>
struct Smem {
  uint4 ring[kWaves][RING][64];
  float act[kMaxDim];  // input of the current projection; during attention: per-wave accumulators
  union {
    float stage[kStageWords];  // merge partials, down-projection partials of this WG's rows
    struct {
      float q[kMaxGroup][kMaxHeadDim];  // rotated queries of this unit's kv head, times 1/sqrt(hd)
      float kp[kMaxHeadDim];            // K and V of the current position, as stored
      float vp[kMaxHeadDim];
      float scores[kWaves][kScorePos][kMaxGroup];
      float ml[kWaves][kMaxGroup][2];
      float sp[kMaxGroup];  // score of the current position
    } att;
  } u;
  float rowpart[kWaves][kRowPart];  // per-wave row sums of the current tile
  float xo[kMaxRowsD];              // this WG's rows of x (then x')
  float a[kMaxSlice];               // SiLU(gate)*up of this WG's FFN slice
  float rope_c[kMaxHeadDim / 2];
  float rope_s[kMaxHeadDim / 2];
  float red[kWaves];
  int32_t redi[kWaves];
  SegEntry segs[kWaves][4 + 2 * kMaxUnits];
  SegEntry lm_seg[kWaves];
  int32_t split[kTiles][kWaves + 1];  // wave boundaries of each tile (packets)
  int32_t first[kTiles][kWaves];      // first row / block of each wave's share
  int abort_flag;
  uint32_t cancel;                    // the cancel word as read at the start of the step
  int32_t next_token;                 // the step's greedy token, for the next step of the launch
};

// step-level facts every workgroup derives from the inputs
struct StepInfo {
  int32_t p;  // position of the input token
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

// Packets of each tile of workgroup w, and how many packets a row (or down block) spans.
template <int WB>
__device__ __forceinline__ void tile_shape(const Dims& m, int w, int tile, int& T, int& C) {
  if (tile == kTileQKV) { C = m.cd; T = (p_lo(m.nqkv, m.nwg, w + 1) - p_lo(m.nqkv, m.nwg, w)) * C; }
  else if (tile == kTileO) { C = m.cq; T = (drow_lo(m, w + 1) - drow_lo(m, w)) * C; }
  else if (tile == kTileGU) { C = m.cd; T = 2 * (ffn_lo32<WB>(m, w + 1) - ffn_lo32<WB>(m, w)) * C; }
  else if (tile == kTileD) { C = (ffn_lo32<WB>(m, w + 1) - ffn_lo32<WB>(m, w)) / kFu<WB>; T = (m.d / kDbr<WB>) * C; }
  else { C = m.cd; T = (p_lo(m.V, m.nwg, w + 1) - p_lo(m.V, m.nwg, w)) * C; }
}

// Packet range [lo, hi) of wave v in a tile. The down tile is cut at whole blocks of dbr rows, so
// each block's sum is finished by one wave.
template <int WB>
__device__ __forceinline__ void wave_range(const Dims& m, int w, int tile, int v, int& lo, int& hi) {
  int T, C;
  tile_shape<WB>(m, w, tile, T, C);
  if (tile == kTileD) {
    const int nb = m.d / kDbr<WB>;
    lo = (int)wave_lo(nb, v) * C;
    hi = (int)wave_lo(nb, v + 1) * C;
  } else {
    lo = (int)wave_lo(T, v);
    hi = (int)wave_lo(T, v + 1);
  }
}

// Fill wave v's segment table (done by the wave itself).
// K/V positions from p_new on were appended earlier in this launch (by a multi-step launch), so
// their packets are loaded coherently; p_new = max_seq when no such position exists.
template <int RING, int WB>
__device__ __forceinline__ void build_segments(const Params& P, const StepInfo& si, int w, int v, Smem<RING>& sm,
                                               int p_new) {
  const Dims& m = P.m;
  if (lane_id() != 0) return;
  auto put = [&](SegEntry& e, const uint8_t* base, int lo, int hi, int kind, int coh = kNoCoherent) {
    e.base = base;
    e.lo = lo;
    e.hi = hi;
    e.kind = kind;
    e.coh = coh;
  };
  SegEntry* t = sm.segs[v];
  int lo, hi;
  wave_range<WB>(m, w, kTileQKV, v, lo, hi);
  put(t[0], P.blob + (m.off_qkv + (int64_t)p_lo(m.nqkv, m.nwg, w) * m.d) * m.wbytes, lo, hi, kSegWeight);
  for (int k = 0; k < si.nunits; ++k) {
    const Unit u = unit_of(si, w, k, m.nwg);
    const int n = u.j1 > u.j0 ? c_div(u.j1 - u.j0, m.ppp) : 0;
    const int64_t kbase = (((int64_t)0 * 2 + 0) * m.hkv + u.g) * m.S + u.j0;
    const int64_t vbase = (((int64_t)0 * 2 + 1) * m.hkv + u.g) * m.S + u.j0;
    const int coh = p_new < u.j1 ? max(p_new - u.j0, 0) / m.ppp : kNoCoherent;  // packet holding p_new
    put(t[1 + 2 * k], P.kv + kbase * m.hd * m.kvbytes, p_lo(n, kWaves, v), p_lo(n, kWaves, v + 1), kSegKV, coh);
    put(t[2 + 2 * k], P.kv + vbase * m.hd * m.kvbytes, p_lo(n, kWaves, v), p_lo(n, kWaves, v + 1), kSegKV, coh);
  }
  const int o = seg_o(si.nunits);
  wave_range<WB>(m, w, kTileO, v, lo, hi);
  put(t[o], P.blob + (m.off_o + (int64_t)drow_lo(m, w) * m.qdim) * m.wbytes, lo, hi, kSegWeight);
  wave_range<WB>(m, w, kTileGU, v, lo, hi);
  put(t[o + 1], P.blob + (m.off_gu + (int64_t)2 * ffn_lo32<WB>(m, w) * m.d) * m.wbytes, lo, hi, kSegWeight);
  wave_range<WB>(m, w, kTileD, v, lo, hi);
  put(t[o + 2], P.blob + (m.off_d + (int64_t)m.d * ffn_lo32<WB>(m, w)) * m.wbytes, lo, hi, kSegWeight);
  wave_range<WB>(m, w, kTileLM, v, lo, hi);
  put(sm.lm_seg[v], P.blob + (m.off_lm + (int64_t)p_lo(m.V, m.nwg, w) * m.d) * m.wbytes, lo, hi, kSegOnce);
}

// Walks this wave's packet sequence ahead of the consumer and issues the loads. COH: the launch
// runs several steps, so packets from a segment's `coh` index on are loaded coherently.
template <bool COH>
struct Issuer {
  const SegEntry* tab;
  const SegEntry* lm;
  int nseg, L;
  int64_t wstride, kvstride;
  int layer, e;  // layer == L: the LM head; layer > L: past the end
  const uint8_t* base;
  int32_t idx, hi, coh;
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
      const SegEntry s = uniform(layer < L ? tab[e] : *lm);
      if (s.hi > s.lo) {
        base = s.base + (s.kind == kSegWeight ? layer * wstride : (s.kind == kSegKV ? layer * kvstride : 0));
        idx = s.lo;
        hi = s.hi;
        coh = s.coh;
        return;
      }
      next_entry();
    }
  }
  // Issue the next packet of the sequence into an LDS slot; past the end, reload the last one,
  // so that every slot is always covered by exactly one load in flight.
  __device__ __forceinline__ void issue(uint32_t slot_addr) {
    const uint8_t* a = last;
    bool c = false;
    if (layer <= L) {
      a = base + (int64_t)idx * kPacketBytes;
      if constexpr (COH) c = idx >= coh;
      last = a;
      if (++idx == hi) { next_entry(); load(); }
    }
    if (COH && c) dma_packet_coherent(a + lane_id() * 16, slot_addr);
    else dma_packet(a + lane_id() * 16, slot_addr);
  }
};

// Consumer side of the ring: take the next packet (waiting for its load), then give the slot back.
template <int RING, bool COH>
struct Ring {
  const uint4* slots;  // this wave's RING x 64 x 16 bytes
  uint32_t slot_lds;   // LDS address of slot 0
  uint32_t cnt;
  Issuer<COH> is;
  __device__ __forceinline__ uint4 take() const {
    // RING loads were issued after the oldest one's slot was last refilled, minus nothing: any
    // other memory operation issued since only makes this wait longer, never shorter.
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
// Eight fp8 E4M3 weights (two 32-bit words) times a[0..8). gfx950's packed conversion reads the
// OCP E4M3 format: byte k of a word becomes element k of the pair it selects.
__device__ __forceinline__ float dot8_fp8(uint32_t lo, uint32_t hi, const float* a) {
  const float4 a0 = *(const float4*)a, a1 = *(const float4*)(a + 4);
  const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false), p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const auto p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false), p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  float s = p0[0] * a0.x;
  s = fmaf(p0[1], a0.y, s);
  s = fmaf(p1[0], a0.z, s);
  s = fmaf(p1[1], a0.w, s);
  s = fmaf(p2[0], a1.x, s);
  s = fmaf(p2[1], a1.y, s);
  s = fmaf(p3[0], a1.z, s);
  s = fmaf(p3[1], a1.w, s);
  return s;
}

// Eight int8 weights (two 32-bit words, byte k is element k) times a[0..8). Each signed byte
// converts to float exactly (one sign-extending byte-select conversion per element).
__device__ __forceinline__ float dot8_i8(uint32_t lo, uint32_t hi, const float* a) {
  const float4 a0 = *(const float4*)a, a1 = *(const float4*)(a + 4);
  float s = (float)(int8_t)lo * a0.x;
  s = fmaf((float)(int8_t)(lo >> 8), a0.y, s);
  s = fmaf((float)(int8_t)(lo >> 16), a0.z, s);
  s = fmaf((float)((int32_t)lo >> 24), a0.w, s);
  s = fmaf((float)(int8_t)hi, a1.x, s);
  s = fmaf((float)(int8_t)(hi >> 8), a1.y, s);
  s = fmaf((float)(int8_t)(hi >> 16), a1.z, s);
  s = fmaf((float)((int32_t)hi >> 24), a1.w, s);
  return s;
}

// Eight 1-byte codes times a[0..8): E4M3 or (I8) int8.
template <bool I8>
__device__ __forceinline__ float dot8_q8(uint32_t lo, uint32_t hi, const float* a) {
  if constexpr (I8) return dot8_i8(lo, hi, a);
  else return dot8_fp8(lo, hi, a);
}

// One 16-byte lane load of weights times the matching activation values (16 one-byte codes, 8 bf16
// or 4 f32). I8: the one-byte codes are int8, else E4M3.
template <int WB, bool I8 = false>
__device__ __forceinline__ float dot16(const uint4 w, const float* a) {
  if constexpr (WB == 1) {
    return dot8_q8<I8>(w.x, w.y, a) + dot8_q8<I8>(w.z, w.w, a + 8);
  } else if constexpr (WB == 2) {
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

// Row-split matrix-vector product over packets [s.lo, s.hi): packets are row chunks of 64*vpl
// values; act is the input vector. A row's lane sums are reduced across the wave when the row (or
// this wave's share of it) ends; part[r - first row] receives the wave's sum.
template <int RING, int WB, bool COH, bool I8>
// (The segment is taken by value: a copy in registers is not reloaded from LDS after every
// LDS-DMA refill, whose asm clobbers memory.)
__device__ __forceinline__ void consume_rows(Ring<RING, COH>& rg, const SegEntry s, int C, const float* act, float* part) {
  constexpr int VPL = 16 / WB;
  const int lane = lane_id();
  int r = s.lo / C;
  const int r_first = r;
  int c = s.lo - r * C;
  float acc = 0.f;
  for (int i = s.lo; i < s.hi; ++i) {
    const uint4 wv = rg.take();
    acc += dot16<WB, I8>(wv, act + c * (64 * VPL) + lane * VPL);
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

// Down projection of this WG's FFN slice over the wave's whole 64-row blocks: packets hold 64 rows
// x vpl columns; lane l owns row 64*b + l, and all lanes read the same slice values. Each finished
// block is published at once as 64 contiguous exchange words.
template <int RING, int WB, bool COH, bool I8>
__device__ __forceinline__ void consume_down(Ring<RING, COH>& rg, const SegEntry s, int g, const float* a, uint64_t* ll,
                                             int64_t dp_at, uint32_t tag) {
  const int lane = lane_id();
  if constexpr (WB == 1) {
    // one-byte codes: 128-row blocks; lane l sums row 128 b + l from the first 8 bytes of its pieces and row
    // 128 b + 64 + l from the last 8, over 8 slice columns per packet
    int b = s.lo / g;
    int j = 0;
    float acc0 = 0.f, acc1 = 0.f;
    for (int i = s.lo; i < s.hi; ++i) {
      const uint4 wv = rg.take();
      acc0 += dot8_q8<I8>(wv.x, wv.y, a + j * 8);
      acc1 += dot8_q8<I8>(wv.z, wv.w, a + j * 8);
      rg.give();
      if (++j == g) {
        ll_store(ll, dp_at + (int64_t)b * 128 + lane, acc0, tag);
        ll_store(ll, dp_at + (int64_t)b * 128 + 64 + lane, acc1, tag);
        acc0 = acc1 = 0.f;
        j = 0;
        ++b;
      }
    }
    return;
  }
  constexpr int VPL = 16 / WB;
  int b = s.lo / g;
  int j = 0;
  float acc = 0.f;
  for (int i = s.lo; i < s.hi; ++i) {
    const uint4 wv = rg.take();
    acc += dot16<WB, I8>(wv, a + j * VPL);
    rg.give();
    if (++j == g) {
      ll_store(ll, dp_at + (int64_t)b * 64 + lane, acc, tag);
      acc = 0.f;
      j = 0;
      ++b;
    }
  }
}

// Lanes 0-31 get the sum of x over lanes l and l ^ 32, lanes 32-63 the sum of y (gfx950's
// permlane32 swap exchanges the upper half of its first operand with the lower half of its
// second). halve16 does the same one level down: even 16-lane rows get x, odd rows get y.
__device__ __forceinline__ float halve32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halve16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scores, then the exp-weighted V sum, of one attention unit over this wave's share of the
// unit's cached positions. lpp lanes hold one position; each lane holds kv_vpl of its dims.
// Leaves (max, sum) in ml[v] and the weighted V sums in accv[h][hd].
//
// Branch-free: all kMaxGroup head slots are computed (slots h >= G get q = 0 and are never read
// back), and positions past the unit's end are masked by selects, so the LDS reads of a packet
// are issued together rather than one per branch.
template <int RING, int KB, int HD, bool COH>
__device__ __forceinline__ void consume_attention(Ring<RING, COH>& rg, const SegEntry sk, const Unit& u, int G, Smem<RING>& sm,
                                                  int v, float* accv) {
  constexpr int KVPL = 16 / KB;
  constexpr int LPP = HD / KVPL;
  constexpr int PPP = 64 / LPP;
  constexpr int H = kMaxGroup;
  static_assert(H == 4, "scores are stored as one float4 per position");
  const int lane = lane_id();
  const int q_in = lane / LPP;  // position inside a packet
  const int dim0 = (lane % LPP) * KVPL;
  float qv[H][KVPL];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int e = 0; e < KVPL; ++e) {
      const float t = sm.u.att.q[h][dim0 + e];
      qv[h][e] = h < G ? t : 0.f;
    }
  float mh[H];
#pragma unroll
  for (int h = 0; h < H; ++h) mh[h] = -INFINITY;
  // pass 1: scores (q already carries 1/sqrt(hd))
  for (int i = sk.lo; i < sk.hi; ++i) {
    const uint4 kw = rg.take();
    float kf[KVPL];
    unpack16<KB>(kw, kf);
    rg.give();
    const bool valid = u.j0 + i * PPP + q_in < u.j1;
    float sc[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < KVPL; ++e) t = fmaf(qv[h][e], kf[e], t);
      sc[h] = sum_lanes<LPP>(t);
      mh[h] = valid ? fmaxf(mh[h], sc[h]) : mh[h];
    }
    if (lane % LPP == 0)
      *(float4*)&sm.u.att.scores[v][(i - sk.lo) * PPP + q_in][0] = make_float4(sc[0], sc[1], sc[2], sc[3]);
  }
#pragma unroll
  for (int h = 0; h < H; ++h) mh[h] = max_positions<LPP>(mh[h]);
  // pass 2: V weighted by exp(score - wave max); masked positions add nothing (their cache
  // slots may hold anything, so the sums are selected rather than multiplied by zero)
  float acc[H][KVPL];
  float lsum[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < KVPL; ++e) acc[h][e] = 0.f;
  }
  for (int i = sk.lo; i < sk.hi; ++i) {
    const uint4 vw = rg.take();
    float vf[KVPL];
    unpack16<KB>(vw, vf);
    rg.give();
    const bool valid = u.j0 + i * PPP + q_in < u.j1;
    const float4 s4 = *(const float4*)&sm.u.att.scores[v][(i - sk.lo) * PPP + q_in][0];
    const float s[H] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const float e = __expf(s[h] - mh[h]);
      lsum[h] = valid ? lsum[h] + e : lsum[h];
#pragma unroll
      for (int k = 0; k < KVPL; ++k) acc[h][k] = valid ? fmaf(e, vf[k], acc[h][k]) : acc[h][k];
    }
  }
#pragma unroll
  for (int h = 0; h < H; ++h) lsum[h] = sum_positions<LPP>(lsum[h]);
  // Sum acc over the PPP position groups by halving: each level pairs value j with value
  // j + n/2 and keeps one of them per half, so lane l ends with the totals of a block of values
  // (block l >> 4 of four when PPP >= 4, l >> 5 of two when PPP == 2).
  constexpr int NV = H * KVPL;
  float a[NV];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int k = 0; k < KVPL; ++k) a[h * KVPL + k] = acc[h][k];
#pragma unroll
  for (int j = 0; j < NV / 2; ++j) a[j] = halve32(a[j], a[j + NV / 2]);
  if constexpr (PPP >= 4) {
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) a[j] = halve16(a[j], a[j + NV / 4]);
  }
  if constexpr (PPP >= 8) {
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) a[j] = xsum8(a[j]);
  }
  constexpr int NR = PPP == 2 ? NV / 2 : NV / 4;  // values each lane ends with
  const int blk = PPP == 2 ? (lane >> 5) : (lane >> 4);
  if (PPP < 8 || (lane & 8) == 0) {
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int vi = blk * NR + j, h = vi / KVPL, k = vi - h * KVPL;
      accv[h * HD + dim0 + k] = a[j];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
      sm.u.att.ml[v][h][0] = mh[h];
      sm.u.att.ml[v][h][1] = lsum[h];
    }
  }
}

// ----------------------------------------------------------------------------------------------
// exchange
// ----------------------------------------------------------------------------------------------
template <int RING>
struct Xchg {
  const Params& P;
  __amdgpu_buffer_rsrc_t llr;
  Smem<RING>& sm;

  // Give up on this launch: record why, and name it (by its tag base) in the abort word, which
  // only the workgroups of this launch compare against. A later launch runs normally.
  __device__ __forceinline__ void fail(uint32_t bit) {
    if (lane_id() == 0) {
      __hip_atomic_fetch_or(P.flags + kFlagStatus, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(P.abortf, P.tag0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sm.abort_flag = 1;
  }

  // All 512 threads: collect npieces 16-byte pieces (two exchange words each) at word offsets
  // off(k); each wave waits until both words of each of its pieces carry `tag`, then hands the two
  // floats of piece k to sink(k, a, b). Ends with a workgroup barrier; returns false if the step
  // was abandoned (timeout here or elsewhere).
  template <class Off, class Sink>
  __device__ __forceinline__ bool gather(uint32_t tag, int npieces, Off off, Sink sink) {
    return gather(tag, npieces, off, sink, [] {});
  }
  // As above; fin() runs on every thread after its last sink call, before the closing barrier.
  template <class Off, class Sink, class Fin>
  __device__ __forceinline__ bool gather(uint32_t tag, int npieces, Off off, Sink sink, Fin fin) {
    constexpr int NB = 4;
    const int tid = (int)threadIdx.x;
    for (int base = 0; base < npieces; base += kThreads * NB) {
      uint4 val[NB];
      uint64_t t0 = 0;
      bool started = false;
      bool dead = false;
      for (int spin = 0;; ++spin) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int k = base + tid + kThreads * i;
          if (k < npieces) val[i] = ll_load2(llr, off(k));
        }
        bool ok = true;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int k = base + tid + kThreads * i;
          if (k < npieces) ok = ok && val[i].y == tag && val[i].w == tag;
        }
        if (__all(ok)) break;
        if (!started) { t0 = now_ticks(); started = true; }
        if ((spin & 15) == 15) {
          if (now_ticks() - t0 > (uint64_t)P.spin_us * 100u) { fail(kStatusTimeout); dead = true; break; }
          if (ld_flag(P.flags + kFlagCancel)) { fail(kStatusCancelled); dead = true; break; }
          if (ld_flag(P.abortf) == P.tag0 || sm.abort_flag) { sm.abort_flag = 1; dead = true; break; }
        }
      }
      if (dead) break;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int k = base + tid + kThreads * i;
        if (k < npieces) sink(k, __uint_as_float(val[i].x), __uint_as_float(val[i].z));
      }
    }
    fin();
    wg_barrier();
    // the same LDS word for every lane: say so, so that the branch on it stays uniform
    return __builtin_amdgcn_readfirstlane(sm.abort_flag) == 0;
  }

  // Gather n consecutive exchange words (n even) starting at word `at` into dst[0..n).
  __device__ __forceinline__ bool gather_vec(uint32_t tag, int64_t at, int n, float* dst) {
    return gather(tag, n / 2, [&](int k) { return at + 2 * (int64_t)k; },
                  [&](int k, float a, float b) {
                    dst[2 * k] = a;
                    dst[2 * k + 1] = b;
                  });
  }
};

// RMSNorm folded into the gather of the vector it normalises. The projection after a norm is
// linear, so W (x r g) = r W (x g) with r = 1 / sqrt(mean(x^2) + eps): the gather stores x g and
// sums x^2 as the pieces arrive, and the projection's outputs are scaled by r when they are
// published. No separate pass over the vector and no extra barrier.
//
// A full-vector gather hands thread tid the pieces tid + kThreads i (elements 2 (tid + kThreads i)
// and + 1), in order of i; the gains of those elements are loaded into registers first, so their
// latency hides behind the wait.
constexpr int kPieceRegs = kMaxDim / (2 * kThreads);
template <int WB>
__device__ __forceinline__ void load_piece_gains(const uint8_t* gain, int d, float2 (&g)[kPieceRegs]) {
  const int tid = (int)threadIdx.x;
  // no branches: loads issued back to back are waited for together, by the gather's first poll
#pragma unroll
  for (int i = 0; i < kPieceRegs; ++i) {
    const int e = min(2 * (tid + kThreads * i), d - 2);
    if constexpr (WB == 2) {
      const uint32_t u = ((const uint32_t*)gain)[e / 2];
      g[i] = make_float2(bf16_lo(u), bf16_hi(u));
    } else {
      g[i] = *(const float2*)((const float*)gain + e);
    }
  }
}

// Per-thread state of a folded norm: the gains of the thread's pieces and its sum of squares.
struct NormFold {
  float2 g[kPieceRegs];
  float ss;
  // piece k (= tid + kThreads i) holds x[2k], x[2k+1]: store them times their gains, add squares
  __device__ __forceinline__ void put(float* act, int k, float a, float b) {
    const int i = (k - (int)threadIdx.x) / kThreads;
    // select rather than index, so the gains stay in registers
    float2 gi = g[0];
#pragma unroll
    for (int j = 1; j < kPieceRegs; ++j) gi = i == j ? g[j] : gi;
    act[2 * k] = a * gi.x;
    act[2 * k + 1] = b * gi.y;
    ss = fmaf(a, a, ss);
    ss = fmaf(b, b, ss);
  }
  // this wave's sum of squares into red[wave] (before the barrier that ends the gather)
  template <class S>
  __device__ __forceinline__ void finish(S& sm) {
    const float t = wave_sum(ss);
    if (lane_id() == 0) sm.red[wave_id()] = t;
  }
};

// The norm's scale r from the waves' sums of squares (after the barrier), summed in wave order.
template <int RING>
__device__ __forceinline__ float norm_scale(const Smem<RING>& sm, int d, float eps) {
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += sm.red[w];
  return 1.0f / sqrtf(tot / (float)d + eps);
}

// Total of row r (C packets per row) of a tile over the waves that touched it, in wave order.
// Branch-free: all the wave bounds, then all the candidate partial sums, are read before use.
template <int RING>
__device__ __forceinline__ float row_total(const Smem<RING>& sm, int tile, int C, int r) {
  const int a = r * C, b = a + C;
  int lo[kWaves + 1], fi[kWaves];
#pragma unroll
  for (int v = 0; v <= kWaves; ++v) lo[v] = sm.split[tile][v];
#pragma unroll
  for (int v = 0; v < kWaves; ++v) fi[v] = sm.first[tile][v];
  float p[kWaves];
#pragma unroll
  for (int v = 0; v < kWaves; ++v) p[v] = sm.rowpart[v][min(max(r - fi[v], 0), kRowPart - 1)];
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const bool touched = lo[v] < lo[v + 1] && lo[v] < b && lo[v + 1] > a;
    s = touched ? s + p[v] : s;
  }
  return s;
}

// Timestamp slot of phase-boundary `ev` (layer < L) or of the final phases (layer == L).
__device__ __forceinline__ int trace_slot(int layer, int ev) { return 2 + kTraceLayerEvents * layer + ev; }

// ----------------------------------------------------------------------------------------------
// the kernel
// ----------------------------------------------------------------------------------------------
// Every wave executes the same sequence of workgroup barriers. A failed wait sets the LDS abort
// flag before the barrier that ends its gather; all waves test the flag right after that barrier
// and leave together, after their LDS-DMA loads have landed.
// MULTI: the launch may run several steps (kd_generate); without it the kernel runs exactly one,
// with no step loop and no coherent-load choice in the streaming loops.
// I8 (with WB = 1): the one-byte matrix codes are int8 instead of E4M3.
template <int RING, int WB, int KB, int HD, bool MULTI, bool I8 = false>
__global__ __launch_bounds__(kThreads, 1) void decode_step_kernel(const Params P_arg) {
  __shared__ Smem<RING> sm;
  // work on a private copy: references into the kernel-argument segment would force a stack copy
  const Params P = P_arg;
  const Dims m = P.m;
  constexpr int EB = WB == 1 ? 2 : WB;  // embedding and norm gains: bf16 when the matrices are 1-byte codes
  constexpr bool Q8 = WB == 1;          // matrices hold E4M3 or int8 codes; each row's total is times its scale
  static_assert(Q8 || !I8, "int8 codes are one byte");
  const ScaleLayout scl_at = Q8 ? scale_layout(m) : ScaleLayout{};
  const int w = (int)blockIdx.x;
  const int tid = (int)threadIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();

  // inputs of the launch; every thread of every workgroup takes the same decision
  const int32_t token0 = P.tokens[0];
  const int32_t p0 = P.positions[0];
  if (token0 < 0 || token0 >= m.V || p0 < 0 || p0 >= P.max_seq) {
    if (w == 0 && tid == 0) {
      uint32_t bit = (token0 < 0 || token0 >= m.V) ? kStatusTokenRange : 0u;
      if (p0 < 0 || p0 >= P.max_seq) bit |= kStatusPosOverflow;
      __hip_atomic_fetch_or(P.flags + kFlagStatus, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  // a launch of several steps appends positions p0, p0 + 1, ... and reads them back in later steps
  const int n_steps = MULTI ? P.n_steps : 1;
  const int p_new = n_steps > 1 ? p0 : P.max_seq;

  const int rd0 = drow_lo(m, w), nrd = drow_lo(m, w + 1) - rd0;  // this WG's d rows (O, x ownership)
  const int f0 = ffn_lo32<WB>(m, w), nf = ffn_lo32<WB>(m, w + 1) - f0;  // this WG's FFN slice
  const int rq0 = p_lo(m.nqkv, m.nwg, w), nq = p_lo(m.nqkv, m.nwg, w + 1) - rq0;
  const int rl0 = p_lo(m.V, m.nwg, w), nl = p_lo(m.V, m.nwg, w + 1) - rl0;
  const int gD = nf / kFu<WB>;  // down packets per block of dbr rows
  const int mc = max_chunks(m);

  // Phase timestamps go to LDS and are copied out at the end of the launch (the last step's): a
  // global store here would hold up the next memory wait of wave 0 (stores share the in-order
  // vector memory counter with the loads).
  uint64_t* const tr = P.trace ? P.trace + (int64_t)w * trace_stride(m.L) : nullptr;
  __shared__ uint64_t trl[kTraceMaxSlots];
  const int trn = (int)trace_stride(m.L);
  if (tr)
    for (int i = tid; i < trn; i += kThreads) trl[i] = 0;
  auto stamp = [&](int slot) {
    if (tr && tid == 0) trl[slot] = now_ticks();
  };

  // ---- once per launch: the wave split of every tile ----
  if (tid == 0) sm.abort_flag = 0;
  if (tid < kTiles) {
    for (int v = 0; v <= kWaves; ++v) {
      int lo, hi;
      wave_range<WB>(m, w, tid, v < kWaves ? v : kWaves - 1, lo, hi);
      sm.split[tid][v] = v < kWaves ? lo : hi;
    }
    int T, C;
    tile_shape<WB>(m, w, tid, T, C);
    for (int v = 0; v < kWaves; ++v) sm.first[tid][v] = C > 0 ? sm.split[tid][v] / C : 0;
  }

  Xchg<RING> xc{P, __builtin_amdgcn_make_buffer_rsrc(P.ll, (short)0, (int)(P.lo.total * 8), 0x00020000), sm};
  const float inv_sqrt_hd = 1.0f / sqrtf((float)m.hd);
  const SegEntry* tab = sm.segs[wave];
  NormFold fold;
  float r_attn = 1.f, r_ffn = 1.f, r_final = 1.f;  // scales of the folded norms
  Ring<RING, MULTI> rg;
  rg.slots = &sm.ring[wave][0][0];
  rg.slot_lds = lds_addr_of(&sm.ring[wave][0][0]);
  int32_t token = token0;

  for (int step = 0; step < n_steps; ++step) {
  const uint32_t tb0 = P.tag0 + (uint32_t)step * tag_stride(m);  // this step's tag base
  StepInfo si{};
  si.p = p0 + step;
  if (step > 0) {
    if (si.p >= P.max_seq) {  // the cache is full: the launch ends here (same decision everywhere)
      if (w == 0 && tid == 0) __hip_atomic_fetch_or(P.flags + kFlagStatus, kStatusPosOverflow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      goto drain;
    }
    // the previous step's loads have landed and every wave is done with the LDS tables
    wait_vm<0>();
    wg_barrier();
    token = __builtin_amdgcn_readfirstlane(sm.next_token);
  }
  stamp(0);
  si.ap = att_plan(m, si.p);
  si.nunits = w < si.ap.units ? c_div(si.ap.units - w, m.nwg) : 0;
  {
  const int mfirst = m.nwg - 1 - w;  // merge units are dealt from the last workgroup down
  const int nmerge_here = mfirst < si.ap.nmerge ? c_div(si.ap.nmerge - mfirst, m.nwg) : 0;
  const int oseg = seg_o(si.nunits);

  // ---- setup of the step: segment tables, ring, RoPE row, embedding row, cancel word ----
  if (tid == 0) sm.cancel = ld_flag(P.flags + kFlagCancel);
  build_segments<RING, WB>(P, si, w, wave, sm, p_new);
  for (int i = tid; i < m.hd / 2; i += kThreads) {
    const float2 cs = P.rope[(int64_t)si.p * (m.hd / 2) + i];
    sm.rope_c[i] = cs.x;
    sm.rope_s[i] = cs.y;
  }
  for (int i = tid; i < m.d; i += kThreads) sm.act[i] = load_w<EB>(P.embed, (int64_t)token * m.d + i);
  wg_barrier();  // segment tables and the cancel word visible

  rg.cnt = 0;
  rg.is.tab = sm.segs[wave];
  rg.is.lm = &sm.lm_seg[wave];
  rg.is.nseg = oseg + 3;
  rg.is.L = m.L;
  rg.is.wstride = m.layer_elems * m.wbytes;
  rg.is.kvstride = (int64_t)2 * m.hkv * m.S * m.hd * m.kvbytes;
  rg.is.layer = 0;
  rg.is.e = 0;
  rg.is.last = P.blob;
  rg.is.load();
  for (int s = 0; s < RING; ++s) rg.is.issue(rg.slot_lds + s * kPacketBytes);
  if (__builtin_amdgcn_readfirstlane(sm.cancel)) {  // cancelled before the step began: leave like a failed wait
    if (tid == 0) {
      __hip_atomic_fetch_or(P.flags + kFlagStatus, kStatusCancelled, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(P.abortf, P.tag0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    goto drain;
  }
  stamp(1);

  for (int layer = 0; layer < m.L; ++layer) {
    const uint8_t* g_attn = P.norms + ((int64_t)layer * 2 + 0) * m.d * EB;
    const uint8_t* g_ffn = P.norms + ((int64_t)layer * 2 + 1) * m.d * EB;
    // row scales of this layer (fp8 or int8 codes): each thread that publishes a row loads its scale ahead of the
    // gather before it, so the load's latency hides behind that wait
    const float* const scl = Q8 ? P.scales + (int64_t)layer * scl_at.layer : nullptr;
    float s_q = 1.f;
    if constexpr (Q8)
      if (tid < nq) s_q = scl[rq0 + tid];
    // ---- x (this WG's rows kept raw for the residual), RMSNorm folded into the gather ----
    load_piece_gains<EB>(g_attn, m.d, fold.g);
    fold.ss = 0.f;
    {
      auto put_x = [&](int k, float a, float b) {
        fold.put(sm.act, k, a, b);
        const int e = 2 * k - rd0;  // rd0 and nrd are even
        if (e >= 0 && e < nrd) {
          sm.xo[e] = a;
          sm.xo[e + 1] = b;
        }
      };
      if (layer > 0) {
        if (!xc.gather(ll_tag(tb0, layer - 1, kX), m.d / 2, [&](int k) -> int64_t { return P.lo.x + 2 * (int64_t)k; },
                       put_x, [&] { fold.finish(sm); }))
          goto drain;
      } else {
        // the embedding row is already in act: fold it in place
#pragma unroll
        for (int i = 0; i < kPieceRegs; ++i) {
          const int k = tid + kThreads * i;
          if (2 * k < m.d) put_x(k, sm.act[2 * k], sm.act[2 * k + 1]);
        }
        fold.finish(sm);
        wg_barrier();
      }
    }
    r_attn = norm_scale(sm, m.d, P.eps);
    stamp(trace_slot(layer, 0));
    stamp(trace_slot(layer, 1));
    // ---- QKV rows ----
    consume_rows<RING, WB, MULTI, I8>(rg, uniform(tab[0]), m.cd, sm.act, sm.rowpart[wave]);
    wg_barrier();
    stamp(trace_slot(layer, 2));
    if (tid < nq)
      ll_store(P.ll, P.lo.qkv + rq0 + tid, row_total(sm, kTileQKV, m.cd, tid) * r_attn * s_q, ll_tag(tb0, layer, kQKV));
    stamp(trace_slot(layer, 3));
    // ---- attention units: one chunk of positions of one kv head each ----
    for (int k = 0; k < si.nunits; ++k) {
      const Unit u = unit_of(si, w, k, m.nwg);
      const int G = m.G;
      const int64_t qoff = P.lo.qkv + (int64_t)u.g * G * m.hd;
      const int64_t koff = P.lo.qkv + m.qdim + (int64_t)u.g * m.hd;
      const int64_t voff = P.lo.qkv + m.qdim + m.kvdim + (int64_t)u.g * m.hd;
      const int nqp = G * m.hd / 2, nkp = m.hd / 2;
      const bool ok = xc.gather(
          ll_tag(tb0, layer, kQKV), nqp + 2 * nkp,
          [&](int k2) -> int64_t {
            return k2 < nqp ? qoff + 2 * k2 : (k2 < nqp + nkp ? koff + 2 * (k2 - nqp) : voff + 2 * (k2 - nqp - nkp));
          },
          [&](int k2, float a, float b) {
            if (k2 < nqp) {
              const int h = (2 * k2) / m.hd, e = (2 * k2) - h * m.hd;
              sm.u.att.q[h][e] = a;
              sm.u.att.q[h][e + 1] = b;
            } else if (k2 < nqp + nkp) {
              sm.u.att.kp[2 * (k2 - nqp)] = a;
              sm.u.att.kp[2 * (k2 - nqp) + 1] = b;
            } else {
              sm.u.att.vp[2 * (k2 - nqp - nkp)] = a;
              sm.u.att.vp[2 * (k2 - nqp - nkp) + 1] = b;
            }
          });
      if (!ok) goto drain;
      if (k == 0) stamp(trace_slot(layer, 4));
      {
        // RoPE on the G queries (with the 1/sqrt(hd) score scale) and on k; K and V rounded to the
        // cache type, and appended by the unit that holds the last chunk
        const int half = m.hd / 2;
        if (tid < (G + 1) * half) {
          const int h = tid / half, i = tid - h * half;
          const float c = sm.rope_c[i], s = sm.rope_s[i];
          float* vec = h < G ? sm.u.att.q[h] : sm.u.att.kp;
          const float a = vec[i], b = vec[i + half];
          const float sc = h < G ? inv_sqrt_hd : 1.0f;
          vec[i] = (a * c - b * s) * sc;
          vec[i + half] = (a * s + b * c) * sc;
        }
        wg_barrier();
        if (k == 0) stamp(trace_slot(layer, 5));
        if (tid < m.hd) {
          const int i = tid;
          float kk = sm.u.att.kp[i], vv = sm.u.att.vp[i];
          if constexpr (KB == 2) {
            kk = __uint_as_float(bf16_rne_bits(kk) << 16);
            vv = __uint_as_float(bf16_rne_bits(vv) << 16);
          }
          sm.u.att.kp[i] = kk;
          sm.u.att.vp[i] = vv;
        }
        wg_barrier();
        if (k == 0) stamp(trace_slot(layer, 6));
        if (u.last) {
          // append K and V at position p as 32-bit words with device-scope stores, so a later step
          // of the same launch reads them on another compute unit (coherent loads, see Issuer)
          constexpr int EPW = 4 / KB;  // cache elements per word
          const int nw = m.hd / EPW;
          if (tid < 2 * nw) {
            const int kvs = tid / nw, j = tid - kvs * nw;  // slot 0: K, 1: V
            const float* src = kvs ? sm.u.att.vp : sm.u.att.kp;
            uint32_t word;
            if constexpr (KB == 2) word = (__float_as_uint(src[2 * j]) >> 16) | (__float_as_uint(src[2 * j + 1]) & 0xffff0000u);
            else word = __float_as_uint(src[j]);
            const int64_t row = (((int64_t)layer * 2 + kvs) * m.hkv + u.g) * m.S + si.p;
            __hip_atomic_store((uint32_t*)(P.kv + row * m.hd * KB) + j, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      // score of the current position (last chunk only), one wave per query head
      if (u.last && wave < G) {
        float t = 0.f;
        for (int i = lane; i < m.hd; i += 64) t = fmaf(sm.u.att.q[wave][i], sm.u.att.kp[i], t);
        t = wave_sum(t);
        if (lane == 0) sm.u.att.sp[wave] = t;
      }
      consume_attention<RING, KB, HD, MULTI>(rg, uniform(tab[1 + 2 * k]), u, G, sm, wave, sm.act + (int64_t)wave * kMaxGroup * HD);
      if (k == 0) stamp(trace_slot(layer, 7));
      wg_barrier();
      if (k == 0) stamp(trace_slot(layer, 8));
      // combine the waves' partial softmax sums (plus the current position in the last chunk)
      if (tid < G * m.hd) {
        const int h = tid / m.hd, i = tid - h * m.hd;
        const float sp = u.last ? sm.u.att.sp[h] : -INFINITY;
        float mv[kWaves], lv[kWaves], av[kWaves];
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
          mv[v] = sm.u.att.ml[v][h][0];
          lv[v] = sm.u.att.ml[v][h][1];
          av[v] = sm.act[((int64_t)v * kMaxGroup + h) * HD + i];
        }
        float M = sp;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) M = lv[v] > 0.f ? fmaxf(M, mv[v]) : M;
        float Lsum = 0.f, acc = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
          // a wave with no positions here contributes nothing (its slots may hold stale values)
          const float sc = __expf(mv[v] - M);
          Lsum = lv[v] > 0.f ? fmaf(sc, lv[v], Lsum) : Lsum;
          acc = lv[v] > 0.f ? fmaf(sc, av[v], acc) : acc;
        }
        if (u.last) {
          const float e = __expf(sp - M);
          Lsum += e;
          acc = fmaf(e, sm.u.att.vp[i], acc);
        }
        const uint32_t tag = ll_tag(tb0, layer, kATTP);
        const int hq = u.g * G + h;
        const int64_t at = P.lo.attp + ((int64_t)hq * mc + u.c) * (m.hd + 2);
        ll_store(P.ll, at + 2 + i, acc, tag);
        if (i == 0) {
          ll_store(P.ll, at, M, tag);
          ll_store(P.ll, at + 1, Lsum, tag);
        }
      }
      if (k == 0) stamp(trace_slot(layer, 9));
      // the per-wave sums must stay readable until every thread has combined them: clear the
      // unused wave slots of the next unit only after this barrier
      wg_barrier();
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
        if (lane == 0) sm.u.att.ml[wave][h][1] = 0.f;
    }
    stamp(trace_slot(layer, 10));
    // ---- merge units: one slice of one head's output, over all chunks ----
    for (int k = 0; k < nmerge_here; ++k) {
      const int mu = mfirst + k * m.nwg;
      const int NC = si.ap.NC, MS = si.ap.MS;
      const int per_head = m.hd / MS;
      const int hq = mu / per_head, sl = mu - hq * per_head;
      const int ppc = 1 + MS / 2;  // pieces per chunk: (m, l), then the slice
      const int64_t head_at = P.lo.attp + (int64_t)hq * mc * (m.hd + 2);
      float* st = sm.u.stage;  // [NC][2 + MS]
      const bool ok = xc.gather(
          ll_tag(tb0, layer, kATTP), NC * ppc,
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
      if (!ok) goto drain;
      if (k == 0) stamp(trace_slot(layer, 11));
      if (wave == 0) {
        float M = -INFINITY;
        for (int c = lane; c < NC; c += 64) M = fmaxf(M, st[c * (2 + MS)]);
        M = wave_max(M);
        // each chunk's weight once (act is free between the attention units and the o gather)
        float* wts = sm.act;
        float Ls = 0.f;
        for (int c = lane; c < NC; c += 64) {
          const float e = __expf(st[c * (2 + MS)] - M);
          wts[c] = e;
          Ls = fmaf(e, st[c * (2 + MS) + 1], Ls);
        }
        Ls = wave_sum(Ls);
        const float invL = 1.0f / Ls;
        const uint32_t tag = ll_tag(tb0, layer, kO);
        if (MS >= 8 && MS <= 64) {
          // lane = (chunk group cg, element i): cg sums chunks cg, cg + CG, ...; then a fixed
          // butterfly over the chunk groups (lanes i + MS, i + 2 MS, ...)
          const int CG = 64 / MS, i = lane % MS, cg = lane / MS;
          float a = 0.f;
#pragma unroll 4
          for (int c = cg; c < NC; c += CG) a = fmaf(wts[c], st[c * (2 + MS) + 2 + i], a);
          if (MS <= 8) a = xsum8(a);
          if (MS <= 16) a = xsum16(a);
          if (MS <= 32) a = xsum32(a);
          if (cg == 0) ll_store(P.ll, P.lo.o + (int64_t)hq * m.hd + (int64_t)sl * MS + i, a * invL, tag);
        } else {
          for (int i = lane; i < MS; i += 64) {
            float a = 0.f;
#pragma unroll 8
            for (int c = 0; c < NC; ++c) a = fmaf(wts[c], st[c * (2 + MS) + 2 + i], a);
            ll_store(P.ll, P.lo.o + (int64_t)hq * m.hd + (int64_t)sl * MS + i, a * invL, tag);
          }
        }
      }
      wg_barrier();
    }
    stamp(trace_slot(layer, 12));
    // ---- output projection rows + residual ----
    float s_o = 1.f;
    if constexpr (Q8)
      if (tid < nrd) s_o = scl[scl_at.o + rd0 + tid];
    if (!xc.gather_vec(ll_tag(tb0, layer, kO), P.lo.o, m.qdim, sm.act)) goto drain;
    stamp(trace_slot(layer, 13));
    consume_rows<RING, WB, MULTI, I8>(rg, uniform(tab[oseg]), m.cq, sm.act, sm.rowpart[wave]);
    wg_barrier();
    stamp(trace_slot(layer, 14));
    if (tid < nrd) {
      const float xp = sm.xo[tid] + row_total(sm, kTileO, m.cq, tid) * s_o;
      sm.xo[tid] = xp;
      ll_store(P.ll, P.lo.xp + rd0 + tid, xp, ll_tag(tb0, layer, kXP));
    }
    stamp(trace_slot(layer, 15));
    // ---- gate/up rows of this workgroup's FFN slice ----
    float s_g = 1.f, s_u = 1.f;
    if constexpr (Q8)
      if (tid < nf) {
        s_g = scl[scl_at.gu + 2 * f0 + tid];
        s_u = scl[scl_at.gu + 2 * f0 + nf + tid];
      }
    load_piece_gains<EB>(g_ffn, m.d, fold.g);
    fold.ss = 0.f;
    if (!xc.gather(ll_tag(tb0, layer, kXP), m.d / 2, [&](int k) -> int64_t { return P.lo.xp + 2 * (int64_t)k; },
                   [&](int k, float a, float b) { fold.put(sm.act, k, a, b); }, [&] { fold.finish(sm); }))
      goto drain;
    r_ffn = norm_scale(sm, m.d, P.eps);
    stamp(trace_slot(layer, 16));
    stamp(trace_slot(layer, 17));
    consume_rows<RING, WB, MULTI, I8>(rg, uniform(tab[oseg + 1]), m.cd, sm.act, sm.rowpart[wave]);
    wg_barrier();
    stamp(trace_slot(layer, 18));
    if (tid < nf) {
      const float gt = row_total(sm, kTileGU, m.cd, tid) * r_ffn * s_g;
      const float up = row_total(sm, kTileGU, m.cd, nf + tid) * r_ffn * s_u;
      sm.a[tid] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;  // hardware reciprocal (1 ulp)
    }
    wg_barrier();
    stamp(trace_slot(layer, 19));
    // ---- down projection of the slice, for all d rows, published block by block ----
    consume_down<RING, WB, MULTI, I8>(rg, uniform(tab[oseg + 2]), gD, sm.a, P.ll, P.lo.dp + (int64_t)w * m.d, ll_tag(tb0, layer, kDP));
    stamp(trace_slot(layer, 20));
    // ---- sum every slice's contribution to this workgroup's rows; residual add ----
    {
      float* st = sm.u.stage;  // [nrd][nwg]: each row's partials contiguous (conflict-free reads)
      const int hp = nrd / 2;  // pieces per producer
      // T = kThreads / nrd threads per row when nrd is a power of two from 8 to 64, else one wave
      // per row (see below); fp8 or int8: the scale of the row this thread finishes, loaded ahead
      float s_d = 1.f;
      if constexpr (Q8) {
        const bool pt = nrd >= 8 && nrd <= 64 && (nrd & (nrd - 1)) == 0;
        const int rr = pt ? tid / (kThreads / max(nrd, 1)) : wave;
        if (rr < nrd) s_d = scl[scl_at.d + rd0 + rr];
      }
      const bool ok = nrd == 0 ||
                      xc.gather(
                          ll_tag(tb0, layer, kDP), m.nwg * hp,
                          [&](int k2) -> int64_t {
                            const int q = k2 / hp, j = k2 - q * hp;
                            return P.lo.dp + (int64_t)q * m.d + rd0 + 2 * j;
                          },
                          [&](int k2, float a, float b) {
                            const int q = k2 / hp, j = k2 - q * hp;
                            st[(2 * j) * m.nwg + q] = a;
                            st[(2 * j + 1) * m.nwg + q] = b;
                          });
      if (!ok) goto drain;
      stamp(trace_slot(layer, 21));
      // T = kThreads / nrd threads per row when nrd is a power of two from 8 to 64: thread j of a
      // row adds producers j, j + T, ... in order, then a fixed butterfly over the T lanes;
      // otherwise one wave per row
      if (nrd >= 8 && nrd <= 64 && (nrd & (nrd - 1)) == 0) {
        const int T = kThreads / nrd, r = tid / T, j = tid - r * T;
        float s = 0.f;
#pragma unroll 8
        for (int q = j; q < m.nwg; q += T) s += st[r * m.nwg + q];
        if (T >= 64) s = wave_sum(s);
        else if (T == 32) s = xsum16(sum_rows16(s));
        else if (T == 16) s = sum_rows16(s);
        else s = sum_rows8(s);
        if (j == 0) ll_store(P.ll, P.lo.x + rd0 + r, sm.xo[r] + s * s_d, ll_tag(tb0, layer, kX));
      } else {
        for (int r = wave; r < nrd; r += kWaves) {
          float s = 0.f;
          for (int q = lane; q < m.nwg; q += 64) s += st[r * m.nwg + q];
          s = wave_sum(s);
          if constexpr (Q8) s *= r == wave ? s_d : scl[scl_at.d + rd0 + r];
          if (lane == 0) ll_store(P.ll, P.lo.x + rd0 + r, sm.xo[r] + s, ll_tag(tb0, layer, kX));
        }
      }
      // no barrier: the staging area is next written after the next layer's x gather, which
      // ends with a workgroup barrier
    }
    stamp(trace_slot(layer, 22));
  }

  // ---- final norm, LM head rows, argmax ----
  float s_l = 1.f;  // fp8 or int8: scale of this thread's first LM-head row
  if constexpr (Q8)
    if (tid < nl) s_l = P.scales[scl_at.lm + rl0 + tid];
  load_piece_gains<EB>(P.norms + (int64_t)m.L * 2 * m.d * EB, m.d, fold.g);
  fold.ss = 0.f;
  if (!xc.gather(ll_tag(tb0, m.L - 1, kX), m.d / 2, [&](int k) -> int64_t { return P.lo.x + 2 * (int64_t)k; },
                 [&](int k, float a, float b) { fold.put(sm.act, k, a, b); }, [&] { fold.finish(sm); }))
    goto drain;
  r_final = norm_scale(sm, m.d, P.eps);
  stamp(trace_slot(m.L, 0));
  consume_rows<RING, WB, MULTI, I8>(rg, uniform(sm.lm_seg[wave]), m.cd, sm.act, sm.rowpart[wave]);
  wg_barrier();
  stamp(trace_slot(m.L, 1));
  {
    float best = -INFINITY;
    int32_t besti = 0x7fffffff;
    bool nan = false;
    for (int r = tid; r < nl; r += kThreads) {
      float val = row_total(sm, kTileLM, m.cd, r) * r_final;
      if constexpr (Q8) val *= r == tid ? s_l : P.scales[scl_at.lm + rl0 + r];
      if (P.logits) P.logits[(int64_t)step * m.V + rl0 + r] = val;
      if (val != val) { nan = true; continue; }
      if (better(val, rl0 + r, best, besti)) { best = val; besti = rl0 + r; }
    }
    wave_argmax(best, besti);
    if (__any(nan) && lane == 0) __hip_atomic_fetch_or(P.flags + kFlagStatus, kStatusNaN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) {
      sm.red[wave] = best;
      sm.redi[wave] = besti;
    }
    wg_barrier();
    if (tid == 0) {
      for (int v = 1; v < kWaves; ++v)
        if (better(sm.red[v], sm.redi[v], best, besti)) { best = sm.red[v]; besti = sm.redi[v]; }
      const uint32_t tag = ll_tag(tb0, m.L, kLM);
      ll_store_bits(P.ll, P.lo.lm + 2 * w, __float_as_uint(best), tag);
      ll_store_bits(P.ll, P.lo.lm + 2 * w + 1, (uint32_t)besti, tag);
    }
  }
  stamp(trace_slot(m.L, 2));
  // Workgroup 0 writes the step's outputs. When another step follows, every workgroup takes the
  // argmax itself (the same bits from the same words), so the next token needs no further hop.
  if (w == 0 || step + 1 < n_steps) {
    const bool ok = xc.gather(ll_tag(tb0, m.L, kLM), m.nwg, [&](int k) -> int64_t { return P.lo.lm + 2 * (int64_t)k; },
                              [&](int k, float a, float b) {
                                sm.u.stage[2 * k] = a;
                                sm.u.stage[2 * k + 1] = b;
                              });
    // (every workgroup's LM words are in, so none of them gave up: the decision is uniform)
    if (!ok) goto drain;
    if (wave == 0) {
      float best = -INFINITY;
      int32_t besti = 0x7fffffff;
      for (int k = lane; k < m.nwg; k += 64) {
        const float a = sm.u.stage[2 * k];
        const int32_t idx = (int32_t)__float_as_uint(sm.u.stage[2 * k + 1]);
        if (better(a, idx, best, besti)) { best = a; besti = idx; }
      }
      wave_argmax(best, besti);
      if (lane == 0) {
        const int32_t next = besti == 0x7fffffff ? 0 : besti;
        sm.next_token = next;  // read after the barrier that opens the next step
        if (w == 0 && (!MULTI || !P.progress)) {
          P.tokens[0] = next;
          P.positions[0] = si.p + 1;
          if (MULTI && P.out_tokens) P.out_tokens[step] = next;
        } else if (MULTI && w == 0) {
          // outputs written through to memory and complete before the count that announces them
          __hip_atomic_store(P.tokens, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          __hip_atomic_store(P.positions, si.p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          if (P.out_tokens) __hip_atomic_store(P.out_tokens + step, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          wait_vm<0>();
          __hip_atomic_store(P.progress, (uint32_t)(step + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
      }
    }
    stamp(trace_slot(m.L, 3));
  }
  }  // the step's plan
  }  // steps
drain:
  wait_vm<0>();
  if (tr) {
    wg_barrier();
    for (int i = tid; i < trn; i += kThreads) tr[i] = trl[i];
  }
}

}  // namespace kd

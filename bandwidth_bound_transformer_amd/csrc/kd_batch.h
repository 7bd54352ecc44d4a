// kd_batch.h -- decode step of B > 1 sessions stepped in lockstep, for gfx950.
//
// All due sessions advance together, so each weight is read once per tick for the whole group
// rather than once per session ("Why is real-time AI inference 56x more expensive? Continuous
// inference and resident kernels", section "advance all active sessions in lockstep"). With
// B sessions the projections become small-M GEMMs: B rows (padded to 64) times the weight matrix.
// They run on the matrix cores (v_mfma_f32_16x16x32_bf16) so that they stay bound by the weight
// stream instead of by fp32 vector arithmetic. Activations are fp32; each is fed to the matrix
// cores as a bf16 pair (hi = bf16(x), lo = bf16(x - hi)), two products per weight, so the result
// keeps about 16 significant bits of the activation instead of 8.
//
// One tick is a fixed sequence of kernels on the caller's stream (no host work between them):
//   check --> embed+norm --> per layer:
//     QKV GEMM --> reduce+RoPE+KV append --> attention chunks --> merge (o as hi/lo)
//     --> O GEMM --> residual+norm --> gate/up GEMM --> SiLU*up (hi/lo) --> down GEMM
//     --> residual+norm (next layer's norm, or the final one)
//   --> LM-head GEMM (logits) --> argmax (next token, position + 1)
// A GEMM writes split-K partial sums; the kernel after it adds them in a fixed order, so results
// are bitwise reproducible.
//
// The same sequence runs a prefill pass (kd_prefill): up to 128 consecutive prompt positions of one
// session as the rows, all sharing its cache. Then the GEMMs take eight 16-row tiles, and the
// attention is prefill_attention_kernel, which loads each chunk of the cache once for every row of
// the pass and computes scores and weighted sums on the matrix cores.
#pragma once
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace kd {
namespace bt {

constexpr int kM = 64;             // sessions padded to four 16-row MFMA tiles
constexpr int kMPrefill = 128;     // prefill positions per pass: eight 16-row tiles
// A GEMM workgroup covers 128 output columns with 8 waves. With 64 activation rows (session
// ticks) each wave owns one 16-column weight block, and two workgroups share a CU, so one's
// start-up and barrier waits overlap the other's streaming (measured: the 11B tick 1% shorter than
// with 4 waves of two blocks). With 128 rows (prefill) each wave owns two blocks, so that every
// activation fragment it reads from LDS feeds two products (one block per wave made the 8B prefill
// 15% slower), and the waves split each 128-K chunk in two halves: waves w and w + 4 take the same
// blocks over K 0-63 and 64-127 of every chunk, and their sums are added once at the end. The
// prefill tile's 139 KB of LDS leaves one workgroup per CU, so this gives every SIMD two waves.
constexpr int kNB = 128;           // GEMM output columns per workgroup
__host__ __device__ constexpr int gemm_waves(int) { return 8; }
__host__ __device__ constexpr int gemm_threads(int mt) { return 64 * gemm_waves(mt); }
constexpr int kKC = 128;           // K per LDS chunk of the activation block
constexpr int kAttThreads = 256;   // 4 waves; 16 lanes per KV position (hd = 128, bf16)
constexpr int kChunk = 512;        // KV positions per attention workgroup (twice that for large session batches)
constexpr int kMaxG = 4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float32 -> bfloat16, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f_to_bf16(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split_hilo(float x, uint16_t& hi, uint16_t& lo) {
  hi = f_to_bf16(x);
  lo = f_to_bf16(x - bf16_to_f(hi));
}

// Sum over each group of 16 lanes (every lane of the group gets the same bits), without LDS.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dppf<0xB1>(v);   // lane ^ 1
  v += dppf<0x4E>(v);   // lane ^ 2
  v += dppf<0x141>(v);  // half-row mirror: groups of 4 -> 8
  v += dppf<0x140>(v);  // row mirror: groups of 8 -> 16
  return v;
}
// {this lane, lane ^ 16} and {this lane, lane ^ 32} (order depends on the lane)
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float wsum(float v) {
  float a, b;
  v = sum16(v);
  swap16(v, a, b);
  v = a + b;
  swap32(v, a, b);
  return a + b;
}

// ---------------------------------------------------------------------------------------------
// tick validation: every later kernel of the tick reads *skip and writes nothing when it is set
// ---------------------------------------------------------------------------------------------
// A nonzero cancel word skips the tick too (status bit 0x10).
__global__ void check_kernel(const int32_t* tokens, const int32_t* positions, int B, int V, int max_seq,
                             uint32_t* status, uint32_t* skip, const uint32_t* cancel) {
  uint32_t bits = 0;
  for (int b = 0; b < B; ++b) {
    if (tokens[b] < 0 || tokens[b] >= V) bits |= 0x1u;
    if (positions[b] < 0 || positions[b] >= max_seq) bits |= 0x2u;
  }
  if (__hip_atomic_load(cancel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) bits |= 0x10u;
  if (bits) __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  *skip = bits ? 1u : 0u;
}

// ---------------------------------------------------------------------------------------------
// one-byte weights (E4M3 or int8 codes with a float32 scale per row) decoded to bf16
// ---------------------------------------------------------------------------------------------
// The prefill engine of an fp8 or int8 model computes with the weights the codes stand for, code
// times its row's scale, rounded to bf16 once here (the pass is bound by the matrix cores, not by
// the weight bytes). Row r of codes[rows][cols] goes to row (r / bin) * bout + boff + r % bin of
// dst (bin = bout = rows, boff = 0 keeps the order; the gate/up interleave uses bin 32, bout 64).
// Grid: one thread per code.
__global__ void dequant_rows_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scale, int rows,
                                    int cols, int int8, int bin, int bout, int boff, uint16_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * cols) return;
  const int64_t r = i / cols, c = i - r * cols;
  const uint32_t code = codes[i];
  const float v = int8 ? (float)(int8_t)code : __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
  dst[((r / bin) * bout + boff + r % bin) * (int64_t)cols + c] = f_to_bf16(v * scale[r]);
}

// ---------------------------------------------------------------------------------------------
// weight tiles: the layout the GEMM streams
// ---------------------------------------------------------------------------------------------
// A weight matrix W[N][K] is stored as tiles of 16 rows x 32 K (1 KB), tile (r, t) at index
// r * (K / 32) + t, each in the lane order of the matrix-core B operand: the 16 bytes of lane l
// are W[16 r + l % 16][32 t + 8 (l / 16) .. + 8]. One 64-lane load then reads one whole tile,
// 1 KB contiguous, and a wave walks its 16 rows as one contiguous run.
// Grid: one thread per 16-byte piece (N * K / 8 of them).
__global__ void tile_pack_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int N, int K) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)N * K / 8) return;
  const int lane = (int)(i & 63);
  const int64_t tile = i >> 6;
  const int64_t per_row_block = K / 32;
  const int64_t rb = tile / per_row_block, t = tile - rb * per_row_block;
  const int64_t row = rb * 16 + (lane & 15), k = t * 32 + (lane >> 4) * 8;
  ((u32x4*)dst)[i] = *(const u32x4*)(src + row * K + k);
}

// ---------------------------------------------------------------------------------------------
// one-byte weight tiles for the session GEMM
// ---------------------------------------------------------------------------------------------
// With fp8 or int8 weights a lane's 16 bytes hold two 32-K tiles: the first 8 codes are its part
// of tile 2 p (W[16 r + l % 16][64 p + 8 (l / 16) .. + 8]), the last 8 its part of tile 2 p + 1
// (the same 8 columns 32 further on), so a 64-lane load reads two tiles, 1 KB contiguous. Tile pair
// (r, p) sits at index r * (K / 64) + p. Grid: one thread per 16-byte piece (N * K / 16).
__global__ void tile_pack_q8_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int N, int K) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)N * K / 16) return;
  const int lane = (int)(i & 63);
  const int64_t pair = i >> 6, per_row_block = K / 64;
  const int64_t rb = pair / per_row_block, p = pair - rb * per_row_block;
  const int64_t row = rb * 16 + (lane & 15), k = p * 64 + (lane >> 4) * 8;
  const uint2 a = *(const uint2*)(src + row * K + k), b = *(const uint2*)(src + row * K + k + 32);
  ((u32x4*)dst)[i] = u32x4{a.x, a.y, b.x, b.y};
}

// Two bf16 values from bytes 2 H and 2 H + 1 of a word of one-byte codes (Q = 1: E4M3, 2: int8).
// Both formats' values are bf16 values, so taking the top half of the float is exact.
template <int Q, bool H>
__device__ __forceinline__ uint32_t code_pair_bf16(uint32_t w) {
  float f0, f1;
  if constexpr (Q == 1) {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, H);
    f0 = f[0];
    f1 = f[1];
  } else {
    f0 = (float)(int8_t)(w >> (H ? 16 : 0));
    f1 = (float)(int8_t)(w >> (H ? 24 : 8));
  }
  return (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
}
// The B operand of one 32-K tile: bf16 weights as loaded (Q = 0), or tile `half` of a two-tile
// load of one-byte codes, decoded.
template <int Q>
__device__ __forceinline__ bf16x8 weight_frag(u32x4 v, int half) {
  if constexpr (Q == 0) {
    return __builtin_bit_cast(bf16x8, v);
  } else {
    const uint32_t w0 = half ? v.z : v.x, w1 = half ? v.w : v.y;
    const u32x4 r = {code_pair_bf16<Q, false>(w0), code_pair_bf16<Q, true>(w0), code_pair_bf16<Q, false>(w1),
                     code_pair_bf16<Q, true>(w1)};
    return __builtin_bit_cast(bf16x8, r);
  }
}

// ---------------------------------------------------------------------------------------------
// small-M GEMM on MFMA: P[s][m][n] = sum over K-range s of (Ahi[m][k] + Alo[m][k]) * W[n][k]
// ---------------------------------------------------------------------------------------------
// Grid: (N / kNB) * KS workgroups of gemm_waves(MT) waves; unit u covers columns [kNB (u / KS), + kNB)
// and K range u % KS, in chunks of 128 K. Wave w owns JW = 1 or 2 16-row tiles of W (16 JW output
// columns), so every activation fragment it reads from LDS feeds JW products, and KH = 1 or 2
// parts of each chunk's four 32-K steps (KH = 2: waves w and w + 4 share blocks, one K half each).
// Per chunk a lane loads the 1 KB tiles of its K part of each of its row blocks (W in the tile
// layout above), straight into registers in the B-operand layout.
//
// The weights (HBM) and the activation block (64 rows x 128 K, hi and lo; it stays in L2) are
// loaded into registers kPF chunks ahead, in the same order, so a wait for one never holds up
// the other. The activation chunk then goes through a double-buffered LDS tile that the
// workgroup's waves share.
constexpr int kPF = 2;  // chunks in flight per wave
// NCH chunks per K range, fully unrolled: with no loop back-edge the compiler places every wait
// exactly (at a back-edge it would drain all loads in flight).
//
// SILU (gate/up without a K split only): instead of partial sums, the workgroup writes
// SiLU(gate) * up of its 64 FFN columns as the hi/lo activation block Ohi/Olo of the down
// projection. Its 128 rows are two groups of [32 gate rows; the 32 up rows of the same columns].
// MT: 16-row tiles of the activation block (4: up to 64 rows, the session ticks; 8: up to 128, prefill).
// Q: 0 bf16 weight tiles; 1 (E4M3) or 2 (int8) one-byte tiles (64 rows only), decoded to bf16 in
// registers, each output column then times scale[n], its row's scale.
template <int NCH, bool SILU, int MT, int Q>
__global__ __launch_bounds__(gemm_threads(MT)) void gemm_kernel(const uint16_t* __restrict__ W, int N, int K,
                                                                const uint16_t* __restrict__ Ahi,
                                                                const uint16_t* __restrict__ Alo, int lda,
                                                                float* __restrict__ P, int KS, int B, const uint32_t* skip,
                                                                uint16_t* __restrict__ Ohi, uint16_t* __restrict__ Olo,
                                                                const float* __restrict__ scale) {
  if (*skip) return;
  // [buffer][hi, lo][row][16-byte piece of the 128-K chunk, padded against bank conflicts]. The pad
  // was measured: two pieces for 64 rows (the 11B tick 1.1% shorter than with one; 72 KB, still two
  // workgroups per CU), one for 128 rows (the 8B prefill 4% shorter than with two).
  constexpr int kRows = 16 * MT;
  constexpr int kPadPieces = MT == 8 ? 1 : 2;
  constexpr int kHiLoShift = MT == 8 ? 11 : 10;  // piece index -> hi/lo half: log2(kRows * 16)
  static_assert(MT == 4 || MT == 8, "64 or 128 rows");
  __shared__ u32x4 As[2][2][kRows][kKC / 8 + kPadPieces];
  const int unit = (int)blockIdx.x;
  const int nb = unit / KS, s = unit - nb * KS;
  const int k0 = s * (NCH * kKC);
  const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q = lane >> 4;
  constexpr int kThr = gemm_threads(MT), KH = MT == 8 ? 2 : 1, JW = kNB / 16 / (gemm_waves(MT) / KH);
  constexpr int NT = 4 / KH;  // 32-K steps of a chunk per wave
  const int kh = KH == 1 ? 0 : wave / (gemm_waves(MT) / KH);  // this wave's K part of every chunk
  const int rb0 = nb * (kNB / 16) + JW * (KH == 1 ? wave : wave % (gemm_waves(MT) / KH));  // its JW 16-row blocks
  static_assert(Q == 0 || MT == 4, "one-byte weights for the 64-row tile only");
  constexpr int TPL = Q ? 2 : 1;  // 32-K tiles per 16-byte lane load
  constexpr int NWL = NT / TPL;   // weight loads per block per chunk
  const u32x4* wt[JW];
#pragma unroll
  for (int j = 0; j < JW; ++j)
    wt[j] = (const u32x4*)W + ((size_t)(rb0 + j) * (K / (32 * TPL)) + k0 / (32 * TPL)) * 64 + lane;

  // activation chunk: 2 x kRows rows x 16 pieces of 16 bytes, 4 (or 8) per thread
  constexpr int kAPer = 2 * kRows * (kKC / 8) / kThr;
  // ext_vector_type registers (HIP's uint4 is a struct with a union, which the compiler keeps in
  // scratch memory when it sits in an array)
  struct Slot {
    u32x4 a[kAPer];
    u32x4 w[JW][NWL];
  };
  auto load_chunk = [&](int c, Slot& sl) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
      const int idx = tid + kThr * j;
      const int hl = idx >> kHiLoShift, r = (idx >> 4) & (kRows - 1), cc = idx & 15;
      sl.a[j] = *(const u32x4*)((hl ? Alo : Ahi) + (size_t)r * lda + k0 + c * kKC + cc * 8);
    }
    // weights are read once per tick: non-temporal loads
#pragma unroll
    for (int j = 0; j < JW; ++j)
#pragma unroll
      for (int t = 0; t < NWL; ++t) sl.w[j][t] = __builtin_nontemporal_load(wt[j] + (size_t)(c * (4 / TPL) + kh * NWL + t) * 64);
  };

  f32x4 acc[JW][MT];
#pragma unroll
  for (int j = 0; j < JW; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one chunk: activation slot -> LDS buffer, barrier, 64 MFMAs, then refill the slot kPF ahead
  auto step = [&](int c, Slot& sl) __attribute__((always_inline)) {
    const int buf = c & 1;
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
      const int idx = tid + kThr * j;
      const int hl = idx >> kHiLoShift, r = (idx >> 4) & (kRows - 1), cc = idx & 15;
      As[buf][hl][r][cc] = sl.a[j];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tk = kh * NT + t;  // 32-K step of the chunk
      bf16x8 bw[JW];
#pragma unroll
      for (int j = 0; j < JW; ++j) bw[j] = weight_frag<Q>(sl.w[j][t / TPL], t % TPL);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // lane l supplies K = 32 tk + 8 (l / 16) .. + 8 of row 16 mt + l % 16: piece 4 tk + l / 16
        const int r = mt * 16 + (lane & 15);
        const bf16x8 ah = __builtin_bit_cast(bf16x8, As[buf][0][r][tk * 4 + q]);
        const bf16x8 al = __builtin_bit_cast(bf16x8, As[buf][1][r][tk * 4 + q]);
#pragma unroll
        for (int j = 0; j < JW; ++j) {
          acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw[j], acc[j][mt], 0, 0, 0);
          acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw[j], acc[j][mt], 0, 0, 0);
        }
      }
    }
    if (c + kPF < NCH) load_chunk(c + kPF, sl);
  };
  Slot ring[kPF];
#pragma unroll
  for (int c = 0; c < kPF && c < NCH; ++c) load_chunk(c, ring[c]);
#pragma unroll
  for (int c = 0; c < NCH; ++c) step(c, ring[c % kPF]);
  const int cw = 16 * (rb0 - nb * (kNB / 16));  // this wave's first column within the workgroup
  if constexpr (Q != 0) {
    // one-byte weights: each output column times its row's scale
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const float sc = scale[(rb0 + j) * 16 + (lane & 15)];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[j][mt] *= sc;
    }
  }
  if constexpr (KH == 2) {
    // the second K half's sums through LDS (As is free once every wave is past its last chunk),
    // added to the first half's; the waves of the second half then write nothing
    constexpr int LDR = kNB + 1;
    static_assert(sizeof(As) >= sizeof(float) * kRows * LDR, "the K-half staging must fit in the activation tile");
    float* Rs = reinterpret_cast<float*>(&As[0][0][0][0]);
    __syncthreads();
    if (kh == 1) {
#pragma unroll
      for (int j = 0; j < JW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) Rs[(mt * 16 + q * 4 + i) * LDR + cw + 16 * j + (lane & 15)] = acc[j][mt][i];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int j = 0; j < JW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][mt][i] += Rs[(mt * 16 + q * 4 + i) * LDR + cw + 16 * j + (lane & 15)];
    }
  }
  if constexpr (SILU) {
    // the workgroup's 128 rows x B sessions through LDS (As is free once every wave is past its
    // last chunk), then SiLU(gate) * up for 64 columns
    constexpr int LDC = kNB + 1;
    static_assert(sizeof(As) >= sizeof(float) * kRows * LDC, "the SiLU staging must fit in the activation tile");
    static_assert(kNB % 64 == 0, "a workgroup's rows must be whole [32 gate; 32 up] groups");
    float* Cs = reinterpret_cast<float*>(&As[0][0][0][0]);
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int j = 0; j < JW; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) Cs[(mt * 16 + q * 4 + i) * LDC + cw + 16 * j + (lane & 15)] = acc[j][mt][i];
    }
    __syncthreads();
    for (int e = tid; e < B * (kNB / 2); e += kThr) {
      const int m = e / (kNB / 2), c = e - m * (kNB / 2), grp = c / 32, ci = c - 32 * grp;
      const float gt = Cs[m * LDC + 64 * grp + ci], up = Cs[m * LDC + 64 * grp + 32 + ci];
      uint16_t hi, lo;
      split_hilo(gt / (1.0f + __expf(-gt)) * up, hi, lo);
      Ohi[(size_t)m * lda + nb * (kNB / 2) + c] = hi;
      Olo[(size_t)m * lda + nb * (kNB / 2) + c] = lo;
    }
    return;
  }
  // lane l holds rows 16 mt + 4 (l / 16) + i of column 16 (rb0 + j) + l % 16
  if (kh != 0) return;
#pragma unroll
  for (int j = 0; j < JW; ++j) {
    const int n = (rb0 + j) * 16 + (lane & 15);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + q * 4 + i;
        if (m < B) P[((size_t)s * B + m) * N + n] = acc[j][mt][i];
      }
  }
}

// ---------------------------------------------------------------------------------------------
// residual + RMSNorm: X[b] (+)= sum of partials (or the embedding row), then H = RMSNorm(X) * g as hi/lo
// ---------------------------------------------------------------------------------------------
// Grid: B workgroups of 1024 threads; thread t owns columns 4t .. 4t+3 (d <= 4096).
// mode 0: X[b] = E[tokens[b]]; mode 1: X[b] += sum_s P[s][b], partials added in order s = 0, 1, ...
__global__ __launch_bounds__(1024) void residual_norm_kernel(int mode, const uint16_t* __restrict__ E,
                                                              const int32_t* __restrict__ tokens,
                                                              const float* __restrict__ P, int KS, float* __restrict__ X,
                                                              const uint16_t* __restrict__ gain, int d, float eps,
                                                              uint16_t* __restrict__ Ahi, uint16_t* __restrict__ Alo,
                                                              int lda, int B, const uint32_t* skip) {
  if (*skip) return;
  __shared__ float red[16];
  const int b = (int)blockIdx.x, tid = (int)threadIdx.x;
  const int i0 = 4 * tid;
  const bool mine = i0 < d;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
  if (mine) {
    if (mode == 0) {
      const uint2 e = *(const uint2*)(E + (int64_t)tokens[b] * d + i0);
      x = make_float4(__uint_as_float(e.x << 16), __uint_as_float(e.x & 0xffff0000u), __uint_as_float(e.y << 16),
                      __uint_as_float(e.y & 0xffff0000u));
    } else {
      x = *(const float4*)(X + (size_t)b * d + i0);
      int s = 0;
      for (; s + 4 <= KS; s += 4) {  // four partials in flight at a time, added in order
        float4 p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) p[u] = *(const float4*)(P + ((size_t)(s + u) * B + b) * d + i0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x.x += p[u].x; x.y += p[u].y; x.z += p[u].z; x.w += p[u].w;
        }
      }
      for (; s < KS; ++s) {
        const float4 p = *(const float4*)(P + ((size_t)s * B + b) * d + i0);
        x.x += p.x; x.y += p.y; x.z += p.z; x.w += p.w;
      }
    }
    *(float4*)(X + (size_t)b * d + i0) = x;
  }
  float ss = x.x * x.x;
  ss = fmaf(x.y, x.y, ss);
  ss = fmaf(x.z, x.z, ss);
  ss = fmaf(x.w, x.w, ss);
  ss = wsum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) tot += red[w];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  if (mine) {
    const uint2 g = *(const uint2*)(gain + i0);
    const float gv[4] = {__uint_as_float(g.x << 16), __uint_as_float(g.x & 0xffff0000u), __uint_as_float(g.y << 16),
                         __uint_as_float(g.y & 0xffff0000u)};
    const float xv[4] = {x.x, x.y, x.z, x.w};
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) split_hilo(xv[u] * r * gv[u], hi[u], lo[u]);
    *(uint2*)(Ahi + (size_t)b * lda + i0) = make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
    *(uint2*)(Alo + (size_t)b * lda + i0) = make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
  }
}

// ---------------------------------------------------------------------------------------------
// QKV: sum partials, RoPE on q and k, scale q by 1/sqrt(hd), append rounded K and V to the cache
// ---------------------------------------------------------------------------------------------
// Grid: (hq + 2 hkv, B) workgroups of hd threads; workgroup (head, b) owns one head vector.
__global__ __launch_bounds__(128) void qkv_epilogue_kernel(const float* __restrict__ P, int KS, int nqkv, int hq, int hkv,
                                                            int hd, const float2* __restrict__ rope,
                                                            const int32_t* __restrict__ positions, float* __restrict__ Qs,
                                                            uint16_t* __restrict__ kv, int64_t kv_slot, int64_t kv_sess,
                                                            int64_t kv_head, int B, const uint32_t* skip) {
  if (*skip) return;
  __shared__ float v[128];
  const int head = (int)blockIdx.x, b = (int)blockIdx.y, i = (int)threadIdx.x;
  const int p = positions[b];
  float x = 0.f;
  for (int s = 0; s < KS; ++s) x += P[((size_t)s * B + b) * nqkv + head * hd + i];
  const int half = hd / 2;
  if (head < hq + hkv) {  // q or k: rotate pair (i, i + hd/2) by the angle of position p
    v[i] = x;
    __syncthreads();
    const float2 cs = rope[(int64_t)p * half + (i % half)];
    x = i < half ? v[i] * cs.x - v[i + half] * cs.y : v[i - half] * cs.y + v[i] * cs.x;
  }
  if (head < hq) {
    Qs[(size_t)b * hq * hd + head * hd + i] = x * (1.0f / sqrtf((float)hd));
  } else {
    const int slot = head < hq + hkv ? 0 : 1;
    const int g = head - hq - slot * hkv;
    kv[kv_slot * slot + kv_sess * b + kv_head * g + (int64_t)p * hd + i] = f_to_bf16(x);
  }
}

// ---------------------------------------------------------------------------------------------
// attention over one chunk of positions of one (session, kv head), for its G query heads
// ---------------------------------------------------------------------------------------------
// Grid: (NCmax, hkv, B) workgroups of 4 waves. Chunk c covers positions [c CHUNK, min((c+1) CHUNK, p+1)),
// where p is the session's current position (already appended). 16 lanes hold one position (8 dims
// each, hd = 128); a wave reads 4 positions per 1 KB load, and waves take packets round-robin.
// Each lane group keeps a running (max, sum, acc) per head; groups and waves are then merged.
// Output: part[((b hq + h) NCmax + c) (hd + 2) + {0: max, 1: sum, 2 + i: acc_i}].
// G = q heads per kv head. Weights are exp2 of base-2 scores on the hardware exp2 (a result below
// 2^-126 may flush to zero; such a weight is far below the sum's rounding).
template <int G, int CHUNK>
__global__ __launch_bounds__(kAttThreads) void attention_kernel(const float* __restrict__ Qs,
                                                                 const uint16_t* __restrict__ kv, int64_t kv_slot,
                                                                 int64_t kv_sess, int64_t kv_head,
                                                                 const int32_t* __restrict__ positions, int hq, int hkv,
                                                                 int NCmax, float* __restrict__ part,
                                                                 const uint32_t* skip) {
  if (*skip) return;
  constexpr int HD = 128;
  __shared__ float sm[4][G][HD + 2];
  const int c = (int)blockIdx.x, g = (int)blockIdx.y, b = (int)blockIdx.z;
  const int P1 = positions[b] + 1;
  const int j0 = c * CHUNK;
  if (j0 >= P1) return;
  const int j1 = min(j0 + CHUNK, P1);
  const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, dim0 = (lane & 15) * 8;
  // scores in base-2 units: q carries 1/sqrt(hd) and log2(e), so exp(s - m) = exp2(s2 - m2)
  constexpr float kLog2e = 1.4426950408889634f;
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[h][e] = Qs[((size_t)b * hq + g * G + h) * HD + dim0 + e] * kLog2e;
  float mx[G], ls[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mx[h] = -INFINITY;
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  const uint16_t* kbase = kv + kv_sess * b + kv_head * g + dim0;
  const uint16_t* vbase = kbase + kv_slot;
  // Wave w reads packets w, w + 4, ... of the chunk (4 positions each), U at a time; the loop is
  // fully unrolled and loads the next U packets before working on the current ones. Positions
  // past the current one are masked out; their loads re-read the chunk's first position. K and V
  // are read once per tick: non-temporal loads.
  constexpr int U = 4;
  constexpr int kIt = CHUNK / (16 * U);
  auto load = [&](int it, u32x4 (&kw)[U], u32x4 (&vw)[U]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pos = j0 + 4 * (wave + 4 * (it * U + u)) + grp;
      const int pl = pos < j1 ? pos : j0;
      kw[u] = __builtin_nontemporal_load((const u32x4*)(kbase + (int64_t)pl * HD));
      vw[u] = __builtin_nontemporal_load((const u32x4*)(vbase + (int64_t)pl * HD));
    }
  };
  u32x4 kb[2][U], vb[2][U];
  load(0, kb[0], vb[0]);
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    // keep each iteration's loads where they are (hoisting them all would need registers for the
    // whole chunk)
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < kIt) load(it + 1, kb[(it + 1) & 1], vb[(it + 1) & 1]);
    const u32x4(&kc)[U] = kb[it & 1];
    const u32x4(&vc)[U] = vb[it & 1];
    // the U positions of this lane group: scores of every head (masked past the current position)
    float sc[G][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = j0 + 4 * (wave + 4 * (it * U + u)) + grp < j1;
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = __uint_as_float(kc[u][e] << 16);
        kf[2 * e + 1] = __uint_as_float(kc[u][e] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        {
          float s2 = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) s2 = fmaf(qv[h][e], kf[e], s2);
          s2 = sum16(s2);
          sc[h][u] = valid ? s2 : -INFINITY;
        }
      }
    }
    // one rescale per block of U positions: new running max, then the block's weights
    float mb[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      {
        float mn = mx[h];
#pragma unroll
        for (int u = 0; u < U; ++u) mn = fmaxf(mn, sc[h][u]);
        mb[h] = mn == -INFINITY ? 0.f : mn;  // nothing valid yet: every weight below is exp2(-inf) = 0
        const float r = __builtin_amdgcn_exp2f(mx[h] - mb[h]);
        mx[h] = mn;
        ls[h] *= r;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= r;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = __uint_as_float(vc[u][e] << 16);
        vf[2 * e + 1] = __uint_as_float(vc[u][e] & 0xffff0000u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        {
          const float w = __builtin_amdgcn_exp2f(sc[h][u] - mb[h]);
          ls[h] += w;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(w, vf[e], acc[h][e]);
        }
      }
    }
    // Make this iteration's running state an opaque input of the next one, so the compiler
    // cannot defer a head's updates to the end of the chunk (which keeps every iteration's K
    // and V in registers).
#pragma unroll
    for (int h = 0; h < G; ++h) {
      asm volatile("" : "+v"(mx[h]), "+v"(ls[h]));
#pragma unroll
      for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(acc[h][e]));
    }
  }
  // merge the four position groups of the wave (lane ^ 16, then lane ^ 32)
  auto merge_pair = [&](int h, float m_a, float m_b, float l_a, float l_b, float* ea, float* eb) {
    const float M = fmaxf(m_a, m_b);
    const float ra = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_a - M), rb = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_b - M);
    mx[h] = M;
    ls[h] = l_a * ra + l_b * rb;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = ea[e] * ra + eb[e] * rb;
  };
#pragma unroll
  for (int h = 0; h < G; ++h) {
    {
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        float ma, mb, la, lb, ea[8], eb[8];
        if (step == 0) {
          swap16(mx[h], ma, mb);
          swap16(ls[h], la, lb);
#pragma unroll
          for (int e = 0; e < 8; ++e) swap16(acc[h][e], ea[e], eb[e]);
        } else {
          swap32(mx[h], ma, mb);
          swap32(ls[h], la, lb);
#pragma unroll
          for (int e = 0; e < 8; ++e) swap32(acc[h][e], ea[e], eb[e]);
        }
        merge_pair(h, ma, mb, la, lb, ea, eb);
      }
      if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm[wave][h][2 + dim0 + e] = acc[h][e];
        if (lane == 0) {
          sm[wave][h][0] = mx[h];
          sm[wave][h][1] = ls[h];
        }
      }
    }
  }
  __syncthreads();
  // merge the four waves; thread t handles (head t / 64, dims 2 (t % 64) .. + 2)
  for (int t = tid; t < G * (HD / 2); t += kAttThreads) {
    const int h = t / (HD / 2), i0 = 2 * (t % (HD / 2));
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][h][0]);
    float L = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[w][h][0] - M);
      L = fmaf(sm[w][h][1], r, L);
      a0 = fmaf(sm[w][h][2 + i0], r, a0);
      a1 = fmaf(sm[w][h][2 + i0 + 1], r, a1);
    }
    float* out = part + (((size_t)b * hq + g * G + h) * NCmax + c) * (HD + 2);
    out[2 + i0] = a0;
    out[2 + i0 + 1] = a1;
    if (i0 == 0) {
      out[0] = M * 0.6931471805599453f;  // back to natural-log units for the merge
      out[1] = L;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// prefill attention: every row of a pass attends over the same session's cache
// ---------------------------------------------------------------------------------------------
// The rows of a prefill pass are consecutive positions of one session, so one chunk of its cache
// serves all of them, and the scores and weighted sums are dense products: queries x positions
// and weights x values. Workgroup (c, g, rg) loads K and V of positions [c kChunkPrefill, + that)
// of kv head g into LDS once, and each of its four waves takes 16 queries (16 / G rows x the G
// q heads of g) through the matrix cores, 32 positions at a time:
//   S^T = K Q^T   (A: 16 positions x 32 dims of K from LDS; B: q as bf16 hi/lo, both products),
//   online softmax per query (base-2 units, running max, the sum kept per lane),
//   O += P V      (A: the weights as bf16 hi/lo; B: V from LDS).
// The weights need no shuffle: lane l holds S^T for query l % 16 at positions 4 (l / 16) + i and
// 16 + 4 (l / 16) + i, which are exactly the eight values of the A operand of P V if the 32
// positions are taken in that order; V's B operand is read from LDS in the same order.
// Output: chunk partials in the layout attention_kernel writes (merge_kernel combines them).
// Grid: (NCmax, hkv, ceil(nb / (64 / G))) workgroups of 256 threads; rows must be consecutive
// positions (prefill_rows_kernel sets them so).
constexpr int kChunkPrefill = 256;
constexpr int kKvPitch = 136;  // bf16 per LDS row: 128 dims + 16 bytes against bank conflicts
template <int G>
__global__ __launch_bounds__(256) void prefill_attention_kernel(const float* __restrict__ Qs, const uint16_t* __restrict__ kv,
                                                                int64_t kv_slot, int64_t kv_head,
                                                                const int32_t* __restrict__ positions, int nb, int hq,
                                                                int NCmax, float* __restrict__ part, const uint32_t* skip) {
  if (*skip) return;
  constexpr int HD = 128, RW = 16 / G;  // rows per wave
  __shared__ uint16_t Ks[kChunkPrefill][kKvPitch], Vs[kChunkPrefill][kKvPitch];
  const int c = (int)blockIdx.x, g = (int)blockIdx.y, rg = (int)blockIdx.z;
  const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j0 = c * kChunkPrefill;
  const int row0 = rg * 4 * RW, nrow = min(4 * RW, nb - row0);
  const int pwg = positions[row0 + nrow - 1];  // the workgroup's last row attends furthest
  if (j0 > pwg) return;
  const int jend = min(j0 + kChunkPrefill, pwg + 1);
  // K and V of positions [j0, jend) into LDS, zeros after (so that masked weights multiply zeros)
  {
    const uint16_t* kb = kv + kv_head * g;
    const uint16_t* vb = kb + kv_slot;
    constexpr int kPer = kChunkPrefill * (HD / 8) / 256;  // 16-byte pieces per thread
    u32x4 kk[kPer], vv[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int e = tid + 256 * t, pr = e >> 4, pc = e & 15;
      kk[t] = vv[t] = u32x4{0u, 0u, 0u, 0u};
      if (j0 + pr < jend) {
        kk[t] = __builtin_nontemporal_load((const u32x4*)(kb + (int64_t)(j0 + pr) * HD + pc * 8));
        vv[t] = __builtin_nontemporal_load((const u32x4*)(vb + (int64_t)(j0 + pr) * HD + pc * 8));
      }
    }
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int e = tid + 256 * t, pr = e >> 4, pc = e & 15;
      *(u32x4*)&Ks[pr][pc * 8] = kk[t];
      *(u32x4*)&Vs[pr][pc * 8] = vv[t];
    }
  }
  __syncthreads();
  constexpr float kLog2e = 1.4426950408889634f;
  const int q = lane & 15, grp = lane >> 4;
  // this lane's query on the S side: row row0 + wave RW + q / G, head g G + q % G
  const int qrow = row0 + wave * RW + q / G;
  const int qlim = qrow < nb ? positions[qrow] : -1;  // it attends 0..qlim
  bf16x8 qhi[4], qlo[4];
  {
    const float* qp = Qs + ((size_t)(qrow < nb ? qrow : row0) * hq + g * G + q % G) * HD + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint16_t h8[8], l8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split_hilo(qp[32 * ks + e] * kLog2e, h8[e], l8[e]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qhi[ks][e] = __builtin_bit_cast(__bf16, h8[e]);
        qlo[ks][e] = __builtin_bit_cast(__bf16, l8[e]);
      }
    }
  }
  float m_run = -INFINITY, l_part = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nblk = (jend - j0 + 31) / 32;
  for (int blk = 0; blk < nblk; ++blk) {
    const int pb = 32 * blk;
    f32x4 sc[2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      sc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4*)&Ks[pb + 16 * pt + q][32 * ks + 8 * grp]);
        sc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qhi[ks], sc[pt], 0, 0, 0);
        sc[pt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qlo[ks], sc[pt], 0, 0, 0);
      }
    }
    // lane: query q at positions pb + 16 pt + 4 grp + i; masked past the query's own position
    float sv[8], mb = m_run;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = j0 + pb + 16 * pt + 4 * grp + i <= qlim ? sc[pt][i] : -INFINITY;
        sv[4 * pt + i] = v;
        mb = fmaxf(mb, v);
      }
    {
      float a, b2;
      swap16(mb, a, b2);
      mb = fmaxf(a, b2);
      swap32(mb, a, b2);
      mb = fmaxf(a, b2);  // the query's max over all four lane groups
    }
    const float mref = mb == -INFINITY ? 0.f : mb;  // nothing valid yet: every weight is exp2(-inf) = 0
    const float r = __builtin_amdgcn_exp2f(m_run - mref);
    m_run = mb;
    l_part *= r;
    bf16x8 phi, plo;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = __builtin_amdgcn_exp2f(sv[k] - mref);
      l_part += w;
      uint16_t h, l;
      split_hilo(w, h, l);
      phi[k] = __builtin_bit_cast(__bf16, h);
      plo[k] = __builtin_bit_cast(__bf16, l);
    }
    // the O rows this lane holds are queries 4 grp + i: their rescale factors
    float rq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rq[i] = __shfl(r, 4 * grp + i);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nt][i] *= rq[i];
      // V's B operand in the same position order: pb + 4 grp + j (j < 4), pb + 12 + 4 grp + j (j >= 4)
      bf16x8 vf;
#pragma unroll
      for (int j = 0; j < 8; ++j) vf[j] = __builtin_bit_cast(__bf16, Vs[pb + (j < 4 ? 0 : 12) + 4 * grp + j][16 * nt + q]);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, vf, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vf, o[nt], 0, 0, 0);
    }
  }
  // the query's sum over its four lane groups
  {
    float a, b2;
    swap16(l_part, a, b2);
    l_part = a + b2;
    swap32(l_part, a, b2);
    l_part = a + b2;
  }
  // partials: lane group 0 writes the max and sum of its query; every lane its O values
  if (grp == 0 && qrow < nb) {
    float* out = part + (((size_t)qrow * hq + g * G + q % G) * NCmax + c) * (HD + 2);
    out[0] = m_run * 0.6931471805599453f;  // natural-log units for the merge
    out[1] = l_part;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qq = 4 * grp + i, orow = row0 + wave * RW + qq / G;
    if (orow < nb) {
      float* out = part + (((size_t)orow * hq + g * G + qq % G) * NCmax + c) * (HD + 2) + 2;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) out[16 * nt + q] = o[nt][i];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// merge the chunks of one (session, q head) and hand o to the O GEMM as hi/lo
// ---------------------------------------------------------------------------------------------
// Grid: (hq, B) workgroups of hd threads.
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part, const int32_t* __restrict__ positions,
                                                     int hq, int hd, int CH, int NCmax, uint16_t* __restrict__ Ahi,
                                                     uint16_t* __restrict__ Alo, int lda, const uint32_t* skip) {
  if (*skip) return;
  const int h = (int)blockIdx.x, b = (int)blockIdx.y, i = (int)threadIdx.x;
  const int NC = (positions[b] + 1 + CH - 1) / CH;
  const float* base = part + ((size_t)b * hq + h) * NCmax * (hd + 2);
  float M = -INFINITY;
  for (int c = 0; c < NC; ++c) M = fmaxf(M, base[(size_t)c * (hd + 2)]);
  float L = 0.f, a = 0.f;
  for (int c = 0; c < NC; ++c) {
    const float* pc = base + (size_t)c * (hd + 2);
    const float r = __expf(pc[0] - M);
    L = fmaf(pc[1], r, L);
    a = fmaf(pc[2 + i], r, a);
  }
  uint16_t hi, lo;
  split_hilo(a / L, hi, lo);
  Ahi[(size_t)b * lda + h * hd + i] = hi;
  Alo[(size_t)b * lda + h * hd + i] = lo;
}

// ---------------------------------------------------------------------------------------------
// SiLU(gate) * up of every FFN column, as hi/lo for the down GEMM
// ---------------------------------------------------------------------------------------------
// The gate/up GEMM's columns come in blocks of 64: 32 gate rows, then the 32 matching up rows.
// Grid: (F / 256, B) workgroups of 256 threads.
__global__ __launch_bounds__(256) void silu_kernel(const float* __restrict__ P, int KS, int F, uint16_t* __restrict__ Ahi,
                                                    uint16_t* __restrict__ Alo, int lda, int B, const uint32_t* skip) {
  if (*skip) return;
  const int f = (int)(blockIdx.x * 256 + threadIdx.x), b = (int)blockIdx.y;
  const int N = 2 * F;
  const int col = 64 * (f / 32) + (f % 32);
  float gt = 0.f, up = 0.f;
  for (int s = 0; s < KS; ++s) {
    gt += P[((size_t)s * B + b) * N + col];
    up += P[((size_t)s * B + b) * N + col + 32];
  }
  uint16_t hi, lo;
  split_hilo(gt / (1.0f + __expf(-gt)) * up, hi, lo);
  Ahi[(size_t)b * lda + f] = hi;
  Alo[(size_t)b * lda + f] = lo;
}

// ---------------------------------------------------------------------------------------------
// greedy argmax of every session: lowest index of the maximum; NaN logits are skipped and flagged
// ---------------------------------------------------------------------------------------------
// Grid: B workgroups of 1024 threads.
// out (optional): the tick's row of the caller's token record.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ logits, int V, int32_t* tokens,
                                                      int32_t* positions, uint32_t* status, const uint32_t* skip,
                                                      int32_t* out) {
  if (*skip) return;
  __shared__ float bv[16];
  __shared__ int32_t bi[16];
  const int b = (int)blockIdx.x, tid = (int)threadIdx.x;
  const float* l = logits + (size_t)b * V;
  float best = -INFINITY;
  int32_t besti = 0x7fffffff;
  bool nan = false;
  // eight loads in flight per thread, then the compares (ties resolve by index in any order)
  int i = tid;
  for (; i + 7 * 1024 < V; i += 8 * 1024) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = l[i + u * 1024];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = i + u * 1024;
      if (v[u] != v[u]) nan = true;
      else if (v[u] > best || (v[u] == best && j < besti)) { best = v[u]; besti = j; }
    }
  }
  for (; i < V; i += 1024) {
    const float v = l[i];
    if (v != v) { nan = true; continue; }
    if (v > best || (v == best && i < besti)) { best = v; besti = i; }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int32_t oi = __shfl_xor(besti, o);
    if (ob > best || (ob == best && oi < besti)) { best = ob; besti = oi; }
  }
  if (__any(nan) && (tid & 63) == 0) __hip_atomic_fetch_or(status, 0x8u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((tid & 63) == 0) {
    bv[tid >> 6] = best;
    bi[tid >> 6] = besti;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w)
      if (bv[w] > best || (bv[w] == best && bi[w] < besti)) { best = bv[w]; besti = bi[w]; }
    tokens[b] = besti == 0x7fffffff ? 0 : besti;
    positions[b] = positions[b] + 1;
    if (out) out[b] = tokens[b];
  }
}

// After a tick of a multi-tick call: the count of completed ticks, written through to memory (the
// tick's outputs were written by the kernels before this one on the stream).
__global__ void progress_kernel(uint32_t* progress, uint32_t value, const uint32_t* skip) {
  if (*skip) return;
  __hip_atomic_store(progress, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------------------------
// prefill: a chunk of prompt positions of one session as the rows of a tick
// ---------------------------------------------------------------------------------------------
// Rows b < nb of a prefill chunk: prompt token first + b at position *pos0 + first + b.
// Grid: one workgroup of kMPrefill threads (nb <= kMPrefill).
__global__ void prefill_rows_kernel(const int32_t* __restrict__ prompt, int first, int nb, const int32_t* __restrict__ pos0,
                                    int32_t* __restrict__ tokens, int32_t* __restrict__ positions) {
  const int b = (int)threadIdx.x;
  if (b >= nb) return;
  tokens[b] = prompt[first + b];
  positions[b] = *pos0 + first + b;
}

// After the last chunk: the last row's greedy token and next position (the argmax already wrote
// them into the row arrays) and its logits go to the caller. Grid: any, 256 threads.
__global__ void prefill_finish_kernel(const int32_t* __restrict__ row_tokens, const int32_t* __restrict__ row_positions,
                                      int last, const float* __restrict__ row_logits, int V, int32_t* tokens,
                                      int32_t* positions, float* logits, const uint32_t* skip) {
  if (*skip) return;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t == 0) {
    tokens[0] = row_tokens[last];
    positions[0] = row_positions[last];
  }
  if (logits)
    for (int64_t v = t; v < V; v += (int64_t)gridDim.x * blockDim.x) logits[v] = row_logits[(int64_t)last * V + v];
}

}  // namespace bt
}  // namespace kd

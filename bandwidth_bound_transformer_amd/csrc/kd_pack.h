// kd_pack.h -- rearrange canonical row-major weights into the streaming layout on the GPU.
//
// The layout follows the access pattern: every compute wave's packets are one
// contiguous, 1 KB-aligned run, so all loads are full 128-bit lane loads with
// no waste ("Kog 3000 tok/s real-time inference", section "three-layer
// strategy", first layer: access patterns matched to the memory subsystem,
// avoiding unaligned accesses).
//  * QKV, O and LM head stay row-major (Q rows, then K rows, then V rows).
//    Each workgroup owns a run of whole rows.
//  * Gate and up rows of one workgroup's FFN slice sit next to each other
//    ([gate slice; up slice]), so SiLU(gate)*up never leaves the workgroup.
//  * The down projection is read column-slice by column-slice. Workgroup w
//    owns FFN columns [f0, f1), and its block holds, for each group of 64
//    output rows and each 16-byte column group, the 64 rows' 16-byte pieces
//    side by side. Lane l of a packet therefore owns row 64*b + l, and one
//    packet is 1 KB of contiguous memory. With fp8 weights a 16-byte lane piece
//    holds 8 columns of two rows instead, row 128*b + l in its first 8 bytes
//    and row 128*b + 64 + l in the last 8, so that FFN slices stay whole
//    8-column units.
#pragma once
#include <hip/hip_runtime.h>

#include "kd_plan.h"

namespace kd {

// Owner workgroup of FFN column f (slices are whole units of fu columns).
__device__ __forceinline__ int ffn_owner(const Dims& m, int64_t f) {
  return (int)part_of(m.F / ffn_unit(m), m.nwg, f / ffn_unit(m));
}

template <typename T>
__global__ void pack_gate_up_kernel(T* dst, const T* gate, const T* up, Dims m) {
  const int64_t total = (int64_t)2 * m.F * m.d;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = e / m.d, col = e % m.d;
    const bool is_up = row >= m.F;
    const int64_t f = is_up ? row - m.F : row;
    const int w = ffn_owner(m, f);
    const int64_t f0 = ffn_lo(m, w), nf = ffn_lo(m, w + 1) - f0;
    const int64_t drow = 2 * f0 + (is_up ? nf : 0) + (f - f0);
    dst[drow * m.d + col] = (is_up ? up : gate)[f * m.d + col];
  }
}

template <typename T>
__global__ void pack_down_kernel(T* dst, const T* down, Dims m) {
  const int64_t total = (int64_t)m.d * m.F;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / m.F, f = e % m.F;  // output row, FFN column
    const int w = ffn_owner(m, f);
    const int64_t fu = ffn_unit(m), db = down_block_rows(m);
    const int64_t f0 = ffn_lo(m, w), g = (ffn_lo(m, w + 1) - f0) / fu;
    const int64_t b = i / db, r = i % db, half = r / 64, lane = r % 64;
    const int64_t j = (f - f0) / fu, el = (f - f0) % fu;
    dst[down_wg_off(m, w) + ((b * g + j) * 64 + lane) * m.vpl + half * fu + el] = down[e];
  }
}

}  // namespace kd

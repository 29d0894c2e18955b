// Pieces shared by the grouped GEMM kernels: the device-side tile lookup
// and the activation functions of the epilogues.
#pragma once

#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// tile lookup: flattened row-tile index -> (group, first row, rows)

struct TileInfo {
  int group;   // -1: no such tile
  int64_t row0;
  int rows;
};

// Executed by the first wave; result broadcast through LDS by the caller.
// off == nullptr: a single group covering rows [0, rows_max).
__device__ inline TileInfo find_row_tile(const int32_t* __restrict__ off, int n_groups, int64_t rows_max,
                                  int BM, int mt) {
  const int lane = threadIdx.x % kWave;
  if (off == nullptr) {
    TileInfo t;
    const int64_t r0 = (int64_t)mt * BM;
    t.group = r0 < rows_max ? 0 : -1;
    t.row0 = r0;
    t.rows = (int)min((int64_t)BM, rows_max - r0);
    return t;
  }
  int64_t before = 0;  // tiles in groups already passed
  for (int g0 = 0; g0 < n_groups; g0 += kWave) {
    const int g = g0 + lane;
    int tiles = 0;
    int64_t start = 0;
    int rows = 0;
    if (g < n_groups) {
      start = off[g];
      rows = off[g + 1] - (int)start;
      tiles = (rows + BM - 1) / BM;
    }
    // inclusive prefix of tiles across the wave
    int inc = tiles;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += v;
    }
    const int64_t hi = before + inc;
    const int64_t lo = hi - tiles;
    const unsigned long long hit = __ballot(g < n_groups && mt >= lo && mt < hi);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      const int64_t lo_s = __shfl(lo, src, kWave);
      const int64_t start_s = __shfl(start, src, kWave);
      const int rows_s = __shfl(rows, src, kWave);
      const int local = mt - (int)lo_s;
      TileInfo t;
      t.group = g0 + src;
      t.row0 = start_s + (int64_t)local * BM;
      t.rows = min(BM, rows_s - local * BM);
      // never touch rows past rows_max, whatever the offsets say
      if (t.row0 + t.rows > rows_max) t.rows = (int)max((int64_t)0, rows_max - t.row0);
      if (t.rows <= 0) t.group = -1;
      return t;
    }
    before += __shfl(inc, kWave - 1, kWave);
  }
  TileInfo t;
  t.group = -1;
  t.row0 = 0;
  t.rows = 0;
  return t;
}

// Number of row tiles over all groups (executed by one full wave; every lane
// gets the total).
__device__ inline int count_row_tiles(const int32_t* __restrict__ off, int n_groups, int64_t rows_max,
                                      int BM) {
  if (off == nullptr) return (int)((rows_max + BM - 1) / BM);
  const int lane = threadIdx.x % kWave;
  int total = 0;
  for (int g0 = 0; g0 < n_groups; g0 += kWave) {
    const int g = g0 + lane;
    int tiles = 0;
    if (g < n_groups) {
      const int64_t lo = min((int64_t)off[g], rows_max), hi = min((int64_t)off[g + 1], rows_max);
      tiles = hi > lo ? (int)((hi - lo + BM - 1) / BM) : 0;
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) tiles += __shfl_xor(tiles, o, kWave);
    total += tiles;
  }
  return total;
}

// silu(g) = g sigmoid(g), the reciprocal from the hardware (1 ulp; the
// quotient's full-precision division costs several times more in the
// epilogues); 1 + e^-g >= 1 or +inf, so the reciprocal is finite or 0
__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// INT8 weight codes: 16 codes (one 16-byte load, code i in byte i) times the
// row scale s, each product rounded to bfloat16 (nearest even), as two
// 16-byte chunks of 8 bf16 (codes 0..7 and 8..15).  codes16_to_bf16 below
// widens the codes alone (no scale) in the same layout.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dequant16(const u32x4_t q, float s, u32x4_t& lo, u32x4_t& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) v[b] = (float)(int8_t)(w[i] >> (8 * b)) * s;
    o[2 * i] = pack2_bf16(v[0], v[1]);
    o[2 * i + 1] = pack2_bf16(v[2], v[3]);
  }
  lo = u32x4_t{o[0], o[1], o[2], o[3]};
  hi = u32x4_t{o[4], o[5], o[6], o[7]};
}
// 16 INT8 codes -> 16 bf16 of the same integer values (exact: |code| <= 128)
__device__ __forceinline__ void codes16_to_bf16(const u32x4_t q, u32x4_t& lo, u32x4_t& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) v[b] = (float)(int8_t)(w[i] >> (8 * b));
    o[2 * i] = pack2_bf16(v[0], v[1]);
    o[2 * i + 1] = pack2_bf16(v[2], v[3]);
  }
  lo = u32x4_t{o[0], o[1], o[2], o[3]};
  hi = u32x4_t{o[4], o[5], o[6], o[7]};
}
__device__ __forceinline__ float gelu_f(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }

}  // namespace moe

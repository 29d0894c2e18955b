// Weighted combine back to token order, atomic-free.
//
// [P1 §2.1]: the layer output is the routing-weighted sum of the selected
// experts' outputs; [P5 §2]: the weights are the normalised routing scores and
// shared experts are always active; [P2 §4.1]: optionally the input is added.
//
// Token-major: each thread owns 8 consecutive columns of one token and sums,
// in float32 and in the fixed order shared, j = 0..k-1, residual, the rows
// inv_row[t, j] of the expert outputs (dropped assignments, -1, add nothing).
// No two threads write the same element, so no atomics are needed.  For
// k <= 8 every row of the token is loaded at once (a dropped one from row 0,
// its value then unused): the loads are independent of each other, so they
// are in flight together instead of one memory round trip per assignment.
#include "moe_internal.h"

namespace moe {
namespace {

template <int DT>
struct Vec8;

template <>
struct Vec8<MOE_DTYPE_BF16> {
  static __device__ __forceinline__ void load(const void* base, int64_t off, float v[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float v[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <>
struct Vec8<MOE_DTYPE_F32> {
  static __device__ __forceinline__ void load(const void* base, int64_t off, float v[8]) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float v[8]) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// k <= KMAX (compile time, 2, 4 or 8): indices, weights and rows held in
// registers.
template <int DT, int KMAX>
__global__ void __launch_bounds__(256)
combine_small_k_kernel(const void* __restrict__ y_perm, const int32_t* __restrict__ inv_row,
                       const float* __restrict__ topk_w, const void* __restrict__ shared_y,
                       const void* __restrict__ residual, void* __restrict__ y, int64_t T, int d,
                       int k) {
  const int cpt = d / 8;  // chunks of 8 columns per token
  const int64_t total = T * cpt;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / cpt;
    const int c = (int)(i % cpt) * 8;
    // every load unconditional (slots past k repeat the last one, dropped
    // rows read row 0); which values count is decided where they are summed
    int32_t rows[KMAX];
    float wts[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int jj = j < k ? j : k - 1;
      rows[j] = inv_row[t * k + jj];
      wts[j] = topk_w[t * k + jj];
    }
    float v[KMAX][8];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      Vec8<DT>::load(y_perm, (int64_t)(rows[j] >= 0 ? rows[j] : 0) * d + c, v[j]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (shared_y) {
      float sv[8];
      Vec8<DT>::load(shared_y, t * d + c, sv);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = sv[q];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool kept = j < k && rows[j] >= 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = kept ? fmaf(wts[j], v[j][q], acc[q]) : acc[q];
    }
    if (residual) {
      float rv[8];
      Vec8<DT>::load(residual, t * d + c, rv);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += rv[q];
    }
    Vec8<DT>::store(y, t * d + c, acc);
  }
}

// Any k: one assignment at a time.
template <int DT>
__global__ void __launch_bounds__(256)
combine_kernel(const void* __restrict__ y_perm, const int32_t* __restrict__ inv_row,
               const float* __restrict__ topk_w, const void* __restrict__ shared_y,
               const void* __restrict__ residual, void* __restrict__ y, int64_t T, int d, int k) {
  const int cpt = d / 8;  // chunks of 8 columns per token
  const int64_t total = T * cpt;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / cpt;
    const int c = (int)(i % cpt) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float v[8];
    if (shared_y) {
      Vec8<DT>::load(shared_y, t * d + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = v[q];
    }
#pragma unroll 4
    for (int j = 0; j < k; ++j) {
      const int32_t row = inv_row[t * k + j];
      if (row < 0) continue;
      const float w = topk_w[t * k + j];
      Vec8<DT>::load(y_perm, (int64_t)row * d + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(w, v[q], acc[q]);
    }
    if (residual) {
      Vec8<DT>::load(residual, t * d + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += v[q];
    }
    Vec8<DT>::store(y, t * d + c, acc);
  }
}

}  // namespace

hipError_t launch_combine(const moe_config& c, const void* y_perm, const int32_t* inv_row,
                          const float* topk_w, const void* shared_y, const void* residual,
                          void* y, hipStream_t s) {
  const int64_t total = c.n_tokens * (c.d_model / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
#define MOE_COMBINE(K_, DT_)                                                                \
  combine_small_k_kernel<DT_, K_><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(              \
      y_perm, inv_row, topk_w, shared_y, residual, y, c.n_tokens, c.d_model, c.top_k)
  if (c.dtype == MOE_DTYPE_BF16) {
    if (c.top_k <= 2) MOE_COMBINE(2, MOE_DTYPE_BF16);
    else if (c.top_k <= 4) MOE_COMBINE(4, MOE_DTYPE_BF16);
    else if (c.top_k <= 8) MOE_COMBINE(8, MOE_DTYPE_BF16);
    else
      combine_kernel<MOE_DTYPE_BF16><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
          y_perm, inv_row, topk_w, shared_y, residual, y, c.n_tokens, c.d_model, c.top_k);
  } else {
    if (c.top_k <= 2) MOE_COMBINE(2, MOE_DTYPE_F32);
    else if (c.top_k <= 4) MOE_COMBINE(4, MOE_DTYPE_F32);
    else if (c.top_k <= 8) MOE_COMBINE(8, MOE_DTYPE_F32);
    else
      combine_kernel<MOE_DTYPE_F32><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
          y_perm, inv_row, topk_w, shared_y, residual, y, c.n_tokens, c.d_model, c.top_k);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe

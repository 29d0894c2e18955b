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
// k is a compile-time constant there (one instantiation per k <= 8), so no
// slot repeats a load and no branch separates the loads (a branch between
// them makes the compiler wait for each load before the next).
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));

// 16 bytes, with the streaming (nontemporal) hint when NT
template <bool NT>
__device__ __forceinline__ u32x4c ld16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(static_cast<const u32x4c*>(p));
  return *static_cast<const u32x4c*>(p);
}
template <bool NT>
__device__ __forceinline__ void st16(void* p, u32x4c v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, static_cast<u32x4c*>(p));
  else
    *static_cast<u32x4c*>(p) = v;
}

template <int DT, bool NT = false>
struct Vec8;

template <bool NT>
struct Vec8<MOE_DTYPE_BF16, NT> {
  static __device__ __forceinline__ void load(const void* base, int64_t off, float v[8]) {
    const u32x4c q = ld16<NT>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float v[8]) {
    u32x4c w;
    w.x = pack2_bf16(v[0], v[1]);
    w.y = pack2_bf16(v[2], v[3]);
    w.z = pack2_bf16(v[4], v[5]);
    w.w = pack2_bf16(v[6], v[7]);
    st16<NT>(static_cast<uint16_t*>(base) + off, w);
  }
};

template <bool NT>
struct Vec8<MOE_DTYPE_F32, NT> {
  static __device__ __forceinline__ void load(const void* base, int64_t off, float v[8]) {
    const float* p = static_cast<const float*>(base) + off;
    const u32x4c a = ld16<NT>(p), b = ld16<NT>(p + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
  static __device__ __forceinline__ void store(void* base, int64_t off, const float v[8]) {
    float* p = static_cast<float*>(base) + off;
    st16<NT>(p, u32x4c{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
    st16<NT>(p + 4, u32x4c{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
  }
};

// k = K (compile time, 1..8): indices, weights and rows held in registers.
// NT: streaming loads and stores, for expert outputs larger than the
// Infinity Cache (the rows are read once; the hint keeps them from evicting
// lines that are reused).
template <int DT, int K, bool NT>
__global__ void __launch_bounds__(256)
combine_small_k_kernel(const void* __restrict__ y_perm, const int32_t* __restrict__ inv_row,
                       const float* __restrict__ topk_w, const void* __restrict__ shared_y,
                       const void* __restrict__ residual, void* __restrict__ y, int64_t T, int d) {
  const int cpt = d / 8;  // chunks of 8 columns per token
  const int64_t total = T * cpt;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / cpt;
    const int c = (int)(i % cpt) * 8;
    // every load unconditional (dropped rows read row 0); which values count
    // is decided where they are summed
    int32_t rows[K];
    float wts[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      rows[j] = inv_row[t * K + j];
      wts[j] = topk_w[t * K + j];
    }
    float v[K][8];
#pragma unroll
    for (int j = 0; j < K; ++j)
      Vec8<DT, NT>::load(y_perm, (int64_t)(rows[j] >= 0 ? rows[j] : 0) * d + c, v[j]);
    // the shared output and the residual are loaded with the rows (from
    // y_perm's first row when absent, then unused), not after a branch
    float sv[8], rv[8];
    Vec8<DT, NT>::load(shared_y ? shared_y : y_perm, shared_y ? t * d + c : c, sv);
    Vec8<DT, NT>::load(residual ? residual : y_perm, residual ? t * d + c : c, rv);
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = shared_y ? sv[q] : 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const bool kept = rows[j] >= 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = kept ? fmaf(wts[j], v[j][q], acc[q]) : acc[q];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = residual ? acc[q] + rv[q] : acc[q];
    Vec8<DT, NT>::store(y, t * d + c, acc);
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
  // streaming hints once the expert outputs outgrow the 256 MB Infinity
  // Cache (measured: 18 % faster at 1.6 GB of rows, 11 % slower at 200 MB)
  const int64_t elt = c.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const bool nt = c.n_tokens * c.top_k * c.d_model * elt > ((int64_t)256 << 20);
#define MOE_COMBINE(K_, DT_)                                                                \
  case K_:                                                                                  \
    if (nt)                                                                                 \
      combine_small_k_kernel<DT_, K_, true><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(    \
          y_perm, inv_row, topk_w, shared_y, residual, y, c.n_tokens, c.d_model);            \
    else                                                                                    \
      combine_small_k_kernel<DT_, K_, false><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(   \
          y_perm, inv_row, topk_w, shared_y, residual, y, c.n_tokens, c.d_model);            \
    break;
#define MOE_COMBINE_ALL(DT_)                                                                \
  switch (c.top_k) {                                                                        \
    MOE_COMBINE(1, DT_)                                                                     \
    MOE_COMBINE(2, DT_)                                                                     \
    MOE_COMBINE(3, DT_)                                                                     \
    MOE_COMBINE(4, DT_)                                                                     \
    MOE_COMBINE(5, DT_)                                                                     \
    MOE_COMBINE(6, DT_)                                                                     \
    MOE_COMBINE(7, DT_)                                                                     \
    MOE_COMBINE(8, DT_)                                                                     \
    default:                                                                                \
      combine_kernel<DT_><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(                     \
          y_perm, inv_row, topk_w, shared_y, residual, y, c.n_tokens, c.d_model, c.top_k);  \
  }
  if (c.dtype == MOE_DTYPE_BF16) {
    MOE_COMBINE_ALL(MOE_DTYPE_BF16)
  } else {
    MOE_COMBINE_ALL(MOE_DTYPE_F32)
  }
#undef MOE_COMBINE_ALL
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe

// Backward pass of the layer: the kernels that are not grouped GEMMs.
//
// [P3 §4.2] trains on loss = task loss + auxiliary loss and back-propagates
// both; [P5 §2] weights load balance 0.01 and z-loss 0.001.  The grouped
// GEMMs of the backward reuse the forward's kernels (dh = d_o W2 and
// dx_rows = da W1 are "row-grouped" products with K-contiguous weights once
// W1 and W2 are transposed; the pre-activations a = x W1^T + b1 come saved
// from the training forward) and the weight-gradient kernel of
// gemm_wgrad.hip.
//
//   combine_bwd     d o_tj = w_tj dy_t into the kept row, dw_tj = dy_t . o_tj
//   router_grad     renormalisation, aux terms, softmax and 1/tau:
//                   scores [T, E] -> dl [T, E] (float32)
//   pad_offsets     per-group columns padded to multiples of the K tile, and
//                   for each padded column its source row (-1: zero padding)
//   transpose       [rows, C] -> [C, columns]: the weights, and d_o and the
//                   gathered x into the padded columns, optional row gather
//   act_bwd_t       a, dh -> da (row-major) and da^T, h^T (padded columns)
//   seg_rowsum      bias gradients: sums of each row of a transposed matrix
//                   over each group's columns
//   dx_gather       dx_t = sum_j dx_rows[row_tj] + shared + router + residual
//   simt_gemm       router gradients (float32, split K)
// Every reduction runs in a fixed order: no atomics.
#include <cmath>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}
__device__ __forceinline__ void unpack8(const u32x4v v, float* o) {
  o[0] = bf_lo(v.x); o[1] = bf_hi(v.x); o[2] = bf_lo(v.y); o[3] = bf_hi(v.y);
  o[4] = bf_lo(v.z); o[5] = bf_hi(v.z); o[6] = bf_lo(v.w); o[7] = bf_hi(v.w);
}
__device__ __forceinline__ u32x4v pack8(const float* o) {
  return u32x4v{pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------
// combine backward: one wave per token, 16-byte chunks of the row per lane

__global__ void __launch_bounds__(kThreads)
combine_bwd_kernel(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ y_perm,
                   const int32_t* __restrict__ inv_row, const float* __restrict__ topk_w, int64_t T,
                   int d, int k, uint16_t* __restrict__ d_yperm, float* __restrict__ d_topk_w) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + wave;
  if (t >= T) return;
  const int nch = d / 8;
  for (int j = 0; j < k; ++j) {
    const int32_t row = inv_row[t * k + j];
    if (row < 0) {  // dropped: no output, no gradient
      if (lane == 0) d_topk_w[t * k + j] = 0.f;
      continue;
    }
    const float wj = topk_w[t * k + j];
    float dot = 0.f;
    for (int c = lane; c < nch; c += kWave) {
      float g[8], o[8], r[8];
      unpack8(*reinterpret_cast<const u32x4v*>(dy + t * d + c * 8), g);
      unpack8(*reinterpret_cast<const u32x4v*>(y_perm + (int64_t)row * d + c * 8), o);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot += g[i] * o[i];
        r[i] = wj * g[i];
      }
      *reinterpret_cast<u32x4v*>(d_yperm + (int64_t)row * d + c * 8) = pack8(r);
    }
    dot = wave_sum(dot);
    if (lane == 0) d_topk_w[t * k + j] = dot;
  }
}

// ---------------------------------------------------------------------------
// router gradient: one wave per token, expert e on lane e % 64

constexpr int kMaxPerLane = kMaxExperts / kWave;

// Per-expert part of dL/dp from the load-balance terms (one workgroup per
// expert): c_lb E f_e / T + c_sq 2 E P_e / T - c_kl / (E (P_e + 1e-8) T),
// with P_e the mean over tokens of p = exp(s - lse) (fixed-order tree sum;
// only summed when a P term is weighted).
__global__ void __launch_bounds__(kThreads)
aux_dp_kernel(const float* __restrict__ scores, const float* __restrict__ lse,
              const int32_t* __restrict__ counts, int64_t T, int E, int k, double c_lb,
              double c_sq, double c_kl, float* __restrict__ aux_dp) {
  __shared__ float red[kThreads];
  const int e = blockIdx.x;
  double P = 0.0;
  if (c_sq != 0.0 || c_kl != 0.0) {
    float acc = 0.f;
    for (int64_t t = threadIdx.x; t < T; t += kThreads) acc += __expf(scores[t * E + e] - lse[t]);
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
      if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
      __syncthreads();
    }
    P = (double)red[0] / (double)T;
  }
  if (threadIdx.x == 0) {
    const double f = (double)counts[e] / (double)(T * k);
    double g = c_lb * E * f + c_sq * 2.0 * E * P;
    if (c_kl != 0.0) g -= c_kl / ((double)E * (P + 1e-8));
    aux_dp[e] = (float)(g / (double)T);
  }
}

__global__ void __launch_bounds__(kThreads)
router_grad_kernel(const float* __restrict__ scores, const float* __restrict__ lse,
                   const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
                   const float* __restrict__ d_topk_w, const float* __restrict__ aux_dp,
                   int64_t T, int E, int k, float c_z, float inv_tau, float* __restrict__ dl) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + wave;
  if (t >= T) return;
  const float l = lse[t];
  // P = sum of the selected probabilities, S1 = sum_j dw_j w_j
  float P = 0.f, S1 = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[t * k + j];
    P += __expf(scores[t * E + e] - l);
    S1 += d_topk_w[t * k + j] * topk_w[t * k + j];
  }
  const float invP = 1.f / P;
  // aux_dp[e]: the load-balance terms; c_z = (z weight) * 2 / T
  float p[kMaxPerLane], dp[kMaxPerLane];
  float sp = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + kWave * i;
    p[i] = 0.f;
    dp[i] = 0.f;
    if (e < E) {
      p[i] = __expf(scores[t * E + e] - l);
      dp[i] = aux_dp[e];
    }
  }
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[t * k + j];
    const float g = (d_topk_w[t * k + j] - S1) * invP;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (e == lane + kWave * i) dp[i] += g;
  }
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) sp += p[i] * dp[i];
  sp = wave_sum(sp);
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + kWave * i;
    if (e < E) dl[t * E + e] = (p[i] * (dp[i] - sp) + c_z * l * p[i]) * inv_tau;
  }
}

// ---------------------------------------------------------------------------
// padded group offsets: poff[g] = sum_{g' < g} roundup(rows_g', pad); for
// every padded column j < ncols: colrow[j] = source row, -1 (padding inside
// a group) or -2 (past the last group).  Every workgroup scans the offsets in
// LDS; workgroup 0 also writes poff.

__global__ void __launch_bounds__(kThreads)
pad_offsets_kernel(const int32_t* __restrict__ offsets, int G, int pad, int64_t ncols,
                   int32_t* __restrict__ poff, int32_t* __restrict__ colrow) {
  __shared__ int32_t s_off[kMaxExperts + 1], s_poff[kMaxExperts + 1];
  for (int g = threadIdx.x; g <= G; g += kThreads) s_off[g] = offsets[g];
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int g = 0; g < G; ++g) {
      s_poff[g] = acc;
      const int32_t rows = s_off[g + 1] - s_off[g];
      acc += (rows + pad - 1) / pad * pad;
    }
    s_poff[G] = acc;
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int g = threadIdx.x; g <= G; g += kThreads) poff[g] = s_poff[g];
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= ncols) return;
  if (j >= s_poff[G]) {
    colrow[j] = -2;
    return;
  }
  int lo = 0, hi = G - 1;  // last g with s_poff[g] <= j
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (s_poff[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int32_t r = s_off[lo] + (int32_t)(j - s_poff[lo]);
  colrow[j] = r < s_off[lo + 1] ? r : -1;
}

// ---------------------------------------------------------------------------
// transpose of 2-byte elements through a 64 x 64 LDS tile, 16-byte global
// loads and stores (C, the destination leading dimension and every chunk
// start are multiples of 8 elements).
// dst[b][c][j] = src[b][row(j)][c] for c < C and destination columns j < ncols,
// with row(j) = colrow ? colrow[j] : (j < nsrc ? j : -1), gathered through
// `gather` when given; rows -1 and -2 (past the last group) read as 0.
// Destination chunks of 8 columns at or past ncols are not written.

constexpr int kTP = 72;  // LDS row pitch (elements): 64 + 8 keeps rows 16-byte aligned

__global__ void __launch_bounds__(kThreads)
transpose_kernel(const uint16_t* __restrict__ src, int64_t src_ld, int64_t src_batch,
                 const int32_t* __restrict__ colrow, const int32_t* __restrict__ gather,
                 int64_t nsrc, int64_t ncols, int C, uint16_t* __restrict__ dst, int64_t dst_ld,
                 int64_t dst_batch) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kTP];
  __shared__ int32_t rows[64];
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const uint16_t* S = src + (int64_t)blockIdx.z * src_batch;
  uint16_t* D = dst + (int64_t)blockIdx.z * dst_batch;
  if (threadIdx.x < 64) {
    const int64_t j = j0 + threadIdx.x;
    int32_t r = -1;
    if (j < ncols) {
      r = colrow ? colrow[j] : (j < nsrc ? (int32_t)j : -1);
      if (r >= 0 && gather) r = gather[r];
    }
    rows[threadIdx.x] = r;
  }
  __syncthreads();
  // load: 64 source rows x 8 chunks of 8 columns
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = threadIdx.x + kThreads * u;
    const int jj = o / 8, ch = o % 8;
    const int32_t r = rows[jj];
    const int c = c0 + ch * 8;
    u32x4v v = {0u, 0u, 0u, 0u};
    if (r >= 0 && c < C) v = *reinterpret_cast<const u32x4v*>(S + (int64_t)r * src_ld + c);
    *reinterpret_cast<u32x4v*>(&tile[jj * kTP + ch * 8]) = v;
  }
  __syncthreads();
  // store: 64 destination rows (c) x 8 chunks of 8 columns (j)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = threadIdx.x + kThreads * u;
    const int cc = o / 8, jc = o % 8;
    const int c = c0 + cc;
    const int64_t j = j0 + jc * 8;
    if (c >= C || j >= ncols) continue;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)tile[(jc * 8 + 2 * q) * kTP + cc] |
             ((uint32_t)tile[(jc * 8 + 2 * q + 1) * kTP + cc] << 16);
    *reinterpret_cast<u32x4v*>(D + (int64_t)c * dst_ld + j) = u32x4v{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// activation backward fused with the transposes the weight gradients need.
// Tile (64 destination columns j) x (64 columns n of one segment s): column j
// takes source row r = colrow ? colrow[j] : (j < nsrc ? j : -1) (-1 and -2:
// zero padding).  SwiGLU: a holds [gate | up] per segment (2f columns),
// h = silu(g) u, dg = dh u silu'(g), du = dh silu(g); GELU: h = gelu(a),
// da = dh gelu'(a).  Writes da row-major (rows r >= 0 only, for the dx
// product) and, through LDS, da^T [S * arow, ldt] and h^T [S * f, ldt] at
// columns j (zeros for padding).

__global__ void __launch_bounds__(kThreads)
act_bwd_t_kernel(const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ dh,
                 int64_t ldh, const int32_t* __restrict__ colrow, int64_t nsrc, int64_t ncols,
                 int f, int act, uint16_t* __restrict__ da, uint16_t* __restrict__ dat,
                 uint16_t* __restrict__ ht, int64_t ldt) {
  __shared__ __attribute__((aligned(16))) uint16_t tg[64 * kTP];
  __shared__ __attribute__((aligned(16))) uint16_t tu[64 * kTP];
  __shared__ __attribute__((aligned(16))) uint16_t th[64 * kTP];
  __shared__ int32_t rows[64];
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int n0 = blockIdx.y * 64, s = blockIdx.z;
  const bool swiglu = act == MOE_ACT_SWIGLU;
  const int arow = swiglu ? 2 * f : f;
  if (threadIdx.x < 64) {
    const int64_t j = j0 + threadIdx.x;
    int32_t r = -1;
    if (j < ncols) r = colrow ? colrow[j] : (j < nsrc ? (int32_t)j : -1);
    rows[threadIdx.x] = r;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = threadIdx.x + kThreads * u;
    const int jj = o / 8, ch = o % 8;
    const int32_t r = rows[jj];
    const int n = n0 + ch * 8;
    float gv[8], uv[8], dv[8], dg[8], du[8], hv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) dg[i] = du[i] = hv[i] = 0.f;
    if (r >= 0 && n < f) {
      const int64_t ab = (int64_t)r * lda + (int64_t)s * arow + n;
      unpack8(*reinterpret_cast<const u32x4v*>(a + ab), gv);
      unpack8(*reinterpret_cast<const u32x4v*>(dh + (int64_t)r * ldh + (int64_t)s * f + n), dv);
      if (swiglu) {
        unpack8(*reinterpret_cast<const u32x4v*>(a + ab + f), uv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sg = 1.f / (1.f + __expf(-gv[i]));
          const float si = gv[i] * sg;
          hv[i] = si * uv[i];
          dg[i] = dv[i] * uv[i] * sg * (1.f + gv[i] * (1.f - sg));
          du[i] = dv[i] * si;
        }
        *reinterpret_cast<u32x4v*>(da + ab) = pack8(dg);
        *reinterpret_cast<u32x4v*>(da + ab + f) = pack8(du);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float Phi = 0.5f * (1.f + erff(gv[i] * 0.70710678118654752f));
          const float phi = 0.39894228040143268f * __expf(-0.5f * gv[i] * gv[i]);
          hv[i] = gv[i] * Phi;
          dg[i] = dv[i] * (Phi + gv[i] * phi);
        }
        *reinterpret_cast<u32x4v*>(da + ab) = pack8(dg);
      }
    }
    // the bf16 values written above, or zeros
    *reinterpret_cast<u32x4v*>(&tg[jj * kTP + ch * 8]) = pack8(dg);
    if (swiglu) *reinterpret_cast<u32x4v*>(&tu[jj * kTP + ch * 8]) = pack8(du);
    *reinterpret_cast<u32x4v*>(&th[jj * kTP + ch * 8]) = pack8(hv);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = threadIdx.x + kThreads * u;
    const int cc = o / 8, jc = o % 8;
    const int c = n0 + cc;
    const int64_t j = j0 + jc * 8;
    if (c >= f || j >= ncols) continue;
    uint32_t wg[4], wu[4], wh[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r0 = (jc * 8 + 2 * q) * kTP + cc, r1 = r0 + kTP;
      wg[q] = (uint32_t)tg[r0] | ((uint32_t)tg[r1] << 16);
      wu[q] = swiglu ? ((uint32_t)tu[r0] | ((uint32_t)tu[r1] << 16)) : 0u;
      wh[q] = (uint32_t)th[r0] | ((uint32_t)th[r1] << 16);
    }
    const int64_t crow = (int64_t)s * arow + c;
    *reinterpret_cast<u32x4v*>(dat + crow * ldt + j) = u32x4v{wg[0], wg[1], wg[2], wg[3]};
    if (swiglu)
      *reinterpret_cast<u32x4v*>(dat + (crow + f) * ldt + j) = u32x4v{wu[0], wu[1], wu[2], wu[3]};
    *reinterpret_cast<u32x4v*>(ht + ((int64_t)s * f + c) * ldt + j) = u32x4v{wh[0], wh[1], wh[2], wh[3]};
  }
}

// ---------------------------------------------------------------------------
// bias gradients: out[g][c] = sum over columns [poff[g], poff[g+1]) of row c
// of the transposed matrix m [C, ld] (zero padding included).  One wave per
// (row, group); poff == null: one group [0, ncols).

__global__ void __launch_bounds__(kThreads)
seg_rowsum_kernel(const uint16_t* __restrict__ m, int64_t ld, int C, const int32_t* __restrict__ poff,
                  int64_t ncols, int G, float* __restrict__ out, int64_t out_ld) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int c = blockIdx.x * (kThreads / kWave) + wave;
  const int g = blockIdx.y;
  if (c >= C) return;
  const int64_t j0 = poff ? poff[g] : 0, j1 = poff ? poff[g + 1] : ncols;
  const uint16_t* row = m + (int64_t)c * ld;
  float acc = 0.f;
  for (int64_t j = j0 + (int64_t)lane * 8; j < j1; j += kWave * 8) {
    float v[8];
    unpack8(*reinterpret_cast<const u32x4v*>(row + j), v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += v[i];
  }
  acc = wave_sum(acc);
  if (lane == 0) out[(int64_t)g * out_ld + c] = acc;
}

// column sums of a float32 [T, E] matrix (router bias gradient): one
// workgroup per column, fixed-order tree
__global__ void __launch_bounds__(kThreads)
colsum_f32_kernel(const float* __restrict__ m, int64_t T, int E, float* __restrict__ out) {
  __shared__ float red[kThreads];
  const int e = blockIdx.x;
  float acc = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += kThreads) acc += m[t * E + e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[e] = red[0];
}

// ---------------------------------------------------------------------------
// dx gather, token-major, 8 columns per thread:
// dx_t = dx_router_t + sum_j kept dx_rows[row_tj] (+ shared_t) (+ dy_t)

__global__ void __launch_bounds__(kThreads)
dx_gather_kernel(const uint16_t* __restrict__ dx_rows, const int32_t* __restrict__ inv_row,
                 const uint16_t* __restrict__ shared, const float* __restrict__ dx_router,
                 const uint16_t* __restrict__ residual, int64_t T, int d, int k,
                 uint16_t* __restrict__ dx) {
  const int nch = d / 8;
  const int64_t o = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (o >= T * nch) return;
  const int64_t t = o / nch;
  const int c = (int)(o % nch) * 8;
  float acc[8], v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = dx_router[t * d + c + i];
  for (int j = 0; j < k; ++j) {
    const int32_t row = inv_row[t * k + j];
    if (row < 0) continue;
    unpack8(*reinterpret_cast<const u32x4v*>(dx_rows + (int64_t)row * d + c), v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  if (shared) {
    unpack8(*reinterpret_cast<const u32x4v*>(shared + t * d + c), v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  if (residual) {
    unpack8(*reinterpret_cast<const u32x4v*>(residual + t * d + c), v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  *reinterpret_cast<u32x4v*>(dx + t * d + c) = pack8(acc);
}

// ---------------------------------------------------------------------------
// float32 SIMT GEMM for the router's gradients:
//   C[m, n] = sum_{k in split} A(m, k) B(k, n),
//   A(m, k) = a[m * sam + k * sak] (float32), B(k, n) = b[k * ldb + n] (bf16),
// 64 x 64 tiles, K chunks of 16 through LDS (the next chunk's loads in
// registers while the current one is used), 4 x 4 outputs per thread.
// blockIdx.z = K split s: rows k in [s * kchunk, (s + 1) * kchunk) go to
// c + s * c_split (partials summed afterwards in split order).

__global__ void __launch_bounds__(kThreads)
simt_gemm_kernel(const float* __restrict__ a, int64_t sam, int64_t sak,
                 const uint16_t* __restrict__ b, int64_t ldb, int M, int N, int64_t K,
                 int64_t kchunk, float* __restrict__ c, int64_t ldc, int64_t c_split) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int64_t kb = (int64_t)blockIdx.z * kchunk;
  const int64_t ke = kb + kchunk < K ? kb + kchunk : K;
  const int tm = threadIdx.x / 16, tn = threadIdx.x % 16;
  float acc[4][4] = {};
  float ra[4], rb[4];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int o = threadIdx.x + kThreads * u, kk = o / 64, mm = o % 64;
      const int64_t kg = k0 + kk;
      ra[u] = (kg < ke && m0 + mm < M) ? a[(int64_t)(m0 + mm) * sam + kg * sak] : 0.f;
      rb[u] = (kg < ke && n0 + mm < N) ? bf(b[kg * ldb + n0 + mm]) : 0.f;
    }
  };
  if (kb < ke) load(kb);
  for (int64_t k0 = kb; k0 < ke; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int o = threadIdx.x + kThreads * u, kk = o / 64, mm = o % 64;
      As[kk][mm] = ra[u];
      Bs[kk][mm] = rb[u];
    }
    __syncthreads();
    if (k0 + 16 < ke) load(k0 + 16);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tm + 16 * i];
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[i] = Bs[kk][tn + 16 * i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jx = 0; jx < 4; ++jx) acc[i][jx] += av[i] * bv[jx];
    }
    __syncthreads();
  }
  float* C = c + (int64_t)blockIdx.z * c_split;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jx = 0; jx < 4; ++jx) {
      const int m = m0 + tm + 16 * i, n = n0 + tn + 16 * jx;
      if (m < M && n < N) C[(int64_t)m * ldc + n] = acc[i][jx];
    }
}

// out[i] = sum_s part[s * n + i], s in order (eight loads in flight)
__global__ void __launch_bounds__(kThreads)
sum_splits_kernel(const float* __restrict__ part, int nsplit, int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  int s = 0;
  for (; s + 8 <= nsplit; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(s + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; s < nsplit; ++s) acc += part[(int64_t)s * n + i];
  out[i] = acc;
}

unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_combine_bwd(const moe_config& c, const void* dy, const void* y_perm,
                              const int32_t* inv_row, const float* topk_w, void* d_yperm,
                              float* d_topk_w, hipStream_t s) {
  combine_bwd_kernel<<<blocks_for(c.n_tokens, kThreads / kWave), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(y_perm), inv_row, topk_w,
      c.n_tokens, c.d_model, c.top_k, static_cast<uint16_t*>(d_yperm), d_topk_w);
  return hipGetLastError();
}

hipError_t launch_router_grad(const moe_config& c, const float* scores, const float* lse,
                              const int32_t* topk_idx, const float* topk_w, const float* d_topk_w,
                              const int32_t* counts, const moe_loss_weights& lw, float* aux_dp,
                              float* dl, hipStream_t s) {
  aux_dp_kernel<<<c.n_experts, kThreads, 0, s>>>(scores, lse, counts, c.n_tokens, c.n_experts,
                                                 c.top_k, lw.load_balance, lw.lb_squares,
                                                 lw.kl_uniform, aux_dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float c_z = (float)(lw.z_loss * 2.0 / (double)c.n_tokens);
  const float inv_tau = c.router_temperature == 0.f ? 1.f : 1.f / c.router_temperature;
  router_grad_kernel<<<blocks_for(c.n_tokens, kThreads / kWave), kThreads, 0, s>>>(
      scores, lse, topk_idx, topk_w, d_topk_w, aux_dp, c.n_tokens, c.n_experts, c.top_k, c_z,
      inv_tau, dl);
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int G, int pad, int64_t ncols, int32_t* poff,
                              int32_t* colrow, hipStream_t s) {
  pad_offsets_kernel<<<blocks_for(ncols, kThreads), kThreads, 0, s>>>(offsets, G, pad, ncols, poff,
                                                                      colrow);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, int64_t src_ld, int64_t src_batch,
                            const int32_t* colrow, const int32_t* gather, int64_t nsrc,
                            int64_t ncols, int C, void* dst, int64_t dst_ld, int64_t dst_batch,
                            int batches, hipStream_t s) {
  if (ncols <= 0 || C <= 0 || batches <= 0) return hipSuccess;
  transpose_kernel<<<dim3(blocks_for(ncols, 64), blocks_for(C, 64), batches), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(src), src_ld, src_batch, colrow, gather, nsrc, ncols, C,
      static_cast<uint16_t*>(dst), dst_ld, dst_batch);
  return hipGetLastError();
}

hipError_t launch_act_bwd_t(const void* a, int64_t lda, const void* dh, int64_t ldh,
                            const int32_t* colrow, int64_t nsrc, int64_t ncols, int S, int f,
                            int act, void* da, void* dat, void* ht, int64_t ldt, hipStream_t s) {
  if (ncols <= 0 || S <= 0) return hipSuccess;
  act_bwd_t_kernel<<<dim3(blocks_for(ncols, 64), blocks_for(f, 64), S), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(a), lda, static_cast<const uint16_t*>(dh), ldh, colrow, nsrc,
      ncols, f, act, static_cast<uint16_t*>(da), static_cast<uint16_t*>(dat),
      static_cast<uint16_t*>(ht), ldt);
  return hipGetLastError();
}

hipError_t launch_seg_rowsum(const void* m, int64_t ld, int C, const int32_t* poff, int64_t ncols,
                             int G, float* out, int64_t out_ld, hipStream_t s) {
  if (C <= 0 || G <= 0) return hipSuccess;
  seg_rowsum_kernel<<<dim3(blocks_for(C, kThreads / kWave), G), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(m), ld, C, poff, ncols, G, out, out_ld);
  return hipGetLastError();
}

hipError_t launch_colsum_f32(const float* m, int64_t T, int E, float* out, hipStream_t s) {
  colsum_f32_kernel<<<E, kThreads, 0, s>>>(m, T, E, out);
  return hipGetLastError();
}

hipError_t launch_dx_gather(const moe_config& c, const void* dx_rows, const int32_t* inv_row,
                            const void* shared, const float* dx_router, const void* residual,
                            void* dx, hipStream_t s) {
  const int64_t n = c.n_tokens * (c.d_model / 8);
  dx_gather_kernel<<<blocks_for(n, kThreads), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(dx_rows), inv_row, static_cast<const uint16_t*>(shared), dx_router,
      static_cast<const uint16_t*>(residual), c.n_tokens, c.d_model, c.top_k,
      static_cast<uint16_t*>(dx));
  return hipGetLastError();
}

// Split count of a SIMT GEMM with long K: enough workgroups to cover the
// chip several times over (each K chunk costs a memory round trip), each
// with at least 64 rows of K.
int simt_splits(int M, int N, int64_t K) {
  const int64_t tiles = (int64_t)((M + 63) / 64) * ((N + 63) / 64);
  int64_t want = (2048 + tiles - 1) / tiles;
  const int64_t most = (K + 63) / 64;
  if (want > most) want = most;
  if (want < 1) want = 1;
  if (want > 256) want = 256;
  return (int)want;
}

hipError_t launch_simt_gemm(const float* a, int64_t sam, int64_t sak, const void* b, int64_t ldb,
                            int M, int N, int64_t K, int nsplit, float* c, int64_t ldc,
                            float* partial, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int64_t kchunk = ((K + nsplit - 1) / nsplit + 15) / 16 * 16;
  const dim3 grid(blocks_for(N, 64), blocks_for(M, 64), nsplit);
  if (nsplit == 1) {
    simt_gemm_kernel<<<grid, kThreads, 0, s>>>(a, sam, sak, static_cast<const uint16_t*>(b), ldb, M,
                                               N, K, kchunk, c, ldc, 0);
    return hipGetLastError();
  }
  // partials [nsplit][M][N] (ldc = N), then the sum in split order
  simt_gemm_kernel<<<grid, kThreads, 0, s>>>(a, sam, sak, static_cast<const uint16_t*>(b), ldb, M, N,
                                             K, kchunk, partial, N, (int64_t)M * N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ldc != N) return hipErrorInvalidValue;
  sum_splits_kernel<<<blocks_for((int64_t)M * N, kThreads), kThreads, 0, s>>>(partial, nsplit,
                                                                              (int64_t)M * N, c);
  return hipGetLastError();
}

}  // namespace moe

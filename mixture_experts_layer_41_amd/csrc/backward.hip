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
//   aux_dp          per-expert load-balance part of dL/dp when it needs the
//                   mean router probability (one workgroup per expert)
//   combine_router  one wave per token: d o_tj = w_tj dy_t into the kept
//                   row, dw_tj = dy_t . o_tj, then renormalisation, aux
//                   terms, softmax and 1/tau: dl [T, E] (float32); extra
//                   workgroups of the same launch pad the group offsets to
//                   multiples of the K tile and map every padded column to
//                   its source row (-1: zero padding)
//   side            one launch of independent parts: [rows, C] -> [C,
//                   columns] transposes, two problems per launch (the
//                   weights, and d_o and the gathered x into the padded
//                   columns), with the router weight gradient's split
//                   products or split sums as extra workgroups
//   act_bwd_t       a, dh -> da (row-major) and da^T, h^T (padded columns)
//   seg_rowsum      bias gradients: sums of each row of a transposed matrix
//                   over each group's columns
//   router_wgrad    dW_r = dl^T x and db_r = column sums of dl (float32,
//                   split over tokens); reduce sums the splits
//   dx_final        dx_t = dl_t W_r + sum_j dx_rows[row_tj] + shared +
//                   residual
// Every reduction runs in a fixed order: no atomics.
#include <algorithm>
#include <cmath>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

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
// router gradient

constexpr int kMaxPerLane = kMaxExperts / kWave;

// Per-expert part of dL/dp from the load-balance terms (one workgroup per
// expert): c_lb E f_e / T + c_sq 2 E P_e / T - c_kl / (E (P_e + 1e-8) T),
// with P_e the mean over tokens of p = exp(s - lse) (fixed-order tree sum).
// Launched only when a P term is weighted; otherwise the combine/router
// kernel takes c_lb E f_e / T from the counts itself.
__global__ void __launch_bounds__(kThreads)
aux_dp_kernel(const float* __restrict__ scores, const float* __restrict__ lse,
              const int32_t* __restrict__ counts, int64_t T, int E, int k, double c_lb,
              double c_sq, double c_kl, float* __restrict__ aux_dp) {
  __shared__ float red[kThreads];
  const int e = blockIdx.x;
  float acc = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += kThreads) acc += __expf(scores[t * E + e] - lse[t]);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double P = (double)red[0] / (double)T;
    const double f = (double)counts[e] / (double)(T * k);
    double g = c_lb * E * f + c_sq * 2.0 * E * P;
    if (c_kl != 0.0) g -= c_kl / ((double)E * (P + 1e-8));
    aux_dp[e] = (float)(g / (double)T);
  }
}

struct CombineRouterArgs {
  // combine backward
  const uint16_t* dy;
  const uint16_t* y_perm;
  const int32_t* inv_row;
  const float* topk_w;
  uint16_t* d_yperm;
  // router backward
  const float* scores;
  const float* lse;
  const int32_t* topk_idx;
  const int32_t* counts;
  const float* aux_dp;  // [E], or null: lb_coef * counts[e]
  double lb_coef;       // load-balance weight * E / (T k T)
  float c_z;            // z-loss weight * 2 / T
  float inv_tau;
  float* dl;
  int64_t T;
  int d, E, k;
  unsigned nb_tok;  // workgroups of the token part; the rest pad the offsets
  // padded group offsets
  const int32_t* offsets;
  int pad;
  int64_t ncols;
  int32_t* poff;
  int32_t* colrow;
};

// poff[g] = sum_{g' < g} roundup(rows_g', pad); for every padded column
// j < ncols: colrow[j] = source row, -1 (padding inside a group) or -2 (past
// the last group).  Every workgroup scans the offsets in LDS; workgroup 0
// also writes poff.
__device__ void pad_offsets_part(const CombineRouterArgs& a, unsigned b) {
  __shared__ int32_t s_off[kMaxExperts + 1], s_poff[kMaxExperts + 1];
  const int G = a.E;
  for (int g = threadIdx.x; g <= G; g += kThreads) s_off[g] = a.offsets[g];
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int g = 0; g < G; ++g) {
      s_poff[g] = acc;
      const int32_t rows = s_off[g + 1] - s_off[g];
      acc += (rows + a.pad - 1) / a.pad * a.pad;
    }
    s_poff[G] = acc;
  }
  __syncthreads();
  if (b == 0)
    for (int g = threadIdx.x; g <= G; g += kThreads) a.poff[g] = s_poff[g];
  const int64_t j = (int64_t)b * kThreads + threadIdx.x;
  if (j >= a.ncols) return;
  if (j >= s_poff[G]) {
    a.colrow[j] = -2;
    return;
  }
  int lo = 0, hi = G - 1;  // last g with s_poff[g] <= j
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (s_poff[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int32_t r = s_off[lo] + (int32_t)(j - s_poff[lo]);
  a.colrow[j] = r < s_off[lo + 1] ? r : -1;
}

// One wave per token.  Combine backward: for each kept assignment j,
// d o_tj = w_tj dy_t goes to its row of d_yperm and dw_tj = dy_t . o_tj (0
// for a dropped one); the dw_tj stay in the wave's LDS row.  Router
// backward, expert e on lane e % 64: with p = softmax(s), P = sum of the
// selected p and w_j = p_j / P, dL/dp_e = (dw_e - sum_j dw_j w_j) / P for a
// selected e, plus the load-balance part; dl = (p (dL/dp - p . dL/dp) +
// c_z lse p) / tau.
template <int NPL>  // experts per lane: E <= 64 * NPL
__global__ void __launch_bounds__(kThreads) combine_router_bwd_kernel(CombineRouterArgs a) {
  __shared__ float s_dw[kThreads / kWave][kMaxExperts];
  if (blockIdx.x >= a.nb_tok) {
    pad_offsets_part(a, blockIdx.x - a.nb_tok);
    return;
  }
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + wave;
  if (t >= a.T) return;
  const int d = a.d, E = a.E, k = a.k;
  float* dw = s_dw[wave];
  const int nch = d / 8;
  // router inputs first, so that they arrive while the combine part runs:
  // the scores of the lane's experts, and lane j < k holds assignment j
  const float l = a.lse[t];
  float sc[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + kWave * i;
    sc[i] = e < E ? a.scores[t * E + e] : 0.f;
  }
  int ej = 0;
  float wl = 0.f, sj = 0.f;
  if (lane < k) {
    ej = a.topk_idx[t * k + lane];
    wl = a.topk_w[t * k + lane];
    sj = a.scores[t * E + ej];
  }

  // combine backward, two assignments at a time (row < 0: dropped, no
  // output and no gradient)
  for (int j0 = 0; j0 < k; j0 += 2) {
    int32_t row[2];
    float wj[2], dot[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bool in = j0 + q < k;
      row[q] = in ? a.inv_row[t * k + j0 + q] : -1;
      wj[q] = in ? a.topk_w[t * k + j0 + q] : 0.f;
      dot[q] = 0.f;
    }
    for (int c = lane; c < nch; c += kWave) {
      float g[8];
      unpack8(*reinterpret_cast<const u32x4v*>(a.dy + t * d + c * 8), g);
      u32x4v raw[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        raw[q] = u32x4v{0u, 0u, 0u, 0u};
        if (row[q] >= 0)
          raw[q] = *reinterpret_cast<const u32x4v*>(a.y_perm + (int64_t)row[q] * d + c * 8);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (row[q] < 0) continue;
        float o[8], r[8];
        unpack8(raw[q], o);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dot[q] += g[i] * o[i];
          r[i] = wj[q] * g[i];
        }
        *reinterpret_cast<u32x4v*>(a.d_yperm + (int64_t)row[q] * d + c * 8) = pack8(r);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (j0 + q >= k) break;
      const float sum = row[q] >= 0 ? wave_sum(dot[q]) : 0.f;  // row is the same on every lane
      if (lane == 0) dw[j0 + q] = sum;
    }
  }
  // LDS accesses of one wave complete in order: the reads below see lane 0's
  // writes; the barrier keeps the compiler from moving them
  __builtin_amdgcn_wave_barrier();

  // P = sum of the selected probabilities, S1 = sum_j dw_j w_j
  float P = 0.f, S1 = 0.f;
  if (lane < k) {
    P = __expf(sj - l);
    S1 = dw[lane] * wl;
  }
  for (int j = kWave + lane; j < k; j += kWave) {
    P += __expf(a.scores[t * E + a.topk_idx[t * k + j]] - l);
    S1 += dw[j] * a.topk_w[t * k + j];
  }
  P = wave_sum(P);
  S1 = wave_sum(S1);
  const float invP = 1.f / P;
  float p[NPL], dp[NPL];
  float sp = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + kWave * i;
    p[i] = 0.f;
    dp[i] = 0.f;
    if (e < E) {
      p[i] = __expf(sc[i] - l);
      dp[i] = a.aux_dp ? a.aux_dp[e] : (float)(a.lb_coef * (double)a.counts[e]);
    }
  }
  // dL/dp of the selected experts: assignment j's (expert, value) from lane j
  const float gl = lane < k ? (dw[lane] - S1) * invP : 0.f;
  const int k0 = k < kWave ? k : kWave;
  for (int j = 0; j < k0; ++j) {
    const int e = __shfl(ej, j);
    const float g = __shfl(gl, j);
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (e == lane + kWave * i) dp[i] += g;
  }
  for (int j = kWave; j < k; ++j) {
    const int e = a.topk_idx[t * k + j];
    const float g = (dw[j] - S1) * invP;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (e == lane + kWave * i) dp[i] += g;
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) sp += p[i] * dp[i];
  sp = wave_sum(sp);
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) a.dl[t * E + e] = (p[i] * (dp[i] - sp) + a.c_z * l * p[i]) * a.inv_tau;
  }
}

// ---------------------------------------------------------------------------
// transpose of 2-byte elements through a 128 x 128 LDS tile, 16-byte global
// loads and stores (C, the destination leading dimension and every chunk
// start are multiples of 8 elements).  One problem:
// dst[b][c][j] = src[b][row(j)][c] for c < C and destination columns j < ncols,
// with row(j) = colrow ? colrow[j] : (j < nsrc ? j : -1), gathered through
// `gather` when given; rows -1 and -2 (past the last group) read as 0.
// Destination chunks of 8 columns at or past ncols are not written.  A
// launch runs two problems, one workgroup per tile: the first problem's
// tiles, then the second's.
//
// LDS: tile row jj (a source row) holds its 16 chunks of 8 columns with
// chunk ch stored at position ch ^ (jj / 8 % 16).  The read phase takes one
// column from rows jc * 8 + r of the 16 chunk-columns jc at once; the XOR
// puts those 16 reads in 16 distinct bank groups.

struct TransposeJob {
  const uint16_t* src;
  int64_t src_ld, src_batch;
  const int32_t* colrow;
  const int32_t* gather;
  int64_t nsrc, ncols;
  int C;
  uint16_t* dst;
  int64_t dst_ld, dst_batch;
  unsigned tx, ty;  // tiles along the columns j and along C
};

constexpr int kTT = 128;
constexpr int kTC = kTT / 8;  // 16-byte chunks per tile row

// Workgroup b of a two-problem transpose launch (tile: kTT * kTC chunks of
// LDS, rows: kTT ints).
__device__ void transpose_part(const TransposeJob& j0, const TransposeJob& j1, unsigned n0,
                               unsigned b, u32x4v* __restrict__ tile, int32_t* __restrict__ rows) {
  const bool second = b >= n0;
  const TransposeJob& J = second ? j1 : j0;
  if (second) b -= n0;
  const unsigned bx = b % J.tx;
  b /= J.tx;
  const unsigned by = b % J.ty, bz = b / J.ty;
  const int64_t jt = (int64_t)bx * kTT;
  const int c0 = (int)by * kTT;
  const int64_t ncols = J.ncols, nsrc = J.nsrc;
  const int C = J.C;
  const int32_t* colrow = J.colrow;
  const int32_t* gather = J.gather;
  const uint16_t* S = J.src + (int64_t)bz * J.src_batch;
  uint16_t* D = J.dst + (int64_t)bz * J.dst_batch;
  const int64_t src_ld = J.src_ld, dst_ld = J.dst_ld;
  if (threadIdx.x < kTT) {
    const int64_t j = jt + threadIdx.x;
    int32_t r = -1;
    if (j < ncols) {
      r = colrow ? colrow[j] : (j < nsrc ? (int32_t)j : -1);
      if (r >= 0 && gather) r = gather[r];
    }
    rows[threadIdx.x] = r;
  }
  __syncthreads();
  // load: 128 source rows x 16 chunks of 8 columns, all loads in flight
  u32x4v v[kTT * kTC / kThreads];
#pragma unroll
  for (int u = 0; u < kTT * kTC / kThreads; ++u) {
    const int o = threadIdx.x + kThreads * u;
    const int jj = o / kTC, ch = o % kTC;
    const int32_t r = rows[jj];
    const int c = c0 + ch * 8;
    // branch-free: out-of-range chunks load the problem's first chunk and
    // are zeroed after
    const bool in = r >= 0 && c < C;
    v[u] = *reinterpret_cast<const u32x4v*>(S + (in ? (int64_t)r * src_ld + c : 0));
    if (!in) v[u] = u32x4v{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kTT * kTC / kThreads; ++u) {
    const int o = threadIdx.x + kThreads * u;
    const int jj = o / kTC, ch = o % kTC;
    tile[jj * kTC + (ch ^ ((jj / 8) % kTC))] = v[u];
  }
  __syncthreads();
  // store: 128 destination rows (c) x 16 chunks of 8 columns (j)
  const uint16_t* t16 = reinterpret_cast<const uint16_t*>(tile);
#pragma unroll 2
  for (int u = 0; u < kTT * kTC / kThreads; ++u) {
    const int o = threadIdx.x + kThreads * u;
    const int cc = o / kTC, jc = o % kTC;
    const int c = c0 + cc;
    const int64_t j = jt + jc * 8;
    if (c >= C || j >= ncols) continue;
    // rows jc * 8 + 0..7 all keep column cc in chunk (cc / 8) ^ jc
    const int base = ((cc / 8) ^ jc) * 8 + cc % 8;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)t16[(jc * 8 + 2 * q) * kTT + base] |
             ((uint32_t)t16[(jc * 8 + 2 * q + 1) * kTT + base] << 16);
    *reinterpret_cast<u32x4v*>(D + (int64_t)c * dst_ld + j) = u32x4v{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// activation backward fused with the transposes the weight gradients need.
// Tile (128 destination columns j) x (64 columns n of one segment s): column
// j takes source row r = colrow ? colrow[j] : (j < nsrc ? j : -1) (-1 and -2:
// zero padding).  SwiGLU: a holds [gate | up] per segment (2f columns),
// h = silu(g) u, dg = dh u silu'(g), du = dh silu(g); GELU: h = gelu(a),
// da = dh gelu'(a).  Writes da row-major (rows r >= 0 only, for the dx
// product) and, through LDS, da^T [S * arow, ldt] and h^T [S * f, ldt] at
// columns j (zeros for padding).  Every thread issues the loads of its four
// (row, 8 columns) items before it computes; LDS rows keep their 8 chunks at
// positions ch ^ (row / 8 % 8), so the column reads of the transposed side
// are at most 2-way bank-conflicted; the transposed stores are 256 bytes
// per destination row.

constexpr int kAJ = 128;                    // destination columns j (source rows) per tile
constexpr int kAN = 64;                     // columns n per tile
constexpr int kACh = kAN / 8;               // 16-byte chunks per LDS row
constexpr int kAI = kAJ * kACh / kThreads;  // (row, chunk) items per thread

__global__ void __launch_bounds__(kThreads)
act_bwd_t_kernel(const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ dh,
                 int64_t ldh, const int32_t* __restrict__ colrow, int64_t nsrc, int64_t ncols,
                 int f, int act, uint16_t* __restrict__ da, uint16_t* __restrict__ dat,
                 uint16_t* __restrict__ ht, int64_t ldt) {
  __shared__ __attribute__((aligned(16))) u32x4v tg[kAJ * kACh];
  __shared__ __attribute__((aligned(16))) u32x4v tu[kAJ * kACh];
  __shared__ __attribute__((aligned(16))) u32x4v th[kAJ * kACh];
  __shared__ int32_t rows[kAJ];
  const int64_t j0 = (int64_t)blockIdx.x * kAJ;
  const int n0 = blockIdx.y * kAN, s = blockIdx.z;
  const bool swiglu = act == MOE_ACT_SWIGLU;
  const int arow = swiglu ? 2 * f : f;
  if (threadIdx.x < kAJ) {
    const int64_t j = j0 + threadIdx.x;
    int32_t r = -1;
    if (j < ncols) r = colrow ? colrow[j] : (j < nsrc ? (int32_t)j : -1);
    rows[threadIdx.x] = r;
  }
  __syncthreads();
  // loads (branch-free: an item outside the problem reads element 0 and is
  // zeroed)
  u32x4v rg[kAI], ru[kAI], rd[kAI];
  int64_t ab[kAI];
  bool ok[kAI];
#pragma unroll
  for (int i = 0; i < kAI; ++i) {
    const int o = threadIdx.x + kThreads * i;
    const int jj = o / kACh, ch = o % kACh;
    const int32_t r = rows[jj];
    const int n = n0 + ch * 8;
    ok[i] = r >= 0 && n < f;
    ab[i] = ok[i] ? (int64_t)r * lda + (int64_t)s * arow + n : 0;
    const int64_t hb = ok[i] ? (int64_t)r * ldh + (int64_t)s * f + n : 0;
    rg[i] = *reinterpret_cast<const u32x4v*>(a + ab[i]);
    rd[i] = *reinterpret_cast<const u32x4v*>(dh + hb);
    ru[i] = u32x4v{0u, 0u, 0u, 0u};
    if (swiglu) ru[i] = *reinterpret_cast<const u32x4v*>(a + ab[i] + f);
  }
#pragma unroll
  for (int i = 0; i < kAI; ++i) {
    const int o = threadIdx.x + kThreads * i;
    const int jj = o / kACh, ch = o % kACh;
    float gv[8], uv[8], dv[8], dg[8], du[8], hv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dg[e] = du[e] = hv[e] = 0.f;
    if (ok[i]) {
      unpack8(rg[i], gv);
      unpack8(rd[i], dv);
      if (swiglu) {
        unpack8(ru[i], uv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sg = 1.f / (1.f + __expf(-gv[e]));
          const float si = gv[e] * sg;
          hv[e] = si * uv[e];
          dg[e] = dv[e] * uv[e] * sg * (1.f + gv[e] * (1.f - sg));
          du[e] = dv[e] * si;
        }
        *reinterpret_cast<u32x4v*>(da + ab[i]) = pack8(dg);
        *reinterpret_cast<u32x4v*>(da + ab[i] + f) = pack8(du);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float Phi = 0.5f * (1.f + erff(gv[e] * 0.70710678118654752f));
          const float phi = 0.39894228040143268f * __expf(-0.5f * gv[e] * gv[e]);
          hv[e] = gv[e] * Phi;
          dg[e] = dv[e] * (Phi + gv[e] * phi);
        }
        *reinterpret_cast<u32x4v*>(da + ab[i]) = pack8(dg);
      }
    }
    // the bf16 values written above, or zeros
    const int pos = jj * kACh + (ch ^ ((jj / 8) % kACh));
    tg[pos] = pack8(dg);
    if (swiglu) tu[pos] = pack8(du);
    th[pos] = pack8(hv);
  }
  __syncthreads();
  const uint16_t* g16 = reinterpret_cast<const uint16_t*>(tg);
  const uint16_t* u16 = reinterpret_cast<const uint16_t*>(tu);
  const uint16_t* h16 = reinterpret_cast<const uint16_t*>(th);
#pragma unroll
  for (int i = 0; i < kAI; ++i) {
    const int o = threadIdx.x + kThreads * i;
    const int cc = o / (kAJ / 8), jc = o % (kAJ / 8);
    const int c = n0 + cc;
    const int64_t j = j0 + jc * 8;
    if (c >= f || j >= ncols) continue;
    // rows jc * 8 + 0..7 keep column cc in chunk (cc / 8) ^ (jc % 8)
    const int base = ((cc / 8) ^ (jc % kACh)) * 8 + cc % 8;
    uint32_t wg[4], wu[4], wh[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r0 = (jc * 8 + 2 * q) * kAN + base, r1 = r0 + kAN;
      wg[q] = (uint32_t)g16[r0] | ((uint32_t)g16[r1] << 16);
      wu[q] = swiglu ? ((uint32_t)u16[r0] | ((uint32_t)u16[r1] << 16)) : 0u;
      wh[q] = (uint32_t)h16[r0] | ((uint32_t)h16[r1] << 16);
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

// ---------------------------------------------------------------------------
// router weight and bias gradients, float32 SIMT, split over tokens:
//   out[s][e][i] = sum_{t in split s} dl[t, e] x[t, i]       (e < E, i < d)
//   bout[s][e]   = sum_{t in split s} dl[t, e]               (first column tile)
// 64 x 64 output tiles, 32 tokens per LDS round (the next round's loads in
// registers while the current one is used), a 4 x 4 block of outputs per
// thread (16-byte LDS reads and stores).
// blockIdx.z = split s: tokens [s * kchunk, (s + 1) * kchunk), kchunk a
// multiple of 32.

constexpr int kRK = 32;

struct RouterWgradArgs {
  const float* dl;
  const uint16_t* x;
  int64_t T;
  int E, d;
  int64_t kchunk;
  float* out;  // split s at out + s * out_split
  int64_t out_split;
  float* bout;  // split s at bout + s * bout_split, or null
  int64_t bout_split;
  unsigned tx, ty;  // column and row tiles; workgroup b = (split * ty + row tile) * tx + column tile
};

// Workgroup b of the router weight gradient (As, Bs: kRK x 64 floats of LDS
// each).
__device__ void router_wgrad_part(const RouterWgradArgs& w, unsigned b, float (*__restrict__ As)[64],
                                  float (*__restrict__ Bs)[64]) {
  const float* __restrict__ dl = w.dl;
  const uint16_t* __restrict__ x = w.x;
  const int64_t T = w.T, kchunk = w.kchunk;
  const int E = w.E, d = w.d;
  const unsigned bx = b % w.tx, by = (b / w.tx) % w.ty, bz = b / (w.tx * w.ty);
  const int m0 = by * 64, n0 = bx * 64;
  const int64_t kb = (int64_t)bz * kchunk;
  const int64_t ke = kb + kchunk < T ? kb + kchunk : T;
  const int tid = threadIdx.x, tm = tid / 16, tn = tid % 16;
  const bool bias = w.bout != nullptr && bx == 0;
  float acc[4][4] = {};
  float bacc = 0.f;
  float ra[8];
  u32x4v rb;
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int o = tid + kThreads * u, kk = o / 64, mm = o % 64;
      const int64_t kg = k0 + kk;
      ra[u] = (kg < ke && m0 + mm < E) ? dl[kg * E + m0 + mm] : 0.f;
    }
    const int kk = tid / 8, c = n0 + (tid % 8) * 8;
    const int64_t kg = k0 + kk;
    rb = u32x4v{0u, 0u, 0u, 0u};
    if (kg < ke && c < d) rb = *reinterpret_cast<const u32x4v*>(x + kg * d + c);
  };
  if (kb < ke) load(kb);
  for (int64_t k0 = kb; k0 < ke; k0 += kRK) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int o = tid + kThreads * u;
      As[o / 64][o % 64] = ra[u];
    }
    {
      float v[8];
      unpack8(rb, v);
      float4* dst = reinterpret_cast<float4*>(&Bs[tid / 8][(tid % 8) * 8]);
      dst[0] = float4{v[0], v[1], v[2], v[3]};
      dst[1] = float4{v[4], v[5], v[6], v[7]};
    }
    __syncthreads();
    if (k0 + kRK < ke) load(k0 + kRK);
#pragma unroll 8
    for (int kk = 0; kk < kRK; ++kk) {
      const float4 av = *reinterpret_cast<const float4*>(&As[kk][tm * 4]);
      const float4 bv = *reinterpret_cast<const float4*>(&Bs[kk][tn * 4]);
      const float a4[4] = {av.x, av.y, av.z, av.w}, b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jx = 0; jx < 4; ++jx) acc[i][jx] += a4[i] * b4[jx];
    }
    if (bias && tid < 64)
      for (int kk = 0; kk < kRK; ++kk) bacc += As[kk][tid];
    __syncthreads();
  }
  float* O = w.out + (int64_t)bz * w.out_split;
  const int n = n0 + tn * 4;  // d is a multiple of 8: four columns all in or all out
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tm * 4 + i;
    if (m < E && n < d)
      *reinterpret_cast<float4*>(O + (int64_t)m * d + n) =
          float4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
  }
  if (bias && tid < 64 && m0 + tid < E) w.bout[(int64_t)bz * w.bout_split + m0 + tid] = bacc;
}

// Sum of the splits (split s at part + s * ld), 64 outputs per workgroup:
// the four waves take every fourth split each (eight loads in flight), then
// wave 0 adds the four partial sums in order.  Outputs i < n_a go to out_a,
// the rest (i < n) to out_b.
struct ReduceArgs {
  const float* part;
  int nsplit;
  int64_t ld, n, n_a;
  float* out_a;
  float* out_b;
};

constexpr int kRG = kThreads / kWave;  // split groups of the sum

// Workgroup b of the sum (red: kRG x kWave floats of LDS).
__device__ void reduce_part(const ReduceArgs& r, unsigned b, float (*__restrict__ red)[kWave]) {
  constexpr int G = kRG;
  const float* __restrict__ part = r.part;
  const int nsplit = r.nsplit;
  const int64_t ld = r.ld, n = r.n, n_a = r.n_a;
  const int g = threadIdx.x / kWave, li = threadIdx.x % kWave;
  const int64_t i = (int64_t)b * kWave + li;
  float acc = 0.f;
  if (i < n) {
    int s = g;
    for (; s + 7 * G < nsplit; s += 8 * G) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(s + u * G) * ld + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; s < nsplit; s += G) acc += part[(int64_t)s * ld + i];
  }
  red[g][li] = acc;
  __syncthreads();
  if (g == 0 && i < n) {
    float sum = red[0][li];
#pragma unroll
    for (int q = 1; q < G; ++q) sum += red[q][li];
    if (i < n_a) r.out_a[i] = sum; else r.out_b[i - n_a] = sum;
  }
}

// ---------------------------------------------------------------------------
// One launch for independent side work of the backward: the workgroups
// [0, n_w) run the router weight gradient's split products, the next n_r
// sum its splits, the rest transpose (two problems).  The latency-bound
// router parts come first in dispatch order, so the bandwidth-bound
// transposes fill the CUs around them.  The parts share one LDS buffer.

struct SideArgs {
  TransposeJob t0, t1;
  unsigned n_t0;
  RouterWgradArgs w;
  unsigned n_w;
  ReduceArgs r;
  unsigned n_r;
};

__global__ void __launch_bounds__(kThreads) side_kernel(SideArgs a) {
  __shared__ __attribute__((aligned(16))) u32x4v lds[kTT * kTC];
  __shared__ int32_t rows[kTT];
  static_assert(2 * kRK * 64 * sizeof(float) <= sizeof(lds), "router tiles fit the buffer");
  static_assert(kRG * kWave * sizeof(float) <= sizeof(lds), "split sums fit the buffer");
  unsigned b = blockIdx.x;
  float* f = reinterpret_cast<float*>(lds);
  if (b < a.n_w) {
    router_wgrad_part(a.w, b, reinterpret_cast<float (*)[64]>(f),
                      reinterpret_cast<float (*)[64]>(f + kRK * 64));
    return;
  }
  b -= a.n_w;
  if (b < a.n_r) {
    reduce_part(a.r, b, reinterpret_cast<float (*)[kWave]>(f));
    return;
  }
  transpose_part(a.t0, a.t1, a.n_t0, b - a.n_r, lds, rows);
}

// ---------------------------------------------------------------------------
// dx, 64 tokens x 64 columns per workgroup:
//   dx_t = sum_j kept dx_rows[row_tj] (+ shared_t) (+ dy_t) + dl_t W_r
// Each thread owns 8 consecutive columns of two tokens: it gathers their
// rows first (four assignments' indices, then their rows, in flight at
// once), so that those loads overlap the router product, which runs through
// LDS in chunks of 32 experts (float32, a 4 x 4 block per thread) and comes
// back through LDS to the same 8-column layout.

__device__ __forceinline__ void add8(float* acc, const uint16_t* p) {
  float v[8];
  unpack8(*reinterpret_cast<const u32x4v*>(p), v);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] += v[i];
}

__global__ void __launch_bounds__(kThreads)
dx_final_kernel(const float* __restrict__ dl, const uint16_t* __restrict__ w_router,
                const uint16_t* __restrict__ dx_rows, const int32_t* __restrict__ inv_row,
                const uint16_t* __restrict__ shared, const uint16_t* __restrict__ residual,
                int64_t T, int d, int E, int k, uint16_t* __restrict__ dx) {
  __shared__ __attribute__((aligned(16))) float As[kRK][64 + 4];
  __shared__ __attribute__((aligned(16))) float Bs[kRK][64];
  __shared__ __attribute__((aligned(16))) float O[64][64 + 4];
  const int64_t t0 = (int64_t)blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tm = tid / 16, tn = tid % 16;
  float ra[8];
  u32x4v rb;
  auto load = [&](int e0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int o = tid + kThreads * u, kk = o % kRK, mm = o / kRK;
      const int e = e0 + kk;
      const int64_t t = t0 + mm;
      ra[u] = (e < E && t < T) ? dl[t * E + e] : 0.f;
    }
    const int e = e0 + tid / 8, c = c0 + (tid % 8) * 8;
    rb = u32x4v{0u, 0u, 0u, 0u};
    if (e < E && c < d) rb = *reinterpret_cast<const u32x4v*>(w_router + (int64_t)e * d + c);
  };
  load(0);

  // the gathered rows of this thread's two (token, 8 columns) items
  int64_t tt[2];
  int cc[2];
  bool ok[2];
  float s8[2][8];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = tid + kThreads * u;
    tt[u] = t0 + o / 8;
    cc[u] = c0 + (o % 8) * 8;
    ok[u] = tt[u] < T && cc[u] < d;
#pragma unroll
    for (int i = 0; i < 8; ++i) s8[u][i] = 0.f;
  }
  for (int j0 = 0; j0 < k; j0 += 4) {
    int32_t row[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        row[u][q] = (ok[u] && j0 + q < k) ? inv_row[tt[u] * k + j0 + q] : -1;
    // every load issued before the first use (a dropped row reads row 0)
    u32x4v raw[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        raw[u][q] = u32x4v{0u, 0u, 0u, 0u};
        if (ok[u] && j0 + q < k) {
          const int64_t r = row[u][q] >= 0 ? row[u][q] : 0;
          raw[u][q] = *reinterpret_cast<const u32x4v*>(dx_rows + r * d + cc[u]);
        }
      }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (row[u][q] >= 0) {
          float v[8];
          unpack8(raw[u][q], v);
#pragma unroll
          for (int i = 0; i < 8; ++i) s8[u][i] += v[i];
        }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!ok[u]) continue;
    if (shared) add8(s8[u], shared + tt[u] * d + cc[u]);
    if (residual) add8(s8[u], residual + tt[u] * d + cc[u]);
  }

  float acc[4][4] = {};
  for (int e0 = 0; e0 < E; e0 += kRK) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int o = tid + kThreads * u;
      As[o % kRK][o / kRK] = ra[u];
    }
    {
      float v[8];
      unpack8(rb, v);
      float4* dst = reinterpret_cast<float4*>(&Bs[tid / 8][(tid % 8) * 8]);
      dst[0] = float4{v[0], v[1], v[2], v[3]};
      dst[1] = float4{v[4], v[5], v[6], v[7]};
    }
    __syncthreads();
    if (e0 + kRK < E) load(e0 + kRK);
#pragma unroll 8
    for (int kk = 0; kk < kRK; ++kk) {
      const float4 av = *reinterpret_cast<const float4*>(&As[kk][tm * 4]);
      const float4 bv = *reinterpret_cast<const float4*>(&Bs[kk][tn * 4]);
      const float a4[4] = {av.x, av.y, av.z, av.w}, b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jx = 0; jx < 4; ++jx) acc[i][jx] += a4[i] * b4[jx];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<float4*>(&O[tm * 4 + i][tn * 4]) =
        float4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!ok[u]) continue;
    const int o = tid + kThreads * u, r = o / 8, ch = o % 8;
    const float4 lo = *reinterpret_cast<const float4*>(&O[r][ch * 8]);
    const float4 hi = *reinterpret_cast<const float4*>(&O[r][ch * 8 + 4]);
    s8[u][0] += lo.x; s8[u][1] += lo.y; s8[u][2] += lo.z; s8[u][3] += lo.w;
    s8[u][4] += hi.x; s8[u][5] += hi.y; s8[u][6] += hi.z; s8[u][7] += hi.w;
    *reinterpret_cast<u32x4v*>(dx + tt[u] * d + cc[u]) = pack8(s8[u]);
  }
}

unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_aux_dp(const moe_config& c, const float* scores, const float* lse,
                         const int32_t* counts, const moe_loss_weights& lw, float* aux_dp,
                         hipStream_t s) {
  aux_dp_kernel<<<c.n_experts, kThreads, 0, s>>>(scores, lse, counts, c.n_tokens, c.n_experts,
                                                 c.top_k, lw.load_balance, lw.lb_squares,
                                                 lw.kl_uniform, aux_dp);
  return hipGetLastError();
}

hipError_t launch_combine_router_bwd(const moe_config& c, const moe_loss_weights& lw,
                                     const CombineRouterBwd& b, hipStream_t s) {
  CombineRouterArgs a;
  a.dy = static_cast<const uint16_t*>(b.dy);
  a.y_perm = static_cast<const uint16_t*>(b.y_perm);
  a.inv_row = b.inv_row;
  a.topk_w = b.topk_w;
  a.d_yperm = static_cast<uint16_t*>(b.d_yperm);
  a.scores = b.scores;
  a.lse = b.lse;
  a.topk_idx = b.topk_idx;
  a.counts = b.counts;
  a.aux_dp = b.aux_dp;
  const double T = (double)c.n_tokens;
  a.lb_coef = lw.load_balance * (double)c.n_experts / (T * (double)c.top_k) / T;
  a.c_z = (float)(lw.z_loss * 2.0 / T);
  a.inv_tau = c.router_temperature == 0.f ? 1.f : 1.f / c.router_temperature;
  a.dl = b.dl;
  a.T = c.n_tokens;
  a.d = c.d_model;
  a.E = c.n_experts;
  a.k = c.top_k;
  a.nb_tok = blocks_for(c.n_tokens, kThreads / kWave);
  a.offsets = b.offsets;
  a.pad = b.pad;
  a.ncols = b.ncols;
  a.poff = b.poff;
  a.colrow = b.colrow;
  const unsigned nb_pad = blocks_for(b.ncols > 0 ? b.ncols : 1, kThreads);
  const unsigned grid = a.nb_tok + nb_pad;
  if (c.n_experts <= kWave)
    combine_router_bwd_kernel<1><<<grid, kThreads, 0, s>>>(a);
  else if (c.n_experts <= 2 * kWave)
    combine_router_bwd_kernel<2><<<grid, kThreads, 0, s>>>(a);
  else if (c.n_experts <= 4 * kWave)
    combine_router_bwd_kernel<4><<<grid, kThreads, 0, s>>>(a);
  else
    combine_router_bwd_kernel<kMaxPerLane><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

static TransposeJob job_of(const TransposeDesc& t) {
  TransposeJob j;
  j.src = static_cast<const uint16_t*>(t.src);
  j.src_ld = t.src_ld;
  j.src_batch = t.src_batch;
  j.colrow = t.colrow;
  j.gather = t.gather;
  j.nsrc = t.nsrc;
  j.ncols = t.ncols;
  j.C = t.C;
  j.dst = static_cast<uint16_t*>(t.dst);
  j.dst_ld = t.dst_ld;
  j.dst_batch = t.dst_batch;
  j.tx = blocks_for(t.ncols, kTT);
  j.ty = blocks_for(t.C, kTT);
  return j;
}

// dW_r goes straight to the caller's buffer (16-byte stores) when there is
// one split and the buffer allows it; otherwise through the split partials.
static bool router_wgrad_direct(const RouterWgradDesc& r) {
  return r.nsplit == 1 && ((uintptr_t)r.dw & 15) == 0;
}

hipError_t launch_side(const TransposeDesc& a, const TransposeDesc& b, const RouterWgradDesc* rp,
                       const RouterWgradDesc* rs, hipStream_t s) {
  SideArgs x{};
  const bool ua = a.ncols > 0 && a.C > 0 && a.batches > 0;
  const bool ub = b.ncols > 0 && b.C > 0 && b.batches > 0;
  uint64_t n_t = 0, n_w = 0, n_r = 0;
  if (ua || ub) {
    x.t0 = job_of(ua ? a : b);  // a lone problem goes first
    x.t1 = ua && ub ? job_of(b) : x.t0;
    const uint64_t n0 = (uint64_t)x.t0.tx * x.t0.ty * (uint64_t)(ua ? a.batches : b.batches);
    const uint64_t n1 = ua && ub ? (uint64_t)x.t1.tx * x.t1.ty * (uint64_t)b.batches : 0;
    if (n0 > 0xFFFFFFFFull) return hipErrorInvalidValue;
    x.n_t0 = (unsigned)n0;
    n_t = n0 + n1;
  }
  if (rp != nullptr) {
    const RouterWgradDesc& r = *rp;
    if (r.nsplit < 1 || r.part == nullptr || ((uintptr_t)r.part & 15) != 0 || r.T < 1)
      return hipErrorInvalidValue;
    const int64_t kchunk = ((r.T + r.nsplit - 1) / r.nsplit + kRK - 1) / kRK * kRK;
    if ((r.T + kchunk - 1) / kchunk != r.nsplit) return hipErrorInvalidValue;
    x.w.dl = r.dl;
    x.w.x = static_cast<const uint16_t*>(r.x);
    x.w.T = r.T;
    x.w.E = r.E;
    x.w.d = r.d;
    x.w.kchunk = kchunk;
    if (router_wgrad_direct(r)) {
      x.w.out = r.dw;
      x.w.out_split = 0;
      x.w.bout = r.db;
      x.w.bout_split = 0;
    } else {
      // partials [nsplit][ld], the bias partials after the weight's
      const int64_t ld = router_wgrad_split_ld(r.E, r.d);
      x.w.out = r.part;
      x.w.out_split = ld;
      x.w.bout = r.db ? r.part + (int64_t)r.E * r.d : nullptr;
      x.w.bout_split = ld;
    }
    x.w.tx = blocks_for(r.d, 64);
    x.w.ty = blocks_for(r.E, 64);
    n_w = (uint64_t)x.w.tx * x.w.ty * (uint64_t)r.nsplit;
  }
  if (rs != nullptr && !router_wgrad_direct(*rs)) {
    const RouterWgradDesc& r = *rs;
    if (r.part == nullptr) return hipErrorInvalidValue;
    const int64_t nw = (int64_t)r.E * r.d;
    x.r.part = r.part;
    x.r.nsplit = r.nsplit;
    x.r.ld = router_wgrad_split_ld(r.E, r.d);
    x.r.n = nw + (r.db ? r.E : 0);
    x.r.n_a = nw;
    x.r.out_a = r.dw;
    x.r.out_b = r.db;
    n_r = blocks_for(x.r.n, kWave);
  }
  const uint64_t total = n_t + n_w + n_r;
  if (total == 0) return hipSuccess;
  if (total > 0xFFFFFFFFull) return hipErrorInvalidValue;
  x.n_w = (unsigned)n_w;
  x.n_r = (unsigned)n_r;
  side_kernel<<<(unsigned)total, kThreads, 0, s>>>(x);
  return hipGetLastError();
}

hipError_t launch_transpose(const TransposeDesc& a, const TransposeDesc& b, hipStream_t s) {
  return launch_side(a, b, nullptr, nullptr, s);
}

hipError_t launch_act_bwd_t(const void* a, int64_t lda, const void* dh, int64_t ldh,
                            const int32_t* colrow, int64_t nsrc, int64_t ncols, int S, int f,
                            int act, void* da, void* dat, void* ht, int64_t ldt, hipStream_t s) {
  if (ncols <= 0 || S <= 0) return hipSuccess;
  act_bwd_t_kernel<<<dim3(blocks_for(ncols, kAJ), blocks_for(f, kAN), S), kThreads, 0, s>>>(
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

// Token splits of the router weight gradient: about 1024 workgroups (each
// split costs a memory round trip per 32 tokens), at least 64 tokens each,
// at most 256 splits.
int router_wgrad_splits(int E, int d, int64_t T) {
  const int64_t tiles = (int64_t)((E + 63) / 64) * ((d + 63) / 64);
  int64_t want = (1024 + tiles - 1) / tiles;
  const int64_t most = (T + 63) / 64;
  if (want > most) want = most;
  if (want > 256) want = 256;
  if (want < 1) want = 1;
  const int64_t kchunk = ((T + want - 1) / want + kRK - 1) / kRK * kRK;
  return (int)((T + kchunk - 1) / kchunk);
}

int64_t router_wgrad_split_ld(int E, int d) { return ((int64_t)E * d + E + 3) / 4 * 4; }

hipError_t launch_dx_final(const moe_config& c, const float* dl, const void* w_router,
                           const void* dx_rows, const int32_t* inv_row, const void* shared,
                           const void* residual, void* dx, hipStream_t s) {
  const dim3 grid(blocks_for(c.d_model, 64), blocks_for(c.n_tokens, 64));
  dx_final_kernel<<<grid, kThreads, 0, s>>>(
      dl, static_cast<const uint16_t*>(w_router), static_cast<const uint16_t*>(dx_rows), inv_row,
      static_cast<const uint16_t*>(shared), static_cast<const uint16_t*>(residual), c.n_tokens,
      c.d_model, c.n_experts, c.top_k, static_cast<uint16_t*>(dx));
  return hipGetLastError();
}

}  // namespace moe

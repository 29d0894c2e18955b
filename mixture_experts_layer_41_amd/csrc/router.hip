// Fused router: logits GEMM (+ bias) -> softmax statistics -> top-k ->
// renormalised weights -> per-block routing statistics.
//
// [P2 §3.2]: the router is one linear layer, d_model -> E logits.
// [P3 §3.1] steps 1-2 and [P4 §3.1]: softmax over experts, top-k, divide the
// k probabilities by their sum.  Selection runs on the float32 logits (the
// softmax is monotone), in the total order (logit descending, index
// ascending), so equal logits pick the lower expert index.
//
// One workgroup (4 waves) owns BT consecutive tokens (BT = 16, 32 or 64,
// chosen so that there are enough workgroups to cover the chip) and all E
// experts.
//  * bf16 logits: v_mfma_f32_16x16x32_bf16 on 16-token x 16-expert tiles; A
//    (x rows) and B (W_r rows) are read straight from memory, 32 contiguous
//    bytes per lane per 64-wide K chunk (both operands use the same K order,
//    so the dot products are unchanged).  When a workgroup has fewer than 4
//    tiles, the waves split K and their partial tiles are added in LDS in a
//    fixed order.
//  * float32 logits: plain FMA dot products.
//  * selection: 256 / BT lanes per token; max, sum of exponentials and each
//    of the k picks are wave-shuffle reductions inside that lane group.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__host__ __device__ inline int round_up(int a, int b) { return (a + b - 1) / b * b; }

struct RouterShape {
  int BT, ep, n_tb, n_eb, n_tiles, nks, tiles_per_wave;
};

// bf16 = false: FMA logits, no K split
__host__ __device__ inline RouterShape router_shape(int64_t T, int E, bool bf16) {
  RouterShape s;
  s.BT = route_block_tokens(T, E);
  s.ep = round_up(E, 16);
  s.n_tb = s.BT / 16;
  s.n_eb = s.ep / 16;
  s.n_tiles = s.n_tb * s.n_eb;
  s.nks = (!bf16 || s.n_tiles >= 4) ? 1 : 4 / s.n_tiles;  // waves per tile (K split)
  const int groups = 4 / s.nks;                 // waves with distinct tiles
  s.tiles_per_wave = (s.n_tiles + groups - 1) / groups;
  return s;
}

// LDS: partial logits [nks][BT][ep + 1] f32, counts [ep] i32, lse^2 [BT] f32
__host__ __device__ inline int router_smem_bytes_for(const RouterShape& s) {
  return s.nks * s.BT * (s.ep + 1) * 4 + s.ep * 4 + s.BT * 4;
}

// Logits of the block's tokens into LDS (bf16, MFMA).  TPW = compile-time
// bound on the tiles a wave owns, so the accumulators stay in registers.  All
// of a wave's tiles share one 16-token row block (tile t = grp + 4 i with the
// row block t mod n_tb, n_tb in {1, 2, 4}), so A is loaded once per chunk.
// U chunks are loaded before their MFMAs are issued, to keep several memory
// requests in flight per wave.
template <int TPW>
__device__ void logits_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                            int64_t T, int d, int E, int64_t t0, const RouterShape& s,
                            float* __restrict__ part) {
  constexpr int U = TPW <= 2 ? 4 : (TPW <= 4 ? 2 : 1);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int ks = wave % s.nks;          // K slice of this wave
  const int grp = wave / s.nks;         // tile group
  const int ngrp = 4 / s.nks;
  const int nch = (d + 63) / 64;        // 64-wide K chunks
  const int c0 = ks * nch / s.nks, c1 = (ks + 1) * nch / s.nks;
  const int kq = 16 * (lane / 16);      // this lane's 16 K elements of a chunk

  f32x4 acc[TPW];
  const uint16_t* brow[TPW];
  bool tok_ok[TPW], bok[TPW];
  const int tb = (grp < s.n_tiles ? grp : 0) % s.n_tb;
  int64_t tok = t0 + tb * 16 + (lane % 16);
  if (tok >= T) tok = T - 1;
  const uint16_t* arow = x + tok * (int64_t)d + kq;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int t = grp + i * ngrp;
    tok_ok[i] = t < s.n_tiles;
    const int eb = tok_ok[i] ? t / s.n_tb : 0;
    const int e = eb * 16 + (lane % 16);
    bok[i] = tok_ok[i] && e < E;
    brow[i] = wr + (int64_t)(bok[i] ? e : 0) * d + kq;
  }
  for (int c = c0; c < c1; c += U) {
    uint4 A[U][2], B[U][TPW][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (c + u) * 64;
      const bool in = c + u < c1;
      const bool ok0 = in && k0 + kq < d, ok1 = in && k0 + kq + 8 < d;
      A[u][0] = ok0 ? *reinterpret_cast<const uint4*>(arow + k0) : make_uint4(0, 0, 0, 0);
      A[u][1] = ok1 ? *reinterpret_cast<const uint4*>(arow + k0 + 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        B[u][i][0] = (bok[i] && ok0) ? *reinterpret_cast<const uint4*>(brow[i] + k0) : make_uint4(0, 0, 0, 0);
        B[u][i][1] = (bok[i] && ok1) ? *reinterpret_cast<const uint4*>(brow[i] + k0 + 8) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        if (!tok_ok[i]) continue;
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[u][0]),
                                                         __builtin_bit_cast(bf16x8, B[u][i][0]), acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[u][1]),
                                                         __builtin_bit_cast(bf16x8, B[u][i][1]), acc[i], 0, 0, 0);
      }
    }
  }
  // 16x16 C layout: lane holds rows 4*(lane/16) + r, column lane%16
  float* pk = part + ks * s.BT * (s.ep + 1);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = grp + i * ngrp;
    if (t >= s.n_tiles) continue;
    const int eb = t / s.n_tb;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      pk[(tb * 16 + 4 * (lane / 16) + r) * (s.ep + 1) + eb * 16 + (lane % 16)] = acc[i][r];
  }
}

// Logits of the block's tokens into LDS (float32, FMA).
__device__ void logits_f32(const float* __restrict__ x, const float* __restrict__ wr, int64_t T,
                           int d, int E, int64_t t0, const RouterShape& s, float* __restrict__ part) {
  for (int o = threadIdx.x; o < s.BT * E; o += kThreads) {
    const int r = o / E, e = o % E;
    int64_t tok = t0 + r;
    if (tok >= T) tok = T - 1;
    const float* xr = x + tok * (int64_t)d;
    const float* wrow = wr + (int64_t)e * d;
    float acc = 0.f;
    for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wrow[c], acc);
    part[r * (s.ep + 1) + e] = acc;
  }
}

template <int DT, int TPW>
__global__ void __launch_bounds__(kThreads)
router_kernel(const void* __restrict__ x, const void* __restrict__ wr,
              const float* __restrict__ rbias, int64_t T, int d, int E, int k,
              int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
              float* __restrict__ token_lse, int32_t* __restrict__ st_cnt,
              float* __restrict__ st_psum, float* __restrict__ st_zsum) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouterShape s = router_shape(T, E, DT == MOE_DTYPE_BF16);
  const int BT = s.BT, ep = s.ep;
  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * BT;
  const int nvalid = (int)((T - t0) < BT ? (T - t0) : BT);
  float* part = reinterpret_cast<float*>(smem);
  float* lg = part;  // K-slice 0 holds the summed logits
  int32_t* cnt = reinterpret_cast<int32_t*>(smem + s.nks * BT * (ep + 1) * 4);
  float* lse2 = reinterpret_cast<float*>(cnt + ep);

  for (int e = threadIdx.x; e < ep; e += kThreads) cnt[e] = 0;
  if (DT == MOE_DTYPE_BF16)
    logits_bf16<TPW>(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr), T, d, E, t0,
                     s, part);
  else
    logits_f32(static_cast<const float*>(x), static_cast<const float*>(wr), T, d, E, t0, s, part);
  __syncthreads();
  // sum the K slices in a fixed order and add the bias
  for (int o = threadIdx.x; o < BT * E; o += kThreads) {
    const int r = o / E, e = o % E;
    float v = lg[r * (ep + 1) + e];
    for (int q = 1; q < s.nks; ++q) v += part[(q * BT + r) * (ep + 1) + e];
    lg[r * (ep + 1) + e] = v + (rbias ? rbias[e] : 0.f);
  }
  __syncthreads();

  // selection: G = 256 / BT consecutive lanes per token
  const int G = kThreads / BT;
  const int r = threadIdx.x / G, sub = threadIdx.x % G;
  const bool valid = r < nvalid;
  const int64_t tok = t0 + r;
  float* row = lg + r * (ep + 1);
  float m = -INFINITY;
#pragma unroll 4
  for (int e = sub; e < E; e += G) m = fmaxf(m, row[e]);
  for (int o = G / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, G));
  float z = 0.f;
#pragma unroll 4
  for (int e = sub; e < E; e += G) z += expf(row[e] - m);
  for (int o = G / 2; o > 0; o >>= 1) z += __shfl_xor(z, o, G);
  const float lse = m + logf(z);
  if (valid && sub == 0) {
    if (token_lse) token_lse[tok] = lse;
    lse2[r] = lse * lse;
  }
  // k picks; each takes the best element strictly after the previous pick in
  // the order (logit desc, index asc)
  float prev_l = INFINITY, wsum = 0.f;
  int prev_e = -1;
  for (int j = 0; j < k; ++j) {
    float bl = -INFINITY;
    int be = 0x7FFFFFFF;
    for (int e = sub; e < E; e += G) {
      const float l = row[e];
      const bool after = (l < prev_l) || (l == prev_l && e > prev_e);
      if (after && (be == 0x7FFFFFFF || l > bl || (l == bl && e < be))) {
        bl = l;
        be = e;
      }
    }
    for (int o = G / 2; o > 0; o >>= 1) {
      const float ol = __shfl_xor(bl, o, G);
      const int oe = __shfl_xor(be, o, G);
      if (oe != 0x7FFFFFFF && (be == 0x7FFFFFFF || ol > bl || (ol == bl && oe < be))) {
        bl = ol;
        be = oe;
      }
    }
    if (be == 0x7FFFFFFF) be = j % E;  // only reachable with NaN logits: keep indices in range
    const float ex = expf(bl - m);
    wsum += ex;
    if (valid && sub == 0) {
      topk_idx[tok * k + j] = be;
      topk_w[tok * k + j] = ex;
      atomicAdd(&cnt[be], 1);
    }
    prev_l = bl;
    prev_e = be;
  }
  if (valid && sub == 0) {
    const float inv = 1.f / wsum;
    for (int j = 0; j < k; ++j) topk_w[tok * k + j] *= inv;
  }
  // probabilities for the per-expert sums
  const float iz = 1.f / z;
  if (valid)
    for (int e = sub; e < E; e += G) row[e] = expf(row[e] - m) * iz;
  __syncthreads();

  for (int e = threadIdx.x; e < E; e += kThreads) {
    float acc = 0.f;
#pragma unroll 8
    for (int q = 0; q < nvalid; ++q) acc += lg[q * (ep + 1) + e];
    st_psum[blk * E + e] = acc;
    st_cnt[blk * E + e] = cnt[e];
  }
  if (threadIdx.x == 0) {
    float acc = 0.f;
#pragma unroll 8
    for (int q = 0; q < nvalid; ++q) acc += lse2[q];
    st_zsum[blk] = acc;
  }
}

template <int DT, int TPW>
hipError_t router_launch_t(const moe_config& c, const void* x, const void* w_router,
                           const float* router_bias, int32_t* topk_idx, float* topk_w,
                           float* token_lse, const RouteStats& st, hipStream_t s) {
  const RouterShape sh = router_shape(c.n_tokens, c.n_experts, DT == MOE_DTYPE_BF16);
  const int64_t nb = (c.n_tokens + sh.BT - 1) / sh.BT;
  const int smem = router_smem_bytes_for(sh);
  auto fn = router_kernel<DT, TPW>;
  if (smem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
  }
  fn<<<dim3((unsigned)nb), dim3(kThreads), smem, s>>>(
      x, w_router, router_bias, c.n_tokens, c.d_model, c.n_experts, c.top_k, topk_idx, topk_w,
      token_lse, st.cnt, st.psum, st.zsum);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const moe_config& c, const void* x, const void* w_router,
                         const float* router_bias, int32_t* topk_idx, float* topk_w,
                         float* token_lse, const RouteStats& st, hipStream_t s) {
  if (c.dtype == MOE_DTYPE_F32)
    return router_launch_t<MOE_DTYPE_F32, 1>(c, x, w_router, router_bias, topk_idx, topk_w,
                                             token_lse, st, s);
  const int tpw = router_shape(c.n_tokens, c.n_experts, true).tiles_per_wave;
#define MOE_ROUTER_CASE(N) \
  if (tpw <= N)            \
    return router_launch_t<MOE_DTYPE_BF16, N>(c, x, w_router, router_bias, topk_idx, topk_w, token_lse, st, s);
  MOE_ROUTER_CASE(1)
  MOE_ROUTER_CASE(2)
  MOE_ROUTER_CASE(4)
  MOE_ROUTER_CASE(8)
  MOE_ROUTER_CASE(16)
#undef MOE_ROUTER_CASE
  return hipErrorInvalidConfiguration;
}

}  // namespace moe

// Fused router: logits GEMM (+ bias) -> softmax statistics -> top-k ->
// renormalised weights -> per-block routing statistics.
//
// [P2 §3.2]: the router is one linear layer, d_model -> E logits.
// [P3 §3.1] steps 1-2 and [P4 §3.1]: softmax over experts, top-k, divide the
// k probabilities by their sum.  Selection runs on the float32 logits (the
// softmax is monotone), in the total order (logit descending, index
// ascending), so equal logits pick the lower expert index.
//
// One workgroup (4 waves) owns BT consecutive tokens and all E experts.
// bf16: the logits tile comes from v_mfma_f32_16x16x32_bf16, A = x rows read
// straight from HBM into registers, B = a 64-wide K-chunk of W_r staged in
// LDS and shared by the 4 waves.  f32: plain FMA dot products.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kKC = 64;            // K chunk of the bf16 router
constexpr int kWrPitch = kKC + 8;  // bf16 elements per LDS row of the W_r chunk (pad: bank spread)

struct RouterSmem {
  // offsets in bytes into dynamic LDS
  int wr;      // bf16 [E_pad][kWrPitch]
  int logits;  // f32 [BT][E_pad + 1]
  int cnt;     // i32 [E_pad]
  int lse2;    // f32 [BT]
  int total;
};

__host__ __device__ inline int round_up(int a, int b) { return (a + b - 1) / b * b; }

__host__ __device__ inline RouterSmem router_smem(int E, int BT, bool bf16) {
  const int ep = round_up(E, 16);
  RouterSmem s;
  int off = 0;
  s.wr = off;
  off += bf16 ? ep * kWrPitch * 2 : 0;
  off = round_up(off, 16);
  s.logits = off;
  off += BT * (ep + 1) * 4;
  s.cnt = off;
  off += ep * 4;
  s.lse2 = off;
  off += BT * 4;
  s.total = round_up(off, 16);
  return s;
}

// Logits of the block's tokens into LDS (bf16, MFMA).  EBW = expert blocks
// of 16 handled by one wave (compile-time so the accumulators stay in registers).
template <int EBW>
__device__ void logits_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                            const float* __restrict__ rbias, int64_t T, int d, int E, int BT,
                            int64_t t0, char* smem, const RouterSmem& L) {
  const int ep = round_up(E, 16);
  const int n_eb = ep / 16;
  const int n_tb = BT / 16;         // token sub-blocks of 16
  const int n_eg = 4 / n_tb;        // expert groups sharing a token sub-block
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int tb = wave % n_tb;
  const int eg = wave / n_tb;
  uint16_t* wr_s = reinterpret_cast<uint16_t*>(smem + L.wr);
  float* lg = reinterpret_cast<float*>(smem + L.logits);

  // this lane's A row (token), clamped into range for the tail block
  int64_t tok = t0 + tb * 16 + (lane % 16);
  if (tok >= T) tok = T - 1;
  const uint16_t* xrow = x + tok * (int64_t)d;
  const int kq = 16 * (lane / 16);  // this lane's 16-element slice of a 64-wide chunk

  f32x4 acc[EBW];
#pragma unroll
  for (int i = 0; i < EBW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < d; k0 += kKC) {
    // stage W_r[:, k0:k0+64] (zero-filled past d and past E)
    for (int c = threadIdx.x; c < ep * (kKC / 8); c += kThreads) {
      const int e = c / (kKC / 8);
      const int kk = (c % (kKC / 8)) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (e < E && k0 + kk < d) v = *reinterpret_cast<const uint4*>(wr + (int64_t)e * d + k0 + kk);
      *reinterpret_cast<uint4*>(wr_s + e * kWrPitch + kk) = v;
    }
    // A fragments: 16 consecutive K elements of this lane's token
    uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
    if (k0 + kq < d) a0 = *reinterpret_cast<const uint4*>(xrow + k0 + kq);
    if (k0 + kq + 8 < d) a1 = *reinterpret_cast<const uint4*>(xrow + k0 + kq + 8);
    __syncthreads();
    const bf16x8 fa0 = __builtin_bit_cast(bf16x8, a0);
    const bf16x8 fa1 = __builtin_bit_cast(bf16x8, a1);
#pragma unroll
    for (int i = 0; i < EBW; ++i) {
      const int eb = eg + i * n_eg;
      if (eb < n_eb) {
        const uint16_t* brow = wr_s + (eb * 16 + (lane % 16)) * kWrPitch + kq;
        const bf16x8 fb0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(brow));
        const bf16x8 fb1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(brow + 8));
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0, fb0, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1, fb1, acc[i], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // C layout of the 16x16 product: lane holds rows 4*(lane/16)+i, column lane%16
#pragma unroll
  for (int i = 0; i < EBW; ++i) {
    const int eb = eg + i * n_eg;
    if (eb < n_eb) {
      const int e = eb * 16 + (lane % 16);
      const float b = (rbias != nullptr && e < E) ? rbias[e] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = tb * 16 + 4 * (lane / 16) + r;
        lg[row * (ep + 1) + e] = acc[i][r] + b;
      }
    }
  }
}

// Logits of the block's tokens into LDS (float32, FMA).
__device__ void logits_f32(const float* __restrict__ x, const float* __restrict__ wr,
                           const float* __restrict__ rbias, int64_t T, int d, int E, int BT,
                           int64_t t0, char* smem, const RouterSmem& L) {
  const int ep = round_up(E, 16);
  float* lg = reinterpret_cast<float*>(smem + L.logits);
  for (int o = threadIdx.x; o < BT * E; o += kThreads) {
    const int r = o / E, e = o % E;
    int64_t tok = t0 + r;
    if (tok >= T) tok = T - 1;
    const float* xr = x + tok * (int64_t)d;
    const float* wrow = wr + (int64_t)e * d;
    float acc = 0.f;
    for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wrow[c], acc);
    lg[r * (ep + 1) + e] = acc + (rbias ? rbias[e] : 0.f);
  }
}

template <int DT, int EBW>
__global__ void __launch_bounds__(kThreads)
router_kernel(const void* __restrict__ x, const void* __restrict__ wr,
              const float* __restrict__ rbias, int64_t T, int d, int E, int k, int BT,
              int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
              float* __restrict__ token_lse, int32_t* __restrict__ st_cnt,
              float* __restrict__ st_psum, float* __restrict__ st_zsum) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouterSmem L = router_smem(E, BT, DT == MOE_DTYPE_BF16);
  const int ep = round_up(E, 16);
  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * BT;
  const int nvalid = (int)((T - t0) < BT ? (T - t0) : BT);
  float* lg = reinterpret_cast<float*>(smem + L.logits);
  int32_t* cnt = reinterpret_cast<int32_t*>(smem + L.cnt);
  float* lse2 = reinterpret_cast<float*>(smem + L.lse2);

  for (int e = threadIdx.x; e < ep; e += kThreads) cnt[e] = 0;
  if (DT == MOE_DTYPE_BF16)
    logits_bf16<EBW>(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr), rbias, T, d, E,
                BT, t0, smem, L);
  else
    logits_f32(static_cast<const float*>(x), static_cast<const float*>(wr), rbias, T, d, E, BT,
               t0, smem, L);
  __syncthreads();

  // one thread per token: softmax statistics, top-k, weights
  if (threadIdx.x < nvalid) {
    const int r = threadIdx.x;
    const int64_t tok = t0 + r;
    float* row = lg + r * (ep + 1);
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmaxf(m, row[e]);
    float z = 0.f;
    for (int e = 0; e < E; ++e) z += expf(row[e] - m);
    const float lse = m + logf(z);
    if (token_lse) token_lse[tok] = lse;
    lse2[r] = lse * lse;

    // k passes in the order (logit desc, index asc): each pass takes the best
    // element strictly after the previous pick in that order.
    float prev_l = INFINITY;
    int prev_e = -1;
    float wsum = 0.f;
    int32_t* out_i = topk_idx + tok * k;
    float* out_w = topk_w + tok * k;
    for (int j = 0; j < k; ++j) {
      float best_l = -INFINITY;
      int best_e = -1;
      for (int e = 0; e < E; ++e) {
        const float l = row[e];
        const bool after = (l < prev_l) || (l == prev_l && e > prev_e);
        if (after && (best_e < 0 || l > best_l)) {
          best_l = l;
          best_e = e;
        }
      }
      if (best_e < 0) best_e = j % E;  // only reachable with NaN logits: keep indices in range
      const float ex = expf(best_l - m);
      out_i[j] = best_e;
      out_w[j] = ex;
      wsum += ex;
      atomicAdd(&cnt[best_e], 1);
      prev_l = best_l;
      prev_e = best_e;
    }
    const float inv = 1.f / wsum;
    for (int j = 0; j < k; ++j) out_w[j] = out_w[j] * inv;
    // probabilities for the per-expert sums
    const float iz = 1.f / z;
    for (int e = 0; e < E; ++e) row[e] = expf(row[e] - m) * iz;
  }
  __syncthreads();

  for (int e = threadIdx.x; e < E; e += kThreads) {
    float s = 0.f;
    for (int r = 0; r < nvalid; ++r) s += lg[r * (ep + 1) + e];
    st_psum[blk * E + e] = s;
    st_cnt[blk * E + e] = cnt[e];
  }
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int r = 0; r < nvalid; ++r) s += lse2[r];
    st_zsum[blk] = s;
  }
}

}  // namespace

// expert blocks of 16 per wave for this E (see logits_bf16)
static int router_ebw(int E) {
  const int BT = route_block_tokens(E);
  const int n_eb = (E + 15) / 16;
  const int n_eg = 4 / (BT / 16);
  const int need = (n_eb + n_eg - 1) / n_eg;
  int ebw = 1;
  while (ebw < need) ebw *= 2;
  return ebw;
}

template <int DT, int EBW>
static hipError_t router_launch_t(const moe_config& c, const void* x, const void* w_router,
                                  const float* router_bias, int32_t* topk_idx, float* topk_w,
                                  float* token_lse, const RouteStats& st, hipStream_t s) {
  const int BT = route_block_tokens(c.n_experts);
  const int64_t nb = (c.n_tokens + BT - 1) / BT;
  const RouterSmem L = router_smem(c.n_experts, BT, DT == MOE_DTYPE_BF16);
  auto fn = router_kernel<DT, EBW>;
  if (L.total > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
    if (e != hipSuccess) return e;
  }
  fn<<<dim3((unsigned)nb), dim3(kThreads), L.total, s>>>(
      x, w_router, router_bias, c.n_tokens, c.d_model, c.n_experts, c.top_k, BT, topk_idx,
      topk_w, token_lse, st.cnt, st.psum, st.zsum);
  return hipGetLastError();
}

hipError_t launch_router(const moe_config& c, const void* x, const void* w_router,
                         const float* router_bias, int32_t* topk_idx, float* topk_w,
                         float* token_lse, const RouteStats& st, hipStream_t s) {
  if (c.dtype == MOE_DTYPE_F32)
    return router_launch_t<MOE_DTYPE_F32, 1>(c, x, w_router, router_bias, topk_idx, topk_w,
                                             token_lse, st, s);
  switch (router_ebw(c.n_experts)) {
    case 1: return router_launch_t<MOE_DTYPE_BF16, 1>(c, x, w_router, router_bias, topk_idx, topk_w, token_lse, st, s);
    case 2: return router_launch_t<MOE_DTYPE_BF16, 2>(c, x, w_router, router_bias, topk_idx, topk_w, token_lse, st, s);
    case 4: return router_launch_t<MOE_DTYPE_BF16, 4>(c, x, w_router, router_bias, topk_idx, topk_w, token_lse, st, s);
    case 8: return router_launch_t<MOE_DTYPE_BF16, 8>(c, x, w_router, router_bias, topk_idx, topk_w, token_lse, st, s);
    default: return router_launch_t<MOE_DTYPE_BF16, 16>(c, x, w_router, router_bias, topk_idx, topk_w, token_lse, st, s);
  }
}

size_t router_smem_bytes(const moe_config& c) {
  const int BT = route_block_tokens(c.n_experts);
  return (size_t)router_smem(c.n_experts, BT, c.dtype == MOE_DTYPE_BF16).total;
}

}  // namespace moe

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
//    (x rows) and B (W_r rows) are read straight from memory, two 16-byte
//    loads per lane per 64-wide K chunk, the four lanes of a row covering 64
//    contiguous bytes per load (both operands use the same K order, so the
//    dot products are unchanged).  When a workgroup has fewer than 4
//    tiles, the waves split K and their partial tiles are added in LDS in a
//    fixed order.
//  * float32 logits: plain FMA dot products.
//  * selection: 256 / BT lanes per token, each holding its share of the
//    token's logits as order keys in registers; max, sum of exponentials
//    and each of the k picks end in DPP reductions inside that lane group.
//  * barriers order LDS data only (lds_barrier): no workgroup reads back
//    global memory it has written, so no barrier waits for stores;
//  * scores: everything after the logits GEMM sees
//    s = (logit + bias) / tau + noise ([P2 §5.1] temperature scaling,
//    [P2 §2.2] noise added before the top-k); with tau = 1 and no noise these
//    are the logits plus bias, bit for bit.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Score of token t (global index; rows past T only fill tile padding and
// read no noise) for expert e from its summed logit v.
__device__ __forceinline__ float router_score(float v, const RouterMod& m, int64_t t, int64_t T,
                                              int E, int e) {
  v += m.bias ? m.bias[e] : 0.f;
  v *= m.inv_tau;
  if (m.noise && t < T) v += m.noise[t * E + e];
  return v;
}

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
  // this lane's K elements of a 64-wide chunk: [kq, kq + 8) for the first
  // MFMA and [kq + 32, kq + 40) for the second, so the four lanes of a row
  // read 64 contiguous bytes per load
  const int kq = 8 * (lane / 16);

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
      const bool ok0 = in && k0 + kq < d, ok1 = in && k0 + kq + 32 < d;
      A[u][0] = ok0 ? *reinterpret_cast<const uint4*>(arow + k0) : make_uint4(0, 0, 0, 0);
      A[u][1] = ok1 ? *reinterpret_cast<const uint4*>(arow + k0 + 32) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        B[u][i][0] = (bok[i] && ok0) ? *reinterpret_cast<const uint4*>(brow[i] + k0) : make_uint4(0, 0, 0, 0);
        B[u][i][1] = (bok[i] && ok1) ? *reinterpret_cast<const uint4*>(brow[i] + k0 + 32) : make_uint4(0, 0, 0, 0);
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

// Order key of a logit: a larger logit has a larger key and -0 and +0 share
// one; NaN gets kNanKey = 1, below every number (-inf has 0x007FFFFF), so a
// NaN score is still picked (last, lower index first, with weight 0) and the
// k picks of a token stay distinct.  0 marks an expert that is absent or
// already picked.
constexpr uint32_t kNanKey = 1u;
__device__ inline uint32_t order_key(float l) {
  const uint32_t u = l == 0.f ? 0u : __float_as_uint(l);
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return l != l ? kNanKey : key;
}
__device__ inline float key_logit(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Lane exchanges inside aligned groups of 4, 8 or 16 lanes (DPP, no LDS
// traffic): xor 1 and xor 2 inside a quad, then the half-row mirror (lane i
// <-> 7 - i) and the row mirror (i <-> 15 - i).  Once every lane of a quad
// holds the quad's result, a mirror pairs each lane with a lane of the other
// half, so every lane of the group ends with the group's result; sums are
// the same in every lane (commutative pairs).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline void argmax_step(uint32_t& bk, int& be) {
  const uint32_t ok = dpp_u32<CTRL>(bk);
  const int oe = (int)dpp_u32<CTRL>((uint32_t)be);
  const bool take = ok > bk || (ok == bk && oe < be);
  bk = take ? ok : bk;
  be = take ? oe : be;
}
template <int CTRL>
__device__ inline void max_step(uint32_t& k) {
  const uint32_t o = dpp_u32<CTRL>(k);
  k = o > k ? o : k;
}
template <int CTRL>
__device__ inline void sum_step(float& z) {
  z += __uint_as_float(dpp_u32<CTRL>(__float_as_uint(z)));
}

// Softmax statistics, top-k selection and per-block routing statistics of
// BT tokens whose logits (bias included) are in lg [BT][ep + 1] (LDS).  cnt
// [ep] (zeroed by the caller) and lse2 [BT] are LDS scratch.  256 threads;
// G = 256 / BT consecutive lanes per token (4, 8 or 16), lane sub of a token
// owns experts e = sub + G i, i < NPL (NPL >= E / G), as order keys in
// registers.  Each of the k picks is a branch-free scan of the lane's keys,
// then a group arg-max in the order (logit descending, index ascending); the
// winner's key is then cleared in its owner lane.
template <int NPL>
__device__ __forceinline__ void select_and_stats_t(float* lg, int ep, int BT, int nvalid, int E, int k, int64_t t0,
                                   int64_t blk, int32_t* __restrict__ topk_idx,
                                   float* __restrict__ topk_w, float* __restrict__ token_lse,
                                   int32_t* __restrict__ st_cnt, float* __restrict__ st_psum,
                                   float* __restrict__ st_zsum, int32_t* cnt, float* lse2) {
  const int G = kThreads / BT;
  const int r = threadIdx.x / G, sub = threadIdx.x % G;
  const bool valid = r < nvalid;
  const int64_t tok = t0 + r;
  float* row = lg + r * (ep + 1);
  constexpr int kNone = 0x7FFFFFFF;
  uint32_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = sub + G * i;
    key[i] = e < E ? order_key(row[e]) : 0u;
  }
  // max over the numbers of the row (NaN ignored)
  uint32_t mk = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) mk = key[i] > mk ? key[i] : mk;
  max_step<kDppXor1>(mk);
  max_step<kDppXor2>(mk);
  if (G >= 8) max_step<kDppHalfMirror>(mk);
  if (G >= 16) max_step<kDppMirror>(mk);
  const float m = key_logit(mk);
  float z = 0.f;
#pragma unroll 4
  for (int e = sub; e < E; e += G) z += expf(row[e] - m);
  sum_step<kDppXor1>(z);
  sum_step<kDppXor2>(z);
  if (G >= 8) sum_step<kDppHalfMirror>(z);
  if (G >= 16) sum_step<kDppMirror>(z);
  const float lse = m + logf(z);
  if (valid && sub == 0) {
    if (token_lse) token_lse[tok] = lse;
    lse2[r] = lse * lse;
  }
  // the first kRegPicks weights stay in registers until they are
  // renormalised (no read-back of global memory); later ones (k > kRegPicks)
  // are stored and rescaled in place
  constexpr int kRegPicks = 8;
  float exv[kRegPicks];
  float wsum = 0.f;
  for (int j = 0; j < k; ++j) {
    // the lane's largest key, then its lowest index holding it
    uint32_t bk = key[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) bk = key[i] > bk ? key[i] : bk;
    int bi = -1;
#pragma unroll
    for (int i = NPL - 1; i >= 0; --i) bi = key[i] == bk ? i : bi;
    if (bk == 0u) bi = -1;
    const int my_e = bi >= 0 ? sub + G * bi : kNone;
    int be = my_e;
    argmax_step<kDppXor1>(bk, be);
    argmax_step<kDppXor2>(bk, be);
    if (G >= 8) argmax_step<kDppHalfMirror>(bk, be);
    if (G >= 16) argmax_step<kDppMirror>(bk, be);
    // the owner lane clears the winner's key
    const bool mine = be == my_e && bi >= 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) key[i] = (mine && i == bi) ? 0u : key[i];
    // every expert holds a key (a number or kNanKey), so k <= E picks always
    // find one; the guard only keeps the index in range
    if (be == kNone) be = j % E;
    const float ex = bk > kNanKey ? expf(key_logit(bk) - m) : 0.f;
    wsum += ex;
    if (valid && sub == 0) {
      topk_idx[tok * k + j] = be;
      if (j >= kRegPicks) topk_w[tok * k + j] = ex;
      atomicAdd(&cnt[be], 1);
    }
#pragma unroll
    for (int q = 0; q < kRegPicks; ++q)
      if (q == j) exv[q] = ex;
  }
  if (valid && sub == 0) {
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;  // only NaN picks: weights 0
#pragma unroll
    for (int q = 0; q < kRegPicks; ++q)
      if (q < k) topk_w[tok * k + q] = exv[q] * inv;
    for (int j = kRegPicks; j < k; ++j) topk_w[tok * k + j] *= inv;
  }
  // probabilities for the per-expert sums
  const float iz = 1.f / z;
  if (valid)
    for (int e = sub; e < E; e += G) row[e] = expf(row[e] - m) * iz;
  lds_barrier();

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

// Register budget chosen at run time (float32 router, split-K selection
// kernel).  The bfloat16 logits kernels instantiate select_and_stats_t with
// NPL = 4 TPW directly: a wave's TPW 16x16 tiles cover (BT / 16) * (ep / 16)
// <= 4 TPW tiles, and E / G <= BT * ep / 256 is that tile count.
__device__ void select_and_stats_any(float* lg, int ep, int BT, int nvalid, int E, int k, int64_t t0,
                                     int64_t blk, int32_t* __restrict__ topk_idx,
                                     float* __restrict__ topk_w, float* __restrict__ token_lse,
                                     int32_t* __restrict__ st_cnt, float* __restrict__ st_psum,
                                     float* __restrict__ st_zsum, int32_t* cnt, float* lse2) {
  const int npl = (E + kThreads / BT - 1) / (kThreads / BT);
#define MOE_SELECT(N)                                                                           \
  select_and_stats_t<N>(lg, ep, BT, nvalid, E, k, t0, blk, topk_idx, topk_w, token_lse, st_cnt, \
                        st_psum, st_zsum, cnt, lse2)
  if (npl <= 4) MOE_SELECT(4);
  else if (npl <= 8) MOE_SELECT(8);
  else if (npl <= 16) MOE_SELECT(16);
  else if (npl <= 32) MOE_SELECT(32);
  else MOE_SELECT(64);
#undef MOE_SELECT
}

template <int DT, int TPW>
__global__ void __launch_bounds__(kThreads)
router_kernel(const void* __restrict__ x, const void* __restrict__ wr,
              const RouterMod mod, int64_t T, int d, int E, int k,
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
  lds_barrier();
  // sum the K slices in a fixed order and add the bias
  for (int o = threadIdx.x; o < BT * E; o += kThreads) {
    const int r = o / E, e = o % E;
    float v = lg[r * (ep + 1) + e];
    for (int q = 1; q < s.nks; ++q) v += part[(q * BT + r) * (ep + 1) + e];
    const float sc = router_score(v, mod, t0 + r, T, E, e);
    lg[r * (ep + 1) + e] = sc;
    if (mod.scores_out && t0 + r < T) mod.scores_out[(t0 + r) * E + e] = sc;
  }
  lds_barrier();

  if (DT == MOE_DTYPE_BF16)
    select_and_stats_t<(4 * TPW < 64 ? 4 * TPW : 64)>(lg, ep, BT, nvalid, E, k, t0, blk, topk_idx,
                                                      topk_w, token_lse, st_cnt, st_psum, st_zsum,
                                                      cnt, lse2);
  else
    select_and_stats_any(lg, ep, BT, nvalid, E, k, t0, blk, topk_idx, topk_w, token_lse, st_cnt,
                         st_psum, st_zsum, cnt, lse2);
}

// ---------------------------------------------------------------------------
// bfloat16 router for batches that fill the chip, logits through a deep LDS
// pipeline.  Same workgroup, tiles and selection as router_kernel, but the
// x rows and the W_r rows of each 64-wide K chunk are copied straight into
// an LDS stage (16-byte direct copies, 8 lanes per 128-byte row: every copy
// covers 8 whole lines), kStagedNS stages deep, and the MFMA fragments are
// read from LDS: W_r is fetched once per workgroup instead of once per wave,
// and each wave keeps two chunks of copies in flight under the MFMAs.
// Stage rows: the BT token rows, then the ep expert rows (padding experts
// repeat expert 0; their logits are never read).  16-byte chunk c of row r
// sits at chunk c ^ ((r / 2) % 8): a fragment read (16 consecutive rows, one
// chunk) then hits 16 distinct 16-byte bank groups.
constexpr int kStagedNS = 3;

__host__ __device__ inline bool router_staged_fits(const RouterShape& s, int d) {
  return s.nks == 1 && d % 64 == 0 && (s.BT + s.ep) % 32 == 0 && s.ep <= 128;
}
__host__ __device__ inline int router_staged_smem_bytes(const RouterShape& s) {
  return kStagedNS * (s.BT + s.ep) * 128 + s.BT * (s.ep + 1) * 4 + s.ep * 4 + s.BT * 4;
}

// s_waitcnt vmcnt(n) lgkmcnt(0) for a wave-uniform n in [0, 15]
__device__ __forceinline__ void wait_vm_lgkm_dyn(int n) {
  __asm__ volatile("" ::: "memory");
  switch (n) {
#define MOE_W(N) case N: __builtin_amdgcn_s_waitcnt(0x0070 | N); break;
    MOE_W(0) MOE_W(1) MOE_W(2) MOE_W(3) MOE_W(4) MOE_W(5) MOE_W(6) MOE_W(7)
    MOE_W(8) MOE_W(9) MOE_W(10) MOE_W(11) MOE_W(12) MOE_W(13) MOE_W(14)
#undef MOE_W
    default: __builtin_amdgcn_s_waitcnt(0x0070 | 15); break;
  }
  __asm__ volatile("" ::: "memory");
}

template <int TPW>
__global__ void __launch_bounds__(kThreads, 2)
router_staged_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                     const RouterMod mod, int64_t T, int d, int E, int k,
                     int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                     float* __restrict__ token_lse, int32_t* __restrict__ st_cnt,
                     float* __restrict__ st_psum, float* __restrict__ st_zsum) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RouterShape s = router_shape(T, E, true);
  const int BT = s.BT, ep = s.ep;
  const int rows = BT + ep;                 // rows per stage (128 bytes each)
  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * BT;
  const int nvalid = (int)((T - t0) < BT ? (T - t0) : BT);
  u32x4* stages = reinterpret_cast<u32x4*>(smem);
  float* part = reinterpret_cast<float*>(smem + kStagedNS * rows * 128);
  int32_t* cnt = reinterpret_cast<int32_t*>(part + BT * (ep + 1));
  float* lse2 = reinterpret_cast<float*>(cnt + ep);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int nch = d / 64;

  // copies: instruction q covers stage rows 8q .. 8q + 7; wave w issues
  // q = w, w + 4, ... (lpw per wave); lane i -> row 8q + i / 8, LDS chunk
  // i % 8, global chunk (i % 8) ^ ((row / 2) % 8)
  const int lpw = rows / 32;
  constexpr int kMaxLpw = 6;                // rows <= 64 + 128
  const uint16_t* src[kMaxLpw];
#pragma unroll
  for (int i = 0; i < kMaxLpw; ++i) {
    const int q = wave + 4 * i;
    const int r = 8 * q + lane / 8;
    const int gc = (lane % 8) ^ ((r / 2) % 8);
    const uint16_t* rowp;
    if (r < BT) {
      int64_t tok = t0 + r;
      if (tok >= T) tok = T - 1;
      rowp = x + tok * (int64_t)d;
    } else {
      const int e = r - BT;
      rowp = wr + (int64_t)(e < E ? e : 0) * d;
    }
    src[i] = rowp + gc * 8;
  }
  auto issue = [&](int c) {
    u32x4* st = stages + (c % kStagedNS) * rows * 8;
#pragma unroll
    for (int i = 0; i < kMaxLpw; ++i)
      if (i < lpw)
        __builtin_amdgcn_global_load_lds(src[i] + (int64_t)c * 64, st + (wave + 4 * i) * 64, 16, 0, 0);
  };

  // tiles of this wave (as in logits_bf16): t = wave + 4 i, token block
  // t % n_tb (the same for all of the wave's tiles), expert block t / n_tb
  const int tb = wave % s.n_tb;
  const int ra = tb * 16 + lane % 16;       // A fragment row (stage row)
  const int ka = ((ra / 2) % 8);
  int rb[TPW], kb[TPW];
  bool tok_ok[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wave + 4 * i;
    tok_ok[i] = t < s.n_tiles;
    rb[i] = BT + (tok_ok[i] ? t / s.n_tb : 0) * 16 + lane % 16;
    kb[i] = (rb[i] / 2) % 8;
  }
  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int e = threadIdx.x; e < ep; e += kThreads) cnt[e] = 0;
  // prologue: chunks 0 .. NS-2 in flight, chunk 0 landed
  for (int c = 0; c < kStagedNS - 1; ++c)
    if (c < nch) issue(c);
  wait_vm_lgkm_dyn(nch > 1 ? lpw : 0);
  lds_barrier();
  for (int c = 0; c < nch; ++c) {
    if (c + kStagedNS - 1 < nch) issue(c + kStagedNS - 1);
    const u32x4* st = stages + (c % kStagedNS) * rows * 8;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // 16-byte chunk of this lane in the 32-wide K step: 4 ks + lane / 16
      const int ch = 4 * ks + lane / 16;
      const u32x4 a = st[ra * 8 + (ch ^ ka)];
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        if (!tok_ok[i]) continue;
        const u32x4 b = st[rb[i] * 8 + (ch ^ kb[i])];
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, b), acc[i], 0, 0, 0);
      }
    }
    // chunk c + 1 landed (the copies of chunk c + 2 may stay in flight);
    // every wave done with chunk c's stage before the next step refills it
    const int after = c + kStagedNS - 1 < nch ? lpw : 0;
    wait_vm_lgkm_dyn(c + 1 < nch ? after : 0);
    lds_barrier();
  }
  // 16x16 C layout: lane holds token rows 4*(lane/16) + r, expert column lane%16
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (!tok_ok[i]) continue;
    const int eb = (wave + 4 * i) / s.n_tb;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      part[(tb * 16 + 4 * (lane / 16) + r) * (ep + 1) + eb * 16 + (lane % 16)] = acc[i][r];
  }
  lds_barrier();
  float* lg = part;
  for (int o = threadIdx.x; o < BT * E; o += kThreads) {
    const int r = o / E, e = o % E;
    const float sc = router_score(lg[r * (ep + 1) + e], mod, t0 + r, T, E, e);
    lg[r * (ep + 1) + e] = sc;
    if (mod.scores_out && t0 + r < T) mod.scores_out[(t0 + r) * E + e] = sc;
  }
  lds_barrier();
  select_and_stats_t<(4 * TPW < 64 ? 4 * TPW : 64)>(lg, ep, BT, nvalid, E, k, t0, blk, topk_idx,
                                                    topk_w, token_lse, st_cnt, st_psum, st_zsum,
                                                    cnt, lse2);
}

template <int TPW>
hipError_t router_staged_launch(const moe_config& c, const void* x, const void* w_router,
                                const RouterMod& mod, int32_t* topk_idx, float* topk_w,
                                float* token_lse, const RouteStats& st, hipStream_t s) {
  const RouterShape sh = router_shape(c.n_tokens, c.n_experts, true);
  const int64_t nb = (c.n_tokens + sh.BT - 1) / sh.BT;
  const int smem = router_staged_smem_bytes(sh);
  auto fn = router_staged_kernel<TPW>;
  if (smem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
  }
  fn<<<dim3((unsigned)nb), dim3(kThreads), smem, s>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router), mod, c.n_tokens,
      c.d_model, c.n_experts, c.top_k, topk_idx, topk_w, token_lse, st.cnt, st.psum, st.zsum);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bfloat16 router: logits GEMM with x and W_r staged through LDS
//
// Workgroup (blk, ks): tokens [blk*BT, +BT), all experts, K chunks
// [c0, c1) of the ks-th split (one split unless the token blocks alone are
// too few to fill the chip).  Per chunk of CH K elements the workgroup copies
// the BT x rows and the ep W_r rows (16 bytes per lane, registers, the next
// chunk loaded while the current one feeds the MFMAs) into an LDS stage,
// rows XOR-swizzled in 16-byte pieces (piece' = piece ^ ((row / rpw) % ppr)
// with ppr pieces per row and rpw rows per 256-byte bank window).
// Waves own 16x16 tiles (v_mfma_f32_16x16x32_bf16); with fewer than four
// tiles, the waves split each chunk's K steps and their partial tiles are
// added in LDS in wave order.
struct Router2Shape {
  int BT, ep, n_tb, n_tiles, nks, tpw, ch, nch, ks, cps;  // cps: chunks per split
};

__host__ __device__ inline Router2Shape router2_shape(int64_t T, int E, int d) {
  Router2Shape s;
  s.BT = route_block_tokens(T, E);
  s.ep = round_up(E, 16);
  s.n_tb = s.BT / 16;
  s.n_tiles = s.n_tb * (s.ep / 16);
  s.nks = s.n_tiles >= 4 ? 1 : 4 / s.n_tiles;
  s.tpw = (s.n_tiles + (4 / s.nks) - 1) / (4 / s.nks);
  // K per chunk: one 32-wide K step per wave when the waves split K four
  // ways; narrower chunks keep two stages of 512 expert rows within LDS
  s.ch = s.nks == 4 ? 128 : (s.ep > 256 ? 32 : 64);
  s.nch = (d + s.ch - 1) / s.ch;
  const int64_t nb = (T + s.BT - 1) / s.BT;
  int ks = 1;
  if (nb < 128) ks = (int)((256 + nb - 1) / nb);
  if (ks > s.nch) ks = s.nch;
  s.cps = (s.nch + ks - 1) / ks;
  s.ks = (s.nch + s.cps - 1) / s.cps;  // no empty split
  return s;
}

// LDS of the logits kernel: 2 stages of (BT + ep) rows x ch bf16, then the
// partial logits [nks][BT][ep + 1] f32, counts [ep], lse^2 [BT]
__host__ __device__ inline int router2_stage_bytes(const Router2Shape& s) {
  return (s.BT + s.ep) * s.ch * 2;
}
__host__ __device__ inline int router2_smem_bytes(const Router2Shape& s) {
  return 2 * router2_stage_bytes(s) + s.nks * s.BT * (s.ep + 1) * 4 + s.ep * 4 + s.BT * 4;
}

template <int TPW>
__global__ void __launch_bounds__(kThreads)
router_bf16_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                   const RouterMod mod, int64_t T, int d, int E, int k,
                   int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                   float* __restrict__ token_lse, int32_t* __restrict__ st_cnt,
                   float* __restrict__ st_psum, float* __restrict__ st_zsum,
                   float* __restrict__ part_out) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const Router2Shape s = router2_shape(T, E, d);
  const int BT = s.BT, ep = s.ep, CH = s.ch;
  const int PPR = CH / 8;                    // 16-byte pieces per row
  const int rows = BT + ep;                  // rows per stage: tokens then experts
  const int64_t blk = blockIdx.x;
  const int ks = blockIdx.y;
  const int64_t t0 = blk * BT;
  const int nvalid = (int)((T - t0) < BT ? (T - t0) : BT);
  u32x4* stage0 = reinterpret_cast<u32x4*>(smem);
  u32x4* stage1 = stage0 + rows * PPR;
  float* part = reinterpret_cast<float*>(smem + 2 * router2_stage_bytes(s));
  int32_t* cnt = reinterpret_cast<int32_t*>(part + s.nks * BT * (ep + 1));
  float* lse2 = reinterpret_cast<float*>(cnt + ep);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int c0 = ks * s.cps, c1 = min(s.nch, c0 + s.cps);

  // copy slots: piece q = tid + 256 i -> row q / PPR, piece q % PPR
  const int RPW = 128 / CH;                  // rows per 256-byte bank window
  const int nload = (rows * PPR + kThreads - 1) / kThreads;
  constexpr int kMaxLoads = 18;  // (16 + 512) rows x 8 pieces / 256 lanes, rounded up
  const uint16_t* src[kMaxLoads];
  int dst[kMaxLoads];
#pragma unroll
  for (int i = 0; i < kMaxLoads; ++i) {
    src[i] = nullptr;
    dst[i] = -1;
    if (i >= nload) continue;
    const int q = tid + kThreads * i;
    if (q >= rows * PPR) continue;
    const int r = q / PPR, pc = q % PPR;
    const uint16_t* rowp;
    if (r < BT) {
      int64_t tok = t0 + r;
      if (tok >= T) tok = T - 1;
      rowp = x + tok * (int64_t)d;
    } else {
      const int e = r - BT;
      rowp = e < E ? wr + (int64_t)e * d : nullptr;  // padding experts: zeros
    }
    src[i] = rowp ? rowp + pc * 8 : nullptr;
    dst[i] = r * PPR + (pc ^ ((r / RPW) % PPR));
  }
  u32x4 reg[kMaxLoads];
#define MOE_ROUTER_LOAD(c_)                                                                  \
  do {                                                                                      \
    const int k0_ = (c_) * CH;                                                              \
    _Pragma("unroll") for (int i_ = 0; i_ < kMaxLoads; ++i_) {                             \
      const int kk_ = k0_ + ((tid + kThreads * i_) % PPR) * 8;                              \
      reg[i_] = (i_ < nload && src[i_] && kk_ < d)                                          \
                    ? *reinterpret_cast<const u32x4*>(src[i_] + k0_)                        \
                    : u32x4{0u, 0u, 0u, 0u};                                                \
    }                                                                                       \
  } while (0)
#define MOE_ROUTER_STORE(st_)                                                                \
  do {                                                                                      \
    _Pragma("unroll") for (int i_ = 0; i_ < kMaxLoads; ++i_)                               \
      if (i_ < nload && dst[i_] >= 0) (st_)[dst[i_]] = reg[i_];                              \
  } while (0)

  // tiles of this wave: t = grp + (4 / nks) * i, token block t % n_tb,
  // expert block t / n_tb; K steps of a chunk: ksub = wave % nks, + nks ...
  const int ngrp = 4 / s.nks, grp = wave / s.nks, ksub = wave % s.nks;
  const int ksteps = CH / 32;
  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (c0 < c1) {
    MOE_ROUTER_LOAD(c0);
    MOE_ROUTER_STORE(stage0);
  }
  lds_barrier();
  for (int c = c0; c < c1; ++c) {
    u32x4* cur = ((c - c0) & 1) ? stage1 : stage0;
    u32x4* nxt = ((c - c0) & 1) ? stage0 : stage1;
    if (c + 1 < c1) MOE_ROUTER_LOAD(c + 1);
    for (int kq = ksub; kq < ksteps; kq += s.nks) {
      // lane: row lane % 16 of its tile, pieces 4 * kq + lane / 16
      const int pc = 4 * kq + lane / 16;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int t = grp + ngrp * i;
        if (t >= s.n_tiles) break;
        const int ra = (t % s.n_tb) * 16 + lane % 16;
        const int rb = BT + (t / s.n_tb) * 16 + lane % 16;
        const u32x4 a = cur[ra * PPR + (pc ^ ((ra / RPW) % PPR))];
        const u32x4 b = cur[rb * PPR + (pc ^ ((rb / RPW) % PPR))];
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, b), acc[i], 0, 0, 0);
      }
    }
    if (c + 1 < c1) MOE_ROUTER_STORE(nxt);
    lds_barrier();
  }

#undef MOE_ROUTER_LOAD
#undef MOE_ROUTER_STORE
  // 16x16 C layout: lane holds token rows 4*(lane/16) + r, expert column lane%16
  float* pk = part + ksub * BT * (ep + 1);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = grp + ngrp * i;
    if (t >= s.n_tiles) break;
    const int tb = t % s.n_tb, eb = t / s.n_tb;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      pk[(tb * 16 + 4 * (lane / 16) + r) * (ep + 1) + eb * 16 + (lane % 16)] = acc[i][r];
  }
  for (int e = tid; e < ep; e += kThreads) cnt[e] = 0;
  lds_barrier();
  float* lg = part;  // wave-split slice 0 receives the sum
  if (s.ks > 1) {
    // K split over workgroups: this split's partial logits go out, in
    // [ks][T][E] order; the selection kernel adds the splits in order
    for (int o = tid; o < nvalid * E; o += kThreads) {
      const int r = o / E, e = o % E;
      float v = lg[r * (ep + 1) + e];
      for (int q = 1; q < s.nks; ++q) v += part[(q * BT + r) * (ep + 1) + e];
      part_out[((int64_t)ks * T + t0 + r) * E + e] = v;
    }
    return;
  }
  for (int o = tid; o < BT * E; o += kThreads) {
    const int r = o / E, e = o % E;
    float v = lg[r * (ep + 1) + e];
    for (int q = 1; q < s.nks; ++q) v += part[(q * BT + r) * (ep + 1) + e];
    const float sc = router_score(v, mod, t0 + r, T, E, e);
    lg[r * (ep + 1) + e] = sc;
    if (mod.scores_out && t0 + r < T) mod.scores_out[(t0 + r) * E + e] = sc;
  }
  lds_barrier();
  select_and_stats_t<(4 * TPW < 64 ? 4 * TPW : 64)>(lg, ep, BT, nvalid, E, k, t0, blk, topk_idx,
                                                    topk_w, token_lse, st_cnt, st_psum, st_zsum,
                                                    cnt, lse2);
}

// Selection after a K-split logits pass: the splits are added in split order.
__global__ void __launch_bounds__(kThreads)
router_select_kernel(const float* __restrict__ part_in, int nsplit, const RouterMod mod,
                     int64_t T, int E, int k, int32_t* __restrict__ topk_idx,
                     float* __restrict__ topk_w, float* __restrict__ token_lse,
                     int32_t* __restrict__ st_cnt, float* __restrict__ st_psum,
                     float* __restrict__ st_zsum) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int BT = route_block_tokens(T, E), ep = round_up(E, 16);
  const int64_t blk = blockIdx.x;
  const int64_t t0 = blk * BT;
  const int nvalid = (int)((T - t0) < BT ? (T - t0) : BT);
  float* lg = reinterpret_cast<float*>(smem);
  int32_t* cnt = reinterpret_cast<int32_t*>(lg + BT * (ep + 1));
  float* lse2 = reinterpret_cast<float*>(cnt + ep);
  for (int e = threadIdx.x; e < ep; e += kThreads) cnt[e] = 0;
  // the splits of each element added in split order.  Loads are
  // unconditional, from clamped addresses (a load under a per-lane condition
  // is waited for before the next one is issued), and the splits' loads are
  // in flight together in batches.
  const int n = nvalid * E;
  auto put_score = [&](int o, float v) {
    const int r = o / E, e = o % E;
    const float sc = router_score(v, mod, t0 + r, T, E, e);
    lg[r * (ep + 1) + e] = sc;
    if (mod.scores_out) mod.scores_out[(t0 + r) * E + e] = sc;
  };
  if (E % 4 == 0 && (reinterpret_cast<uintptr_t>(part_in) & 15u) == 0) {
    // 4 consecutive elements (16 bytes) per load, kV of them per thread,
    // kQ splits per batch
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int kV = 2, kQ = 14;
    const int n4 = n / 4;
    for (int o0 = 0; o0 < n4; o0 += kThreads * kV) {
      f4 v[kV];
#pragma unroll
      for (int i = 0; i < kV; ++i) v[i] = f4{0.f, 0.f, 0.f, 0.f};
      for (int q0 = 0; q0 < nsplit; q0 += kQ) {
        f4 w[kQ][kV];
#pragma unroll
        for (int u = 0; u < kQ; ++u) {
          const int q = min(q0 + u, nsplit - 1);
          const f4* src = reinterpret_cast<const f4*>(part_in + ((int64_t)q * T + t0) * E);
#pragma unroll
          for (int i = 0; i < kV; ++i) w[u][i] = src[min(o0 + (int)threadIdx.x + i * kThreads, n4 - 1)];
        }
#pragma unroll
        for (int u = 0; u < kQ; ++u)
          if (q0 + u < nsplit)
#pragma unroll
            for (int i = 0; i < kV; ++i) v[i] += w[u][i];
      }
#pragma unroll
      for (int i = 0; i < kV; ++i) {
        const int o = o0 + threadIdx.x + i * kThreads;
        if (o < n4)
#pragma unroll
          for (int c = 0; c < 4; ++c) put_score(4 * o + c, v[i][c]);
      }
    }
  } else {
    constexpr int kPer = 16, kQ = 4;
    for (int o0 = 0; o0 < n; o0 += kThreads * kPer) {
      float v[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) v[i] = 0.f;
      for (int q0 = 0; q0 < nsplit; q0 += kQ) {
        float w[kQ][kPer];
#pragma unroll
        for (int u = 0; u < kQ; ++u) {
          const int q = min(q0 + u, nsplit - 1);
#pragma unroll
          for (int i = 0; i < kPer; ++i)
            w[u][i] = part_in[((int64_t)q * T + t0) * E + min(o0 + (int)threadIdx.x + i * kThreads, n - 1)];
        }
#pragma unroll
        for (int u = 0; u < kQ; ++u)
          if (q0 + u < nsplit)
#pragma unroll
            for (int i = 0; i < kPer; ++i) v[i] += w[u][i];
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int o = o0 + threadIdx.x + i * kThreads;
        if (o < n) put_score(o, v[i]);
      }
    }
  }
  lds_barrier();
  select_and_stats_any(lg, ep, BT, nvalid, E, k, t0, blk, topk_idx, topk_w, token_lse, st_cnt,
                       st_psum, st_zsum, cnt, lse2);
}

template <int DT, int TPW>
hipError_t router_launch_t(const moe_config& c, const void* x, const void* w_router,
                           const RouterMod& mod, int32_t* topk_idx, float* topk_w,
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
      x, w_router, mod, c.n_tokens, c.d_model, c.n_experts, c.top_k, topk_idx, topk_w,
      token_lse, st.cnt, st.psum, st.zsum);
  return hipGetLastError();
}

template <int TPW>
hipError_t router_bf16_launch(const moe_config& c, const void* x, const void* w_router,
                              const RouterMod& mod, int32_t* topk_idx, float* topk_w,
                              float* token_lse, const RouteStats& st, hipStream_t s) {
  const Router2Shape sh = router2_shape(c.n_tokens, c.n_experts, c.d_model);
  const int64_t nb = (c.n_tokens + sh.BT - 1) / sh.BT;
  const int smem = router2_smem_bytes(sh);
  auto fn = router_bf16_kernel<TPW>;
  if (smem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
  }
  fn<<<dim3((unsigned)nb, (unsigned)sh.ks), dim3(kThreads), smem, s>>>(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router), mod,
      c.n_tokens, c.d_model, c.n_experts, c.top_k, topk_idx, topk_w, token_lse, st.cnt, st.psum,
      st.zsum, st.logit_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sh.ks == 1) return e;
  const int ssmem = sh.BT * (sh.ep + 1) * 4 + sh.ep * 4 + sh.BT * 4;
  router_select_kernel<<<dim3((unsigned)nb), dim3(kThreads), ssmem, s>>>(
      st.logit_part, sh.ks, mod, c.n_tokens, c.n_experts, c.top_k, topk_idx, topk_w,
      token_lse, st.cnt, st.psum, st.zsum);
  return hipGetLastError();
}

}  // namespace

size_t router_scratch_bytes(const moe_config& c) {
  if (c.dtype != MOE_DTYPE_BF16) return 0;
  const Router2Shape sh = router2_shape(c.n_tokens, c.n_experts, c.d_model);
  return sh.ks > 1 ? (size_t)sh.ks * c.n_tokens * c.n_experts * sizeof(float) : 0;
}

hipError_t launch_router(const moe_config& c, const void* x, const void* w_router,
                         const RouterMod& mod, int32_t* topk_idx, float* topk_w,
                         float* token_lse, const RouteStats& st, hipStream_t s) {
  if (c.dtype == MOE_DTYPE_F32)
    return router_launch_t<MOE_DTYPE_F32, 1>(c, x, w_router, mod, topk_idx, topk_w,
                                             token_lse, st, s);
  const Router2Shape sh2 = router2_shape(c.n_tokens, c.n_experts, c.d_model);
  if (sh2.ks > 1) {
    // decode-sized batch: K split over workgroups, then the selection
#define MOE_ROUTER2_CASE(N) \
    if (sh2.tpw <= N)       \
      return router_bf16_launch<N>(c, x, w_router, mod, topk_idx, topk_w, token_lse, st, s);
    MOE_ROUTER2_CASE(1)
    MOE_ROUTER2_CASE(2)
    MOE_ROUTER2_CASE(4)
    MOE_ROUTER2_CASE(8)
    MOE_ROUTER2_CASE(16)
    MOE_ROUTER2_CASE(32)
#undef MOE_ROUTER2_CASE
    return hipErrorInvalidConfiguration;
  }
  const RouterShape rs = router_shape(c.n_tokens, c.n_experts, true);
  const int tpw = rs.tiles_per_wave;
  if (router_staged_fits(rs, c.d_model)) {
    // batches that fill the chip with at least 4 tiles per workgroup
    if (tpw <= 1) return router_staged_launch<1>(c, x, w_router, mod, topk_idx, topk_w, token_lse, st, s);
    if (tpw <= 2) return router_staged_launch<2>(c, x, w_router, mod, topk_idx, topk_w, token_lse, st, s);
    if (tpw <= 4) return router_staged_launch<4>(c, x, w_router, mod, topk_idx, topk_w, token_lse, st, s);
    if (tpw <= 8) return router_staged_launch<8>(c, x, w_router, mod, topk_idx, topk_w, token_lse, st, s);
  }
#define MOE_ROUTER_CASE(N) \
  if (tpw <= N)            \
    return router_launch_t<MOE_DTYPE_BF16, N>(c, x, w_router, mod, topk_idx, topk_w, token_lse, st, s);
  MOE_ROUTER_CASE(1)
  MOE_ROUTER_CASE(2)
  MOE_ROUTER_CASE(4)
  MOE_ROUTER_CASE(8)
  MOE_ROUTER_CASE(16)
#undef MOE_ROUTER_CASE
  return hipErrorInvalidConfiguration;
}

}  // namespace moe

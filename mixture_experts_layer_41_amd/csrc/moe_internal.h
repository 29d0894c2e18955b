// Internal declarations shared by the HIP translation units of the MoE
// library: device helpers, launch descriptors and launcher prototypes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// constants

constexpr int kMaxExperts = 512;
constexpr int kWave = 64;

// Tokens per routing block: every routing-side kernel (router, histogram,
// scatter) splits the tokens into blocks of this many consecutive tokens, and
// the per-block expert counts feed the stable ranking.  The largest of 64,
// 32, 16 that still gives >= 512 blocks (two per CU), 16 for E > 256.
__host__ __device__ inline int route_block_tokens(int64_t n_tokens, int n_experts) {
  if (n_experts > 256) return 16;
  if (n_tokens >= 64 * 512) return 64;
  if (n_tokens >= 32 * 512) return 32;
  return 16;
}

// ---------------------------------------------------------------------------
// device helpers

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier for LDS data only: this wave's LDS accesses complete,
// then s_barrier.  __syncthreads also waits for every global store and load
// in flight (its release fence), which the callers do not need.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest even: gfx950's conversion
// instruction (v_cvt_pk_bf16_f32; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// two values in one 32-bit word (a in the low half): one instruction
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  const bf16x2_v v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// workspace of the routing side (one region per routing block)

struct RouteStats {
  int32_t* cnt;    // [nb, E] tokens of block b that picked expert e
  float* psum;     // [nb, E] sum over the block's tokens of p[t,e]
  float* zsum;     // [nb]    sum over the block's tokens of lse^2
  int32_t* bad;    // [nb]    invalid expert indices seen by the block (permute input check)
  float* logit_part;  // router K-split partial logits [splits][T][E] (router_scratch_bytes)
};

struct PermuteOut {
  int32_t* counts;      // [E] pre-capacity counts
  int32_t* offsets;     // [E+1] exclusive scan of kept counts
  int32_t* n_dropped;   // [1] (-1: an expert index was out of range)
  int32_t* perm_token;  // [T*k]
  float* perm_w;        // [T*k] or null
  int32_t* inv_row;     // [T*k]
};

// ---------------------------------------------------------------------------
// grouped GEMM descriptor

enum GemmKind : int { kGemmUp = 0, kGemmDown = 1 };

struct GemmDesc {
  // A: row r of the grouped problem reads a + (a_rows ? a_rows[r] : r) * lda
  const void* a;
  const int32_t* a_rows;
  int64_t lda;
  const int32_t* group_off;  // [n_groups + 1], device
  int n_groups;
  int n_seg;                 // FFN segments summed per group
  int64_t rows_max;          // host upper bound of group_off[n_groups]
  // up GEMM (N-segmented): out[r, s*f + n] = act(A[r] . W1[g*S+s] rows), K = d
  // down GEMM (K-segmented): out[r, n] = sum_s H[r, s*f:(s+1)*f] . W2[g*S+s][n], K = S*f
  const void* w;
  const float* w_scale;      // non-null: w holds int8 codes, one scale per weight row
  const void* bias;
  int d;                     // d_model
  int f;                     // d_ffn
  int act;                   // moe_act (up GEMM only)
  void* out;
  int64_t ldo;
  // up GEMM, bf16 only, optional: the pre-activations (bias added) are also
  // stored, at [row, seg * 2f + n] (gate) and [row, seg * 2f + f + n] (up)
  // for SwiGLU, at [row, seg * f + n] for GELU (the training forward keeps
  // them for the backward)
  void* preact;
  int64_t ldp;
};

// ---------------------------------------------------------------------------
// launchers (each returns hipGetLastError() of its launch)

// What turns the router's logits into its scores:
//   s[t, e] = (logit[t, e] + bias[e]) * inv_tau + noise[t, e]
struct RouterMod {
  const float* bias;   // [E] or null
  const float* noise;  // [T, E] or null
  float inv_tau;       // 1 / temperature
  float* scores_out;   // [T, E] or null: the scores are also written here
};

// Bytes of RouteStats::logit_part the router needs (0: no K split).
size_t router_scratch_bytes(const moe_config& c);
hipError_t launch_router(const moe_config& c, const void* x, const void* w_router,
                         const RouterMod& mod, int32_t* topk_idx, float* topk_w,
                         float* token_lse, const RouteStats& st, hipStream_t s);

hipError_t launch_histogram(const moe_config& c, const int32_t* topk_idx, const RouteStats& st,
                            hipStream_t s);

// Counts, offsets and the stable permutation from the per-block histograms
// in st; capacity < 0: no limit.  aux (may be null) needs st.psum / st.zsum.
// scratch: permute_scratch_bytes(c) bytes of device memory (may be 0).
size_t permute_scratch_bytes(const moe_config& c);
hipError_t launch_permute(const moe_config& c, const RouteStats& st, const PermuteOut& po,
                          int64_t capacity, const int32_t* topk_idx, const float* topk_w,
                          const void* x, void* x_perm, moe_aux* aux, void* scratch, hipStream_t s);

hipError_t launch_aux(const moe_config& c, const RouteStats& st, const int32_t* counts,
                      const int32_t* n_dropped, int64_t capacity, moe_aux* aux, hipStream_t s);

hipError_t launch_gemm(const moe_config& c, GemmKind kind, const GemmDesc& g, hipStream_t s);

hipError_t launch_combine(const moe_config& c, const void* y_perm, const int32_t* inv_row,
                          const float* topk_w, const void* shared_y, const void* residual,
                          void* y, hipStream_t s);

// ---------------------------------------------------------------------------
// backward pass (backward.hip, gemm_wgrad.hip); bf16 operands

// per-expert load-balance part of dL/dp when a term needs the mean router
// probability (lb_squares or kl_uniform weighted)
hipError_t launch_aux_dp(const moe_config& c, const float* scores, const float* lse,
                         const int32_t* counts, const moe_loss_weights& lw, float* aux_dp,
                         hipStream_t s);

// Combine and router backward in one launch; extra workgroups of the same
// launch pad the group offsets to multiples of `pad` and map the padded
// columns j < ncols to their source rows.
struct CombineRouterBwd {
  const void* dy;
  const void* y_perm;
  const int32_t* inv_row;
  const float* topk_w;
  void* d_yperm;          // [T k, d] bf16: d o rows (kept rows only)
  const float* scores;
  const float* lse;
  const int32_t* topk_idx;
  const int32_t* counts;
  const float* aux_dp;    // from launch_aux_dp, or null
  float* dl;              // [T, E] float32: dL/d logits
  const int32_t* offsets; // [E + 1]
  int pad;
  int64_t ncols;
  int32_t* poff;          // [E + 1]
  int32_t* colrow;        // [ncols]
};
hipError_t launch_combine_router_bwd(const moe_config& c, const moe_loss_weights& lw,
                                     const CombineRouterBwd& b, hipStream_t s);

// dst[b][c][j] = src[b][row(j)][c], c < C, j < ncols, row(j) = colrow ?
// colrow[j] : (j < nsrc ? j : -1), then through gather when given; negative
// rows read as zero.  Two problems per launch (b.batches = 0: one).
struct TransposeDesc {
  const void* src;
  int64_t src_ld, src_batch;
  const int32_t* colrow;
  const int32_t* gather;
  int64_t nsrc, ncols;
  int C;
  void* dst;
  int64_t dst_ld, dst_batch;
  int batches;
};
hipError_t launch_transpose(const TransposeDesc& a, const TransposeDesc& b, hipStream_t s);

// dW_r = dl^T x (float32 [E, d]) and, when db is given, db_r[e] = sum_t
// dl[t, e], split over tokens: nsplit from router_wgrad_splits, part
// (16-byte aligned) holding nsplit * router_wgrad_split_ld(E, d) floats.
struct RouterWgradDesc {
  const float* dl;  // [T, E]
  const void* x;    // [T, d] bf16
  int64_t T;
  int E, d, nsplit;
  float* part;
  float* dw;
  float* db;
};
int router_wgrad_splits(int E, int d, int64_t T);
int64_t router_wgrad_split_ld(int E, int d);
// The transposes a and b (batches = 0: none) in one launch, with more
// workgroups in the same launch for the router weight gradient: rp (if
// given) runs its split products, rs (if given) sums the splits.  Launch
// rs after rp, in a later launch.
hipError_t launch_side(const TransposeDesc& a, const TransposeDesc& b, const RouterWgradDesc* rp,
                       const RouterWgradDesc* rs, hipStream_t s);
hipError_t launch_act_bwd_t(const void* a, int64_t lda, const void* dh, int64_t ldh,
                            const int32_t* colrow, int64_t nsrc, int64_t ncols, int S, int f,
                            int act, void* da, void* dat, void* ht, int64_t ldt, hipStream_t s);
hipError_t launch_seg_rowsum(const void* m, int64_t ld, int C, const int32_t* poff, int64_t ncols,
                             int G, float* out, int64_t out_ld, hipStream_t s);
// dx_t = dl_t W_r + sum_j kept dx_rows[row_tj] (+ shared_t) (+ residual_t)
hipError_t launch_dx_final(const moe_config& c, const float* dl, const void* w_router,
                           const void* dx_rows, const int32_t* inv_row, const void* shared,
                           const void* residual, void* dx, hipStream_t s);
// Weight gradients C_b = A_b B_b^T (float32) over the K range of batch b:
// kofs[b] .. kofs[b + 1] (K = their total) or 0 .. K.  The plan picks the
// tile and a K split; a split product needs wgrad_partial_floats(...) floats
// of `partial` and a dense C (ldc = N, c_batch = M N).
struct WgradPlan {
  int tile;    // 128 or 256
  int nsplit;  // K splits per batch
};
WgradPlan wgrad_plan(int M, int N, int batches, int64_t k_avg);
size_t wgrad_partial_floats(const WgradPlan& w, int M, int N, int batches);
hipError_t launch_wgrad(const void* a, int64_t lda, int64_t a_batch, const void* b, int64_t ldb,
                        int64_t b_batch, const int32_t* kofs, int64_t K, int M, int N, int batches,
                        float* c, int64_t ldc, int64_t c_batch, float* partial, hipStream_t s);

}  // namespace moe

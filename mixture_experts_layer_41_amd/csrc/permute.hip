// Counts, capacity and the stable expert-contiguous permutation, plus the
// auxiliary statistics.
//
// [P4 §3.1]: capacity C = capacity_factor * tokens / E (taken here with the
// k assignments per token), overflow tokens dropped; in place of a loop over
// experts, flatten the assignments, reorder them by expert, compute, and
// scatter back by the original positions.  [P2 §4.1] keeps an expert_counts
// buffer.  [P1 §2.2]: overflow assignments are dropped (they contribute
// nothing; the caller's residual carries the token).
//
// Three kernels, all integer and atomic-free in global memory:
//   histogram (only when the router did not already count): per routing
//       block of BT tokens, how many tokens picked each expert;
//   scan (one workgroup): per expert the exclusive prefix of those counts
//       over blocks (= the rank base of the block's first token), the
//       pre-capacity totals, the kept counts min(total, C), their exclusive
//       scan (expert offsets) and the number of dropped assignments;
//   scatter (one wave per routing block): the rank of token t among the
//       block's tokens routed to e comes from a 64-bit LDS mask per expert;
//       rank = base + that; kept iff rank < C; row = offset[e] + rank.
// Ranks therefore follow ascending token order inside each expert, which
// makes the permutation unique and the capacity drop first-come.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(64)
histogram_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int E, int BT,
                 int32_t* __restrict__ cnt, int32_t* __restrict__ bad) {
  __shared__ int32_t c[kMaxExperts];
  __shared__ int32_t nbad;
  for (int e = threadIdx.x; e < E; e += 64) c[e] = 0;
  if (threadIdx.x == 0) nbad = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * BT + threadIdx.x;
  if (threadIdx.x < BT && t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E)
        atomicAdd(&c[e], 1);
      else
        atomicAdd(&nbad, 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64) cnt[(int64_t)blockIdx.x * E + e] = c[e];
  if (threadIdx.x == 0) bad[blockIdx.x] = nbad;
}

// Exclusive scan of v[0..n) in LDS (n <= kScanThreads), Hillis-Steele.
__device__ void block_exclusive_scan(int64_t* v, int64_t* tmp, int n) {
  const int i = threadIdx.x;
  int64_t x = (i < n) ? v[i] : 0;
  for (int off = 1; off < n; off <<= 1) {
    if (i < n) tmp[i] = x;
    __syncthreads();
    if (i < n && i >= off) x += tmp[i - off];
    __syncthreads();
  }
  // x is inclusive; shift
  if (i < n) tmp[i] = x;
  __syncthreads();
  if (i < n) v[i] = (i == 0) ? 0 : tmp[i - 1];
  __syncthreads();
}

// do_scan: compute bases/counts/offsets/drops from st.cnt.
// do_aux:  compute the moe_aux record; counts come from the scan (do_scan) or
//          from `counts_in`, drops from the scan or `dropped_in`.
__global__ void __launch_bounds__(kScanThreads)
scan_kernel(int do_scan, int do_aux, int64_t T, int k, int E, int64_t nb, int64_t cap,
            const int32_t* __restrict__ st_cnt, const float* __restrict__ st_psum,
            const float* __restrict__ st_zsum, const int32_t* __restrict__ st_bad,
            int32_t* __restrict__ base, int32_t* __restrict__ counts,
            int32_t* __restrict__ offsets, int32_t* __restrict__ n_dropped,
            const int32_t* __restrict__ counts_in, const int32_t* __restrict__ dropped_in,
            moe_aux* __restrict__ aux) {
  __shared__ int64_t part[kScanThreads];   // [G][E] partial sums of counts
  __shared__ double ppart[kScanThreads];   // [G][E] partial sums of probabilities
  __shared__ int64_t total[kMaxExperts + 1];
  __shared__ int64_t tmp[kScanThreads];
  __shared__ double red[kScanThreads];
  __shared__ int64_t ired[kScanThreads];
  const int tid = threadIdx.x;
  const int G = kScanThreads / E;  // E <= 512 -> G >= 2
  const int g = tid / E, e = tid % E;
  const bool act = tid < G * E;
  const int64_t b0 = act ? (g * nb) / G : 0;
  const int64_t b1 = act ? ((g + 1) * nb) / G : 0;

  // pass 1: per (g, e) partial sums over blocks [b0, b1)
  int64_t s = 0;
  double ps = 0.0;
  if (act) {
    for (int64_t b = b0; b < b1; ++b) {
      if (do_scan) s += st_cnt[b * E + e];
      if (do_aux) ps += (double)st_psum[b * E + e];
    }
    part[tid] = s;
    ppart[tid] = ps;
  }
  __syncthreads();
  // per expert: exclusive prefix over g, totals, P_e
  double P = 0.0;
  if (tid < E) {
    int64_t run = 0;
    for (int gg = 0; gg < G; ++gg) {
      const int64_t v = part[gg * E + tid];
      part[gg * E + tid] = run;
      run += v;
      P += ppart[gg * E + tid];
    }
    total[tid] = do_scan ? run : (int64_t)counts_in[tid];
  }
  __syncthreads();

  int64_t dropped = 0, kept_sum = 0, bad = 0;
  if (do_scan) {
    // pass 2: rank bases of every block
    if (act) {
      int64_t run = part[tid];
      for (int64_t b = b0; b < b1; ++b) {
        base[b * E + e] = (int32_t)run;
        run += st_cnt[b * E + e];
      }
    }
    // kept counts and their exclusive scan
    if (tid < E) {
      const int64_t tot = total[tid];
      const int64_t kept = (cap < 0 || tot < cap) ? tot : cap;
      counts[tid] = (int32_t)tot;
      tmp[tid] = kept;  // staged for the scan below
    }
    __syncthreads();
    if (tid < E) part[tid] = tmp[tid];
    __syncthreads();
    block_exclusive_scan(part, tmp, E);
    if (tid < E) {
      const int64_t tot = total[tid];
      const int64_t kept = (cap < 0 || tot < cap) ? tot : cap;
      offsets[tid] = (int32_t)part[tid];
      if (tid == E - 1) offsets[E] = (int32_t)(part[tid] + kept);
    }
    // dropped assignments and invalid indices: fixed-order block sums
    int64_t my_drop = 0, my_bad = 0;
    if (tid < E) {
      const int64_t tot = total[tid];
      my_drop = tot - ((cap < 0 || tot < cap) ? tot : cap);
    }
    if (st_bad)
      for (int64_t b = tid; b < nb; b += kScanThreads) my_bad += st_bad[b];
    ired[tid] = my_drop;
    tmp[tid] = my_bad;
    __syncthreads();
    for (int off = kScanThreads / 2; off > 0; off >>= 1) {
      if (tid < off) {
        ired[tid] += ired[tid + off];
        tmp[tid] += tmp[tid + off];
      }
      __syncthreads();
    }
    dropped = ired[0];
    bad = tmp[0];
    if (tid == 0) n_dropped[0] = bad ? -1 : (int32_t)dropped;
  } else if (tid == 0) {
    dropped = dropped_in[0];
  }

  if (do_aux) {
    // f_e P_e terms in LDS, then fixed-order sums
    if (tid < E) red[tid] = ((double)total[tid] / (double)(T * k)) * (P / (double)T);
    __syncthreads();
    double zs = 0.0;
    for (int64_t b = tid; b < nb; b += kScanThreads) zs += (double)st_zsum[b];
    __syncthreads();
    if (tid == 0) {
      double lb = 0.0;
      for (int i = 0; i < E; ++i) lb += red[i];
      red[0] = lb * (double)E;
    }
    __syncthreads();
    const double lb = red[0];
    __syncthreads();
    red[tid] = zs;
    __syncthreads();
    for (int off = kScanThreads / 2; off > 0; off >>= 1) {
      if (tid < off) red[tid] += red[tid + off];
      __syncthreads();
    }
    if (tid == 0) {
      for (int i = 0; i < E; ++i) kept_sum += total[i];  // pre-capacity sum = T*k
      const double z = red[0] / (double)T;
      aux->load_balance = lb;
      aux->z_loss = z;
      aux->weighted = 0.01 * lb + 0.001 * z;
      aux->n_dropped = dropped;
      aux->capacity = cap;
      aux->n_kept = kept_sum - dropped;
    }
  }
}

__global__ void __launch_bounds__(64)
scatter_kernel(const int32_t* __restrict__ idx, const float* __restrict__ topk_w, int64_t T,
               int k, int E, int BT, int64_t cap, const int32_t* __restrict__ base,
               const int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
               float* __restrict__ perm_w, int32_t* __restrict__ inv_row,
               const uint8_t* __restrict__ x, uint8_t* __restrict__ x_perm, int64_t row_bytes) {
  __shared__ unsigned long long mask[kMaxExperts];
  const int lane = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int64_t t = blk * BT + lane;
  const bool valid = lane < BT && t < T;
  for (int e = lane; e < E; e += 64) mask[e] = 0ull;
  __syncthreads();
  if (valid) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << lane);
    }
  }
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (valid) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      int32_t row = -1;
      if (e >= 0 && e < E) {
        const int64_t rank = (int64_t)base[blk * E + e] + __popcll(mask[e] & below);
        if (cap < 0 || rank < cap) {
          row = offsets[e] + (int32_t)rank;
          perm_token[row] = (int32_t)t;
          if (perm_w) perm_w[row] = topk_w[t * k + j];
        }
      }
      inv_row[t * k + j] = row;
    }
  }
  if (x_perm == nullptr) return;
  __syncthreads();  // inv_row of every lane is visible below
  // optional gather x_perm[row] = x[t]: the wave copies one row at a time
  for (int i = 0; i < BT * k; ++i) {
    const int r = i / k;
    const int64_t tt = blk * BT + r;
    if (r >= BT || tt >= T) break;
    const int32_t row = inv_row[tt * k + (i % k)];
    if (row < 0) continue;
    const uint4* src = reinterpret_cast<const uint4*>(x + tt * row_bytes);
    uint4* dst = reinterpret_cast<uint4*>(x_perm + (int64_t)row * row_bytes);
    for (int64_t c = lane; c < row_bytes / 16; c += 64) dst[c] = src[c];
  }
}

}  // namespace

hipError_t launch_histogram(const moe_config& c, const int32_t* topk_idx, const RouteStats& st,
                            hipStream_t s) {
  const int BT = route_block_tokens(c.n_tokens, c.n_experts);
  const int64_t nb = (c.n_tokens + BT - 1) / BT;
  histogram_kernel<<<dim3((unsigned)nb), dim3(64), 0, s>>>(topk_idx, c.n_tokens, c.top_k,
                                                           c.n_experts, BT, st.cnt, st.bad);
  return hipGetLastError();
}

hipError_t launch_scan(const moe_config& c, const RouteStats& st, const PermuteMeta& pm,
                       int64_t capacity, moe_aux* aux, hipStream_t s) {
  const int BT = route_block_tokens(c.n_tokens, c.n_experts);
  const int64_t nb = (c.n_tokens + BT - 1) / BT;
  scan_kernel<<<dim3(1), dim3(kScanThreads), 0, s>>>(
      1, aux != nullptr, c.n_tokens, c.top_k, c.n_experts, nb, capacity, st.cnt, st.psum,
      st.zsum, st.bad, pm.base, pm.counts, pm.offsets, pm.n_dropped, nullptr, nullptr, aux);
  return hipGetLastError();
}

hipError_t launch_aux(const moe_config& c, const RouteStats& st, const int32_t* counts,
                      const int32_t* n_dropped, int64_t capacity, moe_aux* aux, hipStream_t s) {
  const int BT = route_block_tokens(c.n_tokens, c.n_experts);
  const int64_t nb = (c.n_tokens + BT - 1) / BT;
  scan_kernel<<<dim3(1), dim3(kScanThreads), 0, s>>>(
      0, 1, c.n_tokens, c.top_k, c.n_experts, nb, capacity, nullptr, st.psum, st.zsum, nullptr,
      nullptr, nullptr, nullptr, nullptr, counts, n_dropped, aux);
  return hipGetLastError();
}

hipError_t launch_scatter(const moe_config& c, const int32_t* topk_idx, const float* topk_w,
                          const PermuteMeta& pm, int64_t capacity, int32_t* perm_token,
                          float* perm_w, int32_t* inv_row, const void* x, void* x_perm,
                          hipStream_t s) {
  const int BT = route_block_tokens(c.n_tokens, c.n_experts);
  const int64_t nb = (c.n_tokens + BT - 1) / BT;
  const int64_t row_bytes = (int64_t)c.d_model * (c.dtype == MOE_DTYPE_BF16 ? 2 : 4);
  scatter_kernel<<<dim3((unsigned)nb), dim3(64), 0, s>>>(
      topk_idx, topk_w, c.n_tokens, c.top_k, c.n_experts, BT, capacity, pm.base, pm.offsets,
      perm_token, perm_w, inv_row, static_cast<const uint8_t*>(x), static_cast<uint8_t*>(x_perm),
      row_bytes);
  return hipGetLastError();
}

}  // namespace moe

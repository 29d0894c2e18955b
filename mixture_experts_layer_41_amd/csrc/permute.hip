// Counts, capacity and the stable expert-contiguous permutation, plus the
// auxiliary statistics.
//
// [P4 §3.1]: capacity C = capacity_factor * tokens / E (taken here with the
// k assignments per token), overflow tokens dropped; in place of a loop over
// experts, flatten the assignments, reorder them by expert, compute, and
// scatter back by the original positions.  [P2 §4.1] keeps an expert_counts
// buffer.  [P1 §2.2]: overflow assignments are dropped (they contribute
// nothing; the caller's residual carries the token).  [P4 §3.1] / [P5 §2]:
// load-balance and router z-loss statistics.
//
// The tokens are cut into routing blocks of BT consecutive tokens; the router
// (or the histogram kernel) leaves cnt[b][e], the number of tokens of block b
// that picked expert e.  The rank of token t inside expert e is
//   (tokens of earlier blocks that picked e) + (earlier tokens of t's block
//   that picked e),
// the second term from a 64-bit LDS mask per expert and a popcount.  Ranks
// thus follow ascending token order inside each expert, which makes the
// permutation unique and the capacity drop first-come.  Kept iff rank < C;
// row = offset[e] + rank with offset the exclusive scan of min(count, C).
//
// Kernels (integer work, no floating-point atomics):
//   histogram   only when the router did not already count;
//   colscan     large tables only: one workgroup per expert scans cnt[.][e]
//               over the blocks (rank bases, totals, probability sums);
//   scatter     4 routing blocks per workgroup (one wave each); small tables
//               are summed in the workgroup itself, so no scan launch; one
//               extra workgroup writes counts, offsets, drops and the aux
//               record while the others scatter.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocksPerScatter = 4;     // routing blocks per scatter workgroup
constexpr int64_t kSmallTable = 8192;    // nb * E up to this: no colscan launch
constexpr int kBatch = 16;               // independent loads issued together
constexpr int kMaxKReg = 8;              // top-k indices of a token kept in registers

// Per-block expert counts of a caller's routing table, with its input check:
// an index outside [0, E) or an expert listed twice by one token is counted
// in bad[] (moe_permute then reports n_dropped = -1) and not in the counts,
// so the ranks of the scatter still cover every counted row.  Each thread
// owns one token and a bit set of the experts it has listed (LDS words only
// that thread touches).
__global__ void __launch_bounds__(64)
histogram_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int E, int BT,
                 int32_t* __restrict__ cnt, int32_t* __restrict__ bad) {
  constexpr int kSetWords = kMaxExperts / 32;
  __shared__ int32_t c[kMaxExperts];
  __shared__ uint32_t seen[64][kSetWords + 1];
  __shared__ int32_t nbad;
  for (int e = threadIdx.x; e < E; e += 64) c[e] = 0;
  if (threadIdx.x == 0) nbad = 0;
  uint32_t* mine = seen[threadIdx.x];
  for (int w = 0; w < kSetWords; ++w) mine[w] = 0u;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * BT + threadIdx.x;
  if (threadIdx.x < BT && t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      bool ok = e >= 0 && e < E;
      if (ok) {
        const uint32_t bit = 1u << (e & 31);
        ok = (mine[e >> 5] & bit) == 0u;
        mine[e >> 5] |= bit;
      }
      if (ok)
        atomicAdd(&c[e], 1);
      else
        atomicAdd(&nbad, 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64) cnt[(int64_t)blockIdx.x * E + e] = c[e];
  if (threadIdx.x == 0) bad[blockIdx.x] = nbad;
}

// Block-wide sums in a fixed order (tree over the thread index).
__device__ double block_sum_f64(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__device__ int64_t block_sum_i64(int64_t v, int64_t* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const int64_t r = red[0];
  __syncthreads();
  return r;
}

// Four block-wide sums at once (two integer, two float64): a butterfly over
// each wave (every lane ends with the same value), then the four wave
// partials added in wave order.  One barrier pair instead of a tree of
// barriers per sum.
__device__ void block_sum4(int64_t& i0, int64_t& i1, double& f0, double& f1, int64_t* ired,
                           double* red) {
  for (int o = kWave / 2; o > 0; o >>= 1) {
    i0 += __shfl_xor(i0, o);
    i1 += __shfl_xor(i1, o);
    f0 += __shfl_xor(f0, o);
    f1 += __shfl_xor(f1, o);
  }
  const int wave = threadIdx.x / kWave, nw = kThreads / kWave;
  if (threadIdx.x % kWave == 0) {
    ired[wave] = i0;
    ired[nw + wave] = i1;
    red[wave] = f0;
    red[nw + wave] = f1;
  }
  __syncthreads();
  i0 = ired[0];
  i1 = ired[nw];
  f0 = red[0];
  f1 = red[nw];
  for (int w = 1; w < nw; ++w) {
    i0 += ired[w];
    i1 += ired[nw + w];
    f0 += red[w];
    f1 += red[nw + w];
  }
  __syncthreads();
}

// Three float64 block-wide sums at once, in the same fixed order as
// block_sum4.
__device__ void block_sum3(double& f0, double& f1, double& f2, double* red) {
  for (int o = kWave / 2; o > 0; o >>= 1) {
    f0 += __shfl_xor(f0, o);
    f1 += __shfl_xor(f1, o);
    f2 += __shfl_xor(f2, o);
  }
  const int wave = threadIdx.x / kWave, nw = kThreads / kWave;
  if (threadIdx.x % kWave == 0) {
    red[wave] = f0;
    red[nw + wave] = f1;
    red[2 * nw + wave] = f2;
  }
  __syncthreads();
  f0 = red[0];
  f1 = red[nw];
  f2 = red[2 * nw];
  for (int w = 1; w < nw; ++w) {
    f0 += red[w];
    f1 += red[nw + w];
    f2 += red[2 * nw + w];
  }
  __syncthreads();
}

// Per-expert terms of the other load-balance forms ([P3 §3.1] E sum P^2;
// [P2 §4.2] KL(uniform || P) with 1e-8 in the logarithm, and the squared
// distance of the selection shares f from 1/E), added to sq, lg, fq.
__device__ __forceinline__ void lb_form_terms(double f, double P, int E, double& sq, double& lg,
                                              double& fq) {
  sq += P * P;
  lg += log(P + 1e-8);
  const double df = f - 1.0 / (double)E;
  fq += df * df;
}

// Writes the float64 statistics of the aux record from the block-summed
// parts (lbp = sum f P, lgp = sum ln(P + 1e-8), ...).
__device__ __forceinline__ void write_lb_forms(moe_aux* aux, int E, double lbp, double z,
                                               double sqp, double lgp, double fqp) {
  const double lb = lbp * (double)E;
  aux->load_balance = lb;
  aux->z_loss = z;
  aux->weighted = 0.01 * lb + 0.001 * z;
  aux->lb_squares = (double)E * sqp;
  aux->kl_uniform = log(1.0 / (double)E) - lgp / (double)E;
  aux->freq_penalty = fqp;
}

// One workgroup per expert e: rank bases base[b][e] = sum_{b' < b} cnt[b'][e],
// total[e], pe[e] = sum_b psum[b][e] (float64, fixed order); workgroup 0 also
// sums the lse^2 partials and the invalid-index counts.
__global__ void __launch_bounds__(kThreads)
colscan_kernel(int64_t nb, int E, const int32_t* __restrict__ cnt, const float* __restrict__ psum,
               const float* __restrict__ zsum, const int32_t* __restrict__ bad,
               int32_t* __restrict__ base, int32_t* __restrict__ total, double* __restrict__ pe,
               double* __restrict__ zs, int32_t* __restrict__ nbad) {
  __shared__ int64_t sc[kThreads];
  __shared__ double red[kThreads];
  __shared__ int64_t ired[kThreads];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  // a contiguous range of blocks per thread
  const int64_t per = (nb + kThreads - 1) / kThreads;
  const int64_t b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
  int64_t s = 0;
  double ps = 0.0;
#pragma unroll 8
  for (int64_t b = b0; b < b1; ++b) {
    s += cnt[b * E + e];
    if (psum) ps += (double)psum[b * E + e];
  }
  // inclusive scan of the per-thread sums (Hillis-Steele)
  sc[tid] = s;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int64_t v = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  int64_t run = sc[tid] - s;
#pragma unroll 8
  for (int64_t b = b0; b < b1; ++b) {
    base[b * E + e] = (int32_t)run;
    run += cnt[b * E + e];
  }
  if (tid == kThreads - 1) total[e] = (int32_t)sc[tid];
  const double P = block_sum_f64(ps, red);
  if (tid == 0) pe[e] = P;
  if (e == 0) {
    double z = 0.0;
    int64_t nbd = 0;
    for (int64_t b = tid; b < nb; b += kThreads) {
      if (zsum) z += (double)zsum[b];
      if (bad) nbd += bad[b];
    }
    z = block_sum_f64(z, red);
    nbd = block_sum_i64(nbd, ired);
    if (tid == 0) {
      *zs = z;
      *nbad = (int32_t)nbd;
    }
  }
}

struct ScatterArgs {
  const int32_t* idx;
  const float* topk_w;
  int64_t T;
  int k, E, BT;
  int64_t nb, cap;
  // per-block counts / partials from the router or the histogram
  const int32_t* cnt;
  const float* psum;
  const float* zsum;
  const int32_t* bad;
  // large tables: the colscan results
  const int32_t* base;
  const int32_t* total;
  const double* pe;
  const double* zs;
  const int32_t* nbad;
  // outputs
  int32_t* counts;
  int32_t* offsets;
  int32_t* n_dropped;
  moe_aux* aux;
  int32_t* perm_token;
  float* perm_w;
  int32_t* inv_row;
  const uint8_t* x;
  uint8_t* x_perm;
  int64_t row_bytes;
};

// Column sums of the count table (and of the probability sums when P) over
// the blocks g, g + G, ... for expert e: the total, the tokens of the blocks
// before each of the workgroup's blocks, and P_e's share.  Batches of
// kBatch unconditional loads (clamped rows, then a select) keep the requests
// in flight together.
template <bool P>
__device__ __forceinline__ void sum_blocks(const ScatterArgs& a, int e, int g, int G, int64_t rb0,
                                           int32_t& s_tot, int32_t (&s_pre)[kBlocksPerScatter],
                                           double& s_p) {
  const int E = a.E;
  for (int64_t b = g; b < a.nb; b += (int64_t)G * kBatch) {
    int32_t v[kBatch];
    float pv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t bb = b + (int64_t)u * G;
      const int64_t bc = bb < a.nb ? bb : a.nb - 1;
      v[u] = a.cnt[bc * E + e];
      if (P) pv[u] = a.psum[bc * E + e];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t bb = b + (int64_t)u * G;
      const bool in = bb < a.nb;
      const int32_t c = in ? v[u] : 0;
      s_tot += c;
      if (P) s_p += in ? (double)pv[u] : 0.0;
#pragma unroll
      for (int w = 0; w < kBlocksPerScatter; ++w) s_pre[w] += (bb < rb0 + w) ? c : 0;
    }
  }
}

template <bool SMALL>
__global__ void __launch_bounds__(kThreads)
scatter_kernel(ScatterArgs a) {
  __shared__ int32_t tot[kMaxExperts];                      // pre-capacity totals
  __shared__ int32_t bases[kBlocksPerScatter][kMaxExperts];  // rank base of each wave's block
  __shared__ int32_t offs[kMaxExperts + 1];
  __shared__ unsigned long long mask[kBlocksPerScatter][kMaxExperts];
  __shared__ double red[kThreads];
  __shared__ int64_t ired[kThreads];
  __shared__ double Pe[kMaxExperts];  // summary: P_e numerators (sum of block prob. sums)
  __shared__ int32_t part[1 + kBlocksPerScatter][kThreads];  // [total, bases][G][E] partials
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int E = a.E;
  // the last workgroup only writes counts, offsets, drops and the aux record;
  // the others scatter (nobody waits for the summary)
  const bool summary = blockIdx.x == gridDim.x - 1;
  const int64_t rb0 = (int64_t)blockIdx.x * kBlocksPerScatter;  // first routing block

  // this lane's token and its expert indices, loaded before anything else
  const int64_t rb = rb0 + wave;
  const int64_t t = rb * a.BT + lane;
  const bool valid = !summary && rb < a.nb && lane < a.BT && t < a.T;
  int32_t ev[kMaxKReg];
#pragma unroll
  for (int j = 0; j < kMaxKReg; ++j) ev[j] = (valid && j < a.k) ? a.idx[t * a.k + j] : -1;
  // the summary workgroup issues its other loads (per-block z sums and
  // invalid-logit flags, probability sums below) in the same round as the
  // count loads: one memory round trip instead of four
  // (unconditional loads from clamped addresses, masked where they are
  // used: a load under a per-lane condition is followed by a wait for it)
  constexpr int kSumReg = 4;
  const bool want_aux = summary && a.aux != nullptr;
  float zv[kSumReg] = {0.f, 0.f, 0.f, 0.f};
  int32_t bv[kSumReg] = {0, 0, 0, 0};
  if (SMALL && want_aux) {
#pragma unroll
    for (int u = 0; u < kSumReg; ++u) {
      const int64_t b = tid + (int64_t)u * kThreads;
      zv[u] = a.zsum[b < a.nb ? b : a.nb - 1];
    }
  }
  if (SMALL && summary && a.bad) {
#pragma unroll
    for (int u = 0; u < kSumReg; ++u) {
      const int64_t b = tid + (int64_t)u * kThreads;
      bv[u] = a.bad[b < a.nb ? b : a.nb - 1];
    }
  }

  // ---- totals and rank bases
  if (SMALL) {
    // G = 256 / E threads per expert (one when E > 256) sum interleaved
    // blocks in registers: the total and, for each of this workgroup's
    // blocks, the tokens of the blocks before it; partials meet in LDS in a
    // fixed order (integer sums, exact)
    const int G = E <= kThreads ? kThreads / E : 1;
    const int EW = E <= kThreads ? E : kThreads;  // experts per pass
    for (int e0 = 0; e0 < E; e0 += kThreads) {
      const int e = e0 + (E <= kThreads ? tid % E : tid);
      const int g = E <= kThreads ? tid / E : 0;
      int32_t s_tot = 0, s_pre[kBlocksPerScatter] = {0, 0, 0, 0};
      double s_p = 0.0;  // summary: this thread's share of P_e (interleaved blocks, in order)
      if (g < G && e < E) {
        if (want_aux)
          sum_blocks<true>(a, e, g, G, rb0, s_tot, s_pre, s_p);
        else
          sum_blocks<false>(a, e, g, G, rb0, s_tot, s_pre, s_p);
      }
      // all partials meet in LDS in one round: the total, this workgroup's
      // rank bases (not needed by the summary) and P_e (summary only)
      if (g < G && e < E) {
        const int slot = g * EW + (e - e0);
        part[0][slot] = s_tot;
        if (!summary) {
#pragma unroll
          for (int w = 0; w < kBlocksPerScatter; ++w) part[1 + w][slot] = s_pre[w];
        }
        if (want_aux) red[slot] = s_p;
      }
      __syncthreads();
      const int ne = min(EW, E - e0);
      const int rows = summary ? 1 : 1 + kBlocksPerScatter;
      for (int o = tid; o < (rows + (want_aux ? 1 : 0)) * ne; o += kThreads) {
        const int row = o / ne, c = o % ne;
        if (row < rows) {  // the G partials added in order (integers: exact anyway)
          int32_t sum = 0;
#pragma unroll 8
          for (int q = 0; q < G; ++q) sum += part[row][q * EW + c];
          if (row == 0)
            tot[e0 + c] = sum;
          else
            bases[row - 1][e0 + c] = sum;
        } else {  // P_e: the G partials added in order
          double P = 0.0;
#pragma unroll 8
          for (int q = 0; q < G; ++q) P += red[q * EW + c];
          Pe[e0 + c] = P;
        }
      }
      __syncthreads();
      if (E <= kThreads) break;
    }
  } else {
    for (int e = tid; e < E; e += kThreads) {
      tot[e] = a.total[e];
      for (int w = 0; w < kBlocksPerScatter; ++w) {
        const int64_t b = rb0 + w;
        bases[w][e] = b < a.nb ? a.base[b * E + e] : 0;
      }
    }
  }
  for (int w = 0; w < kBlocksPerScatter; ++w)
    for (int e = tid; e < E; e += kThreads) mask[w][e] = 0ull;
  __syncthreads();

  // ---- kept counts and their exclusive scan (offsets): wave 0 scans 64
  // experts at a time with lane shuffles and carries the running total
  if (wave == 0) {
    int32_t carry = 0;
    for (int c0 = 0; c0 < E; c0 += kWave) {
      const int e = c0 + lane;
      int32_t v = 0;
      if (e < E) {
        const int64_t te = tot[e];
        v = (int32_t)((a.cap < 0 || te < a.cap) ? te : a.cap);
      }
      for (int o = 1; o < kWave; o <<= 1) {
        const int32_t n = __shfl_up(v, o);
        if (lane >= o) v += n;
      }
      if (e < E) offs[e + 1] = carry + v;
      carry += __shfl(v, kWave - 1);
    }
    if (lane == 0) offs[0] = 0;
  }
  __syncthreads();

  // ---- summary workgroup: counts, offsets, drops, aux
  if (summary) {
    int64_t my_drop = 0, my_bad = 0;
    for (int e = tid; e < E; e += kThreads) {
      a.counts[e] = tot[e];
      a.offsets[e] = offs[e];
      my_drop += tot[e] - (offs[e + 1] - offs[e]);
    }
    if (tid == 0) a.offsets[E] = offs[E];
    if (SMALL) {
#pragma unroll
      for (int u = 0; u < kSumReg; ++u) my_bad += tid + (int64_t)u * kThreads < a.nb ? bv[u] : 0;
      if (a.bad)
        for (int64_t b = tid + (int64_t)kSumReg * kThreads; b < a.nb; b += kThreads) my_bad += a.bad[b];
    }
    // lb = E * sum_e f_e P_e with f_e = total_e / (T k), P_e = sum_t p / T
    double lbp = 0.0, zp = 0.0, sqp = 0.0, lgp = 0.0, fqp = 0.0;
    if (a.aux) {
      if (SMALL) {
        // P_e was summed with the counts: G = 256 / E threads per expert
        // over interleaved blocks, the G partials added in order (E > 256:
        // one thread per expert, blocks in order)
        for (int e = tid; e < E; e += kThreads) {
          const double fe = (double)tot[e] / (double)(a.T * a.k), P = Pe[e] / (double)a.T;
          lbp += fe * P;
          lb_form_terms(fe, P, E, sqp, lgp, fqp);
        }
#pragma unroll
        for (int u = 0; u < kSumReg; ++u)
          zp += tid + (int64_t)u * kThreads < a.nb ? (double)zv[u] : 0.0;
        for (int64_t b = tid + (int64_t)kSumReg * kThreads; b < a.nb; b += kThreads)
          zp += (double)a.zsum[b];
      } else {
        for (int e = tid; e < E; e += kThreads) {
          const double fe = (double)tot[e] / (double)(a.T * a.k), P = a.pe[e] / (double)a.T;
          lbp += fe * P;
          lb_form_terms(fe, P, E, sqp, lgp, fqp);
        }
      }
    }
    block_sum4(my_drop, my_bad, lbp, zp, ired, red);
    if (a.aux) block_sum3(sqp, lgp, fqp, red);
    const int64_t dropped = my_drop;
    const int64_t nbd = SMALL ? my_bad : (int64_t)*a.nbad;
    if (tid == 0) a.n_dropped[0] = nbd ? -1 : (int32_t)dropped;
    if (a.aux && tid == 0) {
      const double z = (SMALL ? zp : *a.zs) / (double)a.T;
      write_lb_forms(a.aux, E, lbp, z, sqp, lgp, fqp);
      a.aux->n_dropped = dropped;
      a.aux->capacity = a.cap;
      a.aux->n_kept = a.T * a.k - dropped;
    }
  }

  if (summary) return;

  // ---- ranks and scatter: wave w owns routing block rb0 + w, lane = token
  // (the first kMaxKReg indices come from registers: constant indices only)
  if (valid) {
#pragma unroll
    for (int j = 0; j < kMaxKReg; ++j)
      if (j < a.k && ev[j] >= 0 && ev[j] < E) atomicOr(&mask[wave][ev[j]], 1ull << lane);
    for (int j = kMaxKReg; j < a.k; ++j) {
      const int e = a.idx[t * a.k + j];
      if (e >= 0 && e < E) atomicOr(&mask[wave][e], 1ull << lane);
    }
  }
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (valid) {
#pragma unroll
    for (int j = 0; j < kMaxKReg; ++j) {
      if (j >= a.k) break;
      const int e = ev[j];
      int32_t row = -1;
      if (e >= 0 && e < E) {
        const int64_t rank = (int64_t)bases[wave][e] + __popcll(mask[wave][e] & below);
        if (a.cap < 0 || rank < a.cap) {
          row = offs[e] + (int32_t)rank;
          a.perm_token[row] = (int32_t)t;
          if (a.perm_w) a.perm_w[row] = a.topk_w[t * a.k + j];
        }
      }
      a.inv_row[t * a.k + j] = row;
    }
    for (int j = kMaxKReg; j < a.k; ++j) {
      const int e = a.idx[t * a.k + j];
      int32_t row = -1;
      if (e >= 0 && e < E) {
        const int64_t rank = (int64_t)bases[wave][e] + __popcll(mask[wave][e] & below);
        if (a.cap < 0 || rank < a.cap) {
          row = offs[e] + (int32_t)rank;
          a.perm_token[row] = (int32_t)t;
          if (a.perm_w) a.perm_w[row] = a.topk_w[t * a.k + j];
        }
      }
      a.inv_row[t * a.k + j] = row;
    }
  }
  if (a.x_perm == nullptr) return;
  __syncthreads();  // inv_row of every lane is visible below
  // optional gather x_perm[row] = x[t]: each wave copies its block's rows
  for (int r = 0; r < a.BT; ++r) {
    const int64_t tt = rb * a.BT + r;
    if (rb >= a.nb || tt >= a.T) break;
    for (int j = 0; j < a.k; ++j) {
      const int32_t row = a.inv_row[tt * a.k + j];
      if (row < 0) continue;
      const uint4* src = reinterpret_cast<const uint4*>(a.x + tt * a.row_bytes);
      uint4* dst = reinterpret_cast<uint4*>(a.x_perm + (int64_t)row * a.row_bytes);
      for (int64_t c = lane; c < a.row_bytes / 16; c += kWave) dst[c] = src[c];
    }
  }
}

// moe_aux_stats on its own: counts and drops given, partials from the router.
__global__ void __launch_bounds__(kThreads)
aux_kernel(int64_t T, int k, int E, int64_t nb, int64_t cap, const float* __restrict__ psum,
           const float* __restrict__ zsum, const int32_t* __restrict__ counts,
           const int32_t* __restrict__ n_dropped, moe_aux* __restrict__ aux) {
  __shared__ double red[kThreads];
  double lbp = 0.0, zp = 0.0, sqp = 0.0, lgp = 0.0, fqp = 0.0;
  for (int e = threadIdx.x; e < E; e += kThreads) {
    double P = 0.0;
    for (int64_t b = 0; b < nb; ++b) P += (double)psum[b * E + e];
    const double fe = (double)counts[e] / (double)(T * k);
    P /= (double)T;
    lbp += fe * P;
    lb_form_terms(fe, P, E, sqp, lgp, fqp);
  }
  for (int64_t b = threadIdx.x; b < nb; b += kThreads) zp += (double)zsum[b];
  const double lbs = block_sum_f64(lbp, red);
  const double z = block_sum_f64(zp, red) / (double)T;
  block_sum3(sqp, lgp, fqp, red);
  if (threadIdx.x == 0) {
    const int64_t dropped = n_dropped[0];
    write_lb_forms(aux, E, lbs, z, sqp, lgp, fqp);
    aux->n_dropped = dropped;
    aux->capacity = cap;
    aux->n_kept = T * k - dropped;
  }
}

}  // namespace

size_t permute_scratch_bytes(const moe_config& c) {
  const int BT = route_block_tokens(c.n_tokens, c.n_experts);
  const int64_t nb = (c.n_tokens + BT - 1) / BT;
  if (nb * c.n_experts <= kSmallTable) return 0;
  // base [nb*E] i32, total [E] i32, pe [E] f64, zs f64 + nbad i32, each 256-aligned
  return ((size_t)nb * c.n_experts * 4 + 255) / 256 * 256 + ((size_t)c.n_experts * 4 + 255) / 256 * 256 +
         ((size_t)c.n_experts * 8 + 255) / 256 * 256 + 256;
}

hipError_t launch_histogram(const moe_config& c, const int32_t* topk_idx, const RouteStats& st,
                            hipStream_t s) {
  const int BT = route_block_tokens(c.n_tokens, c.n_experts);
  const int64_t nb = (c.n_tokens + BT - 1) / BT;
  histogram_kernel<<<dim3((unsigned)nb), dim3(64), 0, s>>>(topk_idx, c.n_tokens, c.top_k,
                                                           c.n_experts, BT, st.cnt, st.bad);
  return hipGetLastError();
}

hipError_t launch_permute(const moe_config& c, const RouteStats& st, const PermuteOut& po,
                          int64_t capacity, const int32_t* topk_idx, const float* topk_w,
                          const void* x, void* x_perm, moe_aux* aux, void* scratch, hipStream_t s) {
  const int BT = route_block_tokens(c.n_tokens, c.n_experts);
  const int64_t nb = (c.n_tokens + BT - 1) / BT;
  const int E = c.n_experts;
  ScatterArgs a{};
  a.idx = topk_idx;
  a.topk_w = topk_w;
  a.T = c.n_tokens;
  a.k = c.top_k;
  a.E = E;
  a.BT = BT;
  a.nb = nb;
  a.cap = capacity;
  a.cnt = st.cnt;
  a.psum = st.psum;
  a.zsum = st.zsum;
  a.bad = st.bad;
  a.counts = po.counts;
  a.offsets = po.offsets;
  a.n_dropped = po.n_dropped;
  a.aux = aux;
  a.perm_token = po.perm_token;
  a.perm_w = po.perm_w;
  a.inv_row = po.inv_row;
  a.x = static_cast<const uint8_t*>(x);
  a.x_perm = static_cast<uint8_t*>(x_perm);
  a.row_bytes = (int64_t)c.d_model * (c.dtype == MOE_DTYPE_BF16 ? 2 : 4);
  // scatter workgroups plus one summary workgroup
  const int64_t grid = (nb + kBlocksPerScatter - 1) / kBlocksPerScatter + 1;
  if (nb * E <= kSmallTable) {
    scatter_kernel<true><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
  }
  // large tables: carve the colscan results out of the scratch area
  char* p = static_cast<char*>(scratch);
  int32_t* base = reinterpret_cast<int32_t*>(p);
  p += ((size_t)nb * E * 4 + 255) / 256 * 256;
  int32_t* total = reinterpret_cast<int32_t*>(p);
  p += ((size_t)E * 4 + 255) / 256 * 256;
  double* pe = reinterpret_cast<double*>(p);
  p += ((size_t)E * 8 + 255) / 256 * 256;
  double* zs = reinterpret_cast<double*>(p);
  int32_t* nbad = reinterpret_cast<int32_t*>(p + 8);
  colscan_kernel<<<dim3(E), dim3(kThreads), 0, s>>>(nb, E, st.cnt, aux ? st.psum : nullptr,
                                                   aux ? st.zsum : nullptr, st.bad, base, total,
                                                   pe, zs, nbad);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  a.base = base;
  a.total = total;
  a.pe = pe;
  a.zs = zs;
  a.nbad = nbad;
  scatter_kernel<false><<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_aux(const moe_config& c, const RouteStats& st, const int32_t* counts,
                      const int32_t* n_dropped, int64_t capacity, moe_aux* aux, hipStream_t s) {
  const int BT = route_block_tokens(c.n_tokens, c.n_experts);
  const int64_t nb = (c.n_tokens + BT - 1) / BT;
  aux_kernel<<<dim3(1), dim3(kThreads), 0, s>>>(c.n_tokens, c.top_k, c.n_experts, nb, capacity,
                                               st.psum, st.zsum, counts, n_dropped, aux);
  return hipGetLastError();
}

}  // namespace moe

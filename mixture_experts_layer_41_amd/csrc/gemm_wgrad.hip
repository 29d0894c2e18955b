// Weight-gradient GEMM of the backward pass:
//   C_b[m, n] = sum_{k in [k0_b, k1_b)} A_b[m, k] * B_b[n, k]     (float32 out)
// for batches b (one per expert, or per shared expert), with A_b = a +
// b * a_batch, B_b = b + b * b_batch, rows of length lda / ldb (K
// contiguous), and the K range of batch b from kofs[b], kofs[b + 1] (the
// padded column offsets of the transposed activations; every range is a
// multiple of the K tile and the padding is zero) or [0, K) for all.
//
// dW2_e = d_o_e^T h_e and dW1_e = da_e^T x_e take their operands from the
// transposed activations, so both operands are read along K like the
// forward's grouped GEMMs: 128 x 128 x 64 tiles over 4 waves, or, for long K
// and enough output tiles, 256 x 256 x 64 tiles over 8 waves (half the bytes
// per flop); each wave holds 64 x 64 or 128 x 64 of the tile in
// v_mfma_f32_32x32x16_bf16 accumulators.  Global loads of K tile t+1 are
// staged in registers while tile t feeds the MFMAs from LDS; 16-byte LDS
// chunks are XOR-swizzled so the 16 lanes of a fragment read hit distinct
// bank groups.  Rows past M or N are clamped on load and masked on store.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BK = 64;
constexpr int CPR = BK / 8;               // 16-byte chunks per tile row
constexpr int RPW = 256 / (BK * 2);       // tile rows per 256-byte bank window
constexpr int KS = BK / 16;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct WgradArgs {
  const uint16_t* a;
  int64_t lda, a_batch;
  const uint16_t* b;
  int64_t ldb, b_batch;
  const int32_t* kofs;
  int64_t K;
  int M, N;
  float* c;
  int64_t ldc, c_batch;
  int nsplit;       // K splits per batch: blockIdx.z = batch * nsplit + split
  int64_t c_split;  // output offset of split s: s * c_split
};

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN, BM * BN > 128 * 128 ? 1 : 2)
wgrad_kernel(WgradArgs p) {
  constexpr int kThreads = 64 * WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN, MI = TM / 32, NI = TN / 32;
  constexpr int A_LD = BM * CPR / kThreads;
  constexpr int B_LD = BN * CPR / kThreads;
  __shared__ __attribute__((aligned(16))) u32x4 sA[2][BM * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sB[2][BN * CPR];
  const int bt = blockIdx.z / p.nsplit, sp = blockIdx.z % p.nsplit;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  // this split's share of the batch's K range (whole K tiles)
  const int64_t kb0 = p.kofs ? p.kofs[bt] : 0;
  const int64_t kb1 = p.kofs ? p.kofs[bt + 1] : p.K;
  const int64_t chunk = ((kb1 - kb0 + p.nsplit - 1) / p.nsplit + BK - 1) / BK * BK;
  const int64_t k0 = kb0 + sp * chunk < kb1 ? kb0 + sp * chunk : kb1;
  const int64_t k1 = k0 + chunk < kb1 ? k0 + chunk : kb1;
  const int nk = (int)((k1 - k0) / BK);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / WN, wn = wave % WN;

  const uint16_t* A = p.a + (int64_t)bt * p.a_batch;
  const uint16_t* B = p.b + (int64_t)bt * p.b_batch;
  const uint16_t* aptr[A_LD];
  const uint16_t* bptr[B_LD];
  int aoff[A_LD], boff[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int c = tid + kThreads * i, r = c / CPR, ch = c % CPR;
    const int m = min(m0 + r, p.M - 1);
    aptr[i] = A + (int64_t)m * p.lda + k0 + ch * 8;
    aoff[i] = r * CPR + (ch ^ ((r / RPW) % CPR));
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int c = tid + kThreads * i, r = c / CPR, ch = c % CPR;
    const int n = min(n0 + r, p.N - 1);
    bptr[i] = B + (int64_t)n * p.ldb + k0 + ch * 8;
    boff[i] = r * CPR + (ch ^ ((r / RPW) % CPR));
  }
  u32x4 ra[A_LD], rb[B_LD];
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *reinterpret_cast<const u32x4*>(aptr[i] + (int64_t)kt * BK);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bptr[i] + (int64_t)kt * BK);
  };
  auto store = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) sA[st][aoff[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) sB[st][boff[i]] = rb[i];
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int fr = lane % 32, half = lane / 32;
  int arow[MI], brow[NI];
#pragma unroll
  for (int i = 0; i < MI; ++i) arow[i] = (wm * TM + i * 32 + fr) * CPR;
#pragma unroll
  for (int j = 0; j < NI; ++j) brow[j] = (wn * TN + j * 32 + fr) * CPR;
  const int sw = (fr / RPW) % CPR;

  if (nk > 0) {
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      if (kt + 1 < nk) load(kt + 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // lanes of half h take the K elements [h*BK/2, (h+1)*BK/2) of the
        // tile, one chunk per step; A and B use the same order
        const int c = (half * KS + ks) ^ sw;
        bf16x8 fa[MI], fb[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = __builtin_bit_cast(bf16x8, sA[st][arow[i] + c]);
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[j] = __builtin_bit_cast(bf16x8, sB[st][brow[j] + c]);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store(st ^ 1);
      __syncthreads();
    }
  }

  // 32x32 C layout: column lane%32, rows 8*(q/4) + 4*(lane/32) + q%4
  float* C = p.c + (int64_t)sp * p.c_split + (int64_t)bt * p.c_batch;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = m0 + wm * TM + i * 32 + 8 * (q / 4) + 4 * half + (q % 4);
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int n = n0 + wn * TN + j * 32 + fr;
        if (n < p.N) C[(int64_t)m * p.ldc + n] = acc[i][j][q];
      }
    }
}

// out[i] = sum over the splits s of part[s * n + i], in split order
__global__ void __launch_bounds__(256)
wgrad_reduce_kernel(const float* __restrict__ part, int nsplit, int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = part[i];
  int s = 1;
  for (; s + 4 <= nsplit; s += 4) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = part[(int64_t)(s + u) * n + i];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += v[u];
  }
  for (; s < nsplit; ++s) acc += part[(int64_t)s * n + i];
  out[i] = acc;
}

}  // namespace

// Tile and K split of a weight-gradient product, from a cost model in units
// of one K tile of a 128 x 128 tile pair on a CU: a round of resident
// workgroups (256 tiles of 256 x 256, one per CU, or 512 of 128 x 128, two
// per CU) costs its K tiles per split, times 1.5 for the large tile (it does
// twice the work of a pair at the higher efficiency measured for it).
// A split product also writes and reads back its float32 partials (one such
// unit moves about 8.5 MB at HBM rate).  The large tile needs batches of 512
// K rows on average; splits keep at least 512 K rows each, at most 64; the
// fewest splits win a tie.
WgradPlan wgrad_plan(int M, int N, int batches, int64_t k_avg) {
  WgradPlan best{128, 1};
  if (M <= 0 || N <= 0 || batches <= 0 || k_avg <= 0) return best;
  double best_cost = 1e300;
  for (const int tile : {256, 128}) {
    const int64_t t = (int64_t)((M + tile - 1) / tile) * ((N + tile - 1) / tile) * batches;
    const int64_t slots = tile == 256 ? 256 : 512;
    const int64_t min_rows = 512;
    if (k_avg < min_rows && tile == 256) continue;
    const int64_t ns_max = std::max<int64_t>(1, std::min<int64_t>(k_avg / min_rows, 64));
    for (int64_t ns = 1; ns <= ns_max; ++ns) {
      const int64_t rounds = (t * ns + slots - 1) / slots;
      const int64_t ksteps = ((k_avg + ns - 1) / ns + BK - 1) / BK;
      const double partial_bytes = ns > 1 ? 8.0 * (double)ns * batches * M * N : 0.0;
      const double cost =
          (double)rounds * (double)ksteps * (tile == 256 ? 1.5 : 1.0) + partial_bytes / 8.5e6;
      if (cost < best_cost) {
        best_cost = cost;
        best = WgradPlan{tile, (int)ns};
      }
    }
  }
  return best;
}

size_t wgrad_partial_floats(const WgradPlan& w, int M, int N, int batches) {
  return w.nsplit > 1 ? (size_t)w.nsplit * batches * M * N : 0;
}

hipError_t launch_wgrad(const void* a, int64_t lda, int64_t a_batch, const void* b, int64_t ldb,
                        int64_t b_batch, const int32_t* kofs, int64_t K, int M, int N, int batches,
                        float* c, int64_t ldc, int64_t c_batch, float* partial, hipStream_t s) {
  if (M <= 0 || N <= 0 || batches <= 0) return hipSuccess;
  if (lda % 8 != 0 || ldb % 8 != 0 || K < 0 || (!kofs && K % BK != 0))
    return hipErrorInvalidValue;
  const WgradPlan w = wgrad_plan(M, N, batches, kofs ? K / batches : K);
  WgradArgs p;
  p.a = static_cast<const uint16_t*>(a);
  p.lda = lda;
  p.a_batch = a_batch;
  p.b = static_cast<const uint16_t*>(b);
  p.ldb = ldb;
  p.b_batch = b_batch;
  p.kofs = kofs;
  p.K = K;
  p.M = M;
  p.N = N;
  p.nsplit = w.nsplit;
  const int64_t n = (int64_t)batches * M * N;
  if (w.nsplit > 1) {
    // partials [nsplit][batches][M][N], summed into c (which must be dense)
    if (partial == nullptr || ldc != N || c_batch != (int64_t)M * N) return hipErrorInvalidValue;
    p.c = partial;
    p.ldc = N;
    p.c_batch = (int64_t)M * N;
    p.c_split = n;
  } else {
    p.c = c;
    p.ldc = ldc;
    p.c_batch = c_batch;
    p.c_split = 0;
  }
  const unsigned z = (unsigned)(batches * w.nsplit);
  if (w.tile == 256) {
    const dim3 grid((unsigned)((N + 255) / 256), (unsigned)((M + 255) / 256), z);
    wgrad_kernel<256, 256, 2, 4><<<grid, 512, 0, s>>>(p);
  } else {
    const dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128), z);
    wgrad_kernel<128, 128, 2, 2><<<grid, 256, 0, s>>>(p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || w.nsplit == 1) return e;
  wgrad_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(partial, w.nsplit, n, c);
  return hipGetLastError();
}

}  // namespace moe

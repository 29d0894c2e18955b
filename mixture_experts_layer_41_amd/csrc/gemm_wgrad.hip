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
// forward's grouped GEMMs: 128 x 128 x 64 tiles over 4 waves (64 x 64 each,
// v_mfma_f32_32x32x16_bf16), global loads of K tile t+1 staged in registers
// while tile t feeds the MFMAs from LDS, 16-byte LDS chunks XOR-swizzled so
// the 16 lanes of a fragment read hit distinct bank groups.  Rows past M or
// N are clamped on load and masked on store.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, WM = 2, WN = 2;
constexpr int kThreads = 64 * WM * WN;
constexpr int TM = BM / WM, TN = BN / WN, MI = TM / 32, NI = TN / 32;
constexpr int CPR = BK / 8;               // 16-byte chunks per tile row
constexpr int RPW = 256 / (BK * 2);       // tile rows per 256-byte bank window
constexpr int A_LD = BM * CPR / kThreads;
constexpr int B_LD = BN * CPR / kThreads;
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
};

__global__ void __launch_bounds__(kThreads, 2) wgrad_kernel(WgradArgs p) {
  __shared__ __attribute__((aligned(16))) u32x4 sA[2][BM * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sB[2][BN * CPR];
  const int bt = blockIdx.z;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int64_t k0 = p.kofs ? p.kofs[bt] : 0;
  const int64_t k1 = p.kofs ? p.kofs[bt + 1] : p.K;
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
  float* C = p.c + (int64_t)bt * p.c_batch;
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

}  // namespace

hipError_t launch_wgrad(const void* a, int64_t lda, int64_t a_batch, const void* b, int64_t ldb,
                        int64_t b_batch, const int32_t* kofs, int64_t K, int M, int N, int batches,
                        float* c, int64_t ldc, int64_t c_batch, hipStream_t s) {
  if (M <= 0 || N <= 0 || batches <= 0) return hipSuccess;
  if (lda % 8 != 0 || ldb % 8 != 0 || (!kofs && K % BK != 0)) return hipErrorInvalidValue;
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
  p.c = c;
  p.ldc = ldc;
  p.c_batch = c_batch;
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM), (unsigned)batches);
  wgrad_kernel<<<grid, kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe

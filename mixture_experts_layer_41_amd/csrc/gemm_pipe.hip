// Pipelined persistent grouped GEMM for bf16 on gfx950.
//
// Same operation as the other grouped GEMM kernels (expert FFN up GEMM with
// the SwiGLU / GELU epilogue; down GEMM summing the shared-expert segments
// along K), built for long runs of tiles:
//   * K advances 32 elements per stage; NS = 4 LDS stages rotate (8 in the
//     deep variant, for few tiles with long K).  The
//     global -> LDS copies use the direct-to-LDS load (global_load_lds,
//     16 bytes per lane), so no registers stage the data, and each stage
//     lives in its own __shared__ array, which lets the compiler see that
//     reading stage s does not depend on the copies into the other stages
//     (it then waits only for what it needs);
//   * the grid holds only resident workgroups; each walks a contiguous run of
//     its XCD's share of the tile list, and the copies for the first stages
//     of its next tile are issued while the current tile finishes, so the
//     epilogue and the next tile's first loads overlap;
//   * the MFMA takes the weight fragment as its first operand, so each lane
//     ends up with 4 consecutive output columns of one row; the output tile
//     then leaves through LDS as 16-byte stores of whole rows (the training
//     forward's SwiGLU variant stores from the registers, lane pairs joined);
//   * LDS rows (64 bytes) are XOR-swizzled in 16-byte chunks on the global
//     side of the copy: chunk' = chunk ^ ((row / 4) % 4).  A fragment read
//     (16 lanes, 16 consecutive rows, one chunk each) then touches 16
//     distinct 16-byte bank groups of the 256-byte bank window.
// Requirements (checked by the host): K per segment a multiple of 32 and the
// total K steps a multiple of NS; output widths a multiple of the tile.
#include <algorithm>

#include "moe_internal.h"
#include "gemm_common.h"

namespace moe {
namespace pipe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

constexpr int BK = 32;              // K elements per stage
constexpr int NS = 4;               // LDS stages (default; the deep variant uses 8)
constexpr int CPR = BK / 8;         // 16-byte chunks per tile row
constexpr int KS = BK / 16;         // MFMA K steps per stage
static_assert(CPR == 4, "the swizzle below assumes 64-byte rows");

// 16 bytes per lane from global memory straight into LDS; lane i of the wave
// lands at lds + 16 * i (lds is wave-uniform).
__device__ __forceinline__ void copy16(const void* g, u32x4* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// 4 bytes per lane into LDS; lane i lands at lds + 4 * i.
__device__ __forceinline__ void copy4(const void* g, int* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read(const u32x4* __restrict__ p, int i) { return p[i]; }
// LDS read of a gather index.  Written as one asm block (read and its wait
// together) so that the compiler does not tie it to the outstanding copies:
// the callers order it after the copy of the index with explicit waits.
__device__ __forceinline__ int lds_read_i32(const int* p, int i) {
  int v;
  const uint32_t addr = (uint32_t)(uintptr_t)(p + i);
  __asm__ volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// Workgroup barrier without a memory fence (the fence would also wait for
// every outstanding global load); the empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(N) lgkmcnt(0): also every LDS read of this wave has landed.
// The asm statement keeps LDS reads issued before it from being moved past
// the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}

template <int BM, int BN, int WM, int WN>
struct Shape {
  static constexpr int NW = WM * WN;
  static constexpr int NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int MI = TM / 32, NI = TN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int A_IW = BM / (16 * NW);       // copies per wave per stage (A)
  static constexpr int B_IW = BN / (16 * NW);       // (B)
  static constexpr int LPS = A_IW + B_IW;           // copies per lane per stage
  static_assert(MI >= 1 && NI >= 1 && A_IW >= 1 && B_IW >= 1, "tile shape");
  static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "tile shape");
};

// Per-lane source rows of one tile's copies, at K = 0 (the swizzled chunk
// included).
template <int A_IW, int B_IW>
struct TileSrc {
  const uint16_t* a[A_IW];
  const uint16_t* b[B_IW];
};

// PAIRED (SwiGLU up GEMM that also stores the pre-activations): the
// epilogue pairs lanes l and l ^ 32, which hold the two 4-column halves of
// each 8-column run of a row, so that every store is 16 bytes.  A separate
// instantiation, so the inference kernel keeps its registers.
template <int BM, int BN, int WM, int WN, int KIND, int ACT, bool BIAS, int NSt, bool PAIRED>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_pipe_kernel(GemmDesc p, int tiles_n) {
  constexpr int NS = NSt;  // LDS stages: 4, or 8 for the deep variant
  static_assert(NS == 4 || NS == 8, "stages");
  using Sh = Shape<BM, BN, WM, WN>;
  constexpr int NT = Sh::NT, TM = Sh::TM, TN = Sh::TN, MI = Sh::MI, NI = Sh::NI;
  constexpr int A_IW = Sh::A_IW, B_IW = Sh::B_IW, LPS = Sh::LPS;
  constexpr int RW = 16 * A_IW;  // A rows copied by one wave (a contiguous block)
  static_assert(RW <= kWave, "one gather-index copy per wave");
  constexpr bool kSwiglu = (KIND == kGemmUp && ACT == MOE_ACT_SWIGLU);
  static_assert(!kSwiglu || (NI % 2 == 0), "SwiGLU pairs gate and up blocks");
  static_assert((NS - 3) * LPS < 64, "vmcnt range");
  constexpr int XS = NS > 4 ? 1 : 0;  // the deep variant's extra stages

  __shared__ __attribute__((aligned(16))) u32x4 sA0[BM * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sA1[BM * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sA2[BM * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sA3[BM * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sB0[BN * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sB1[BN * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sB2[BN * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sB3[BN * CPR];
  __shared__ __attribute__((aligned(16))) u32x4 sA4[XS * BM * CPR + 1], sA5[XS * BM * CPR + 1];
  __shared__ float s_bias[BIAS ? BN : 1];   // bias of the current tile's output columns
  __shared__ __attribute__((aligned(16))) u32x4 sA6[XS * BM * CPR + 1], sA7[XS * BM * CPR + 1];
  __shared__ __attribute__((aligned(16))) u32x4 sB4[XS * BN * CPR + 1], sB5[XS * BN * CPR + 1];
  __shared__ __attribute__((aligned(16))) u32x4 sB6[XS * BN * CPR + 1], sB7[XS * BN * CPR + 1];
  __shared__ int s_idx[3][BM];               // gather indices of three consecutive tiles
  __shared__ int s_off[kMaxExperts + 1];     // group row offsets
  __shared__ int s_tstart[kMaxExperts + 1];  // first row tile of each group
  __shared__ int s_scan[kMaxExperts + 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;

  // ---- row-tile table of the groups (exact, from the device offsets)
  const int G = p.group_off ? p.n_groups : 1;
  for (int g = tid; g <= G; g += NT)
    s_off[g] = p.group_off ? p.group_off[g] : (g == 0 ? 0 : (int)p.rows_max);
  __syncthreads();
  for (int g = tid; g <= G; g += NT) {
    const int rows = g < G ? min(s_off[g + 1], (int)p.rows_max) - min(s_off[g], (int)p.rows_max) : 0;
    s_tstart[g] = rows > 0 ? (rows + BM - 1) / BM : 0;
  }
  __syncthreads();
  for (int o = 1; o <= G; o <<= 1) {  // inclusive scan over g = 0..G
    for (int g = tid; g <= G; g += NT) s_scan[g] = g >= o ? s_tstart[g - o] : 0;
    __syncthreads();
    for (int g = tid; g <= G; g += NT) s_tstart[g] += s_scan[g];
    __syncthreads();
  }
  const int m_tiles = s_tstart[G - 1];
  for (int g = tid; g <= G; g += NT) s_scan[g] = g == 0 ? 0 : s_tstart[g - 1];
  __syncthreads();
  for (int g = tid; g <= G; g += NT) s_tstart[g] = s_scan[g];
  __syncthreads();

  // ---- this workgroup's tiles: XCD x = blockIdx % 8 owns the x-th eighth of
  // the tile list; its workgroups stride through it
  const int total = m_tiles * tiles_n;
  const int xcd = blockIdx.x % 8, per_xcd = gridDim.x / 8;
  const int t_lo = (int)((int64_t)total * xcd / 8), t_hi = (int)((int64_t)total * (xcd + 1) / 8);
  int L = t_lo + (int)(blockIdx.x / 8);
  if (L >= t_hi) return;

  const int S = p.n_seg, d = p.d, f = p.f;
  const bool gather = p.a_rows != nullptr;
  const uint16_t* A = static_cast<const uint16_t*>(p.a);
  const uint16_t* W = static_cast<const uint16_t*>(p.w);
  const int nk_seg = ((KIND == kGemmUp) ? d : f) / BK;     // K stages per FFN segment
  const int nk = (KIND == kGemmUp) ? nk_seg : S * nk_seg;  // K stages per tile

  // copy geometry: copy i of wave w covers tile rows w*RW + i*16 + lane/4 at
  // LDS chunk lane%4, which holds the global chunk (lane%4) ^ ((row/4)%4) =
  // (lane%4) ^ ((lane/16)%4)
  const int lrow = lane / 4;
  const int chk = ((lane % 4) ^ ((lane / 16) % 4)) * 8;

  struct Tile {
    int group, rows, seg, n0;
    int64_t row0;
  };
  auto tile_of = [&](int l) {
    Tile t;
    const int mt = l / tiles_n, nt = l % tiles_n;
    int glo = 0, ghi = G - 1;  // last g with s_tstart[g] <= mt
    while (glo < ghi) {
      const int mid = (glo + ghi + 1) / 2;
      if (s_tstart[mid] <= mt) glo = mid; else ghi = mid - 1;
    }
    t.group = glo;
    t.row0 = (int64_t)s_off[glo] + (int64_t)(mt - s_tstart[glo]) * BM;
    t.rows = min(BM, min(s_off[glo + 1], (int)p.rows_max) - (int)t.row0);
    if (KIND == kGemmUp) {
      constexpr int bnh = kSwiglu ? BN / 2 : BN;
      const int tpn = f / bnh;
      t.seg = nt / tpn;
      t.n0 = (nt % tpn) * bnh;
    } else {
      t.seg = 0;
      t.n0 = nt * BN;
    }
    return t;
  };

  // gather indices of this wave's rows of tile t_ -> s_idx[buf_] (one 4-byte
  // copy per lane; rows past the tile end repeat its last row)
#define MOE_PIPE_IDX(t_, buf_)                                                              \
  do {                                                                                      \
    if (lane < RW) {                                                                        \
      const int r_ = wave * RW + lane;                                                      \
      const int64_t gr_ = (t_).row0 + (r_ < (t_).rows ? r_ : (t_).rows - 1);               \
      copy4(p.a_rows + gr_, &s_idx[buf_][wave * RW]);                                       \
    }                                                                                       \
  } while (0)
  // source rows of this lane's copies for tile t_ (gather indices in s_idx[buf_])
#define MOE_PIPE_SRC(src_, t_, buf_)                                                        \
  do {                                                                                      \
    _Pragma("unroll") for (int i_ = 0; i_ < A_IW; ++i_) {                                  \
      const int r_ = wave * RW + i_ * 16 + lrow;                                            \
      const int64_t row_ = gather ? (int64_t)lds_read_i32(s_idx[buf_], r_)                  \
                                  : (t_).row0 + (r_ < (t_).rows ? r_ : (t_).rows - 1);      \
      (src_).a[i_] = A + row_ * p.lda + chk;                                                \
    }                                                                                       \
    const int rows1_ = (KIND == kGemmUp) ? (kSwiglu ? 2 * f : f) : d;                      \
    const int kw_ = (KIND == kGemmUp) ? d : f;                                              \
    const uint16_t* wb_ = W + ((int64_t)(t_).group * S + (t_).seg) * rows1_ * (int64_t)kw_; \
    _Pragma("unroll") for (int i_ = 0; i_ < B_IW; ++i_) {                                  \
      const int r_ = (wave * B_IW + i_) * 16 + lrow;                                        \
      int wr_;                                                                              \
      if (kSwiglu)                                                                          \
        wr_ = (r_ < BN / 2) ? (t_).n0 + r_ : f + (t_).n0 + (r_ - BN / 2);                   \
      else                                                                                  \
        wr_ = (t_).n0 + r_;                                                                 \
      (src_).b[i_] = wb_ + (int64_t)wr_ * kw_ + chk;                                        \
    }                                                                                       \
  } while (0)
  // copies of K stage kt_ of the tile with sources src_ into LDS stage (sa_, sb_)
#define MOE_PIPE_LOAD(src_, kt_, sa_, sb_)                                                  \
  do {                                                                                      \
    int64_t ao_, bo_;                                                                       \
    if (KIND == kGemmUp) {                                                                  \
      ao_ = (int64_t)(kt_) * BK;                                                            \
      bo_ = ao_;                                                                            \
    } else {                                                                                \
      const int s_ = (kt_) / nk_seg, kk_ = ((kt_) % nk_seg) * BK;                           \
      ao_ = (int64_t)s_ * f + kk_;                                                          \
      bo_ = (int64_t)s_ * d * f + kk_;                                                      \
    }                                                                                       \
    _Pragma("unroll") for (int i_ = 0; i_ < A_IW; ++i_)                                    \
        copy16((src_).a[i_] + ao_, (sa_) + (wave * A_IW + i_) * 64);                        \
    _Pragma("unroll") for (int i_ = 0; i_ < B_IW; ++i_)                                    \
        copy16((src_).b[i_] + bo_, (sb_) + (wave * B_IW + i_) * 64);                        \
  } while (0)

  // fragment rows of this wave (row bases are multiples of 32, so the swizzle
  // key depends on the lane's row only)
  const int wm = wave / WN, wn = wave % WN;
  const int fr = lane % 32, half = lane / 32;
  int arow[MI], brow[NI];
#pragma unroll
  for (int i = 0; i < MI; ++i) arow[i] = (wm * TM + i * 32 + fr) * CPR;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    int r;
    if (kSwiglu)
      r = (j < NI / 2) ? wn * (TN / 2) + j * 32 + fr : BN / 2 + wn * (TN / 2) + (j - NI / 2) * 32 + fr;
    else
      r = wn * TN + j * 32 + fr;
    brow[j] = r * CPR;
  }
  const int sw = (fr / 4) % 4;

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // ---- prologue: gather indices of the first two tiles, their sources,
  // stages 0 .. NS-2 of the first tile
  int ib = 0;  // s_idx buffer of the current tile; the next two follow cyclically
  Tile tc = tile_of(L);
  bool has_next = L + per_xcd < t_hi;
  Tile tn = has_next ? tile_of(L + per_xcd) : tc;
  TileSrc<A_IW, B_IW> cur, nxt;
  if (gather) {
    MOE_PIPE_IDX(tc, 0);
    MOE_PIPE_IDX(tn, 1);
    wait_vmcnt<0>();
  }
  MOE_PIPE_SRC(cur, tc, 0);
  MOE_PIPE_SRC(nxt, tn, 1);
  MOE_PIPE_LOAD(cur, 0, sA0, sB0);
  MOE_PIPE_LOAD(cur, 1, sA1, sB1);
  MOE_PIPE_LOAD(cur, 2, sA2, sB2);
  if constexpr (NS == 8) {
    MOE_PIPE_LOAD(cur, 3, sA3, sB3);
    MOE_PIPE_LOAD(cur, 4, sA4, sB4);
    MOE_PIPE_LOAD(cur, 5, sA5, sB5);
    MOE_PIPE_LOAD(cur, 6, sA6, sB6);
  }
  wait_vmcnt<(NS - 3) * LPS>();  // stages 0 and 1 landed (this lane's copies)
  wg_barrier();

  // MFMA operands: the first K step of a stage (R0 / R1, alternating between
  // steps) is read one step ahead; the second K step (RK) within the step
  bf16x8 R0a[MI], R0b[NI], R1a[MI], R1b[NI], RKa[MI], RKb[NI];
#define MOE_PIPE_FRAGS(va_, vb_, sa_, sb_, ks_)                                             \
  do {                                                                                      \
    const int c_ = (half * KS + (ks_)) ^ sw;                                                \
    _Pragma("unroll") for (int i_ = 0; i_ < MI; ++i_)                                      \
        (va_)[i_] = __builtin_bit_cast(bf16x8, lds_read(sa_, arow[i_] + c_));               \
    _Pragma("unroll") for (int j_ = 0; j_ < NI; ++j_)                                      \
        (vb_)[j_] = __builtin_bit_cast(bf16x8, lds_read(sb_, brow[j_] + c_));               \
  } while (0)
#define MOE_PIPE_MFMA(va_, vb_)                                                             \
  do {                                                                                      \
    _Pragma("unroll") for (int i_ = 0; i_ < MI; ++i_)                                      \
        _Pragma("unroll") for (int j_ = 0; j_ < NI; ++j_) acc[i_][j_] =                     \
            __builtin_amdgcn_mfma_f32_32x32x16_bf16((vb_)[j_], (va_)[i_], acc[i_][j_], 0, 0, 0); \
  } while (0)
  MOE_PIPE_FRAGS(R0a, R0b, sA0, sB0, 0);

  uint16_t* out = static_cast<uint16_t*>(p.out);
  const uint16_t* bias = static_cast<const uint16_t*>(p.bias);

  for (;;) {
    // gather indices of the tile after next (landed long before they are read)
    const bool has_next2 = has_next && L + 2 * per_xcd < t_hi;
    Tile tn2;
    if (has_next2) {
      tn2 = tile_of(L + 2 * per_xcd);
      if (gather) MOE_PIPE_IDX(tn2, ib == 0 ? 2 : ib - 1);
    }

    // one K stage.  On entry stages kk and kk + 1 are in LDS and visible to
    // every wave, stage kk's first K step is in registers (Rc), and later
    // stages may still be in flight.  Read stage kk's second K step, refill
    // the stage consumed by the previous step with stage kk + NS - 1 (of this
    // tile, of the next one, or, past the last tile, a harmless repeat of
    // stage 0 that keeps one copy group per step), run the first K step's
    // MFMAs, read stage kk + 1's first K step into Rn, run the second K
    // step's MFMAs, then wait until stage kk + 2 has landed and this wave's
    // LDS reads are done, and meet the other waves.
#define MOE_PIPE_STEP(kk_, sa_, sb_, na_, nb_, fa_, fb_, Rca, Rcb, Rna, Rnb)               \
  do {                                                                                      \
    MOE_PIPE_FRAGS(RKa, RKb, sa_, sb_, 1);                                                  \
    {                                                                                       \
      const int kn_ = (kk_) + NS - 1;                                                       \
      const bool in_cur_ = kn_ < nk;                                                        \
      const int kt_ = in_cur_ ? kn_ : (has_next ? kn_ - nk : 0);                            \
      TileSrc<A_IW, B_IW> ls_;                                                              \
      _Pragma("unroll") for (int i_ = 0; i_ < A_IW; ++i_) ls_.a[i_] = in_cur_ ? cur.a[i_] : nxt.a[i_]; \
      _Pragma("unroll") for (int i_ = 0; i_ < B_IW; ++i_) ls_.b[i_] = in_cur_ ? cur.b[i_] : nxt.b[i_]; \
      MOE_PIPE_LOAD(ls_, kt_, fa_, fb_);                                                    \
    }                                                                                       \
    /* keep the copies at the head of the step (the scheduler would sink them) */          \
    __builtin_amdgcn_sched_barrier(0);                                                      \
    MOE_PIPE_MFMA(Rca, Rcb);                                                                \
    /* first K step's MFMAs first: their operands are already in registers */              \
    __builtin_amdgcn_sched_barrier(0);                                                      \
    MOE_PIPE_FRAGS(Rna, Rnb, na_, nb_, 0);                                                  \
    __builtin_amdgcn_sched_barrier(0); /* next operands in flight under these MFMAs */     \
    MOE_PIPE_MFMA(RKa, RKb);                                                                \
    wait_vmcnt_lds<(NS - 3) * LPS>();                                                       \
    wg_barrier();                                                                           \
  } while (0)

    if constexpr (NS == 4) {
      for (int kk = 0; kk < nk; kk += NS) {
        MOE_PIPE_STEP(kk + 0, sA0, sB0, sA1, sB1, sA3, sB3, R0a, R0b, R1a, R1b);
        MOE_PIPE_STEP(kk + 1, sA1, sB1, sA2, sB2, sA0, sB0, R1a, R1b, R0a, R0b);
        MOE_PIPE_STEP(kk + 2, sA2, sB2, sA3, sB3, sA1, sB1, R0a, R0b, R1a, R1b);
        MOE_PIPE_STEP(kk + 3, sA3, sB3, sA0, sB0, sA2, sB2, R1a, R1b, R0a, R0b);
      }
    } else {
      for (int kk = 0; kk < nk; kk += NS) {
        MOE_PIPE_STEP(kk + 0, sA0, sB0, sA1, sB1, sA7, sB7, R0a, R0b, R1a, R1b);
        MOE_PIPE_STEP(kk + 1, sA1, sB1, sA2, sB2, sA0, sB0, R1a, R1b, R0a, R0b);
        MOE_PIPE_STEP(kk + 2, sA2, sB2, sA3, sB3, sA1, sB1, R0a, R0b, R1a, R1b);
        MOE_PIPE_STEP(kk + 3, sA3, sB3, sA4, sB4, sA2, sB2, R1a, R1b, R0a, R0b);
        MOE_PIPE_STEP(kk + 4, sA4, sB4, sA5, sB5, sA3, sB3, R0a, R0b, R1a, R1b);
        MOE_PIPE_STEP(kk + 5, sA5, sB5, sA6, sB6, sA4, sB4, R1a, R1b, R0a, R0b);
        MOE_PIPE_STEP(kk + 6, sA6, sB6, sA7, sB7, sA5, sB5, R0a, R0b, R1a, R1b);
        MOE_PIPE_STEP(kk + 7, sA7, sB7, sA0, sB0, sA6, sB6, R1a, R1b, R0a, R0b);
      }
    }
#undef MOE_PIPE_STEP

    // ---- epilogue.  acc[i][j] holds the transposed 32x32 block: lane l has
    // tile row i*32 + l%32 and output columns j*32 + 8*(q/4) + 4*(l/32) + q%4.
    // The bias of the tile's columns goes to LDS as float32 once per tile
    // (the down kind: the segments' biases summed in segment order): one
    // round of loads instead of a load and its wait for every accumulator.
    if (BIAS) {
      for (int c = tid; c < BN; c += NT) {
        float b = 0.f;
        if (kSwiglu) {
          const uint16_t* bb = bias + ((int64_t)tc.group * S + tc.seg) * 2 * f;
          b = bf16_to_f32(bb[c < BN / 2 ? tc.n0 + c : f + tc.n0 + (c - BN / 2)]);
        } else if (KIND == kGemmUp) {
          b = bf16_to_f32(bias[((int64_t)tc.group * S + tc.seg) * f + tc.n0 + c]);
        } else {
          for (int sg = 0; sg < S; ++sg) b += bf16_to_f32(bias[((int64_t)tc.group * S + sg) * d + tc.n0 + c]);
        }
        s_bias[c] = b;
      }
      lds_barrier();
    }
    if constexpr (kSwiglu && PAIRED) {
      // training forward (pre-activations too): 16-byte stores from the
      // registers, lane pairs l, l ^ 32 joining their 4-column halves
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm * TM + i * 32 + fr;
        if (r < tc.rows) {
          const int64_t grow = tc.row0 + r;
          // lane l keeps its own half of runs 0, 2 (lower 32 lanes) or 1, 3
          // (upper), gives the partner its half of the other two runs and
          // stores 16 bytes per run it keeps
#pragma unroll
          for (int j = 0; j < NI / 2; ++j) {
            uint32_t hw[4][2], gw[4][2], uw[4][2];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int cidx = wn * (TN / 2) + j * 32 + 8 * g4 + 4 * half;
              uint16_t h[4], pg[4], pu[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float gv = acc[i][j][4 * g4 + e], uv = acc[i][j + NI / 2][4 * g4 + e];
                if (BIAS) {
                  gv += s_bias[cidx + e];
                  uv += s_bias[BN / 2 + cidx + e];
                }
                h[e] = f32_to_bf16(silu_f(gv) * uv);
                pg[e] = f32_to_bf16(gv);
                pu[e] = f32_to_bf16(uv);
              }
              hw[g4][0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
              hw[g4][1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
              gw[g4][0] = (uint32_t)pg[0] | ((uint32_t)pg[1] << 16);
              gw[g4][1] = (uint32_t)pg[2] | ((uint32_t)pg[3] << 16);
              uw[g4][0] = (uint32_t)pu[0] | ((uint32_t)pu[1] << 16);
              uw[g4][1] = (uint32_t)pu[2] | ((uint32_t)pu[3] << 16);
            }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
              const int gs = 2 * pr + (half ? 0 : 1), gk = 2 * pr + (half ? 1 : 0);
              const int cidx = wn * (TN / 2) + j * 32 + 8 * gk;
              // the partner's half of run gk arrives for this lane's half of run gs
              auto run = [&](const uint32_t (*w)[2]) {
                const uint32_t r0 = (uint32_t)__shfl_xor((int)w[gs][0], 32);
                const uint32_t r1 = (uint32_t)__shfl_xor((int)w[gs][1], 32);
                return half ? uint4{r0, r1, w[gk][0], w[gk][1]} : uint4{w[gk][0], w[gk][1], r0, r1};
              };
              *reinterpret_cast<uint4*>(out + grow * p.ldo + (int64_t)tc.seg * f + tc.n0 + cidx) = run(hw);
              uint16_t* pa = static_cast<uint16_t*>(p.preact) + grow * p.ldp +
                             (int64_t)tc.seg * 2 * f + tc.n0 + cidx;
              *reinterpret_cast<uint4*>(pa) = run(gw);
              *reinterpret_cast<uint4*>(pa + f) = run(uw);
            }
          }
        }
      }
    } else {
      // The output tile leaves through LDS (the last stage's buffers, free
      // until the next tile's first step refills them): each pass, every
      // wave writes IPP of its row blocks (bf16, 8 bytes per lane, 16-byte
      // chunks XOR-swizzled by row), then the workgroup stores 16-byte chunks
      // of whole rows, so a wave's store covers full 128-byte lines (storing
      // from the accumulators writes 16 bytes of 32 rows per instruction).
      static_assert(WM == 2, "two half bands");
      constexpr int OC = kSwiglu ? BN / 2 : BN;  // output columns of the tile
      constexpr int NCH = OC / 8;                // 16-byte chunks per output row
      constexpr int HB = (BM < BN ? BM : BN) * CPR * 16;  // bytes per half band
      constexpr int IPP0 = HB / (32 * OC * 2);
      constexpr int IPP = IPP0 > MI ? MI : IPP0;  // row blocks per pass
      constexpr int NP = MI / IPP;                // passes
      constexpr int RCH = IPP * 32 * NCH;         // chunks per half band
      // swizzle key: rows sharing a 256-byte bank window get distinct keys
      constexpr int RPWIN = OC * 2 >= 256 ? 1 : 256 / (OC * 2);
      static_assert(IPP >= 1 && MI % IPP == 0 && (2 * RCH) % NT == 0, "epilogue band");
      char* hb0;
      char* hb1;
      if constexpr (NS == 4) {
        hb0 = reinterpret_cast<char*>(sA3);
        hb1 = reinterpret_cast<char*>(sB3);
      } else {
        hb0 = reinterpret_cast<char*>(sA7);
        hb1 = reinterpret_cast<char*>(sB7);
      }
      char* band = wm == 0 ? hb0 : hb1;
      const int64_t col0 = (KIND == kGemmUp) ? (int64_t)tc.seg * f + tc.n0 : tc.n0;
      auto put = [&](int lr, int oc, const uint16_t* h) {
        const uint2 w = {(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
        const int ch = (oc / 8) ^ ((lr / RPWIN) & (NCH - 1));
        *reinterpret_cast<uint2*>(band + lr * (OC * 2) + ch * 16 + (oc % 8) * 2) = w;
      };
#pragma unroll
      for (int q = 0; q < NP; ++q) {
#pragma unroll
        for (int ii = 0; ii < IPP; ++ii) {
          const int i = q * IPP + ii;
          const int lr = ii * 32 + fr;
          const int r = wm * TM + i * 32 + fr;
          const int64_t grow = tc.row0 + r;
          const bool live = r < tc.rows;
          if (kSwiglu) {
#pragma unroll
            for (int j = 0; j < NI / 2; ++j) {
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const int cidx = wn * (TN / 2) + j * 32 + 8 * g4 + 4 * half;
                uint16_t h[4], pg[4], pu[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  float gv = acc[i][j][4 * g4 + e], uv = acc[i][j + NI / 2][4 * g4 + e];
                  if (BIAS) {
                    gv += s_bias[cidx + e];
                    uv += s_bias[BN / 2 + cidx + e];
                  }
                  h[e] = f32_to_bf16(silu_f(gv) * uv);
                  pg[e] = f32_to_bf16(gv);
                  pu[e] = f32_to_bf16(uv);
                }
                put(lr, cidx, h);
                if (p.preact && live) {
                  uint16_t* pa = static_cast<uint16_t*>(p.preact) + grow * p.ldp +
                                 (int64_t)tc.seg * 2 * f + tc.n0 + cidx;
                  *reinterpret_cast<uint2*>(pa) =
                      uint2{(uint32_t)pg[0] | ((uint32_t)pg[1] << 16), (uint32_t)pg[2] | ((uint32_t)pg[3] << 16)};
                  *reinterpret_cast<uint2*>(pa + f) =
                      uint2{(uint32_t)pu[0] | ((uint32_t)pu[1] << 16), (uint32_t)pu[2] | ((uint32_t)pu[3] << 16)};
                }
              }
            }
          } else {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const int cidx = wn * TN + j * 32 + 8 * g4 + 4 * half;
                uint16_t h[4], pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  float v = acc[i][j][4 * g4 + e];
                  if (KIND == kGemmUp) {
                    if (BIAS) v += s_bias[cidx + e];
                    pv[e] = f32_to_bf16(v);
                    h[e] = f32_to_bf16(gelu_f(v));
                  } else {
                    if (BIAS) v += s_bias[cidx + e];
                    h[e] = f32_to_bf16(v);
                  }
                }
                put(lr, cidx, h);
                if (KIND == kGemmUp && p.preact && live)
                  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.preact) + grow * p.ldp + col0 + cidx) =
                      uint2{(uint32_t)pv[0] | ((uint32_t)pv[1] << 16), (uint32_t)pv[2] | ((uint32_t)pv[3] << 16)};
              }
            }
          }
        }
        lds_barrier();
        // whole rows out: chunk c of the band (the rows of wm = 0, then wm = 1)
#pragma unroll
        for (int u = 0; u < 2 * RCH / NT; ++u) {
          const int c = tid + u * NT;
          const int hb = c / RCH, lc = c % RCH;
          const int lr = lc / NCH, cc = lc % NCH;
          const u32x4 v = *reinterpret_cast<const u32x4*>((hb == 0 ? hb0 : hb1) + lr * (OC * 2) +
                                                          ((cc ^ ((lr / RPWIN) & (NCH - 1))) * 16));
          const int trow = hb * TM + q * IPP * 32 + lr;
          if (trow < tc.rows)
            *reinterpret_cast<u32x4*>(out + (tc.row0 + trow) * p.ldo + col0 + cc * 8) = v;
        }
        lds_barrier();
      }
    }
    if (!has_next) {
      wait_vmcnt<0>();  // no copy may still target LDS when the workgroup ends
      break;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    // advance: next becomes current; the tile after next becomes next (its
    // indices were copied at the start of this tile, LPS or more copies ago,
    // so the waits of this tile's steps have seen them land)
    L += per_xcd;
    tc = tn;
    cur = nxt;
    ib = ib == 2 ? 0 : ib + 1;
    has_next = has_next2;
    if (has_next) {
      tn = tn2;
      MOE_PIPE_SRC(nxt, tn, ib == 2 ? 0 : ib + 1);
    }
  }
#undef MOE_PIPE_FRAGS
#undef MOE_PIPE_MFMA
#undef MOE_PIPE_IDX
#undef MOE_PIPE_SRC
#undef MOE_PIPE_LOAD
}

}  // namespace pipe

namespace {

int device_cus() {
  static int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

template <int BM, int BN, int WM, int WN, int KIND, int ACT, bool BIAS, int NSt, bool PAIRED>
hipError_t run_pipe(const GemmDesc& g, int occ, hipStream_t s) {
  constexpr int NT = 64 * WM * WN;
  constexpr bool kSwiglu = (KIND == kGemmUp && ACT == MOE_ACT_SWIGLU);
  const int tiles_n = KIND == kGemmUp ? g.n_seg * (g.f / (kSwiglu ? BN / 2 : BN)) : g.d / BN;
  const int64_t tiles_m = (g.rows_max + BM - 1) / BM + (g.group_off ? g.n_groups : 0);
  const int64_t upper = tiles_m * tiles_n;
  if (upper <= 0 || g.rows_max <= 0) return hipSuccess;
  int64_t grid = std::min<int64_t>(upper, (int64_t)device_cus() * occ);
  grid = (grid + 7) / 8 * 8;  // a multiple of 8 (XCDs)
  pipe::gemm_pipe_kernel<BM, BN, WM, WN, KIND, ACT, BIAS, NSt, PAIRED>
      <<<dim3((unsigned)grid), dim3(NT), 0, s>>>(g, tiles_n);
  return hipGetLastError();
}

template <int KIND, int ACT, bool BIAS, bool PAIRED = false>
hipError_t dispatch_pipe(const GemmDesc& g, int shape, int occ, hipStream_t s) {
  switch (shape) {
    case 0: return run_pipe<256, 256, 2, 2, KIND, ACT, BIAS, 4, PAIRED>(g, occ, s);
    case 1: return run_pipe<256, 128, 2, 2, KIND, ACT, BIAS, 4, PAIRED>(g, occ, s);
    case 2: return run_pipe<128, 128, 2, 2, KIND, ACT, BIAS, 4, PAIRED>(g, occ, s);
    default: return run_pipe<128, 128, 2, 2, KIND, ACT, BIAS, 8, PAIRED>(g, occ, s);
  }
}

}  // namespace

// Shape index 0: 256x256, 1: 256x128, 2: 128x128 (4 stages), 3: 128x128 with
// 8 stages (all 4 waves, 2 x 2).
bool pipe_shape_fits(GemmKind kind, const GemmDesc& g, int bm, int bn, int stages) {
  (void)bm;
  const bool swiglu = kind == kGemmUp && g.act == MOE_ACT_SWIGLU;
  const int K = kind == kGemmUp ? g.d : g.f;
  if (K % pipe::BK != 0) return false;
  const int nk = (kind == kGemmUp ? 1 : g.n_seg) * (K / pipe::BK);
  if (nk % stages != 0) return false;
  const int ncol = kind == kGemmUp ? (swiglu ? bn / 2 : bn) : bn;
  const int width = kind == kGemmUp ? g.f : g.d;
  // 16-byte output stores
  if (g.ldo % 8 != 0 || reinterpret_cast<uintptr_t>(g.out) % 16 != 0) return false;
  return width % ncol == 0;
}

hipError_t launch_gemm_pipe(GemmKind kind, const GemmDesc& g, int shape, int occ, hipStream_t s) {
  const bool bias = g.bias != nullptr;
  if (kind == kGemmDown)
    return bias ? dispatch_pipe<kGemmDown, 0, true>(g, shape, occ, s)
                : dispatch_pipe<kGemmDown, 0, false>(g, shape, occ, s);
  if (g.act == MOE_ACT_SWIGLU && g.preact)  // training forward: 16-byte epilogue stores
    return bias ? dispatch_pipe<kGemmUp, MOE_ACT_SWIGLU, true, true>(g, shape, occ, s)
                : dispatch_pipe<kGemmUp, MOE_ACT_SWIGLU, false, true>(g, shape, occ, s);
  if (g.act == MOE_ACT_SWIGLU)
    return bias ? dispatch_pipe<kGemmUp, MOE_ACT_SWIGLU, true>(g, shape, occ, s)
                : dispatch_pipe<kGemmUp, MOE_ACT_SWIGLU, false>(g, shape, occ, s);
  return bias ? dispatch_pipe<kGemmUp, MOE_ACT_GELU, true>(g, shape, occ, s)
              : dispatch_pipe<kGemmUp, MOE_ACT_GELU, false>(g, shape, occ, s);
}

}  // namespace moe

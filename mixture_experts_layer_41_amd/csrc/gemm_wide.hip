// Wide-tile persistent grouped GEMM for bf16 on gfx950, for groups of
// thousands of rows (the FLAME-shaped and skewed layers, and the dense
// shared-expert products).
//
// Same operation as the other grouped GEMM kernels (expert FFN up GEMM with
// the SwiGLU / GELU epilogue; down GEMM summing the shared-expert segments
// along K).  Design:
//   * 256 x 256 output tiles (the largest whose float32 accumulators fit the
//     register file: 256 per lane of a CU), 8 waves as 2 x 4, each wave a
//     128 x 64 block of 4 x 2 v_mfma_f32_32x32x16_bf16 tiles, two waves per
//     SIMD.  With one wave per SIMD the in-order issue of the LDS reads and
//     copies stalls that SIMD's matrix pipe (a loop of 16-byte LDS reads and
//     MFMAs measured 1.3 PFLOP/s at one wave per SIMD and 1.9 at two); with
//     two, one wave's memory instructions issue while the other's MFMAs run;
//   * K advances 32 per stage through 4 LDS stages (32 KB each); global data
//     goes straight into LDS (16-byte direct copies, no staging registers);
//   * one barrier per stage, placed between the stage's two K steps: the
//     first K step's MFMAs run on fragments read before the barrier, the
//     second's on fragments read right after it, and the copies for stage
//     s + 3 are issued at the top of stage s, so a copy has two and a half
//     stages to land; group barriers place one LDS read or copy after each
//     MFMA;
//   * two sets of MFMA operand registers (the two K steps), 128 accumulators
//     per lane: no spills in the K loop;
//   * persistent workgroups, one per CU, walk a contiguous run of their XCD's
//     share of the tile list; the copies of the next tile's first stages are
//     issued during the current tile's last stages, so the epilogue overlaps
//     them.  The list runs in groups of 8 row tiles, column-major inside a
//     group, when the output has 8 or more column tiles (the skewed layer's
//     products and the shared experts: 2-5 % faster, fewer re-reads from
//     beyond L2);
//   * LDS rows (64 bytes) are XOR-swizzled in 16-byte chunks on the global
//     side of the copy: chunk' = chunk ^ ((row / 4) % 4), so the 16 lanes of
//     a fragment read hit 16 distinct 16-byte bank groups;
//   * the weight fragment is the MFMA's first operand: each lane ends up with
//     4 consecutive output columns of one row;
//   * the output tile leaves through LDS, a band of rows at a time, as
//     16-byte stores of whole rows (full 128-byte lines) through buffer
//     resources whose range check drops rows past the group's end.  Storing
//     straight from the accumulators wrote 16 bytes per row per instruction,
//     eight times the L2 write requests; those stores, which the next tile's
//     first stage has to wait for, cost 10-20 % of the kernel's time.
// What bounds it: the global -> LDS copies.  With the MFMAs removed the
// copies and LDS reads alone take as long as the whole kernel; with every
// tile reading the same (L2-resident) data the kernel gains only about 15 %.
// Requirements (checked by the host): K per segment a multiple of 32, the
// K stages per tile a multiple of 4, output widths a multiple of the tile
// (of half a tile for the down kind: a last half tile clamps its weight rows
// to the width and stores only its first half).
#include <algorithm>

#include "moe_internal.h"
#include "gemm_common.h"

namespace moe {
namespace wide {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

constexpr int BM = 256, BN = 256;   // output tile
constexpr int BK = 32;              // K elements per stage
constexpr int NS = 4;               // LDS stages
constexpr int CPR = BK / 8;         // 16-byte chunks per LDS row
constexpr int SCH = BM * CPR;       // u32x4 per operand stage
static_assert(CPR == 4, "64-byte LDS rows");

// Wave layout: WM x WN waves, each a (BM / WM) x (BN / WN) block of 32x32
// MFMA tiles.
template <int WM, int WN>
struct Layout {
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
  static constexpr int MI = TM / 32, NI = TN / 32;
  static constexpr int A_IW = BM / (16 * NW);        // 16-row copies per wave per stage (A)
  static constexpr int B_IW = BN / (16 * NW);        // (B)
  static constexpr int LPS = A_IW + B_IW;            // copies per lane per stage
  static_assert(A_IW >= 1 && B_IW >= 1 && MI >= 1 && NI >= 2, "layout");
};

__device__ __forceinline__ void copy16(const void* g, u32x4* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// 4 bytes per lane into LDS; lane i lands at lds + 4 * i
__device__ __forceinline__ void copy4(const void* g, int* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}

// LDS read of a gather index, with its wait in the same asm block (the
// callers order it after the copy of the index with explicit waits)
__device__ __forceinline__ int lds_read_i32(const int* p, int i) {
  int v;
  const uint32_t addr = (uint32_t)(uintptr_t)(p + i);
  __asm__ volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// workgroup barrier without a memory fence; the empty asm statements keep the
// compiler from moving memory accesses across it
__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}
// s_waitcnt vmcnt(0)
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Buffer resource word 3 for raw (untyped, unswizzled) access.
constexpr int kBufFlags = 0x00020000;
// cache-policy operand of a buffer store: the nontemporal (nt) bit
constexpr int kStoreNT = 2;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 4 floats rounded to bf16 (nearest even), one 8-byte buffer store at byte
// offset off (dropped by the range check when past the resource's end)
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, int off, const float* v) {
  const u32x2 w = {pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, 0);
}

// ONE_SEG (down kind): every group has one FFN segment, so stage kt reads
// K chunk kt with no segment arithmetic in the K loop
template <int WM, int WN, int KIND, int ACT, bool BIAS, bool ONE_SEG>
__global__ void __launch_bounds__(64 * WM * WN, 1)
gemm_wide_kernel(GemmDesc p, int tiles_n) {
  constexpr bool kSwiglu = (KIND == kGemmUp && ACT == MOE_ACT_SWIGLU);
  using Ly = Layout<WM, WN>;
  constexpr int NT = Ly::NT, TM = Ly::TM, TN = Ly::TN, MI = Ly::MI, NI = Ly::NI;
  constexpr int A_IW = Ly::A_IW, B_IW = Ly::B_IW, LPS = Ly::LPS;
  constexpr int RW = 16 * A_IW;      // A rows copied by one wave (a contiguous block)
  constexpr int BW = 16 * B_IW;      // B rows copied by one wave
  // the group barriers below hand out one LDS read or copy after each MFMA
  constexpr int MF = MI * NI;        // MFMAs per K step
  constexpr int DSR = MI + NI;       // fragment reads per K step
  static_assert(DSR <= MF && LPS <= MF, "interleave pattern");

  __shared__ __attribute__((aligned(16))) u32x4 sA0[SCH];
  __shared__ __attribute__((aligned(16))) u32x4 sA1[SCH];
  __shared__ __attribute__((aligned(16))) u32x4 sA2[SCH];
  __shared__ __attribute__((aligned(16))) u32x4 sB0[SCH];
  __shared__ __attribute__((aligned(16))) u32x4 sB1[SCH];
  __shared__ __attribute__((aligned(16))) u32x4 sB2[SCH];
  // stage 3 is one array holding both operands: the epilogue's band (either
  // half of it) is then one LDS object, which the compiler knows the copies
  // in flight to stages 0-2 do not write
  __shared__ __attribute__((aligned(16))) u32x4 s3[2 * SCH];
  u32x4* const sA3 = s3;
  u32x4* const sB3 = s3 + SCH;
  __shared__ int s_off[kMaxExperts + 1];     // group row offsets
  __shared__ int s_tstart[kMaxExperts + 1];  // first row tile of each group
  __shared__ int s_idx[3][BM];               // gather indices of three consecutive tiles
  __shared__ float s_bias[BIAS ? BN : 1];    // bias of the current tile's output columns

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;

  // ---- row-tile table of the groups (exact, from the device offsets)
  const int G = p.group_off ? p.n_groups : 1;
  for (int g = tid; g <= G; g += NT)
    s_off[g] = p.group_off ? p.group_off[g] : (g == 0 ? 0 : (int)p.rows_max);
  __syncthreads();
  // first row tile of each group (s_tstart[G] = all row tiles): one wave,
  // each lane owning a run of consecutive groups, the runs' totals scanned
  // across the lanes
  if (wave == 0) {
    const int per = (G + kWave - 1) / kWave;
    const int g0 = min(lane * per, G), g1 = min(g0 + per, G);
    auto row_tiles = [&](int g) {
      const int rows = min(s_off[g + 1], (int)p.rows_max) - min(s_off[g], (int)p.rows_max);
      return rows > 0 ? (rows + BM - 1) / BM : 0;
    };
    int own = 0;
    for (int g = g0; g < g1; ++g) own += row_tiles(g);
    int incl = own;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int run = incl - own;
    for (int g = g0; g < g1; ++g) {
      s_tstart[g] = run;
      run += row_tiles(g);
    }
    if (lane == kWave - 1) s_tstart[G] = incl;
  }
  __syncthreads();
  const int m_tiles = s_tstart[G];

  // ---- this workgroup's tiles: XCD x = blockIdx % 8 owns the x-th eighth of
  // the tile list; its workgroups stride through it
  const int total = m_tiles * tiles_n;
  const int xcd = blockIdx.x % 8, per_xcd = gridDim.x / 8;
  const int t_lo = (int)((int64_t)total * xcd / 8), t_hi = (int)((int64_t)total * (xcd + 1) / 8);
  int L = t_lo + (int)(blockIdx.x / 8);
  if (L >= t_hi) return;

  const int S = p.n_seg, d = p.d, f = p.f;
  const uint16_t* A = static_cast<const uint16_t*>(p.a);
  const uint16_t* W = static_cast<const uint16_t*>(p.w);
  const int kw = (KIND == kGemmUp) ? d : f;                // weight row length (one segment)
  const int rows1 = (KIND == kGemmUp) ? (kSwiglu ? 2 * f : f) : d;  // weight rows per segment
  const int nk_seg = kw / BK;                              // stages per FFN segment
  const int nk = (KIND == kGemmUp) ? nk_seg : S * nk_seg;  // stages per tile
  // stage kt of the down kind reads chunk kt % nk_seg of FFN segment
  // kt / nk_seg; the quotient as a multiply-high by ceil(2^32 / nk_seg),
  // exact while kt and nk_seg stay below 2^16 (the host checks nk, and
  // nk_seg >= 2 for the down kind)
  const uint32_t seg_mul = (uint32_t)((0x100000000ull + nk_seg - 1) / nk_seg);
  const int64_t seg_w = (int64_t)d * f;                    // weight elements per segment

  // copy geometry: copy i of wave w covers tile rows w*64 + i*16 + lane/4 at
  // LDS chunk lane%4, which holds global chunk (lane%4) ^ ((row/4)%4) =
  // (lane%4) ^ ((lane/16)%4)
  const int lrow = lane / 4;
  const int chk = ((lane % 4) ^ ((lane / 16) % 4)) * 8;

  struct Tile {
    int group, rows, seg, n0;
    int64_t row0;
  };
  auto tile_of = [&](int l) {
    Tile t;
    // tile order: groups of gm row tiles, column-major inside a group, so
    // an XCD's concurrent tiles form a block of about 8 x 4 tiles (fewer
    // distinct operand panels than 3 rows of 11 tiles); narrow outputs
    // (4 column tiles) are already that shape row by row
    const int gm = tiles_n >= 8 ? 8 : 1;
    const int gsz = gm * tiles_n, gi = l / gsz, rem = l % gsz;
    const int rig = min(gm, m_tiles - gi * gm);
    const int mt = gi * gm + rem % rig, nt = rem / rig;
    int glo = 0, ghi = G - 1;  // last g with s_tstart[g] <= mt
    while (glo < ghi) {
      const int mid = (glo + ghi + 1) / 2;
      if (s_tstart[mid] <= mt) glo = mid; else ghi = mid - 1;
    }
    // the values are the same in every lane: keep them in scalar registers
    t.group = __builtin_amdgcn_readfirstlane(glo);
    const int r0 = __builtin_amdgcn_readfirstlane(s_off[glo] + (mt - s_tstart[glo]) * BM);
    t.row0 = r0;
    t.rows = __builtin_amdgcn_readfirstlane(min(BM, min(s_off[glo + 1], (int)p.rows_max) - r0));
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

  // per-lane copy sources of one tile at K = 0: A rows (gathered or direct)
  // and the first B row (the wave's B rows are 16 apart per copy)
  struct Src {
    const uint16_t* a[A_IW];
    const uint16_t* b;
  };
  const bool gather = p.a_rows != nullptr;
  // gather indices of this wave's 64 rows of tile t_ -> s_idx[buf_] (one
  // 4-byte copy per lane; rows past the tile end repeat its last row)
#define MOE_WIDE_IDX(t_, buf_)                                                              \
  do {                                                                                      \
    if (lane < RW) {                                                                        \
      const int r_ = wave * RW + lane;                                                      \
      const int64_t gr_ = (t_).row0 + (r_ < (t_).rows ? r_ : (t_).rows - 1);               \
      copy4(p.a_rows + gr_, &s_idx[buf_][wave * RW]);                                       \
    }                                                                                       \
  } while (0)
  auto src_of = [&](const Tile& t, int buf) {
    Src s;
#pragma unroll
    for (int i = 0; i < A_IW; ++i) {
      const int rr = wave * RW + i * 16 + lrow;
      const int64_t row = gather ? (int64_t)lds_read_i32(s_idx[buf], rr)
                                 : t.row0 + (rr < t.rows ? rr : t.rows - 1);
      s.a[i] = A + row * p.lda + chk;
    }
    const uint16_t* wb = W + ((int64_t)t.group * S + t.seg) * rows1 * (int64_t)kw;
    // the wave's B rows (BW of them, never across the gate / up boundary at
    // BN / 2 for SwiGLU)
    const int rb = wave * BW + lrow;
    int wr;
    if (kSwiglu)
      wr = (rb < BN / 2) ? t.n0 + rb : f + t.n0 + (rb - BN / 2);
    else
      wr = min(t.n0 + rb, rows1 - 1);  // a last column tile may be half outside the width
    s.b = wb + (int64_t)wr * kw + chk;
    return s;
  };
  // copies of K stage kt_ of the tile with sources src_ into LDS (sa_, sb_)
#define MOE_WIDE_LOAD(src_, kt_, sa_, sb_)                                                  \
  do {                                                                                      \
    int64_t ao_, bo_;                                                                       \
    if (KIND == kGemmUp) {                                                                  \
      ao_ = (int64_t)(kt_) * BK;                                                            \
      bo_ = ao_;                                                                            \
    } else {                                                                                \
      const int s_ = ONE_SEG ? 0 : (int)__umulhi((uint32_t)(kt_), seg_mul);               \
      const int kk_ = ((kt_) - s_ * nk_seg) * BK;                                           \
      ao_ = (int64_t)s_ * f + kk_;                                                          \
      bo_ = s_ * seg_w + kk_;                                                               \
    }                                                                                       \
    _Pragma("unroll") for (int i_ = 0; i_ < A_IW; ++i_)                                    \
        copy16((src_).a[i_] + ao_, (sa_) + (wave * A_IW + i_) * 64);                        \
    _Pragma("unroll") for (int i_ = 0; i_ < B_IW; ++i_)                                    \
        copy16((src_).b + (int64_t)i_ * 16 * kw + bo_, (sb_) + (wave * B_IW + i_) * 64);   \
  } while (0)

  // fragment rows of this wave (row bases are multiples of 32, so the
  // swizzle key depends on the lane's row only)
  const int wm = wave / WN, wn = wave % WN;  // wave position in the tile
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
  // stages 0..2 of the first tile
  int ib = 0;  // s_idx buffer of the current tile; the next two follow cyclically
  Tile tc = tile_of(L);
  bool has_next = L + per_xcd < t_hi;
  Tile tn = has_next ? tile_of(L + per_xcd) : tc;
  if (gather) {
    MOE_WIDE_IDX(tc, 0);
    MOE_WIDE_IDX(tn, 1);
    wait_vm0();
  }
  Src cur = src_of(tc, 0);
  Src nxt = src_of(tn, 1);
  MOE_WIDE_LOAD(cur, 0, sA0, sB0);
  MOE_WIDE_LOAD(cur, 1, sA1, sB1);
  MOE_WIDE_LOAD(cur, 2, sA2, sB2);
  wait_vm_lgkm<2 * LPS>();  // stage 0 landed (this lane's copies)
  wg_barrier();

  bf16x8 F0a[MI], F0b[NI], F1a[MI], F1b[NI];
#define MOE_WIDE_FRAGS(va_, vb_, sa_, sb_, ks_)                                             \
  do {                                                                                      \
    const int c_ = (half + 2 * (ks_)) ^ sw;                                                 \
    _Pragma("unroll") for (int i_ = 0; i_ < MI; ++i_)                                      \
        (va_)[i_] = __builtin_bit_cast(bf16x8, (sa_)[arow[i_] + c_]);                       \
    _Pragma("unroll") for (int j_ = 0; j_ < NI; ++j_)                                      \
        (vb_)[j_] = __builtin_bit_cast(bf16x8, (sb_)[brow[j_] + c_]);                       \
  } while (0)
#define MOE_WIDE_MFMA(va_, vb_)                                                             \
  do {                                                                                      \
    _Pragma("unroll") for (int i_ = 0; i_ < MI; ++i_)                                      \
        _Pragma("unroll") for (int j_ = 0; j_ < NI; ++j_) acc[i_][j_] =                     \
            __builtin_amdgcn_mfma_f32_32x32x16_bf16((vb_)[j_], (va_)[i_], acc[i_][j_], 0, 0, 0); \
  } while (0)
  MOE_WIDE_FRAGS(F0a, F0b, sA0, sB0, 0);

  uint16_t* out = static_cast<uint16_t*>(p.out);
  const uint16_t* bias = static_cast<const uint16_t*>(p.bias);

  for (;;) {
    // gather indices of the tile after next (landed long before they are read)
    const bool has_next2 = has_next && L + 2 * per_xcd < t_hi;
    Tile tn2 = tn;
    if (has_next2) {
      tn2 = tile_of(L + 2 * per_xcd);
      if (gather) MOE_WIDE_IDX(tn2, ib == 0 ? 2 : ib - 1);
    }

    // one stage, in two halves around one barrier.  On entry stage kk is in
    // LDS and visible to every wave, its first K step is in F0, and stages
    // kk+1, kk+2 may be in flight.
    //   first half: refill the buffer of stage kk - 1 (free since the last
    //   barrier) with stage kk + 3 (of this tile, of the next one, or past
    //   the last tile a harmless repeat of stage 0, which keeps one copy
    //   group per stage) and read the second K step (F1), both interleaved
    //   with the MFMAs on F0;
    //   wait until stage kk + 1 has landed and F1 is in registers; barrier;
    //   second half: read stage kk + 1's first K step into F0, interleaved
    //   with the MFMAs on F1.
    // The group barriers place one LDS read or one copy after each MFMA, so
    // the matrix pipe is fed while the memory instructions issue.
#define MOE_WIDE_STAGE(kk_, sa_, sb_, na_, nb_, fa_, fb_)                                   \
  do {                                                                                      \
    {                                                                                       \
      const int kn_ = (kk_) + NS - 1;                                                       \
      const bool in_cur_ = kn_ < nk;                                                        \
      const int kt_ = in_cur_ ? kn_ : (has_next ? kn_ - nk : 0);                            \
      Src ls_;                                                                              \
      _Pragma("unroll") for (int i_ = 0; i_ < A_IW; ++i_) ls_.a[i_] = in_cur_ ? cur.a[i_] : nxt.a[i_]; \
      ls_.b = in_cur_ ? cur.b : nxt.b;                                                      \
      MOE_WIDE_LOAD(ls_, kt_, fa_, fb_);                                                    \
    }                                                                                       \
    MOE_WIDE_FRAGS(F1a, F1b, sa_, sb_, 1);                                                  \
    MOE_WIDE_MFMA(F0a, F0b);                                                                \
    _Pragma("unroll") for (int g_ = 0; g_ < MF; ++g_) {                                    \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* MFMA */                         \
      if (g_ < DSR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); /* LDS read */       \
      if (g_ < LPS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* copy */           \
    }                                                                                       \
    wait_vm_lgkm<(NS - 2) * LPS>();                                                         \
    wg_barrier();                                                                           \
    MOE_WIDE_FRAGS(F0a, F0b, na_, nb_, 0);                                                  \
    MOE_WIDE_MFMA(F1a, F1b);                                                                \
    _Pragma("unroll") for (int g_ = 0; g_ < MF; ++g_) {                                    \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1); /* MFMA */                         \
      if (g_ < DSR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1); /* LDS read */       \
    }                                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                      \
  } while (0)

    for (int kk = 0; kk < nk; kk += NS) {
      MOE_WIDE_STAGE(kk + 0, sA0, sB0, sA1, sB1, sA3, sB3);
      MOE_WIDE_STAGE(kk + 1, sA1, sB1, sA2, sB2, sA0, sB0);
      MOE_WIDE_STAGE(kk + 2, sA2, sB2, sA3, sB3, sA1, sB1);
      MOE_WIDE_STAGE(kk + 3, sA3, sB3, sA0, sB0, sA2, sB2);
    }
#undef MOE_WIDE_STAGE

    // ---- epilogue.  acc[i][j] holds the transposed 32x32 block: lane l has
    // tile row i*32 + l%32 and output columns j*32 + 8*(q/4) + 4*(l/32) + q%4.
    // The output tile leaves through LDS (stage buffer 3, free from the last
    // stage's barrier until the next tile's first stage refills it): in each
    // pass every wave writes its accumulators of IPP row blocks (bf16, 8
    // bytes per lane, 16-byte chunks XOR-swizzled by row), then every lane
    // stores 16-byte chunks of whole rows, so a wave's store covers full
    // 128-byte lines.  Stores go through buffer resources that span the
    // tile's valid rows: a row past the group's end is dropped by the range
    // check.  Pre-activations (training) are stored from the registers.
    {
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          out + tc.row0 * p.ldo, (short)0, (int)(tc.rows * p.ldo * 2), kBufFlags);
      __amdgpu_buffer_rsrc_t rp = ro;
      if (KIND == kGemmUp && p.preact)
        rp = __builtin_amdgcn_make_buffer_rsrc(static_cast<uint16_t*>(p.preact) + tc.row0 * p.ldp,
                                              (short)0, (int)(tc.rows * p.ldp * 2), kBufFlags);
      constexpr int OC = kSwiglu ? BN / 2 : BN;   // output columns of the tile
      constexpr int NCH = OC / 8;                 // 16-byte chunks per output row
      constexpr int IPP = (SCH * 16) / (32 * OC * 2);  // row blocks per pass (16 KB per wave row)
      constexpr int NP = MI / IPP;                // passes
      constexpr int RCH = SCH;                    // chunks per half band (16 KB)
      static_assert(IPP >= 1 && MI % IPP == 0 && (2 * RCH) % NT == 0, "epilogue band");
      static_assert(OC * 2 >= 256, "a row per 256-byte bank window at least (swizzle key = row)");
      const int col0 = (KIND == kGemmUp) ? tc.seg * f + tc.n0 : tc.n0;
      // bias of the tile's columns as float32, once per tile (the down kind:
      // the segments' biases summed in segment order): one round of loads
      // instead of a load and its wait for every accumulator
      if (BIAS) {
        for (int c = tid; c < BN; c += NT) {
          float b = 0.f;
          if (kSwiglu) {
            const uint16_t* bb = bias + ((int64_t)tc.group * S + tc.seg) * 2 * f;
            b = bf16_to_f32(bb[c < BN / 2 ? tc.n0 + c : f + tc.n0 + (c - BN / 2)]);
          } else if (KIND == kGemmUp) {
            b = bf16_to_f32(bias[((int64_t)tc.group * S + tc.seg) * f + tc.n0 + c]);
          } else {
            for (int sg = 0; sg < S; ++sg)
              b += bf16_to_f32(bias[((int64_t)tc.group * S + sg) * d + min(tc.n0 + c, d - 1)]);
          }
          s_bias[c] = b;
        }
        lds_barrier();
      }
      u32x2* const band = reinterpret_cast<u32x2*>(s3) + wm * (2 * SCH);  // this wave's half
      // 4 values of output column oc (a multiple of 4) of band row lr.  The
      // write is an asm statement: the compiler would otherwise wait for
      // every copy in flight (the next tile's stages 1 and 2, which target
      // other buffers) before the first write.
      auto put = [&](int lr, int oc, const float* v) {
        const u32x2 w = {pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
        const int ch = (oc / 8) ^ (lr & (NCH - 1));
        const uint32_t a = (uint32_t)(uintptr_t)(band + lr * (OC / 4) + ch * 2 + (oc % 8) / 4);
        __asm__ volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(w) : "memory");
      };
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ii = 0; ii < IPP; ++ii) {
          const int i = q * IPP + ii;
          const int lr = ii * 32 + fr;
          const int r = wm * TM + i * 32 + fr;
          const int prow = r * (int)p.ldp;
          if (kSwiglu) {
#pragma unroll
            for (int j = 0; j < NI / 2; ++j) {
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const int cidx = wn * (TN / 2) + j * 32 + 8 * g4 + 4 * half;
                float hv[4], gv[4], uv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  gv[e] = acc[i][j][4 * g4 + e];
                  uv[e] = acc[i][j + NI / 2][4 * g4 + e];
                  if (BIAS) {
                    gv[e] += s_bias[cidx + e];
                    uv[e] += s_bias[BN / 2 + cidx + e];
                  }
                  hv[e] = silu_f(gv[e]) * uv[e];
                }
                put(lr, cidx, hv);
                if (p.preact) {
                  const int pc = tc.seg * 2 * f + tc.n0 + cidx;
                  store4(rp, (prow + pc) * 2, gv);
                  store4(rp, (prow + pc + f) * 2, uv);
                }
              }
            }
          } else {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const int cidx = wn * TN + j * 32 + 8 * g4 + 4 * half;
                float hv[4], pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  float v = acc[i][j][4 * g4 + e];
                  if (KIND == kGemmUp) {
                    if (BIAS) v += s_bias[cidx + e];
                    pv[e] = v;
                    hv[e] = gelu_f(v);
                  } else {
                    if (BIAS) v += s_bias[cidx + e];
                    hv[e] = v;
                  }
                }
                put(lr, cidx, hv);
                if (KIND == kGemmUp && p.preact) store4(rp, (prow + col0 + cidx) * 2, pv);
              }
            }
          }
        }
        lds_barrier();
        // whole rows out: chunk c of the band (two halves of RCH chunks: the
        // rows of wm = 0, then wm = 1)
#pragma unroll
        for (int u = 0; u < 2 * RCH / NT; ++u) {
          const int c = tid + u * NT;
          const int hb = c / RCH, lc = c % RCH;
          const int lr = lc / NCH, cc = lc % NCH;
          const u32x4 v = s3[hb * SCH + lr * NCH + (cc ^ (lr & (NCH - 1)))];
          const int trow = hb * TM + q * IPP * 32 + lr;
          // streaming store (nt): the output is read back only by the next
          // kernel, so it need not displace this kernel's operand lines in L2
          if (KIND == kGemmUp || tc.n0 + cc * 8 < d)  // columns past the width (down: half tiles)
            __builtin_amdgcn_raw_buffer_store_b128(v, ro, (trow * (int)p.ldo + col0 + cc * 8) * 2, 0, kStoreNT);
        }
        lds_barrier();
      }
    }
    if (!has_next) {
      wait_vm0();  // no copy may still target LDS when the workgroup ends
      break;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    // advance: next becomes current; the tile after next becomes next (its
    // indices were copied at the start of this tile, many stages ago, and
    // the stage waits since then have seen them land)
    L += per_xcd;
    tc = tn;
    cur = nxt;
    ib = ib == 2 ? 0 : ib + 1;
    has_next = has_next2;
    if (has_next) {
      tn = tn2;
      nxt = src_of(tn, ib == 2 ? 0 : ib + 1);
    }
  }
#undef MOE_WIDE_FRAGS
#undef MOE_WIDE_MFMA
#undef MOE_WIDE_LOAD
#undef MOE_WIDE_IDX
}


}  // namespace wide

namespace {

int wide_cus() {
  static int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

template <int WM, int WN, int KIND, int ACT, bool BIAS, bool ONE_SEG = false>
hipError_t run_wide(const GemmDesc& g, hipStream_t s) {
  constexpr bool kSwiglu = (KIND == kGemmUp && ACT == MOE_ACT_SWIGLU);
  // down: the last column tile may cover half a tile (widths multiple of 128)
  const int tiles_n = KIND == kGemmUp ? g.n_seg * (g.f / (kSwiglu ? wide::BN / 2 : wide::BN))
                                      : (g.d + wide::BN - 1) / wide::BN;
  const int64_t tiles_m = (g.rows_max + wide::BM - 1) / wide::BM + (g.group_off ? g.n_groups : 0);
  const int64_t upper = tiles_m * tiles_n;
  if (upper <= 0 || g.rows_max <= 0) return hipSuccess;
  int64_t grid = std::min<int64_t>(upper, (int64_t)wide_cus());
  grid = (grid + 7) / 8 * 8;  // a multiple of 8 (XCDs)
  wide::gemm_wide_kernel<WM, WN, KIND, ACT, BIAS, ONE_SEG>
      <<<dim3((unsigned)grid), dim3(64 * WM * WN), 0, s>>>(g, tiles_n);
  return hipGetLastError();
}

}  // namespace

// Whether the wide kernel covers the problem: bf16 weights (no INT8 codes),
// K per segment a multiple of 32 with a multiple of 4 stages per tile, and
// output widths that fill whole tiles.
bool wide_fits(GemmKind kind, const GemmDesc& g) {
  if (g.w_scale) return false;
  // the epilogue's 32-bit buffer offsets: 256 rows of output (and
  // pre-activations) stay below 2 GiB
  if (g.ldo >= ((int64_t)1 << 22) || (g.preact && g.ldp >= ((int64_t)1 << 22))) return false;
  // 16-byte output stores
  if (g.ldo % 8 != 0 || reinterpret_cast<uintptr_t>(g.out) % 16 != 0) return false;
  const bool swiglu = kind == kGemmUp && g.act == MOE_ACT_SWIGLU;
  const int K = kind == kGemmUp ? g.d : g.f;
  if (K % wide::BK != 0) return false;
  const int nk = (kind == kGemmUp ? 1 : g.n_seg) * (K / wide::BK);
  // the down kind's segment quotient: nk below 2^16, two stages per segment at least
  if (nk % wide::NS != 0 || nk >= (1 << 16) || (kind == kGemmDown && K / wide::BK < 2)) return false;
  // output widths in whole tiles; the down kind also takes a last half tile
  // (the backward's dh product: width f = 1408 on the skewed layer)
  const int ncol = kind == kGemmUp ? (swiglu ? wide::BN / 2 : wide::BN) : wide::BN / 2;
  const int width = kind == kGemmUp ? g.f : g.d;
  return width % ncol == 0;
}

// 8 waves (2 x 4, wave tile 128 x 64, two waves per SIMD)
hipError_t launch_gemm_wide(GemmKind kind, const GemmDesc& g, hipStream_t s) {
  constexpr int WM = 2, WN = 4;
  const bool bias = g.bias != nullptr;
  if (kind == kGemmDown) {
    if (g.n_seg == 1)
      return bias ? run_wide<WM, WN, kGemmDown, 0, true, true>(g, s)
                  : run_wide<WM, WN, kGemmDown, 0, false, true>(g, s);
    return bias ? run_wide<WM, WN, kGemmDown, 0, true>(g, s) : run_wide<WM, WN, kGemmDown, 0, false>(g, s);
  }
  if (g.act == MOE_ACT_SWIGLU)
    return bias ? run_wide<WM, WN, kGemmUp, MOE_ACT_SWIGLU, true>(g, s)
                : run_wide<WM, WN, kGemmUp, MOE_ACT_SWIGLU, false>(g, s);
  return bias ? run_wide<WM, WN, kGemmUp, MOE_ACT_GELU, true>(g, s)
              : run_wide<WM, WN, kGemmUp, MOE_ACT_GELU, false>(g, s);
}

}  // namespace moe

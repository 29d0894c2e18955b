// Large-tile grouped GEMM for bf16 on gfx950 (the path taken whenever the
// reduction length is a multiple of the K tile and the output width fills
// whole tiles; everything else goes to the generic kernel in gemm.hip).
//
// Same math as the generic kernel (expert FFN up GEMM with the SwiGLU / GELU
// epilogue, down GEMM summing shared-expert segments); differences:
//   * BM x BN workgroup tiles (up to 256 x 256) over 4 or 8 waves; each wave owns
//     (BM/WM) x (BN/WN) of v_mfma_f32_32x32x16_bf16 blocks, so every 16-byte
//     LDS fragment feeds several MFMAs;
//   * global loads of K tile t+1 go to registers while tile t feeds the
//     MFMAs from LDS, then land in the other LDS stage (one barrier per K
//     tile);
//   * LDS rows are XOR-swizzled in 16-byte chunks.  gfx950 serves a 16-byte
//     LDS read 16 lanes at a time over 64 four-byte banks (a 256-byte
//     window); the 16 lanes of a fragment read 16 consecutive rows at one
//     chunk, and chunk' = chunk ^ ((row / rows_per_window) % chunks_per_row)
//     puts them in 16 distinct 16-byte bank groups;
//   * workgroups are remapped so each XCD (blockIdx % 8) takes a contiguous
//     run of tiles: the tiles of one expert, which share its weights, then
//     hit the same L2;
//   * INT8 weights (Q8 != 0): the weight tile is loaded as codes (half the
//     bytes) and widened to bf16 on the way from the staging registers to
//     LDS; the MFMA loop is the bf16 one.  Q8 = 1: the codes enter the MFMAs
//     as they are (small integers are exact in bf16) and the epilogue
//     multiplies each output column by its weight row's scale; this covers
//     every GEMM whose K range is one weight matrix.  Q8 = 2 (the down GEMM
//     summing several shared experts, whose K segments each bring their own
//     row scales): each code is multiplied by its row scale and rounded to
//     bf16 while staging.
#include <algorithm>
#include <cmath>

#include "moe_internal.h"
#include "gemm_common.h"

namespace moe {
namespace tiled {


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

// One output tile: K loop over the group's rows and the tile's weight rows,
// then the epilogue.  sA / sB are the two LDS stages.  PD = K tiles whose
// global loads are in flight at once (1, or 2 with two register sets; PD = 2
// needs an even number of K tiles).  STREAM_W: the tile is its group's only
// row tile, so it reads each weight byte once (bf16 weight loads then carry
// the nontemporal hint).
template <int BM, int BN, int BK, int WM, int WN, int KIND, int ACT, bool BIAS, int Q8, int PD,
          bool STREAM_W = false>
__device__ __forceinline__ void gemm_tile_body(const GemmDesc& p, const TileInfo& tile, int nt,
                                               u32x4 (*sA)[BM * (BK / 8)],
                                               u32x4 (*sB)[BN * (BK / 8)]) {
  constexpr int NW = WM * WN;
  constexpr int kTileThreads = 64 * NW;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int MI = TM / 32, NI = TN / 32;  // 32x32 MFMA blocks per wave
  constexpr bool kSwiglu = (KIND == kGemmUp && ACT == MOE_ACT_SWIGLU);
  constexpr int CPR = BK / 8;                // 16-byte chunks per tile row
  constexpr int RPW = 256 / (BK * 2);        // tile rows per 256-byte bank window
  constexpr int A_LD = BM * CPR / kTileThreads;  // 16-byte loads per thread per K tile
  constexpr int B_LD = Q8 ? 1 : BN * CPR / kTileThreads;  // (unused with Q8)
  constexpr int CPR8 = BK / 16;                  // 16-byte chunks of codes per tile row (Q8)
  constexpr int B8_LD = BN * CPR8 / kTileThreads;  // 16-byte code loads per thread (Q8)
  constexpr int KS = BK / 16;                // MFMA K steps per K tile
  static_assert(BK == 32 || BK == 64, "K tile");
  static_assert(MI >= 1 && NI >= 1 && A_LD >= 1 && B_LD >= 1, "tile shape");
  static_assert(!Q8 || (B8_LD >= 1 && BN * CPR8 % kTileThreads == 0), "tile shape");
  static_assert(Q8 != 2 || KIND == kGemmDown, "row scales while staging: the shared down GEMM only");
  static_assert(!kSwiglu || (NI % 2 == 0), "SwiGLU pairs gate and up blocks");
  static_assert(PD == 1 || PD == 2, "prefetch depth");
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int S = p.n_seg, d = p.d, f = p.f;

  int seg = 0, n0;
  int64_t wbase;  // element offset of the tile's weight slab
  int K;
  const int rows1 = (KIND == kGemmUp) ? (kSwiglu ? 2 * f : f) : d;  // weight rows per segment
  if (KIND == kGemmUp) {
    constexpr int bnh = kSwiglu ? BN / 2 : BN;
    const int tpn = f / bnh;
    seg = nt / tpn;
    n0 = (nt % tpn) * bnh;
    wbase = ((int64_t)tile.group * S + seg) * rows1 * (int64_t)d;
    K = d;
  } else {
    n0 = nt * BN;
    wbase = (int64_t)tile.group * S * (int64_t)d * f;
    K = f;
  }
  const int nk_seg = K / BK;
  const int nk = (KIND == kGemmUp) ? nk_seg : S * nk_seg;

  // --- load slots: chunk c = tid + 256 i -> row c / CPR, chunk c % CPR
  const uint16_t* A = static_cast<const uint16_t*>(p.a);
  const uint16_t* aptr[A_LD];
  const uint16_t* bptr[B_LD];
  int aoff[A_LD], boff[B_LD];  // swizzled LDS slot (uint4 units)
  const int8_t* bptr8[B8_LD];
  int boff8[B8_LD][2];   // LDS slots of the two bf16 chunks a code chunk becomes
  int brow8[B8_LD];      // weight row (within the segment) of each code load
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int c = tid + kTileThreads * i;
    const int r = c / CPR, ch = c % CPR;
    const int64_t gr = tile.row0 + (r < tile.rows ? r : tile.rows - 1);
    const int64_t src = p.a_rows ? (int64_t)p.a_rows[gr] : gr;
    aptr[i] = A + src * p.lda + ch * 8;
    aoff[i] = r * CPR + (ch ^ ((r / RPW) % CPR));
  }
  if constexpr (!Q8) {
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int c = tid + kTileThreads * i;
      const int r = c / CPR, ch = c % CPR;
      int wr;
      if (kSwiglu)
        wr = (r < BN / 2) ? n0 + r : f + n0 + (r - BN / 2);
      else
        wr = n0 + r;
      bptr[i] = static_cast<const uint16_t*>(p.w) + wbase + (int64_t)wr * K + ch * 8;
      boff[i] = r * CPR + (ch ^ ((r / RPW) % CPR));
    }
  } else {
#pragma unroll
    for (int i = 0; i < B8_LD; ++i) {
      const int c = tid + kTileThreads * i;
      const int r = c / CPR8, c8 = c % CPR8;  // 16 codes = K [16 c8, 16 c8 + 16)
      int wr;
      if (kSwiglu)
        wr = (r < BN / 2) ? n0 + r : f + n0 + (r - BN / 2);
      else
        wr = n0 + r;
      brow8[i] = wr;
      bptr8[i] = static_cast<const int8_t*>(p.w) + wbase + (int64_t)wr * K + c8 * 16;
      boff8[i][0] = r * CPR + ((2 * c8) ^ ((r / RPW) % CPR));
      boff8[i][1] = r * CPR + ((2 * c8 + 1) ^ ((r / RPW) % CPR));
    }
  }

  // bf16 weight loads of a tile that is its group's only row tile (decode
  // batches: groups of at most 32 rows) carry the nontemporal hint: each
  // weight byte is read once, and a K tile is one whole 128-byte line of
  // each weight row, so the lines need not stay in the caches (a plain
  // streaming read of HBM runs 7-10 % faster with the hint).  Not for INT8
  // codes: their K tile is half a line, whose other half the next K tile
  // reads (with the hint that half came from HBM again: 40 % slower).  A
  // group of several row tiles keeps its weight panels cached for the others.
  auto ld_w = [](const u32x4* q) -> u32x4 {
    if constexpr (STREAM_W) return __builtin_nontemporal_load(q);
    return *q;
  };
  u32x4 ra[PD][A_LD], rb[PD][B_LD];  // staging registers of the next K tile(s)
  u32x4 rb8[PD][B8_LD];              // (Q8) codes of the next K tile(s)
  float sc8[PD][B8_LD];              // (Q8 = 2) their row scales
  // load K tile kt_ into register set r_ (a compile-time constant)
#define MOE_TILE_LOAD(kt_, r_)                                                              \
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
    _Pragma("unroll") for (int i_ = 0; i_ < A_LD; ++i_)                                    \
        ra[r_][i_] = *reinterpret_cast<const u32x4*>(aptr[i_] + ao_);                       \
    if constexpr (!Q8) {                                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < B_LD; ++i_)                                  \
          rb[r_][i_] = ld_w(reinterpret_cast<const u32x4*>(bptr[i_] + bo_));                \
    } else {                                                                                \
      _Pragma("unroll") for (int i_ = 0; i_ < B8_LD; ++i_)                                 \
          rb8[r_][i_] = *reinterpret_cast<const u32x4*>(bptr8[i_] + bo_);                   \
      if constexpr (Q8 == 2) {                                                              \
        const int s_ = (kt_) / nk_seg;                                                      \
        _Pragma("unroll") for (int i_ = 0; i_ < B8_LD; ++i_)                               \
            sc8[r_][i_] = p.w_scale[((int64_t)tile.group * S + s_) * rows1 + brow8[i_]];    \
      }                                                                                     \
    }                                                                                       \
  } while (0)
  // store register set r_ into LDS stage st_
#define MOE_TILE_STORE(st_, r_)                                                             \
  do {                                                                                      \
    _Pragma("unroll") for (int i_ = 0; i_ < A_LD; ++i_) sA[st_][aoff[i_]] = ra[r_][i_];     \
    if constexpr (!Q8) {                                                                    \
      _Pragma("unroll") for (int i_ = 0; i_ < B_LD; ++i_) sB[st_][boff[i_]] = rb[r_][i_];   \
    } else {                                                                                \
      _Pragma("unroll") for (int i_ = 0; i_ < B8_LD; ++i_) {                               \
        /* codes stay packed until here: no unpacking next to the load */                   \
        if constexpr (PD == 2) asm volatile("" : "+v"(rb8[r_][i_]));                       \
        u32x4 lo_, hi_;                                                                     \
        if constexpr (Q8 == 2)                                                              \
          dequant16(rb8[r_][i_], sc8[r_][i_], lo_, hi_);                                    \
        else                                                                                \
          codes16_to_bf16(rb8[r_][i_], lo_, hi_);                                           \
        sB[st_][boff8[i_][0]] = lo_;                                                        \
        sB[st_][boff8[i_][1]] = hi_;                                                        \
      }                                                                                     \
    }                                                                                       \
  } while (0)

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // LDS rows of this wave's fragments (row bases are multiples of 32, so the
  // swizzle key depends on the fragment row only)
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
  const int sw = (fr / RPW) % CPR;

  // (Q8 = 1) row scale of each output column this lane holds: fragment j's
  // column fr is weight row brow[j] / CPR of the tile
  float esc[Q8 == 1 ? NI : 1];
  if constexpr (Q8 == 1) {
    const int64_t sbase = ((int64_t)tile.group * S + seg) * rows1;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = brow[j] / CPR;
      int wr;
      if (kSwiglu)
        wr = (r < BN / 2) ? n0 + r : f + n0 + (r - BN / 2);
      else
        wr = n0 + r;
      esc[j] = p.w_scale[sbase + wr];
    }
  }

  // MFMAs over the K tile in LDS stage st_
#define MOE_TILE_COMPUTE(st_)                                                               \
  do {                                                                                      \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                    \
      /* lanes of half h take the K elements [h*BK/2, (h+1)*BK/2) of the tile, */           \
      /* one chunk per K step; A and B use the same order */                                \
      const int c = (half * KS + ks) ^ sw;                                                  \
      bf16x8 fa[MI], fb[NI];                                                                \
      _Pragma("unroll") for (int i = 0; i < MI; ++i)                                       \
          fa[i] = __builtin_bit_cast(bf16x8, sA[st_][arow[i] + c]);                         \
      _Pragma("unroll") for (int j = 0; j < NI; ++j)                                       \
          fb[j] = __builtin_bit_cast(bf16x8, sB[st_][brow[j] + c]);                         \
      _Pragma("unroll") for (int i = 0; i < MI; ++i)                                       \
          _Pragma("unroll") for (int j = 0; j < NI; ++j)                                   \
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j],  \
                                                                  0, 0, 0);                 \
    }                                                                                       \
  } while (0)

  if constexpr (PD == 1) {
    MOE_TILE_LOAD(0, 0);
    MOE_TILE_STORE(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      if (kt + 1 < nk) MOE_TILE_LOAD(kt + 1, 0);
      MOE_TILE_COMPUTE(st);
      if (kt + 1 < nk) MOE_TILE_STORE(st ^ 1, 0);
      __syncthreads();
    }
  } else {
    // two K tiles in flight: register set r holds the tile bound for LDS
    // stage r, loaded one step before the step that stores it.  nk is even;
    // the loads past the end re-read the last tile (clamped, so no branch
    // splits the loads from the MFMAs) and the stores after the last tile go
    // to a stage nobody reads again.  The scheduling barriers keep each
    // step's loads ahead of its MFMAs and the dequantizing stores behind
    // them, so a load has two steps to land.
    MOE_TILE_LOAD(0, 0);
    MOE_TILE_LOAD(1, 1);
    MOE_TILE_STORE(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      MOE_TILE_LOAD(min(kt + 2, nk - 1), 0);
      __builtin_amdgcn_sched_barrier(0);
      MOE_TILE_COMPUTE(0);
      __builtin_amdgcn_sched_barrier(0);
      MOE_TILE_STORE(1, 1);
      __syncthreads();
      MOE_TILE_LOAD(min(kt + 3, nk - 1), 1);
      __builtin_amdgcn_sched_barrier(0);
      MOE_TILE_COMPUTE(1);
      __builtin_amdgcn_sched_barrier(0);
      MOE_TILE_STORE(0, 0);
      __syncthreads();
    }
  }
#undef MOE_TILE_LOAD
#undef MOE_TILE_STORE
#undef MOE_TILE_COMPUTE

  // epilogue.  The bf16 SwiGLU up GEMM and the down GEMMs stage the output
  // tile through LDS; the GELU and INT8-scaled up GEMMs, whose epilogues
  // would spill with the band addressing, store from the registers.
  constexpr bool kStage = !(KIND == kGemmUp && (Q8 == 1 || !kSwiglu));
  // bias of this lane's output columns (one per j; SwiGLU: gate and up),
  // float32, loaded once instead of once per accumulator (the down kind: the
  // segments' biases summed in segment order)
  float bsa[NI], bsb[NI];
  if (BIAS) {
    const uint16_t* bias = static_cast<const uint16_t*>(p.bias);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      bsa[j] = bsb[j] = 0.f;
      if (kSwiglu) {
        if (j < NI / 2) {
          const int cidx = wn * (TN / 2) + j * 32 + fr;
          const uint16_t* b = bias + ((int64_t)tile.group * S + seg) * 2 * f;
          bsa[j] = bf16_to_f32(b[n0 + cidx]);
          bsb[j] = bf16_to_f32(b[f + n0 + cidx]);
        }
      } else {
        const int cidx = wn * TN + j * 32 + fr;
        if (KIND == kGemmUp) {
          bsa[j] = bf16_to_f32(bias[((int64_t)tile.group * S + seg) * f + n0 + cidx]);
        } else {
          for (int sg = 0; sg < S; ++sg) bsa[j] += bf16_to_f32(bias[((int64_t)tile.group * S + sg) * d + n0 + cidx]);
        }
      }
    }
  }
  if constexpr (kStage) {
    // 32x32 C layout: column lane%32, rows 8*(q/4) + 4*(lane/32) + q%4.
    // The output tile goes through LDS (free since the K loop's last barrier):
    // each lane writes its values (bf16) into a [BM][OC] band, output columns
    // [0, 128) in sA's bytes and [128, 256) in sB's, 256-byte rows whose
    // 16-byte chunks are XOR-swizzled by row; then every lane stores 16-byte
    // chunks of whole rows (a 2-byte store per value would write 64 bytes of
    // two rows per instruction).  Pre-activations are stored from the registers.
    static_assert(BK == 64, "256-byte band rows in the LDS stages");
    constexpr int OC = kSwiglu ? BN / 2 : BN;  // output columns of the tile
    constexpr int NCH = OC / 8;                // 16-byte chunks per output row
    static_assert(OC % 8 == 0 && OC <= 256 && (OC <= 128 || BN >= BM), "epilogue band");
    static_assert((BM * NCH) % kTileThreads == 0, "epilogue band");
    uint16_t* out = static_cast<uint16_t*>(p.out);
    char* const bandA = reinterpret_cast<char*>(&sA[0][0]);
    char* const bandB = reinterpret_cast<char*>(&sB[0][0]);
    auto band_at = [&](int r, int c) -> char* {
      const int cc = c % 128;
      return (c < 128 ? bandA : bandB) + r * 256 + (((cc / 8) ^ (r & 15)) * 16) + (cc % 8) * 2;
    };
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = wm * TM + i * 32 + 8 * (q / 4) + 4 * half + (q % 4);
        const bool live = r < tile.rows;
        const int64_t grow = tile.row0 + r;
        if (kSwiglu) {
#pragma unroll
          for (int j = 0; j < NI / 2; ++j) {
            const int cidx = wn * (TN / 2) + j * 32 + fr;
            float g = acc[i][j][q], u = acc[i][j + NI / 2][q];
            if constexpr (Q8 == 1) {
              g *= esc[j];
              u *= esc[j + NI / 2];
            }
            if (BIAS) {
              g += bsa[j];
              u += bsb[j];
            }
            *reinterpret_cast<uint16_t*>(band_at(r, cidx)) = f32_to_bf16(silu_f(g) * u);
            if (p.preact && live) {
              uint16_t* pa = static_cast<uint16_t*>(p.preact) + grow * p.ldp + (int64_t)seg * 2 * f + n0 + cidx;
              pa[0] = f32_to_bf16(g);
              pa[f] = f32_to_bf16(u);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int cidx = wn * TN + j * 32 + fr;
            float v = acc[i][j][q];
            if constexpr (Q8 == 1) v *= esc[j];
            if (KIND == kGemmUp) {
              if (BIAS) v += bsa[j];
              if (p.preact && live)
                static_cast<uint16_t*>(p.preact)[grow * p.ldp + (int64_t)seg * f + n0 + cidx] = f32_to_bf16(v);
              *reinterpret_cast<uint16_t*>(band_at(r, cidx)) = f32_to_bf16(gelu_f(v));
            } else {
              if (BIAS) v += bsa[j];
              *reinterpret_cast<uint16_t*>(band_at(r, cidx)) = f32_to_bf16(v);
            }
          }
        }
      }
    }
    __syncthreads();
    const int64_t col0 = (KIND == kGemmUp) ? (int64_t)seg * f + n0 : n0;
#pragma unroll
    for (int u = 0; u < BM * NCH / kTileThreads; ++u) {
      const int c = tid + u * kTileThreads;
      const int r = c / NCH, cc = c % NCH;
      const u32x4 v = *reinterpret_cast<const u32x4*>(band_at(r, cc * 8));
      if (r < tile.rows) *reinterpret_cast<u32x4*>(out + (tile.row0 + r) * p.ldo + col0 + cc * 8) = v;
    }
    __syncthreads();  // the band is read before the next tile's loads land in LDS

  } else {
    // epilogue (32x32 C layout: column lane%32, rows 8*(q/4) + 4*(lane/32) + q%4)
    uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = wm * TM + i * 32 + 8 * (q / 4) + 4 * half + (q % 4);
        if (r >= tile.rows) continue;
        const int64_t grow = tile.row0 + r;
        if (kSwiglu) {
#pragma unroll
          for (int j = 0; j < NI / 2; ++j) {
            const int cidx = wn * (TN / 2) + j * 32 + fr;
            float g = acc[i][j][q], u = acc[i][j + NI / 2][q];
            if constexpr (Q8 == 1) {
              g *= esc[j];
              u *= esc[j + NI / 2];
            }
            if (BIAS) {
              g += bsa[j];
              u += bsb[j];
            }
            out[grow * p.ldo + (int64_t)seg * f + n0 + cidx] = f32_to_bf16(silu_f(g) * u);
            if (p.preact) {
              uint16_t* pa = static_cast<uint16_t*>(p.preact) + grow * p.ldp + (int64_t)seg * 2 * f + n0 + cidx;
              pa[0] = f32_to_bf16(g);
              pa[f] = f32_to_bf16(u);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int cidx = wn * TN + j * 32 + fr;
            float v = acc[i][j][q];
            if constexpr (Q8 == 1) v *= esc[j];
            if (KIND == kGemmUp) {
              if (BIAS) v += bsa[j];
              if (p.preact)
                static_cast<uint16_t*>(p.preact)[grow * p.ldp + (int64_t)seg * f + n0 + cidx] = f32_to_bf16(v);
              out[grow * p.ldo + (int64_t)seg * f + n0 + cidx] = f32_to_bf16(gelu_f(v));
            } else {
              if (BIAS) v += bsa[j];
              out[grow * p.ldo + n0 + cidx] = f32_to_bf16(v);
            }
          }
        }
      }
    }

  }
}

// One workgroup per tile slot; the row tile is looked up from the group
// offsets.  Blocks are remapped so that each XCD (blockIdx % 8) takes a
// contiguous run of tiles: the tiles of one expert share its weights in that
// XCD's L2.
template <int BM, int BN, int BK, int WM, int WN, int KIND, int ACT, bool BIAS, int Q8, int PD>
__global__ void __launch_bounds__(64 * WM * WN, PD == 2 ? 2 : 1)
gemm_tile_kernel(GemmDesc p, int tiles_n) {
  __shared__ __attribute__((aligned(16))) u32x4 sA[2][BM * (BK / 8)];
  __shared__ __attribute__((aligned(16))) u32x4 sB[2][BN * (BK / 8)];
  __shared__ TileInfo s_tile;
  __shared__ int s_nt;
  // XCD x = blockIdx % 8 takes the x-th eighth of the exact tile list (the
  // grid is sized for an upper bound; surplus blocks leave at once)
  if (threadIdx.x < kWave) {
    const int64_t total = (int64_t)count_row_tiles(p.group_off, p.n_groups, p.rows_max, BM) * tiles_n;
    const int xcd = blockIdx.x % 8;
    const int64_t lo = total * xcd / 8, hi = total * (xcd + 1) / 8;
    const int64_t L = lo + blockIdx.x / 8;
    TileInfo t;
    t.group = -1;
    t.row0 = 0;
    t.rows = 0;
    if (L < hi) t = find_row_tile(p.group_off, p.n_groups, p.rows_max, BM, (int)(L / tiles_n));
    if (threadIdx.x == 0) {
      s_tile = t;
      s_nt = (int)(L % tiles_n);
    }
  }
  __syncthreads();
  const TileInfo tile = s_tile;
  const int nt = s_nt;
  if (tile.group < 0) return;
  if constexpr (BM <= 32 && !Q8) {
    const int64_t grows = p.group_off ? (int64_t)p.group_off[tile.group + 1] - p.group_off[tile.group]
                                      : p.rows_max;
    if (grows <= BM) {
      gemm_tile_body<BM, BN, BK, WM, WN, KIND, ACT, BIAS, Q8, PD, true>(p, tile, nt, sA, sB);
      return;
    }
  }
  gemm_tile_body<BM, BN, BK, WM, WN, KIND, ACT, BIAS, Q8, PD>(p, tile, nt, sA, sB);
}

// (With two tiles in flight the extra staging registers would otherwise push
// the kernel past 256 VGPRs, i.e. to one wave per SIMD; every shape here runs
// two waves per SIMD, which the second bound asks for.)
//
// Persistent variant: the grid holds only the resident workgroups; the
// row-tile table of the groups is built once per workgroup in LDS, and XCD
// x = blockIdx % 8 walks a contiguous run of the (exact) tile list.
template <int BM, int BN, int BK, int WM, int WN, int KIND, int ACT, bool BIAS, int Q8, int PD>
__global__ void __launch_bounds__(64 * WM * WN, PD == 2 ? 2 : 1)
gemm_tile_persistent(GemmDesc p, int tiles_n) {
  constexpr int kTileThreads = 64 * WM * WN;
  __shared__ __attribute__((aligned(16))) u32x4 sA[2][BM * (BK / 8)];
  __shared__ __attribute__((aligned(16))) u32x4 sB[2][BN * (BK / 8)];
  __shared__ int s_off[kMaxExperts + 1];     // group row offsets
  __shared__ int s_tstart[kMaxExperts + 1];  // first row tile of each group
  __shared__ int s_scan[kMaxExperts + 1];

  const int G = p.group_off ? p.n_groups : 1;
  for (int g = threadIdx.x; g <= G; g += kTileThreads)
    s_off[g] = p.group_off ? p.group_off[g] : (g == 0 ? 0 : (int)p.rows_max);
  __syncthreads();
  for (int g = threadIdx.x; g <= G; g += kTileThreads) {
    const int rows = g < G ? min(s_off[g + 1], (int)p.rows_max) - min(s_off[g], (int)p.rows_max) : 0;
    s_tstart[g] = rows > 0 ? (rows + BM - 1) / BM : 0;  // tiles of group g, scanned below
  }
  __syncthreads();
  for (int o = 1; o <= G; o <<= 1) {  // inclusive scan over g = 0..G
    for (int g = threadIdx.x; g <= G; g += kTileThreads) s_scan[g] = g >= o ? s_tstart[g - o] : 0;
    __syncthreads();
    for (int g = threadIdx.x; g <= G; g += kTileThreads) s_tstart[g] += s_scan[g];
    __syncthreads();
  }
  const int m_tiles = s_tstart[G - 1];
  for (int g = threadIdx.x; g <= G; g += kTileThreads) s_scan[g] = g == 0 ? 0 : s_tstart[g - 1];
  __syncthreads();
  for (int g = threadIdx.x; g <= G; g += kTileThreads) s_tstart[g] = s_scan[g];
  __syncthreads();

  const int total = m_tiles * tiles_n;
  const int xcd = blockIdx.x % 8, per_xcd = gridDim.x / 8;
  const int lo = (int)((int64_t)total * xcd / 8), hi = (int)((int64_t)total * (xcd + 1) / 8);
  for (int L = lo + (int)(blockIdx.x / 8); L < hi; L += per_xcd) {
    const int mt = L / tiles_n, nt = L % tiles_n;
    // group of row tile mt: last g with s_tstart[g] <= mt (binary search)
    int glo = 0, ghi = G - 1;
    while (glo < ghi) {
      const int mid = (glo + ghi + 1) / 2;
      if (s_tstart[mid] <= mt) glo = mid; else ghi = mid - 1;
    }
    TileInfo tile;
    tile.group = glo;
    tile.row0 = (int64_t)s_off[glo] + (int64_t)(mt - s_tstart[glo]) * BM;
    tile.rows = min(BM, min(s_off[glo + 1], (int)p.rows_max) - (int)tile.row0);
    if constexpr (BM <= 32 && !Q8) {
      if (min(s_off[glo + 1], (int)p.rows_max) - s_off[glo] <= BM) {
        gemm_tile_body<BM, BN, BK, WM, WN, KIND, ACT, BIAS, Q8, PD, true>(p, tile, nt, sA, sB);
        continue;
      }
    }
    gemm_tile_body<BM, BN, BK, WM, WN, KIND, ACT, BIAS, Q8, PD>(p, tile, nt, sA, sB);
  }
}

}  // namespace tiled

bool pipe_shape_fits(GemmKind kind, const GemmDesc& g, int bm, int bn, int stages);
hipError_t launch_gemm_pipe(GemmKind kind, const GemmDesc& g, int shape, int occ, hipStream_t s);
bool wide_fits(GemmKind kind, const GemmDesc& g);
hipError_t launch_gemm_wide(GemmKind kind, const GemmDesc& g, hipStream_t s);

namespace {
using namespace tiled;

struct TileCfg {
  int bm, bn, bk, occ;  // occ: workgroups resident per CU
  double eff;           // relative MFMA efficiency of the shape
};

constexpr int kVariants = 9;
constexpr int kFirstPipe = 4;  // variants 4..7 are the pipelined kernel (gemm_pipe.hip)
constexpr int kWide = 8;       // the wide-tile kernel (gemm_wide.hip)
constexpr TileCfg kTiles[kVariants] = {
    {256, 256, 64, 1, 1.0},   // 8 waves, wave tile 128 x 64
    {256, 128, 64, 1, 0.85},  // 8 waves, wave tile 64 x 64
    {128, 128, 64, 2, 0.9},   // wave tile 64 x 64
    {32, 256, 64, 2, 0.6},    // decode-shaped: few rows per expert
    {256, 256, 32, 1, 1.3},   // pipelined, 4 waves, wave tile 128 x 128
    {256, 128, 32, 1, 1.1},   // pipelined, 4 waves, wave tile 128 x 64
    {128, 128, 32, 2, 1.1},   // pipelined, 4 waves, wave tile 64 x 64
    {128, 128, 32, 1, 1.0},   // pipelined, 8 stages (long K, few tiles)
    {256, 256, 32, 1, 1.6},   // wide: 8 waves, wave tile 128 x 64, 4 stages
};

int cu_count();

template <int BM, int BN, int BK, int WM, int WN, bool PERSIST, int KIND, int ACT, bool BIAS, int Q8,
          int PD>
hipError_t run(const GemmDesc& g, int occ, hipStream_t s) {
  constexpr int kTileThreads = 64 * WM * WN;
  constexpr bool kSwiglu = (KIND == kGemmUp && ACT == MOE_ACT_SWIGLU);
  int tiles_n;
  if (KIND == kGemmUp)
    tiles_n = g.n_seg * (g.f / (kSwiglu ? BN / 2 : BN));
  else
    tiles_n = g.d / BN;
  // upper bound of the row tiles (the exact count is known on the device)
  const int64_t tiles_m = (g.rows_max + BM - 1) / BM + (g.group_off ? g.n_groups : 0);
  const int64_t upper = tiles_m * tiles_n;
  if (upper <= 0 || g.rows_max <= 0) return hipSuccess;
  int64_t grid = PERSIST ? std::min<int64_t>(upper, (int64_t)cu_count() * occ) : upper;
  grid = (grid + 7) / 8 * 8;  // a multiple of 8 (XCDs)
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if constexpr (PERSIST)
    gemm_tile_persistent<BM, BN, BK, WM, WN, KIND, ACT, BIAS, Q8, PD>
        <<<dim3((unsigned)grid), dim3(kTileThreads), 0, s>>>(g, tiles_n);
  else
    gemm_tile_kernel<BM, BN, BK, WM, WN, KIND, ACT, BIAS, Q8, PD>
        <<<dim3((unsigned)grid), dim3(kTileThreads), 0, s>>>(g, tiles_n);
  return hipGetLastError();
}

// INT8 weights keep two K tiles in flight (their K is a multiple of 128, so
// the K tile count is even): a tile of codes is half the bytes of a bf16 one.
// The decode-shaped tile (weight streaming) does so for bf16 too when the K
// tile count is even.
template <int KIND, int ACT, bool BIAS, int Q8>
hipError_t dispatch(const GemmDesc& g, int variant, hipStream_t s) {
  constexpr int PD = Q8 ? 2 : 1;
  const bool even_k_tiles = (KIND == kGemmUp ? g.d : g.f) % 128 == 0;
  switch (variant) {
    case 0: return run<256, 256, 64, 2, 4, false, KIND, ACT, BIAS, Q8, PD>(g, kTiles[0].occ, s);
    case 1: return run<256, 128, 64, 4, 2, true, KIND, ACT, BIAS, Q8, PD>(g, kTiles[1].occ, s);
    case 2: return run<128, 128, 64, 2, 2, true, KIND, ACT, BIAS, Q8, PD>(g, kTiles[2].occ, s);
    default:
      // one group (a shared expert over a decode batch): half-width column
      // tiles over 2 waves, up to 4 per CU, so that twice the CUs stream
      // its weights (many groups already give every CU tiles)
      if (!g.group_off || g.n_groups == 1) {
        if (even_k_tiles) return run<32, 128, 64, 1, 2, true, KIND, ACT, BIAS, Q8, 2>(g, 4, s);
        return run<32, 128, 64, 1, 2, true, KIND, ACT, BIAS, Q8, PD>(g, 4, s);
      }
      if (even_k_tiles) return run<32, 256, 64, 1, 4, true, KIND, ACT, BIAS, Q8, 2>(g, kTiles[3].occ, s);
      return run<32, 256, 64, 1, 4, true, KIND, ACT, BIAS, Q8, PD>(g, kTiles[3].occ, s);
  }
}

template <int KIND, int ACT, bool BIAS>
hipError_t dispatch_w(const GemmDesc& g, int variant, hipStream_t s) {
  if (!g.w_scale) return dispatch<KIND, ACT, BIAS, 0>(g, variant, s);
  if constexpr (KIND == kGemmDown)
    if (g.n_seg > 1) return dispatch<KIND, ACT, BIAS, 2>(g, variant, s);
  return dispatch<KIND, ACT, BIAS, 1>(g, variant, s);
}

int cu_count() {
  static int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}

}  // namespace

// Shape preference by expected rows per group, from kernel-time sweeps of
// every shape on MI355X: weight streaming (up to 128 rows per group) is
// fastest with the 32-row decode tile on both GEMMs (on the decode layer the
// routed down GEMM 1 % faster than with the pipelined 128x128 tile, and the
// shared expert's 128 rows take twice the tiles, so twice the CUs stream its
// weights: the step 0.9 % faster); a few hundred rows per group with the
// pipelined 128x128
// (up) and the 128x128 persistent tile (down); thousands of rows with the
// pipelined 256x128 (up) and the 8-wave 256x256 (down).
const int* preferred_variants(GemmKind kind, double rows_per_group) {
  static const int up_decode[] = {3, 6, 2, -1}, dn_decode[] = {3, 6, 2, -1};
  static const int up_small[] = {6, 2, 5, -1}, dn_small[] = {2, 1, 6, -1};
  static const int up_large[] = {8, 5, 0, 4, -1}, dn_large[] = {8, 0, 2, 5, -1};
  if (rows_per_group <= 128) return kind == kGemmUp ? up_decode : dn_decode;
  if (rows_per_group < 1024) return kind == kGemmUp ? up_small : dn_small;
  return kind == kGemmUp ? up_large : dn_large;
}

// Picks a tile shape, or -1 if no shape covers the problem: the first
// preferred shape that covers it, else the cost model below.  Expected rows
// per group = rows_max spread evenly over the groups (plus half a tile of
// padding per group in the model).  Predicted time ~ rounds of resident
// workgroups x tile work / shape efficiency.
// force >= 0 selects that shape if it covers the problem.
int pick_tile_variant(const moe_config& c, GemmKind kind, const GemmDesc& g, int force) {
  if (c.dtype != MOE_DTYPE_BF16) return -1;
  const bool swiglu = kind == kGemmUp && g.act == MOE_ACT_SWIGLU;
  const int K = kind == kGemmUp ? g.d : g.f;
  const double groups = g.group_off ? g.n_groups : 1;
  const double rows_per_group = (double)g.rows_max / groups;
  const int cus = cu_count();
  auto fits = [&](int v) {
    const TileCfg& tc = kTiles[v];
    if (g.w_scale && v >= kFirstPipe) return false;  // INT8 weights: register-staged tiles only
    // 16-byte output stores
    if (g.ldo % 8 != 0 || reinterpret_cast<uintptr_t>(g.out) % 16 != 0) return false;
    if (v == kWide) return wide_fits(kind, g);
    if (K % tc.bk != 0) return false;
    const int ncol = kind == kGemmUp ? (swiglu ? tc.bn / 2 : tc.bn) : tc.bn;
    const int nwidth = kind == kGemmUp ? g.f : g.d;
    if (nwidth % ncol != 0) return false;
    if (v >= kFirstPipe && !pipe_shape_fits(kind, g, tc.bm, tc.bn, v == 7 ? 8 : 4)) return false;
    return true;
  };
  if (force >= 0) return force < kVariants && fits(force) ? force : -1;
  for (const int* v = preferred_variants(kind, rows_per_group); *v >= 0; ++v)
    if (fits(*v)) return *v;
  int best = -1;
  double best_t = 0;
  for (int v = 0; v < kVariants; ++v) {
    const TileCfg& tc = kTiles[v];
    if (!fits(v)) continue;
    const int ncol = kind == kGemmUp ? (swiglu ? tc.bn / 2 : tc.bn) : tc.bn;
    const int nwidth = kind == kGemmUp ? g.f : g.d;
    const double tiles_n = (double)(kind == kGemmUp ? g.n_seg : 1) * (nwidth / ncol);
    const double tiles = groups * (g.group_off ? rows_per_group / tc.bm + 0.5
                                               : std::ceil(rows_per_group / tc.bm)) * tiles_n;
    const double rounds = std::ceil(tiles / ((double)cus * tc.occ));
    const double t = rounds * tc.occ * (double)tc.bm * tc.bn / tc.eff;
    if (best < 0 || t < best_t) {
      best = v;
      best_t = t;
    }
  }
  return best;
}

hipError_t launch_gemm_tiled(const moe_config& c, GemmKind kind, const GemmDesc& g, int variant,
                             hipStream_t s) {
  if (variant == kWide) return launch_gemm_wide(kind, g, s);
  if (variant >= kFirstPipe)
    return launch_gemm_pipe(kind, g, variant - kFirstPipe, kTiles[variant].occ, s);
  const bool bias = g.bias != nullptr;
  if (kind == kGemmDown)
    return bias ? dispatch_w<kGemmDown, 0, true>(g, variant, s)
                : dispatch_w<kGemmDown, 0, false>(g, variant, s);
  if (g.act == MOE_ACT_SWIGLU)
    return bias ? dispatch_w<kGemmUp, MOE_ACT_SWIGLU, true>(g, variant, s)
                : dispatch_w<kGemmUp, MOE_ACT_SWIGLU, false>(g, variant, s);
  return bias ? dispatch_w<kGemmUp, MOE_ACT_GELU, true>(g, variant, s)
              : dispatch_w<kGemmUp, MOE_ACT_GELU, false>(g, variant, s);
}

}  // namespace moe

// One 256x256 output tile of C = A * B^T on CDNA4 bf16 MFMA, with A [M][K] and
// B [N][K] both K-contiguous ("NT"). Every contraction of the path has this
// shape: the forward logit tile X W_s^T and its backward recompute (K = H),
// dX = G (W_s^T)^T (K = vocabulary chunk) and dW_s = G^T (X^T)^T (K = token
// chunk), the last two fed with transposed copies so both operands stay
// K-contiguous.
//
// Workgroup: 256 threads = 4 waves of 64, arranged WM x WN over the tile; each
// wave owns a (256/WM) x (256/WN) sub-tile held as 32x32 MFMA accumulators.
// K advances 64 at a time through two LDS stages of 64 KB (A and B, 32 KB
// each), filled by direct global->LDS 16-byte loads (no VGPR staging) while
// the MFMAs run on the other stage.
//
// LDS layout of one operand stage: 256 rows x 128 bytes (64 bf16 of K), as
// 16-byte chunks. Chunk kc of row r sits in slot kc ^ (r & 7) ^ ((r >> 3) & 1),
// so the 16-byte fragment reads of 8 consecutive rows (32-bank phases) and of
// 16 consecutive rows (64-bank phases) each touch distinct banks.
#pragma once
#include "cdna4.hpp"

namespace lce {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kTileBytes = kBM * kBK * 2;      // one operand, one stage: 32 KB
constexpr int kStageBytes = 2 * kTileBytes;    // A + B
constexpr int kMainLds = 2 * kStageBytes;      // double-buffered: 128 KB

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Global -> LDS loader for one 256-row operand. Rows at or past rows_valid are
// clamped to the last valid row: they load real (finite) data whose results the
// epilogues discard.
struct OperandLoader {
  const char* base;
  uint32_t off[8];

  __device__ __forceinline__ void init(const uint16_t* p, int ld, int row0, int rows_valid, int wave, int lane) {
    base = reinterpret_cast<const char*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int r = wave * 64 + j * 8 + (lane >> 3);
      int kc = (lane & 7) ^ (((lane >> 3) & 7) ^ (j & 1));
      int gr = min(row0 + r, rows_valid - 1);
      off[j] = (uint32_t)gr * (uint32_t)ld * 2u + (uint32_t)kc * 16u;
    }
  }
  __device__ __forceinline__ void issue(int k0, LCE_LDS char* tile, int wave) const {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      g2lds16(base + off[j] + (uint32_t)k0 * 2u, tile + (wave * 8 + j) * 1024);
  }
};

template <int WM, int WN>
struct TileShape {
  static constexpr int kWaveM = kBM / WM;
  static constexpr int kWaveN = kBN / WN;
  static constexpr int kMI = kWaveM / 32;
  static constexpr int kNI = kWaveN / 32;
  static_assert(WM * WN == 4, "four waves per workgroup");
};

// One K=64 stage: 4 MFMA k-steps of 16 over the wave's MI x NI accumulators.
// With kZeroInit the first k-step starts from a literal-zero accumulator, so a
// tile never spends instructions clearing its accumulators.
template <int MI, int NI, bool kZeroInit>
__device__ __forceinline__ void mma_stage(const LCE_LDS char* a_tile, const LCE_LDS char* b_tile, int a_wrow,
                                          int b_wrow, int lane, f32x16 (&acc)[MI][NI]) {
  const int sw = swz(lane);
  const int half = lane >> 5;
  const int ra = (a_wrow + (lane & 31)) * 128;
  const int rb = (b_wrow + (lane & 31)) * 128;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int slot = ((ks * 2 + half) ^ sw) * 16;
    bf16x8 a[MI], b[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) a[i] = *reinterpret_cast<const LCE_LDS bf16x8*>(a_tile + ra + i * 4096 + slot);
#pragma unroll
    for (int j = 0; j < NI; ++j) b[j] = *reinterpret_cast<const LCE_LDS bf16x8*>(b_tile + rb + j * 4096 + slot);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        if (kZeroInit && ks == 0) {
          const f32x16 zero = {};
          acc[i][j] = mfma32(a[i], b[j], zero);
        } else {
          acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
        }
      }
  }
}

// Full K loop for one tile (K >= 64). If stage0_issued, the caller already
// issued the loads of k-block 0 into stage 0. The accumulators need no
// initialisation. On return all waves have passed a barrier and both LDS
// stages are free.
template <int WM, int WN>
__device__ __forceinline__ void tile_mainloop(const OperandLoader& la, const OperandLoader& lb, int K,
                                              LCE_LDS char* lds,
                                              f32x16 (&acc)[TileShape<WM, WN>::kMI][TileShape<WM, WN>::kNI],
                                              bool stage0_issued) {
  using S = TileShape<WM, WN>;
  const int wave = wave_id();
  const int lane = lane_id();
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int kt_n = K / kBK;
  if (!stage0_issued) {
    la.issue(0, lds, wave);
    lb.issue(0, lds + kTileBytes, wave);
  }
  wait_vm0();
  __syncthreads();
  for (int kt = 0; kt < kt_n; ++kt) {
    LCE_LDS char* cur = lds + (kt & 1) * kStageBytes;
    if (kt + 1 < kt_n) {
      LCE_LDS char* nxt = lds + ((kt + 1) & 1) * kStageBytes;
      la.issue((kt + 1) * kBK, nxt, wave);
      lb.issue((kt + 1) * kBK, nxt + kTileBytes, wave);
    }
    if (kt == 0)
      mma_stage<S::kMI, S::kNI, true>(cur, cur + kTileBytes, wm * S::kWaveM, wn * S::kWaveN, lane, acc);
    else
      mma_stage<S::kMI, S::kNI, false>(cur, cur + kTileBytes, wm * S::kWaveM, wn * S::kWaveN, lane, acc);
    wait_vm0();
    __syncthreads();
  }
}

// Row / column (within the 256x256 tile) of accumulator element e of block (i, j).
template <int WM, int WN>
__device__ __forceinline__ int acc_row(int wave, int lane, int i, int e) {
  return (wave / WN) * TileShape<WM, WN>::kWaveM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
template <int WM, int WN>
__device__ __forceinline__ int acc_col(int wave, int lane, int j) {
  return (wave % WN) * TileShape<WM, WN>::kWaveN + j * 32 + (lane & 31);
}

}  // namespace lce

// One 256x256 output tile of C[m][n] = sum_k A(m, k) B(n, k) on CDNA4 bf16 MFMA.
//
// Every contraction of the path is one of these, with each operand stored in
// global memory either K-contiguous ("row" m holds its K values contiguously)
// or K-major (row k holds 256+ consecutive m values contiguously):
//   logit tile (forward and backward recompute)  A = W_s rows, B = X rows, K = H,
//                                                both K-contiguous;
//   dX += G W_s       A = G [token][vocab] (K-contiguous), B = W_s [vocab][H] (K-major);
//   dW_s += G^T X     A = G [token][vocab] (K-major), B = X [token][H] (K-major).
// No operand is ever transposed in memory: K-major tiles are copied to LDS as
// they are, and the fragment reads transpose them (ds_read_tr16_b64).
//
// Workgroup: 512 threads = 8 waves, two per SIMD, arranged 2 (M) x 4 (N); each
// wave owns a 128 x 64 sub-tile held as 4 x 2 accumulators of the 32x32x16 bf16
// MFMA (128 fp32 per lane). Two waves per SIMD let one wave's LDS traffic and
// waits hide under the other's MFMAs.
//
// K advances 64 per stage through two LDS stages (A and B, 32 KB each, 128 KB
// total) filled by direct global->LDS 16-byte loads. Within a stage, the
// fragments of k-step s+1 are read from LDS while the MFMAs of k-step s run;
// the loads of the next stage are in flight during the whole stage.
//
// LDS layouts (one operand, one stage, 32 KB):
//  K-contiguous: 256 rows x 128 bytes (64 bf16 of K), as 16-byte chunks; chunk
//    kc of row r sits in slot kc ^ swz(r), so the 16-byte fragment reads of 8
//    (and 16) consecutive rows fall in distinct banks.
//  K-major: 64 rows (k) x 512 bytes (256 bf16 of m); 16-byte chunk c of row k
//    sits in slot c ^ kmaj_swz(k), so the four 32-byte row segments one 16-lane
//    group of a transposing read touches (rows k..k+3) fall in distinct banks.
#pragma once
#include "cdna4.hpp"

namespace lce {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kOpBytes = kBM * kBK * 2;      // one operand, one stage: 32 KB
constexpr int kStageBytes = 2 * kOpBytes;    // A + B
constexpr int kMainLds = 2 * kStageBytes;    // double-buffered: 128 KB

constexpr int kWM = 2, kWN = 4;              // wave grid over the tile
constexpr int kWaveM = kBM / kWM;            // 128
constexpr int kWaveN = kBN / kWN;            // 64
constexpr int kMI = kWaveM / 32;             // 4 accumulator rows of blocks
constexpr int kNI = kWaveN / 32;             // 2 accumulator columns of blocks

typedef f32x16 Acc[kMI][kNI];

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int kmaj_swz(int k) { return (2 * (k & 3)) ^ (8 * (k & 1)); }

// ---- global -> LDS loaders ------------------------------------------------
// Each wave issues 4 loads of 1 KB (64 lanes x 16 bytes) per operand and stage.

// K-contiguous operand: tile rows row0..row0+255 of a [rows][ld] bf16 matrix.
// Rows at or past rows_valid are clamped to the last valid row: they load real
// (finite) data whose results the epilogues discard or whose partner operand
// is zero there.
struct KContigLoader {
  const char* base;
  uint32_t off[4];

  __device__ __forceinline__ void init(const uint16_t* p, int ld, int row0, int rows_valid, int wave, int lane) {
    base = reinterpret_cast<const char*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wave * 32 + j * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ swz(r);
      const int gr = min(row0 + r, rows_valid - 1);
      off[j] = (uint32_t)gr * (uint32_t)ld * 2u + (uint32_t)kc * 16u;
    }
  }
  __device__ __forceinline__ void issue(int k0, LCE_LDS char* tile, int wave) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) g2lds16(base, off[j] + (uint32_t)k0 * 2u, tile + (wave * 4 + j) * 1024);
  }
};

// K-major operand: element (m, k) at p[k * ld + m]; the tile covers columns
// m0..m0+255 and rows k0..k0+63. Columns past m_valid (a multiple of 8) and
// rows past k_valid are clamped to the last valid ones.
struct KMajorLoader {
  const char* base;
  uint32_t ld2;       // row pitch in bytes
  uint32_t col[4];    // byte offset of this lane's 16-byte chunk within a row
  int row[4];         // tile row (k) this lane fills, per load
  int k_last;

  __device__ __forceinline__ void init(const uint16_t* p, int ld, int m0, int m_valid, int k_valid, int wave,
                                       int lane) {
    base = reinterpret_cast<const char*>(p);
    ld2 = (uint32_t)ld * 2u;
    k_last = k_valid - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = wave * 4 + j;           // 1 KB piece = tile rows 2q, 2q+1
      const int r = 2 * q + (lane >> 5);
      const int c = (lane & 31) ^ kmaj_swz(r);
      const int m = min(m0 + c * 8, m_valid - 8);
      row[j] = r;
      col[j] = (uint32_t)m * 2u;
    }
  }
  __device__ __forceinline__ void issue(int k0, LCE_LDS char* tile, int wave) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t kr = (uint32_t)min(k0 + row[j], k_last);
      g2lds16(base, kr * ld2 + col[j], tile + (wave * 4 + j) * 1024);
    }
  }
};

// ---- LDS -> register fragments --------------------------------------------
// Fragment of block i (32 rows of the wave's sub-tile) for k-step ks: lane l
// holds operand row (l % 32) and k = 16 ks + 8 (l / 32) + 0..7.

template <int NB>
struct KContigReader {
  int base;  // byte offset of this lane's row in the operand tile
  int sw;
  __device__ __forceinline__ void init(int wrow, int lane) {
    base = (wrow + (lane & 31)) * 128;
    sw = swz(lane & 31);
  }
  __device__ __forceinline__ void read(const LCE_LDS char* tile, int ks, int lane, bf16x8 (&f)[NB]) const {
    const int slot = ((ks * 2 + (lane >> 5)) ^ sw) * 16;
#pragma unroll
    for (int i = 0; i < NB; ++i) f[i] = *reinterpret_cast<const LCE_LDS bf16x8*>(tile + base + i * 4096 + slot);
  }
};

// Transposing read of a K-major tile. ds_read_tr16_b64 works on groups of 16
// lanes: each lane loads 4 consecutive bf16 and lane i of the group receives
// element (i % 4) of lanes 4q + i / 4, q = 0..3. A lane at position 4q + r of
// its group therefore loads row k = kbase + q, columns mbase + 4r .. +3, so
// that lane i receives column mbase + i at rows kbase .. kbase + 3; two such
// reads (k + 0..3, k + 4..7) make one 8-element fragment.
template <int NB>
struct KMajorReader {
  int off[NB];  // byte offset for k-step 0, first half
  __device__ __forceinline__ void init(int wrow, int lane) {
    const int q = (lane & 15) >> 2, r = lane & 3;
    const int k = 8 * (lane >> 5) + q;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int m = wrow + 32 * i + 16 * ((lane >> 4) & 1) + 4 * r;
      off[i] = k * 512 + (((m >> 3) ^ kmaj_swz(k)) << 4) + (m & 7) * 2;
    }
  }
  __device__ __forceinline__ void read(const LCE_LDS char* tile, int ks, int lane, bf16x8 (&f)[NB]) const {
    (void)lane;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      // rows k and k + 4 have the same (k & 3), so the same swizzle
      const bf16x4 lo = ds_read_tr16(tile + off[i] + ks * 16 * 512);
      const bf16x4 hi = ds_read_tr16(tile + off[i] + ks * 16 * 512 + 4 * 512);
      f[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
};

template <bool KMAJ, int NB>
struct ReaderFor {
  typedef KContigReader<NB> type;
};
template <int NB>
struct ReaderFor<true, NB> {
  typedef KMajorReader<NB> type;
};

template <int MI, int NI>
__device__ __forceinline__ void mma_step(Acc& acc, const bf16x8 (&a)[MI], const bf16x8 (&b)[NI]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
}

// Ask the scheduler to put one LDS read after each of the first n MFMAs of the
// step, then the remaining MFMAs.
// Ask the scheduler to spread NVM global->LDS loads and NDS LDS reads evenly
// over the NMFMA MFMAs of a k-step (masks: 0x008 MFMA, 0x020 global load,
// 0x100 LDS read).
template <int I, int NMFMA, int NVM, int NDS>
__device__ __forceinline__ void interleave_from() {
  if constexpr (I < NMFMA) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int nv = NVM / NMFMA + (I < NVM % NMFMA ? 1 : 0);
    constexpr int nd = NDS / NMFMA + (I < NDS % NMFMA ? 1 : 0);
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);
    if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nd, 0);
    interleave_from<I + 1, NMFMA, NVM, NDS>();
  }
}
template <int NMFMA, int NDS>
__device__ __forceinline__ void interleave_mfma_ds() {
  interleave_from<0, NMFMA, 0, NDS>();
}
template <int NMFMA, int NVM, int NDS>
__device__ __forceinline__ void interleave_mfma_vmem_ds() {
  interleave_from<0, NMFMA, NVM, NDS>();
}

// One stage (64 of K) of the main loop, branch-free so the scheduling
// barriers can interleave across the whole body. On entry the fragments of
// k-step 0 of this stage are in (a0, b0) and the stage's tiles are in LDS
// buffer kt & 1; the next stage's tiles are in flight into the other buffer.
// k-steps 0..2: read the next k-step's fragments while the MFMAs of the
// current one run. Then wait for the next stage's tiles and pass a barrier
// (after which no wave reads this stage's buffer again), and during k-step 3
// issue the loads of stage kt + 2 into this stage's buffer (kIssue) and read
// k-step 0 of the next stage (kNext).
template <bool A_KMAJ, bool B_KMAJ, bool kIssue, bool kNext, class LA, class LB, class RA, class RB>
__device__ __forceinline__ void mainloop_stage(int kt, const LA& la, const LB& lb, const RA& ra, const RB& rb,
                                               LCE_LDS char* lds, int wave, int lane, Acc& acc, bf16x8 (&a0)[kMI],
                                               bf16x8 (&b0)[kNI], bf16x8 (&a1)[kMI], bf16x8 (&b1)[kNI]) {
  constexpr int kReads = (A_KMAJ ? 2 : 1) * kMI + (B_KMAJ ? 2 : 1) * kNI;
  constexpr int kLoads = 8;  // global->LDS loads per wave per stage
  LCE_LDS char* cur = lds + (kt & 1) * kStageBytes;
  LCE_LDS char* nxt = lds + ((kt + 1) & 1) * kStageBytes;
  ra.read(cur, 1, lane, a1);
  rb.read(cur + kOpBytes, 1, lane, b1);
  mma_step<kMI, kNI>(acc, a0, b0);
  interleave_mfma_ds<kMI * kNI, kReads>();
  ra.read(cur, 2, lane, a0);
  rb.read(cur + kOpBytes, 2, lane, b0);
  mma_step<kMI, kNI>(acc, a1, b1);
  interleave_mfma_ds<kMI * kNI, kReads>();
  ra.read(cur, 3, lane, a1);
  rb.read(cur + kOpBytes, 3, lane, b1);
  mma_step<kMI, kNI>(acc, a0, b0);
  interleave_mfma_ds<kMI * kNI, kReads>();
  wait_vm0();
  wait_lgkm0();
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  if (kIssue) {
    la.issue((kt + 2) * kBK, cur, wave);
    lb.issue((kt + 2) * kBK, cur + kOpBytes, wave);
  }
  if (kNext) {
    ra.read(nxt, 0, lane, a0);
    rb.read(nxt + kOpBytes, 0, lane, b0);
  }
  mma_step<kMI, kNI>(acc, a1, b1);
  if (kIssue && kNext) {
    interleave_mfma_vmem_ds<kMI * kNI, kLoads, kReads>();
  } else if (kNext) {
    interleave_mfma_ds<kMI * kNI, kReads>();
  }
}

// Issues the loads of the first two stages of a tile (one if K = 64). A caller
// that has a next tile can issue them as soon as the previous tile_mainloop
// returned (both LDS stages are then free) and do other work, such as an
// epilogue, while they fly; it then passes kIssued = true.
template <class LA, class LB>
__device__ __forceinline__ void tile_prologue(const LA& la, const LB& lb, int K, LCE_LDS char* lds) {
  const int wave = wave_id();
  la.issue(0, lds, wave);
  lb.issue(0, lds + kOpBytes, wave);
  if (K > kBK) {
    la.issue(kBK, lds + kStageBytes, wave);
    lb.issue(kBK, lds + kStageBytes + kOpBytes, wave);
  }
}

// Full K loop for one tile (K a positive multiple of 64). The accumulators are
// zeroed here. With kIssued the first stages were issued by tile_prologue and
// the wave has issued no other memory operation since. On return every wave
// has passed a barrier after its last LDS read and no load into LDS is in
// flight, so both LDS stages are free for the caller.
template <bool A_KMAJ, bool B_KMAJ, bool kIssued = false, class LA, class LB>
__device__ __forceinline__ void tile_mainloop(const LA& la, const LB& lb, int K, LCE_LDS char* lds, Acc& acc) {
  const int wave = wave_id();
  const int lane = lane_id();
  const int wm = wave / kWN, wn = wave % kWN;
  typename ReaderFor<A_KMAJ, kMI>::type ra;
  typename ReaderFor<B_KMAJ, kNI>::type rb;
  ra.init(wm * kWaveM, lane);
  rb.init(wn * kWaveN, lane);
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j) acc[i][j] = f32x16{};
  const int kt_n = K / kBK;
  if (!kIssued) tile_prologue(la, lb, K, lds);
  if (kt_n > 1)
    wait_vm<8>();  // stage 0 landed (the 8 loads of stage 1 may still fly)
  else
    wait_vm0();
  __syncthreads();
  bf16x8 a0[kMI], b0[kNI], a1[kMI], b1[kNI];
  ra.read(lds, 0, lane, a0);
  rb.read(lds + kOpBytes, 0, lane, b0);
  int kt = 0;
  for (; kt < kt_n - 2; ++kt)
    mainloop_stage<A_KMAJ, B_KMAJ, true, true>(kt, la, lb, ra, rb, lds, wave, lane, acc, a0, b0, a1, b1);
  if (kt_n >= 2)
    mainloop_stage<A_KMAJ, B_KMAJ, false, true>(kt_n - 2, la, lb, ra, rb, lds, wave, lane, acc, a0, b0, a1, b1);
  mainloop_stage<A_KMAJ, B_KMAJ, false, false>(kt_n - 1, la, lb, ra, rb, lds, wave, lane, acc, a0, b0, a1, b1);
}

// Tile (r, c) of workgroup b within a problem of rows x cols tiles occupying
// workgroups [0, rows * cols) of a launch. The hardware hands workgroups to the
// eight XCDs round-robin (b % 8), and each XCD has its own L2. Here each XCD
// gets a contiguous run of the tile order, which walks bands of kBand rows
// column by column, so the 32 workgroups an XCD runs at once cover a
// kBand x 8 rectangle and share 4 + 8 operand tiles instead of up to 64.
constexpr int kBand = 4;
__device__ __forceinline__ void xcd_tile(int b, int rows, int cols, int& r, int& c) {
  const int n = rows * cols;
  const int x = b & 7, l = b >> 3;
  const int q = n >> 3, rem = n & 7;
  const int t = x * q + min(x, rem) + l;
  const int band = t / (kBand * cols);
  const int r0 = band * kBand;
  const int h = min(rows - r0, kBand);
  const int w = t - band * kBand * cols;
  r = r0 + w % h;
  c = w / h;
}

// Row / column (within the 256x256 tile) of accumulator element e of block (i, j).
__device__ __forceinline__ int acc_row(int wave, int lane, int i, int e) {
  return (wave / kWN) * kWaveM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
__device__ __forceinline__ int acc_col(int wave, int lane, int j) {
  return (wave % kWN) * kWaveN + j * 32 + (lane & 31);
}

}  // namespace lce

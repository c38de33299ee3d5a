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
// wave owns a 128 x 64 sub-tile held as 8 x 4 accumulators of the 16x16x32 bf16
// MFMA (128 fp32 per lane). Two waves per SIMD let one wave's LDS traffic and
// waits hide under the other's MFMAs. The 16x16x32 shape does the same work
// per LDS byte as 32x32x16 here but draws less power per flop, and this chip
// reaches its power limit before its peak clock on dense bf16 work.
//
// K advances 64 per stage (two k-steps of 32) through two LDS stages (A and B,
// 32 KB each, 128 KB total) filled by direct global->LDS 16-byte loads. The
// fragments of k-step 1 are read from LDS while the MFMAs of k-step 0 run, and
// those of the next stage's k-step 0 while the MFMAs of k-step 1 run; the
// loads of the next stage are in flight during the whole stage.
//
// LDS layouts (one operand, one stage, 32 KB):
//  K-contiguous: 256 rows x 128 bytes (64 bf16 of K), as 16-byte chunks; chunk
//    kc of row r sits in slot kc ^ swz(r). A fragment read has lane l read
//    chunk 4 ks + l / 16 of row l % 16 (of a 16-row block). The LDS serves a
//    16-byte read in four passes of 256 bytes (64 banks); the bank counters
//    show that lanes l and l + 32 share a pass (eight lanes from each half).
//    swz permutes row bits 1..3 into slot bits 0..2 so that both the 16
//    consecutive lanes and the 8 + 8 lanes of a pass fall in distinct banks:
//    the even (and the odd) rows of a 16-row block get 8 different swizzles,
//    and rows 0, 2, 4, 6 (or 8, 10, 12, 14) get swizzles that stay distinct
//    after XOR with 2, the chunk difference between lanes l and l + 32.
//  K-major: 64 rows (k) x 512 bytes (256 bf16 of m); 16-byte chunk c of row k
//    sits in slot c ^ kmaj_swz(k). A transposing read has 16-lane group g read
//    rows 8 g + 0..3 (then + 4..7), 32 bytes each. kmaj_swz spreads the four
//    rows of a group over distinct banks, and its bit-3/bit-4 term moves groups
//    g and g ^ 1, and g and g ^ 2, onto the complementary banks, so that a
//    pass of 32 lanes (either lanes 0-31, or l and l + 32) is conflict-free
//    too.
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
constexpr int kBlk = 16;                     // MFMA block edge
constexpr int kKStep = 32;                   // K per MFMA
constexpr int kMI = kWaveM / kBlk;           // 8 accumulator rows of blocks
constexpr int kNI = kWaveN / kBlk;           // 4 accumulator columns of blocks

typedef f32x4 Acc[kMI][kNI];

__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 1) | ((r >> 2) & 2) | (r & 4); }
__device__ __forceinline__ int kmaj_swz(int k) { return (2 * (k & 3)) ^ (8 * (k & 1)) ^ (2 * (((k >> 3) ^ (k >> 4)) & 1)); }

// ---- global -> LDS loaders ------------------------------------------------
// Only the first kLoadWaves waves (one per SIMD) issue a stage's loads, kLoadJ
// loads of 1 KB (64 lanes x 16 bytes) per operand each. After a stage barrier
// the other wave on each SIMD starts its MFMAs at once while the loading wave
// issues, so the MFMA pipe does not sit idle behind the issue of the loads;
// the skew this leaves between the two waves of a SIMD is absorbed at the next
// barrier, where the late wave's MFMAs keep the pipe busy.
constexpr int kLoadWaves = 4;
constexpr int kLoadJ = (kOpBytes / 1024) / kLoadWaves;  // 8

// K-contiguous operand: tile rows row0..row0+255 of a [rows][ld] bf16 matrix.
// Rows at or past rows_valid are clamped to the last valid row: they load real
// (finite) data whose results the epilogues discard or whose partner operand
// is zero there. Load j of loading wave w fills tile rows 64 w + 8 j + lane / 8;
// the per-lane state is two registers, and each load's address is formed when
// it is issued (a few VALU per 16-byte load), which keeps the main loop's
// register footprint small.
struct KContigLoader {
  const char* base;
  uint32_t ld2;   // row pitch in bytes
  int row;        // this lane's row for load 0 (absolute)
  int last;       // last valid row
  uint32_t kc16;  // byte offset of this lane's chunk for even j (odd j: ^ 32)

  __device__ __forceinline__ void init(const uint16_t* p, int ld, int row0, int rows_valid, int wave, int lane) {
    base = reinterpret_cast<const char*>(p);
    ld2 = (uint32_t)ld * 2u;
    row = row0 + wave * (8 * kLoadJ) + (lane >> 3);
    last = rows_valid - 1;
    // chunk (lane & 7) of row r sits in slot (lane & 7) ^ swz(r); these rows
    // have r % 16 = 8 (j & 1) + lane / 8, so swz(r) = swz(lane / 8) ^ 2 (j & 1)
    kc16 = (uint32_t)(((lane & 7) ^ swz(lane >> 3)) * 16);
  }
  // kOpaque: the row goes through an empty asm first, so that the kLoadJ
  // addresses are formed at each issue instead of being hoisted out of the
  // main loop as invariants. Hoisting saves VALU but holds 8 registers per
  // loader across the loop, which the forward (running state per token in
  // registers) cannot spare.
  template <bool kOpaque = false>
  __device__ __forceinline__ void issue(int k0, LCE_LDS char* tile, int wave) const {
    if (wave >= kLoadWaves) return;
    int r = row;
    if (kOpaque) asm volatile("" : "+v"(r));
#pragma unroll
    for (int j = 0; j < kLoadJ; ++j) {
      const uint32_t gr = (uint32_t)min(r + 8 * j, last);
      g2lds16(base, gr * ld2 + (kc16 ^ (32u * (j & 1))) + (uint32_t)k0 * 2u, tile + (wave * kLoadJ + j) * 1024);
    }
  }
};

// K-major operand: element (m, k) at p[k * ld + m]; the tile covers columns
// m0..m0+255 and rows k0..k0+63. Columns past m_valid (a multiple of 8) and
// rows past k_valid are clamped to the last valid ones. Load j of loading wave
// w fills tile rows 2 q and 2 q + 1 (lanes 0-31 and 32-63), 16 bytes per lane,
// q = 4 w + (j & 3) + 16 (j >> 2): the wave's rows are 8 w .. 8 w + 7 and
// 32 + 8 w .. 32 + 8 w + 7, which share bits 3 and 4 of the row, so kmaj_swz
// of a lane's row takes only two values (by j & 1).
struct KMajorLoader {
  const char* base;
  uint32_t ld2;       // row pitch in bytes
  uint32_t col[2];    // byte offset of this lane's chunk within a row, for even / odd j
  int row;            // tile row (k) this lane fills for load 0
  int k_last;

  __device__ __forceinline__ void init(const uint16_t* p, int ld, int m0, int m_valid, int k_valid, int wave,
                                       int lane) {
    base = reinterpret_cast<const char*>(p);
    ld2 = (uint32_t)ld * 2u;
    k_last = k_valid - 1;
    static_assert(kLoadWaves == 4 && kLoadJ == 8, "row assignment written for 4 loading waves x 8 loads");
    row = 8 * wave + (lane >> 5);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = row + 2 * h;             // same row bits 0, 1, 3, 4 as the rows of loads with j & 1 = h
      const int c = (lane & 31) ^ kmaj_swz(r);
      col[h] = (uint32_t)min(m0 + c * 8, m_valid - 8) * 2u;
    }
  }
  template <bool kOpaque = false>
  __device__ __forceinline__ void issue(int k0, LCE_LDS char* tile, int wave) const {
    if (wave >= kLoadWaves) return;
    int r = row;  // kOpaque: as in KContigLoader::issue
    if (kOpaque) asm volatile("" : "+v"(r));
#pragma unroll
    for (int j = 0; j < kLoadJ; ++j) {
      const uint32_t kr = (uint32_t)min(k0 + r + 2 * (j & 3) + 32 * (j >> 2), k_last);
      g2lds16(base, kr * ld2 + col[j & 1], tile + (4 * wave + (j & 3) + 16 * (j >> 2)) * 1024);
    }
  }
};

// ---- LDS -> register fragments --------------------------------------------
// Fragment of block i (16 rows of the wave's sub-tile) for k-step ks: lane l
// holds operand row (l % 16) and k = 32 ks + 8 (l / 16) + 0..7.

template <int NB>
struct KContigReader {
  int base;  // byte offset of this lane's row in the operand tile
  int sw;
  __device__ __forceinline__ void init(int wrow, int lane) {
    base = (wrow + (lane & 15)) * 128;
    sw = swz(lane & 15);  // wrow + 16 i adds nothing to the low four row bits
  }
  __device__ __forceinline__ void read(const LCE_LDS char* tile, int ks, int lane, bf16x8 (&f)[NB]) const {
    read_range<0, NB>(tile, ks, lane, f);
  }
  // fragments [I0, I1) into f[0 .. I1 - I0) (f may be shorter than NB)
  template <int I0, int I1, int NF>
  __device__ __forceinline__ void read_range(const LCE_LDS char* tile, int ks, int lane, bf16x8 (&f)[NF]) const {
    static_assert(I1 - I0 <= NF && I1 <= NB, "fragment range");
    const int slot = ((ks * 4 + (lane >> 4)) ^ sw) * 16;
#pragma unroll
    for (int i = I0; i < I1; ++i)
      f[i - I0] = *reinterpret_cast<const LCE_LDS bf16x8*>(tile + base + i * kBlk * 128 + slot);
  }
};

// Transposing read of a K-major tile. ds_read_tr16_b64 works on groups of 16
// lanes: each lane loads 4 consecutive bf16 and lane i of the group receives
// element (i % 4) of lanes 4q + i / 4, q = 0..3. A lane at position 4q + r of
// group g = l / 16 therefore loads row k = 8 g + q, columns mbase + 4r .. +3, so
// that lane i of the group receives column mbase + i at rows 8 g .. 8 g + 3; two
// such reads (rows + 0..3, + 4..7) make the 8-element fragment of k-group g.
template <int NB>
struct KMajorReader {
  int off[NB];  // byte offset for k-step 0, first half
  __device__ __forceinline__ void init(int wrow, int lane) {
    const int q = (lane & 15) >> 2, r = lane & 3;
    const int k = 8 * (lane >> 4) + q;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int m = wrow + kBlk * i + 4 * r;
      off[i] = k * 512 + (((m >> 3) ^ kmaj_swz(k)) << 4) + (m & 7) * 2;
    }
  }
  __device__ __forceinline__ void read(const LCE_LDS char* tile, int ks, int lane, bf16x8 (&f)[NB]) const {
    read_range<0, NB>(tile, ks, lane, f);
  }
  // fragments [I0, I1) into f[0 .. I1 - I0) (f may be shorter than NB)
  template <int I0, int I1, int NF>
  __device__ __forceinline__ void read_range(const LCE_LDS char* tile, int ks, int lane, bf16x8 (&f)[NF]) const {
    static_assert(I1 - I0 <= NF && I1 <= NB, "fragment range");
    (void)lane;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      // rows k, k + 4 and k + 32 ks share bits 0, 1, 3 and 4 (k % 8 < 4), so
      // the same swizzle
      const bf16x4 lo = ds_read_tr16(tile + off[i] + ks * kKStep * 512);
      const bf16x4 hi = ds_read_tr16(tile + off[i] + ks * kKStep * 512 + 4 * 512);
      f[i - I0] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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
    for (int j = 0; j < NI; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
}

// Ask the scheduler for the order of one k-step (masks: 0x008 MFMA, 0x100 LDS
// read): after MFMA t, X(t) of the next k-step's fragment reads, where the
// reads are issued in source order. mma_step runs j fastest, so MFMA 4 i + 3
// is the last one that uses A fragment i; a read that refills A fragment i
// must not be issued before it, or its register could not be reused.
//  kSteady: the B reads (NB) one per MFMA from the start, then the AR reads of
//    A fragment i after MFMA 4 i + 3. Source order: B, then A by block.
//  !kSteady (before a barrier): the same, but the reads of A fragments 6 and 7
//    go into spare registers right after the B reads, so that the last refill
//    (fragment 5) follows MFMA 23 and its latency is hidden before the barrier
//    at the end of the k-step. Source order: B, A6, A7, then A0 .. A5.
// In both cases each read lands at or after its planned MFMA, never before.
template <int I, int NMFMA, int NB, int AR, bool kSteady>
__device__ __forceinline__ void interleave_from() {
  if constexpr (I < NMFMA) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int early = kSteady ? NB : NB + 2 * AR;
    constexpr int last_refill = kSteady ? kMI - 1 : kMI - 3;
    constexpr int nd = (I < early ? 1 : 0) + (I % kNI == kNI - 1 && I / kNI <= last_refill ? AR : 0);
    if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nd, 0);
    interleave_from<I + 1, NMFMA, NB, AR, kSteady>();
  }
}

// One stage (64 of K) of the main loop. On entry the fragments of k-step 0 of
// this stage are in (a, b0) and the stage's tiles are in LDS buffer kt & 1;
// the next stage's tiles are in flight into the other buffer. k-step 0: read
// k-step 1's fragments into (a, b1) while its MFMAs run (fragments 6 and 7 of
// A via a6, a7). Then wait for the next stage's tiles and pass a barrier
// (after which no wave reads this stage's buffer again), issue the loads of
// stage kt + 2 into this stage's buffer (if there is one), and during k-step 1
// read k-step 0 of the next stage into (a, b0). The last stage reads the other
// buffer too, whatever it holds then (the values are never used): keeping
// those reads unconditional keeps them in the same basic block as the MFMAs
// they interleave with.
template <bool A_KMAJ, bool B_KMAJ, bool kOpaque, class LA, class LB, class RA, class RB>
__device__ __forceinline__ void mainloop_stage(int kt, int kt_n, const LA& la, const LB& lb, const RA& ra,
                                               const RB& rb, LCE_LDS char* lds, int wave, int lane, Acc& acc,
                                               bf16x8 (&a)[kMI], bf16x8 (&b0)[kNI], bf16x8 (&b1)[kNI]) {
  constexpr int kAR = A_KMAJ ? 2 : 1;            // LDS reads per A fragment
  constexpr int kBR = (B_KMAJ ? 2 : 1) * kNI;    // LDS reads of the B fragments
  LCE_LDS char* cur = lds + (kt & 1) * kStageBytes;
  LCE_LDS char* nxt = lds + ((kt + 1) & 1) * kStageBytes;
  static_assert(kBK == 2 * kKStep, "two k-steps per stage");
  static_assert(kMI == 8 && kNI == 4, "read schedule written for 8 x 4 blocks");
  mma_step<kMI, kNI>(acc, a, b0);
  rb.read(cur + kOpBytes, 1, lane, b1);
  bf16x8 a67[2];
  ra.template read_range<6, 8>(cur, 1, lane, a67);
  ra.template read_range<0, 6>(cur, 1, lane, a);
  interleave_from<0, kMI * kNI, kBR, kAR, false>();
  __builtin_amdgcn_sched_barrier(0);  // all of k-step 0 before the barrier
  a[6] = a67[0];
  a[7] = a67[1];
  wait_vm0();
  wait_lgkm0();
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  if (kt + 2 < kt_n) {
    la.template issue<kOpaque>((kt + 2) * kBK, cur, wave);
    lb.template issue<kOpaque>((kt + 2) * kBK, cur + kOpBytes, wave);
  }
  mma_step<kMI, kNI>(acc, a, b1);
  rb.read(nxt + kOpBytes, 0, lane, b0);
  ra.read(nxt, 0, lane, a);
  interleave_from<0, kMI * kNI, kBR, kAR, true>();
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
// has passed a barrier after its last LDS read whose value is used, and no
// load into LDS is in flight, so both LDS stages are free for the caller (the
// discarded reads of the last stage may still be in flight: they read, never
// write, and nothing uses what they return).
//
// idle (uniform over the wave): the caller discards every row of this wave's
// 128 x 64 sub-tile (a tile past the end of A's valid rows, such as a shard's
// last vocabulary tile with at most 128 live rows, in the waves with wm = 1).
// Such a wave reads no fragments and issues no MFMA; its accumulators stay
// zero, and it passes the same barriers as the others (one before the loop,
// one per stage). Only waves with wm = 1 may be idle, and those never issue
// loads (the loading waves are waves 0 .. kLoadWaves - 1, all with wm = 0).
template <bool A_KMAJ, bool B_KMAJ, bool kIssued = false, bool kOpaque = false, class LA, class LB>
__device__ __forceinline__ void tile_mainloop(const LA& la, const LB& lb, int K, LCE_LDS char* lds, Acc& acc,
                                              bool idle = false) {
  static_assert(kLoadWaves <= kWN, "loading waves must all have wm = 0");
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
    for (int j = 0; j < kNI; ++j) acc[i][j] = f32x4{};
  const int kt_n = K / kBK;
  if (!kIssued) tile_prologue(la, lb, K, lds);
  // a scalar branch (the condition is made uniform explicitly), so a wave that
  // does not take it never runs these barriers with its lanes masked off
  if (__builtin_amdgcn_readfirstlane(idle && wm == 1 ? 1 : 0)) {
    for (int kt = 0; kt <= kt_n; ++kt) __syncthreads();
    return;
  }
  if (kt_n > 1)
    wait_vm<2 * kLoadJ>();  // stage 0 landed (the loads of stage 1 may still fly)
  else
    wait_vm0();
  __syncthreads();
  bf16x8 a[kMI], b0[kNI], b1[kNI];
  ra.read(lds, 0, lane, a);
  rb.read(lds + kOpBytes, 0, lane, b0);
  // one loop body (no peeled last stages): it keeps the register allocation
  // within the 256 registers of a wave without spills
  for (int kt = 0; kt < kt_n; ++kt)
    mainloop_stage<A_KMAJ, B_KMAJ, kOpaque>(kt, kt_n, la, lb, ra, rb, lds, wave, lane, acc, a, b0, b1);
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
  return (wave / kWN) * kWaveM + i * kBlk + 4 * (lane >> 4) + e;
}
__device__ __forceinline__ int acc_col(int wave, int lane, int j) {
  return (wave % kWN) * kWaveN + j * kBlk + (lane & 15);
}

}  // namespace lce

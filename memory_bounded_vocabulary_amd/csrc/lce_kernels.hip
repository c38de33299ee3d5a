// HIP kernels (gfx950) for the memory-bounded vocabulary projection +
// cross-entropy, and the host-side launchers the C ABI calls.
//
// Method: "Flattening Every Memory Peak in Long-Context Mixture-of-Experts
// Training", section 3.2 (Ring-DTP). One vocabulary shard per round; its
// logit tiles update a per-token running (max m, exp-sum z) by the online
// softmax rule (Eq. 3) and are never stored. loss_i = lse_i - y_{t_i} with
// lse_i = m_i + log z_i; the backward rebuilds each logit tile from X, W and
// the stored lse.
#include <hip/hip_runtime.h>

#include "lce_internal.hpp"
#include "tile_gemm.hpp"

namespace lce {

// --------------------------------------------------------------------------
// Forward round: fold X W_s^T into the running per-token state.
//
// The logit tile is computed transposed, W_s rows (vocabulary) x X rows
// (tokens), so that in the MFMA accumulator layout each lane owns whole token
// columns: lane l of wave (wm, wn) holds tokens wn*64 + 16 j + l % 16
// (j = 0..3) and, for each, 32 of the tile's 256 vocabulary rows. The online
// (m, z) of a token (log2 domain) therefore lives in two registers per lane
// and token and the fold needs no cross-lane traffic until the end of the
// round.
//
// A launch covers rounds [k_begin, k_end) (round k meets shards.p[k], the
// shard a ring would deliver then; the host permutes the table into ring
// order). Grid: token blocks x S splits, in the XCD-grouped order of xcd_tile.
// Workgroup (tb, s) owns tokens [256 tb, 256 tb + 256) and, in each of its
// rounds, the shard's vocabulary tiles [s*tps, min((s+1)*tps, n_vtiles)),
// keeping (m, z) in registers across them; while it folds a tile, the first
// two LDS stages of its next tile are already loading. At the end its (m, z)
// per token is merged into state[s][token] after the earlier launches' (one
// writer per entry per launch, launches ordered on the stream: no atomics on
// data). When the grid fits on the CUs at once, one launch covers all rounds;
// otherwise one launch per round keeps every CU on the same shard, which then
// stays in the caches. The split states are merged by finalize_kernel after
// the last round's launch.
// --------------------------------------------------------------------------
__device__ __forceinline__ void fold_full(const Acc& acc, float (&m)[kNI], float (&z)[kNI]) {
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    float mx = acc[0][j][0];
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, acc[i][j][e]);
    const float mn = fmaxf(m[j], mx * kLog2e);
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += fast_exp2(fmaf(acc[i][j][e], kLog2e, -mn));
    z[j] = fmaf(z[j], fast_exp2(m[j] - mn), (s[0] + s[1]) + (s[2] + s[3]));
    m[j] = mn;
  }
}

// Same, for a shard's last tile: vocabulary rows at or past `live` (relative
// to this lane's first row) act as -infinity.
__device__ __forceinline__ void fold_masked(const Acc& acc, float (&m)[kNI], float (&z)[kNI], int live) {
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    float v[kMI][4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = kBlk * i + e;
        v[i][e] = r < live ? acc[i][j][e] : -__builtin_inff();
        mx = fmaxf(mx, v[i][e]);
      }
    const float mn = fmaxf(m[j], mx * kLog2e);
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += fast_exp2(fmaf(v[i][e], kLog2e, -mn));
    z[j] = fmaf(z[j], fast_exp2(m[j] - mn), (s[0] + s[1]) + (s[2] + s[3]));
    m[j] = mn;
  }
}

// The target logit: tile row r_lane + 16 i + e of column j is held by this lane
// (r_lane = the lane's first row, 4 (lane / 16) within its wave's 128 rows).
// rel[j] is the target's row relative to the wave's first row; the wave's
// rows that belong to the shard are [0, wave_live) (a shard's last tile is
// padded past its rows, and those padding rows must not be taken for the
// next shard's ids). Each target that lies in the tile sits in exactly one
// lane, which writes it out; the test is uniform over the wave, so waves
// without a target skip the selection.
__device__ __forceinline__ void capture_target(const Acc& acc, const int (&rel)[kNI], int wave_live, int lane,
                                               float* __restrict__ yt, int row0) {
  bool mine[kNI];
  bool any = false;
  const int lim = min(kWaveM, wave_live);
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    mine[j] = rel[j] >= 0 && rel[j] < lim && ((rel[j] >> 2) & 3) == (lane >> 4);
    any |= mine[j];
  }
  if (!__any(any)) return;
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    if (!mine[j]) continue;
    const int ii = rel[j] >> 4, ee = rel[j] & 3;
    float y = 0.0f;
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) y = (i == ii && e == ee) ? acc[i][j][e] : y;
    yt[row0 + kBlk * j + (lane & 15)] = y;
  }
}

// Fixed-order tree sum over the first 256 threads of a block (deterministic).
__device__ __forceinline__ void block_sum256(double& a, long long& b, double* sa, long long* sb) {
  const int t = threadIdx.x;
  if (t < 256) {
    sa[t] = a;
    sb[t] = b;
  }
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      sa[t] += sa[t + w];
      sb[t] += sb[t + w];
    }
    __syncthreads();
  }
  a = sa[0];
  b = sb[0];
}

// A workgroup's end: merge the lanes' and waves' (m, z) of its 256 tokens and
// merge that into state[split][token] (after the earlier rounds').
__device__ __forceinline__ void fwd_finish_item(const FwdArgs& a, int tb, int split, const float (&m_in)[kNI],
                                               const float (&z_in)[kNI], int first, char* lds_raw) {
  const int wave = wave_id();
  const int lane = lane_id();
  const int wm = wave / kWN, wn = wave % kWN;
  float m[kNI], z[kNI];
  // lanes l, l ^ 16, l ^ 32 and l ^ 48 hold the same tokens (different
  // vocabulary rows)
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    m[j] = m_in[j];
    z[j] = z_in[j];
#pragma unroll
    for (int x = 16; x <= 32; x *= 2) {
      const float m2 = __shfl_xor(m[j], x);
      const float z2 = __shfl_xor(z[j], x);
      lse_merge(m[j], z[j], m2, z2);
    }
  }
  // waves wm = 1 hand their tokens' state to waves wm = 0 (LDS is free: the
  // main loop ended on a barrier and no load is in flight)
  __syncthreads();
  float2* red = reinterpret_cast<float2*>(lds_raw);
  if (wm == 1 && lane < kBlk) {
#pragma unroll
    for (int j = 0; j < kNI; ++j) red[wn * kWaveN + kBlk * j + lane] = make_float2(m[j], z[j]);
  }
  __syncthreads();
  if (wm == 0 && lane < kBlk) {
#pragma unroll
    for (int j = 0; j < kNI; ++j) {
      const float2 o = red[wn * kWaveN + kBlk * j + lane];
      float M = m[j], Z = z[j];
      lse_merge(M, Z, o.x, o.y);
      const int row = tb * kBN + wn * kWaveN + kBlk * j + lane;
      if (row < a.N) {
        float2* sp = a.state + (size_t)split * a.state_ld + row;
        if (!first) {  // earlier rounds come first in the merge
          const float2 p = *sp;
          float M0 = p.x, Z0 = p.y;
          lse_merge(M0, Z0, M, Z);
          M = M0;
          Z = Z0;
        }
        *sp = make_float2(M, Z);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void fwd_round_kernel(FwdArgs a, ShardTable shards, int k_begin,
                                                                int k_end, int first) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kMainLds];
  __shared__ int tgt[kBN];  // the targets of this block's tokens (-1: none)
  LCE_LDS char* lds = (LCE_LDS char*)lds_raw;
  const int wave = wave_id();
  const int lane = lane_id();
  const int wm = wave / kWN, wn = wave % kWN;
  int tb, split;
  xcd_tile(blockIdx.x, a.token_blocks, a.S, tb, split);
  const int t0 = split * a.tiles_per_split;
  const int n_my = min(t0 + a.tiles_per_split, a.n_vtiles) - t0;  // tiles per shard
  const int n_all = (k_end - k_begin) * n_my;
  if (threadIdx.x < kBN) {  // read before the first tile's epilogue (the main loop passes barriers)
    const int row = tb * kBN + threadIdx.x;
    const int t = row < a.N ? a.targets[row] : -1;
    // ignored and out-of-range targets are never captured (their yt stays 0 / NaN)
    tgt[threadIdx.x] = (t == a.ignore_index || t < 0 || t >= a.Vs * a.P) ? -1 : t;
  }
  const int row0 = tb * kBN + wn * kWaveN;  // first token of this wave's columns

  float m[kNI], z[kNI];
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    m[j] = kNegBig;
    z[j] = 0.0f;
  }
  const int lane_row = wm * kWaveM + 4 * (lane >> 4);  // first vocabulary row of this lane in a tile
  KContigLoader lx, lw;
  lx.init(a.X, a.H, tb * kBN, a.N, wave, lane);
  lw.init(shards.p[k_begin], a.H, t0 * kBM, a.Vs, wave, lane);
  tile_prologue(lw, lx, a.H, lds);
  for (int i = 0; i < n_all; ++i) {
    const int vt = t0 + i % n_my;
    Acc acc;
    // a shard's last tile with at most 128 live rows gets its own copy of the
    // loop, in which the waves of rows 128-255 skip the MFMAs
    if (__builtin_amdgcn_readfirstlane(a.Vs - vt * kBM <= kWaveM ? 1 : 0))
      tile_mainloop<false, false, true, true>(lw, lx, a.H, lds, acc, true);
    else
      tile_mainloop<false, false, true, true>(lw, lx, a.H, lds, acc);
    if (i + 1 < n_all) {  // the next tile's first stages load while this one folds
      lw.init(shards.p[k_begin + (i + 1) / n_my], a.H, (t0 + (i + 1) % n_my) * kBM, a.Vs, wave, lane);
      tile_prologue(lw, lx, a.H, lds);
    }
    const int live = a.Vs - vt * kBM;
    // the target logits that lie in this tile (vocabulary rows of this wave:
    // from the shard's id, the tile and the wave's half)
    const int wave_v0 = shards.id[k_begin + i / n_my] * a.Vs + vt * kBM + wm * kWaveM;
    int rel[kNI];
#pragma unroll
    for (int j = 0; j < kNI; ++j) {
      const int t = tgt[wn * kWaveN + kBlk * j + (lane & 15)];
      rel[j] = t < 0 ? -1 : t - wave_v0;
    }
    capture_target(acc, rel, live - wm * kWaveM, lane, a.yt, row0);
    if (live >= kBM)
      fold_full(acc, m, z);
    else
      fold_masked(acc, m, z, live - lane_row);
  }
  fwd_finish_item(a, tb, split, m, z, first, lds_raw);
}

// --------------------------------------------------------------------------
// Before the first round: yt = 0 for ignored tokens, NaN for the others.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void init_target_logits_kernel(const int* __restrict__ targets, int N,
                                                                 int ignore_index, float* __restrict__ yt) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row < N) yt[row] = targets[row] == ignore_index ? 0.0f : __builtin_nanf("");
}

// --------------------------------------------------------------------------
// Backward preparation (one workgroup of 1024 threads): count the tokens whose
// target is not ignore_index, decide whether leaving the others out saves a
// 256-token tile (compact mode), and write the token info of every position
// the backward runs over, kept tokens in ascending order. Thread t owns a run
// of consecutive tokens; a block-wide prefix sum of the runs' counts gives
// each thread its first position. The loss scale g = dloss / n_valid (mean)
// or dloss (sum) is formed here, on the device, so dloss can come straight
// from autograd; with reduction "none" each token carries its own dloss.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void bwd_prep_kernel(const int* __restrict__ targets,
                                                        const float* __restrict__ lse, int N, int ignore_index,
                                                        const float* __restrict__ dloss, int reduction,
                                                        int allow_compact, BwdPrep* __restrict__ prep,
                                                        TokInfo* __restrict__ tinfo) {
  __shared__ int wave_base[16];
  __shared__ int s_total;
  const int t = threadIdx.x;
  const int lane = lane_id(), wave = t >> 6;
  const int per = (((N + 1023) >> 10) + 3) & ~3;  // tokens per thread, a multiple of 4
  const int r0 = min(t * per, N), r1 = min(r0 + per, N);
  int cnt = 0;
  int r = r0;
  for (; r + 4 <= r1; r += 4) {
    const int4 v = *reinterpret_cast<const int4*>(targets + r);  // r0 is a multiple of 4: aligned
    cnt += (v.x != ignore_index) + (v.y != ignore_index) + (v.z != ignore_index) + (v.w != ignore_index);
  }
  for (; r < r1; ++r) cnt += targets[r] != ignore_index;
  int incl = cnt;  // inclusive prefix sum over the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_base[wave] = incl;
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int w = 0; w < 16; ++w) {
      const int v = wave_base[w];
      wave_base[w] = acc;
      acc += v;
    }
    s_total = acc;
  }
  __syncthreads();
  const int n_valid = s_total;
  const bool compact = allow_compact && ((n_valid + 255) & ~255) < ((N + 255) & ~255);
  float gscale = 0.0f;
  if (reduction == 0) gscale = (float)((double)dloss[0] / (double)n_valid);  // NaN / inf if n_valid = 0: unused then
  if (reduction == 1) gscale = dloss[0];
  int pos = compact ? wave_base[wave] + incl - cnt : r0;
  auto put = [&](int row, int tg, float l, float g) {
    if (compact && tg == ignore_index) return;
    TokInfo ti;
    ti.lse = l;
    ti.target = tg;
    ti.g = g;
    ti.row = row;
    tinfo[pos++] = ti;
  };
  for (r = r0; r + 4 <= r1; r += 4) {  // 16-byte loads of four tokens at a time
    const int4 tg = *reinterpret_cast<const int4*>(targets + r);
    const float4 l = *reinterpret_cast<const float4*>(lse + r);
    float4 g = make_float4(gscale, gscale, gscale, gscale);
    if (reduction == 2) g = *reinterpret_cast<const float4*>(dloss + r);
    put(r, tg.x, l.x, g.x);
    put(r + 1, tg.y, l.y, g.y);
    put(r + 2, tg.z, l.z, g.z);
    put(r + 3, tg.w, l.w, g.w);
  }
  for (; r < r1; ++r) put(r, targets[r], lse[r], reduction == 2 ? dloss[r] : gscale);
  if (t == 0) {
    BwdPrep p;
    p.n_valid = n_valid;
    p.n_eff = compact ? n_valid : N;
    p.compact = compact ? 1 : 0;
    p.gscale = gscale;
    *prep = p;
  }
}

// Compact mode: copy the hidden rows of positions [n0, n0 + nc) (those that
// exist) into xv, one block per row, 16-byte accesses; and, when dX is given,
// zero the dX [N][H] rows of ignored tokens (the contractions never write
// them in compact mode).
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ X, uint16_t* __restrict__ xv,
                                                          const BwdPrep* __restrict__ prep,
                                                          const TokInfo* __restrict__ tinfo, int n0, int nc, int H,
                                                          float* __restrict__ dX, const int* __restrict__ targets,
                                                          int N, int ignore_index) {
  if (!prep->compact) return;
  const int nv = min(nc, prep->n_eff - n0);
  const int c8 = H >> 3;
  for (int i = blockIdx.x; i < nv; i += gridDim.x) {
    const u32x4* src = reinterpret_cast<const u32x4*>(X + (size_t)tinfo[n0 + i].row * H);
    u32x4* dst = reinterpret_cast<u32x4*>(xv + (size_t)i * H);
    for (int c = threadIdx.x; c < c8; c += 256) dst[c] = src[c];
  }
  if (!dX) return;
  const int c4 = H >> 2;
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int r = blockIdx.x; r < N; r += gridDim.x) {
    if (targets[r] != ignore_index) continue;
    f32x4* d = reinterpret_cast<f32x4*>(dX + (size_t)r * H);
    for (int c = threadIdx.x; c < c4; c += 256) d[c] = z;
  }
}

// --------------------------------------------------------------------------
// Backward, one unit = (shard, vocabulary chunk, token chunk).
//
// recompute_g_tile: one 256 x 256 block of the unit's logits, recomputed from
// X and W_s, and its gradient G = g_i (exp(y - lse_i) - [v == t_i]) in bf16
// (round to nearest even), written to G [token][vocabulary] (row pitch ldg).
// As in the forward the tile is computed vocabulary x token, so each lane owns
// four token columns and their (lse, g, target) sit in registers. Rows past the
// token chunk (g = 0, lse = +inf) and columns past the vocabulary chunk are
// written as 0, so G is a dense zero-padded [nc_pad][vc_pad] matrix. The tile
// is staged in LDS (16-byte chunks of each token row XOR-swizzled by the row)
// and written out with 16-byte stores.
//
// grad_tile: one 256 x 256 output tile of the unit's two contractions
//   dX[n0 + m][h]   (+)= sum_v G[m][v] W_s[v0 + v][h]   (K = vc_pad)
//   dW_s[v0 + m][h] (+)= sum_t G[t][m] X[n0 + t][h]     (K = nc_pad)
// G is read as it was written: K-contiguous for dX, K-major for dW; W_s and X
// are K-major for both. The problem with the longer K takes the first slots
// (padded to a multiple of 8 so both start on XCD 0) so the long tiles are
// dispatched first; within each problem the tiles follow xcd_tile.
//
// bwd_step_kernel runs, in one launch, the gradient tiles of unit u - 1 (first
// slots) and the recompute tiles of unit u (after them), with the two units'
// G in different buffers: the short recompute tiles fill in behind the long
// gradient tiles, and the backward needs one launch per unit instead of two.
// --------------------------------------------------------------------------
// G of one recomputed tile into the LDS staging area: token row tok holds the
// tile's 256 vocabulary values as bf16, 16-byte chunk c in slot c ^ (tok & 31).
template <bool kMask, bool kOneHot>
__device__ __forceinline__ void stage_g(const Acc& acc, const float (&lse2)[kNI], const float (&g)[kNI],
                                        const int (&tcol)[kNI], int live, char* ldsg) {
  const int wave = wave_id();
  const int lane = lane_id();
  const int wm = wave / kWN, wn = wave % kWN;
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    const int tok = wn * kWaveN + kBlk * j + (lane & 15);  // token row of the staged tile
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      const int r0 = wm * kWaveM + kBlk * i + 4 * (lane >> 4);  // 4 consecutive vocabulary rows
      float gv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + q;
        const float p = fast_exp2(fmaf(acc[i][j][q], kLog2e, -lse2[j]));
        const float v = kOneHot ? g[j] * (p - (r == tcol[j] ? 1.0f : 0.0f)) : g[j] * p;
        gv[q] = (!kMask || r < live) ? v : 0.0f;
      }
      const int slot = (r0 >> 3) ^ (tok & 31);
      uint2 packed = make_uint2(pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]));
      *reinterpret_cast<uint2*>(ldsg + tok * 512 + slot * 16 + (r0 & 7) * 2) = packed;
    }
  }
}

__device__ __forceinline__ void recompute_g_tile(const BwdGArgs& a, int id, LCE_LDS char* lds, char* ldsg) {
  const int wave = wave_id();
  const int lane = lane_id();
  const int wm = wave / kWN, wn = wave % kWN;
  int tt, tv;
  xcd_tile(id, a.n_tt, a.n_tv, tt, tv);
  // positions of this unit that exist (the host plans for every token; the
  // backward runs over n_eff of them)
  const int nv = min(a.nc, a.prep->n_eff - a.n0);
  if (tt * kBN >= nv) return;
  // the hidden rows of the unit's positions: gathered (compact mode) or X's own
  const uint16_t* xs = a.prep->compact ? a.xv : a.X + (size_t)a.n0 * a.H;

  // per-lane token info, loaded before the main loop (unconditionally, from a
  // clamped position, so that the loads complete under the loop's first wait)
  // and turned into (log2-domain lse, gradient scale, target row in this
  // tile) after it
  TokInfo ti[kNI];
  bool valid[kNI];
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    const int rr = tt * kBN + wn * kWaveN + kBlk * j + (lane & 15);
    valid[j] = rr < nv;
    ti[j] = a.tinfo[a.n0 + (valid[j] ? rr : tt * kBN)];
  }
  KContigLoader lw, lx;
  lw.init(a.Ws, a.H, a.v0 + tv * kBM, a.Vs, wave, lane);
  lx.init(xs, a.H, tt * kBN, nv, wave, lane);
  Acc acc;
  // load addresses formed at each issue (as in the forward): with the two
  // K-contiguous operands this loop runs about 10 % faster than with the
  // addresses hoisted out of it
  tile_mainloop<false, false, false, true>(lw, lx, a.H, lds, acc, a.vc - tv * kBM <= kWaveM);

  float lse2[kNI], g[kNI];
  int tcol[kNI];
#pragma unroll
  for (int j = 0; j < kNI; ++j) {
    lse2[j] = __builtin_inff();
    g[j] = 0.0f;
    tcol[j] = -1;
    if (valid[j]) {
      lse2[j] = ti[j].lse * kLog2e;
      const int t = ti[j].target;
      if (t != a.ignore_index) {
        if (t < 0 || t >= a.V) {
          g[j] = __builtin_nanf("");
        } else {
          g[j] = ti[j].g;
          tcol[j] = t - (a.vocab_base + tv * kBM);
        }
      }
    }
  }
  const int live = a.vc - tv * kBM;  // vocabulary rows of this tile inside the chunk
  // The row mask matters only in a chunk's last, partial tile, and the one-hot
  // only in a wave whose 128 vocabulary rows hold some lane's target: both are
  // uniform over the wave, so the common case skips their compares (the
  // values are the same: p - 0 is p).
  bool has_target = false;
#pragma unroll
  for (int j = 0; j < kNI; ++j) has_target |= tcol[j] >= wm * kWaveM && tcol[j] < wm * kWaveM + kWaveM;
  const bool one_hot = __any(has_target);
  if (live < kBM) {
    if (one_hot)
      stage_g<true, true>(acc, lse2, g, tcol, live, ldsg);
    else
      stage_g<true, false>(acc, lse2, g, tcol, live, ldsg);
  } else {
    if (one_hot)
      stage_g<false, true>(acc, lse2, g, tcol, live, ldsg);
    else
      stage_g<false, false>(acc, lse2, g, tcol, live, ldsg);
  }
  __syncthreads();
  uint16_t* gt = a.G + (size_t)tt * kBN * a.ldg + (size_t)tv * kBM;
  // G is read back by the next launch, from other XCDs' L2s: a chunk that
  // fits the last-level cache is stored normally, so that it is read from
  // there; a larger one non-temporally
  if (a.g_cached) {
#pragma unroll 4
    for (int it = 0; it < kBN * kBM / 8 / kThreads; ++it) {
      const int q = it * kThreads + threadIdx.x;
      const int r = q >> 5, c = q & 31;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ldsg + r * 512 + ((c ^ (r & 31)) << 4));
      *reinterpret_cast<u32x4*>(gt + (size_t)r * a.ldg + c * 8) = v;
    }
  } else {
#pragma unroll 4
    for (int it = 0; it < kBN * kBM / 8 / kThreads; ++it) {
      const int q = it * kThreads + threadIdx.x;
      const int r = q >> 5, c = q & 31;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ldsg + r * 512 + ((c ^ (r & 31)) << 4));
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(gt + (size_t)r * a.ldg + c * 8));
    }
  }
}

// Stores (accumulate = 0) or adds (accumulate = 1) the fp32 tile into
// C[row(m0 + r)][n0 + c] for r < m_valid - m0, c < n_valid - n0 (n_valid a
// multiple of 4), where row(m0 + r) = rowmap[r] when a row map is given (the
// dX rows of the tile's positions, staged in LDS) and m0 + r otherwise. The
// tile goes through LDS in two halves of 128 rows (the rows of the waves with
// wm = 0, then wm = 1), so that global memory sees 16-byte accesses along
// whole rows. For each half, a thread issues all of its loads of C before the
// half is staged, so they fly while the accumulators are written to LDS and
// the half costs one round trip to memory. LDS row r holds the 256 floats of
// the row, with column c stored at c ^ (16 ((r >> 2) & 3)), so the four
// 16-lane groups of an accumulator write (rows r, r + 4, r + 8, r + 12, 16
// columns each) use different banks. Needs the 128 KB of LDS free (the main
// loop ends on a barrier). Thread t handles 16-byte chunk (t & 63) of rows
// (t >> 6) + 8 k, k < kIt; a row's index is read again where it is used
// rather than kept in registers across the staging. With a row map the
// element's byte offset from C is formed in 32 bits (the host allows a row
// map only when the whole of C is below 4 GiB), one register per access.
__device__ __forceinline__ float* elem(float* C, int ldc, const int* rowmap, int m0, int r, int gc) {
  if (rowmap)
    return reinterpret_cast<float*>(reinterpret_cast<char*>(C) +
                                    ((uint32_t)rowmap[r] * (uint32_t)ldc + (uint32_t)gc) * 4u);
  return C + (size_t)(m0 + r) * ldc + gc;
}
template <int kIt, bool kFull>
__device__ __forceinline__ void load_half(const float* __restrict__ C, int ldc, const int* rowmap, int m0, int h,
                                          int m_valid, int n0, int n_valid, float4 (&old)[kIt]) {
  const int c = threadIdx.x & 63;
  const int gc = n0 + 4 * c;
#pragma unroll
  for (int k = 0; k < kIt; ++k) {
    const int r = 128 * h + k * (kThreads / 64) + (threadIdx.x >> 6);
    old[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (kFull || (m0 + r < m_valid && gc < n_valid))
      old[k] = *reinterpret_cast<const float4*>(elem(const_cast<float*>(C), ldc, rowmap, m0, r, gc));
  }
}
template <int kIt, bool kFull, bool kAcc>
__device__ __forceinline__ void store_half(float* __restrict__ C, int ldc, const int* rowmap, int m0, int h,
                                           int m_valid, int n0, int n_valid, const float* tile,
                                           const float4 (&old)[kIt]) {
  const int c = threadIdx.x & 63;
  const int gc = n0 + 4 * c;
#pragma unroll
  for (int k = 0; k < kIt; ++k) {
    const int rl = k * (kThreads / 64) + (threadIdx.x >> 6);  // row within the half
    const int r = 128 * h + rl;
    if (kFull || (m0 + r < m_valid && gc < n_valid)) {
      float4 v = *reinterpret_cast<const float4*>(tile + rl * 256 + 4 * (c ^ (4 * ((rl >> 2) & 3))));
      if (kAcc) {
        v.x += old[k].x;
        v.y += old[k].y;
        v.z += old[k].z;
        v.w += old[k].w;
      }
      // non-temporal: the next add to this tile comes from a later launch
      const f32x4 nv = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(elem(C, ldc, rowmap, m0, r, gc)));
    }
  }
}

template <bool kFull, bool kAcc>
__device__ __forceinline__ void store_tile_impl(const Acc& acc, float* __restrict__ C, int ldc, const int* rowmap,
                                                int m0, int m_valid, int n0, int n_valid, char* ldsg) {
  const int wave = wave_id();
  const int lane = lane_id();
  const int wm = wave / kWN, wn = wave % kWN;
  constexpr int kIt = 128 * 64 / kThreads;  // 16-byte chunks per thread and half
  float* tile = reinterpret_cast<float*>(ldsg);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float4 old[kIt];
    if (kAcc) load_half<kIt, kFull>(C, ldc, rowmap, m0, h, m_valid, n0, n_valid, old);
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = kBlk * i + 4 * (lane >> 4) + e;
#pragma unroll
          for (int j = 0; j < kNI; ++j) {
            const int c = wn * kWaveN + kBlk * j + (lane & 15);
            tile[r * 256 + (c ^ (16 * ((r >> 2) & 3)))] = acc[i][j][e];
          }
        }
    }
    __syncthreads();
    store_half<kIt, kFull, kAcc>(C, ldc, rowmap, m0, h, m_valid, n0, n_valid, tile, old);
    __syncthreads();
  }
}

// rowmap: NULL, or the LDS row map of the tile's 256 rows (see store_tile_impl).
__device__ __forceinline__ void store_tile(const Acc& acc, float* __restrict__ C, int ldc, const int* rowmap, int m0,
                                           int m_valid, int n0, int n_valid, int accumulate, char* ldsg) {
  const bool full = m0 + kBM <= m_valid && n0 + kBN <= n_valid;
  if (full && accumulate)
    store_tile_impl<true, true>(acc, C, ldc, rowmap, m0, m_valid, n0, n_valid, ldsg);
  else if (full)
    store_tile_impl<true, false>(acc, C, ldc, rowmap, m0, m_valid, n0, n_valid, ldsg);
  else if (accumulate)
    store_tile_impl<false, true>(acc, C, ldc, rowmap, m0, m_valid, n0, n_valid, ldsg);
  else
    store_tile_impl<false, false>(acc, C, ldc, rowmap, m0, m_valid, n0, n_valid, ldsg);
}

// The K loop of a gradient tile runs over the live part of its contraction
// only: the vocabulary chunk rounded up to the 64 of a stage for dX (the G
// columns past the chunk are zero), and for dW the positions of the unit that
// exist, rounded up likewise (G rows past them are zero; their X rows are
// clamped to the last existing one). A dW tile with nothing to contract
// writes zeros (or, accumulating, leaves its rows as they are); a dX tile
// past the existing positions has no rows to write.
__device__ __forceinline__ void grad_tile(const GradArgs& a, int id, LCE_LDS char* lds, char* ldsg, int* rowmap) {
  const int wave = wave_id();
  const int lane = lane_id();
  const int dx_rows = a.nc_pad / kBM, dw_rows = a.vc_pad / kBM;
  bool is_dx;
  if (id < a.first_slots) {
    is_dx = !a.dw_first;
  } else {
    is_dx = a.dw_first;
    id -= a.first_slots;
  }
  const int rows = is_dx ? dx_rows : dw_rows;
  if (id >= rows * a.n_tiles) return;  // padding slot
  int tm, tn;
  xcd_tile(id, rows, a.n_tiles, tm, tn);
  const int nv = min(a.nc, a.prep->n_eff - a.n0);
  Acc acc;
  if (is_dx) {
    if (tm * kBM >= nv) return;
    // the dX rows of the tile's positions, staged in LDS while the main loop
    // runs (its barriers order these writes before the epilogue's reads)
    const bool mapped = a.prep->compact;
    if (mapped && threadIdx.x < kBM) {
      const int pos = tm * kBM + threadIdx.x;
      rowmap[threadIdx.x] = pos < nv ? a.tinfo[a.n0 + pos].row : 0;
    }
    KContigLoader la;
    KMajorLoader lb;
    la.init(a.G, a.ldg, tm * kBM, nv, wave, lane);
    lb.init(a.Wc, a.H, tn * kBN, a.H, a.vc, wave, lane);
    tile_mainloop<false, true>(la, lb, (a.vc + kBK - 1) / kBK * kBK, lds, acc, nv - tm * kBM <= kWaveM);
    // without a row map position n0 + i is row n0 + i
    store_tile(acc, mapped ? a.dX : a.dX + (size_t)a.n0 * a.H, a.H, mapped ? rowmap : nullptr, tm * kBM, nv,
               tn * kBN, a.H, a.acc_dx, ldsg);
  } else {
    if (nv <= 0) {
      if (a.acc_dw) return;
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kNI; ++j) acc[i][j] = f32x4{};
    } else {
      const int k_live = (nv + kBK - 1) / kBK * kBK;
      const uint16_t* xs = a.prep->compact ? a.xv : a.X + (size_t)a.n0 * a.H;
      KMajorLoader la, lb;
      la.init(a.G, a.ldg, tm * kBM, a.vc_pad, k_live, wave, lane);
      lb.init(xs, a.H, tn * kBN, a.H, nv, wave, lane);
      tile_mainloop<true, true>(la, lb, k_live, lds, acc, a.vc - tm * kBM <= kWaveM);
    }
    store_tile(acc, a.dW, a.H, nullptr, tm * kBM, a.vc, tn * kBN, a.H, a.acc_dw, ldsg);
  }
}

__global__ __launch_bounds__(kThreads, 1) void bwd_step_kernel(GradArgs gr, int grad_slots, BwdGArgs bg,
                                                               int g_tiles) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kMainLds];
  __shared__ int rowmap[kBM];
  LCE_LDS char* lds = (LCE_LDS char*)lds_raw;
  const int id = blockIdx.x;
  if (id < grad_slots) {
    grad_tile(gr, id, lds, lds_raw, rowmap);
  } else if (id - grad_slots < g_tiles) {
    recompute_g_tile(bg, id - grad_slots, lds, lds_raw);
  }
}

// --------------------------------------------------------------------------
// Finalize, after the last round's launch: block tb merges the S split states
// of its 256 tokens in split order, writes lse = (m + log2 z) ln 2 and the
// token losses, and the block's (loss sum, count) in fixed tree order;
// loss_kernel then sums the block partials in block order. Two launches, so
// the only ordering between workgroups is the launch boundary: a device-wide
// fence inside a launch (an L2 write-back and invalidate on this GPU) cost
// each workgroup tens of microseconds and evicted its neighbours' operands.
// Every sum runs in a fixed order, so the result is bitwise reproducible.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void finalize_kernel(FwdArgs a) {
  __shared__ double sa[256];
  __shared__ long long sb[256];
  const int tb = blockIdx.x;
  const int row = tb * 256 + threadIdx.x;
  double l = 0.0;
  long long cnt = 0;
  if (row < a.N) {
    float M = kNegBig, Z = 0.0f;
    for (int s = 0; s < a.S; ++s) {
      const float2 p = a.state[(size_t)s * a.state_ld + row];
      lse_merge(M, Z, p.x, p.y);
    }
    const float lse = (M + fast_log2(Z)) * kLn2;
    a.lse[row] = lse;
    float tl = 0.0f;
    if (a.targets[row] != a.ignore_index) {
      tl = lse - a.yt[row];
      cnt = 1;
    }
    if (a.token_loss) a.token_loss[row] = tl;
    l = tl;
  }
  block_sum256(l, cnt, sa, sb);
  if (threadIdx.x == 0) a.partials[tb] = make_double2(l, (double)cnt);
}

__global__ __launch_bounds__(256) void loss_kernel(FwdArgs a) {
  __shared__ double sa[256];
  __shared__ long long sb[256];
  double s = 0.0;
  long long c = 0;
  for (int b = threadIdx.x; b < a.token_blocks; b += 256) {
    const double2 p = a.partials[b];
    s += p.x;
    c += (long long)p.y;
  }
  block_sum256(s, c, sa, sb);
  if (threadIdx.x == 0) a.loss[0] = (float)(a.reduction == 0 ? s / (double)c : s);
}

// --------------------------------------------------------------------------
// bf16 gradient outputs: the contractions accumulate in fp32 scratch; these
// convert between that scratch and the caller's bf16 buffers, 8 elements per
// thread with 16-byte accesses (round to nearest even on narrowing).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void widen_bf16_kernel(const uint16_t* __restrict__ src, float* __restrict__ dst,
                                                         int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const u32x4 v = reinterpret_cast<const u32x4*>(src)[i];
    float4 lo, hi;
    lo.x = __uint_as_float(v[0] << 16);
    lo.y = __uint_as_float(v[0] & 0xffff0000u);
    lo.z = __uint_as_float(v[1] << 16);
    lo.w = __uint_as_float(v[1] & 0xffff0000u);
    hi.x = __uint_as_float(v[2] << 16);
    hi.y = __uint_as_float(v[2] & 0xffff0000u);
    hi.z = __uint_as_float(v[3] << 16);
    hi.w = __uint_as_float(v[3] & 0xffff0000u);
    reinterpret_cast<float4*>(dst)[2 * i] = lo;
    reinterpret_cast<float4*>(dst)[2 * i + 1] = hi;
  }
}

__global__ __launch_bounds__(256) void narrow_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                          int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const float4 lo = reinterpret_cast<const float4*>(src)[2 * i];
    const float4 hi = reinterpret_cast<const float4*>(src)[2 * i + 1];
    u32x4 v;
    v[0] = pack_bf16x2(lo.x, lo.y);
    v[1] = pack_bf16x2(lo.z, lo.w);
    v[2] = pack_bf16x2(hi.x, hi.y);
    v[3] = pack_bf16x2(hi.z, hi.w);
    reinterpret_cast<u32x4*>(dst)[i] = v;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(u32x4* __restrict__ p, int64_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) p[i] = z;
}

__global__ void set_scalar_kernel(float* p, float v) {
  if (threadIdx.x == 0) *p = v;
}

// ============================ host launchers ==============================
static inline hipError_t last() { return hipGetLastError(); }

hipError_t launch_fwd_rounds(const FwdArgs& a, const ShardTable& shards, int k_begin, int k_end, int first,
                             hipStream_t st) {
  hipLaunchKernelGGL(fwd_round_kernel, dim3(a.token_blocks * a.S), dim3(kThreads), 0, st, a, shards, k_begin, k_end,
                     first);
  return last();
}

hipError_t launch_finalize(const FwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(finalize_kernel, dim3(a.token_blocks), dim3(256), 0, st, a);
  hipError_t e = last();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(256), 0, st, a);
  return last();
}

hipError_t launch_init_target_logits(const int* targets, int N, int ignore_index, float* yt, hipStream_t st) {
  hipLaunchKernelGGL(init_target_logits_kernel, dim3((N + 255) / 256), dim3(256), 0, st, targets, N, ignore_index, yt);
  return last();
}

hipError_t launch_bwd_prep(const int* targets, const float* lse, int N, int ignore_index, const float* dloss,
                           int reduction, int allow_compact, BwdPrep* prep, TokInfo* tinfo, hipStream_t st) {
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(1), dim3(1024), 0, st, targets, lse, N, ignore_index, dloss, reduction,
                     allow_compact, prep, tinfo);
  return last();
}

hipError_t launch_gather_rows(const uint16_t* X, uint16_t* xv, const BwdPrep* prep, const TokInfo* tinfo, int n0,
                              int nc, int H, float* dX, const int* targets, int N, int ignore_index, hipStream_t st) {
  const int rows = dX ? (nc > N ? nc : N) : nc;
  const int blocks = rows < 2048 ? (rows < 1 ? 1 : rows) : 2048;  // grid-stride over rows beyond that
  hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(256), 0, st, X, xv, prep, tinfo, n0, nc, H, dX, targets,
                     N, ignore_index);
  return last();
}

hipError_t launch_bwd_step(const GradArgs* gr, const BwdGArgs* bg, hipStream_t st) {
  GradArgs g{};
  BwdGArgs b{};
  int grad_slots = 0, g_tiles = 0;
  if (gr) {
    g = *gr;
    g.n_tiles = g.H / kBN + (g.H % kBN ? 1 : 0);
    const int dx_tiles = (g.nc_pad / kBM) * g.n_tiles;
    const int dw_tiles = (g.vc_pad / kBM) * g.n_tiles;
    g.dw_first = g.nc_pad > g.vc_pad ? 1 : 0;  // dW tiles have K = nc_pad, dX tiles K = vc_pad
    const int first = g.dw_first ? dw_tiles : dx_tiles, second = g.dw_first ? dx_tiles : dw_tiles;
    g.first_slots = (first + 7) & ~7;
    grad_slots = (g.first_slots + second + 7) & ~7;
  }
  if (bg) {
    b = *bg;
    b.n_tt = b.nc_pad / kBN;
    b.n_tv = b.vc_pad / kBM;
    g_tiles = b.n_tt * b.n_tv;
  }
  if (grad_slots + g_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_step_kernel, dim3(grad_slots + g_tiles), dim3(kThreads), 0, st, g, grad_slots, b, g_tiles);
  return last();
}

static inline unsigned elementwise_blocks(int64_t n8) {
  const int64_t b = (n8 + 255) / 256;
  return (unsigned)(b < 4096 ? (b < 1 ? 1 : b) : 4096);  // grid-stride beyond 4096 blocks
}

hipError_t launch_widen_bf16(const uint16_t* src, float* dst, int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t n8 = rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(widen_bf16_kernel, dim3(elementwise_blocks(n8)), dim3(256), 0, st, src, dst, n8);
  return last();
}

hipError_t launch_narrow_bf16(const float* src, uint16_t* dst, int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t n8 = rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(narrow_bf16_kernel, dim3(elementwise_blocks(n8)), dim3(256), 0, st, src, dst, n8);
  return last();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(elementwise_blocks(n16)), dim3(256), 0, st, static_cast<u32x4*>(p), n16);
  return last();
}

hipError_t launch_set_scalar(float* p, float v, hipStream_t st) {
  hipLaunchKernelGGL(set_scalar_kernel, dim3(1), dim3(64), 0, st, p, v);
  return last();
}

}  // namespace lce

// HIP kernels (gfx950) for the memory-bounded vocabulary projection +
// cross-entropy, and the host-side launchers the C ABI calls.
//
// Method: "Flattening Every Memory Peak in Long-Context Mixture-of-Experts
// Training", section 3.2 (Ring-DTP). Each round meets one vocabulary shard,
// folds its logits into a per-token running (max, exp-sum) by the online
// softmax update (Eq. 3), and never stores the logits; after the last round
// the loss is m + log z - y_t. Backward recomputes each logit block from the
// saved normalizer lse = m + log z.
#include <hip/hip_runtime.h>

#include "lce_internal.hpp"
#include "tile_gemm.hpp"

namespace lce {

// --------------------------------------------------------------------------
// Forward round: fold X W_s^T into the running per-token state.
//
// Grid (row_blocks, S). Workgroup (rb, j) owns tokens [256 rb, 256 rb + 256)
// and the column tiles [j*tps, min((j+1)*tps, n_col_tiles)) of shard s. It
// keeps, per lane and per token it holds in the MFMA accumulator layout, an
// online (m, z) in the log2 domain over every column it sees, and merges the
// lanes and waves once at the end, in a fixed order. The state of split j,
// state[j][token], is read-modified-written once per round, so over the rounds
// each split meets the shards in ring order. No atomics: every (j, token) has
// exactly one writer per launch, and launches are ordered on the stream.
// --------------------------------------------------------------------------
template <int MI, int NI>
__device__ __forceinline__ void fold_tile(const f32x16 (&acc)[MI][NI], float (&m)[MI * 16], float (&z)[MI * 16],
                                          const bool (&live)[NI]) {
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    // One row-block at a time: its NI accumulator vectors leave the AGPRs
    // together (16 x NI values), are folded row by row, and are released
    // before the next row-block is touched.
    f32x16 blk[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) blk[j] = acc[i][j];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j) v[j] = live[j] ? blk[j][e] : -__builtin_inff();
      float mx = v[0];
#pragma unroll
      for (int j = 1; j < NI; ++j) mx = fmaxf(mx, v[j]);
      const int k = i * 16 + e;
      const float mn = fmaxf(m[k], mx * kLog2e);
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < NI; ++j) s += fast_exp2(fmaf(v[j], kLog2e, -mn));
      z[k] = fmaf(z[k], fast_exp2(m[k] - mn), s);
      m[k] = mn;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int WM, int WN>
__global__ __launch_bounds__(kThreads, 1) void fwd_round_kernel(const uint16_t* __restrict__ X, int N, int H,
                                                                const uint16_t* __restrict__ W, int Vs,
                                                                float2* __restrict__ state, int state_ld,
                                                                int tiles_per_split, int n_col_tiles, int first) {
  using S = TileShape<WM, WN>;
  constexpr int MI = S::kMI, NI = S::kNI;
  constexpr int kRedCols = WN * 32;
  constexpr int kRedStride = kRedCols * 8 + 8;
  constexpr int kRedBytes = kBM * kRedStride;
  constexpr int kLdsBytes = kRedBytes > kMainLds ? kRedBytes : kMainLds;
  __shared__ __attribute__((aligned(1024))) char lds_raw[kLdsBytes];
  LCE_LDS char* lds = (LCE_LDS char*)lds_raw;
  char* ldsg = lds_raw;

  const int wave = wave_id();
  const int lane = lane_id();
  const int row0 = blockIdx.x * kBM;
  const int split = blockIdx.y;
  const int t0 = split * tiles_per_split;
  const int t1 = min(t0 + tiles_per_split, n_col_tiles);

  OperandLoader la;
  la.init(X, H, row0, N, wave, lane);
  float m[MI * 16], z[MI * 16];
#pragma unroll
  for (int k = 0; k < MI * 16; ++k) {
    m[k] = kNegBig;
    z[k] = 0.0f;
  }
  const int col_lane = (wave % WN) * S::kWaveN + (lane & 31);
  for (int ct = t0; ct < t1; ++ct) {
    OperandLoader lb;
    lb.init(W, H, ct * kBN, Vs, wave, lane);
    f32x16 acc[MI][NI];
    tile_mainloop<WM, WN>(la, lb, H, lds, acc, false);
    // columns past the end of the shard (last tile only) act as -infinity
    const int cvalid = Vs - ct * kBN;
    bool live[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) live[j] = col_lane + j * 32 < cvalid;
    fold_tile<MI, NI>(acc, m, z, live);
  }

  // Merge lanes and waves: every lane parks its (m, z) per token in LDS, then
  // thread t merges token t's partials in column order.
  const int rcol = (wave % WN) * 32 + (lane & 31);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = acc_row<WM, WN>(wave, lane, i, e);
      float* d = reinterpret_cast<float*>(ldsg + r * kRedStride + rcol * 8);
      d[0] = m[i * 16 + e];
      d[1] = z[i * 16 + e];
    }
  __syncthreads();
  const int r = threadIdx.x;
  float M = kNegBig, Z = 0.0f;
  for (int c = 0; c < kRedCols; ++c) {
    const float* p = reinterpret_cast<const float*>(ldsg + r * kRedStride + c * 8);
    lse_merge(M, Z, p[0], p[1]);
  }
  const int row = row0 + r;
  if (row < N) {
    float2* sp = state + (size_t)split * state_ld + row;
    if (!first) {
      const float2 o = *sp;
      float M0 = o.x, Z0 = o.y;
      lse_merge(M0, Z0, M, Z);
      M = M0;
      Z = Z0;
    }
    *sp = make_float2(M, Z);
  }
}

// --------------------------------------------------------------------------
// Target logit y_t = x_i . w_{t_i} (fp32 accumulation), one wave per token, read
// from the shard that owns t_i. Ignored tokens get 0; a target outside [0, V)
// gets NaN so the token's loss, and the mean, become NaN.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void target_logit_kernel(const uint16_t* __restrict__ X, int N, int H,
                                                           ShardTable shards, int Vs, int V,
                                                           const int* __restrict__ targets, int ignore_index,
                                                           float* __restrict__ yt) {
  const int lane = lane_id();
  const int row = blockIdx.x * 4 + wave_id();
  if (row >= N) return;
  const int t = __builtin_amdgcn_readfirstlane(targets[row]);
  if (t == ignore_index || t < 0 || t >= V) {
    if (lane == 0) yt[row] = (t == ignore_index) ? 0.0f : __builtin_nanf("");
    return;
  }
  const int s = t / Vs;
  const uint16_t* w = shards.p[s] + (size_t)(t - s * Vs) * H;
  const uint16_t* x = X + (size_t)row * H;
  float acc = 0.0f;
  for (int c = lane * 8; c < H; c += 512) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(x + c);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(w + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc = fmaf(__uint_as_float(xv[q] << 16), __uint_as_float(wv[q] << 16), acc);
      acc = fmaf(__uint_as_float(xv[q] & 0xffff0000u), __uint_as_float(wv[q] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) yt[row] = acc;
}

// Fixed-order tree sum over a 256-thread block (deterministic).
__device__ __forceinline__ void block_sum2(double& a, long long& b) {
  __shared__ double sa[256];
  __shared__ long long sb[256];
  sa[threadIdx.x] = a;
  sb[threadIdx.x] = b;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      sa[threadIdx.x] += sa[threadIdx.x + w];
      sb[threadIdx.x] += sb[threadIdx.x + w];
    }
    __syncthreads();
  }
  a = sa[0];
  b = sb[0];
}

// --------------------------------------------------------------------------
// Finalize: merge the S split states in order; lse = (m + log2 z) ln 2; token
// loss lse - y_t for valid tokens, 0 for ignored ones; per-block partial sums.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void finalize_kernel(const float2* __restrict__ state, int state_ld, int S,
                                                       const float* __restrict__ yt,
                                                       const int* __restrict__ targets, int N, int ignore_index,
                                                       float* __restrict__ lse_out,
                                                       float* __restrict__ token_loss,
                                                       double2* __restrict__ partials) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  double l = 0.0;
  long long cnt = 0;
  if (row < N) {
    float M = kNegBig, Z = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float2 p = state[(size_t)s * state_ld + row];
      lse_merge(M, Z, p.x, p.y);
    }
    const float lse = (M + fast_log2(Z)) * kLn2;
    lse_out[row] = lse;
    float tl = 0.0f;
    if (targets[row] != ignore_index) {
      tl = lse - yt[row];
      cnt = 1;
    }
    if (token_loss) token_loss[row] = tl;
    l = tl;
  }
  block_sum2(l, cnt);
  if (threadIdx.x == 0) partials[blockIdx.x] = make_double2(l, (double)cnt);
}

__global__ __launch_bounds__(256) void loss_reduce_kernel(const double2* __restrict__ partials, int n, int reduction,
                                                          float* __restrict__ loss, float* __restrict__ n_valid_out) {
  double s = 0.0;
  long long c = 0;
  for (int i = threadIdx.x; i < n; i += 256) {
    s += partials[i].x;
    c += (long long)partials[i].y;
  }
  block_sum2(s, c);
  if (threadIdx.x == 0) {
    loss[0] = (float)(reduction == 0 ? s / (double)c : s);
    if (n_valid_out) n_valid_out[0] = (float)c;
  }
}

// --------------------------------------------------------------------------
// Backward scale: g = dloss / n_valid (mean) or dloss (sum), on the device so
// dloss can come straight from autograd.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_scale_kernel(const int* __restrict__ targets, int N, int ignore_index,
                                                        const float* __restrict__ dloss, int reduction,
                                                        float* __restrict__ gscale) {
  double unused = 0.0;
  long long c = 0;
  for (int i = threadIdx.x; i < N; i += 256) c += (targets[i] != ignore_index) ? 1 : 0;
  block_sum2(unused, c);
  if (threadIdx.x == 0) gscale[0] = reduction == 0 ? (float)((double)dloss[0] / (double)c) : dloss[0];
}

// --------------------------------------------------------------------------
// Backward recompute of one 256x256 logit tile of the (token chunk, vocabulary
// chunk) block and its gradient G = g_i (exp(y - lse_i) - [v == t_i]) in bf16
// (round to nearest even). Rows past the token chunk and columns past the
// vocabulary chunk are written as 0, so G is a dense zero-padded
// [nc_pad][vc_pad] matrix.
// --------------------------------------------------------------------------
struct RowInfo {
  float lse2;
  float g;
  int tcol;
  int pad;
};

template <int WM, int WN>
__global__ __launch_bounds__(kThreads, 1) void bwd_g_kernel(const uint16_t* __restrict__ X, int N, int H,
                                                            const uint16_t* __restrict__ Ws, int Vs, int v0,
                                                            int vc, int n0, int nc,
                                                            const int* __restrict__ targets,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ gscale, int ignore_index,
                                                            int vocab_base, int V, uint16_t* __restrict__ G,
                                                            int ldg) {
  using S = TileShape<WM, WN>;
  constexpr int MI = S::kMI, NI = S::kNI;
  constexpr int kStgStride = (kBN + 8) * 2;  // bytes per staged bf16 row
  constexpr int kStgBytes = kBM * kStgStride;
  constexpr int kBodyBytes = kStgBytes > kMainLds ? kStgBytes : kMainLds;
  __shared__ __attribute__((aligned(1024))) char lds_raw[kBodyBytes + kBM * (int)sizeof(RowInfo)];
  LCE_LDS char* lds = (LCE_LDS char*)lds_raw;
  char* ldsg = lds_raw;
  RowInfo* info = reinterpret_cast<RowInfo*>(ldsg + kBodyBytes);

  const int wave = wave_id();
  const int lane = lane_id();
  const int tm = blockIdx.x, tn = blockIdx.y;
  {
    const int rr = tm * kBM + threadIdx.x;
    const int row = n0 + rr;
    RowInfo ri{__builtin_inff(), 0.0f, -1, 0};
    if (rr < nc && row < N) {
      ri.lse2 = lse[row] * kLog2e;
      const int t = targets[row];
      if (t != ignore_index) {
        if (t < 0 || t >= V) {
          ri.g = __builtin_nanf("");
        } else {
          ri.g = gscale[0];
          ri.tcol = t - (vocab_base + tn * kBN);
        }
      }
    }
    info[threadIdx.x] = ri;
  }
  OperandLoader la, lb;
  la.init(X, H, n0 + tm * kBM, N, wave, lane);
  lb.init(Ws, H, v0 + tn * kBN, Vs, wave, lane);
  f32x16 acc[MI][NI];
  tile_mainloop<WM, WN>(la, lb, H, lds, acc, false);  // its barriers also publish info[]

  const int cvalid = vc - tn * kBN;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = acc_row<WM, WN>(wave, lane, i, e);
      const RowInfo ri = info[r];
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int c = acc_col<WM, WN>(wave, lane, j);
        const float p = fast_exp2(fmaf(acc[i][j][e], kLog2e, -ri.lse2));
        float gv = ri.g * (p - (c == ri.tcol ? 1.0f : 0.0f));
        if (c >= cvalid) gv = 0.0f;
        *reinterpret_cast<uint16_t*>(ldsg + r * kStgStride + c * 2) = f32_to_bf16(gv);
      }
    }
  __syncthreads();
  uint16_t* gt = G + (size_t)tm * kBM * ldg + (size_t)tn * kBN;
#pragma unroll 4
  for (int it = 0; it < kBM * kBN / 8 / kThreads; ++it) {
    const int q = it * kThreads + threadIdx.x;
    const int r = q >> 5, c8 = q & 31;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ldsg + r * kStgStride + c8 * 16);
    *reinterpret_cast<u32x4*>(gt + (size_t)r * ldg + c8 * 8) = v;
  }
}

// --------------------------------------------------------------------------
// out[c][r] = in[r][c] for r < R, c < C; out[c][r] = 0 for R <= r < R_pad.
// 64x64 tiles through LDS. C, ld_in, ld_out and R_pad are multiples of 8.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in, int R, int C,
                                                             int ld_in, uint16_t* __restrict__ out, int ld_out,
                                                             int R_pad) {
  __shared__ uint16_t t[64][72];
  const int br = blockIdx.x * 64, bc = blockIdx.y * 64;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = threadIdx.x + 256 * k;
    const int r = q >> 3, c8 = (q & 7) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (br + r < R && bc + c8 < C) v = *reinterpret_cast<const u32x4*>(in + (size_t)(br + r) * ld_in + bc + c8);
    *reinterpret_cast<u32x4*>(&t[r][c8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = threadIdx.x + 256 * k;
    const int c = q >> 3, r8 = (q & 7) * 8;
    if (bc + c < C && br + r8 < R_pad) {
      u32x4 v;
#pragma unroll
      for (int p = 0; p < 4; ++p) v[p] = (uint32_t)t[r8 + 2 * p][c] | ((uint32_t)t[r8 + 2 * p + 1][c] << 16);
      *reinterpret_cast<u32x4*>(out + (size_t)(bc + c) * ld_out + br + r8) = v;
    }
  }
}

// --------------------------------------------------------------------------
// C[M][Nn] (+)= A[M][K] B[Nn][K]^T in fp32, one 256x256 tile per workgroup.
// K is a multiple of 64. Rows of A past M and of B past Nn load clamped rows;
// their results are not stored.
// --------------------------------------------------------------------------
template <int WM, int WN>
__global__ __launch_bounds__(kThreads, 1) void gemm_acc_kernel(const uint16_t* __restrict__ A, int lda, int M,
                                                               const uint16_t* __restrict__ B, int ldb, int Nn,
                                                               int K, float* __restrict__ C, int ldc,
                                                               int accumulate) {
  using S = TileShape<WM, WN>;
  constexpr int MI = S::kMI, NI = S::kNI;
  __shared__ __attribute__((aligned(1024))) char lds_raw[kMainLds];
  LCE_LDS char* lds = (LCE_LDS char*)lds_raw;
  const int wave = wave_id();
  const int lane = lane_id();
  const int tm = blockIdx.x, tn = blockIdx.y;
  OperandLoader la, lb;
  la.init(A, lda, tm * kBM, M, wave, lane);
  lb.init(B, ldb, tn * kBN, Nn, wave, lane);
  f32x16 acc[MI][NI];
  tile_mainloop<WM, WN>(la, lb, K, lds, acc, false);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = tm * kBM + acc_row<WM, WN>(wave, lane, i, e);
      if (r >= M) continue;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int c = tn * kBN + acc_col<WM, WN>(wave, lane, j);
        if (c < Nn) {
          float* p = C + (size_t)r * ldc + c;
          *p = accumulate ? *p + acc[i][j][e] : acc[i][j][e];
        }
      }
    }
}

// ============================ host launchers ==============================
// Wave layouts (WM x WN): the forward keeps a per-lane online state for every
// token it holds, so it uses 4x1 (64 tokens x 256 columns per wave, 32 tokens
// per lane); the others use 2x2 (128 x 128 per wave).
constexpr int kFwdWM = 4, kFwdWN = 1;
constexpr int kWM = 2, kWN = 2;

static inline hipError_t last() { return hipGetLastError(); }

hipError_t launch_fwd_round(const uint16_t* X, int N, int H, const uint16_t* W, int Vs, float2* state, int state_ld,
                            int row_blocks, int S, int tiles_per_split, int n_col_tiles, int first, hipStream_t st) {
  hipLaunchKernelGGL((fwd_round_kernel<kFwdWM, kFwdWN>), dim3(row_blocks, S), dim3(kThreads), 0, st, X, N, H, W, Vs,
                     state, state_ld, tiles_per_split, n_col_tiles, first);
  return last();
}

hipError_t launch_target_logit(const uint16_t* X, int N, int H, const ShardTable& shards, int Vs, int V,
                               const int* targets, int ignore_index, float* yt, hipStream_t st) {
  hipLaunchKernelGGL(target_logit_kernel, dim3((N + 3) / 4), dim3(256), 0, st, X, N, H, shards, Vs, V, targets,
                     ignore_index, yt);
  return last();
}

hipError_t launch_finalize(const float2* state, int state_ld, int S, const float* yt, const int* targets, int N,
                           int ignore_index, float* lse, float* token_loss, double2* partials, int reduction,
                           float* loss, float* n_valid_out, hipStream_t st) {
  const int nb = (N + 255) / 256;
  hipLaunchKernelGGL(finalize_kernel, dim3(nb), dim3(256), 0, st, state, state_ld, S, yt, targets, N, ignore_index,
                     lse, token_loss, partials);
  hipError_t e = last();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(256), 0, st, partials, nb, reduction, loss, n_valid_out);
  return last();
}

hipError_t launch_bwd_scale(const int* targets, int N, int ignore_index, const float* dloss, int reduction,
                            float* gscale, hipStream_t st) {
  hipLaunchKernelGGL(bwd_scale_kernel, dim3(1), dim3(256), 0, st, targets, N, ignore_index, dloss, reduction, gscale);
  return last();
}

hipError_t launch_bwd_g(const uint16_t* X, int N, int H, const uint16_t* Ws, int Vs, int v0, int vc, int n0, int nc,
                        const int* targets, const float* lse, const float* gscale, int ignore_index, int vocab_base,
                        int V, uint16_t* G, int ldg, int nc_pad, int vc_pad, hipStream_t st) {
  hipLaunchKernelGGL((bwd_g_kernel<kWM, kWN>), dim3(nc_pad / kBM, vc_pad / kBN), dim3(kThreads), 0, st, X, N, H, Ws,
                     Vs, v0, vc, n0, nc, targets, lse, gscale, ignore_index, vocab_base, V, G, ldg);
  return last();
}

hipError_t launch_transpose(const uint16_t* in, int R, int C, int ld_in, uint16_t* out, int ld_out, int R_pad,
                            hipStream_t st) {
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((R_pad + 63) / 64, (C + 63) / 64), dim3(256), 0, st, in, R, C, ld_in,
                     out, ld_out, R_pad);
  return last();
}

hipError_t launch_gemm_acc(const uint16_t* A, int lda, int M, const uint16_t* B, int ldb, int Nn, int K, float* C,
                           int ldc, int accumulate, hipStream_t st) {
  hipLaunchKernelGGL((gemm_acc_kernel<kWM, kWN>), dim3((M + kBM - 1) / kBM, (Nn + kBN - 1) / kBN), dim3(kThreads), 0,
                     st, A, lda, M, B, ldb, Nn, K, C, ldc, accumulate);
  return last();
}

}  // namespace lce

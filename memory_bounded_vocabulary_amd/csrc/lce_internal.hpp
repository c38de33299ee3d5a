// Internal interface between the C ABI (lce_api.cpp) and the kernel launchers
// (lce_kernels.hip). Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

constexpr int kMaxShards = 256;

// Device pointers of the vocabulary shards (and their ids), passed by value
// as a kernel argument (3 KB) so no host->device copy is needed.
struct ShardTable {
  const uint16_t* p[kMaxShards];
  int id[kMaxShards];
};

// Forward rounds [k_begin, k_end) in one launch (shards.p[k] is the shard met in
// round k). `first`: no earlier state to merge with.
struct FwdArgs {
  const uint16_t* X;        // hidden [N][H]
  const int* targets;
  float* yt;                // target logits, written by the tile that holds each
  float2* state;            // [S][state_ld] per-split (m, z), log2 domain
  double2* partials;        // [token_blocks] (loss sum, count)
  float* lse;               // [N]
  float* token_loss;        // [N] or NULL
  float* loss;              // scalar
  int N, H, Vs, P, state_ld, token_blocks, S, tiles_per_split, n_vtiles, ignore_index, reduction;
};
hipError_t launch_fwd_rounds(const FwdArgs& a, const ShardTable& shards, int k_begin, int k_end, int first,
                             hipStream_t st);
// After the last round: lse, token losses, block partials, then the loss (two launches).
hipError_t launch_finalize(const FwdArgs& a, hipStream_t st);
// Before the first round: yt = 0 for ignored tokens, NaN for the others (the
// rounds fill in each target logit when its tile is folded; a target outside
// [0, V) is never filled, so its token's loss, and the mean, stay NaN).
hipError_t launch_init_target_logits(const int* targets, int N, int ignore_index, float* yt, hipStream_t st);
// Backward preparation, written on the device by launch_bwd_prep. Only
// tokens whose target is not ignore_index can have a nonzero gradient row.
// When leaving the ignored ones out saves at least one 256-token tile,
// `compact` is set: the backward runs over the n_eff = n_valid kept tokens in
// ascending order ("positions"), tinfo[0 .. n_eff) describes them, and
// launch_gather_rows copies a range of their hidden rows into a buffer the
// contractions read. Otherwise n_eff = N, position i is token i, and the
// kernels read X itself.
struct BwdPrep {
  int n_valid;              // tokens with target != ignore_index
  int n_eff;                // positions the backward runs over (n_valid or N)
  int compact;              // 1: positions are the kept tokens only
  float gscale;             // dloss / n_valid (mean) or dloss (sum)
};
// What the G formation needs of the token at one position.
struct TokInfo {
  float lse;                // from the forward
  int target;
  float g;                  // gscale (mean / sum) or the token's dloss (none)
  int row;                  // the token's row in X, dX
};
// allow_compact = 0 keeps every token (no gathered copy exists then).
hipError_t launch_bwd_prep(const int* targets, const float* lse, int N, int ignore_index, const float* dloss,
                           int reduction, int allow_compact, BwdPrep* prep, TokInfo* tinfo, hipStream_t st);
// Compact mode only (else it does nothing): xv[i] = X[tinfo[n0 + i].row] for
// the positions n0 + i < min(n0 + nc, n_eff); and, when dX is non-NULL, zero
// the rows of dX [N][H] fp32 whose target is ignore_index (the contractions
// never write them in compact mode).
hipError_t launch_gather_rows(const uint16_t* X, uint16_t* xv, const BwdPrep* prep, const TokInfo* tinfo, int n0,
                              int nc, int H, float* dX, const int* targets, int N, int ignore_index, hipStream_t st);
// Recompute + G of one backward unit (shard, vocabulary chunk, token chunk).
// Token indices n0, nc are positions (see BwdPrep).
struct BwdGArgs {
  const uint16_t* X;        // hidden [N][H]
  const uint16_t* xv;       // compact mode: the hidden rows of positions n0 ..
  const BwdPrep* prep;
  const TokInfo* tinfo;
  const uint16_t* Ws;       // the unit's shard [Vs][H]
  uint16_t* G;              // [nc_pad][vc_pad], pitch ldg
  int H, Vs, v0, vc, n0, nc, nc_pad, vc_pad;
  int ignore_index, vocab_base, V, ldg;
  int g_cached;             // 1: G stored normally (it fits the last-level cache), 0: non-temporally
  int n_tt, n_tv;           // set by the launcher
};

// The two gradient contractions of one backward unit.
struct GradArgs {
  const uint16_t* G;        // [nc_pad][vc_pad], pitch ldg
  const uint16_t* Wc;       // shard rows v0.. [vc][H]
  const uint16_t* X;        // hidden [N][H]
  const uint16_t* xv;       // compact mode: the hidden rows of positions n0 ..
  const BwdPrep* prep;
  const TokInfo* tinfo;
  float* dX;                // d_hidden [N][H] (rows through tinfo)
  float* dW;                // d_shard rows v0..
  int n0;                   // the unit's first position
  int ldg, nc_pad, vc_pad, vc, nc, H, acc_dx, acc_dw;
  int n_tiles, dw_first, first_slots;  // set by the launcher
};

// One launch: the gradient tiles of `gr` (may be NULL) and the recompute tiles
// of `bg` (may be NULL); their G buffers must differ.
hipError_t launch_bwd_step(const GradArgs* gr, const BwdGArgs* bg, hipStream_t st);

// bf16 gradient outputs: rows x cols fp32 <-> bf16 (round to nearest even),
// row pitch `cols` on both sides; cols a multiple of 8, pointers 16-byte aligned.
hipError_t launch_widen_bf16(const uint16_t* src, float* dst, int64_t rows, int64_t cols, hipStream_t st);
hipError_t launch_narrow_bf16(const float* src, uint16_t* dst, int64_t rows, int64_t cols, hipStream_t st);

// Empty batches: zero `bytes` (a multiple of 16) at p; write one float.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);
hipError_t launch_set_scalar(float* p, float v, hipStream_t st);

}  // namespace lce

// C ABI of the memory-bounded vocabulary projection + cross-entropy: argument
// checks, workspace layout and the host-side schedule of kernel launches.
//
// Schedule (one rank's share of "Flattening Every Memory Peak in Long-Context
// Mixture-of-Experts Training", section 3.2, Ring-DTP):
//   forward   round k = 0..P-1 folds shard order[k] into the per-token
//             running (m, z), and the tile holding a token's target writes
//             its target logit; then a finalize launch merges the split
//             states into lse = m + log z and the token losses, and a
//             one-block launch sums the loss.
//   backward  a preparation launch forms the loss scale and the list of
//             positions the backward runs over (only the tokens whose target
//             is not ignore_index, when leaving the others out saves a token
//             tile; their hidden rows are gathered per token chunk); then for
//             every unit (token chunk, shard in ring order, vocabulary chunk):
//             recompute the logit block from lse and form G in bf16, then
//             dX += G W_chunk and dW_chunk += G^T X_chunk (fp32). One launch
//             runs the GEMMs of unit j - 1 with the recompute of unit j (two
//             G buffers alternate). The GEMMs read W, X and G as they lie in
//             memory; nothing is transposed.
// Transient device memory is O(N) per-token state, the gathered hidden rows
// (at most N x H bf16) and fixed-size G chunks: no logit strip (N x V/P) is
// ever formed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/lce.h"
#include "lce_internal.hpp"

namespace {

constexpr int64_t kTile = 256;
constexpr int64_t kGChunkElems = int64_t(1) << 27;  // bf16 elements of one G chunk (256 MiB)
constexpr int64_t kVocabChunkMax = 16384;           // vocabulary rows per backward chunk
constexpr size_t kGCachedBytes = size_t(64) << 20;  // G chunks up to this size are stored cacheable
constexpr int kMaxSplits = 16;             // forward vocabulary splits per shard
constexpr int kTargetWorkgroups = 256;     // one per compute unit
constexpr int kKnownFlags =
    LCE_FLAG_ACCUMULATE_DX | LCE_FLAG_ACCUMULATE_DW | LCE_FLAG_BF16_GRADS | LCE_FLAG_KEEP_IGNORED_ROWS;

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Plan {
  int64_t N, H, V, P, Vs;
  int64_t n_pad, token_blocks, vocab_tiles;
  int64_t splits, tiles_per_split;
  int64_t vs_pad, vcs, ncs;
  // forward workspace
  size_t off_state, off_yt, off_part, fwd_bytes;
  // backward workspace (off_dx32 / off_dw32: fp32 accumulators for bf16 gradients)
  size_t off_prep, off_tinfo, off_xv, xv_bytes, off_g, g_bytes, off_dx32, off_dw32, bwd_bytes;
  bool xv_whole;  // the gathered hidden rows: all positions at once, or two token chunks
  bool compact;   // the backward may leave ignored tokens out
  size_t state_bytes;  // leading bytes that carry state from one call of a sequence to the next
  bool bf16_grads;
  size_t bytes;
};

int check_dims(const lce_dims* d) {
  if (!d) return fail(LCE_ERR_INVALID_ARG, "dims is NULL");
  if (d->n_tokens < 0) return fail(LCE_ERR_INVALID_ARG, "n_tokens must be >= 0 (got %lld)", (long long)d->n_tokens);
  if (d->hidden < 1) return fail(LCE_ERR_INVALID_ARG, "hidden must be >= 1 (got %lld)", (long long)d->hidden);
  if (d->vocab < 1) return fail(LCE_ERR_INVALID_ARG, "vocab must be >= 1 (got %lld)", (long long)d->vocab);
  if (d->n_shards < 1 || d->n_shards > LCE_MAX_SHARDS)
    return fail(LCE_ERR_INVALID_ARG, "n_shards must be in [1, %d] (got %d)", LCE_MAX_SHARDS, d->n_shards);
  if (d->vocab % d->n_shards)
    return fail(LCE_ERR_INVALID_ARG, "vocab (%lld) is not divisible by n_shards (%d)", (long long)d->vocab,
                d->n_shards);
  if (d->reduction != LCE_REDUCTION_MEAN && d->reduction != LCE_REDUCTION_SUM && d->reduction != LCE_REDUCTION_NONE)
    return fail(LCE_ERR_INVALID_ARG, "reduction must be LCE_REDUCTION_MEAN, _SUM or _NONE (got %d)", d->reduction);
  if (d->flags & ~kKnownFlags) return fail(LCE_ERR_INVALID_ARG, "unknown flag bits 0x%x", d->flags & ~kKnownFlags);
  if (d->hidden % 64) return fail(LCE_ERR_UNSUPPORTED, "hidden (%lld) must be a multiple of 64", (long long)d->hidden);
  const int64_t vs = d->vocab / d->n_shards;
  const int64_t lim = int64_t(1) << 31;
  const int64_t n_pad = round_up(d->n_tokens, kTile);
  if (n_pad * d->hidden >= lim || round_up(vs, kTile) * d->hidden >= lim || n_pad * vs >= lim)
    return fail(LCE_ERR_UNSUPPORTED, "sizes exceed 2^31 elements (N=%lld H=%lld V/P=%lld)",
                (long long)d->n_tokens, (long long)d->hidden, (long long)vs);
  return LCE_OK;
}

Plan make_plan(const lce_dims* d) {
  Plan p{};
  p.N = d->n_tokens;
  p.H = d->hidden;
  p.V = d->vocab;
  p.P = d->n_shards;
  p.Vs = p.V / p.P;
  p.n_pad = round_up(p.N, kTile);
  p.token_blocks = p.n_pad / kTile;
  p.vocab_tiles = ceil_div(p.Vs, kTile);
  // Split each shard's vocabulary tiles: at least 8 ways (the XCD-grouped
  // tile order puts 4 token blocks x 8 splits on an XCD at once), more while
  // the grid would not give every CU a workgroup.
  int64_t s = std::min<int64_t>(
      {kMaxSplits, p.vocab_tiles, std::max<int64_t>(8, ceil_div(kTargetWorkgroups, std::max<int64_t>(1, p.token_blocks)))});
  p.tiles_per_split = ceil_div(p.vocab_tiles, s);
  p.splits = ceil_div(p.vocab_tiles, p.tiles_per_split);
  // Backward chunks (vocabulary rows vc x tokens nc): tile-aligned, balanced,
  // nc * vc within the G-chunk budget and vc within kVocabChunkMax, so the
  // workspace does not grow with V. Each vocabulary chunk reads and writes
  // the whole fp32 dX once, each token chunk after the first the shard's
  // whole fp32 dW: among the admissible shapes take the one that moves the
  // fewest such bytes, preferring fewer token chunks within 2 %.
  p.vs_pad = round_up(p.Vs, kTile);
  p.vcs = std::min(p.vs_pad, kVocabChunkMax);
  p.ncs = p.n_pad;
  if (p.n_pad > 0) {
    struct Shape { int64_t vc, nc, ct; double bytes; };
    std::vector<Shape> shapes;
    const double dx_pass = 8.0 * double(p.N) * double(p.H), dw_pass = 8.0 * double(p.V) * double(p.H);
    for (int64_t cv = ceil_div(p.vs_pad, kVocabChunkMax); cv <= p.vs_pad / kTile; ++cv) {
      const int64_t vc = round_up(ceil_div(p.vs_pad, cv), kTile);
      const int64_t nc_max = kGChunkElems / vc / kTile * kTile;
      if (nc_max < kTile) continue;
      const int64_t ct = ceil_div(p.n_pad, nc_max);
      const int64_t nc = round_up(ceil_div(p.n_pad, ct), kTile);
      shapes.push_back({vc, nc, ct, double(p.P * ceil_div(p.vs_pad, vc)) * dx_pass + double(ct - 1) * dw_pass});
    }
    double best = shapes[0].bytes;
    for (const Shape& sh : shapes) best = std::min(best, sh.bytes);
    const Shape* pick = nullptr;
    for (const Shape& sh : shapes)
      if (sh.bytes <= 1.02 * best && (!pick || sh.ct < pick->ct || (sh.ct == pick->ct && sh.bytes < pick->bytes)))
        pick = &sh;
    p.vcs = pick->vc;
    p.ncs = pick->nc;
  }

  size_t o = 0;
  p.off_state = o;
  o = align256(o + size_t(p.splits) * p.n_pad * 8);
  p.off_yt = o;
  o = align256(o + size_t(p.n_pad) * 4);
  p.off_part = o;
  o = align256(o + size_t(std::max<int64_t>(1, p.token_blocks)) * 16);
  p.fwd_bytes = o;

  // Backward. What persists between the calls of one sequence sits first
  // (the bf16 gradients' dX accumulator), so the state of a sequence is always
  // a prefix of the workspace: state_bytes.
  o = 0;
  p.bf16_grads = (d->flags & LCE_FLAG_BF16_GRADS) != 0;
  p.off_dx32 = p.off_dw32 = 0;
  if (p.bf16_grads) {
    p.off_dx32 = o;
    o = align256(o + size_t(p.N) * p.H * 4);
  }
  const size_t bwd_state = o;
  p.off_prep = o;  // BwdPrep
  o = align256(o + sizeof(lce::BwdPrep));
  p.off_tinfo = o;  // TokInfo per position
  o = align256(o + size_t(p.n_pad) * sizeof(lce::TokInfo));
  // hidden rows of the kept tokens (compact mode): all of them when that is
  // no more than two token chunks, else two token-chunk buffers that the
  // units' chunks alternate in
  // (the dX rows of kept tokens are addressed with 32-bit byte offsets)
  p.compact = (d->flags & LCE_FLAG_KEEP_IGNORED_ROWS) == 0 && p.N * p.H * 4 < (int64_t(1) << 32);
  p.xv_whole = p.N <= 2 * p.ncs;
  p.xv_bytes = !p.compact ? 0 : p.xv_whole ? size_t(p.N) * p.H * 2 : align256(size_t(p.ncs) * p.H * 2);
  p.off_xv = o;
  o = align256(o + (p.xv_whole ? 1 : 2) * p.xv_bytes);
  p.g_bytes = align256(size_t(p.ncs) * p.vcs * 2);
  p.off_g = o;  // two G chunks: consecutive backward units alternate
  o += 2 * p.g_bytes;
  if (p.bf16_grads) {
    p.off_dw32 = o;
    o = align256(o + size_t(p.vcs) * p.H * 4);
  }
  p.state_bytes = std::max(p.fwd_bytes, bwd_state);
  p.bwd_bytes = o;
  p.bytes = std::max(p.fwd_bytes, p.bwd_bytes);
  return p;
}

int check_order(const int32_t* order, int P, int32_t* out) {
  if (!order) {
    for (int k = 0; k < P; ++k) out[k] = (P - k) % P;
    return LCE_OK;
  }
  bool seen[LCE_MAX_SHARDS] = {};
  for (int k = 0; k < P; ++k) {
    const int s = order[k];
    if (s < 0 || s >= P || seen[s])
      return fail(LCE_ERR_INVALID_ARG, "shard_order is not a permutation of 0..%d (entry %d = %d)", P - 1, k, s);
    seen[s] = true;
    out[k] = s;
  }
  return LCE_OK;
}

int check_common(const lce_dims* d, const void* hidden, const void* const* w_shards, const int32_t* targets,
                 void* workspace, size_t workspace_bytes, Plan* plan) {
  int st = check_dims(d);
  if (st) return st;
  if (!w_shards || (d->n_tokens > 0 && (!hidden || !targets)))
    return fail(LCE_ERR_INVALID_ARG, "hidden, w_shards and targets must be non-NULL");
  for (int s = 0; s < d->n_shards; ++s) {
    if (!w_shards[s]) return fail(LCE_ERR_INVALID_ARG, "w_shards[%d] is NULL", s);
    if (!aligned16(w_shards[s])) return fail(LCE_ERR_UNSUPPORTED, "w_shards[%d] is not 16-byte aligned", s);
  }
  if (!aligned16(hidden) || !aligned16(targets)) return fail(LCE_ERR_UNSUPPORTED, "hidden/targets not 16-byte aligned");
  *plan = make_plan(d);
  if (!workspace) return fail(LCE_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned16(workspace)) return fail(LCE_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  if (workspace_bytes < plan->bytes)
    return fail(LCE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, plan->bytes);
  return LCE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return LCE_OK;
  return fail(LCE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- optional per-launch event trace (see lce_trace_enable) ----
enum Kind { kTargetLogit, kFwdRound, kFinalize, kBwdPrep, kGather, kBwdG, kBwdStep, kGradGemm, kConvert, kKinds };
const char* const kKindName[kKinds] = {"target_init", "fwd_round", "finalize", "bwd_prep",     "gather",
                                       "bwd_g",        "bwd_step",  "grad_gemm", "bf16_convert"};

// Algorithmic work of one launch: a fixed part plus, for backward launches,
// parts per position that exist (known on the device only: the positions of
// a unit past the kept-token count do no work), read back when the trace is
// collected.
struct Work {
  double flops = 0.0, bytes = 0.0;
  const lce::BwdPrep* prep = nullptr;
  int n0[2] = {0, 0}, nc[2] = {0, 0};
  double flops_pp[2] = {0.0, 0.0}, bytes_pp[2] = {0.0, 0.0};
  Work() = default;
  Work(double f, double b) : flops(f), bytes(b) {}
};

struct Trace {
  std::vector<hipEvent_t> ev;  // pairs: [2i] before, [2i+1] after launch i
  struct Rec {
    int kind;
    Work work;
  };
  std::vector<Rec> recs;
  int64_t dropped[kKinds] = {};
};
thread_local Trace g_trace;

template <class F>
hipError_t traced(Kind kind, const Work& work, hipStream_t s, F&& launch) {
  Trace& t = g_trace;
  if (t.ev.empty()) return launch();
  const size_t i = t.recs.size();
  if (2 * i + 2 > t.ev.size()) {
    t.dropped[kind]++;
    return launch();
  }
  hipError_t e = hipEventRecord(t.ev[2 * i], s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(t.ev[2 * i + 1], s);
  if (e != hipSuccess) return e;
  t.recs.push_back({int(kind), work});
  return hipSuccess;
}

// ---- shared pieces of the schedule ----------------------------------------

lce::FwdArgs fwd_args(const Plan& p, const lce_dims* d, const void* hidden, const int32_t* targets, char* ws,
                      float* loss, float* lse, float* token_loss) {
  lce::FwdArgs a{};
  a.X = static_cast<const uint16_t*>(hidden);
  a.targets = targets;
  a.yt = reinterpret_cast<float*>(ws + p.off_yt);
  a.state = reinterpret_cast<float2*>(ws + p.off_state);
  a.partials = reinterpret_cast<double2*>(ws + p.off_part);
  a.lse = lse;
  a.token_loss = token_loss;
  a.loss = loss;
  a.N = int(p.N);
  a.H = int(p.H);
  a.Vs = int(p.Vs);
  a.P = int(p.P);
  a.state_ld = int(p.n_pad);
  a.token_blocks = int(p.token_blocks);
  a.S = int(p.splits);
  a.tiles_per_split = int(p.tiles_per_split);
  a.n_vtiles = int(p.vocab_tiles);
  a.ignore_index = d->ignore_index;
  a.reduction = d->reduction;
  return a;
}

int run_init_target_logits(const Plan& p, const lce::FwdArgs& a, hipStream_t s) {
  return hip_status(traced(kTargetLogit, Work(0.0, 8.0 * double(p.N)), s,
                           [&] { return lce::launch_init_target_logits(a.targets, a.N, a.ignore_index, a.yt, s); }),
                    "target logit init");
}

int run_fwd_rounds(const Plan& p, const lce::FwdArgs& a, const lce::ShardTable& by_round, int k0, int k1, int first,
                   hipStream_t s) {
  const double dN = double(p.N), dH = double(p.H), dS = double(p.splits), dVs = double(p.Vs);
  const int nr = k1 - k0;
  const double flops = 2.0 * dN * dVs * dH * nr;
  const double bytes = 2.0 * dN * dH + 2.0 * dVs * dH * nr + (first ? 8.0 : 16.0) * dS * dN;
  return hip_status(
      traced(kFwdRound, Work(flops, bytes), s, [&] { return lce::launch_fwd_rounds(a, by_round, k0, k1, first, s); }),
      "forward rounds");
}

int run_finalize(const Plan& p, const lce::FwdArgs& a, hipStream_t s) {
  return hip_status(traced(kFinalize, Work(0.0, 8.0 * double(p.splits) * double(p.N) + 16.0 * double(p.N)), s,
                           [&] { return lce::launch_finalize(a, s); }),
                    "finalize");
}

// One backward unit: a (vocabulary chunk, token chunk) block of one shard.
// Token chunks are ranges of positions (see lce::BwdPrep).
struct Unit {
  int sh, v0, vc, vc_pad, n0, nc, nc_pad;
  const uint16_t* W;  // the shard
  float* dW;          // fp32 target of the dW contraction for rows v0.. (output, or the chunk accumulator)
  uint16_t* dW_bf16;  // bf16 gradient rows v0.. (LCE_FLAG_BF16_GRADS), else NULL
  int acc_dx, acc_dw;
  bool chunk_first, chunk_last;  // first / last unit of its (shard, vocabulary chunk)
};

// The units of the shards `ids` (in ring order). Each token chunk's first
// unit writes dX (adds, with acc_dx), later ones add; each (shard, vocabulary
// chunk)'s first token chunk writes its dW rows (adds, with acc_dw). With fp32
// gradients the token chunk is the outer loop, so that each chunk's hidden
// rows are gathered once; with bf16 gradients a (shard, vocabulary chunk) runs
// all its token chunks back to back, for its one fp32 accumulator. Every dX
// and dW element gets its terms in the same order either way (shards in ring
// order for dX, token chunks in order for dW), so the results are equal.
std::vector<Unit> backward_units(const Plan& p, const int32_t* ids, int n_ids, const void* const* w_by_id,
                                 void* const* dw_by_id, char* ws, bool acc_dx, bool acc_dw) {
  std::vector<Unit> out;
  std::vector<bool> dx_written(size_t(ceil_div(p.N, p.ncs)), acc_dx);
  auto add = [&](int k, int64_t v0, int64_t n0) {
    const int sh = ids[k];
    const int vc = int(std::min<int64_t>(p.vcs, p.Vs - v0));
    const int nc = int(std::min<int64_t>(p.ncs, p.N - n0));
    const size_t nchunk = size_t(n0 / p.ncs);
    Unit u{sh, int(v0), vc, int(round_up(vc, kTile)), int(n0), nc, int(round_up(nc, kTile)),
           static_cast<const uint16_t*>(w_by_id[k]), nullptr, nullptr, 0, 0, n0 == 0, n0 + p.ncs >= p.N};
    if (p.bf16_grads) {
      u.dW = reinterpret_cast<float*>(ws + p.off_dw32);
      u.dW_bf16 = static_cast<uint16_t*>(dw_by_id[k]) + size_t(v0) * p.H;
    } else {
      u.dW = static_cast<float*>(dw_by_id[k]) + size_t(v0) * p.H;
    }
    u.acc_dx = dx_written[nchunk] ? 1 : 0;
    dx_written[nchunk] = true;
    u.acc_dw = (acc_dw || n0 > 0) ? 1 : 0;
    out.push_back(u);
  };
  if (p.bf16_grads) {
    for (int k = 0; k < n_ids; ++k)
      for (int64_t v0 = 0; v0 < p.Vs; v0 += p.vcs)
        for (int64_t n0 = 0; n0 < p.N; n0 += p.ncs) add(k, v0, n0);
  } else {
    for (int64_t n0 = 0; n0 < p.N; n0 += p.ncs)
      for (int k = 0; k < n_ids; ++k)
        for (int64_t v0 = 0; v0 < p.Vs; v0 += p.vcs) add(k, v0, n0);
  }
  return out;
}

// Token info of the positions the backward runs over (kept tokens only when
// that saves a token tile) and the loss scale.
int run_bwd_prep(const Plan& p, const lce_dims* d, const int32_t* targets, const float* lse, const float* dloss,
                 char* ws, hipStream_t s) {
  lce::BwdPrep* prep = reinterpret_cast<lce::BwdPrep*>(ws + p.off_prep);
  lce::TokInfo* tinfo = reinterpret_cast<lce::TokInfo*>(ws + p.off_tinfo);
  int st = hip_status(traced(kBwdPrep, Work(0.0, 4.0 * double(p.N) + 16.0 * double(p.N)), s,
                             [&] {
                               return lce::launch_bwd_prep(targets, lse, int(p.N), d->ignore_index, dloss,
                                                           d->reduction, p.compact ? 1 : 0, prep, tinfo, s);
                             }),
                      "backward preparation");
  return st;
}

int run_convert(bool widen, const void* src, void* dst, int64_t rows, int64_t cols, hipStream_t s) {
  const double n = double(rows) * double(cols);
  return hip_status(traced(kConvert, Work(0.0, 6.0 * n), s,
                           [&] {
                             return widen ? lce::launch_widen_bf16(static_cast<const uint16_t*>(src),
                                                                   static_cast<float*>(dst), rows, cols, s)
                                          : lce::launch_narrow_bf16(static_cast<const float*>(src),
                                                                    static_cast<uint16_t*>(dst), rows, cols, s);
                           }),
                    widen ? "widen" : "narrow");
}

// Launch j runs the gradient GEMMs of unit j - 1 and the recompute of unit j.
// With bf16 gradients each vocabulary chunk's dW accumulates in the chunk
// accumulator and is narrowed into the caller's buffer after the launch that
// ends it (and, when accumulating, widened from it before the launch that
// starts it). In compact mode the units read their token chunk's hidden rows
// from a gathered copy: all positions in one buffer when they fit
// (xv_whole), else two chunk buffers; a unit whose chunk is not in a buffer
// gets it gathered, before its recompute launch, into the buffer the
// previous unit does not use (whose GEMMs run in that same launch). The first
// gather also zeroes the ignored tokens' rows of `dx_zero` (NULL: leave them,
// when accumulating): in compact mode no contraction writes them.
int run_bwd_units(const Plan& p, const lce_dims* d, const std::vector<Unit>& units, const uint16_t* X,
                  const int32_t* targets, float* dX, float* dx_zero, bool acc_dw, char* ws, hipStream_t s) {
  const double dH = double(p.H);
  auto gbuf = [&](size_t u) { return reinterpret_cast<uint16_t*>(ws + p.off_g + (u & 1) * p.g_bytes); };
  float* dw32 = reinterpret_cast<float*>(ws + p.off_dw32);
  const lce::BwdPrep* prep = reinterpret_cast<const lce::BwdPrep*>(ws + p.off_prep);
  const lce::TokInfo* tinfo = reinterpret_cast<const lce::TokInfo*>(ws + p.off_tinfo);
  uint16_t* xv_base = reinterpret_cast<uint16_t*>(ws + p.off_xv);
  bool zero_pending = dx_zero != nullptr;
  auto gather = [&](uint16_t* dst, int n0, int nc) {
    float* z = zero_pending ? dx_zero : nullptr;
    zero_pending = false;
    return hip_status(traced(kGather, Work(0.0, 4.0 * double(nc) * dH), s,
                             [&] {
                               return lce::launch_gather_rows(X, dst, prep, tinfo, n0, nc, int(p.H), z, targets,
                                                              int(p.N), d->ignore_index, s);
                             }),
                      "gather rows");
  };
  // the gathered rows of each unit's positions
  std::vector<uint16_t*> xv(units.size());
  std::vector<int> gather_before(units.size(), -1);  // launch j gathers unit j's chunk first
  int st;
  if (!p.compact) {
    for (size_t j = 0; j < units.size(); ++j) xv[j] = nullptr;  // the kernels read X
  } else if (p.xv_whole) {
    st = gather(xv_base, 0, int(p.N));
    if (st) return st;
    for (size_t j = 0; j < units.size(); ++j) xv[j] = xv_base + size_t(units[j].n0) * p.H;
  } else {
    int held[2] = {-1, -1}, prev = 1;
    for (size_t j = 0; j < units.size(); ++j) {
      int b = held[0] == units[j].n0 ? 0 : held[1] == units[j].n0 ? 1 : -1;
      if (b < 0) {
        b = prev ^ 1;
        held[b] = units[j].n0;
        gather_before[j] = b;
      }
      xv[j] = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(xv_base) + b * p.xv_bytes);
      prev = b;
    }
  }
  if (!units.empty() && units[0].dW_bf16 && acc_dw) {
    st = run_convert(true, units[0].dW_bf16, dw32, units[0].vc, p.H, s);
    if (st) return st;
  }
  for (size_t j = 0; j <= units.size(); ++j) {
    if (j < units.size() && gather_before[j] >= 0) {
      st = gather(xv[j], units[j].n0, units[j].nc);
      if (st) return st;
    }
    lce::GradArgs ga{};
    lce::BwdGArgs ba{};
    Work work;
    work.prep = prep;
    if (j > 0) {
      const Unit& u = units[j - 1];
      ga.G = gbuf(j - 1);
      ga.ldg = u.vc_pad;
      ga.nc_pad = u.nc_pad;
      ga.vc_pad = u.vc_pad;
      ga.Wc = u.W + size_t(u.v0) * p.H;
      ga.vc = u.vc;
      ga.X = X;
      ga.xv = xv[j - 1];
      ga.prep = prep;
      ga.tinfo = tinfo;
      ga.n0 = u.n0;
      ga.nc = u.nc;
      ga.H = int(p.H);
      ga.dX = dX;
      ga.acc_dx = u.acc_dx;
      ga.dW = u.dW;
      ga.acc_dw = u.acc_dw;
      // per position: the two contractions, G read twice, the position's X
      // row and dX row (read when adding); fixed: the W chunk, the dW rows
      const double dvc = u.vc;
      work.n0[0] = u.n0;
      work.nc[0] = u.nc;
      work.flops_pp[0] = 4.0 * dvc * dH;
      work.bytes_pp[0] = 4.0 * double(u.vc_pad) + 2.0 * dH + (4.0 + 4.0 * u.acc_dx) * dH;
      work.bytes += 2.0 * dvc * dH + (4.0 + 4.0 * u.acc_dw) * dvc * dH;
    }
    if (j < units.size()) {
      const Unit& u = units[j];
      ba.X = X;
      ba.xv = xv[j];
      ba.prep = prep;
      ba.tinfo = tinfo;
      ba.Ws = u.W;
      ba.G = gbuf(j);
      ba.H = int(p.H);
      ba.Vs = int(p.Vs);
      ba.v0 = u.v0;
      ba.vc = u.vc;
      ba.n0 = u.n0;
      ba.nc = u.nc;
      ba.nc_pad = u.nc_pad;
      ba.vc_pad = u.vc_pad;
      ba.ignore_index = d->ignore_index;
      ba.vocab_base = int(u.sh * p.Vs + u.v0);
      ba.V = int(p.V);
      ba.ldg = u.vc_pad;
      // G chunks up to a quarter of the 256 MB last-level cache stay cached
      // for the next launch's reads
      ba.g_cached = size_t(u.nc_pad) * size_t(u.vc_pad) * 2 <= kGCachedBytes ? 1 : 0;
      // per position: the recompute, its X row, its G row, its token info;
      // fixed: the W chunk
      const double dvc = u.vc;
      work.n0[1] = u.n0;
      work.nc[1] = u.nc;
      work.flops_pp[1] = 2.0 * dvc * dH;
      work.bytes_pp[1] = 2.0 * dH + 2.0 * double(u.vc_pad) + 16.0;
      work.bytes += 2.0 * dvc * dH;
    }
    const Kind kind = j == 0 ? kBwdG : (j == units.size() ? kGradGemm : kBwdStep);
    st = hip_status(traced(kind, work, s,
                           [&] {
                             return lce::launch_bwd_step(j > 0 ? &ga : nullptr, j < units.size() ? &ba : nullptr,
                                                         s);
                           }),
                    "backward step");
    if (st) return st;
    if (j > 0 && units[j - 1].dW_bf16 && units[j - 1].chunk_last) {
      st = run_convert(false, dw32, units[j - 1].dW_bf16, units[j - 1].vc, p.H, s);
      if (st) return st;
    }
    if (j > 0 && j < units.size() && units[j].dW_bf16 && units[j].chunk_first && acc_dw) {
      st = run_convert(true, units[j].dW_bf16, dw32, units[j].vc, p.H, s);
      if (st) return st;
    }
  }
  return LCE_OK;
}

// Empty batch (N = 0): the loss is the mean of no tokens (NaN, as 0/0) or a
// sum of none (0); a shard gradient is zero.
int run_empty_loss(const lce_dims* d, float* loss, hipStream_t s) {
  const float v = d->reduction == LCE_REDUCTION_MEAN ? __builtin_nanf("") : 0.0f;
  return hip_status(traced(kFinalize, Work(0.0, 4.0), s, [&] { return lce::launch_set_scalar(loss, v, s); }), "empty loss");
}

int run_zero(const Plan& p, void* d_w_shard, hipStream_t s) {
  const size_t bytes = size_t(p.Vs) * p.H * (p.bf16_grads ? 2 : 4);
  return hip_status(traced(kConvert, Work(0.0, double(bytes)), s, [&] { return lce::launch_zero(d_w_shard, bytes, s); }),
                    "zero gradient");
}

int check_round_args(const lce_dims* d, int round, int shard_index, const void* hidden, const void* w_shard,
                     const int32_t* targets, void* workspace, size_t workspace_bytes, Plan* plan) {
  int st = check_dims(d);
  if (st) return st;
  if (round < 0 || round >= d->n_shards)
    return fail(LCE_ERR_INVALID_ARG, "round must be in [0, %d) (got %d)", d->n_shards, round);
  if (shard_index < 0 || shard_index >= d->n_shards)
    return fail(LCE_ERR_INVALID_ARG, "shard_index must be in [0, %d) (got %d)", d->n_shards, shard_index);
  if (!w_shard || (d->n_tokens > 0 && (!hidden || !targets)))
    return fail(LCE_ERR_INVALID_ARG, "hidden, w_shard and targets must be non-NULL");
  if (!aligned16(w_shard) || !aligned16(hidden) || !aligned16(targets))
    return fail(LCE_ERR_UNSUPPORTED, "hidden/w_shard/targets not 16-byte aligned");
  *plan = make_plan(d);
  if (!workspace) return fail(LCE_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned16(workspace)) return fail(LCE_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  if (workspace_bytes < plan->bytes)
    return fail(LCE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, plan->bytes);
  return LCE_OK;
}

}  // namespace

extern "C" {

size_t lce_workspace_bytes(const lce_dims* dims) {
  if (check_dims(dims) != LCE_OK) return 0;
  return make_plan(dims).bytes;
}

size_t lce_state_bytes(const lce_dims* dims) {
  if (check_dims(dims) != LCE_OK) return 0;
  return make_plan(dims).state_bytes;
}

int lce_ring_payload(const lce_dims* d, size_t* weight_bytes, size_t* activation_bytes) {
  int st = check_dims(d);
  if (st) return st;
  const Plan p = make_plan(d);
  const size_t gb = p.bf16_grads ? 2 : 4;  // bytes of a gradient element
  // one hop of the forward plus one of the backward
  const size_t w = size_t(p.Vs) * p.H * 2 * 2 + size_t(p.Vs) * p.H * gb;
  const size_t x = size_t(p.N) * p.H * 2 * 2 + size_t(p.N) * 4 * 2 + p.fwd_bytes + size_t(p.N) * 4 +
                   size_t(p.N) * p.H * 4;
  if (weight_bytes) *weight_bytes = w;
  if (activation_bytes) *activation_bytes = x;
  return x < w ? LCE_PAYLOAD_ACTIVATIONS : LCE_PAYLOAD_WEIGHTS;
}

}  // extern "C"

namespace {

// Argument checks of the forward that do not involve the workspace.
int check_forward(const lce_dims* d, const void* hidden, const void* const* w_shards, const int32_t* shard_order,
                  const int32_t* targets, float* loss, float* lse, float* token_loss, int32_t* order, Plan* p) {
  int st = check_dims(d);
  if (st) return st;
  if (!w_shards || (d->n_tokens > 0 && (!hidden || !targets)))
    return fail(LCE_ERR_INVALID_ARG, "hidden, w_shards and targets must be non-NULL");
  for (int s = 0; s < d->n_shards; ++s) {
    if (!w_shards[s]) return fail(LCE_ERR_INVALID_ARG, "w_shards[%d] is NULL", s);
    if (!aligned16(w_shards[s])) return fail(LCE_ERR_UNSUPPORTED, "w_shards[%d] is not 16-byte aligned", s);
  }
  if (!aligned16(hidden) || !aligned16(targets)) return fail(LCE_ERR_UNSUPPORTED, "hidden/targets not 16-byte aligned");
  if (!loss || (d->n_tokens > 0 && !lse)) return fail(LCE_ERR_INVALID_ARG, "loss and lse must be non-NULL");
  if (d->n_tokens > 0 && !token_loss && d->reduction == LCE_REDUCTION_NONE)
    return fail(LCE_ERR_INVALID_ARG, "token_loss must be non-NULL for LCE_REDUCTION_NONE");
  if (!aligned16(lse) || (token_loss && !aligned16(token_loss)))
    return fail(LCE_ERR_UNSUPPORTED, "lse/token_loss not 16-byte aligned");
  st = check_order(shard_order, d->n_shards, order);
  if (st) return st;
  *p = make_plan(d);
  return LCE_OK;
}

// The forward schedule on a checked workspace of at least p.fwd_bytes.
int run_forward(const Plan& p, const lce_dims* d, const void* hidden, const void* const* w_shards,
                const int32_t* order, const int32_t* targets, float* loss, float* lse, float* token_loss, char* ws,
                hipStream_t s) {
  if (d->n_tokens == 0) return run_empty_loss(d, loss, s);
  lce::ShardTable by_round{};
  for (int k = 0; k < d->n_shards; ++k) {
    by_round.p[k] = static_cast<const uint16_t*>(w_shards[order[k]]);
    by_round.id[k] = order[k];
  }
  const lce::FwdArgs a = fwd_args(p, d, hidden, targets, ws, loss, lse, token_loss);
  int st = run_init_target_logits(p, a, s);
  if (st) return st;
  // All rounds in one launch when every workgroup is resident at once (its
  // state then stays in registers); else one launch per round.
  const int P = d->n_shards;
  const int per_launch = p.token_blocks * p.splits <= kTargetWorkgroups ? P : 1;
  for (int k = 0; k < P; k += per_launch) {
    const int k1 = std::min(P, k + per_launch);
    st = run_fwd_rounds(p, a, by_round, k, k1, k == 0, s);
    if (st) return st;
  }
  return run_finalize(p, a, s);
}

// ---- the forward without a caller workspace --------------------------------
// For callers that cannot allocate device memory: the forward's scratch (split
// states, target logits, loss partials) lives in this file-scope array, one
// copy per GPU, held until the process ends. In host code `scratch` is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress,
// fetched once per device (with that device current) and kept in
// g_scratch_addr; only that address ever reaches a kernel.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = -1;
  int st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(LCE_ERR_UNSUPPORTED, "device %d is beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* addr = nullptr;
    st = hip_status(hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st) return st;
    if (!addr) return fail(LCE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_addr[dev] = addr;
  }
  *out = g_scratch_addr[dev];
  return LCE_OK;
}

}  // namespace

extern "C" {

int lce_forward(const lce_dims* d, const void* hidden, const void* const* w_shards, const int32_t* shard_order,
                const int32_t* targets, float* loss, float* lse, float* token_loss, void* workspace,
                size_t workspace_bytes, void* stream) {
  Plan p;
  int32_t order[LCE_MAX_SHARDS];
  int st = check_forward(d, hidden, w_shards, shard_order, targets, loss, lse, token_loss, order, &p);
  if (st) return st;
  if (!workspace) return fail(LCE_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned16(workspace)) return fail(LCE_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  // the forward uses only its own leading part of the workspace
  if (workspace_bytes < p.fwd_bytes)
    return fail(LCE_ERR_WORKSPACE, "workspace has %zu bytes, the forward needs %zu", workspace_bytes, p.fwd_bytes);
  g_last_error.clear();
  return run_forward(p, d, hidden, w_shards, order, targets, loss, lse, token_loss, static_cast<char*>(workspace),
                     reinterpret_cast<hipStream_t>(stream));
}

size_t lce_forward_noalloc_max_bytes(void) { return kStaticScratchBytes; }

int lce_forward_noalloc(const lce_dims* d, const void* hidden, const void* const* w_shards, const int32_t* shard_order,
                        const int32_t* targets, float* loss, float* lse, float* token_loss, void* stream) {
  Plan p;
  int32_t order[LCE_MAX_SHARDS];
  int st = check_forward(d, hidden, w_shards, shard_order, targets, loss, lse, token_loss, order, &p);
  if (st) return st;
  if (p.fwd_bytes > kStaticScratchBytes)
    return fail(LCE_ERR_WORKSPACE,
                "the forward needs %zu bytes of scratch for N=%lld (%lld splits); the built-in scratch holds %zu",
                p.fwd_bytes, (long long)p.N, (long long)p.splits, kStaticScratchBytes);
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st) return st;
  g_last_error.clear();
  return run_forward(p, d, hidden, w_shards, order, targets, loss, lse, token_loss, static_cast<char*>(ws),
                     reinterpret_cast<hipStream_t>(stream));
}

int lce_backward(const lce_dims* d, const void* hidden, const void* const* w_shards, const int32_t* shard_order,
                 const int32_t* targets, const float* lse, const float* dloss, void* d_hidden,
                 void* const* d_w_shards, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int st = check_common(d, hidden, w_shards, targets, workspace, workspace_bytes, &p);
  if (st) return st;
  if (!d_w_shards || (d->n_tokens > 0 && (!lse || !dloss || !d_hidden)))
    return fail(LCE_ERR_INVALID_ARG, "lse, dloss, d_hidden and d_w_shards must be non-NULL");
  if (!aligned16(lse) || !aligned16(d_hidden)) return fail(LCE_ERR_UNSUPPORTED, "lse/d_hidden not 16-byte aligned");
  for (int k = 0; k < d->n_shards; ++k) {
    if (!d_w_shards[k]) return fail(LCE_ERR_INVALID_ARG, "d_w_shards[%d] is NULL", k);
    if (!aligned16(d_w_shards[k])) return fail(LCE_ERR_UNSUPPORTED, "d_w_shards[%d] is not 16-byte aligned", k);
  }
  int32_t order[LCE_MAX_SHARDS];
  st = check_order(shard_order, d->n_shards, order);
  if (st) return st;
  g_last_error.clear();

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bool acc_dx = (d->flags & LCE_FLAG_ACCUMULATE_DX) != 0, acc_dw = (d->flags & LCE_FLAG_ACCUMULATE_DW) != 0;
  if (d->n_tokens == 0) {  // no tokens: the shard gradients are zero (or unchanged when accumulating)
    for (int k = 0; k < d->n_shards && !acc_dw; ++k) {
      st = run_zero(p, d_w_shards[k], s);
      if (st) return st;
    }
    return LCE_OK;
  }
  float* dx32 = p.bf16_grads ? reinterpret_cast<float*>(ws + p.off_dx32) : static_cast<float*>(d_hidden);
  if (p.bf16_grads && acc_dx) {
    st = run_convert(true, d_hidden, dx32, p.N, p.H, s);
    if (st) return st;
  }
  st = run_bwd_prep(p, d, targets, lse, dloss, ws, s);
  if (st) return st;
  const void* w_by_round[LCE_MAX_SHARDS];
  void* dw_by_round[LCE_MAX_SHARDS];
  for (int k = 0; k < d->n_shards; ++k) {
    w_by_round[k] = w_shards[order[k]];
    dw_by_round[k] = d_w_shards[order[k]];
  }
  const std::vector<Unit> units = backward_units(p, order, d->n_shards, w_by_round, dw_by_round, ws, acc_dx, acc_dw);
  st = run_bwd_units(p, d, units, static_cast<const uint16_t*>(hidden), targets, dx32, acc_dx ? nullptr : dx32, acc_dw,
                     ws, s);
  if (st || !p.bf16_grads) return st;
  return run_convert(false, dx32, d_hidden, p.N, p.H, s);
}

int lce_fwd_round(const lce_dims* d, int round, int shard_index, const void* hidden, const void* w_shard,
                  const int32_t* targets, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int st = check_round_args(d, round, shard_index, hidden, w_shard, targets, workspace, workspace_bytes, &p);
  if (st) return st;
  g_last_error.clear();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  lce::ShardTable by_round{};
  by_round.p[0] = static_cast<const uint16_t*>(w_shard);
  by_round.id[0] = shard_index;
  const lce::FwdArgs a = fwd_args(p, d, hidden, targets, ws, nullptr, nullptr, nullptr);
  if (d->n_tokens == 0) return LCE_OK;  // nothing to fold
  if (round == 0) {
    st = run_init_target_logits(p, a, s);
    if (st) return st;
  }
  return run_fwd_rounds(p, a, by_round, 0, 1, round == 0, s);
}

int lce_fwd_finish(const lce_dims* d, const int32_t* targets, float* loss, float* lse, float* token_loss,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (!loss || !workspace || (d->n_tokens > 0 && (!targets || !lse)))
    return fail(LCE_ERR_INVALID_ARG, "targets, loss, lse and workspace must be non-NULL");
  if (d->n_tokens > 0 && !token_loss && d->reduction == LCE_REDUCTION_NONE)
    return fail(LCE_ERR_INVALID_ARG, "token_loss must be non-NULL for LCE_REDUCTION_NONE");
  if (!aligned16(targets) || !aligned16(lse) || (token_loss && !aligned16(token_loss)) || !aligned16(workspace))
    return fail(LCE_ERR_UNSUPPORTED, "targets/lse/token_loss/workspace not 16-byte aligned");
  const Plan p = make_plan(d);
  if (workspace_bytes < p.bytes) return fail(LCE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, p.bytes);
  g_last_error.clear();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d->n_tokens == 0) return run_empty_loss(d, loss, s);
  const lce::FwdArgs a = fwd_args(p, d, nullptr, targets, static_cast<char*>(workspace), loss, lse, token_loss);
  return run_finalize(p, a, s);
}

int lce_bwd_round(const lce_dims* d, int round, int shard_index, const void* hidden, const void* w_shard,
                  const int32_t* targets, const float* lse, const float* dloss, void* d_hidden, void* d_w_shard,
                  int accumulate_dw, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int st = check_round_args(d, round, shard_index, hidden, w_shard, targets, workspace, workspace_bytes, &p);
  if (st) return st;
  if (!d_w_shard || (d->n_tokens > 0 && (!lse || !dloss || !d_hidden)))
    return fail(LCE_ERR_INVALID_ARG, "lse, dloss, d_hidden and d_w_shard must be non-NULL");
  if (!aligned16(lse) || !aligned16(d_hidden) || !aligned16(d_w_shard))
    return fail(LCE_ERR_UNSUPPORTED, "lse/d_hidden/d_w_shard not 16-byte aligned");
  g_last_error.clear();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bool acc_dx = round > 0 || (d->flags & LCE_FLAG_ACCUMULATE_DX) != 0;
  const bool acc_dw = accumulate_dw != 0 || (d->flags & LCE_FLAG_ACCUMULATE_DW) != 0;
  if (d->n_tokens == 0) return acc_dw ? LCE_OK : run_zero(p, d_w_shard, s);
  float* dx32 = p.bf16_grads ? reinterpret_cast<float*>(ws + p.off_dx32) : static_cast<float*>(d_hidden);
  if (p.bf16_grads && round == 0 && acc_dx) {
    st = run_convert(true, d_hidden, dx32, p.N, p.H, s);
    if (st) return st;
  }
  st = run_bwd_prep(p, d, targets, lse, dloss, ws, s);
  if (st) return st;
  const int32_t id = shard_index;
  const void* w_one[1] = {w_shard};
  void* dw_one[1] = {d_w_shard};
  const std::vector<Unit> units = backward_units(p, &id, 1, w_one, dw_one, ws, acc_dx, acc_dw);
  st = run_bwd_units(p, d, units, static_cast<const uint16_t*>(hidden), targets, dx32, acc_dx ? nullptr : dx32, acc_dw,
                     ws, s);
  if (st || !p.bf16_grads || round != d->n_shards - 1) return st;
  return run_convert(false, dx32, d_hidden, p.N, p.H, s);
}

int lce_trace_enable(int capacity) {
  Trace& t = g_trace;
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.clear();
  t.recs.clear();
  for (auto& d : t.dropped) d = 0;
  if (capacity < 0) return fail(LCE_ERR_INVALID_ARG, "trace capacity must be >= 0");
  t.ev.resize(size_t(2) * capacity);
  for (auto& e : t.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      t.ev.clear();
      return hip_status(r, "hipEventCreate");
    }
  }
  t.recs.reserve(capacity);
  return LCE_OK;
}

int lce_trace_collect(lce_trace_entry* out, int max_entries) {
  Trace& t = g_trace;
  if (max_entries > 0 && !out) return fail(LCE_ERR_INVALID_ARG, "out is NULL");
  lce_trace_entry agg[kKinds];
  std::memset(agg, 0, sizeof agg);
  for (int k = 0; k < kKinds; ++k) {
    std::snprintf(agg[k].name, sizeof agg[k].name, "%s", kKindName[k]);
    agg[k].dropped = t.dropped[k];
  }
  if (!t.recs.empty()) {
    int st = hip_status(hipEventSynchronize(t.ev[2 * t.recs.size() - 1]), "hipEventSynchronize");
    if (st) return st;
  }
  // positions that exist, per backward preparation record (as it stands now:
  // the last backward on that workspace)
  std::vector<std::pair<const lce::BwdPrep*, int>> n_eff;
  auto positions = [&](const lce::BwdPrep* prep, int* n) {
    for (const auto& e : n_eff)
      if (e.first == prep) {
        *n = e.second;
        return LCE_OK;
      }
    lce::BwdPrep host{};
    int st = hip_status(hipMemcpy(&host, prep, sizeof host, hipMemcpyDeviceToHost), "hipMemcpy(trace)");
    if (st) return st;
    n_eff.push_back({prep, host.n_eff});
    *n = host.n_eff;
    return LCE_OK;
  };
  for (size_t i = 0; i < t.recs.size(); ++i) {
    float ms = 0.0f;
    int st = hip_status(hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]), "hipEventElapsedTime");
    if (st) return st;
    const Work& w = t.recs[i].work;
    double flops = w.flops, bytes = w.bytes;
    if (w.prep) {
      int n = 0;
      st = positions(w.prep, &n);
      if (st) return st;
      for (int h = 0; h < 2; ++h) {
        const double live = double(std::max(0, std::min(w.nc[h], n - w.n0[h])));
        flops += w.flops_pp[h] * live;
        bytes += w.bytes_pp[h] * live;
      }
    }
    lce_trace_entry& a = agg[t.recs[i].kind];
    a.launches += 1;
    a.total_ms += ms;
    a.flops += flops;
    a.bytes += bytes;
  }
  int n = 0;
  for (int k = 0; k < kKinds; ++k) {
    if (agg[k].launches == 0 && agg[k].dropped == 0) continue;
    if (n < max_entries) out[n] = agg[k];
    ++n;
  }
  t.recs.clear();
  for (auto& d : t.dropped) d = 0;
  return n;
}

const char* lce_status_string(int status) {
  switch (status) {
    case LCE_OK: return "ok";
    case LCE_ERR_INVALID_ARG: return "invalid argument";
    case LCE_ERR_UNSUPPORTED: return "unsupported size or alignment";
    case LCE_ERR_WORKSPACE: return "workspace too small";
    case LCE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* lce_last_error(void) { return g_last_error.c_str(); }

int lce_version(void) { return (1 << 16) | 2; }

}  // extern "C"

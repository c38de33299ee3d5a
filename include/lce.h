/*
 * lce.h - memory-bounded vocabulary projection + cross-entropy on MI355X (C ABI).
 *
 * Computes the exact cross-entropy of the logits X W^T, where the vocabulary
 * weight W (V x H) arrives as P column shards (contiguous vocabulary
 * intervals of V/P ids), and its gradients, without ever forming the N x V
 * logit tensor. This is one rank's share of the ring data-tensor-parallel
 * vocabulary projection of "Flattening Every Memory Peak in Long-Context
 * Mixture-of-Experts Training", section 3.2 (Ring-DTP). The rank's batch is
 * multiplied by one shard after another, in ring delivery order; every
 * product tile updates a per-token running maximum m and exponential sum z
 * (online softmax, Eq. 3 of that section) and is then dropped. With
 * lse_i = m_i + log z_i, token i's loss is lse_i - y_{t_i}. The backward
 * rebuilds each logit tile from X, W and the stored lse (fp32, one value per
 * token). Loss and gradients equal those of the plain full-logit
 * cross-entropy up to floating-point rounding order (the exactness condition
 * in the introduction to section 3).
 *
 * Conventions shared by every entry point:
 *  - Pointers marked "device" are HIP device pointers; "host" pointers are
 *    read before the call returns. The caller owns and frees every buffer,
 *    including the workspace; the library never allocates device memory and
 *    never synchronizes the stream.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *    Results are valid once the stream reaches the enqueued work.
 *  - Every argument check runs on the host before any GPU work is enqueued;
 *    a failed check returns a negative status and enqueues nothing.
 *  - Layouts: hidden bf16 [N][H] row-major; shard s bf16 [V/P][H] row-major,
 *    holding vocabulary ids [s*V/P, (s+1)*V/P); targets int32 [N].
 *    bf16 is passed as raw 16-bit patterns.
 *  - Alignment: every device pointer must be 16-byte aligned. H must be a
 *    positive multiple of 64.
 *  - Limits: N*H, (V/P)*H and N*(V/P) below 2^31 elements; 1 <= P <= 256.
 *  - Calls are thread-safe; concurrent calls need distinct workspaces.
 *  - An empty batch (N = 0) is valid: the per-token pointers (hidden,
 *    targets, lse, token_loss, d_hidden, a per-token dloss) may be NULL; the
 *    loss is NaN for a mean over no tokens and 0 for a sum; the shard
 *    gradients are zero (left unchanged when accumulating).
 */
#ifndef LCE_H
#define LCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef LCE_API
#define LCE_API __attribute__((visibility("default")))
#endif

#define LCE_OK 0
#define LCE_ERR_INVALID_ARG (-1) /* null pointer, bad size, order not a permutation */
#define LCE_ERR_UNSUPPORTED (-2) /* H not a multiple of 64, misaligned pointer, size limit */
#define LCE_ERR_WORKSPACE (-3)   /* workspace smaller than lce_workspace_bytes() */
#define LCE_ERR_HIP (-4)         /* a HIP launch failed; see lce_last_error() */

#define LCE_REDUCTION_MEAN 0 /* mean over tokens whose target != ignore_index */
#define LCE_REDUCTION_SUM 1  /* sum over tokens whose target != ignore_index */
#define LCE_REDUCTION_NONE 2 /* per token: token_loss is the result (loss gets
                                their sum); backward takes a per-token dloss [N] */

/* lce_dims.flags bits */
#define LCE_FLAG_ACCUMULATE_DX 1 /* backward adds into d_hidden instead of overwriting it */
#define LCE_FLAG_ACCUMULATE_DW 2 /* backward adds into the shard gradients */
#define LCE_FLAG_BF16_GRADS 4    /* d_hidden and the shard gradients are bf16 (accumulated
                                    in fp32 inside the workspace, rounded once at the end) */
#define LCE_FLAG_KEEP_IGNORED_ROWS 8 /* the backward runs over every token, ignored ones
                                        included (their gradient rows are zero either way):
                                        no gathered copy of the hidden rows in the workspace,
                                        so less memory, and more time when ignored tokens
                                        would have saved a 256-token tile */

#define LCE_MAX_SHARDS 256

typedef struct lce_dims {
  int64_t n_tokens;     /* N >= 0 (an empty batch: see below) */
  int64_t hidden;       /* H >= 64, multiple of 64 */
  int64_t vocab;        /* V >= 1, divisible by n_shards */
  int32_t n_shards;     /* P, 1..LCE_MAX_SHARDS */
  int32_t ignore_index; /* targets equal to this are skipped (e.g. -100) */
  int32_t reduction;    /* LCE_REDUCTION_MEAN, _SUM or _NONE */
  int32_t flags;        /* LCE_FLAG_* bits; other bits must be 0 */
} lce_dims;

/*
 * Bytes of device workspace lce_forward and lce_backward need for `dims`.
 * Pure host function. The size is bounded independently of V: it holds
 * per-token state (O(N)), a bf16 copy of hidden rows whose target is not
 * ignore_index (the backward leaves ignored tokens out when that saves a
 * 256-token tile; at most N x H, or two token chunks of rows when that is
 * less; none with LCE_FLAG_KEEP_IGNORED_ROWS) and two gradient chunks of at
 * most 2^27 bf16 elements each (fixed-size, whatever N and V), never a logit
 * strip; with
 * LCE_FLAG_BF16_GRADS also fp32 accumulators for d_hidden (N x H) and one
 * gradient chunk (at most 16384 x H).
 * Returns 0 if dims is invalid.
 */
LCE_API size_t lce_workspace_bytes(const lce_dims* dims);

/*
 * Forward: loss and lse (the per-token log-sum-exp the backward reuses).
 *  hidden       device bf16 [N][H]
 *  w_shards     host array of P device pointers, each bf16 [V/P][H]
 *  shard_order  host int32 [P], a permutation of 0..P-1: round k meets shard
 *               shard_order[k]. NULL = the ring order of rank 0, k -> (P-k) % P.
 *               The result does not depend on the order except for fp32
 *               rounding.
 *  targets      device int32 [N]; ids in [0, V) or ignore_index. An id outside
 *               [0, V) that is not ignore_index makes that token's loss NaN
 *               (and so the mean); no host synchronization is done to detect it.
 *  loss         device fp32 scalar, written: mean (or sum) over non-ignored
 *               tokens; NaN for a mean over zero tokens. With
 *               LCE_REDUCTION_NONE the sum (token_loss is then the result).
 *  lse          device fp32 [N], written: log-sum-exp of each token's full
 *               logit row (every token, ignored ones included). Keep it for
 *               lce_backward: it is the only state backward needs.
 *  token_loss   device fp32 [N] or NULL (required for LCE_REDUCTION_NONE);
 *               written: lse - target logit, 0 for ignored tokens.
 *  workspace    device buffer of at least lce_workspace_bytes(dims) bytes
 *               (the size both passes need); the forward itself uses and
 *               checks only its leading part, lce_state_bytes(dims) of dims
 *               without flags, so one workspace sized for a backward with
 *               any flags serves it.
 */
LCE_API int lce_forward(const lce_dims* dims, const void* hidden, const void* const* w_shards, const int32_t* shard_order,
                const int32_t* targets, float* loss, float* lse, float* token_loss, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * Forward without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, kernels and results as lce_forward (bit
 * for bit), but the forward's scratch (per-token split states, target logits,
 * loss partials: the first part of lce_workspace_bytes) comes from a
 * fixed-size device array built into the library, one copy per GPU, held
 * until the process ends; lce_forward_noalloc_max_bytes() gives its size
 * (32 MiB: N up to about 250 000 tokens). The call allocates nothing: the
 * array's device address is looked up once per device, on the first call with
 * that device current (the stream must belong to the current device).
 * Returns LCE_ERR_WORKSPACE, enqueuing nothing, when the batch needs more
 * scratch than the array holds. Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (two streams, or two threads) race and
 * must be ordered by the caller. Nothing in the array needs to start at zero:
 * each call writes what it reads.
 */
LCE_API int lce_forward_noalloc(const lce_dims* dims, const void* hidden, const void* const* w_shards,
                                const int32_t* shard_order, const int32_t* targets, float* loss, float* lse,
                                float* token_loss, void* stream);
LCE_API size_t lce_forward_noalloc_max_bytes(void);

/*
 * Backward: gradients of the (mean or sum) loss; each shard's logit tiles
 * are rebuilt from X, W and lse.
 *  hidden, w_shards, shard_order, targets   as for lce_forward
 *  lse          device fp32 [N] from lce_forward on the same inputs
 *  dloss        device fp32 scalar: d(objective)/d(loss); for
 *               LCE_REDUCTION_NONE device fp32 [N]: d(objective)/d(token_loss).
 *  d_hidden     device fp32 [N][H] (bf16 with LCE_FLAG_BF16_GRADS), overwritten
 *               with dL/dX scaled by dloss (added to it with
 *               LCE_FLAG_ACCUMULATE_DX). Ignored tokens contribute exactly 0.
 *  d_w_shards   host array of P device pointers, each fp32 [V/P][H] (bf16
 *               with LCE_FLAG_BF16_GRADS), overwritten with that shard's
 *               dL/dW scaled by dloss (added to with LCE_FLAG_ACCUMULATE_DW).
 *  workspace    as for lce_forward (the forward's contents are not needed).
 * A target outside [0, V) that is not ignore_index makes every output NaN.
 */
LCE_API int lce_backward(const lce_dims* dims, const void* hidden, const void* const* w_shards, const int32_t* shard_order,
                 const int32_t* targets, const float* lse, const float* dloss, void* d_hidden,
                 void* const* d_w_shards, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One ring round at a time (same page, section 3.2 and Fig. 3: in each of
 * the P rounds a rank computes against the shard it currently holds, then
 * passes it on; backward makes the same trip). A ring driver holding one
 * shard at a time calls these in place of lce_forward / lce_backward, moving
 * the shards between rounds itself:
 *
 *   for k in 0..P-1: lce_fwd_round(dims, k, id_k, hidden, shard_k, targets, ws)
 *   lce_fwd_finish(dims, targets, loss, lse, token_loss, ws)
 *   for k in 0..P-1: lce_bwd_round(dims, k, id_k, hidden, shard_k, targets,
 *                                  lse, dloss, d_hidden, d_shard_k, acc, ws)
 *
 * id_k is the shard id (0..P-1) of the shard held in round k; the ids of the
 * P rounds must be a permutation of 0..P-1. The per-token running state
 * (m, z) and the target logits stay in `workspace` between the calls of one
 * forward, so every call of a sequence gets the same workspace (at least
 * lce_workspace_bytes(dims) bytes) and nothing else may use it meanwhile; the
 * stream order between the calls is the caller's to keep (one stream, or
 * events). Results match lce_forward / lce_backward with shard_order[k] = id_k:
 * the backward bit for bit, the forward up to fp32 rounding (its running state
 * is merged once per round here, possibly once per call there).
 *
 * lce_fwd_round
 *  round        k, 0..P-1. Round 0 starts a new forward (resets the state).
 *  shard_index  the id of the shard passed in w_shard.
 *  hidden, targets  as for lce_forward; w_shard device bf16 [V/P][H].
 *  Folds the logits of every token against this shard into the state and
 *  fills the target logits that fall in this shard.
 *
 * lce_fwd_finish
 *  After the P rounds: writes loss, lse and (if non-NULL) token_loss exactly
 *  as lce_forward does. Calling it before all P rounds have run gives the
 *  loss of the shards seen so far, with NaN token losses for targets in the
 *  missing shards.
 *
 * lce_bwd_round
 *  round, shard_index, hidden, w_shard, targets  as for lce_fwd_round.
 *  lse, dloss   as for lce_backward (every round reads them).
 *  d_hidden     as for lce_backward: round 0 overwrites it (or adds, with
 *               LCE_FLAG_ACCUMULATE_DX), later rounds add this shard's part,
 *               so after round P-1 it holds dL/dX. With LCE_FLAG_BF16_GRADS the
 *               sum is kept in fp32 in the workspace and written to the bf16
 *               d_hidden by round P-1 only.
 *  d_w_shard    this shard's gradient, overwritten, or added to what it holds
 *               when accumulate_dw != 0 or LCE_FLAG_ACCUMULATE_DW is set (a
 *               driver that sums a travelling partial, or accumulates over
 *               micro-batches); bf16 with LCE_FLAG_BF16_GRADS.
 * The forward's workspace contents are not needed by the backward rounds;
 * lce_fwd_round must not run between backward rounds on the same workspace.
 */
/*
 * Two ways to run the ring (same page, section 3.2: the ring can circulate
 * either the weight shards or the activations). The calls above serve both:
 *  - weights move: rank r keeps its batch and workspace; in round k it gets
 *    shard (r - k) mod P, and in the backward that shard's gradient partial
 *    travels with it (accumulate_dw from round 1 on).
 *  - activations move: rank r keeps shard r; in round k it gets batch
 *    b = (r - k) mod P with that batch's targets, lse (backward), d_hidden
 *    partial (backward) and the first lce_state_bytes(dims) bytes of the
 *    batch's workspace, and calls with shard_index = r on them; its own shard
 *    gradient stays put and accumulates over the batches (accumulate_dw from
 *    round 1 on).
 * lce_state_bytes: the leading workspace bytes that carry state from one call
 * of a sequence to the next (forward state; the fp32 dX accumulator with
 * LCE_FLAG_BF16_GRADS); the rest of the workspace is scratch. 0 if dims is
 * invalid.
 * lce_ring_payload: which payload moves fewer bytes per hop (one forward hop
 * plus one backward hop): LCE_PAYLOAD_WEIGHTS (shard + gradient partial) or
 * LCE_PAYLOAD_ACTIVATIONS (hidden, targets, lse, state and dX partial); the
 * two byte counts are written to the non-NULL out-pointers. Pure host
 * function; a negative status if dims is invalid.
 */
#define LCE_PAYLOAD_WEIGHTS 0
#define LCE_PAYLOAD_ACTIVATIONS 1
LCE_API size_t lce_state_bytes(const lce_dims* dims);
LCE_API int lce_ring_payload(const lce_dims* dims, size_t* weight_bytes, size_t* activation_bytes);

LCE_API int lce_fwd_round(const lce_dims* dims, int round, int shard_index, const void* hidden, const void* w_shard,
                          const int32_t* targets, void* workspace, size_t workspace_bytes, void* stream);
LCE_API int lce_fwd_finish(const lce_dims* dims, const int32_t* targets, float* loss, float* lse, float* token_loss,
                           void* workspace, size_t workspace_bytes, void* stream);
LCE_API int lce_bwd_round(const lce_dims* dims, int round, int shard_index, const void* hidden, const void* w_shard,
                          const int32_t* targets, const float* lse, const float* dloss, void* d_hidden,
                          void* d_w_shard, int accumulate_dw, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing trace, for measurement (off by default).
 * lce_trace_enable(capacity) creates `capacity` pairs of HIP events for the
 * calling thread (capacity 0 disables the trace and frees them). While enabled,
 * every kernel launch made by lce_forward / lce_backward on this thread is
 * bracketed by an event pair recorded on the call's stream, until the pairs
 * run out. lce_trace_collect waits for the recorded events, adds the elapsed
 * times into one entry per kernel kind, writes up to max_entries entries and
 * returns how many kinds it saw (or a negative status); it then empties the
 * trace for reuse. Entries also carry the launches' algorithmic work: MFMA
 * flops (2 x M x N x K of each contraction) and the bytes the kernel must move
 * at minimum (each operand read once, each output written once). Backward
 * launches count the tokens the backward ran over: when it left ignored
 * tokens out, only the others (the count is read back from the workspace of
 * the last backward that used it).
 */
typedef struct lce_trace_entry {
  char name[32];    /* kernel kind, e.g. "fwd_round", "gemm_dx" */
  int64_t launches; /* traced launches of this kind */
  int64_t dropped;  /* launches not traced because the event pairs ran out */
  double total_ms;  /* sum of event-measured durations of the traced launches */
  double flops;     /* algorithmic MFMA flops of the traced launches */
  double bytes;     /* algorithmic bytes of the traced launches */
} lce_trace_entry;

LCE_API int lce_trace_enable(int capacity);
LCE_API int lce_trace_collect(lce_trace_entry* out, int max_entries);

/* Static text for a status code. */
LCE_API const char* lce_status_string(int status);

/* Text of the last failure on the calling thread ("" if none). */
LCE_API const char* lce_last_error(void);

/* ABI version: (major << 16) | minor. */
LCE_API int lce_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H */

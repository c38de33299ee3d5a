"""CPU oracle for the exact vocabulary projection + cross-entropy, forward and backward.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import or run this module. The product path (the HIP
library and its Python binding) never imports it, and shares no code with it.

Everything here is plain float64 numpy on the host, written from:

* "Flattening Every Memory Peak in Long-Context Mixture-of-Experts Training",
  section 3.2 (Ring-DTP; the section label is inferred, the extracted page has
  no headings). Per token the loss depends on three numbers only: the largest
  logit, the sum of exponentials and the target's logit. Rank r holds one
  contiguous block of V/P vocabulary ids (columns of the H x V projection
  weight). A round multiplies the batch by one block and merges the resulting
  strip into the per-token (m, z, y_t) with the online-softmax rule (Eq. 3,
  missing from the extraction); at the end loss_i = m_i + log z_i - y_{t_i}.
  The backward multiplies again, block by block, and needs only lse from the
  forward.
* The exactness condition in the introduction to section 3: the operator may
  reorder the arithmetic but must produce the same loss and gradients as the
  plain implementation.

Because of that exactness requirement, ``cross_entropy`` below is the plain
definition written out (full logit rows, two-pass stable log-sum-exp, textbook
softmax-minus-one-hot gradient). ``ring_fold`` is the pages' algorithm in their
order (strip by strip in ring order, online fold, then the backward strip by
strip from lse); it exists so the tests can show the two agree.

Readings where the pages are silent (each also listed in the design notes):
* Eq. 3 (missing) is read as the standard update m' = max(m, max_j y_j),
  z' = z e^(m - m') + sum_j e^(y_j - m').
* Reduction is the mean over non-ignored tokens (sum optional); ignored tokens
  (target == ignore_index) have zero loss and zero gradient rows. "none"
  keeps the per-token losses: the objective is sum_i u_i loss_i for a given
  per-token upstream gradient u (``dloss`` an array), and ``loss`` reports the
  plain sum.
* Gradients: G = g_i (softmax_i - onehot(t_i)) with g_i = dloss / n_valid for
  valid rows (dloss for "sum", dloss[i] for "none"), 0 for ignored rows; dX = G W, dW = G^T X, where
  W is the V x H (vocabulary-major) weight, i.e. the transpose of the pages'
  H x V W_voc.
* n_valid = 0 under "mean" gives loss NaN (0/0) and all-zero gradients.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

IGNORE_INDEX = -100


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Result:
    loss: float                 # mean (or sum) over valid tokens
    loss_sum: float             # sum over valid tokens
    n_valid: int
    token_loss: np.ndarray      # [N]; 0 for ignored tokens
    lse: np.ndarray             # [N]; log-sum-exp of each full logit row (all rows)
    d_hidden: Optional[np.ndarray]   # [N][H]
    d_weight: Optional[np.ndarray]   # [V][H], vocabulary order

    def d_shards(self, n_shards: int) -> List[np.ndarray]:
        vs = self.d_weight.shape[0] // n_shards
        return [self.d_weight[s * vs:(s + 1) * vs] for s in range(n_shards)]


def _prepare(x, t, ignore_index, vocab, dloss, reduction):
    t = np.asarray(t, dtype=np.int64)
    valid = t != ignore_index
    bad = valid & ((t < 0) | (t >= vocab))
    if bad.any():
        raise ValueError(f"target id out of [0, {vocab}) at rows {np.nonzero(bad)[0][:8].tolist()}")
    n_valid = int(valid.sum())
    if reduction == "mean":
        scale = dloss / n_valid if n_valid else 0.0
    elif reduction == "sum":
        scale = dloss
    elif reduction == "none":
        scale = np.asarray(dloss, dtype=np.float64)
        if scale.shape != t.shape:
            raise ValueError("reduction 'none' takes one dloss per token")
    else:
        raise ValueError(f"reduction must be 'mean', 'sum' or 'none', got {reduction!r}")
    g = np.where(valid, scale, 0.0)
    return t, valid, n_valid, g


def _reduce(token_loss, n_valid, reduction):
    loss_sum = math.fsum(token_loss.tolist())
    if reduction in ("sum", "none"):
        return loss_sum, loss_sum
    return (loss_sum / n_valid if n_valid else float("nan")), loss_sum


def cross_entropy(x, w, targets, ignore_index: int = IGNORE_INDEX, dloss: float = 1.0,
                  reduction: str = "mean", grad: bool = True,
                  row_block: Optional[int] = None) -> Result:
    """Plain cross-entropy of the logits x @ w.T against ``targets``, with gradients.

    x: [N][H] float64, w: [V][H] float64 (vocabulary order). Full logit rows are
    formed one block of rows at a time; blocking over rows does not change any
    value (each row is independent, and dW sums the blocks in row order).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n, h = x.shape
    v = w.shape[0]
    t, valid, n_valid, g = _prepare(x, targets, ignore_index, v, dloss, reduction)
    lse = np.empty(n)
    token_loss = np.zeros(n)
    dx = np.zeros((n, h)) if grad else None
    dw = np.zeros((v, h)) if grad else None
    rb = row_block or max(1, min(n, (1 << 26) // max(v, 1)))
    for r0 in range(0, n, rb):
        r1 = min(n, r0 + rb)
        z = x[r0:r1] @ w.T                                   # logits, full rows
        m = z.max(axis=1)
        lse_b = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
        lse[r0:r1] = lse_b
        rows = np.nonzero(valid[r0:r1])[0]
        token_loss[r0 + rows] = lse_b[rows] - z[rows, t[r0 + rows]]
        if grad:
            p = np.exp(z - lse_b[:, None])                   # softmax
            p[rows, t[r0 + rows]] -= 1.0                     # minus one-hot
            p *= g[r0:r1, None]                              # dloss/dlogits
            dx[r0:r1] = p @ w
            dw += p.T @ x[r0:r1]
    loss, loss_sum = _reduce(token_loss, n_valid, reduction)
    return Result(loss, loss_sum, n_valid, token_loss, lse, dx, dw)


def ring_fold(x, shards: Sequence[np.ndarray], order: Sequence[int], targets,
              ignore_index: int = IGNORE_INDEX, dloss: float = 1.0,
              reduction: str = "mean", grad: bool = True) -> Result:
    """The pages' per-round algorithm in float64, one strip per round in ``order``.

    Round k forms the strip Y = x @ shards[order[k]].T (shard s holds vocabulary
    ids [s*Vs, (s+1)*Vs)), folds it into the running (m, z, y_t) by the online
    update, and drops it. After the last round: lse = m + log z and
    nll = lse - y_t. Backward visits the shards again in the same order and
    rebuilds each strip's gradient from the saved lse.
    """
    x = np.asarray(x, dtype=np.float64)
    shards = [np.asarray(s, dtype=np.float64) for s in shards]
    p_count = len(shards)
    vs = shards[0].shape[0]
    if sorted(int(s) for s in order) != list(range(p_count)):
        raise ValueError("order must be a permutation of the shard indices")
    n, h = x.shape
    t, valid, n_valid, g = _prepare(x, targets, ignore_index, vs * p_count, dloss, reduction)
    owner = np.where(valid, t // vs, -1)
    m = np.full(n, -np.inf)
    z = np.zeros(n)
    yt = np.full(n, np.nan)
    for s in order:
        y = x @ shards[s].T                                  # strip of this round
        m_new = np.maximum(m, y.max(axis=1))
        z = z * np.exp(m - m_new) + np.exp(y - m_new[:, None]).sum(axis=1)
        m = m_new
        rows = np.nonzero(owner == s)[0]
        yt[rows] = y[rows, t[rows] - s * vs]
    lse = m + np.log(z)
    token_loss = np.where(valid, lse - np.where(valid, yt, 0.0), 0.0)
    loss, loss_sum = _reduce(token_loss, n_valid, reduction)
    dx = dw = None
    if grad:
        dx = np.zeros((n, h))
        dws = [None] * p_count
        for s in order:
            y = x @ shards[s].T                              # recomputed strip
            gs = np.exp(y - lse[:, None])
            rows = np.nonzero(owner == s)[0]
            gs[rows, t[rows] - s * vs] -= 1.0
            gs *= g[:, None]
            dx += gs @ shards[s]
            dws[s] = gs.T @ x
        dw = np.concatenate(dws, axis=0)
    return Result(loss, loss_sum, n_valid, token_loss, lse, dx, dw)


def token_rows(x_rows, w, t_rows, g_rows, ignore_index: int = IGNORE_INDEX):
    """Per-row lse, loss and dX for selected rows, given each row's loss scale g.

    Rows are independent given g (= dloss / n_valid of the whole batch for valid
    rows, 0 for ignored rows), so a few rows of a large batch can be checked one
    by one. Returns (lse, token_loss, d_hidden_rows).
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    t = np.asarray(t_rows, dtype=np.int64)
    g = np.asarray(g_rows, dtype=np.float64)
    v = w.shape[0]
    valid = t != ignore_index
    if (valid & ((t < 0) | (t >= v))).any():
        raise ValueError("target id out of range")
    z = x_rows @ w.T
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    rows = np.nonzero(valid)[0]
    tok = np.zeros(len(t))
    tok[rows] = lse[rows] - z[rows, t[rows]]
    p = np.exp(z - lse[:, None])
    p[rows, t[rows]] -= 1.0
    p *= np.where(valid, g, 0.0)[:, None]
    return lse, tok, p @ w


def weight_rows(x, w_rows, v_ids, targets, lse, g, ignore_index: int = IGNORE_INDEX):
    """Selected rows of dW, given every token's normalizer lse and loss scale g.

    The gradient of vocabulary row v is a sum over tokens:
        dW_v = sum_i g_i (exp(x_i . w_v - lse_i) - [t_i = v]) x_i,
    which needs only that row of W, all of X and the per-token lse and g (g_i
    = dloss / n_valid for valid tokens, 0 for ignored ones), so a few rows of a
    large problem can be checked one by one at N x H cost each. x: [N][H],
    w_rows: [k][H] (the rows v_ids of W), lse, g: [N]. Returns [k][H].
    """
    x = np.asarray(x, dtype=np.float64)
    w_rows = np.asarray(w_rows, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    lse = np.asarray(lse, dtype=np.float64)
    g = np.where(t != ignore_index, np.asarray(g, dtype=np.float64), 0.0)
    ids = np.asarray(v_ids, dtype=np.int64)
    z = x @ w_rows.T                                         # the rows' logits, every token: [N][k]
    coef = g[:, None] * (np.exp(z - lse[:, None]) - (t[:, None] == ids[None, :]))   # dloss/dlogit
    return coef.T @ x

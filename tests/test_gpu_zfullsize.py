"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default ring order, one workspace from alloc_workspace).

The oracle cannot form every full logit row at these sizes in a test's time,
so:
* per-token results are checked on sampled rows, which the oracle computes one
  by one (a row's lse, loss and dX row depend only on that row, given the
  batch's loss scale g = dloss / n_valid, which is counted from the targets);
* the shard gradients are checked through properties that hold at any size:
  sum_ij dX_ij X_ij = sum_vh dW_vh W_vh, since both equal sum_iv G_iv z_iv
  (exact even for the bf16-rounded G both GEMMs share); and every row of
  softmax - onehot sums to zero, so for each column h the dW rows sum to zero
  up to the rounding of G to bf16 (unit roundoff 2^-8 per element, random
  sign: about 2^-8/sqrt(3) times the root-sum-square of the column; the bound
  used is 2^-5 times it);
* the mean loss must equal the mean of the per-token losses;
* a dozen vocabulary rows of dW (shard edges, the most frequent target, the
  last id, random ones) are computed one by one in float64 from the row's
  definition, given every token's lse and loss scale (oracle.weight_rows, at
  N x H cost per row); lse is the GPU's, itself checked on the sampled rows
  above, and an lse error e moves a row by a relative e at most.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_support import GRAD_TOL, LOSS_TOL, say, to_device

pytestmark = pytest.mark.gpu


def _sample_rows(targets, k=12, seed=0):
    n = len(targets)
    rng = np.random.default_rng(seed)
    rows = {0, n - 1, n // 2}
    ign = np.nonzero(targets == -100)[0]
    if len(ign):
        rows.add(int(ign[0]))
    rows.update(int(r) for r in rng.choice(n, size=min(n, k), replace=False))
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["small", "large", "long", "stress"])
def test_full_size_sampled(name):
    import torch
    import memory_bounded_vocabulary_amd as lce
    w = workloads.WORKLOADS[name]
    say("full size", name, dict(N=w.n_tokens, H=w.hidden, V=w.vocab, P=w.n_shards))
    b = workloads.make(w)
    hidden, shards, targets = to_device(b)
    ws = lce.alloc_workspace(w.n_tokens, w.hidden, w.vocab, w.n_shards, hidden.device)
    loss, lse, tl = lce.forward(hidden, shards, targets, workspace=ws, token_loss=True)
    dx, dws = lce.backward(hidden, shards, targets, lse, torch.ones((), device=hidden.device), workspace=ws)
    torch.cuda.synchronize()

    n_valid = int(np.sum(b.targets != -100))
    g = np.where(b.targets != -100, 1.0 / n_valid, 0.0)
    rows = _sample_rows(b.targets)
    ref_lse, ref_tok, ref_dx = oracle.token_rows(oracle.bf16_to_f64(b.hidden[rows]), oracle.bf16_to_f64(b.weight),
                                                 b.targets[rows], g[rows])
    got_lse = lse[rows.tolist()].double().cpu().numpy()
    got_tok = tl[rows.tolist()].double().cpu().numpy()
    got_dx = dx[rows.tolist()].double().cpu().numpy()
    e_lse = float(np.max(np.abs(got_lse - ref_lse)))
    e_tok = float(np.max(np.abs(got_tok - ref_tok)))
    e_dx = float(np.max(np.abs(got_dx - ref_dx)) / np.max(np.abs(ref_dx)))
    say(f"{name}: rows {len(rows)}: max|dlse|={e_lse:.2e} max|dtok|={e_tok:.2e} dX rows rel={e_dx:.2e}")
    assert e_lse <= LOSS_TOL * max(1.0, float(np.max(np.abs(ref_lse))) / 10)
    assert e_tok <= 10 * LOSS_TOL
    assert e_dx <= GRAD_TOL
    ign = b.targets[rows] == -100
    assert np.all(got_tok[ign] == 0.0) and np.all(got_dx[ign] == 0.0)

    # mean loss = mean of the token losses (all tokens)
    mean_tok = float(tl.double().sum().item()) / n_valid
    assert abs(loss.item() - mean_tok) <= LOSS_TOL, (loss.item(), mean_tok)

    # sum over vocabulary rows of dW vanishes (G rows sum to 0; G is bf16)
    col = sum(d.double().sum(dim=0) for d in dws)
    rss = sum((d.double() ** 2).sum(dim=0) for d in dws).sqrt()
    e_col = float((col.abs() / rss).max().item())
    # <dX, X> = <dW, W>
    lhs = float((dx.double() * hidden.double()).sum().item())
    rhs = float(sum((d.double() * s.double()).sum().item() for d, s in zip(dws, shards)))
    e_ip = abs(lhs - rhs) / max(abs(lhs), abs(rhs))
    say(f"{name}: max_h |sum_v dW_vh|/rss_h={e_col:.2e} <dX,X>={lhs:.6e} <dW,W>={rhs:.6e} rel={e_ip:.2e}")
    assert e_col <= 2.0 ** -5
    assert e_ip <= 1e-3

    # sampled dW rows against their float64 definition
    vs = w.shard_rows
    rng = np.random.default_rng(1)
    ids = sorted({0, vs - 1, vs, w.vocab - vs, w.vocab - 1, int(np.bincount(b.targets[b.targets >= 0]).argmax())} |
                 {int(i) for i in rng.choice(w.vocab, size=6, replace=False)})
    lse_all = lse.double().cpu().numpy()
    x64 = oracle.bf16_to_f64(b.hidden)
    ref_dw = oracle.weight_rows(x64, oracle.bf16_to_f64(b.weight[ids]), ids, b.targets, lse_all, g)
    del x64
    got_dw = np.stack([dws[i // vs][i % vs].double().cpu().numpy() for i in ids])
    e_dw = float(np.max(np.abs(got_dw - ref_dw)) / np.max(np.abs(ref_dw)))
    say(f"{name}: dW rows {ids}: rel={e_dw:.2e}")
    assert e_dw <= GRAD_TOL
    assert all(bool(torch.isfinite(d).all().item()) for d in dws) and bool(torch.isfinite(dx).all().item())


def test_full_size_rounds_match_whole_pass():
    """The one-round-at-a-time calls at the large workload's full size (two
    vocabulary chunks per shard) against the whole-pass calls: the backward bit
    for bit, the forward's lse within the loss gate."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    w = workloads.WORKLOADS["large"]
    say("full size rounds", dict(N=w.n_tokens, H=w.hidden, V=w.vocab, P=w.n_shards))
    b = workloads.make(w)
    hidden, shards, targets = to_device(b)
    p = w.n_shards
    order = [(p - k) % p for k in range(p)]
    loss, lse = lce.forward(hidden, shards, targets)
    dx, dws = lce.backward(hidden, shards, targets, lse, torch.ones((), device=hidden.device))
    dims = lce.make_dims(w.n_tokens, w.hidden, w.vocab, p)
    ws = lce.alloc_workspace(w.n_tokens, w.hidden, w.vocab, p)
    for k, s in enumerate(order):
        lce.fwd_round(dims, k, s, hidden, shards[s], targets, ws)
    loss_r, lse_r = lce.fwd_finish(dims, targets, ws)
    dl = torch.ones((), device=hidden.device)
    dx_r = torch.empty_like(dx)
    dws_r = [torch.empty_like(d) for d in dws]
    for k, s in enumerate(order):
        lce.bwd_round(dims, k, s, hidden, shards[s], targets, lse, dl, dx_r, dws_r[s], False, ws)
    torch.cuda.synchronize()
    e = float((lse_r - lse).abs().max().item())
    say(f"rounds: |dloss|={abs(loss_r.item() - loss.item()):.2e} max|dlse|={e:.2e}")
    assert abs(loss_r.item() - loss.item()) <= LOSS_TOL
    assert e <= LOSS_TOL
    assert torch.equal(dx_r, dx)
    assert all(torch.equal(a, c) for a, c in zip(dws_r, dws))

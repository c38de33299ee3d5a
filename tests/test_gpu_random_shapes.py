"""GPU parity on seeded random shapes: token counts, widths, shard sizes and
shard counts drawn at random (ragged against the 256 x 256 tiles and the
64-wide K steps), with random ignore fractions, weight scales, reductions and
shard orders. Each case is checked against the oracle at the gate
(|d loss| <= 2e-3, max|d grad| / max|grad| <= 2e-2) and ignored rows must
have exactly zero loss and gradient."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_support import compare, run_lce, say, to_device

pytestmark = pytest.mark.gpu

BASE = workloads.WORKLOADS["tiny"]


def _cases(n_cases=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_cases):
        p = int(rng.integers(1, 9))
        vs = int(rng.integers(1, 1300))
        n = int(rng.integers(1, 2600))
        h = 64 * int(rng.integers(1, 13))
        ign = float(rng.choice([0.0, 0.05, 0.3]))
        std = float(rng.choice([0.02, 0.1, 0.5]))
        red = str(rng.choice(["mean", "sum"]))
        order = [int(x) for x in rng.permutation(p)] if rng.random() < 0.5 else None
        out.append((f"case{i}: N={n} H={h} V/P={vs} P={p}", n, h, vs * p, p, ign, std, red, order))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0].split(":")[0] for c in CASES])
def test_random_shape_parity(case):
    name, n, h, v, p, ign, std, red, order = case
    say(name, dict(ignore=ign, w_std=std, reduction=red, order=order))
    w = BASE.with_dims(name=name, n_tokens=n, hidden=h, vocab=v, n_shards=p, ignore_frac=ign, w_std=std)
    b = workloads.make(w, seed=n + h + v)
    gpu = run_lce(*to_device(b), order=order, reduction=red, dloss=0.75)
    ref = oracle.cross_entropy(oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight), b.targets,
                               reduction=red, dloss=0.75)
    if np.isfinite(ref.loss):
        compare(gpu, ref, name, loss_tol=2e-3 * (max(1.0, abs(ref.loss) / 10) if red == "sum" else 1.0))
    ign_rows = b.targets == -100
    assert np.all(gpu["token_loss"][ign_rows] == 0.0)
    assert np.all(gpu["d_hidden"][ign_rows] == 0.0)


RING_CASES = _cases(n_cases=10, seed=77)


@pytest.mark.parametrize("case", RING_CASES, ids=[c[0].split(":")[0] for c in RING_CASES])
def test_random_shape_round_calls(case):
    """The round calls in a random shard order on random shapes: the backward
    equals the whole pass bit for bit, the forward within the gate."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    name, n, h, v, p, ign, std, red, order = case
    order = order or [(p - k) % p for k in range(p)]
    say("rounds", name, dict(order=order, reduction=red))
    w = BASE.with_dims(name=name, n_tokens=n, hidden=h, vocab=v, n_shards=p, ignore_frac=ign, w_std=std)
    b = workloads.make(w, seed=n + 2 * h + v)
    hidden, shards, targets = to_device(b)
    loss, lse, tl = lce.forward(hidden, shards, targets, order=order, reduction=red, token_loss=True)
    dloss = torch.full((), 0.75, device="cuda")
    dx, dws = lce.backward(hidden, shards, targets, lse, dloss, order=order, reduction=red)
    dims = lce.make_dims(n, h, v, p, reduction=red)
    ws = lce.alloc_workspace(n, h, v, p, reduction=red)
    for k, s in enumerate(order):
        lce.fwd_round(dims, k, s, hidden, shards[s], targets, ws)
    loss_r, lse_r, tl_r = lce.fwd_finish(dims, targets, ws, token_loss=True)
    dx_r = torch.empty_like(dx)
    dws_r = [torch.empty_like(d) for d in dws]
    for k, s in enumerate(order):
        lce.bwd_round(dims, k, s, hidden, shards[s], targets, lse, dloss, dx_r, dws_r[s], False, ws)
    torch.cuda.synchronize()
    assert float((lse_r - lse).abs().max().item()) <= 2e-3
    assert float((tl_r - tl).abs().max().item()) <= 2e-2
    if np.isfinite(loss.item()):
        assert abs(loss_r.item() - loss.item()) <= 2e-3 * max(1.0, abs(loss.item()) / 10)
    assert torch.equal(dx_r, dx)
    assert all(torch.equal(a, c) for a, c in zip(dws_r, dws))

"""GPU parity of the one-round-at-a-time entry points, driven as a simulated
ring on one GPU.

P virtual ranks each hold a distinct batch (hidden, targets) and share one
vocabulary weight cut into P shards. In round k rank r holds shard
(r - k) mod P, the shard its left neighbour held in round k - 1, so each shard
visits every rank once ("Flattening Every Memory Peak in Long-Context
Mixture-of-Experts Training", section 3.2 and Fig. 3). Backward makes the same
trip, and each shard's gradient travels with the shard: a rank adds its part
to the partial it receives (accumulate_dw from round 1 on), so after P rounds
the shard's gradient holds the sum over all ranks' batches.

Each rank is checked against the oracle's ring fold of its own batch in its own
shard order; the shard gradients against the sum of the ranks' oracle
gradients.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_support import GRAD_TOL, LOSS_TOL, compare, rel_max, say, to_device

pytestmark = pytest.mark.gpu

BASE = workloads.WORKLOADS["tiny"]

RINGS = [
    # name, N per rank, H, V, P
    ("4 ranks, ragged shard", 600, 256, 4 * 300, 4),
    ("2 ranks, two vocab chunks", 300, 64, 2 * 20000, 2),
    ("3 ranks, ragged N", 257, 192, 3 * 256, 3),
    ("8 ranks", 512, 128, 8 * 512, 8),
]


def _ring(name, n, h, v, p, seed0=20):
    import torch
    import memory_bounded_vocabulary_amd as lce
    w = BASE.with_dims(name=name, n_tokens=n, hidden=h, vocab=v, n_shards=p, ignore_frac=0.1, w_std=0.05)
    weight = workloads.make(w, seed=seed0).weight
    batches = [workloads.make(w, seed=seed0 + 1 + r, weight=weight) for r in range(p)]
    dev = [to_device(b) for b in batches]
    shards = dev[0][1]  # the weight is the same for every rank
    dims = lce.make_dims(n, h, v, p)
    ws = [lce.alloc_workspace(n, h, v, p) for _ in range(p)]
    for k in range(p):
        for r in range(p):
            s = (r - k) % p
            lce.fwd_round(dims, k, s, dev[r][0], shards[s], dev[r][2], ws[r])
    outs = [lce.fwd_finish(dims, dev[r][2], ws[r], token_loss=True) for r in range(p)]
    dloss = torch.ones((), dtype=torch.float32, device="cuda")
    dx = [torch.empty((n, h), dtype=torch.float32, device="cuda") for _ in range(p)]
    dws = [torch.empty((v // p, h), dtype=torch.float32, device="cuda") for _ in range(p)]
    for k in range(p):
        for r in range(p):
            s = (r - k) % p
            lce.bwd_round(dims, k, s, dev[r][0], shards[s], dev[r][2], outs[r][1], dloss, dx[r], dws[s], k > 0, ws[r])
    torch.cuda.synchronize()
    return batches, dev, outs, dx, dws


@pytest.mark.parametrize("case", RINGS, ids=[c[0] for c in RINGS])
def test_ring_simulation_parity(case):
    name, n, h, v, p = case
    say("ring", name, dict(N=n, H=h, V=v, P=p))
    batches, dev, outs, dx, dws = _ring(name, n, h, v, p)
    vs = v // p
    w64 = oracle.bf16_to_f64(batches[0].weight)
    w_shards = [w64[s * vs:(s + 1) * vs] for s in range(p)]
    dw_sum = np.zeros_like(w64)
    for r, b in enumerate(batches):
        order = [(r - k) % p for k in range(p)]
        ref = oracle.ring_fold(oracle.bf16_to_f64(b.hidden), w_shards, order, b.targets)
        dw_sum += ref.d_weight
        loss, lse, tl = outs[r]
        got = {
            "loss": float(loss.item()),
            "lse": lse.cpu().numpy().astype(np.float64),
            "token_loss": tl.cpu().numpy().astype(np.float64),
            "d_hidden": dx[r].cpu().numpy().astype(np.float64),
            "d_weight": ref.d_weight,  # compared summed over ranks below
        }
        compare(got, ref, f"{name} rank {r}")
        ign = b.targets == -100
        assert np.all(got["token_loss"][ign] == 0.0) and np.all(got["d_hidden"][ign] == 0.0)
    got_dw = np.concatenate([d.cpu().numpy() for d in dws]).astype(np.float64)
    e = rel_max(got_dw, dw_sum)
    say(f"{name}: summed dW rel={e:.2e}")
    assert e <= GRAD_TOL


def test_rounds_match_whole_pass():
    """Per-round calls against lce_forward / lce_backward with the same shard
    order: the backward bit for bit (the same launches on the same data), the
    forward within the loss tolerance (the running state is merged once per
    round instead of once per call)."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    w = BASE.with_dims(name="rounds vs whole", n_tokens=700, hidden=256, vocab=4 * 1000, n_shards=4,
                       ignore_frac=0.1, w_std=0.05)
    b = workloads.make(w, seed=5)
    hidden, shards, targets = to_device(b)
    order = [2, 0, 3, 1]
    say("rounds vs whole pass", order)
    loss, lse, tl = lce.forward(hidden, shards, targets, order=order, token_loss=True)
    dx, dws = lce.backward(hidden, shards, targets, lse, 1.0, order=order)
    dims = lce.make_dims(w.n_tokens, w.hidden, w.vocab, w.n_shards)
    ws = lce.alloc_workspace(w.n_tokens, w.hidden, w.vocab, w.n_shards)
    for k, s in enumerate(order):
        lce.fwd_round(dims, k, s, hidden, shards[s], targets, ws)
    loss_r, lse_r, tl_r = lce.fwd_finish(dims, targets, ws, token_loss=True)
    dloss = torch.ones((), dtype=torch.float32, device="cuda")
    dx_r = torch.empty_like(dx)
    dws_r = [torch.empty_like(d) for d in dws]
    for k, s in enumerate(order):
        lce.bwd_round(dims, k, s, hidden, shards[s], targets, lse, dloss, dx_r, dws_r[s], False, ws)
    torch.cuda.synchronize()
    assert abs(loss_r.item() - loss.item()) <= LOSS_TOL
    assert float((lse_r - lse).abs().max().item()) <= LOSS_TOL
    assert float((tl_r - tl).abs().max().item()) <= LOSS_TOL
    assert torch.equal(dx_r, dx)
    for a, c in zip(dws_r, dws):
        assert torch.equal(a, c)


def test_accumulate_into_existing_gradient():
    """accumulate_dw adds the shard gradient to what the buffer holds (gradient
    accumulation over micro-batches): two micro-batches accumulated into a
    buffer with prior content equal the prior content plus both gradients."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    w = BASE.with_dims(name="accumulate", n_tokens=300, hidden=128, vocab=2 * 700, n_shards=2, ignore_frac=0.1,
                       w_std=0.05)
    weight = workloads.make(w, seed=7).weight
    mbs = [workloads.make(w, seed=8 + i, weight=weight) for i in range(2)]
    say("accumulate over micro-batches")
    dims = lce.make_dims(w.n_tokens, w.hidden, w.vocab, w.n_shards)
    ws = lce.alloc_workspace(w.n_tokens, w.hidden, w.vocab, w.n_shards)
    rng = np.random.default_rng(1)
    prior = [rng.standard_normal((w.shard_rows, w.hidden)).astype(np.float32) * 1e-3 for _ in range(2)]
    dws = [torch.from_numpy(pr.copy()).cuda() for pr in prior]
    dloss = torch.ones((), dtype=torch.float32, device="cuda")
    expect = np.concatenate(prior).astype(np.float64)
    for mb in mbs:
        hidden, shards, targets = to_device(mb)
        for k in range(2):
            lce.fwd_round(dims, k, k, hidden, shards[k], targets, ws)
        _, lse = lce.fwd_finish(dims, targets, ws)
        dx = torch.empty((w.n_tokens, w.hidden), dtype=torch.float32, device="cuda")
        for k in range(2):
            lce.bwd_round(dims, k, k, hidden, shards[k], targets, lse, dloss, dx, dws[k], True, ws)
        expect += oracle.cross_entropy(oracle.bf16_to_f64(mb.hidden), oracle.bf16_to_f64(weight), mb.targets).d_weight
    torch.cuda.synchronize()
    got = np.concatenate([d.cpu().numpy() for d in dws]).astype(np.float64)
    e = rel_max(got, expect)
    say(f"accumulate: rel={e:.2e}")
    assert e <= GRAD_TOL


ACT_RINGS = [
    ("4 ranks", 600, 256, 4 * 300, 4),
    ("3 ranks, two vocab chunks", 257, 64, 3 * 20000, 3),
]


@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
@pytest.mark.parametrize("case", ACT_RINGS, ids=[c[0] for c in ACT_RINGS])
def test_activation_ring_simulation_parity(case, bf16):
    """The other payload: rank r keeps shard r and its gradient; batch b visits
    rank (b + k) mod P in round k, carrying its targets, lse, dX partial and the
    first lce_state_bytes of its workspace, copied from rank to rank here."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    name, n, h, v, p = case
    say("activation ring", name, dict(N=n, H=h, V=v, P=p, bf16=bf16))
    w = BASE.with_dims(name=name, n_tokens=n, hidden=h, vocab=v, n_shards=p, ignore_frac=0.1, w_std=0.05)
    weight = workloads.make(w, seed=60).weight
    batches = [workloads.make(w, seed=61 + b, weight=weight) for b in range(p)]
    dev = [to_device(b) for b in batches]
    shards = dev[0][1]
    flags = lce.FLAG_BF16_GRADS if bf16 else 0
    dims = lce.make_dims(n, h, v, p, flags=flags)
    sb = lce.state_bytes(dims)
    ws = [lce.alloc_workspace(n, h, v, p, flags=flags) for _ in range(p)]  # rank r's own workspace

    def hop():  # every rank passes the state it holds to rank r + 1
        transit = [ws[r][:sb].clone() for r in range(p)]
        for r in range(p):
            ws[r][:sb].copy_(transit[(r - 1) % p])

    for k in range(p):
        if k:
            hop()
        for r in range(p):
            b = (r - k) % p
            lce.fwd_round(dims, k, r, dev[b][0], shards[r], dev[b][2], ws[r])
    outs = [None] * p
    for r in range(p):
        b = (r - (p - 1)) % p
        outs[b] = lce.fwd_finish(dims, dev[b][2], ws[r], token_loss=True)
    dt = torch.bfloat16 if bf16 else torch.float32
    dloss = torch.ones((), dtype=torch.float32, device="cuda")
    dx = [torch.empty((n, h), dtype=dt, device="cuda") for _ in range(p)]       # travels with batch b
    dws = [torch.empty((v // p, h), dtype=dt, device="cuda") for _ in range(p)]  # stays on rank r
    for k in range(p):
        if k:
            hop()
        for r in range(p):
            b = (r - k) % p
            lce.bwd_round(dims, k, r, dev[b][0], shards[r], dev[b][2], outs[b][1], dloss, dx[b], dws[r], k > 0, ws[r])
    torch.cuda.synchronize()

    vs = v // p
    w64 = oracle.bf16_to_f64(weight)
    w_shards = [w64[s * vs:(s + 1) * vs] for s in range(p)]
    dw_sum = np.zeros_like(w64)
    for b, bt in enumerate(batches):
        ref = oracle.ring_fold(oracle.bf16_to_f64(bt.hidden), w_shards, [(b + k) % p for k in range(p)], bt.targets)
        dw_sum += ref.d_weight
        loss, lse, tl = outs[b]
        got = {"loss": float(loss.item()), "lse": lse.cpu().numpy().astype(np.float64),
               "token_loss": tl.cpu().numpy().astype(np.float64),
               "d_hidden": dx[b].float().cpu().numpy().astype(np.float64), "d_weight": ref.d_weight}
        compare(got, ref, f"{name} batch {b}")
    got_dw = np.concatenate([d.float().cpu().numpy() for d in dws]).astype(np.float64)
    e = rel_max(got_dw, dw_sum)
    say(f"{name}: stationary dW rel={e:.2e}")
    assert e <= GRAD_TOL


VARIANTS = [
    # reduction, bf16 gradients, accumulate into prior contents
    ("mean", True, False),
    ("none", False, False),
    ("sum", True, True),
    ("mean", False, True),
]


@pytest.mark.parametrize("variant", VARIANTS, ids=["-".join(map(str, v)) for v in VARIANTS])
def test_round_variants_match_whole_pass(variant):
    """Per-round backward with the flags and reductions equals the whole-pass
    backward with the same ones, bit for bit (same launches, same data)."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    reduction, bf16, acc = variant
    w = BASE.with_dims(name="round variants", n_tokens=24000, hidden=64, vocab=3 * 20000, n_shards=3,
                       ignore_frac=0.1, w_std=0.3)
    b = workloads.make(w, seed=12)
    hidden, shards, targets = to_device(b)
    say("round variants", variant)
    n, h, v, p = w.n_tokens, w.hidden, w.vocab, w.n_shards
    order = [1, 2, 0]
    dt = torch.bfloat16 if bf16 else torch.float32
    flags = (lce.FLAG_BF16_GRADS if bf16 else 0) | (lce.FLAG_ACCUMULATE_DX | lce.FLAG_ACCUMULATE_DW if acc else 0)
    out = lce.forward(hidden, shards, targets, order=order, reduction=reduction, token_loss=True)
    lse = out[1]
    gen = torch.Generator(device="cuda").manual_seed(4)
    dloss = (torch.rand((n,), generator=gen, device="cuda") if reduction == "none"
             else torch.full((), 0.5, device="cuda"))
    u = dloss.double().cpu().numpy() if reduction == "none" else 0.5
    ref = oracle.cross_entropy(oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight), b.targets,
                               reduction=reduction, dloss=u)
    # priors at the gradients' own scale, so that an accumulation that drops
    # or doubles them shows
    sx, sw = float(np.max(np.abs(ref.d_hidden))), float(np.max(np.abs(ref.d_weight)))
    prior_x = (torch.randn((n, h), generator=gen, device="cuda") * sx).to(dt)
    prior_w = [(torch.randn((v // p, h), generator=gen, device="cuda") * sw).to(dt) for _ in range(p)]
    dx = prior_x.clone()
    dws = [t.clone() for t in prior_w]
    lce.backward(hidden, shards, targets, lse, dloss, order=order, reduction=reduction, d_hidden=dx, d_shards=dws,
                 accumulate=acc, grad_dtype=dt)
    dims = lce.make_dims(n, h, v, p, reduction=reduction, flags=flags)
    ws = lce.alloc_workspace(n, h, v, p, reduction=reduction, flags=flags)
    dx_r = prior_x.clone()
    dws_r = [t.clone() for t in prior_w]
    for k, s in enumerate(order):
        lce.bwd_round(dims, k, s, hidden, shards[s], targets, lse, dloss, dx_r, dws_r[s], False, ws)
    torch.cuda.synchronize()
    assert torch.equal(dx_r, dx)
    for a, c in zip(dws_r, dws):
        assert torch.equal(a, c)
    # and against prior (when accumulating) + the oracle's gradient; bf16
    # outputs add one rounding of the sum (2^-8 relative)
    ex = ref.d_hidden + (prior_x.double().cpu().numpy() if acc else 0.0)
    ew = ref.d_weight + (np.concatenate([pw.double().cpu().numpy() for pw in prior_w]) if acc else 0.0)
    e_dx = float(np.max(np.abs(dx.double().cpu().numpy() - ex)))
    e_dw = float(np.max(np.abs(np.concatenate([d.double().cpu().numpy() for d in dws]) - ew)))
    tx = GRAD_TOL * sx + (2.0 ** -8 * float(np.max(np.abs(ex))) if bf16 else 0.0)
    tw = GRAD_TOL * sw + (2.0 ** -8 * float(np.max(np.abs(ew))) if bf16 else 0.0)
    say(f"{variant}: dX max|err|={e_dx:.2e} (bound {tx:.2e}) dW max|err|={e_dw:.2e} (bound {tw:.2e})")
    assert e_dx <= tx and e_dw <= tw

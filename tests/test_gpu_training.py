"""GPU parity of the training-loop extras: per-token upstream gradients
(reduction "none"), bf16 gradient outputs, accumulation into existing
gradients, and the recompute contract under activation checkpointing (apart
from the inputs the backward uses only lse from the forward; "Flattening
Every Memory Peak in Long-Context Mixture-of-Experts Training", section 3.2).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_support import GRAD_TOL, LOSS_TOL, rel_max, say, to_device

pytestmark = pytest.mark.gpu

BASE = workloads.WORKLOADS["tiny"]

SHAPES = [
    # name, N, H, V, P
    ("ragged shard", 600, 256, 4 * 300, 4),
    ("two token and two vocab chunks", 24000, 64, 2 * 20000, 2),
    ("two vocab chunks", 300, 64, 2 * 20000, 2),
]


def _batch(name, n, h, v, p, seed=31):
    w = BASE.with_dims(name=name, n_tokens=n, hidden=h, vocab=v, n_shards=p, ignore_frac=0.1, w_std=0.05)
    return workloads.make(w, seed=seed)


def _np(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else t.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
def test_per_token_dloss(case):
    import torch
    import memory_bounded_vocabulary_amd as lce
    b = _batch(*case)
    say("reduction none", case)
    hidden, shards, targets = to_device(b)
    u = np.random.default_rng(2).standard_normal(b.workload.n_tokens)
    loss, lse, tl = lce.forward(hidden, shards, targets, reduction="none")
    du = torch.from_numpy(u.astype(np.float32)).cuda()
    dx, dws = lce.backward(hidden, shards, targets, lse, du, reduction="none")
    torch.cuda.synchronize()
    ref = oracle.cross_entropy(oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight), b.targets,
                               reduction="none", dloss=u.astype(np.float32).astype(np.float64))
    e_tok = float(np.max(np.abs(_np(tl) - ref.token_loss)))
    e_sum = abs(loss.item() - ref.loss) / max(1.0, abs(ref.loss))
    e_dx = rel_max(_np(dx), ref.d_hidden)
    e_dw = rel_max(np.concatenate([_np(d) for d in dws]), ref.d_weight)
    say(f"{case[0]}: tok={e_tok:.2e} sum rel={e_sum:.2e} dX={e_dx:.2e} dW={e_dw:.2e}")
    assert e_tok <= 10 * LOSS_TOL
    assert e_sum <= LOSS_TOL
    assert e_dx <= GRAD_TOL and e_dw <= GRAD_TOL
    ign = b.targets == -100
    assert np.all(_np(dx)[ign] == 0.0)


@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
def test_bf16_gradients_are_rounded_fp32_gradients(case):
    """bf16 outputs equal the fp32 outputs rounded to nearest even, bit for bit
    (same contractions in the same order, one rounding at the end)."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    b = _batch(*case)
    say("bf16 gradients", case)
    hidden, shards, targets = to_device(b)
    loss, lse = lce.forward(hidden, shards, targets)
    dx32, dws32 = lce.backward(hidden, shards, targets, lse, 1.0)
    dx16, dws16 = lce.backward(hidden, shards, targets, lse, 1.0, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert dx16.dtype == torch.bfloat16 and all(d.dtype == torch.bfloat16 for d in dws16)
    assert torch.equal(dx16, dx32.to(torch.bfloat16))
    for a, c in zip(dws16, dws32):
        assert torch.equal(a, c.to(torch.bfloat16))
    ref = oracle.cross_entropy(oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight), b.targets)
    assert rel_max(_np(dx16), ref.d_hidden) <= GRAD_TOL
    assert rel_max(np.concatenate([_np(d) for d in dws16]), ref.d_weight) <= GRAD_TOL


@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
def test_accumulate_into_existing_gradients(case, bf16):
    import torch
    import memory_bounded_vocabulary_amd as lce
    b = _batch(*case)
    say("accumulate", case, "bf16" if bf16 else "fp32")
    hidden, shards, targets = to_device(b)
    loss, lse = lce.forward(hidden, shards, targets)
    dx, dws = lce.backward(hidden, shards, targets, lse, 1.0)
    dt = torch.bfloat16 if bf16 else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(3)
    scale = float(dx.abs().max().item())
    rx = (torch.randn(dx.shape, generator=gen, device="cuda") * scale).to(dt)
    rws = [(torch.randn(d.shape, generator=gen, device="cuda") * scale).to(dt) for d in dws]
    ax, aws = rx.clone(), [r.clone() for r in rws]
    lce.backward(hidden, shards, targets, lse, 1.0, d_hidden=ax, d_shards=aws, accumulate=True, grad_dtype=dt)
    torch.cuda.synchronize()
    ref = oracle.cross_entropy(oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight), b.targets)
    # prior + the oracle's gradient: the gate on the gradient, plus (bf16) one
    # rounding of the sum
    ex = rx.double().cpu().numpy() + ref.d_hidden
    e = float(np.max(np.abs(_np(ax) - ex)))
    tol_x = GRAD_TOL * np.max(np.abs(ref.d_hidden)) + (2.0 ** -8 * np.max(np.abs(ex)) if bf16 else 0.0)
    say(f"dX: max|err|={e:.3e} bound={tol_x:.3e}")
    assert e <= tol_x
    ew = np.concatenate([r.double().cpu().numpy() for r in rws]) + ref.d_weight
    e = float(np.max(np.abs(np.concatenate([_np(a) for a in aws]) - ew)))
    tol_w = GRAD_TOL * np.max(np.abs(ref.d_weight)) + (2.0 ** -8 * np.max(np.abs(ew)) if bf16 else 0.0)
    say(f"dW: max|err|={e:.3e} bound={tol_w:.3e}")
    assert e <= tol_w


def test_backward_after_recompute_needs_only_lse():
    """The backward run on a recomputed copy of the activations (new buffer,
    original freed) with only lse kept equals the backward on the original."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    b = _batch("recompute", 700, 256, 4 * 1000, 4)
    say("recompute contract")
    hidden, shards, targets = to_device(b)
    loss, lse = lce.forward(hidden, shards, targets)
    dx, dws = lce.backward(hidden, shards, targets, lse, 1.0)
    torch.cuda.synchronize()
    saved_lse = lse.clone()
    del hidden, loss, lse
    torch.cuda.empty_cache()
    hidden2 = to_device(b)[0]   # the caller's recompute: same values, a new buffer
    dx2, dws2 = lce.backward(hidden2, shards, targets, saved_lse, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(dx2, dx)
    for a, c in zip(dws2, dws):
        assert torch.equal(a, c)


def test_autograd_under_checkpointing():
    """linear_cross_entropy inside torch.utils.checkpoint: the forward runs again
    before the backward; gradients match the plain autograd run bit for bit and
    the oracle within the gate."""
    import torch
    from torch.utils.checkpoint import checkpoint
    from memory_bounded_vocabulary_amd.autograd import linear_cross_entropy
    b = _batch("autograd", 700, 256, 4 * 1000, 4)
    say("autograd + checkpoint")
    hidden, shards, targets = to_device(b)

    def run(use_ckpt):
        x = hidden.clone().requires_grad_(True)
        ws = [s.clone().requires_grad_(True) for s in shards]

        def head(xx, *ss):
            return linear_cross_entropy(xx * 1, list(ss), targets)

        loss = checkpoint(head, x, *ws, use_reentrant=False) if use_ckpt else head(x, *ws)
        loss.backward()
        torch.cuda.synchronize()
        return loss.detach(), x.grad, [w.grad for w in ws]

    l0, gx0, gw0 = run(False)
    l1, gx1, gw1 = run(True)
    assert gx0.dtype == torch.bfloat16 and all(g.dtype == torch.bfloat16 for g in gw0)
    assert torch.equal(l0, l1) and torch.equal(gx0, gx1)
    for a, c in zip(gw0, gw1):
        assert torch.equal(a, c)
    ref = oracle.cross_entropy(oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight), b.targets)
    assert abs(l0.item() - ref.loss) <= LOSS_TOL
    assert rel_max(_np(gx0), ref.d_hidden) <= GRAD_TOL
    assert rel_max(np.concatenate([_np(g) for g in gw0]), ref.d_weight) <= GRAD_TOL

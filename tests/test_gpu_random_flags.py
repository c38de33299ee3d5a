"""GPU parity on seeded random shapes crossed with the backward's options:
token counts and shard sizes drawn near the 256-row tile edges (127, 128,
129, 255, 256 past a multiple of 256) or at random, ignore fractions up to
0.9, mean, sum or per-token losses (random dloss per token), random shard
orders, and at random: every token kept in
the backward (LCE_FLAG_KEEP_IGNORED_ROWS), accumulation into prior
gradients (LCE_FLAG_ACCUMULATE_DX / _DW), bf16 gradient outputs
(LCE_FLAG_BF16_GRADS). Checked against the oracle at the gate; with bf16
outputs that accumulate, the stored sum prior + gradient is compared,
allowing one bf16 rounding of it."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_support import compare, say, to_device

pytestmark = pytest.mark.gpu

BASE = workloads.WORKLOADS["tiny"]


def _rows(rng, hi):
    if rng.random() < 0.4:
        return max(1, int(256 * rng.integers(0, hi // 256 + 1) + rng.choice([1, 127, 128, 129, 255, 256])))
    return int(rng.integers(1, hi))


def _cases(n_cases=100, seed=31337):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_cases):
        p = int(rng.integers(1, 11))
        vs, n = _rows(rng, 2000), _rows(rng, 3000)
        h = 64 * int(rng.integers(1, 13))
        opts = dict(ign=float(rng.choice([0.0, 0.1, 0.5, 0.9])), std=float(rng.choice([0.02, 0.1, 0.5])),
                    red=str(rng.choice(["mean", "sum", "none"])), keep=bool(rng.random() < 0.3),
                    acc=bool(rng.random() < 0.3), bf16=bool(rng.random() < 0.3),
                    order=[int(x) for x in rng.permutation(p)] if rng.random() < 0.5 else None)
        out.append((f"case{i}: N={n} H={h} V/P={vs} P={p}", n, h, vs, p, opts))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0].split(":")[0] for c in CASES])
def test_random_shape_and_flags_parity(case):
    import torch
    import memory_bounded_vocabulary_amd as lce
    name, n, h, vs, p, o = case
    say(name, o)
    w = BASE.with_dims(name=name, n_tokens=n, hidden=h, vocab=vs * p, n_shards=p, ignore_frac=o["ign"],
                       w_std=o["std"])
    b = workloads.make(w, seed=3 * n + h + vs)
    hidden, shards, targets = to_device(b)
    loss, lse, tl = lce.forward(hidden, shards, targets, order=o["order"], reduction=o["red"], token_loss=True)
    if o["red"] == "none":
        dl_ref = np.random.default_rng(n + h).standard_normal(n).astype(np.float32) * 0.5
        dloss = torch.from_numpy(dl_ref).cuda()
        dl_ref = dl_ref.astype(np.float64)
    else:
        dl_ref = 0.75
        dloss = torch.tensor(0.75, dtype=torch.float32, device="cuda")
    gdt = torch.bfloat16 if o["bf16"] else torch.float32
    kw, px, pw = {}, None, None
    if o["acc"]:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(n + vs)
        sc = 1e-3 if o["red"] == "mean" else 1e-1  # about the gradients' own scale
        px = (torch.randn((n, h), device="cuda", generator=gen) * sc).to(gdt)
        pw = [(torch.randn(s.shape, device="cuda", generator=gen) * sc).to(gdt) for s in shards]
        kw = dict(d_hidden=px.clone(), d_shards=[t.clone() for t in pw], accumulate=True)
    dx, dws = lce.backward(hidden, shards, targets, lse, dloss, order=o["order"], reduction=o["red"],
                           keep_ignored_rows=o["keep"], grad_dtype=gdt, **kw)
    torch.cuda.synchronize()
    ref = oracle.cross_entropy(oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight), b.targets,
                               reduction=o["red"], dloss=dl_ref)
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    got_dx, got_dw = f64(dx), np.concatenate([f64(g) for g in dws])
    loss_tol = 2e-3 * (max(1.0, abs(ref.loss) / 10) if o["red"] != "mean" else 1.0)
    gpu = {"loss": float(loss.item()), "lse": f64(lse), "token_loss": f64(tl)}
    if o["acc"] and o["bf16"]:
        # the stored value is bf16(prior + gradient): compare the sum, with one bf16 rounding of it allowed
        for got, prior_t, want, what in ((got_dx, px, ref.d_hidden, "dX"), (got_dw, torch.cat(pw), ref.d_weight, "dW")):
            prior = f64(prior_t)
            err = np.abs(got - (want + prior))
            allowed = 2e-2 * np.max(np.abs(want)) + 2.0 ** -8 * np.abs(want + prior)
            assert np.all(err <= allowed), (name, what, float(np.max(err - allowed)))
        gpu.update(d_hidden=ref.d_hidden, d_weight=ref.d_weight)  # the rest of the gate: loss, lse, token losses
    else:
        if o["acc"]:
            got_dx, got_dw = got_dx - f64(px), got_dw - np.concatenate([f64(t) for t in pw])
        gpu.update(d_hidden=got_dx, d_weight=got_dw)
    if np.isfinite(ref.loss):
        compare(gpu, ref, name, loss_tol=loss_tol)
    ign_rows = b.targets == -100
    assert np.all(gpu["token_loss"][ign_rows] == 0.0)
    # an ignored token's dX row is exactly zero, or exactly its prior when accumulating
    assert np.all(f64(dx)[ign_rows] == (f64(px)[ign_rows] if o["acc"] else 0.0))

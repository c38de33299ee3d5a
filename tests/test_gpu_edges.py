"""GPU parity on small and degenerate shapes, closed forms and invariants.

Every case runs the HIP path through the C ABI and compares with the CPU
oracle on the same seeded inputs (gates: |d loss| <= 2e-3, max|d grad| /
max|grad| <= 2e-2).
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_support import GRAD_TOL, compare, oracle_for, rel_max, run_lce, say, to_device

pytestmark = pytest.mark.gpu

BASE = workloads.WORKLOADS["tiny"]

SHAPES = [
    # name, N, H, V, P, ignore fraction, weight std
    ("one token", 1, 128, 1024, 4, 0.0, 0.02),
    ("ragged N=17", 17, 64, 512, 2, 0.2, 0.05),
    ("N=255 one short of a tile", 255, 192, 768, 3, 0.1, 0.05),
    ("N=257 one past a tile", 257, 128, 1000, 4, 0.1, 0.05),
    ("shard of 300 rows (ragged vocab tile)", 600, 256, 1200, 4, 0.05, 0.05),
    ("single shard", 300, 128, 700, 1, 0.0, 0.05),
    ("one vocab row per shard", 3, 64, 4, 4, 0.0, 1.0),
    ("V=1", 5, 64, 1, 1, 0.0, 1.0),
    ("256 shards", 300, 64, 256 * 3, 256, 0.1, 0.3),
    # backward chunking (G chunks of at most 2^27 elements, vocabulary chunks of
    # at most 16384 rows): two token chunks and two vocabulary chunks per shard
    ("two token and two vocab chunks", 24000, 64, 2 * 20000, 2, 0.05, 0.3),
    ("two vocab chunks", 300, 64, 2 * 20000, 2, 0.05, 0.3),
    # ignored tokens left out of the backward (a token tile saved): ragged,
    # and with the second token chunk left empty
    ("ignored tokens left out", 1000, 128, 3000, 3, 0.3, 0.1),
    ("half ignored, empty second token chunk", 24000, 64, 2 * 20000, 2, 0.5, 0.3),
    ("large logits", 333, 512, 2048, 2, 0.1, 0.5),
    # the backward's last vocabulary and token tiles with exactly 128 live rows
    # (the waves of rows 128-255 skip their MFMAs) and with 129 (they do not)
    ("last tiles with 128 live rows", 384, 128, 2 * 384, 2, 0.0, 0.05),
    ("last tiles with 129 live rows", 385, 128, 2 * 385, 2, 0.0, 0.05),
]


@pytest.mark.parametrize("case", SHAPES, ids=[s[0] for s in SHAPES])
def test_shape_parity(case):
    name, n, h, v, p, ign, std = case
    say("case", name, dict(N=n, H=h, V=v, P=p))
    w = BASE.with_dims(name=name, n_tokens=n, hidden=h, vocab=v, n_shards=p, ignore_frac=ign, w_std=std)
    b = workloads.make(w, seed=3)
    gpu = run_lce(*to_device(b))
    compare(gpu, oracle_for(b), name)
    # ignored tokens: zero loss and exactly zero gradient rows
    ign_rows = b.targets == -100
    assert np.all(gpu["token_loss"][ign_rows] == 0.0)
    assert np.all(gpu["d_hidden"][ign_rows] == 0.0)


def test_zero_weight_closed_form():
    say("case W=0")
    b = workloads.make("tiny")
    wz = np.zeros_like(b.weight)
    gpu = run_lce(*to_device(b, weight=wz))
    v = BASE.vocab
    assert abs(gpu["loss"] - math.log(v)) <= 1e-5
    assert np.all(np.abs(gpu["lse"] - math.log(v)) <= 1e-5)
    assert np.all(gpu["d_hidden"] == 0.0)
    x = oracle.bf16_to_f64(b.hidden)
    g = 1.0 / len(b.targets)
    expect = np.repeat((g / v) * x.sum(axis=0)[None, :], v, axis=0)
    np.subtract.at(expect, b.targets, g * x)
    assert rel_max(gpu["d_weight"], expect) <= GRAD_TOL


def test_dlogit_rows_sum_to_zero():
    """Each token's row of dloss/dlogits sums to zero. The last 64 hidden
    features are 0 in X and 1.0 in every row of W: the logits are unchanged,
    and each of those dX columns is the token's sum over the vocabulary of
    dloss/dlogits (G rounded to bf16, as the contractions take it). Checked
    against the oracle on the same inputs and, explicitly, for being small
    against the real dX columns."""
    import torch
    say("case dlogit row sums")
    w = BASE.with_dims(name="rowsum", n_tokens=700, hidden=256, vocab=4 * 500, n_shards=4, ignore_frac=0.1,
                       w_std=0.1)
    b = workloads.make(w, seed=11)
    x_bits = np.ascontiguousarray(b.hidden).copy()
    w_bits = np.ascontiguousarray(b.weight).copy()
    x_bits[:, -64:] = 0             # bf16 +0.0
    w_bits[:, -64:] = 0x3F80        # bf16 1.0
    hidden = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    vs = w.shard_rows
    shards = [torch.from_numpy(w_bits[s * vs:(s + 1) * vs].view(np.int16)).view(torch.bfloat16).cuda()
              for s in range(w.n_shards)]
    targets = torch.from_numpy(np.ascontiguousarray(b.targets, dtype=np.int32)).cuda()
    gpu = run_lce(hidden, shards, targets)
    ref = oracle.cross_entropy(oracle.bf16_to_f64(x_bits), oracle.bf16_to_f64(w_bits), b.targets)
    compare(gpu, ref, "dlogit row sums")
    assert np.max(np.abs(ref.d_hidden[:, -64:])) <= 1e-12 * np.max(np.abs(ref.d_hidden))  # fp64 rounding only
    sums = gpu["d_hidden"][:, -64:]
    assert np.all(sums == sums[:, :1])  # the 64 columns read the same sum
    assert np.max(np.abs(sums)) <= GRAD_TOL * np.max(np.abs(ref.d_hidden[:, :-64]))


def test_ring_order_invariance_and_determinism():
    say("case ring order")
    w = BASE.with_dims(name="order", n_tokens=700, hidden=256, vocab=8 * 300, n_shards=8, ignore_frac=0.1, w_std=0.2)
    b = workloads.make(w, seed=5)
    dev = to_device(b)
    ref = oracle_for(b)
    runs = {}
    for order in ([0, 1, 2, 3, 4, 5, 6, 7], [7, 6, 5, 4, 3, 2, 1, 0], [3, 0, 6, 1, 7, 2, 5, 4], None):
        r = run_lce(*dev, order=order)
        compare(r, ref, f"order {order}")
        runs[str(order)] = r
    a, c = runs[str([0, 1, 2, 3, 4, 5, 6, 7])], runs[str([7, 6, 5, 4, 3, 2, 1, 0])]
    assert abs(a["loss"] - c["loss"]) <= 1e-5 * abs(a["loss"])
    assert rel_max(a["d_hidden"], c["d_hidden"]) <= 2e-3
    # same order twice: bit-identical (fixed-order reductions, no atomics)
    again = run_lce(*dev, order=[3, 0, 6, 1, 7, 2, 5, 4])
    first = runs[str([3, 0, 6, 1, 7, 2, 5, 4])]
    for k in ("lse", "token_loss", "d_hidden", "d_weight"):
        assert np.array_equal(again[k], first[k]), k
    assert again["loss"] == first["loss"]


def test_sum_reduction_and_dloss_scale():
    say("case sum reduction")
    w = BASE.with_dims(name="sum", n_tokens=300, hidden=128, vocab=1024, n_shards=4, ignore_frac=0.1, w_std=0.1)
    b = workloads.make(w, seed=7)
    gpu = run_lce(*to_device(b), reduction="sum", dloss=0.37)
    ref = oracle_for(b, reduction="sum", dloss=0.37)
    compare(gpu, ref, "sum", loss_tol=2e-3 * ref.n_valid)


def test_all_tokens_ignored():
    say("case all ignored")
    w = BASE.with_dims(name="ignored", n_tokens=100, hidden=64, vocab=512, n_shards=2, ignore_frac=1.0)
    b = workloads.make(w, seed=1)
    gpu = run_lce(*to_device(b))
    assert math.isnan(gpu["loss"])
    assert np.all(gpu["token_loss"] == 0.0)
    assert np.all(gpu["d_hidden"] == 0.0) and np.all(gpu["d_weight"] == 0.0)


def test_out_of_range_target_gives_nan():
    say("case bad target")
    w = BASE.with_dims(name="bad", n_tokens=50, hidden=64, vocab=512, n_shards=2, ignore_frac=0.0)
    b = workloads.make(w, seed=1)
    b.targets[7] = 512
    gpu = run_lce(*to_device(b))
    assert math.isnan(gpu["loss"]) and math.isnan(gpu["token_loss"][7])
    assert np.all(np.isfinite(np.delete(gpu["token_loss"], 7)))
    assert np.all(np.isnan(gpu["d_hidden"][7])) and np.all(np.isnan(gpu["d_weight"]))
    assert np.all(np.isfinite(np.delete(gpu["d_hidden"], 7, axis=0)))


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_empty_batch(reduction):
    """N = 0: the loss is NaN (mean of nothing) or 0 (sum of nothing); the shard
    gradients are zero, or unchanged when accumulating; the round calls agree."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    say("empty batch", reduction)
    h, v, p = 128, 4 * 300, 4
    gen = torch.Generator(device="cuda").manual_seed(1)
    shards = [(torch.randn((v // p, h), generator=gen, device="cuda") * 0.05).to(torch.bfloat16) for _ in range(p)]
    hidden = torch.empty((0, h), dtype=torch.bfloat16, device="cuda")
    targets = torch.empty((0,), dtype=torch.int32, device="cuda")
    loss, lse = lce.forward(hidden, shards, targets, reduction=reduction)
    garbage = [torch.full((v // p, h), 3.0, device="cuda") for _ in range(p)]
    dx, dws = lce.backward(hidden, shards, targets, lse, 1.0, reduction=reduction,
                           d_shards=[g.clone() for g in garbage])
    acc = [g.clone() for g in garbage]
    lce.backward(hidden, shards, targets, lse, 1.0, reduction=reduction, d_hidden=dx, d_shards=acc, accumulate=True)
    dims = lce.make_dims(0, h, v, p, reduction=reduction)
    ws = lce.alloc_workspace(0, h, v, p, reduction=reduction)
    for k in range(p):
        lce.fwd_round(dims, k, k, hidden, shards[k], targets, ws)
    loss_r, _ = lce.fwd_finish(dims, targets, ws)
    dws_r = [g.clone() for g in garbage]
    dl = torch.ones((), device="cuda")
    for k in range(p):
        lce.bwd_round(dims, k, k, hidden, shards[k], targets, lse, dl, dx, dws_r[k], False, ws)
    torch.cuda.synchronize()
    if reduction == "mean":
        assert math.isnan(loss.item()) and math.isnan(loss_r.item())
    else:
        assert loss.item() == 0.0 and loss_r.item() == 0.0
    assert lse.numel() == 0 and dx.numel() == 0
    assert all(bool((d == 0).all().item()) for d in dws)
    assert all(bool((d == 0).all().item()) for d in dws_r)
    assert all(torch.equal(a, g) for a, g in zip(acc, garbage))


def test_binding_refuses_host_buffers_beside_device_inputs():
    """A host workspace or gradient buffer never reaches the kernels as a pointer."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    b = workloads.make("tiny")
    hidden, shards, targets = to_device(b)
    w = b.workload
    say("host buffers beside device inputs")
    ws_host = torch.zeros(lce.workspace_bytes(w.n_tokens, w.hidden, w.vocab, w.n_shards), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        lce.forward(hidden, shards, targets, workspace=ws_host)
    loss, lse = lce.forward(hidden, shards, targets)
    with pytest.raises(ValueError, match="GPU"):
        lce.backward(hidden, shards, targets, lse, 1.0, workspace=ws_host)
    with pytest.raises(ValueError, match="GPU"):
        lce.backward(hidden, shards, targets, lse, 1.0, d_hidden=torch.zeros((w.n_tokens, w.hidden)))
    with pytest.raises(ValueError, match="GPU"):
        lce.backward(hidden, shards, targets, lse, 1.0,
                     d_shards=[torch.zeros((w.shard_rows, w.hidden)) for _ in range(w.n_shards)])
    dims = lce.make_dims(w.n_tokens, w.hidden, w.vocab, w.n_shards)
    with pytest.raises(ValueError, match="GPU"):
        lce.fwd_round(dims, 0, 0, hidden, shards[0], targets, ws_host)
    torch.cuda.synchronize()

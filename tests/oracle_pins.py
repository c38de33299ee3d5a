"""Checks that pin the CPU oracle to things other than itself.

Each check takes the oracle module (or a stand-in with the same functions) so
that the planted-mistake test can run the same checks against deliberately
broken copies of it and confirm that every copy fails at least one check.

What each check pins, and where the fact comes from:
* brute_force: scalar pure-Python evaluation of the cross-entropy definition
  (log of a sum of exponentials minus the target logit; gradient of the mean)
  on tiny random instances, without the max shift the oracle uses.
* torch_reference: torch's float64 cross_entropy + autograd on the CPU.
* finite_differences: central differences of the mean loss in every entry of
  X and W; independent of any gradient formula. The per-token reduction is
  pinned the same way, on the objective sum_i u_i loss_i for a random u, and
  against torch's reduction="none" backward with upstream gradient u.
* zero_weight: W = 0 makes every logit 0, so each valid token's loss is ln V,
  dX = 0, and dW_v = g (sum of valid x_i / V - sum of valid x_i with t_i = v).
* logistic: V = 2 reduces to the logistic loss log(1 + exp(y_other - y_t)).
* bf16_widening: the widening of bfloat16 bit patterns, over all 65536 of
  them, against the format's own definition (1 sign bit, 8 exponent bits with
  bias 127, 7 fraction bits; subnormals at exponent field 0; all-ones exponent
  for infinities and NaN) evaluated with math.ldexp, and against torch's
  bfloat16 -> float64 conversion; plus hand-checked patterns.
* invariants: softmax-minus-one-hot rows sum to 0, token by token (a
  hidden feature that is 0 in X and 1 in W reads the sum) and so
  sum_v dW_v = 0;
  adding one vector c to every vocabulary row leaves loss and gradients
  unchanged; an ignored row contributes nothing (equal to dropping it while
  keeping n_valid); mean * n_valid = sum; the pages' ring fold over any shard
  order and any shard count equals the plain definition.
"""
from __future__ import annotations

import math

import numpy as np


def rand_instance(rng, n, h, v, ignore=0, scale=1.0):
    x = rng.standard_normal((n, h)) * scale
    w = rng.standard_normal((v, h)) * scale
    t = rng.integers(0, v, size=n)
    if ignore:
        t[rng.choice(n, size=ignore, replace=False)] = -100
    return x, w, t


def _brute(x, w, t, ignore_index=-100):
    n, h = x.shape
    v = w.shape[0]
    valid = [int(t[i]) != ignore_index for i in range(n)]
    n_valid = sum(valid)
    z = [[math.fsum(x[i][k] * w[j][k] for k in range(h)) for j in range(v)] for i in range(n)]
    tok = []
    lse = []
    for i in range(n):
        s = math.log(math.fsum(math.exp(zz) for zz in z[i]))
        lse.append(s)
        tok.append(s - z[i][int(t[i])] if valid[i] else 0.0)
    loss = math.fsum(tok) / n_valid
    dx = [[0.0] * h for _ in range(n)]
    dw = [[0.0] * h for _ in range(v)]
    for i in range(n):
        if not valid[i]:
            continue
        den = math.fsum(math.exp(zz) for zz in z[i])
        for j in range(v):
            gij = (math.exp(z[i][j]) / den - (1.0 if j == int(t[i]) else 0.0)) / n_valid
            for k in range(h):
                dx[i][k] += gij * w[j][k]
                dw[j][k] += gij * x[i][k]
    return loss, np.array(tok), np.array(lse), np.array(dx), np.array(dw)


def check_brute_force(orc, seeds=range(6)):
    for seed in seeds:
        rng = np.random.default_rng(1000 + seed)
        n, h, v = 1 + seed % 7, 1 + (seed * 3) % 8, 2 + (seed * 5) % 31
        x, w, t = rand_instance(rng, n, h, v, ignore=(n - 1) // 3)
        loss, tok, lse, dx, dw = _brute(x, w, t)
        for rb in (None, 1, 2):
            r = orc.cross_entropy(x, w, t, row_block=rb)
            assert abs(r.loss - loss) <= 1e-12 * max(1.0, abs(loss)), (seed, rb, r.loss, loss)
            np.testing.assert_allclose(r.token_loss, tok, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(r.lse, lse, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(r.d_hidden, dx, rtol=1e-10, atol=1e-13)
            np.testing.assert_allclose(r.d_weight, dw, rtol=1e-10, atol=1e-13)


def _bf16_by_definition(bits):
    """Value of one bfloat16 bit pattern from the format's fields."""
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)          # subnormal: 0.f x 2^-126
    return sign * math.ldexp(128 + f, e - 127 - 7)     # normal: 1.f x 2^(e - 127)


def check_bf16_widening(orc):
    import torch
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns are widened to NaN
        got = orc.bf16_to_f64(allbits)
    assert got.dtype == np.float64 and got.shape == (1 << 16,)
    ref = np.array([_bf16_by_definition(int(b)) for b in range(1 << 16)])
    lib = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for expect in (ref, lib):
        nan = np.isnan(expect)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], expect[~nan])
        # signed zeros keep their sign
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(expect[~nan]))
    hand = {0x3F80: 1.0, 0xC020: -2.5, 0x0001: 2.0 ** -133, 0x7F80: math.inf, 0xFF80: -math.inf,
            0x4049: 3.140625, 0x0080: 2.0 ** -126, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127}
    for b, v in hand.items():
        assert orc.bf16_to_f64(np.array([b], dtype=np.uint16))[0] == v, hex(b)
    assert math.copysign(1.0, orc.bf16_to_f64(np.array([0x8000], dtype=np.uint16))[0]) == -1.0
    assert math.isnan(orc.bf16_to_f64(np.array([0x7FC0], dtype=np.uint16))[0])
    # a 2-D array keeps its shape
    assert orc.bf16_to_f64(np.array([[0x3F80, 0x4000]], dtype=np.uint16)).tolist() == [[1.0, 2.0]]


def check_torch_reference(orc, x, w, t, tol=1e-10, row_block=None):
    import torch
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    tt = torch.tensor(np.asarray(t, dtype=np.int64))
    logits = xt @ wt.T
    loss = torch.nn.functional.cross_entropy(logits, tt, ignore_index=-100, reduction="mean")
    loss.backward()
    tok = torch.nn.functional.cross_entropy(logits.detach(), tt, ignore_index=-100, reduction="none")
    r = orc.cross_entropy(x, w, t, row_block=row_block)
    assert abs(r.loss - loss.item()) <= tol * max(1.0, abs(loss.item())), (r.loss, loss.item())
    np.testing.assert_allclose(r.token_loss, tok.numpy(), rtol=tol, atol=tol)
    np.testing.assert_allclose(r.lse, torch.logsumexp(logits.detach(), dim=1).numpy(), rtol=tol, atol=tol)
    gx, gw = xt.grad.numpy(), wt.grad.numpy()
    assert np.max(np.abs(r.d_hidden - gx)) <= tol * max(1e-30, np.max(np.abs(gx)))
    assert np.max(np.abs(r.d_weight - gw)) <= tol * max(1e-30, np.max(np.abs(gw)))


def check_finite_differences(orc, seed=7):
    rng = np.random.default_rng(seed)
    x, w, t = rand_instance(rng, 5, 3, 6, ignore=1)
    r = orc.cross_entropy(x, w, t)

    def loss_at(xx, ww):
        return orc.cross_entropy(xx, ww, t, grad=False).loss

    for arr, grad in ((x, r.d_hidden), (w, r.d_weight)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            hstep = 1e-6 * max(1.0, abs(arr[idx]))
            old = arr[idx]
            arr[idx] = old + hstep
            lp = loss_at(x, w)
            arr[idx] = old - hstep
            lm = loss_at(x, w)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * hstep)
        err = np.max(np.abs(num - grad)) / max(1e-30, np.max(np.abs(grad)))
        assert err <= 1e-6, err


def check_per_token_reduction(orc, seed=8):
    """reduction 'none': gradients of sum_i u_i loss_i, by finite differences of
    the token losses and by torch's backward of the unreduced loss."""
    import torch
    rng = np.random.default_rng(seed)
    x, w, t = rand_instance(rng, 6, 3, 7, ignore=2)
    u = rng.standard_normal(6)
    r = orc.cross_entropy(x, w, t, reduction="none", dloss=u)

    def objective(xx, ww):
        return float(np.dot(u, orc.cross_entropy(xx, ww, t, grad=False).token_loss))

    for arr, grad in ((x, r.d_hidden), (w, r.d_weight)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            hstep = 1e-6 * max(1.0, abs(arr[idx]))
            old = arr[idx]
            arr[idx] = old + hstep
            lp = objective(x, w)
            arr[idx] = old - hstep
            lm = objective(x, w)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * hstep)
        err = np.max(np.abs(num - grad)) / max(1e-30, np.max(np.abs(grad)))
        assert err <= 1e-6, err
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    tok = torch.nn.functional.cross_entropy(xt @ wt.T, torch.tensor(t), ignore_index=-100, reduction="none")
    tok.backward(torch.tensor(u))
    assert abs(r.loss - float(tok.sum().item())) <= 1e-12 * max(1.0, abs(r.loss))
    np.testing.assert_allclose(r.token_loss, tok.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r.d_hidden, xt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(r.d_weight, wt.grad.numpy(), rtol=1e-10, atol=1e-13)


def check_zero_weight(orc, seed=3):
    rng = np.random.default_rng(seed)
    n, h, v = 9, 4, 11
    x = rng.standard_normal((n, h))
    t = rng.integers(0, v, size=n)
    t[[2, 5]] = -100
    w = np.zeros((v, h))
    r = orc.cross_entropy(x, w, t)
    assert abs(r.loss - math.log(v)) <= 1e-14, r.loss
    valid = t != -100
    np.testing.assert_allclose(r.token_loss[valid], math.log(v), rtol=0, atol=1e-14)
    assert np.all(r.d_hidden == 0.0)
    g = 1.0 / valid.sum()
    expect = np.zeros((v, h))
    xs = x[valid].sum(axis=0)
    for j in range(v):
        expect[j] = g * (xs / v - x[valid & (t == j)].sum(axis=0))
    np.testing.assert_allclose(r.d_weight, expect, rtol=1e-12, atol=1e-15)


def check_logistic(orc, seed=4):
    rng = np.random.default_rng(seed)
    x, w, t = rand_instance(rng, 8, 5, 2)
    r = orc.cross_entropy(x, w, t)
    z = x @ w.T
    for i in range(8):
        other = 1 - int(t[i])
        expect = math.log1p(math.exp(z[i, other] - z[i, int(t[i])]))
        assert abs(r.token_loss[i] - expect) <= 1e-13 * max(1.0, expect)


def check_invariants(orc, seed=5):
    rng = np.random.default_rng(seed)
    n, h, v = 12, 6, 24
    x, w, t = rand_instance(rng, n, h, v, ignore=3)
    base = orc.cross_entropy(x, w, t)
    # rows of softmax - onehot sum to zero, so the vocabulary rows of dW sum to zero
    assert np.max(np.abs(base.d_weight.sum(axis=0))) <= 1e-14 * max(1.0, np.max(np.abs(base.d_weight)) * v)
    # the same, token by token: a feature that is 0 in every hidden row and 1 in
    # every vocabulary row leaves the logits unchanged, and its column of dX is
    # then each token's sum of dloss/dlogits over the vocabulary
    aug = orc.cross_entropy(np.hstack([x, np.zeros((n, 1))]), np.hstack([w, np.ones((v, 1))]), t)
    assert abs(aug.loss - base.loss) <= 1e-13 * max(1.0, abs(base.loss))
    assert np.max(np.abs(aug.d_hidden[:, h])) <= 1e-14 * max(1.0, np.max(np.abs(base.d_hidden)) * v)
    np.testing.assert_allclose(aug.d_hidden[:, :h], base.d_hidden, rtol=1e-12, atol=1e-15)
    # a constant vector added to every vocabulary row shifts each row's logits uniformly
    c = rng.standard_normal(h)
    sh = orc.cross_entropy(x, w + c[None, :], t)
    assert abs(sh.loss - base.loss) <= 1e-12
    np.testing.assert_allclose(sh.d_hidden, base.d_hidden, atol=1e-13)
    np.testing.assert_allclose(sh.d_weight, base.d_weight, atol=1e-13)
    # ignored rows: zero loss, zero dX row, and the same as dropping them (same n_valid)
    ign = t == -100
    assert np.all(base.token_loss[ign] == 0.0) and np.all(base.d_hidden[ign] == 0.0)
    kept = orc.cross_entropy(x[~ign], w, t[~ign])
    assert abs(kept.loss - base.loss) <= 1e-13
    np.testing.assert_allclose(kept.d_hidden, base.d_hidden[~ign], atol=1e-14)
    np.testing.assert_allclose(kept.d_weight, base.d_weight, atol=1e-14)
    # mean * n_valid = sum, and "sum" gradients are n_valid times the mean ones
    sm = orc.cross_entropy(x, w, t, reduction="sum")
    assert abs(sm.loss - base.loss * base.n_valid) <= 1e-12 * abs(sm.loss)
    np.testing.assert_allclose(sm.d_hidden, base.d_hidden * base.n_valid, rtol=1e-12, atol=1e-14)
    # a row's loss does not depend on the other rows
    perm = rng.permutation(n)
    pr = orc.cross_entropy(x[perm], w, t[perm])
    np.testing.assert_allclose(pr.token_loss, base.token_loss[perm], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(pr.d_hidden, base.d_hidden[perm], rtol=1e-12, atol=1e-15)
    # the pages' per-round fold gives the same result for every shard count and order
    for p_count in (1, 2, 3, 4, 6, 8, 12, 24):
        vs = v // p_count
        shards = [w[s * vs:(s + 1) * vs] for s in range(p_count)]
        for order in (list(range(p_count)), [(-k) % p_count for k in range(p_count)],
                      list(rng.permutation(p_count))):
            rf = orc.ring_fold(x, shards, order, t)
            assert abs(rf.loss - base.loss) <= 1e-12 * max(1.0, abs(base.loss))
            np.testing.assert_allclose(rf.token_loss, base.token_loss, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(rf.lse, base.lse, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(rf.d_hidden, base.d_hidden, rtol=1e-10, atol=1e-14)
            np.testing.assert_allclose(rf.d_weight, base.d_weight, rtol=1e-10, atol=1e-14)


def check_row_samples(orc, seed=6):
    rng = np.random.default_rng(seed)
    x, w, t = rand_instance(rng, 10, 4, 9, ignore=2)
    base = orc.cross_entropy(x, w, t)
    g = np.where(t != -100, 1.0 / base.n_valid, 0.0)
    rows = np.array([0, 3, 7, 9])
    lse, tok, dx = orc.token_rows(x[rows], w, t[rows], g[rows])
    np.testing.assert_allclose(lse, base.lse[rows], rtol=1e-13)
    np.testing.assert_allclose(tok, base.token_loss[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dx, base.d_hidden[rows], rtol=1e-12, atol=1e-15)


def check_weight_rows(orc, seed=10):
    """Selected dW rows given lse and g equal the rows of the full definition's
    dW (and of torch's autograd), ignored tokens and a row with several
    targets included."""
    import torch
    rng = np.random.default_rng(seed)
    x, w, t = rand_instance(rng, 14, 5, 9, ignore=3)
    t[[0, 4]] = 2                                   # two tokens share target 2
    base = orc.cross_entropy(x, w, t)
    g = np.where(t != -100, 1.0 / base.n_valid, 0.0)
    ids = [0, 2, 8]
    got = orc.weight_rows(x, w[ids], ids, t, base.lse, g)
    np.testing.assert_allclose(got, base.d_weight[ids], rtol=1e-12, atol=1e-15)
    wt = torch.tensor(w, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(torch.tensor(x) @ wt.T, torch.tensor(t), ignore_index=-100)
    loss.backward()
    np.testing.assert_allclose(got, wt.grad.numpy()[ids], rtol=1e-10, atol=1e-15)


def all_small_checks(orc):
    """Every pin that runs in about a second (used by the planted-mistake test)."""
    check_bf16_widening(orc)
    check_brute_force(orc)
    rng = np.random.default_rng(11)
    x, w, t = rand_instance(rng, 16, 8, 40, ignore=4)
    check_torch_reference(orc, x, w, t, row_block=5)
    check_finite_differences(orc)
    check_per_token_reduction(orc)
    check_zero_weight(orc)
    check_logistic(orc)
    check_invariants(orc)
    check_row_samples(orc)
    check_weight_rows(orc)

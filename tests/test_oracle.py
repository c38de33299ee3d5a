"""Pins of the CPU oracle (no GPU): see oracle_pins for what each check rests on."""
import inspect
import math
import sys
import types

import numpy as np
import pytest

import oracle
from oracle import lce_oracle
import oracle_pins as pins
import workloads


def test_bf16_widening():
    pins.check_bf16_widening(oracle)


def test_brute_force():
    pins.check_brute_force(oracle)


def test_torch_reference_random():
    rng = np.random.default_rng(0)
    for (n, h, v, ign, rb) in [(16, 8, 40, 4, 5), (33, 16, 97, 0, None), (7, 3, 2, 2, 1)]:
        x, w, t = pins.rand_instance(rng, n, h, v, ignore=ign)
        pins.check_torch_reference(oracle, x, w, t, row_block=rb)


def test_torch_reference_tiny_workload():
    b = workloads.make("tiny")
    x, w = oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight)
    pins.check_torch_reference(oracle, x, w, b.targets, row_block=100)


def test_finite_differences():
    pins.check_finite_differences(oracle)


def test_per_token_reduction():
    pins.check_per_token_reduction(oracle)


def test_zero_weight_closed_form():
    pins.check_zero_weight(oracle)


def test_zero_weight_tiny_is_ln_v():
    b = workloads.make("tiny")
    x = oracle.bf16_to_f64(b.hidden)
    r = oracle.cross_entropy(x, np.zeros((1024, 128)), b.targets)
    assert abs(r.loss - 6.931471805599453) <= 1e-14


def test_logistic_special_case():
    pins.check_logistic(oracle)


def test_invariants():
    pins.check_invariants(oracle)


def test_row_samples():
    pins.check_row_samples(oracle)


def test_weight_rows():
    pins.check_weight_rows(oracle)


def test_large_logits_stay_finite():
    # logits of order 1e3 overflow a naive exp; the max-shifted form must not
    rng = np.random.default_rng(9)
    x, w, t = pins.rand_instance(rng, 6, 4, 10, scale=20.0)
    r = oracle.cross_entropy(x, w, t)
    assert np.isfinite(r.loss) and np.all(np.isfinite(r.d_hidden)) and np.all(np.isfinite(r.d_weight))
    z = x @ w.T
    for i in range(6):
        m = max(z[i])
        expect = m + math.log(math.fsum(math.exp(v - m) for v in z[i])) - z[i, t[i]]
        assert abs(r.token_loss[i] - expect) <= 1e-12 * max(1.0, abs(expect))


def test_no_valid_tokens():
    x = np.ones((3, 2))
    w = np.ones((4, 2))
    r = oracle.cross_entropy(x, w, np.full(3, -100))
    assert math.isnan(r.loss) and r.n_valid == 0
    assert np.all(r.d_hidden == 0) and np.all(r.d_weight == 0)


def test_out_of_range_target_raises():
    with pytest.raises(ValueError):
        oracle.cross_entropy(np.ones((2, 2)), np.ones((3, 2)), np.array([0, 3]))
    with pytest.raises(ValueError):
        oracle.ring_fold(np.ones((2, 2)), [np.ones((3, 2))], [0], np.array([-1, 0]))


# --- planted mistakes -------------------------------------------------------
# Each entry breaks one step of a copy of the oracle's source. The copy is run
# through the same pins; every one of them must fail at least one pin.
MUTANTS = {
    "bf16 widening shifted by 15": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "bf16 widening drops the low fraction bit": ("u = np.asarray(bits, dtype=np.uint16).astype(np.uint32)",
                                                 "u = (np.asarray(bits, dtype=np.uint16) & 0xFFFE).astype(np.uint32)"),
    "lse without the max": ("lse_b = m + np.log(", "lse_b = np.log("),
    "one-hot added, not subtracted": ("p[rows, t[r0 + rows]] -= 1.0", "p[rows, t[r0 + rows]] += 1.0"),
    "target index without block offset": ("z[rows, t[r0 + rows]]", "z[rows, t[rows]]"),
    "gradient scale dropped": ("p *= g[r0:r1, None]", "pass"),
    "mean over all tokens": ("scale = dloss / n_valid if n_valid else 0.0", "scale = dloss / len(t)"),
    "ignored rows keep gradient": ("g = np.where(valid, scale, 0.0)", "g = np.full(len(t), scale)"),
    "loss divided by N": ("return (loss_sum / n_valid if n_valid", "return (loss_sum / len(token_loss) if n_valid"),
    "dX from transposed weight order": ("dx[r0:r1] = p @ w", "dx[r0:r1] = p @ w[::-1]"),
    "dW rows from the wrong block": ("dw += p.T @ x[r0:r1]", "dw += p.T @ x[:r1 - r0]"),
    "fold without rescale": ("z = z * np.exp(m - m_new) + ", "z = z + "),
    "fold target off by one column": ("yt[rows] = y[rows, t[rows] - s * vs]", "yt[rows] = y[rows, (t[rows] - s * vs + 1) % vs]"),
    "fold keeps stale max": ("        m = m_new\n", "        pass\n"),
    "ring backward one-hot in wrong shard": ("gs[rows, t[rows] - s * vs] -= 1.0", "gs[rows, (t[rows] - s * vs + 1) % vs] -= 1.0"),
    "token loss sign": ("token_loss[r0 + rows] = lse_b[rows] - z[", "token_loss[r0 + rows] = -lse_b[rows] + z["),
    "row sample one-hot dropped": ("p[rows, t[rows]] -= 1.0\n    p *= np.where", "p *= np.where"),
    "per-token scale ignores the token": ("scale = np.asarray(dloss, dtype=np.float64)",
                                          "scale = np.full(t.shape, np.mean(dloss))"),
    "weight row one-hot at the wrong id": ("(t[:, None] == ids[None, :])", "(t[:, None] == ids[None, :] + 1)"),
    "weight row without the normalizer": ("np.exp(z - lse[:, None])", "np.exp(z)"),
    "per-token loss reported as a mean": ('if reduction in ("sum", "none"):', 'if reduction == "sum":'),
    "softmax with another token's normalizer": ("p = np.exp(z - lse_b[:, None])", "p = np.exp(z - lse_b[::-1, None])"),
}


def _mutant(src_from, src_to):
    src = inspect.getsource(lce_oracle)
    assert src.count(src_from) >= 1, f"mutation anchor not found: {src_from!r}"
    name = "oracle_mutant_%d" % len(sys.modules)
    mod = types.ModuleType(name)
    sys.modules[name] = mod          # dataclasses look their module up by name
    exec(compile(src.replace(src_from, src_to, 1), name, "exec"), mod.__dict__)
    assert callable(mod.cross_entropy) and callable(mod.ring_fold)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(*MUTANTS[name])      # built outside the check: a broken copy must load
    with pytest.raises((AssertionError, IndexError, ValueError, FloatingPointError)):
        pins.all_small_checks(mod)


def test_unmodified_copy_passes_all_pins():
    mod = _mutant("IGNORE_INDEX = -100", "IGNORE_INDEX = -100")
    pins.all_small_checks(mod)


def test_golden_tiny_unchanged():
    """The oracle's tiny-workload results match the stored fixture (written by the oracle)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")) as f:
        gold = json.load(f)
    b = workloads.make("tiny", seed=0)
    assert b.digest() == gold["inputs_sha256_16"]
    r = oracle.cross_entropy(oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight), b.targets)
    assert abs(r.loss - gold["loss"]) <= 1e-13 and r.n_valid == gold["n_valid"]
    rows = gold["rows"]
    np.testing.assert_allclose(r.lse[rows], gold["lse"], rtol=1e-13)
    np.testing.assert_allclose(r.token_loss[rows], gold["token_loss"], rtol=1e-13)
    np.testing.assert_allclose(r.d_hidden[rows, :4], gold["d_hidden_rows_first4"], rtol=1e-11, atol=1e-18)
    np.testing.assert_allclose(r.d_weight[[0, 255, 256, 1023], :4], gold["d_weight_rows_first4"],
                               rtol=1e-11, atol=1e-18)
    assert abs(np.sqrt((r.d_weight ** 2).sum()) - gold["d_weight_fro"]) <= 1e-12 * gold["d_weight_fro"]

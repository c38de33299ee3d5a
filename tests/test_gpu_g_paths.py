"""GPU parity for the placements of targets that select the recompute
epilogue's variants: whether a tile is a vocabulary chunk's last, partial one
(rows past the chunk masked to zero), and whether a wave's 128 vocabulary rows
hold any target (the one-hot subtraction of G = g (softmax - onehot),
"Flattening Every Memory Peak in Long-Context Mixture-of-Experts Training",
section 3.2). Targets are placed by hand so that each variant is hit, and a
tenth of the tokens are ignored. Everything is compared with the oracle.

Shape: N = 600, H = 128, V = 4 x 1000, so each shard is one vocabulary chunk
of four 256-row tiles, the last holding 232 rows.
"""
import numpy as np
import pytest

import workloads
from gpu_support import compare, oracle_for, run_lce, say, to_device

pytestmark = pytest.mark.gpu

BASE = workloads.WORKLOADS["tiny"].with_dims(name="g-paths", n_tokens=600, hidden=128, vocab=4000, n_shards=4,
                                             w_std=0.05)


def _targets(kind: str, n: int, vs: int, p: int, rng) -> np.ndarray:
    t = np.empty(n, dtype=np.int32)
    shard = rng.integers(0, p, n)
    if kind == "partial tile":
        # rows 768..999 of each shard: the chunk's last, partial tile
        t[:] = shard * vs + rng.integers(768, vs, n)
    elif kind == "first waves only":
        # rows 0..127 of the first tile: only the waves with wm = 0 of that tile
        # see a target; every other wave of every tile takes the no-one-hot path
        t[:] = shard * vs + rng.integers(0, 128, n)
    elif kind == "one shard, second waves":
        # rows 128..255 of shard 2's first tile only
        t[:] = 2 * vs + rng.integers(128, 256, n)
    elif kind == "mixed":
        t[:] = rng.integers(0, p * vs, n)
    else:
        raise ValueError(kind)
    t[rng.random(n) < 0.1] = -100
    return t


@pytest.mark.parametrize("kind", ["partial tile", "first waves only", "one shard, second waves", "mixed"])
def test_recompute_epilogue_variants(kind):
    b = workloads.make(BASE, seed=5)
    rng = np.random.default_rng(11)
    b.targets = _targets(kind, BASE.n_tokens, BASE.shard_rows, BASE.n_shards, rng)
    say("g paths", kind, dict(N=BASE.n_tokens, H=BASE.hidden, V=BASE.vocab, P=BASE.n_shards))
    hidden, shards, targets = to_device(b)
    gpu = run_lce(hidden, shards, targets)
    ref = oracle_for(b)
    compare(gpu, ref, kind)
    ign = b.targets == -100
    assert np.all(gpu["d_hidden"][ign] == 0.0)

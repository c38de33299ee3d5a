"""Seeded synthetic inputs for the vocabulary projection + cross-entropy path.

This module only draws inputs: hidden states, vocabulary weight shards and
target ids, with the sizes and value distributions of the five workloads below,
packed as bfloat16 bit patterns (round to nearest even). It holds none of the
arithmetic of the method itself. Both the CPU oracle and the GPU path consume
what it returns, so the two sides always see bit-identical inputs.

Recipe (the same for every workload):

* One ``numpy.random.SeedSequence(seed)`` per instance. Each array draws from
  its own child stream, identified by a fixed spawn key, so an array never
  depends on how many other arrays were drawn or on the thread count:
  hidden = key (0, block), weight = key (1, block), targets = key (2,),
  ignore mask = key (3,). Hidden and weight rows are drawn in fixed blocks of
  ``BLOCK_ROWS`` rows (one PCG64 stream per block), so the first ``n`` rows of
  an instance are the same for every ``N >= n`` except for the ignore mask.
* hidden: standard normal float32; for RMS-normalised workloads each row is
  divided by ``sqrt(mean(x**2) + 1e-6)`` in float32; then bf16 RNE.
* weight: normal(0, w_std) float32 over all ``V`` rows, bf16 RNE, split into
  ``P`` contiguous row blocks of ``V/P`` rows (shard s owns vocabulary ids
  ``[s*V/P, (s+1)*V/P)``).
* targets: uniform integers in ``[0, V)``, or a finite Zipf law over ranks
  ``k = 1..V`` with ``p_k`` proportional to ``k**-s`` sampled by inverse CDF on
  the float64 cumulative sum (token id = k - 1, so frequent ids sit in shard 0).
* ignore: exactly ``floor(f*N + 0.5)`` positions, drawn without replacement,
  are set to ``ignore_index`` (-100).
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

IGNORE_INDEX = -100
BLOCK_ROWS = 4096
RMS_EPS = 1e-6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int
    hidden: int
    vocab: int
    n_shards: int
    rms_norm: bool
    w_std: float
    targets: str          # "uniform" or "zipf"
    zipf_s: float
    ignore_frac: float
    description: str = ""

    @property
    def shard_rows(self) -> int:
        return self.vocab // self.n_shards

    def with_tokens(self, n_tokens: int) -> "Workload":
        """Same hidden width, vocabulary, shards and distributions, fewer tokens."""
        return dataclasses.replace(self, name=f"{self.name}[N={n_tokens}]", n_tokens=n_tokens)

    def with_dims(self, **kw) -> "Workload":
        name = kw.pop("name", None) or self.name + "[" + ",".join(f"{k}={v}" for k, v in kw.items()) + "]"
        return dataclasses.replace(self, name=name, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 256, 128, 1024, 4, False, 0.02, "uniform", 0.0, 0.0,
                     "N=256 H=128 V=1024 P=4; hidden N(0,1); weight N(0,0.02); uniform targets; none ignored"),
    "small": Workload("small", 4096, 2048, 32000, 8, True, 0.02, "zipf", 1.1, 0.05,
                      "small LM head: N=4096 H=2048 V=32000 P=8; RMS-normalised hidden; Zipf(1.1); 5% ignored"),
    "large": Workload("large", 16384, 4096, 128256, 8, True, 0.02, "zipf", 1.1, 0.02,
                      "large vocabulary: N=16384 H=4096 V=128256 P=8; Zipf(1.1); 2% ignored"),
    "long": Workload("long", 65536, 7168, 129280, 8, True, 0.015, "zipf", 1.05, 0.01,
                     "long-context rank share: N=65536 H=7168 V=129280 P=8; Zipf(1.05); 1% ignored"),
    "stress": Workload("stress", 131071, 4096, 151936, 16, False, 0.5, "uniform", 0.0, 0.10,
                       "tail/stability stress: N=131071 H=4096 V=151936 P=16; weight N(0,0.5); 10% ignored"),
}
ORDER = ["tiny", "small", "large", "long", "stress"]


@dataclasses.dataclass
class Batch:
    workload: Workload
    seed: int
    hidden: np.ndarray    # uint16 [N][H], bf16 bit patterns
    weight: np.ndarray    # uint16 [V][H], bf16 bit patterns, vocabulary order
    targets: np.ndarray   # int32 [N]

    @property
    def shards(self) -> List[np.ndarray]:
        vs = self.workload.shard_rows
        return [self.weight[s * vs:(s + 1) * vs] for s in range(self.workload.n_shards)]

    def digest(self) -> Dict[str, str]:
        return {k: hashlib.sha256(np.ascontiguousarray(getattr(self, k)).tobytes()).hexdigest()[:16]
                for k in ("hidden", "weight", "targets")}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal_rows(seed: int, stream: int, rows: int, cols: int, std: float, rms: bool) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS

    def one(b: int) -> None:
        r0, r1 = b * BLOCK_ROWS, min(rows, (b + 1) * BLOCK_ROWS)
        x = _rng(seed, (stream, b)).standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if rms:
            ms = np.mean(np.square(x, dtype=np.float32), axis=1, dtype=np.float32, keepdims=True)
            x /= np.sqrt(ms + np.float32(RMS_EPS), dtype=np.float32)
        out[r0:r1] = f32_to_bf16_bits(x)

    if nblk == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nblk)))
    return out


def zipf_cdf(vocab: int, s: float) -> np.ndarray:
    k = np.arange(1, vocab + 1, dtype=np.float64)
    p = k ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


def make_targets(w: Workload, seed: int, n_tokens: Optional[int] = None) -> np.ndarray:
    n = w.n_tokens if n_tokens is None else n_tokens
    rng = _rng(seed, (2,))
    if w.targets == "uniform":
        t = rng.integers(0, w.vocab, size=n, dtype=np.int64)
    elif w.targets == "zipf":
        u = rng.random(n)
        t = np.minimum(np.searchsorted(zipf_cdf(w.vocab, w.zipf_s), u, side="right"), w.vocab - 1)
    else:
        raise ValueError(f"unknown target law {w.targets!r}")
    t = t.astype(np.int32)
    k = int(np.floor(w.ignore_frac * n + 0.5))
    if k:
        pos = _rng(seed, (3,)).choice(n, size=k, replace=False)
        t[pos] = IGNORE_INDEX
    return t


def make(w, seed: int = 0, weight: Optional[np.ndarray] = None) -> Batch:
    """Draw one instance of workload ``w`` (a name or a Workload)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w.vocab % w.n_shards:
        raise ValueError("vocabulary must split into equal shards")
    hidden = _normal_rows(seed, 0, w.n_tokens, w.hidden, 1.0, w.rms_norm)
    if weight is None:
        weight = _normal_rows(seed, 1, w.vocab, w.hidden, w.w_std, False)
    targets = make_targets(w, seed)
    return Batch(w, seed, hidden, weight, targets)


def bf16_bits_as_float32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for distribution checks)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)

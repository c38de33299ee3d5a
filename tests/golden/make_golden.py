"""Writes tiny_oracle.json: the CPU oracle's results on the tiny workload (seed 0).

The pages print no worked example for the vocabulary projection, so this file
pins the oracle against later changes of its own arithmetic: the stored values
come only from ``oracle`` (and the seeded inputs from ``workloads``). Rerun it
only when a change to the oracle's arithmetic is justified by the pages, and
say which passage in the commit message.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    b = workloads.make("tiny", seed=0)
    x, w = oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight)
    r = oracle.cross_entropy(x, w, b.targets)
    rows = [0, 1, 17, 128, 255]
    out = {
        "source": "oracle.cross_entropy on workloads.make('tiny', seed=0); written by make_golden.py",
        "inputs_sha256_16": b.digest(),
        "loss": r.loss,
        "loss_sum": r.loss_sum,
        "n_valid": r.n_valid,
        "rows": rows,
        "lse": [r.lse[i] for i in rows],
        "token_loss": [r.token_loss[i] for i in rows],
        "d_hidden_rows_first4": [r.d_hidden[i, :4].tolist() for i in rows],
        "d_weight_rows_first4": [r.d_weight[i, :4].tolist() for i in (0, 255, 256, 1023)],
        "d_hidden_fro": float(np.sqrt((r.d_hidden ** 2).sum())),
        "d_weight_fro": float(np.sqrt((r.d_weight ** 2).sum())),
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

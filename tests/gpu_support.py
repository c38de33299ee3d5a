"""Helpers shared by the GPU tests: device transfer, comparison against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle

LOSS_TOL = 2e-3      # |loss_gpu - loss_oracle| on the mean (or per-token) loss
GRAD_TOL = 2e-2      # max|grad_gpu - grad_oracle| / max|grad_oracle|


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def to_device(batch, weight=None):
    import torch
    hidden = torch.from_numpy(np.ascontiguousarray(batch.hidden).view(np.int16)).view(torch.bfloat16).cuda()
    w = batch.weight if weight is None else weight
    vs = batch.workload.shard_rows
    shards = [torch.from_numpy(np.ascontiguousarray(w[s * vs:(s + 1) * vs]).view(np.int16)).view(torch.bfloat16).cuda()
              for s in range(batch.workload.n_shards)]
    targets = torch.from_numpy(np.ascontiguousarray(batch.targets, dtype=np.int32)).cuda()
    return hidden, shards, targets


def run_lce(hidden, shards, targets, order=None, reduction="mean", dloss=1.0, ignore_index=-100):
    import torch
    import memory_bounded_vocabulary_amd as lce
    loss, lse, tl = lce.forward(hidden, shards, targets, ignore_index=ignore_index, order=order,
                                reduction=reduction, token_loss=True)
    dl = torch.tensor(float(dloss), dtype=torch.float32, device=hidden.device)
    dx, dws = lce.backward(hidden, shards, targets, lse, dl, ignore_index=ignore_index, order=order,
                           reduction=reduction)
    torch.cuda.synchronize()
    return {
        "loss": float(loss.item()),
        "lse": lse.cpu().numpy().astype(np.float64),
        "token_loss": tl.cpu().numpy().astype(np.float64),
        "d_hidden": dx.cpu().numpy().astype(np.float64),
        "d_weight": np.concatenate([g.cpu().numpy() for g in dws]).astype(np.float64),
    }


def rel_max(a, b):
    den = float(np.max(np.abs(b)))
    return float(np.max(np.abs(a - b))) / den if den > 0 else float(np.max(np.abs(a - b)))


def compare(gpu, ref: oracle.Result, name: str, loss_tol=LOSS_TOL, grad_tol=GRAD_TOL):
    dl = abs(gpu["loss"] - ref.loss)
    e_lse = float(np.max(np.abs(gpu["lse"] - ref.lse)))
    e_tok = float(np.max(np.abs(gpu["token_loss"] - ref.token_loss)))
    e_dx = rel_max(gpu["d_hidden"], ref.d_hidden)
    e_dw = rel_max(gpu["d_weight"], ref.d_weight)
    say(f"{name}: loss gpu={gpu['loss']:.6f} oracle={ref.loss:.6f} |d|={dl:.2e}; max|dlse|={e_lse:.2e} "
        f"max|dtok|={e_tok:.2e}; dX rel={e_dx:.2e}; dW rel={e_dw:.2e}")
    assert dl <= loss_tol, (name, dl)
    assert e_lse <= loss_tol * max(1.0, float(np.max(np.abs(ref.lse))) / 10), (name, e_lse)
    assert e_tok <= 10 * loss_tol, (name, e_tok)
    assert e_dx <= grad_tol, (name, e_dx)
    assert e_dw <= grad_tol, (name, e_dw)
    return dict(loss=dl, lse=e_lse, tok=e_tok, dx=e_dx, dw=e_dw)


def oracle_for(batch, weight=None, reduction="mean", dloss=1.0):
    x = oracle.bf16_to_f64(batch.hidden)
    w = oracle.bf16_to_f64(batch.weight if weight is None else weight)
    return oracle.cross_entropy(x, w, batch.targets, reduction=reduction, dloss=dloss)

"""torch.autograd wrapper over the C-ABI calls (argument marshalling only).

    loss = linear_cross_entropy(hidden, shards, targets)      # mean over valid tokens
    loss.backward()                                           # hidden.grad, shard.grad

Forward keeps only the per-token normalizer lse (fp32, N values) besides the
inputs; backward recomputes every logit block from it, so the wrapper also
works under activation checkpointing, where the forward is run again before
the backward. Gradients come back in the inputs' dtype: bf16 inputs get bf16
gradients, accumulated in fp32 inside the library and rounded once.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import backward as _backward
from . import forward as _forward


class LinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, targets, ignore_index, reduction, order, *shards):
        out = _forward(hidden, shards, targets, ignore_index=ignore_index, order=order, reduction=reduction,
                       token_loss=reduction == "none")
        loss, lse = out[0], out[1]
        ctx.save_for_backward(hidden, targets, lse, *shards)
        ctx.cfg = (ignore_index, reduction, order)
        if reduction == "none":
            return out[2]
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        hidden, targets, lse, *shards = ctx.saved_tensors
        ignore_index, reduction, order = ctx.cfg
        g = grad_out.detach().to(torch.float32).contiguous()
        dx, dws = _backward(hidden, shards, targets, lse, g, ignore_index=ignore_index, order=order,
                            reduction=reduction, grad_dtype=hidden.dtype)
        return (dx, None, None, None, None, *dws)


def linear_cross_entropy(hidden, shards: Sequence, targets, ignore_index: int = -100, reduction: str = "mean",
                         order: Optional[Sequence[int]] = None):
    """Cross-entropy of hidden @ concat(shards).T against targets, differentiable in
    hidden and every shard; hidden and the shards share one dtype (bf16)."""
    if any(s.dtype != hidden.dtype for s in shards):
        raise ValueError("hidden and the shards must share one dtype")
    return LinearCrossEntropy.apply(hidden, targets, ignore_index, reduction,
                                    None if order is None else tuple(order), *shards)

"""The forward without a caller workspace (lce_forward_noalloc, built-in
scratch) against lce_forward on the same inputs: the same kernels run, so
loss, lse and token losses must agree bit for bit. Two calls in a row, the
second on a smaller batch (the scratch keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_support import say, to_device

pytestmark = pytest.mark.gpu


def _noalloc(lce, hidden, shards, targets, reduction="mean"):
    import torch
    n = hidden.shape[0]
    loss = torch.full((), float("nan"), dtype=torch.float32, device=hidden.device)
    lse = torch.full((n,), float("nan"), dtype=torch.float32, device=hidden.device)
    tl = torch.full((n,), float("nan"), dtype=torch.float32, device=hidden.device)
    p = len(shards)
    d = lce.make_dims(n, hidden.shape[1], p * shards[0].shape[0], p, reduction=reduction)
    arr = (ctypes.c_void_p * p)(*[s.data_ptr() for s in shards])
    st = lce.lib().lce_forward_noalloc(ctypes.byref(d), hidden.data_ptr(), arr, None, targets.data_ptr(),
                                       loss.data_ptr(), lse.data_ptr(), tl.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == 0, lce.lib().lce_last_error().decode()
    return loss, lse, tl


def test_noalloc_forward_equals_forward_twice():
    import torch
    import memory_bounded_vocabulary_amd as lce
    for name, w in (("stress slice", workloads.WORKLOADS["stress"].with_tokens(1500)),
                    ("tiny", workloads.WORKLOADS["tiny"])):
        say("noalloc forward", name, dict(N=w.n_tokens, H=w.hidden, V=w.vocab, P=w.n_shards))
        b = workloads.make(w)
        hidden, shards, targets = to_device(b)
        loss_n, lse_n, tl_n = _noalloc(lce, hidden, shards, targets)
        loss, lse, tl = lce.forward(hidden, shards, targets, token_loss=True)
        torch.cuda.synchronize()
        say(f"{name}: loss noalloc={loss_n.item():.6f} forward={loss.item():.6f}")
        assert np.isfinite(loss.item())
        assert torch.equal(loss_n, loss)
        assert torch.equal(lse_n, lse)
        assert torch.equal(tl_n, tl)

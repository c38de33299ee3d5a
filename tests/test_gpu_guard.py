"""Guard bands: every buffer the library writes (loss, lse, token losses,
d_hidden, the shard gradients, the workspace) is carved out of a larger
allocation with 4 KiB of poison before and after it; after the calls the
poison must be bit for bit unchanged. Shapes with a ragged last token tile,
a shard that is not a tile multiple, the full stress workload (N = 131071),
bf16 gradients with accumulation, the per-token reduction, the per-round
calls and the forward without a workspace."""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_support import say, to_device

pytestmark = pytest.mark.gpu

GUARD = 4096                       # bytes before and after each buffer
POISON = 0x5A                      # byte pattern (a NaN-free, denormal-free float pattern: 0x5A5A5A5A)


class Guarded:
    """A device buffer of `shape` and `dtype` with poisoned guard bytes around it."""

    def __init__(self, shape, dtype):
        import torch
        self.nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((GUARD + self.nbytes + GUARD,), POISON, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(shape)

    def intact(self):
        import torch
        head = self.raw[:GUARD]
        tail = self.raw[GUARD + self.nbytes:]
        return bool(torch.all(head == POISON).item()) and bool(torch.all(tail == POISON).item())


def _check_all(bufs, what):
    import torch
    torch.cuda.synchronize()
    bad = [name for name, g in bufs.items() if not g.intact()]
    say(what, "guards intact" if not bad else f"guards broken: {bad}")
    assert not bad, (what, bad)


def _run_case(w, grad_dtype="fp32", accumulate=False, reduction="mean", seed=0):
    import torch
    import memory_bounded_vocabulary_amd as lce
    b = workloads.make(w, seed=seed)
    hidden, shards, targets = to_device(b)
    n, h, v, p = w.n_tokens, w.hidden, w.vocab, w.n_shards
    vs = v // p
    gdt = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
    flags = (lce.FLAG_BF16_GRADS if grad_dtype == "bf16" else 0) | \
        (lce.FLAG_ACCUMULATE_DX | lce.FLAG_ACCUMULATE_DW if accumulate else 0)
    wsb = lce.workspace_bytes(n, h, v, p, reduction=reduction, flags=flags)
    bufs = {"loss": Guarded((), torch.float32), "lse": Guarded((n,), torch.float32),
            "token_loss": Guarded((n,), torch.float32), "d_hidden": Guarded((n, h), gdt),
            "workspace": Guarded((wsb,), torch.uint8)}
    for s in range(p):
        bufs[f"d_shard{s}"] = Guarded((vs, h), gdt)
    if accumulate:
        for name, g in bufs.items():
            if name.startswith("d_"):
                g.t.copy_(torch.randn(g.t.shape, device="cuda").to(gdt) * 1e-3)
    d = lce.make_dims(n, h, v, p, reduction=reduction, flags=flags)
    L = lce.lib()
    sp = (ctypes.c_void_p * p)(*[s.data_ptr() for s in shards])
    stream = torch.cuda.current_stream().cuda_stream
    st = L.lce_forward(ctypes.byref(d), hidden.data_ptr(), sp, None, targets.data_ptr(), bufs["loss"].t.data_ptr(),
                       bufs["lse"].t.data_ptr(), bufs["token_loss"].t.data_ptr(), bufs["workspace"].t.data_ptr(), wsb,
                       stream)
    assert st == 0, L.lce_last_error().decode()
    dloss = torch.rand((n,), device="cuda") if reduction == "none" else torch.ones((), device="cuda")
    dp = (ctypes.c_void_p * p)(*[bufs[f"d_shard{s}"].t.data_ptr() for s in range(p)])
    st = L.lce_backward(ctypes.byref(d), hidden.data_ptr(), sp, None, targets.data_ptr(), bufs["lse"].t.data_ptr(),
                        dloss.data_ptr(), bufs["d_hidden"].t.data_ptr(), dp, bufs["workspace"].t.data_ptr(), wsb,
                        stream)
    assert st == 0, L.lce_last_error().decode()
    _check_all(bufs, f"{w.name} {grad_dtype} acc={accumulate} {reduction}")
    assert bool(torch.isfinite(bufs["loss"].t).item())
    return lce, d, hidden, shards, targets, bufs


CASES = [
    ("ragged N, ragged shard", dict(n_tokens=777, hidden=256, vocab=4 * 1000, n_shards=4, ignore_frac=0.1,
                                    w_std=0.05), "fp32", False, "mean"),
    ("bf16 gradients, accumulating", dict(n_tokens=1000, hidden=128, vocab=3 * 700, n_shards=3, ignore_frac=0.3,
                                          w_std=0.1), "bf16", True, "mean"),
    ("per-token reduction", dict(n_tokens=513, hidden=64, vocab=2 * 20000, n_shards=2, ignore_frac=0.05,
                                 w_std=0.3), "fp32", False, "none"),
    ("two token chunks, half ignored", dict(n_tokens=24000, hidden=64, vocab=2 * 20000, n_shards=2,
                                            ignore_frac=0.5, w_std=0.3), "fp32", False, "mean"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_guard_bands(case):
    name, dims, gdt, acc, red = case
    w = workloads.WORKLOADS["tiny"].with_dims(name=name, **dims)
    say("guard bands", name, dims)
    _run_case(w, gdt, acc, red, seed=5)


def test_guard_bands_stress_full_size():
    w = workloads.WORKLOADS["stress"]
    say("guard bands, full stress workload", dict(N=w.n_tokens, H=w.hidden, V=w.vocab, P=w.n_shards))
    _run_case(w)


def test_guard_bands_round_calls_and_noalloc():
    import torch
    w = workloads.WORKLOADS["tiny"].with_dims(name="rounds", n_tokens=700, hidden=192, vocab=3 * 500, n_shards=3,
                                              ignore_frac=0.4, w_std=0.1)
    say("guard bands, round calls")
    lce, d, hidden, shards, targets, bufs = _run_case(w)
    n, h, p = w.n_tokens, w.hidden, w.n_shards
    wsb = lce.workspace_bytes(n, h, w.vocab, p)
    L = lce.lib()
    stream = torch.cuda.current_stream().cuda_stream
    order = [(p - k) % p for k in range(p)]
    ws = bufs["workspace"].t.data_ptr()
    for k, s in enumerate(order):
        assert L.lce_fwd_round(ctypes.byref(d), k, s, hidden.data_ptr(), shards[s].data_ptr(), targets.data_ptr(), ws,
                               wsb, stream) == 0
    assert L.lce_fwd_finish(ctypes.byref(d), targets.data_ptr(), bufs["loss"].t.data_ptr(), bufs["lse"].t.data_ptr(),
                            bufs["token_loss"].t.data_ptr(), ws, wsb, stream) == 0
    dloss = torch.ones((), device="cuda")
    for k, s in enumerate(order):
        assert L.lce_bwd_round(ctypes.byref(d), k, s, hidden.data_ptr(), shards[s].data_ptr(), targets.data_ptr(),
                               bufs["lse"].t.data_ptr(), dloss.data_ptr(), bufs["d_hidden"].t.data_ptr(),
                               bufs[f"d_shard{s}"].t.data_ptr(), 0, ws, wsb, stream) == 0
    _check_all(bufs, "round calls")
    sp = (ctypes.c_void_p * p)(*[s.data_ptr() for s in shards])
    assert L.lce_forward_noalloc(ctypes.byref(d), hidden.data_ptr(), sp, None, targets.data_ptr(),
                                 bufs["loss"].t.data_ptr(), bufs["lse"].t.data_ptr(),
                                 bufs["token_loss"].t.data_ptr(), stream) == 0
    _check_all(bufs, "forward without a workspace")

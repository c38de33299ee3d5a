"""Device memory of the path on the GPU: the transient (peak minus inputs and
outputs) is bounded independently of the vocabulary, and the library itself
allocates nothing.

V sweeps {16032, 32064, 64128, 128256} at N = 16384, H = 4096, P = 8. The
backward's two bf16 gradient chunks hold at most 2^27 elements each (at
N = 16384 they are min(V/P, 8192) vocabulary rows wide), so the transient
grows with V/P until that budget and is flat after it, bounded by the same
figure whatever V is. At the largest V it is below the
one-strip live set N x V/P x 4 bytes of the pages' own scheme ("Flattening
Every Memory Peak in Long-Context Mixture-of-Experts Training", section 3.2),
and at every V far below the full logits. Values are random (the check is
about memory only); the loss must still be finite.
"""
import pytest

from gpu_support import say

pytestmark = pytest.mark.gpu

N, H, P = 16384, 4096, 8
VOCABS = [16032, 32064, 64128, 128256]


def _run(v, keep_ignored_rows=False):
    import torch
    import memory_bounded_vocabulary_amd as lce
    dev = torch.device("cuda:0")
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(dev)
    g = torch.Generator(device=dev).manual_seed(v)
    vs = v // P
    hidden = torch.randn((N, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    shards = [(torch.randn((vs, H), generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
              for _ in range(P)]
    targets = torch.randint(0, v, (N,), generator=g, device=dev, dtype=torch.int32)
    d_hidden = torch.empty((N, H), dtype=torch.float32, device=dev)
    d_shards = [torch.empty((vs, H), dtype=torch.float32, device=dev) for _ in range(P)]
    dloss = torch.ones((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize(dev)
    # what the caching allocator holds for the inputs and gradient outputs
    # (their sizes plus its own rounding), before the workspace exists
    io_alloc = torch.cuda.memory_allocated(dev) - base
    flags = lce.FLAG_KEEP_IGNORED_ROWS if keep_ignored_rows else 0
    ws = lce.alloc_workspace(N, H, v, P, dev, flags=flags)
    torch.cuda.synchronize(dev)
    # warm-up call, then the measured one
    loss, lse = lce.forward(hidden, shards, targets, workspace=ws)
    lce.backward(hidden, shards, targets, lse, dloss, workspace=ws, d_hidden=d_hidden, d_shards=d_shards,
                 keep_ignored_rows=keep_ignored_rows)
    del loss, lse
    torch.cuda.synchronize(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    free0 = torch.cuda.mem_get_info(dev)[0]
    loss, lse = lce.forward(hidden, shards, targets, workspace=ws)
    lce.backward(hidden, shards, targets, lse, dloss, workspace=ws, d_hidden=d_hidden, d_shards=d_shards,
                 keep_ignored_rows=keep_ignored_rows)
    torch.cuda.synchronize(dev)
    free1 = torch.cuda.mem_get_info(dev)[0]
    peak = torch.cuda.max_memory_allocated(dev) - base
    transient = peak - io_alloc   # workspace, lse, loss
    res = dict(v=v, transient=transient, workspace=ws.numel(), free_delta=free0 - free1,
               strip=N * vs * 4, logits=N * v * 4, loss=float(loss.item()))
    del hidden, shards, targets, d_hidden, d_shards, ws, loss, lse
    torch.cuda.empty_cache()
    return res


@pytest.mark.parametrize("keep_ignored_rows", [False, True], ids=["default", "keep ignored rows"])
def test_transient_bounded_independently_of_vocab(keep_ignored_rows):
    """Default: the workspace also holds the gathered hidden rows of the kept
    tokens (at N = 16384 all of them, N x H bf16), which lets the backward skip
    ignored tokens; with LCE_FLAG_KEEP_IGNORED_ROWS it does not, and the
    transient is the G chunks and O(N) state alone."""
    import math
    import memory_bounded_vocabulary_amd as lce
    flags = lce.FLAG_KEEP_IGNORED_ROWS if keep_ignored_rows else 0
    copy = 0 if keep_ignored_rows else N * H * 2
    rows = []
    for v in VOCABS:
        say("memory sweep", dict(N=N, H=H, V=v, P=P, keep_ignored_rows=keep_ignored_rows))
        r = _run(v, keep_ignored_rows)
        say(r)
        rows.append(r)
        assert math.isfinite(r["loss"])
        # nothing beyond what torch allocated: the library itself allocates no device memory
        assert r["free_delta"] == 0, r
        # the transient is the workspace plus lse and loss (plus allocator rounding)
        assert r["transient"] <= r["workspace"] + (2 << 20), r
        # the gathered copy aside, far below the full logits at every V
        assert r["transient"] - copy < r["logits"] / 4, r
    bound = lce.workspace_bytes(N, H, P * 8192, P, flags=flags)
    assert max(r["transient"] for r in rows) <= bound + (2 << 20)
    # flat once the G chunks reach their budget (64128 / 8 = 8016 rows pads to 8192)
    assert rows[-1]["workspace"] == rows[-2]["workspace"]
    assert abs(rows[-1]["transient"] - rows[-2]["transient"]) <= (2 << 20)
    assert rows[-1]["transient"] < rows[-1]["strip"]
    if not keep_ignored_rows:
        assert lce.workspace_bytes(N, H, P * 8192, P) - bound == 0
        assert lce.workspace_bytes(N, H, P * 8192, P, flags=lce.FLAG_KEEP_IGNORED_ROWS) == bound - copy

"""The calls under HIP graph capture and from several host threads.

The library enqueues kernels only (no allocation, no memset, no host
synchronisation), so a forward + backward can be captured into a graph and
replayed. Each replay here follows eager work of the program's own (other
calls of the library on other buffers, refills of the graph's outputs, a
device synchronisation) and must reproduce the eager result bit for bit; the
kernels are deterministic (fixed-order merges, atomics only count arrivals).
"""
import threading

import pytest

import workloads
from gpu_support import say, to_device

pytestmark = pytest.mark.gpu

BASE = workloads.WORKLOADS["tiny"]


def _case(n=700, h=256, v=4 * 1000, p=4, seed=9):
    w = BASE.with_dims(name="graph", n_tokens=n, hidden=h, vocab=v, n_shards=p, ignore_frac=0.1, w_std=0.05)
    return workloads.make(w, seed=seed)


def _run(lce, hidden, shards, targets, ws, dx, dws, dloss):
    loss, lse = lce.forward(hidden, shards, targets, workspace=ws)
    lce.backward(hidden, shards, targets, lse, dloss, workspace=ws, d_hidden=dx, d_shards=dws)
    return loss, lse


@pytest.mark.parametrize("dims", [(700, 256, 4 * 1000, 4), (24000, 64, 2 * 20000, 2)],
                         ids=["one chunk", "two token and two vocab chunks"])
def test_graph_replays_match_eager(dims):
    import torch
    import memory_bounded_vocabulary_amd as lce
    n, h, v, p = dims
    say("graph capture", dict(N=n, H=h, V=v, P=p))
    b = _case(n, h, v, p)
    hidden, shards, targets = to_device(b)
    dloss = torch.ones((), dtype=torch.float32, device="cuda")

    def bufs():
        return (lce.alloc_workspace(n, h, v, p), torch.empty((n, h), dtype=torch.float32, device="cuda"),
                [torch.empty((v // p, h), dtype=torch.float32, device="cuda") for _ in range(p)])

    ws_e, dx_e, dws_e = bufs()
    loss_e, lse_e = _run(lce, hidden, shards, targets, ws_e, dx_e, dws_e, dloss)
    torch.cuda.synchronize()

    ws_g, dx_g, dws_g = bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(lce, hidden, shards, targets, ws_g, dx_g, dws_g, dloss)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loss_g, lse_g = _run(lce, hidden, shards, targets, ws_g, dx_g, dws_g, dloss)

    other = _case(n, h, v, p, seed=10)
    oh, osh, ot = to_device(other)
    ws_o, dx_o, dws_o = bufs()
    for rep in range(3):
        # the program's own eager work between replays
        _run(lce, oh, osh, ot, ws_o, dx_o, dws_o, dloss)
        dx_g.fill_(float("nan"))
        for d in dws_g:
            d.fill_(float("nan"))
        lse_g.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}: loss {loss_g.item():.6f} (eager {loss_e.item():.6f})")
        assert torch.equal(loss_g, loss_e)
        assert torch.equal(lse_g, lse_e)
        assert torch.equal(dx_g, dx_e)
        for a, c in zip(dws_g, dws_e):
            assert torch.equal(a, c)


def test_concurrent_host_threads():
    """Two host threads, each with its own stream and workspace, calling at the
    same time, get the results of serial calls bit for bit."""
    import torch
    import memory_bounded_vocabulary_amd as lce
    say("two host threads")
    batches = [_case(seed=20 + i) for i in range(2)]
    dev = [to_device(b) for b in batches]
    ref = []
    for hidden, shards, targets in dev:
        loss, lse = lce.forward(hidden, shards, targets)
        dx, dws = lce.backward(hidden, shards, targets, lse, 1.0)
        ref.append((loss, lse, dx, dws))
    torch.cuda.synchronize()
    out = [None, None]
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                hidden, shards, targets = dev[i]
                res = []
                for _ in range(5):
                    loss, lse = lce.forward(hidden, shards, targets)
                    dx, dws = lce.backward(hidden, shards, targets, lse, 1.0)
                    res.append((loss, lse, dx, dws))
            s.synchronize()
            out[i] = res
        except Exception as e:  # surfaced in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(2):
        for loss, lse, dx, dws in out[i]:
            assert torch.equal(loss, ref[i][0]) and torch.equal(lse, ref[i][1]) and torch.equal(dx, ref[i][2])
            for a, c in zip(dws, ref[i][3]):
                assert torch.equal(a, c)

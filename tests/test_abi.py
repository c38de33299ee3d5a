"""C-ABI library: loads, exports what include/lce.h declares, and rejects bad
arguments on the host before any GPU work (no GPU needed)."""
import ctypes
import os
import re

import pytest

import memory_bounded_vocabulary_amd as lce
from memory_bounded_vocabulary_amd import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lce.h")
FAKE = 0x10000          # a 16-byte-aligned stand-in for a device pointer; never dereferenced


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^LCE_API\s+[\w\s\*]+?\b(lce_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_symbols():
    assert declared_symbols() == sorted(lce.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = lce.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert lce.version() == (1, 2)


def test_single_hip_runtime_in_process():
    lce.lib()
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def _dims(n=256, h=128, v=1024, p=4, ignore=-100, red=0, flags=0):
    return Dims(n, h, v, p, ignore, red, flags)


def _fwd(d, hidden=FAKE, shards=None, order=None, targets=FAKE, loss=FAKE, lse=FAKE, tl=None, ws=FAKE,
         ws_bytes=None):
    L = lce.lib()
    p = d.n_shards if d is not None else 1
    shards = [FAKE] * max(p, 1) if shards is None else shards
    arr = (ctypes.c_void_p * len(shards))(*shards)
    if ws_bytes is None:
        ws_bytes = L.lce_workspace_bytes(ctypes.byref(d)) if d is not None else 0
    dp = ctypes.byref(d) if d is not None else None
    ordp = (ctypes.c_int32 * len(order))(*order) if order is not None else None
    return L.lce_forward(dp, hidden, arr, ordp, targets, loss, lse, tl, ws, ws_bytes, None)


def _bwd(d, hidden=FAKE, lse=FAKE, dloss=FAKE, dx=FAKE, dws=None, ws=FAKE, ws_bytes=None, order=None):
    L = lce.lib()
    shards = (ctypes.c_void_p * d.n_shards)(*([FAKE] * d.n_shards))
    dws = [FAKE] * d.n_shards if dws is None else dws
    dwa = (ctypes.c_void_p * len(dws))(*dws)
    if ws_bytes is None:
        ws_bytes = L.lce_workspace_bytes(ctypes.byref(d))
    ordp = (ctypes.c_int32 * len(order))(*order) if order is not None else None
    return L.lce_backward(ctypes.byref(d), hidden, shards, ordp, FAKE, lse, dloss, dx, dwa, ws, ws_bytes, None)


@pytest.mark.parametrize("dims,status", [
    (_dims(n=-1), lce.ERR_INVALID_ARG),
    (_dims(h=0), lce.ERR_INVALID_ARG),
    (_dims(v=0), lce.ERR_INVALID_ARG),
    (_dims(p=0), lce.ERR_INVALID_ARG),
    (_dims(p=257, v=257 * 4), lce.ERR_INVALID_ARG),
    (_dims(v=1000, p=3), lce.ERR_INVALID_ARG),
    (_dims(flags=16), lce.ERR_INVALID_ARG),
    (_dims(red=3), lce.ERR_INVALID_ARG),
    (_dims(h=100), lce.ERR_UNSUPPORTED),
    (_dims(n=1 << 22, h=1024), lce.ERR_UNSUPPORTED),
])
def test_bad_dims_rejected(dims, status):
    L = lce.lib()
    assert L.lce_workspace_bytes(ctypes.byref(dims)) == 0
    assert _fwd(dims, ws_bytes=1 << 30) == status
    assert L.lce_last_error().decode()


def test_null_and_misaligned_pointers_rejected():
    d = _dims()
    assert _fwd(None) == lce.ERR_INVALID_ARG
    assert _fwd(d, hidden=None) == lce.ERR_INVALID_ARG
    assert _fwd(d, targets=None) == lce.ERR_INVALID_ARG
    assert _fwd(d, loss=None) == lce.ERR_INVALID_ARG
    assert _fwd(d, lse=None) == lce.ERR_INVALID_ARG
    assert _fwd(d, ws=None) == lce.ERR_INVALID_ARG
    assert _fwd(d, shards=[FAKE, FAKE, None, FAKE]) == lce.ERR_INVALID_ARG
    assert _fwd(d, hidden=FAKE + 8) == lce.ERR_UNSUPPORTED
    assert _fwd(d, shards=[FAKE, FAKE + 2, FAKE, FAKE]) == lce.ERR_UNSUPPORTED
    assert _fwd(d, lse=FAKE + 4) == lce.ERR_UNSUPPORTED
    assert _fwd(d, ws=FAKE + 4) == lce.ERR_UNSUPPORTED
    assert _bwd(d, dx=None) == lce.ERR_INVALID_ARG
    assert _bwd(d, dloss=None) == lce.ERR_INVALID_ARG
    assert _bwd(d, lse=None) == lce.ERR_INVALID_ARG
    assert _bwd(d, dws=[FAKE, None, FAKE, FAKE]) == lce.ERR_INVALID_ARG
    assert _bwd(d, dx=FAKE + 4) == lce.ERR_UNSUPPORTED


def test_order_must_be_permutation():
    d = _dims()
    for bad in ([0, 1, 2, 2], [0, 1, 2, 4], [-1, 0, 1, 2]):
        assert _fwd(d, order=bad) == lce.ERR_INVALID_ARG
        assert "permutation" in lce.lib().lce_last_error().decode()
        assert _bwd(d, order=bad) == lce.ERR_INVALID_ARG


def test_workspace_too_small():
    d = _dims()
    need = lce.lib().lce_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert _fwd(d, ws_bytes=lce.state_bytes(d) - 1) == lce.ERR_WORKSPACE
    assert "forward needs %d" % lce.state_bytes(d) in lce.lib().lce_last_error().decode()
    assert _bwd(d, ws_bytes=need - 1) == lce.ERR_WORKSPACE
    assert "needs %d" % need in lce.lib().lce_last_error().decode()


def test_status_strings():
    L = lce.lib()
    for st in (0, -1, -2, -3, -4):
        assert L.lce_status_string(st).decode()
    assert L.lce_status_string(99).decode() == "unknown status"


def test_workspace_is_bounded_independently_of_vocab():
    # N and H fixed, V swept: the workspace never holds a logit strip (N x V/P).
    # It is O(N) per-token state, the kept tokens' hidden rows (N x H bf16) and
    # two G chunks of at most 2^27 bf16 elements each, whatever V is.
    n, h, p = 16384, 4096, 8
    bound = 64 * n + n * h * 2 + 2 * (2 ** 27) * 2 + 4096
    for vs in (2004, 4008, 8016, 16032, 32064, 64128, 256512):
        assert lce.workspace_bytes(n, h, p * vs, p) <= bound, vs
    assert bound < n * 16032 * 4          # far below one logit strip at the large workload
    assert lce.workspace_bytes(n, h, 8 * 128256 * 2, 8) <= bound


def _fwd_round(d, rnd=0, shard=0, hidden=FAKE, w=FAKE, targets=FAKE, ws=FAKE, ws_bytes=None):
    L = lce.lib()
    if ws_bytes is None:
        ws_bytes = L.lce_workspace_bytes(ctypes.byref(d))
    return L.lce_fwd_round(ctypes.byref(d), rnd, shard, hidden, w, targets, ws, ws_bytes, None)


def _fwd_finish(d, targets=FAKE, loss=FAKE, lse=FAKE, tl=None, ws=FAKE, ws_bytes=None):
    L = lce.lib()
    if ws_bytes is None:
        ws_bytes = L.lce_workspace_bytes(ctypes.byref(d))
    return L.lce_fwd_finish(ctypes.byref(d), targets, loss, lse, tl, ws, ws_bytes, None)


def _bwd_round(d, rnd=0, shard=0, w=FAKE, lse=FAKE, dloss=FAKE, dx=FAKE, dw=FAKE, ws=FAKE, ws_bytes=None):
    L = lce.lib()
    if ws_bytes is None:
        ws_bytes = L.lce_workspace_bytes(ctypes.byref(d))
    return L.lce_bwd_round(ctypes.byref(d), rnd, shard, FAKE, w, FAKE, lse, dloss, dx, dw, 0, ws, ws_bytes, None)


def test_round_entry_points_reject_bad_arguments():
    d = _dims()
    for bad in (-1, 4):
        assert _fwd_round(d, rnd=bad) == lce.ERR_INVALID_ARG
        assert "round" in lce.lib().lce_last_error().decode()
        assert _fwd_round(d, shard=bad) == lce.ERR_INVALID_ARG
        assert _bwd_round(d, rnd=bad) == lce.ERR_INVALID_ARG
        assert _bwd_round(d, shard=bad) == lce.ERR_INVALID_ARG
    assert _fwd_round(d, w=None) == lce.ERR_INVALID_ARG
    assert _fwd_round(d, hidden=None) == lce.ERR_INVALID_ARG
    assert _fwd_round(d, w=FAKE + 8) == lce.ERR_UNSUPPORTED
    assert _fwd_round(d, ws=None) == lce.ERR_INVALID_ARG
    assert _fwd_round(_dims(h=100)) == lce.ERR_UNSUPPORTED
    assert _fwd_finish(d, loss=None) == lce.ERR_INVALID_ARG
    assert _fwd_finish(d, lse=FAKE + 4) == lce.ERR_UNSUPPORTED
    assert _fwd_finish(d, tl=FAKE + 4) == lce.ERR_UNSUPPORTED
    assert _bwd_round(d, dw=None) == lce.ERR_INVALID_ARG
    assert _bwd_round(d, dloss=None) == lce.ERR_INVALID_ARG
    assert _bwd_round(d, dw=FAKE + 4) == lce.ERR_UNSUPPORTED
    need = lce.lib().lce_workspace_bytes(ctypes.byref(d))
    assert _fwd_round(d, ws_bytes=need - 1) == lce.ERR_WORKSPACE
    assert _fwd_finish(d, ws_bytes=need - 1) == lce.ERR_WORKSPACE
    assert _bwd_round(d, ws_bytes=need - 1) == lce.ERR_WORKSPACE


def test_per_token_reduction_needs_token_loss():
    d = _dims(red=2)
    assert _fwd(d, tl=None) == lce.ERR_INVALID_ARG
    assert "token_loss" in lce.lib().lce_last_error().decode()
    assert _fwd_finish(d, tl=None) == lce.ERR_INVALID_ARG


def test_bf16_gradient_workspace():
    # fp32 accumulators for d_hidden (N x H) and one gradient chunk (at most 16384 x H)
    n, h, v, p = 1000, 512, 8 * 20000, 8
    plain = lce.workspace_bytes(n, h, v, p)
    bf16 = lce.workspace_bytes(n, h, v, p, flags=lce.FLAG_BF16_GRADS)
    assert n * h * 4 + 256 * h * 4 <= bf16 - plain <= n * h * 4 + 16384 * h * 4 + 1024
    assert lce.workspace_bytes(n, h, v, p, flags=lce.FLAG_ACCUMULATE_DX | lce.FLAG_ACCUMULATE_DW) == plain
    # the accumulator does not grow with V past the chunk bound
    assert lce.workspace_bytes(n, h, 8 * 200000, 8, flags=lce.FLAG_BF16_GRADS) - \
        lce.workspace_bytes(n, h, 8 * 200000, 8) <= n * h * 4 + 16384 * h * 4 + 1024


def test_ring_payload_choice():
    # one forward + one backward hop: a shard moves (V/P) H (2 + 2 + 4) bytes,
    # a batch N H (2 + 2 + 4) bytes plus O(N) state: the smaller side moves
    for name, n, h, v, p, want in [("long", 65536, 7168, 129280, 8, "weights"),
                                   ("stress", 131071, 4096, 151936, 16, "weights"),
                                   ("short batch", 1024, 4096, 128256, 8, "activations"),
                                   ("many shards", 16384, 4096, 128256 * 4, 8, "activations")]:
        choice, wb, xb = lce.ring_payload(lce.make_dims(n, h, v, p))
        assert choice == want, (name, wb, xb)
        assert wb == (v // p) * h * 8
        assert n * h * 8 <= xb <= n * h * 8 + 256 * n + 4096  # state: up to 16 (m, z) pairs per token
    assert lce.lib().lce_ring_payload(ctypes.byref(_dims(h=100)), None, None) == lce.ERR_UNSUPPORTED


def test_state_bytes_is_a_prefix_of_the_workspace():
    for flags in (0, lce.FLAG_BF16_GRADS):
        d = lce.make_dims(5000, 1024, 8 * 3000, 8, flags=flags)
        sb, wsb = lce.state_bytes(d), lce.workspace_bytes(5000, 1024, 8 * 3000, 8, flags=flags)
        assert 0 < sb <= wsb
        assert sb >= 8 * 5000  # at least one (m, z) pair per token
        if flags:
            assert sb >= 5000 * 1024 * 4  # the fp32 dX accumulator
        else:
            assert sb < 5000 * 1024  # O(N), no H-sized term
    assert lce.state_bytes(_dims(v=1000, p=3)) == 0


def test_last_error_is_per_thread():
    import threading
    results = {}

    def work(i):
        d = _dims(v=1000 + 3 * i + 1, p=3) if i % 2 else _dims(h=100 + 2 * i)  # never a valid shape
        msgs = set()
        for _ in range(200):
            st = _fwd(d, ws_bytes=1 << 30)
            msgs.add((st, lce.lib().lce_last_error().decode()))
        results[i] = msgs

    threads = [threading.Thread(target=work, args=(i,)) for i in range(6)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i, msgs in results.items():
        assert len(msgs) == 1, (i, msgs)          # never another thread's message
        st, msg = next(iter(msgs))
        if i % 2:
            assert st == lce.ERR_INVALID_ARG and "divisible" in msg
        else:
            assert st == lce.ERR_UNSUPPORTED and "multiple of 64" in msg


def test_plain_c_caller(tmp_path):
    """The ABI from C: compile tests/c_abi_check.c with gcc against include/lce.h,
    link the built library, run it (host-side checks only)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib_dir = os.path.dirname(lce.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe, "-L", lib_dir, "-llce",
                    f"-Wl,-rpath,{lib_dir}"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout


def test_empty_batch_is_a_valid_shape():
    d = _dims(n=0)
    assert lce.lib().lce_workspace_bytes(ctypes.byref(d)) > 0
    assert lce.state_bytes(d) > 0
    # per-token pointers may be NULL, the loss and the shard gradients may not
    assert _fwd(d, loss=None) == lce.ERR_INVALID_ARG
    assert _bwd(d, dws=[FAKE, None, FAKE, FAKE]) == lce.ERR_INVALID_ARG


def test_binding_rejects_layouts_the_abi_cannot_take():
    """The binding checks dtypes, shapes and contiguity before any pointer reaches
    the library (host tensors are enough: the checks run before the device check)."""
    import torch
    h = torch.zeros((8, 64), dtype=torch.bfloat16)
    sh = [torch.zeros((16, 64), dtype=torch.bfloat16) for _ in range(2)]
    t = torch.zeros((8,), dtype=torch.int32)
    with pytest.raises(ValueError, match="bf16"):
        lce.forward(h.float(), sh, t)
    with pytest.raises(ValueError, match="contiguous"):
        lce.forward(torch.zeros((64, 8), dtype=torch.bfloat16).t(), sh, t)
    with pytest.raises(ValueError, match="shard"):
        lce.forward(h, [sh[0], torch.zeros((15, 64), dtype=torch.bfloat16)], t)
    with pytest.raises(ValueError, match="int32"):
        lce.forward(h, sh, t.long())
    with pytest.raises(ValueError, match="lse"):
        lce.backward(h, sh, t, torch.zeros((7,)), 1.0)
    with pytest.raises(ValueError, match="GPU"):
        lce.forward(h, sh, t)


def test_binding_round_calls_check_dims_against_tensors():
    """The per-round calls take N, H and V/P from dims: a mismatch, a gradient
    buffer of the wrong dtype or shape, or a dloss of the wrong size is refused
    before any pointer reaches the library (it would otherwise read or write
    past a buffer)."""
    import torch
    n, h, vs, p = 8, 64, 16, 2
    x = torch.zeros((n, h), dtype=torch.bfloat16)
    w = torch.zeros((vs, h), dtype=torch.bfloat16)
    t = torch.zeros((n,), dtype=torch.int32)
    lse = torch.zeros((n,))
    dl = torch.ones(())
    dims = lce.make_dims(n, h, vs * p, p)
    ws = torch.zeros(lce.workspace_bytes(n, h, vs * p, p), dtype=torch.uint8)
    dx, dw = torch.zeros((n, h)), torch.zeros((vs, h))

    def fr(d=dims, **kw):
        a = dict(hidden=x, shard=w, targets=t, workspace=ws)
        a.update(kw)
        lce.fwd_round(d, 0, 0, a["hidden"], a["shard"], a["targets"], a["workspace"])

    def br(d=dims, **kw):
        a = dict(hidden=x, shard=w, targets=t, lse=lse, dloss=dl, d_hidden=dx, d_shard=dw, workspace=ws)
        a.update(kw)
        lce.bwd_round(d, 0, 0, a["hidden"], a["shard"], a["targets"], a["lse"], a["dloss"], a["d_hidden"],
                      a["d_shard"], False, a["workspace"])

    for bad in (lce.make_dims(n + 8, h, vs * p, p), lce.make_dims(n, 2 * h, vs * p, p),
                lce.make_dims(n, h, 2 * vs * p, p), lce.make_dims(n, h, vs * p + 1, p)):
        with pytest.raises(ValueError, match="dims"):
            fr(bad)
        with pytest.raises(ValueError, match="dims"):
            br(bad)
    with pytest.raises(ValueError, match="targets"):
        lce.fwd_finish(lce.make_dims(n + 1, h, vs * p, p), t, ws)
    with pytest.raises(ValueError, match="workspace"):
        fr(workspace=ws[:-16])
    with pytest.raises(ValueError, match="workspace"):
        lce.fwd_finish(dims, t, ws[:16])
    # bf16 gradient buffers without the bf16 flag (and fp32 ones with it)
    with pytest.raises(ValueError, match="d_shard"):
        br(d_shard=dw.bfloat16())
    with pytest.raises(ValueError, match="d_hidden"):
        br(d_hidden=dx.bfloat16())
    d16 = lce.make_dims(n, h, vs * p, p, flags=lce.FLAG_BF16_GRADS)
    ws16 = torch.zeros(lce.workspace_bytes(n, h, vs * p, p, flags=lce.FLAG_BF16_GRADS), dtype=torch.uint8)
    with pytest.raises(ValueError, match="d_hidden"):
        br(d16, workspace=ws16)
    with pytest.raises(ValueError, match="d_hidden"):
        br(d_hidden=torch.zeros((n, h + 64)))
    with pytest.raises(ValueError, match="d_shard"):
        br(d_shard=torch.zeros((vs + 1, h)))
    with pytest.raises(ValueError, match="dloss"):
        br(dloss=torch.ones((n,)))
    with pytest.raises(ValueError, match="dloss"):
        br(dloss=torch.ones((), dtype=torch.float64))
    with pytest.raises(ValueError, match="dloss"):
        br(lce.make_dims(n, h, vs * p, p, reduction="none"), dloss=dl)
    with pytest.raises(ValueError, match="lse"):
        br(lse=torch.zeros((n + 1,)))
    # consistent host tensors pass every layout check and stop at the device check
    with pytest.raises(ValueError, match="GPU"):
        fr()
    with pytest.raises(ValueError, match="GPU"):
        br()
    with pytest.raises(ValueError, match="GPU"):
        br(d16, workspace=ws16, d_hidden=dx.bfloat16(), d_shard=dw.bfloat16())
    with pytest.raises(ValueError, match="GPU"):
        lce.fwd_finish(dims, t, ws)
    with pytest.raises(ValueError, match="GPU"):
        lce.backward(x, [w, w], t, lse, torch.ones((n,)))


def test_noalloc_forward_refuses_a_batch_beyond_its_scratch():
    """lce_forward_noalloc checks the forward's scratch size on the host before
    any GPU work (N = 2^19 tokens with 8 vocabulary splits need 34 MiB)."""
    L = lce.lib()
    assert L.lce_forward_noalloc_max_bytes() == 32 << 20
    d = lce.make_dims(1 << 19, 64, 16 * 2048, 16)
    arr = (ctypes.c_void_p * 16)(*([FAKE] * 16))
    st = L.lce_forward_noalloc(ctypes.byref(d), FAKE, arr, None, FAKE, FAKE, FAKE, None, None)
    assert st == lce.ERR_WORKSPACE
    assert "scratch" in L.lce_last_error().decode()
    # argument checks come first, as in lce_forward
    assert L.lce_forward_noalloc(ctypes.byref(d), None, arr, None, FAKE, FAKE, FAKE, None, None) == lce.ERR_INVALID_ARG
    assert L.lce_forward_noalloc(ctypes.byref(_dims(h=100)), FAKE, arr, None, FAKE, FAKE, FAKE, None, None) == \
        lce.ERR_UNSUPPORTED

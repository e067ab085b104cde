"""dvm_launch_noalloc (the launch for callers that cannot allocate) against
dvm_launch, through the C ABI.

Reduce-all programs are the ones whose kernels use scratch (one partial per
workgroup, combined by a second launch).  Both entry points run the same
kernels, tile order and partial combine, so the results must be
bit-identical.  Two calls in a row, the second over a smaller input, so the
second call runs on an array that still holds the first call's partials.
"""
import numpy as np
import pytest

import workloads as W
from oracle import ops as O
from tests.dvm_helpers import host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dvm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import device_bytecode_vm_amd as m
    return m


def say(*a):
    print("CASE", *a, flush=True)


def encode_reduce_all(dvm, ectx, x, out, op):
    """The reduce-all program over device tensor x into out, encoded on an
    encode-only context (which holds it instead of launching it)."""
    g = dvm.Graph(ectx)
    g.op(op, g.input(x), out=out, live=True, axis=0x7FFFFFFF)
    p = g.take_program()
    assert p is not None and p.header()["tmpl"] == 2
    return p


@pytest.mark.parametrize("op", ["reduce_sum", "reduce_max"])
def test_noalloc_equals_launch(dvm, op):
    import torch
    ectx, dctx = dvm.Context(-1), dvm.Context(0)
    stream = torch.cuda.current_stream()
    for n in (16384, 3001):                          # the second call is smaller
        say("noalloc", op, n)
        x = W.device_normal((n, 4096), seed=50 + n)
        s_ref = torch.full((), -1.0, dtype=torch.float32, device="cuda")
        s_new = torch.full((), -2.0, dtype=torch.float32, device="cuda")
        p_ref = encode_reduce_all(dvm, ectx, x, s_ref, op)
        p_new = encode_reduce_all(dvm, ectx, x, s_new, op)
        assert p_new.header()["block_dim"] > 1
        p_ref.launch(stream, ctx=dctx)
        p_new.launch_noalloc(stream, ctx=dctx)
        torch.cuda.synchronize()
        a, b = float(s_ref.item()), float(s_new.item())
        assert np.float32(a).tobytes() == np.float32(b).tobytes(), (a, b)
        xh = host64(x)
        if op == "reduce_sum":
            assert abs(b - float(np.sum(xh))) <= O.sum_guard_band(xh)
        else:
            assert b == float(np.max(xh))


def test_noalloc_elementwise_and_limit(dvm):
    import torch
    from device_bytecode_vm_amd import _lib as L
    ectx, dctx = dvm.Context(-1), dvm.Context(0)
    stream = torch.cuda.current_stream()
    say("noalloc_elementwise")
    x = W.device_normal((513, 1031), seed=3)
    out = torch.empty_like(x)
    g = dvm.Graph(ectx)
    g.op("exp", g.input(x), out=out, live=True)
    p = g.flush()
    p.launch_noalloc(stream, ctx=dctx)
    ref = torch.empty_like(x)
    g2 = dvm.Graph(ectx)
    g2.op("exp", g2.input(x), out=ref, live=True)
    g2.flush().launch(stream, ctx=dctx)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # a reduce-all over more tiles than the static array has partial slots
    # (65536) still fits: partials are per workgroup, and the tiling launches
    # at most 4096 workgroups
    say("noalloc_many_tiles")
    big = np.random.default_rng(5).standard_normal((200000, 4096), dtype=np.float32)   # 123077 tiles
    dbig = torch.from_numpy(big).cuda()
    s = torch.full((), 7.0, dtype=torch.float32, device="cuda")
    s2 = torch.full((), 7.0, dtype=torch.float32, device="cuda")
    p = encode_reduce_all(dvm, ectx, dbig, s, "reduce_sum")
    assert p.header()["block_dim"] > 65536 and p.header()["grid"] <= 4096
    p.launch_noalloc(stream, ctx=dctx)
    encode_reduce_all(dvm, ectx, dbig, s2, "reduce_sum").launch(stream, ctx=dctx)
    torch.cuda.synchronize()
    assert float(s.item()) == float(s2.item())
    assert abs(float(s.item()) - float(np.sum(big, dtype=np.float64))) <= O.sum_guard_band(big)
    del big, dbig

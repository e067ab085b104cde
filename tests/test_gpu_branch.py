"""GPU parity of device-side control flow (branch programs) against the
oracle, through the C ABI: if sum(x) > 0 then x + y else x - y (the
if-else-add workload of the DVM review page, section 6.2), with the branch
decided by the VM from the reduce-all's device-resident result, so several
calls queue on one stream with a single host sync at the end.  The branch
outputs are correctly rounded fp32 adds or subtractions: bit-exact.
"""
import numpy as np
import pytest

import workloads as W
from oracle import ops as O
from tests.dvm_helpers import empty_dev, host64, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dvm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import device_bytecode_vm_amd as m
    return m


@pytest.fixture(scope="module")
def ctx(dvm):
    return dvm.Context(0)


def say(*a):
    print("CASE", *a, flush=True)


def queue_if_else(g, dx, dy, s, out, thr=0.0):
    vx, vy = g.input(dx), g.input(dy)
    vs = g.op("reduce_sum", vx, out=s, live=True, axis=0x7FFFFFFF)
    g.begin_branch(vs, thr)
    g.op("add", vx, vy, out=out, live=True)
    g.else_branch()
    g.op("sub", vx, vy, out=out, live=True)
    g.end_branch()


@pytest.mark.parametrize("n", [1, 37, 1000, 4096, 16384])
def test_device_branch_if_else(dvm, ctx, n):
    import torch
    g = dvm.Graph(ctx)
    cases = []
    for i in range(2):
        say("device_branch", n, i)
        x, y, sign = W.ifelse_inputs(n, 7 + i, (n, 4096))
        dx, dy = torch_dev(x, "f32"), torch_dev(y, "f32")
        s = empty_dev((), "f32")
        out = empty_dev(x.shape, "f32")
        queue_if_else(g, dx, dy, s, out)
        cases.append((x, y, s, out))
    torch.cuda.synchronize()                 # one host sync for every call
    for x, y, s, out in cases:
        ref, branch, s64 = O.if_else_add(x, y)
        band = O.sum_guard_band(x)
        assert abs(s64) > band and abs(float(s.item()) - s64) <= band
        assert np.array_equal(host64(out), ref.astype(np.float32).astype(np.float64))


def test_device_branch_stream_of_calls(dvm, ctx):
    """Sixteen calls of the if-else stream queued back to back, each with its
    own output, both branches taken."""
    import torch
    say("device_branch_stream")
    shapes = W.ifelse_shapes(3, 16, nmax=3000)
    g = dvm.Graph(ctx)
    cases = []
    for i, (r, c) in enumerate(shapes):
        x, y, sign = W.ifelse_inputs(3, i, (r, c))
        dx, dy = torch_dev(x, "f32"), torch_dev(y, "f32")
        s = empty_dev((), "f32")
        out = empty_dev((r, c), "f32")
        queue_if_else(g, dx, dy, s, out)
        cases.append((x, y, out, sign))
    torch.cuda.synchronize()
    signs = set()
    for x, y, out, sign in cases:
        ref, branch, _ = O.if_else_add(x, y)
        assert branch == (sign > 0)
        signs.add(branch)
        assert np.array_equal(host64(out), ref.astype(np.float32).astype(np.float64))
    assert signs == {True, False}


def test_device_branch_threshold_and_nan(dvm, ctx):
    """The then-body runs iff cond > threshold, strictly: equal values and
    NaN run the else-body."""
    import torch
    say("device_branch_threshold")
    x = W.normal(np.random.default_rng(5), (33, 1000), 0.5, 1.0)
    y = W.normal(np.random.default_rng(6), (33, 1000), 0.0, 1.0)
    dx, dy = torch_dev(x, "f32"), torch_dev(y, "f32")
    g = dvm.Graph(ctx)
    for cval, thr, take_then in [(1.0, 0.0, True), (0.0, 0.0, False), (2.5, 2.5, False), (-1.0, -2.0, True),
                                 (float("nan"), 0.0, False), (float("inf"), 1e30, True)]:
        cond = torch.full((), cval, dtype=torch.float32, device="cuda")
        out = empty_dev(x.shape, "f32")
        vx, vy = g.input(dx), g.input(dy)
        g.begin_branch(g.input(cond), thr)
        g.op("add", vx, vy, out=out, live=True)
        g.else_branch()
        g.op("sub", vx, vy, out=out, live=True)
        g.end_branch()
        torch.cuda.synchronize()
        ref = (x.astype(np.float64) + y) if take_then else (x.astype(np.float64) - y)
        assert np.array_equal(host64(out), ref.astype(np.float32).astype(np.float64)), (cval, thr)

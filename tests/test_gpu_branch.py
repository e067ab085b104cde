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


def queue_if_else(g, dx, dy, s, out, thr=0.0, fold=False):
    """fold: the branch opens on a reduce-all it issues itself
    (begin_branch_reduce), so the branch program folds the partials."""
    vx, vy = g.input(dx), g.input(dy)
    if fold:
        g.begin_branch_reduce(vx, s, thr)
    else:
        vs = g.op("reduce_sum", vx, out=s, live=True, axis=0x7FFFFFFF)
        g.begin_branch(vs, thr)
    g.op("add", vx, vy, out=out, live=True)
    g.else_branch()
    g.op("sub", vx, vy, out=out, live=True)
    g.end_branch()


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("n", [1, 37, 1000, 4096, 16384])
def test_device_branch_if_else(dvm, ctx, n, fold):
    import torch
    g = dvm.Graph(ctx)
    cases = []
    for i in range(2):
        say("device_branch", n, i, fold)
        x, y, sign = W.ifelse_inputs(n, 7 + i, (n, 4096))
        dx, dy = torch_dev(x, "f32"), torch_dev(y, "f32")
        s = empty_dev((), "f32")
        out = empty_dev(x.shape, "f32")
        queue_if_else(g, dx, dy, s, out, fold=fold)
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
        queue_if_else(g, dx, dy, s, out, fold=i % 2 == 1)
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


def _sum_by_combine(g, dx):
    """The reduce-all's scalar through its own combine launch (no branch)."""
    import torch
    s = empty_dev((), "f32")
    g.op("reduce_sum", g.input(dx), out=s, live=True, axis=0x7FFFFFFF)
    g.sync()
    return s.cpu().view(torch.int32).item()


@pytest.mark.parametrize("n", [1, 1000, 16384])
def test_folded_condition_equals_combine(dvm, ctx, n):
    """A branch opened on a reduce-all it issues (begin_branch_reduce) folds the
    workgroups' partials itself (the combine launch is left out): the scalar it
    writes and the body it picks equal those of the reduce-all's own combine,
    bit for bit."""
    import torch
    say("folded_condition", n)
    x, y, sign = W.ifelse_inputs(n, 21, (n, 4096))
    dx, dy = torch_dev(x, "f32"), torch_dev(y, "f32")
    g = dvm.Graph(ctx)
    bits = _sum_by_combine(g, dx)
    s = empty_dev((), "f32")
    out = empty_dev(x.shape, "f32")
    queue_if_else(g, dx, dy, s, out, fold=True)
    g.sync()
    assert s.cpu().view(torch.int32).item() == bits
    ref, branch, _ = O.if_else_add(x, y)
    assert np.array_equal(host64(out), ref.astype(np.float32).astype(np.float64))


def test_branch_body_reading_its_condition(dvm, ctx):
    """A body that reads the condition keeps the combine launch (the branch
    program would otherwise write the scalar while its tiles read it)."""
    import torch
    say("branch_reads_condition")
    x, y, sign = W.ifelse_inputs(2000, 4, (2000, 1024))
    dx, dy = torch_dev(x, "f32"), torch_dev(y, "f32")
    g = dvm.Graph(ctx)
    bits = _sum_by_combine(g, dx)
    s = empty_dev((), "f32")
    out = empty_dev(x.shape, "f32")
    vx, vy = g.input(dx), g.input(dy)
    vs = g.begin_branch_reduce(vx, s, 0.0)
    g.op("sub", vx, vs, out=out, live=True)
    g.else_branch()
    g.op("add", vx, vs, out=out, live=True)
    g.end_branch()
    g.sync()
    sv = s.cpu()
    assert sv.view(torch.int32).item() == bits
    s32 = np.float32(sv.item())
    ref = (x - s32) if s32 > 0 else (x + s32)
    assert np.array_equal(host64(out), ref.astype(np.float32).astype(np.float64))


def test_other_graph_between_branch_open_and_close(dvm, ctx):
    """A second graph on the same stream runs a reduce-all (rewriting the
    stream's partials) and reads the first graph's condition while that graph's
    branch is open: the held combine runs before it, so both graphs see the
    condition's true value and the branch still picks the right body."""
    import torch
    say("other_graph_inside_branch")
    x, y, sign = W.ifelse_inputs(3000, 9, (3000, 2048))
    z, _, _ = W.ifelse_inputs(700, 10, (700, 512))
    dx, dy, dz = torch_dev(x, "f32"), torch_dev(y, "f32"), torch_dev(z, "f32")
    ga, gb = dvm.Graph(ctx), dvm.Graph(ctx)
    bits = _sum_by_combine(ga, dx)
    zbits = _sum_by_combine(gb, dz)
    s = empty_dev((), "f32")
    sz = empty_dev((), "f32")
    t = empty_dev((), "f32")
    out = empty_dev(x.shape, "f32")
    vx, vy = ga.input(dx), ga.input(dy)
    ga.begin_branch_reduce(vx, s, 0.0)
    gb.op("reduce_sum", gb.input(dz), out=sz, live=True, axis=0x7FFFFFFF)
    gb.op("add", gb.input(s), gb.input(s), out=t, live=True)   # reads the held condition
    gb.flush_launch()
    ga.op("add", vx, vy, out=out, live=True)
    ga.else_branch()
    ga.op("sub", vx, vy, out=out, live=True)
    ga.end_branch()
    ga.sync()
    gb.sync()
    assert s.cpu().view(torch.int32).item() == bits
    assert sz.cpu().view(torch.int32).item() == zbits
    sv = np.float32(s.cpu().item())
    assert np.float32(t.cpu().item()) == np.float32(sv + sv)
    ref, branch, _ = O.if_else_add(x, y)
    assert np.array_equal(host64(out), ref.astype(np.float32).astype(np.float64))


def test_folded_branches_on_two_streams(dvm, ctx):
    """Two graphs on two streams open their branches on reduce-alls they
    issue before either closes: each stream holds its own combine and each
    branch program folds its own reduce-all's partials (each stream has its
    own scratch), so both scalars equal their combine's and both bodies are
    right."""
    import torch
    say("folded_two_streams")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ins = [W.ifelse_inputs(n, 30 + n % 7, (n, 4096)) for n in (2500, 7000)]
    devs = [(torch_dev(x, "f32"), torch_dev(y, "f32")) for x, y, _ in ins]
    g0 = dvm.Graph(ctx)
    bits = [_sum_by_combine(g0, dx) for dx, _ in devs]
    ss = [empty_dev((), "f32") for _ in ins]
    outs = [empty_dev(x.shape, "f32") for x, _, _ in ins]
    torch.cuda.synchronize()
    gs = [dvm.Graph(ctx, sa), dvm.Graph(ctx, sb)]
    vals = []
    for g, (dx, dy), s in zip(gs, devs, ss):
        vx, vy = g.input(dx), g.input(dy)
        g.begin_branch_reduce(vx, s, 0.0)
        vals.append((vx, vy))
    for g, (vx, vy), o in zip(gs, vals, outs):
        g.op("add", vx, vy, out=o, live=True)
        g.else_branch()
        g.op("sub", vx, vy, out=o, live=True)
        g.end_branch()
    torch.cuda.synchronize()
    for (x, y, _), s, o, b in zip(ins, ss, outs, bits):
        assert s.cpu().view(torch.int32).item() == b
        ref, _, _ = O.if_else_add(x, y)
        assert np.array_equal(host64(o), ref.astype(np.float32).astype(np.float64))


def test_open_branch_dropped_with_its_graph(dvm, ctx):
    """A graph destroyed with its branch open (on a reduce-all it issued)
    launches the held combine, so the scalar still lands."""
    import torch
    say("open_branch_destroyed")
    x, y, _ = W.ifelse_inputs(1500, 12, (1500, 4096))
    dx = torch_dev(x, "f32")
    g0 = dvm.Graph(ctx)
    bits = _sum_by_combine(g0, dx)
    s = empty_dev((), "f32")
    g = dvm.Graph(ctx)
    g.begin_branch_reduce(g.input(dx), s, 0.0)
    g.close()
    torch.cuda.synchronize()
    assert s.cpu().view(torch.int32).item() == bits

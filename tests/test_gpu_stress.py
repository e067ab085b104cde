"""Race-stress runs: representative programs launched through
dvm_launch_stress (the profiling twin with seeded, per-wave delays before
every dispatch) must store bit-identical results to a normal launch.  The
programs cover every place the encoder inserts a barrier or the VM relies on
an ordering: cross-wave row reductions (one, nine and seventeen per tile,
the buffers wrapping), the reduce-all's partials and last-workgroup combine,
LDS staging of invariant and prefetched operands, a prefetched operand read
twice, the wide build and a branch program.
"""
import numpy as np
import pytest

import workloads as W
from tests.dvm_helpers import empty_dev

pytestmark = pytest.mark.gpu
SEEDS = (1, 77, 4093)


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


def layernorm(dvm, ctx, rows, cols):
    from device_bytecode_vm_amd import composites as CP
    x = W.device_normal((rows, cols), seed=rows + cols, dtype="bf16")
    gam = W.device_normal((cols,), seed=1, mu=1.0, sd=0.1)
    bet = W.device_normal((cols,), seed=2, sd=0.1)
    out = empty_dev((rows, cols), "bf16")
    g = dvm.Graph(ctx)
    CP.layer_norm(g, g.input(x), g.input(gam), g.input(bet), W.LN_EPS, out=out)
    return g.flush(), [out]


def chained(dvm, ctx, n_red):
    x = W.device_normal((4096, 6000), seed=n_red)
    out = empty_dev((4096, 6000), "f32")
    g = dvm.Graph(ctx)
    v = g.input(x)
    for k in range(n_red):
        s = g.op("reduce_sum", v)
        m = g.op("mul", s, 1.0 / 6000)
        last = k == n_red - 1
        nv = g.op("add", v, m, out=out if last else None, live=last)
        g.release(s, m)
        if k:
            g.release(v)
        v = nv
    return g.flush(), [out]


def softmax(dvm, ctx):
    from device_bytecode_vm_amd import composites as CP
    x = W.device_normal((40 * 300, 6484), seed=9, dtype="bf16")
    out = empty_dev(x.shape, "bf16")
    g = dvm.Graph(ctx)
    CP.softmax(g, g.input(x), out=out)
    return g.flush(), [out]


def reduce_all(dvm, ctx):
    x = W.device_normal((16384, 4096), seed=5)
    s = empty_dev((), "f32")
    e = dvm.Context(-1)
    g = dvm.Graph(e)
    g.op("reduce_sum", g.input(x), out=s, live=True, axis=0x7FFFFFFF)
    p = g.take_program()
    p.ctx = ctx
    return p, [s]


def branch(dvm, ctx):
    x = W.device_normal((3000, 4096), seed=6, mu=0.1)
    y = W.device_normal((3000, 4096), seed=7)
    c = W.device_normal((), seed=8)
    out = empty_dev((3000, 4096), "f32")
    e = dvm.Context(-1)
    g = dvm.Graph(e)
    vx, vy = g.input(x), g.input(y)
    g.begin_branch(g.input(c), 0.0)
    g.op("add", vx, vy, out=out, live=True)
    g.else_branch()
    g.op("sub", vx, vy, out=out, live=True)
    g.end_branch()
    p = g.take_program()
    p.ctx = ctx
    return p, [out]


def prefetch_reuse(dvm, ctx):
    x = W.device_normal((4096, 5120), seed=10)
    out = empty_dev((4096, 5120), "f32")
    g = dvm.Graph(ctx)
    vx = g.input(x)
    a = g.op("sub", vx, vx)
    b = g.op("sub", vx, a)
    c = g.op("mul", b, b)
    g.op("add", c, c, out=out, live=True)
    g.release(a, b, c)
    return g.flush(), [out]


def swiglu(dvm, ctx):
    from device_bytecode_vm_amd import composites as CP
    a = W.device_normal((3487, 17408), seed=11, dtype="bf16")
    b = W.device_normal((3487, 17408), seed=12, dtype="bf16")
    out = empty_dev((3487, 17408), "bf16")
    g = dvm.Graph(ctx)
    CP.swiglu(g, g.input(a), g.input(b), out=out)
    return g.flush(), [out]


CASES = {
    "layernorm_wide_20000x5120": lambda d, c: layernorm(d, c, 20000, 5120),
    "layernorm_cross_wave_3000x8192": lambda d, c: layernorm(d, c, 3000, 8192),
    "layernorm_standard_37x5120": lambda d, c: layernorm(d, c, 37, 5120),
    "chained_1": lambda d, c: chained(d, c, 1),
    "chained_9": lambda d, c: chained(d, c, 9),
    "chained_17": lambda d, c: chained(d, c, 17),
    "softmax_12000x6484": softmax,
    "reduce_all_16384x4096": reduce_all,
    "branch_3000x4096": branch,
    "prefetch_reuse": prefetch_reuse,
    "swiglu_3487x17408": swiglu,
}


@pytest.mark.parametrize("name", list(CASES))
def test_stress_bit_identical(dvm, ctx, name):
    import torch
    print("CASE stress", name, flush=True)
    p, outs = CASES[name](dvm, ctx)
    assert p.verify() is None
    p.launch()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    counters = torch.zeros(p.PROF_COUNTERS * max(p.header()["grid"], 1), dtype=torch.int64, device="cuda")
    for seed in SEEDS:
        for o in outs:
            o.fill_(float("nan"))
        p.launch_stress(seed, counters)
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(-1).view(torch.uint8), r.view(-1).view(torch.uint8)), (name, seed)

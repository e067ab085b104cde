"""GPU parity of the wide VM variant (one tile register of 10 chunks per lane).

The encoder runs a row-reduction program on the wide VM when every tile value
stays in the accumulator and either no standard tile fits its rows (rows of
10241 to 20480 columns) or a wide tile holds more rows than a standard one
with the same LDS staging.
These cases check that choice from the header and the results against the
oracle: softmax and RMSNorm over long rows (bf16 within 2 ulp, fp32 within
1e-5 of the largest value), ragged row ends bit for bit under the oracle's
fp32 emulation, and the profiling launch on the wide kernel.
"""
import numpy as np
import pytest

import workloads as W
from oracle import numerics as N
from oracle import ops as O
from oracle.graph import evaluate
from tests.dvm_helpers import empty_dev, host64, torch_dev

pytestmark = pytest.mark.gpu

WIDE = 2


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


# (rows, cols, kernel type for bf16 / fp32 input): a few rows of 6484 stay on
# the standard VM (the cost model puts one row in a tile on either variant);
# rows of 6484-8192 take the wide VM in both dtypes (a prefetch slot holds the
# tile's nv chunks: 7-8 chunks of fp32 per lane fit next to the reduction
# buffers); rows of 10241 and more fit only the wide VM
@pytest.mark.parametrize("rows,cols,kts", [(3, 6484, (0, 0)), (3000, 6484, (WIDE, WIDE)), (3000, 8192, (WIDE, WIDE)),
                                           (64, 10241, (WIDE, WIDE)), (40, 16384, (WIDE, WIDE)),
                                           (7, 20480, (WIDE, WIDE)), (3000, 6485, (WIDE, WIDE)),
                                           (3000, 6487, (WIDE, WIDE)), (9, 12345, (WIDE, WIDE))])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_wide_softmax(dvm, ctx, rows, cols, kts, dt):
    kt = kts[0] if dt == "bf16" else kts[1]
    import torch
    from device_bytecode_vm_amd import composites as CP
    print("CASE wide softmax", rows, cols, dt, flush=True)
    x = W.normal(np.random.default_rng(rows + cols), (rows, cols), 0, 1, dt)
    dx = torch_dev(x, dt)
    out = empty_dev(x.shape, dt)
    g = dvm.Graph(ctx)
    CP.softmax(g, g.input(dx), out=out)
    p = g.flush()
    assert p.header()["kernel_type"] == kt
    p.launch()
    torch.cuda.synchronize()
    ref = O.softmax(x)
    if dt == "bf16":
        ok, d = N.check_bf16(host64(out), ref)
        assert ok, f"max ulp {d}"
    else:
        err = np.max(np.abs(host64(out) - ref)) / np.max(np.abs(ref))
        assert err <= 1e-5, err


@pytest.mark.parametrize("rows,h", [(2000, 12000), (33, 12000)])
def test_wide_rmsnorm(dvm, ctx, rows, h):
    import torch
    from device_bytecode_vm_amd import composites as CP
    print("CASE wide rmsnorm", rows, h, flush=True)
    rg = np.random.default_rng(rows * 3 + h)
    x = W.normal(rg, (rows, h), 0, 1, "bf16")
    w = W.normal(rg, (h,), 1, 0.1)
    out = empty_dev((rows, h), "bf16")
    g = dvm.Graph(ctx)
    CP.rms_norm(g, g.input(torch_dev(x, "bf16")), g.input(torch_dev(w, "f32")), W.RMS_EPS, out=out)
    p = g.flush()
    assert p.header()["kernel_type"] == WIDE
    p.launch()
    torch.cuda.synchronize()
    ok, d = N.check_bf16(host64(out), O.rms_norm(x, w, W.RMS_EPS))
    assert ok, f"max ulp {d}"


@pytest.mark.parametrize("rem", range(1, 8))
@pytest.mark.parametrize("rows", [3000, 6000])
def test_wide_ragged_exact(dvm, ctx, rem, rows):
    """(x - rowmax(x)) * 2 to fp32 and bf16 over rows of 8 * 811 + rem
    columns: every remainder of the row-end chunk on the wide VM."""
    import torch
    C = 8 * 811 + rem
    print("CASE wide ragged", rem, rows, C, flush=True)
    x = W.normal(np.random.default_rng(rem * 31 + rows), (rows, C), 0, 2, "bf16")
    y32, y16 = empty_dev((rows, C), "f32"), empty_dev((rows, C), "bf16")
    g = dvm.Graph(ctx)
    with g.group():
        xf = g.op("cast", g.input(torch_dev(x, "bf16")), dtype="f32")
        m = g.op("reduce_max", xf)
        d = g.op("sub", xf, m)
        y = g.op("mul", d, 2.0, out=y32, live=True)
        g.op("cast", y, out=y16, dtype="bf16", live=True)
        g.release(xf, m, d)
    p = g.flush()
    assert p.header()["kernel_type"] == WIDE
    p.launch()
    torch.cuda.synchronize()
    ops = [{"op": "reduce_max", "in": ["x"], "out": "m", "dtype": "f32", "axis": -1},
           {"op": "sub", "in": ["x", "m"], "out": "d", "dtype": "f32"},
           {"op": "mul", "in": ["d", 2.0], "out": "y", "dtype": "f32"},
           {"op": "cast", "in": ["y"], "out": "yb", "dtype": "bf16"}]
    ref, _ = evaluate(ops, {"x": x}, emulate_f32=True)
    assert np.array_equal(host64(y32), ref["y"])
    assert np.array_equal(host64(y16), ref["yb"])


def test_wide_profiled_launch(dvm, ctx):
    import torch
    from device_bytecode_vm_amd import composites as CP
    rows, cols = 3000, 6484
    print("CASE wide profiled", rows, cols, flush=True)
    x = torch_dev(W.normal(np.random.default_rng(5), (rows, cols), 0, 1, "bf16"), "bf16")
    y1, y2 = empty_dev((rows, cols), "bf16"), empty_dev((rows, cols), "bf16")
    progs = []
    for y in (y1, y2):
        g = dvm.Graph(ctx)
        CP.softmax(g, g.input(x), out=y)
        progs.append(g.flush())
    h = progs[1].header()
    assert h["kernel_type"] == WIDE
    c = torch.zeros(progs[1].PROF_COUNTERS * h["grid"], dtype=torch.int64, device="cuda")
    progs[0].launch()
    progs[1].launch_profiled(c)
    torch.cuda.synchronize()
    assert np.array_equal(host64(y1), host64(y2))
    cnt = c.view(-1, progs[1].PROF_COUNTERS).cpu().numpy()
    assert (cnt[:, 1] > 0).all() and (cnt[:, 1] + cnt[:, 2] + cnt[:, 3] <= cnt[:, 0]).all()

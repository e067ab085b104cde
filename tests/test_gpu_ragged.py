"""GPU parity at ragged row ends.

Rows whose length is not a multiple of the VM's 8-element chunk leave one
partial chunk per row.  The VM reads that chunk whole when its bytes lie
inside the operand's extent (the values past the row's end are never used)
and element by element otherwise (the tensor's last row), reduces it with a
per-element mask, and stores it in pieces of four, two and one elements.
These cases take every remainder 1..7, dense rows and rows that are views
into a wider buffer (a gap between rows), fp32 and bf16 inputs, one tile
(direct loads) and several tiles per workgroup (loads prefetched into LDS),
lane groups inside one wave and across waves, and
write fp32, bf16 and u8 outputs from one program.  The arithmetic is exact in
fp32 (a row max, one subtraction, a doubling; isfinite), so the oracle's fp32
emulation is matched bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from oracle.graph import evaluate
from tests.dvm_helpers import empty_dev, host64

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


def _specials(rg, shape):
    z = W.normal(rg, shape, 0, 1)
    flat = z.reshape(-1)
    for i, v in enumerate([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-30]):
        flat[(i * 7919 + 13) % flat.size] = v
    return z


def _device(arr, dtype, gap):
    """arr [R, C] on the GPU as `dtype`; with a gap, a view of the first C
    columns of a [R, C + gap] buffer whose other columns hold garbage."""
    import torch
    td = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    R, C = arr.shape
    base = torch.full((R, C + gap), 7168.0, dtype=torch.float32)
    base[:, :C] = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    base = base.to(td).cuda()
    return base, base[:, :C]


# (rows, whole chunks per row, tiles per workgroup at least): one tile of one
# row over 256 lanes (direct loads); tens of rows of 4 or 8 lanes per tile
# (the wide or the standard build, by remainder) and 2 rows of 128 lanes per
# tile (reduction across waves), all with prefetched loads
SHAPES = [(3, 37, 1), (50000, 37, 2), (5000, 400, 2)]


@pytest.mark.parametrize("rem", range(1, 8))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{8 * s[1]}")
@pytest.mark.parametrize("gap", [0, 5])
@pytest.mark.parametrize("in_dt", ["f32", "bf16"])
def test_ragged_row_end(dvm, ctx, rem, shape, gap, in_dt):
    import torch
    rows, chunks, min_body = shape
    C = 8 * chunks + rem
    print("CASE ragged", rem, rows, C, gap, in_dt, flush=True)
    rg = np.random.default_rng(100 * rem + rows + gap)
    x = W.normal(rg, (rows, C), 0, 2, in_dt)
    z = _specials(rg, (rows, C))
    bx, dx = _device(x, in_dt, gap)
    bz, dz = _device(z, "f32", gap)
    y32, y16, fin = empty_dev((rows, C), "f32"), empty_dev((rows, C), "bf16"), empty_dev((rows, C), "u8")
    g = dvm.Graph(ctx)
    with g.group():
        vx = g.input(dx)
        xf = g.op("cast", vx, dtype="f32") if in_dt == "bf16" else vx
        m = g.op("reduce_max", xf)
        d = g.op("sub", xf, m)
        y = g.op("mul", d, 2.0, out=y32, live=True)
        g.op("cast", y, out=y16, dtype="bf16", live=True)
        g.op("isfinite", g.input(dz), out=fin, live=True)
        g.release(m, d, *([xf] if in_dt == "bf16" else []))
    p = g.flush()
    p.launch()
    torch.cuda.synchronize()
    assert p.header()["body_tile"] >= min_body
    ops = [{"op": "reduce_max", "in": ["x"], "out": "m", "dtype": "f32", "axis": -1},
           {"op": "sub", "in": ["x", "m"], "out": "d", "dtype": "f32"},
           {"op": "mul", "in": ["d", 2.0], "out": "y", "dtype": "f32"},
           {"op": "cast", "in": ["y"], "out": "yb", "dtype": "bf16"},
           {"op": "isfinite", "in": ["z"], "out": "f", "dtype": "u8"}]
    ref, _ = evaluate(ops, {"x": x, "z": z}, emulate_f32=True)
    assert np.array_equal(host64(y32), ref["y"])
    assert np.array_equal(host64(y16), ref["yb"])
    assert np.array_equal(host64(fin), ref["f"])
    # the gap columns of the inputs are untouched
    if gap:
        assert torch.all(bx[:, C:].float() == 7168.0).item()

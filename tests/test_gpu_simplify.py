"""GPU parity of graphs the encoder's clean-up rewrites (exact identities,
same-dtype casts nobody stores, dead ops): the stored values equal the
oracle's evaluation of the graph as written, bit for bit under its fp32
emulation, with signed zeros, infinities and NaNs among the inputs."""
import numpy as np
import pytest

import workloads as W
from oracle.graph import evaluate
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


def _with_specials(rg, shape):
    x = W.normal(rg, shape, 0, 3)
    flat = x.reshape(-1)
    for i, v in enumerate([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-40, -1e-40, 3e38]):
        flat[(i * 7919 + 5) % flat.size] = v
    return x


def _same_bits(dev, ref, dt):
    got = host64(dev)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    assert np.array_equal(np.signbit(got[m]), np.signbit(ref[m])), f"signed zeros differ ({dt})"


@pytest.mark.parametrize("rows,cols", [(1, 1), (7, 333), (3000, 1000)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rewritten_graph_matches_oracle(dvm, ctx, rows, cols, dt):
    import torch
    print("CASE simplify", rows, cols, dt, flush=True)
    rg = np.random.default_rng(rows * 7 + cols)
    x = _with_specials(rg, (rows, cols))
    if dt == "bf16":
        from oracle.numerics import round_to
        x = round_to(x, "bf16")
    else:
        from oracle.numerics import round_f32
        x = round_f32(x)
    shape = (rows, cols)
    y_copy, y_neg, y_plus0, y_row = (empty_dev(shape, "f32"), empty_dev(shape, dt), empty_dev(shape, "f32"),
                                     empty_dev(shape, "f32"))
    g = dvm.Graph(ctx)
    with g.group():
        vx = g.input(torch_dev(x, dt))
        a = g.op("mul", vx, 1.0, out=y_copy, dtype="f32", live=True)     # stored: a copy to fp32
        b = g.op("div", a, 1.0)
        c = g.op("sub", b, 0.0)
        d = g.op("add", -0.0, c)
        e = g.op("cast", d, dtype="f32")
        g.op("neg", e, out=y_neg, live=True)
        g.op("add", e, 0.0, out=y_plus0, live=True)                   # -0 + 0 = +0: kept
        dead = g.op("reduce_max", e)
        dead2 = g.op("mul", dead, 2.0)
        g.op("mul", 1.0, e, out=y_row, live=True)
        g.release(b, c, d, e, dead, dead2)
    p = g.flush()
    assert p.header()["tmpl"] == 0, "the dead row reduction was not dropped"
    p.launch()
    torch.cuda.synchronize()
    ops = [{"op": "mul", "in": ["x", 1.0], "out": "a", "dtype": "f32"},
           {"op": "div", "in": ["a", 1.0], "out": "b", "dtype": "f32"},
           {"op": "sub", "in": ["b", 0.0], "out": "c", "dtype": "f32"},
           {"op": "add", "in": [-0.0, "c"], "out": "d", "dtype": "f32"},
           {"op": "cast", "in": ["d"], "out": "e", "dtype": "f32"},
           {"op": "neg", "in": ["e"], "out": "n", "dtype": dt},
           {"op": "add", "in": ["e", 0.0], "out": "p", "dtype": "f32"},
           {"op": "reduce_max", "in": ["e"], "out": "m", "dtype": "f32", "axis": -1},
           {"op": "mul", "in": ["m", 2.0], "out": "m2", "dtype": "f32"},
           {"op": "mul", "in": [1.0, "e"], "out": "r", "dtype": "f32"}]
    ref, _ = evaluate(ops, {"x": x}, emulate_f32=True)
    _same_bits(y_copy, ref["a"], dt)
    _same_bits(y_neg, ref["n"], dt)
    _same_bits(y_plus0, ref["p"], dt)
    _same_bits(y_row, ref["r"], dt)
    # where x is -0: a = x keeps the sign, x + 0 does not
    z = (x == 0) & np.signbit(x)
    if z.any():
        assert np.signbit(host64(y_copy)[z]).all() and not np.signbit(host64(y_plus0)[z]).any()

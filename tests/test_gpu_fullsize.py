"""GPU parity at the workloads' full sizes, through the C ABI.

* if-else-add at N = 4096, 11000 and 16384 rows of 4096: the reduce-all then
  runs several tiles per workgroup with the LDS prefetch and thousands of
  partials (DVM review page, section 6.2, Figure 13);
* the transformer op stream's motifs at T = 3487, T_kv = 6484 (the sizes
  the stream draws for seed 0): add + RMSNorm fused, SwiGLU over [T, 17408]
  and softmax over [40, T, T_kv], checked on seeded sampled rows (each output
  row depends only on its input row, so a row sample is an exact check of
  those rows);
* chains of 9 and 17 cross-wave row reductions with several tiles per
  workgroup (the cross-wave reduction buffers wrap around);
* reduce-alls queued on two streams at once (each stream has its own scratch).

Large inputs are drawn on the device (torch generator); the oracle reads D2H
copies of the exact device inputs.  Every case prints its name first.
"""
import numpy as np
import pytest

import workloads as W
from oracle import numerics as N
from oracle import ops as O
from oracle import tiling as TL
from oracle.graph import evaluate
from tests.dvm_helpers import empty_dev, host64, torch_dev

pytestmark = pytest.mark.gpu

T_STREAM, TKV_STREAM = 3487, 6484


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


def sample_rows(n, k, seed):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], g.integers(0, n, k)]))


def test_stream_draw_sizes():
    t, tkv, _ = W.stream_step(0, 10)
    assert (t, tkv) == (T_STREAM, TKV_STREAM)


@pytest.mark.parametrize("n", [4096, 11000, 16384])
def test_if_else_add_full_size(dvm, ctx, n):
    C = 4096
    # the reduce-all's geometry at this size: several tiles per workgroup
    col = TL.collapse(TL.ALLREDUCE, (n, C), [(C, 1)])
    plan = TL.plan(TL.ALLREDUCE, col[0], col[1], [TL.Operand(4, s_r, s_c, 0) for s_r, s_c in col[2]])
    assert plan.body_tile > 1 and plan.block_dim >= 2048, (plan.body_tile, plan.block_dim)
    for i in range(2):
        say("if_else_add_full", n, i)
        x, y, sign = W.ifelse_inputs(n, i, (n, C))
        dx, dy = torch_dev(x, "f32"), torch_dev(y, "f32")
        s = empty_dev((), "f32")
        g = dvm.Graph(ctx)
        vx, vy = g.input(dx), g.input(dy)
        g.op("reduce_sum", vx, out=s, live=True, axis=0x7FFFFFFF)
        g.sync()
        sv = float(s.item())
        out = empty_dev(x.shape, "f32")
        g.op("add" if sv > 0 else "sub", vx, vy, out=out, live=True)
        g.sync()
        ref, branch, s64 = O.if_else_add(x, y)
        band = O.sum_guard_band(x)
        assert abs(s64) > band
        assert abs(sv - s64) <= band, (sv, s64, band)
        assert (sv > 0) == branch == (sign > 0)
        assert np.array_equal(host64(out), ref.astype(np.float32).astype(np.float64))


def test_add_rmsnorm_stream_size(dvm, ctx):
    import torch
    from device_bytecode_vm_amd import composites as CP
    T, H = T_STREAM, W.H_LN
    say("add_rmsnorm_full", T)
    d0 = W.device_normal((T, H), seed=20, dtype="bf16")
    dr = W.device_normal((T, H), seed=21, dtype="bf16")
    dw = W.device_normal((H,), seed=25, mu=1.0, sd=0.1)
    h1 = empty_dev((T, H), "bf16")
    n = empty_dev((T, H), "bf16")
    g = dvm.Graph(ctx)
    vh = g.op("add", g.input(d0), g.input(dr), out=h1)
    CP.rms_norm(g, vh, g.input(dw), W.RMS_EPS, out=n)
    p = g.flush()
    hd = p.header()
    assert hd["body_tile"] > 1, hd
    p.launch()
    torch.cuda.synchronize()
    idx = sample_rows(T, 256, 5)
    h0, r0 = host64(d0[idx]), host64(dr[idx])
    h1_ref = N.round_bf16(h0 + r0)
    assert np.array_equal(host64(h1[idx]), h1_ref)
    ok, d = N.check_bf16(host64(n[idx]), O.rms_norm(h1_ref, host64(dw), W.RMS_EPS))
    assert ok, f"max ulp {d}"


def test_swiglu_stream_size(dvm, ctx):
    import torch
    from device_bytecode_vm_amd import composites as CP
    T, F = T_STREAM, W.N_FFN
    say("swiglu_full", T, F)
    gt = W.device_normal((T, F), seed=26, dtype="bf16")
    up = W.device_normal((T, F), seed=28, dtype="bf16")
    out = empty_dev((T, F), "bf16")
    g = dvm.Graph(ctx)
    CP.swiglu(g, g.input(gt), g.input(up), out=out)
    p = g.flush()
    hd = p.header()
    assert hd["body_tile"] > 1, hd
    p.launch()
    torch.cuda.synchronize()
    idx = sample_rows(T, 128, 6)
    ok, d = N.check_bf16(host64(out[idx]), O.swiglu(host64(gt[idx]), host64(up[idx])))
    assert ok, f"max ulp {d}"


def test_softmax_stream_size(dvm, ctx):
    import torch
    from device_bytecode_vm_amd import composites as CP
    T, TKV, NH = T_STREAM, TKV_STREAM, W.HEADS
    say("softmax_full", NH, T, TKV)
    s = W.device_normal((NH, T, TKV), seed=30, dtype="bf16")
    out = empty_dev((NH, T, TKV), "bf16")
    g = dvm.Graph(ctx)
    CP.softmax(g, g.input(s), out=out)
    p = g.flush()
    hd = p.header()
    assert hd["body_tile"] > 1 and hd["R"] == NH * T and hd["C"] == TKV, hd
    p.launch()
    torch.cuda.synchronize()
    s2, o2 = s.view(NH * T, TKV), out.view(NH * T, TKV)
    idx = sample_rows(NH * T, 256, 7)
    ok, d = N.check_bf16(host64(o2[idx]), O.softmax(host64(s2[idx])))
    assert ok, f"max ulp {d}"
    del s, out


def _chain_ops(n_red, cols):
    """v <- v + rowsum(v) / cols, n_red times: every step's row sum is
    non-trivial (it doubles the row mean), so a wrong partial shows."""
    ops, v = [], "x"
    for k in range(n_red):
        ops.append({"op": "reduce_sum", "in": [v], "out": f"s{k}", "dtype": "f32", "axis": -1})
        ops.append({"op": "mul", "in": [f"s{k}", 1.0 / cols], "out": f"m{k}", "dtype": "f32"})
        ops.append({"op": "add", "in": [v, f"m{k}"], "out": f"v{k}", "dtype": "f32"})
        v = f"v{k}"
    return ops, v


@pytest.mark.parametrize("n_red,shape", [(9, (4096, 6000)), (17, (4096, 6000)), (9, (1024, 16384))])
def test_chained_cross_wave_reductions(dvm, ctx, n_red, shape):
    say("chained_reductions", n_red, shape)
    rg = np.random.default_rng(n_red)
    x = (rg.normal(0, 1, shape) + rg.normal(0, 4, (shape[0], 1))).astype(np.float32)
    dx = torch_dev(x, "f32")
    out = empty_dev(shape, "f32")
    g = dvm.Graph(ctx)
    v = g.input(dx)
    for k in range(n_red):
        s = g.op("reduce_sum", v)
        m = g.op("mul", s, 1.0 / shape[1])
        last = k == n_red - 1
        nv = g.op("add", v, m, out=out if last else None, live=last)
        g.release(s, m)
        if k:
            g.release(v)
        v = nv
    p = g.flush()
    hd = p.header()
    assert hd["body_tile"] > 1 and hd["g"] > 64, hd
    p.launch()
    import torch
    torch.cuda.synchronize()
    ops, last = _chain_ops(n_red, shape[1])
    ref, _ = evaluate(ops, {"x": x})
    ok, err = N.check_f32(host64(out), ref[last])
    assert ok, f"relative error {err}"


def test_reduce_all_on_two_streams(dvm, ctx):
    """Reduce-alls queued on two streams with no host sync between them: each
    stream's launches use that stream's scratch, so the sums stay exact."""
    import torch
    say("reduce_all_two_streams")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    xs = [W.device_normal((3000 + 7 * i, 4096), seed=40 + i) for i in range(8)]
    outs = [torch.empty((), dtype=torch.float32, device="cuda") for _ in xs]
    torch.cuda.synchronize()
    ga, gb = dvm.Graph(ctx, sa), dvm.Graph(ctx, sb)
    for rep in range(4):
        for i, (x, o) in enumerate(zip(xs, outs)):
            g = ga if i % 2 == 0 else gb
            g.op("reduce_sum", g.input(x), out=o, live=True, axis=0x7FFFFFFF)
    torch.cuda.synchronize()
    for x, o in zip(xs, outs):
        xh = host64(x)
        band = O.sum_guard_band(xh)
        assert abs(float(o.item()) - float(np.sum(xh))) <= band


def test_prefetched_operand_read_twice(dvm, ctx):
    """x is staged in a prefetch slot and read twice per tile (a = x - x,
    b = x - a) with four tiles per workgroup: both reads must see this
    tile's x (the slot is refilled for the next tile only by its last read).
    Correctly rounded ops: bit-exact against the fp32-emulating oracle."""
    import torch
    say("prefetch_reuse")
    x = W.normal(np.random.default_rng(8), (4096, 5120), 0, 1)
    out = empty_dev(x.shape, "f32")
    g = dvm.Graph(ctx)
    vx = g.input(torch_dev(x, "f32"))
    a = g.op("sub", vx, vx)
    b = g.op("sub", vx, a)
    c = g.op("mul", b, b)
    g.op("add", c, c, out=out, live=True)
    g.release(a, b, c)
    p = g.flush()
    assert p.header()["body_tile"] > 1
    assert p.verify() is None
    p.launch()
    torch.cuda.synchronize()
    ref, _ = evaluate([{"op": "sub", "in": ["x", "x"], "out": "a", "dtype": "f32"},
                       {"op": "sub", "in": ["x", "a"], "out": "b", "dtype": "f32"},
                       {"op": "mul", "in": ["b", "b"], "out": "c", "dtype": "f32"},
                       {"op": "add", "in": ["c", "c"], "out": "o", "dtype": "f32"}], {"x": x}, emulate_f32=True)
    assert np.array_equal(host64(out), ref["o"])

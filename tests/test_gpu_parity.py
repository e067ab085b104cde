"""GPU parity of the VM against the oracle, through the C ABI.

Every case prints its name before it launches anything, so a failing run
names the case.  Sizes span several tiles and ragged tails; tolerances:
fp32 max|d|/max|ref| <= 1e-5, bf16 <= 2 ulp (floored), predicted-bit-exact
chains (sqrt(a + b), the if-else branch) compared bit for bit, tiling and
tile maps compared exactly.
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


def test_sqrt_add_bit_exact(dvm, ctx):
    import torch
    for shape in [(513, 1031), (1, 1), (1, 7), (3, 5), (64, 4096)]:
        say("sqrt_add", shape)
        a, b = W.vv_sqrt_add(0, shape)
        da, db = torch_dev(a, "f32"), torch_dev(b, "f32")
        out = empty_dev(shape, "f32")
        g = dvm.Graph(ctx)
        va, vb = g.input(da), g.input(db)
        t = g.op("add", va, vb)
        g.op("sqrt", t, out=out, live=True)
        g.release(t)
        g.sync()
        torch.cuda.synchronize()
        ref, _ = evaluate([{"op": "add", "in": ["a", "b"], "out": "t", "dtype": "f32"},
                           {"op": "sqrt", "in": ["t"], "out": "c", "dtype": "f32"}],
                          {"a": a, "b": b}, emulate_f32=True)
        got = host64(out)
        assert np.array_equal(got, ref["c"]), f"{shape}: {np.sum(got != ref['c'])} mismatches"


def _ln(dvm, ctx, x, gam, bet, eps=W.LN_EPS):
    from device_bytecode_vm_amd import composites as CP
    dx, dg, db = torch_dev(x, "bf16"), torch_dev(gam, "f32"), torch_dev(bet, "f32")
    out = empty_dev(x.shape, "bf16")
    g = dvm.Graph(ctx)
    CP.layer_norm(g, g.input(dx), g.input(dg), g.input(db), eps, out=out)
    g.sync()
    return host64(out)


@pytest.mark.parametrize("rows,h", [(1, 5120), (3, 5120), (37, 5120), (5, 96), (9, 1001), (2, 8192), (300, 24),
                                    (1500, 5122), (700, 1030)])
def test_layernorm(dvm, ctx, rows, h):
    say("layernorm", rows, h)
    x = W.layernorm_x(0, rows, rows, h)
    gam, bet = W.layernorm_params(h)
    got = _ln(dvm, ctx, x, gam, bet)
    ref = O.layer_norm(x, gam, bet, W.LN_EPS)
    ok, d = N.check_bf16(got, ref)
    assert ok, f"max ulp {d}"


def test_layernorm_workload_sampled(dvm, ctx):
    """Three calls of the LayerNorm stream at full size; rows sampled.  The
    third is tiled 4 rows at a time although no ceil(R / 2^j) equals 4 (the
    row count comes from the power-of-two floor on the shrink path), so its
    last tile is ragged in rows."""
    shapes = W.layernorm_shapes(0, 64)
    gam, bet = W.layernorm_params()
    g = np.random.default_rng(99)

    def from_floor(r):
        return r % 4 != 0 and all(-(-r // (1 << j)) != 4 for j in range(40))
    i_floor = next(i for i, (r, _) in enumerate(shapes) if r > 20000 and from_floor(r))
    from device_bytecode_vm_amd import composites as CP
    from device_bytecode_vm_amd import TensorDesc as TD
    r_f = shapes[i_floor][0]
    gh = dvm.Graph(dvm.Context(-1))
    CP.layer_norm(gh, gh.input(TD(1 << 34, "bf16", (r_f, W.H_LN))), gh.input(TD(2 << 34, "f32", (W.H_LN,))),
                  gh.input(TD(3 << 34, "f32", (W.H_LN,))), W.LN_EPS, out=TD(4 << 34, "bf16", (r_f, W.H_LN)))
    assert gh.flush().header()["tr"] == 4
    for i in (0, int(np.argmax([r for r, _ in shapes])), i_floor):
        rows, h = shapes[i]
        say("layernorm_stream", i, rows)
        x = W.layernorm_x(0, i, rows, h)
        got = _ln(dvm, ctx, x, gam, bet)
        idx = np.unique(np.concatenate([[0, rows - 1], g.integers(0, rows, 256)]))
        ref = O.layer_norm(x[idx], gam, bet, W.LN_EPS)
        ok, d = N.check_bf16(got[idx], ref)
        assert ok, f"call {i}: max ulp {d}"


@pytest.mark.parametrize("rows,cols", [(1, 16), (7, 3001), (40, 512), (3, 8192), (513, 17), (1200, 6484),
                                       (900, 1030)])
def test_softmax(dvm, ctx, rows, cols):
    from device_bytecode_vm_amd import composites as CP
    say("softmax", rows, cols)
    x = W.normal(np.random.default_rng(rows * 7 + cols), (rows, cols), 0, 1, "bf16")
    dx = torch_dev(x, "bf16")
    out = empty_dev(x.shape, "bf16")
    g = dvm.Graph(ctx)
    CP.softmax(g, g.input(dx), out=out)
    g.sync()
    ok, d = N.check_bf16(host64(out), O.softmax(x))
    assert ok, f"max ulp {d}"


@pytest.mark.parametrize("rows", [1, 5, 33])
def test_add_rmsnorm_fused(dvm, ctx, rows):
    from device_bytecode_vm_amd import composites as CP
    say("add_rmsnorm", rows)
    h = 5120
    rg = np.random.default_rng(rows)
    h0 = W.normal(rg, (rows, h), 0, 1, "bf16")
    r0 = W.normal(rg, (rows, h), 0, 1, "bf16")
    w = W.normal(rg, (h,), 1, 0.1)
    d0, dr, dw = torch_dev(h0, "bf16"), torch_dev(r0, "bf16"), torch_dev(w, "f32")
    h1 = empty_dev((rows, h), "bf16")
    n = empty_dev((rows, h), "bf16")
    g = dvm.Graph(ctx)
    vh = g.op("add", g.input(d0), g.input(dr), out=h1)
    CP.rms_norm(g, vh, g.input(dw), W.RMS_EPS, out=n)
    g.sync()
    st = g.stats()
    assert st["graphs"] == 1, st          # residual add and RMSNorm fused into one graph
    h1_ref = N.round_bf16(h0.astype(np.float64) + r0)
    assert np.array_equal(host64(h1), h1_ref)
    ok, d = N.check_bf16(host64(n), O.rms_norm(h1_ref, w, W.RMS_EPS))
    assert ok, f"max ulp {d}"


@pytest.mark.parametrize("rows,cols", [(3, 17408), (1, 100), (17, 777), (600, 2052)])
def test_swiglu(dvm, ctx, rows, cols):
    from device_bytecode_vm_amd import composites as CP
    say("swiglu", rows, cols)
    rg = np.random.default_rng(cols)
    gt = W.normal(rg, (rows, cols), 0, 1, "bf16")
    up = W.normal(rg, (rows, cols), 0, 1, "bf16")
    out = empty_dev((rows, cols), "bf16")
    g = dvm.Graph(ctx)
    CP.swiglu(g, g.input(torch_dev(gt, "bf16")), g.input(torch_dev(up, "bf16")), out=out)
    g.sync()
    ok, d = N.check_bf16(host64(out), O.swiglu(gt, up))
    assert ok, f"max ulp {d}"


def _if_else(dvm, ctx, x, y):
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
    return sv, host64(out)


@pytest.mark.parametrize("n", [1, 2, 37, 1000])
def test_if_else_add(dvm, ctx, n):
    for i in range(2):
        say("if_else_add", n, i)
        x, y, sign = W.ifelse_inputs(n, i, (n, 4096))
        sv, got = _if_else(dvm, ctx, x, y)
        ref, branch, s64 = O.if_else_add(x, y)
        band = O.sum_guard_band(x)
        assert abs(s64) > band
        assert abs(sv - s64) <= band
        assert (sv > 0) == branch
        assert np.array_equal(got, ref.astype(np.float32).astype(np.float64))


def test_reduce_all_max_and_empty(dvm, ctx):
    say("reduce_all_max")
    x = W.normal(np.random.default_rng(3), (999, 31), 0, 1)
    s = empty_dev((), "f32")
    g = dvm.Graph(ctx)
    g.op("reduce_max", g.input(torch_dev(x, "f32")), out=s, live=True, axis=0x7FFFFFFF)
    g.sync()
    assert float(s.item()) == float(x.max())


def _collapsed_operands(shape, n):
    st, acc = [], 1
    for d in reversed(shape):
        st.append(acc)
        acc *= d
    return [tuple(reversed(st))] * n


@pytest.mark.parametrize("tmpl,shape", [("elemwise", (513, 1031)), ("rowreduce", (1000, 5120)),
                                        ("rowreduce", (280, 3001)), ("elemwise", (3, 9)),
                                        ("rowreduce", (777, 16)), ("rowreduce", (3000, 6484)),
                                        ("rowreduce", (9, 15000)), ("rowreduce", (20000, 5120))])
def test_tilemap_bit_exact(dvm, ctx, tmpl, shape):
    """The VM's element -> tile and tile -> workgroup maps equal the oracle's."""
    import torch
    say("tilemap", tmpl, shape)
    x = torch.zeros(shape, dtype=torch.float32, device="cuda")
    out = empty_dev(shape, "f32")
    g = dvm.Graph(ctx)
    vx = g.input(x)
    if tmpl == "elemwise":
        g.op("exp", vx, out=out, live=True)
    else:
        m = g.op("reduce_max", vx)
        g.op("sub", vx, m, out=out, live=True)
        g.release(m)
    p = g.flush()
    h = p.header()
    R, Cc = h["R"], h["C"]
    tiles = empty_dev((R, Cc), "f32")
    wgs = empty_dev((R, Cc), "f32")
    dbg = p.debug_tilemap(tiles, wgs)
    dbg.launch()
    torch.cuda.synchronize()
    # oracle: same workload through the tiling rules
    tm = TL.ELEMWISE if tmpl == "elemwise" else TL.ROWREDUCE
    col = TL.collapse(tm, shape, _collapsed_operands(shape, 2))
    ops = [TL.Operand(4, s_r, s_c, 0) for s_r, s_c in col[2]]
    plan = TL.plan(tm, col[0], col[1], ops, TL.NV_WIDE if h["kernel_type"] == 2 else TL.NV_MAX)
    assert (h["tr"], h["tc"], h["block_dim"], h["body_tile"], h["grid"], h["g"], h["nv"]) == \
        (plan.tr, plan.tc, plan.block_dim, plan.body_tile, plan.grid, plan.g, plan.nv)
    et, ew = TL.element_tile_map(plan)
    assert np.array_equal(host64(tiles), et)
    assert np.array_equal(host64(wgs), ew)


def _with_specials(rg, shape):
    """N(0, 1) values with NaN, +inf, -inf and signed zeros sprinkled in."""
    x = W.normal(rg, shape, 0, 1)
    flat = x.reshape(-1)
    k = max(1, flat.size // 50)
    for v in (np.nan, np.inf, -np.inf, 0.0, -0.0):
        flat[rg.choice(flat.size, size=k, replace=False)] = v
    return x


@pytest.mark.parametrize("op", ["max", "min"])
def test_max_min_nan_propagation(dvm, ctx, op):
    """Binary max/min propagate NaN (IEEE 754-2019 maximum/minimum), as the
    oracle's; values compared exactly, NaN positions included."""
    say("binary", op, "nan")
    rg = np.random.default_rng(5)
    a = _with_specials(rg, (77, 1031))
    b = _with_specials(rg, (77, 1031))
    out = empty_dev(a.shape, "f32")
    g = dvm.Graph(ctx)
    g.op(op, g.input(torch_dev(a, "f32")), g.input(torch_dev(b, "f32")), out=out, live=True)
    g.sync()
    ref = O.maximum(a, b) if op == "max" else O.minimum(a, b)
    got = host64(out)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_row_max_nan_propagation(dvm, ctx):
    """A row max (rows inside one wave and rows across waves) is NaN exactly
    where the row holds a NaN, else the row's largest value."""
    for shape in [(61, 300), (9, 5120)]:
        say("row_max", "nan", shape)
        rg = np.random.default_rng(shape[1])
        x = W.normal(rg, shape, 0, 1)
        x[3, 7] = np.nan
        x[5, shape[1] - 1] = np.nan
        x[6, 0] = np.inf
        m = empty_dev((shape[0], 1), "f32")
        g = dvm.Graph(ctx)
        g.op("reduce_max", g.input(torch_dev(x, "f32")), out=m, live=True)
        g.sync()
        ref = O.reduce_max(x)
        got = host64(m)
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        ok = ~np.isnan(ref)
        assert np.array_equal(got[ok], ref[ok])


def test_empty_inputs(dvm, ctx):
    """Zero-size operands: nothing is launched for tile programs (outputs keep
    their contents), a reduce-all of nothing is the reduction's identity, and
    a MatMul with K = 0 is its epilogue on zeros."""
    import torch
    from device_bytecode_vm_amd import composites as CP
    for shape in [(0, 5120), (5, 0), (0,)]:
        say("empty elementwise", shape)
        x = torch.zeros(shape, dtype=torch.float32, device="cuda")
        out = torch.full(shape, 7.0, dtype=torch.float32, device="cuda")
        g = dvm.Graph(ctx)
        g.op("exp", g.input(x), out=out, live=True)
        g.sync()
        assert out.numel() == 0 or bool((out == 7.0).all())
    say("empty layernorm")
    x = torch.zeros((0, 5120), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    gam = torch.ones(5120, device="cuda")
    bet = torch.zeros(5120, device="cuda")
    g = dvm.Graph(ctx)
    CP.layer_norm(g, g.input(x), g.input(gam), g.input(bet), W.LN_EPS, out=y)
    g.sync()
    for op, ident in [("reduce_sum", 0.0), ("reduce_max", -np.inf)]:
        say("empty reduce-all", op)
        x = torch.zeros((0, 4096), dtype=torch.float32, device="cuda")
        s = torch.full((), 7.0, dtype=torch.float32, device="cuda")
        g = dvm.Graph(ctx)
        g.op(op, g.input(x), out=s, live=True, axis=0x7FFFFFFF)
        g.sync()
        assert float(s.item()) == ident
    say("matmul M = 0")
    a = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros(128, device="cuda")
    y = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    g = dvm.Graph(ctx)
    CP.matmul_bias_silu(g, g.input(a), g.input(b), g.input(bias), out=y)
    g.sync()
    say("matmul K = 0")
    bias_h = W.normal(np.random.default_rng(8), (136,), 0, 1)
    a = torch.zeros((37, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((0, 136), dtype=torch.bfloat16, device="cuda")
    y = empty_dev((37, 136), "bf16")
    g = dvm.Graph(ctx)
    CP.matmul_bias_silu(g, g.input(a), g.input(b), g.input(torch_dev(bias_h, "f32")), out=y)
    g.sync()
    torch.cuda.synchronize()
    ref = O.matmul_bias_silu(np.zeros((37, 0)), np.zeros((0, 136)), bias_h)
    ok, e = N.check_matmul(host64(y), ref)
    assert ok, f"max rel err {e:.3g}"


def test_operand_beyond_2gib(dvm, ctx):
    """One fp32 operand of 2.3 GB (offsets past 2^31 bytes from the base):
    y = sqrt(x * x + 1) over [70001, 8200], rows near the start, the middle
    and the end compared bit for bit with the fp32-emulating oracle."""
    import torch
    shape = (70001, 8200)
    say("beyond_2gib", shape)
    x = W.device_normal(shape, seed=17)
    y = torch.empty_like(x)
    g = dvm.Graph(ctx)
    vx = g.input(x)
    t = g.op("mul", vx, vx)
    u = g.op("add", t, 1.0)
    g.op("sqrt", u, out=y, live=True)
    g.release(t, u)
    g.sync()
    torch.cuda.synchronize()
    assert x.numel() * 4 > 2 ** 31
    rows = np.array([0, 1, 2, 35000, 52000, 65500, shape[0] - 2, shape[0] - 1])
    idx = torch.as_tensor(rows, device="cuda")
    xs, ys = host64(x[idx]), host64(y[idx])
    ops = [{"op": "mul", "in": ["x", "x"], "out": "t", "dtype": "f32"},
           {"op": "add", "in": ["t", 1.0], "out": "u", "dtype": "f32"},
           {"op": "sqrt", "in": ["u"], "out": "y", "dtype": "f32"}]
    ref, _ = evaluate(ops, {"x": xs}, emulate_f32=True)
    assert np.array_equal(ys, ref["y"]), f"{np.sum(ys != ref['y'])} mismatches"
    del x, y
    torch.cuda.empty_cache()


def test_views_elementwise(dvm, ctx):
    """ViewLoad/ViewStore: transposed and column-sliced inputs (row stride !=
    columns, misaligned base), row and column broadcasts, and a strided
    output view; fp32 chains compared bit for bit with the fp32-emulating
    oracle."""
    import torch
    rg = np.random.default_rng(21)
    R, C = 301, 1027
    xt_h = W.normal(rg, (C, R), 0, 1)            # stored [C, R]; used as its transpose
    wide_h = W.normal(rg, (R, C + 9), 0, 1)      # used as wide[:, 5:5 + C]
    row_h = W.normal(rg, (C,), 0, 1)             # broadcast along rows
    col_h = W.normal(rg, (R, 1), 0, 1)           # broadcast along columns
    xt = torch_dev(xt_h, "f32").t()
    ws = torch_dev(wide_h, "f32")[:, 5:5 + C]
    rowv, colv = torch_dev(row_h, "f32"), torch_dev(col_h, "f32")
    assert not xt.is_contiguous() and not ws.is_contiguous()
    big = torch.full((R, 2 * C), 7.0, dtype=torch.float32, device="cuda")
    out = big[:, ::2]                            # strided store, the other columns untouched
    say("views", R, C)
    g = dvm.Graph(ctx)
    t1 = g.op("add", g.input(xt), g.input(ws))
    t2 = g.op("mul", t1, g.input(rowv))
    g.op("sub", t2, g.input(colv), out=out, live=True)
    g.release(t1, t2)
    g.sync()
    torch.cuda.synchronize()
    ops = [{"op": "add", "in": ["a", "b"], "out": "t1", "dtype": "f32"},
           {"op": "mul", "in": ["t1", "r"], "out": "t2", "dtype": "f32"},
           {"op": "sub", "in": ["t2", "c"], "out": "y", "dtype": "f32"}]
    ref, _ = evaluate(ops, {"a": xt_h.T, "b": wide_h[:, 5:5 + C], "r": row_h, "c": col_h}, emulate_f32=True)
    got = host64(big)
    assert np.array_equal(got[:, ::2], ref["y"])
    assert np.all(got[:, 1::2] == 7.0)


@pytest.mark.parametrize("cols", [6484, 12000, 3000, 777])
def test_softmax_special_rows(dvm, ctx, cols):
    """Softmax rows with -inf (a whole row; all of one wave's elements of a
    row, following the lane layout: column c sits in lane (c // 8) mod g of
    its row, wave ((c // 8) mod g) // 64), NaN and +inf entries, at widths
    whose rows span waves (one exchange of each wave's max and sum) and fit
    one wave.  NaN exactly where the oracle has NaN; the rest within 2 bf16
    ulp."""
    import torch
    from device_bytecode_vm_amd import composites as CP
    say("softmax_special", cols)
    R = 64
    dx = torch.zeros((R, cols), dtype=torch.bfloat16, device="cuda")
    out = empty_dev((R, cols), "bf16")
    g = dvm.Graph(ctx)
    CP.softmax(g, g.input(dx), out=out)
    p = g.flush()
    gl = p.header()["g"]
    wave_of = ((np.arange(cols) // 8) % gl) // 64
    rg = np.random.default_rng(cols)
    x = rg.normal(0, 3, (R, cols))
    x[0] = -np.inf                                   # no finite maximum: a NaN row
    x[1, wave_of == 0] = -np.inf                     # one wave's elements all -inf
    x[2, cols // 3] = np.nan
    x[3, cols - 5] = np.inf
    x[4, wave_of != wave_of.max()] = -np.inf         # only the last wave of the row is finite
    x[5] = -1e30
    x[5, 7] = 0.0                                    # one finite spike far above the rest
    x[6, :] = 88.0                                   # large equal values
    xb = N.round_bf16(x)
    dx.copy_(torch.tensor(xb, dtype=torch.float64).to(torch.bfloat16))
    p.launch()
    torch.cuda.synchronize()
    got = host64(out)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = O.softmax(xb)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), [int(r) for r in np.where(np.isnan(got) != np.isnan(ref))[0][:5]]
    fin = ~np.isnan(ref).any(axis=1)
    ok, d = N.check_bf16(got[fin], ref[fin])
    assert ok, f"max ulp {d}"


@pytest.mark.parametrize("cols,n_after", [(6484, 0), (6484, 1), (6484, 7), (12000, 2), (3000, 7)])
def test_softmax_then_row_reductions(dvm, ctx, cols, n_after):
    """A softmax followed in the same program by n_after row reductions of its
    output (a row sum, then row maxes, each subtracted): 4096 rows, so each
    workgroup runs many tiles and the cross-wave buffers of consecutive tiles
    alternate or are fenced.  Sampled rows against the fp64 oracle graph, fp32
    criterion."""
    from device_bytecode_vm_amd import composites as CP
    say("softmax_then_reductions", cols, n_after)
    R = 4096
    x = W.normal(np.random.default_rng(cols + n_after), (R, cols), 0, 2, "f32")
    out = empty_dev((R, cols), "f32")
    g = dvm.Graph(ctx)
    v = y = CP.softmax(g, g.input(torch_dev(x, "f32")), out=out if n_after == 0 else None)
    ops = [{"op": "reduce_max", "in": ["x"], "out": "m", "dtype": "f32"},
           {"op": "sub", "in": ["x", "m"], "out": "d", "dtype": "f32"},
           {"op": "exp", "in": ["d"], "out": "e", "dtype": "f32"},
           {"op": "reduce_sum", "in": ["e"], "out": "s", "dtype": "f32"},
           {"op": "div", "in": ["e", "s"], "out": "v0", "dtype": "f32"}]
    for k in range(n_after):
        kind = "reduce_sum" if k == 0 else "reduce_max"
        r = g.op(kind, v)
        last = k == n_after - 1
        nv = g.op("sub", v, r, out=out if last else None, live=last)
        g.release(r)
        if k:
            g.release(v)
        v = nv
        ops += [{"op": kind, "in": [f"v{k}"], "out": f"r{k}", "dtype": "f32"},
                {"op": "sub", "in": [f"v{k}", f"r{k}"], "out": f"v{k + 1}", "dtype": "f32"}]
    if n_after:
        g.release(y)
    p = g.flush()
    assert p.header()["body_tile"] > 1
    p.launch()
    import torch
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, R - 1], np.random.default_rng(7).integers(0, R, 45)]))
    ref, _ = evaluate(ops, {"x": x[rows]})
    got = host64(out)[rows]
    ok, e = N.check_f32(got, ref[f"v{n_after}"])
    assert ok, f"rel err {e}"


def test_views_layernorm_and_softmax(dvm, ctx):
    """Row reductions over views: LayerNorm of a column slice (row stride
    5200) and softmax over a transposed view (unit stride along rows)."""
    import torch
    from device_bytecode_vm_amd import composites as CP
    say("view layernorm")
    rg = np.random.default_rng(22)
    x_wide = W.normal(rg, (45, 5200), 0, 1, "bf16")
    gam, bet = W.layernorm_params(5120)
    xv = torch_dev(x_wide, "bf16")[:, 40:40 + 5120]
    out = empty_dev((45, 5120), "bf16")
    g = dvm.Graph(ctx)
    CP.layer_norm(g, g.input(xv), g.input(torch_dev(gam, "f32")), g.input(torch_dev(bet, "f32")), W.LN_EPS, out=out)
    g.sync()
    ok, d = N.check_bf16(host64(out), O.layer_norm(x_wide[:, 40:40 + 5120], gam, bet, W.LN_EPS))
    assert ok, f"layernorm view: max ulp {d}"
    say("view softmax")
    s_h = W.normal(rg, (700, 33), 0, 1, "bf16")  # softmax over the 700 axis of its transpose
    sv = torch_dev(s_h, "bf16").t()
    out = empty_dev((33, 700), "bf16")
    g = dvm.Graph(ctx)
    CP.softmax(g, g.input(sv), out=out)
    g.sync()
    ok, d = N.check_bf16(host64(out), O.softmax(s_h.T))
    assert ok, f"softmax view: max ulp {d}"


def _specials_input(seed, shape, positive=False):
    rg = np.random.default_rng(seed)
    x = W.normal(rg, shape, 0, 3)
    if positive:
        x = np.abs(x) + 1e-3
    flat = x.reshape(-1)
    specials = [np.nan, np.inf, -np.inf, 0.0, -0.0, 0.5, -0.5, 1.5, 2.5, -2.5, 1e-30, -1e-30]
    for i, v in enumerate(specials):
        flat[(i * 7919) % flat.size] = v
    return x


def _same_specials(got, ref):
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = np.isfinite(ref)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
    return fin


def _check(got, ref, exact):
    fin = _same_specials(got, ref)
    if exact:
        assert np.array_equal(got[fin], ref[fin])
    else:
        scale = np.max(np.abs(ref[fin])) if fin.any() else 1.0
        assert np.max(np.abs(got[fin] - ref[fin])) <= 1e-5 * scale


UNARY_CASES = [("sqrt", True), ("abs", True), ("neg", True), ("round", True), ("floor", True),
               ("recip", True), ("exp", False), ("log", False)]


@pytest.mark.parametrize("op,exact", UNARY_CASES)
def test_unary_ops(dvm, ctx, op, exact):
    """Each unary instruction against the oracle on fp32 input with NaN, +-inf,
    signed zeros, ties and tiny values; correctly rounded ops bit for bit."""
    say("unary", op)
    shape = (129, 1037)
    x = _specials_input(31, shape)
    if op == "exp":
        # |x| <= 20 keeps max|ref| meaningful for the max-relative tolerance
        x = np.clip(x, -20, 20)
        x.reshape(-1)[5] = np.nan
    out = empty_dev(shape, "f32")
    g = dvm.Graph(ctx)
    g.op(op, g.input(torch_dev(x, "f32")), out=out, live=True)
    g.sync()
    ref, _ = evaluate([{"op": op, "in": ["x"], "out": "y", "dtype": "f32"}], {"x": x}, emulate_f32=True)
    _check(host64(out), ref["y"], exact)


def test_isfinite_u8(dvm, ctx):
    say("isfinite")
    x = _specials_input(32, (33, 515))
    out = empty_dev(x.shape, "u8")
    g = dvm.Graph(ctx)
    g.op("isfinite", g.input(torch_dev(x, "f32")), out=out, live=True)
    g.sync()
    assert np.array_equal(host64(out), O.isfinite(x).astype(np.float64))


BINARY_CASES = [("add", True), ("sub", True), ("mul", True), ("div", True), ("max", True), ("min", True),
                ("pow", False)]


@pytest.mark.parametrize("op,exact", BINARY_CASES)
def test_binary_ops(dvm, ctx, op, exact):
    """Each binary instruction, tile (op) tile in both orders and with a
    scalar on either side, against the oracle (fp32 emulation)."""
    shape = (77, 1031)
    a = _specials_input(41, shape, positive=(op == "pow"))
    b = _specials_input(42, shape)
    if op == "pow":
        b = np.clip(b, -4, 4)
        b.reshape(-1)[3] = np.nan
    da, db = torch_dev(a, "f32"), torch_dev(b, "f32")
    for form in ("tt", "tt_rev", "ts", "st"):
        say("binary", op, form)
        out = empty_dev(shape, "f32")
        g = dvm.Graph(ctx)
        va, vb = g.input(da), g.input(db)
        if form == "tt":
            g.op(op, va, vb, out=out, live=True)
            ins = ["a", "b"]
        elif form == "tt_rev":
            g.op(op, vb, va, out=out, live=True)
            ins = ["b", "a"]
        elif form == "ts":
            g.op(op, va, 1.75, out=out, live=True)
            ins = ["a", 1.75]
        else:
            g.op(op, -0.625, va, out=out, live=True)
            ins = [-0.625, "a"]
        g.sync()
        ref, _ = evaluate([{"op": op, "in": ins, "out": "y", "dtype": "f32"}], {"a": a, "b": b}, emulate_f32=True)
        _check(host64(out), ref["y"], exact)

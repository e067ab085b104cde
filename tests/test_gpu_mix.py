"""GPU parity of the MIX kernel (MatMul + elementwise epilogue) against the
oracle, through the C ABI.  Tolerance for matmul graphs: max|d|/max|ref| <=
1e-2 (bf16 inputs, fp32 accumulation); an fp32 matmul result is also held to
1e-4.  Shapes span several 128 x 128 tiles with ragged M, N and K tails (K
shorter than the loads in flight included); the
full MatMul+bias+SiLU shape is checked on seeded sampled rows (each output row
depends only on its own row of A, so sampled rows are exact checks)."""
import numpy as np
import pytest

import workloads as W
from oracle import numerics as N
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


def _inputs(seed, m, k, n):
    g = W.rng(seed)
    a = W.normal(g, (m, k), 0.0, 0.02, "bf16")
    b = W.normal(g, (k, n), 0.0, 0.02, "bf16")
    bias = W.normal(g, (n,), 0.0, 0.02)
    return a, b, bias


@pytest.mark.parametrize("m,k,n", [(1, 64, 128), (37, 72, 200), (3, 8, 128), (65, 40, 136), (128, 128, 128), (300, 136, 1000),
                                   (129, 5120, 264), (256, 5120, 1024), (4096, 256, 4096), (2100, 136, 4000)])
def test_matmul_bias_silu(dvm, ctx, m, k, n):
    import torch
    from device_bytecode_vm_amd import composites as CP
    say("matmul_bias_silu", m, k, n)
    a, b, bias = _inputs(7, m, k, n)
    y = empty_dev((m, n), "bf16")
    g = dvm.Graph(ctx)
    CP.matmul_bias_silu(g, g.input(torch_dev(a, "bf16")), g.input(torch_dev(b, "bf16")),
                        g.input(torch_dev(bias, "f32")), out=y)
    hdr = g.flush().header()
    from oracle import tiling as TL
    plan = TL.plan_matmul(m, n, k, 2, 2, [TL.Operand(4, 0, 1), TL.Operand(2, n, 1)])
    assert hdr["kernel_type"] == 1 and (hdr["tr"], hdr["block_dim"]) == (plan.tr, plan.block_dim)
    g2 = dvm.Graph(ctx)
    CP.matmul_bias_silu(g2, g2.input(torch_dev(a, "bf16")), g2.input(torch_dev(b, "bf16")),
                        g2.input(torch_dev(bias, "f32")), out=y)
    g2.sync()
    torch.cuda.synchronize()
    ref = O.matmul_bias_silu(a, b, bias)
    ok, e = N.check_matmul(host64(y), ref)
    assert ok, f"max rel err {e:.3g}"


def test_matmul_plain_f32(dvm, ctx):
    import torch
    for (m, k, n) in [(130, 200, 136), (5, 5120, 256)]:
        say("matmul_f32", m, k, n)
        a, b, _ = _inputs(3, m, k, n)
        z = empty_dev((m, n), "f32")
        g = dvm.Graph(ctx)
        g.op("matmul", g.input(torch_dev(a, "bf16")), g.input(torch_dev(b, "bf16")), out=z, live=True)
        g.sync()
        torch.cuda.synchronize()
        ref = O.matmul(a, b)
        e = N.max_rel_err(host64(z), ref)
        assert e <= 1e-4, f"max rel err {e:.3g}"


def test_matmul_residual_epilogue(dvm, ctx):
    """Epilogue with a full [M, N] operand, a scalar and a max: y = max(A@B + r, 0) * 0.5, bf16."""
    import torch
    m, k, n = 200, 96, 392
    say("matmul_residual", m, k, n)
    a, b, _ = _inputs(11, m, k, n)
    r = W.normal(W.rng(12), (m, n), 0.0, 0.05, "bf16")
    y = empty_dev((m, n), "bf16")
    # the device tensors are only referenced by the graph (the binding keeps
    # them alive until the launch)
    g = dvm.Graph(ctx)
    with g.group():
        z = g.op("matmul", g.input(torch_dev(a, "bf16")), g.input(torch_dev(b, "bf16")), dtype="f32")
        s = g.op("add", z, g.input(torch_dev(r, "bf16")))
        q = g.op("max", s, 0.0)
        h = g.op("mul", q, 0.5)
        g.op("cast", h, out=y, live=True)
        g.release(z, s, q, h)
    g.sync()
    torch.cuda.synchronize()
    ref = np.maximum(O.matmul(a, b) + r, 0.0) * 0.5
    ok, e = N.check_matmul(host64(y), ref)
    assert ok, f"max rel err {e:.3g}"


def test_matmul_bias_silu_full_size_sampled_rows(dvm, ctx):
    """The MatMul+bias+SiLU shape (K = 5120, N = 17408) at the largest M of
    the call list, all rows computed on the GPU, 48 seeded rows checked."""
    import torch
    from device_bytecode_vm_amd import composites as CP
    ms = W.matmul_ms(0)
    m = max(ms)
    say("matmul_bias_silu_full", m, W.K_MM, W.N_FFN)
    b, bias = W.matmul_weights()
    a = W.matmul_a(0, int(np.argmax(ms)), m)
    y = empty_dev((m, W.N_FFN), "bf16")
    g = dvm.Graph(ctx)
    CP.matmul_bias_silu(g, g.input(torch_dev(a, "bf16")), g.input(torch_dev(b, "bf16")),
                        g.input(torch_dev(bias, "f32")), out=y)
    g.sync()
    torch.cuda.synchronize()
    rows = np.sort(W.rng(5).choice(m, size=48, replace=False))
    rows[0], rows[-1] = 0, m - 1
    ref = O.matmul_bias_silu(a[rows], b, bias)
    got = host64(y[torch.as_tensor(rows, device=y.device)])
    ok, e = N.check_matmul(got, ref)
    assert ok, f"max rel err {e:.3g}"


def test_matmul_output_beyond_2gib(dvm, ctx):
    """Y [65536, 17408] bf16 is 2.3 GB: rows past 2^31 bytes from its base are
    stored through tile-based resources like the others.  K = 64 keeps the
    run short; sampled rows (first, middle, last, around 2^31 bytes) are
    checked against the oracle."""
    import torch
    from device_bytecode_vm_amd import composites as CP
    m, k, n = 65536, 64, 17408
    say("matmul_beyond_2gib", m, k, n)
    a, b, bias = _inputs(13, m, k, n)
    y = empty_dev((m, n), "bf16")
    assert y.numel() * 2 > 2 ** 31
    g = dvm.Graph(ctx)
    CP.matmul_bias_silu(g, g.input(torch_dev(a, "bf16")), g.input(torch_dev(b, "bf16")),
                        g.input(torch_dev(bias, "f32")), out=y)
    g.sync()
    torch.cuda.synchronize()
    boundary = (2 ** 31) // (n * 2)
    rows = np.array([0, 1, m // 2, boundary - 1, boundary, boundary + 1, m - 2, m - 1])
    got = host64(y[torch.as_tensor(rows, device=y.device)])
    ref = O.matmul_bias_silu(a[rows], b, bias)
    ok, e = N.check_matmul(got, ref)
    assert ok, f"max rel err {e:.3g}"
    del y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m,n", [(300, 1000), (2000, 17408), (8192, 17408), (1, 128), (129, 4000)])
def test_mix_tilemap_bit_exact(dvm, ctx, m, n):
    """The MIX kernel's element -> tile and tile -> workgroup maps equal the
    oracle's statement of the grouped, XCD-aware tile order."""
    import torch
    from device_bytecode_vm_amd import composites as CP
    from oracle import tiling as TL
    say("mix_tilemap", m, n)
    k = 64
    a = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((k, n), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros((n,), dtype=torch.float32, device="cuda")
    y = empty_dev((m, n), "bf16")
    g = dvm.Graph(ctx)
    CP.matmul_bias_silu(g, g.input(a), g.input(b), g.input(bias), out=y)
    p = g.flush()
    h = p.header()
    plan = TL.plan_matmul(m, n, k, 2, 2, [TL.Operand(4, 0, 1), TL.Operand(2, n, 1)])
    assert (h["tr"], h["tc"], h["block_dim"], h["body_tile"], h["grid"]) == \
        (plan.tr, plan.tc, plan.block_dim, plan.body_tile, plan.grid)
    tiles = torch.full((m, n), -1.0, dtype=torch.float32, device="cuda")
    wgs = torch.full((m, n), -1.0, dtype=torch.float32, device="cuda")
    dbg = p.debug_tilemap(tiles, wgs)
    dbg.launch()
    torch.cuda.synchronize()
    et, ew = TL.mix_element_tile_map(plan)
    assert np.array_equal(host64(tiles), et)
    assert np.array_equal(host64(wgs), ew)

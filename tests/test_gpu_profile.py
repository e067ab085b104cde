"""The VM's profiling twin (dvm_launch_profiled): the same results as the
product kernel, bit for bit, and a sane per-workgroup cycle split."""
import numpy as np
import pytest

import workloads as W
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


def _layernorm_program(dvm, ctx, rows, out):
    from device_bytecode_vm_amd import composites as CP
    rg = np.random.default_rng(7)
    x = torch_dev(W.normal(rg, (rows, W.H_LN), 0, 1, "bf16"), "bf16")
    gam = torch_dev(W.normal(rg, (W.H_LN,), 1, 0.1), "f32")
    bet = torch_dev(W.normal(rg, (W.H_LN,), 0, 0.1), "f32")
    g = dvm.Graph(ctx)
    CP.layer_norm(g, g.input(x), g.input(gam), g.input(bet), W.LN_EPS, out=out)
    p = g.flush()
    p._keep += [x, gam, bet]
    return p


def test_profiled_launch_matches_and_splits(dvm, ctx):
    import torch
    rows = 4096
    print("CASE profile layernorm", rows, flush=True)
    y1, y2 = empty_dev((rows, W.H_LN), "bf16"), empty_dev((rows, W.H_LN), "bf16")
    p1 = _layernorm_program(dvm, ctx, rows, y1)
    p2 = _layernorm_program(dvm, ctx, rows, y2)
    h = p2.header()
    assert h["body_tile"] >= 2
    c = torch.zeros(p2.PROF_COUNTERS * h["grid"], dtype=torch.int64, device="cuda")
    p1.launch()
    p2.launch_profiled(c)
    torch.cuda.synchronize()
    assert np.array_equal(host64(y1), host64(y2))
    cnt = c.view(-1, p2.PROF_COUNTERS).cpu().numpy()
    total, dec, exe, tile, n = (cnt[:, k] for k in range(5))
    assert (total > 0).all() and (dec > 0).all() and (exe > 0).all() and (tile > 0).all()
    assert (dec + exe + tile <= total).all()
    # dispatches: the prologue once, the body once per tile (row-register
    # runs inside a handler are not dispatches of their own)
    w = p2.words()
    n_pro, n_body = (w[15] - w[14]) // 2, (w[17] - w[16]) // 2
    # workgroup b runs tiles b, b + grid, ... below block_dim
    tiles = np.array([len(range(b, h["block_dim"], h["grid"])) for b in range(h["grid"])])
    assert (n >= tiles).all() and (n <= n_pro + tiles * n_body).all()
    for t in np.unique(tiles):
        assert len(np.unique(n[tiles == t])) == 1


def test_profiled_launch_rejects(dvm, ctx):
    import torch
    y = empty_dev((64, W.H_LN), "bf16")
    p = _layernorm_program(dvm, ctx, 64, y)
    short = torch.zeros(p.PROF_COUNTERS * p.header()["grid"] - 1, dtype=torch.int64, device="cuda")
    with pytest.raises(dvm.DvmError):
        p.launch_profiled(short)
    a = torch_dev(np.ones((16, 64)), "bf16")
    b = torch_dev(np.ones((64, 32)), "bf16")
    g = dvm.Graph(ctx)
    g.op("matmul", g.input(a), g.input(b), out=empty_dev((16, 32), "f32"), live=True)
    q = g.flush()
    assert q.header()["kernel_type"] == 1
    c = torch.zeros(q.PROF_COUNTERS * max(q.header()["grid"], 1), dtype=torch.int64, device="cuda")
    with pytest.raises(dvm.DvmError):
        q.launch_profiled(c)

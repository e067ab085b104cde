"""GPU parity of stacked launches (independent graphs packed into one launch,
the stacking-based fusion of the DVM review page, section 5.1, spatial and
temporal), through the C ABI.  A stacked program runs every segment with its
own header and tiling (spatial: on its own workgroups; temporal: every
workgroup walks the segments in sequence), so each output must equal, bit
for bit, what the same graph computes when launched alone; LayerNorm outputs
are also checked against the oracle, and the temporal tile map against the
oracle's statement of it.
"""
import numpy as np
import pytest

import workloads as W
from oracle import numerics as N
from oracle import ops as O
from oracle import tiling as TL
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


def say(*a):
    print("CASE", *a, flush=True)


def run_layernorms(dvm, ctx, xs, gam, bet, stacking, temporal=False):
    from device_bytecode_vm_amd import composites as CP
    g = dvm.Graph(ctx)
    g.set_stacking(stacking, temporal)
    ys = [empty_dev(x.shape, "bf16") for x in xs]
    for x, y in zip(xs, ys):
        CP.layer_norm(g, g.input(x), g.input(gam), g.input(bet), W.LN_EPS, out=y)
    g.sync()
    return ys, g.stats()


@pytest.mark.parametrize("stacking,temporal", [(2, False), (7, False), (2, True), (7, True)])
def test_stacked_layernorm_stream(dvm, ctx, stacking, temporal):
    import torch
    say("stacked_layernorm", stacking, "temporal" if temporal else "spatial")
    shapes = W.layernorm_shapes(0, 64)[:12]
    xs = [W.device_normal((min(r, 20000), W.H_LN), seed=1000 + i, dtype="bf16") for i, (r, _) in enumerate(shapes)]
    gam = W.device_normal((W.H_LN,), seed=1, mu=1.0, sd=0.1)
    bet = W.device_normal((W.H_LN,), seed=2, sd=0.1)
    ys, st = run_layernorms(dvm, ctx, xs, gam, bet, stacking, temporal)
    ref, st1 = run_layernorms(dvm, ctx, xs, gam, bet, 1)
    assert st["stacked"] > 0 and st["launches"] < st1["launches"]
    for y, r in zip(ys, ref):
        assert torch.equal(y, r)
    gh, bh = host64(gam), host64(bet)
    rg = np.random.default_rng(3)
    for x, y in zip(xs, ys):
        idx = np.unique(np.concatenate([[0, x.shape[0] - 1], rg.integers(0, x.shape[0], 64)]))
        ok, d = N.check_bf16(host64(y[idx]), O.layer_norm(host64(x[idx]), gh, bh, W.LN_EPS))
        assert ok, f"max ulp {d}"


@pytest.mark.parametrize("temporal", [False, True])
def test_stacked_op_stream_with_dependences(dvm, ctx, temporal):
    """A short transformer op stream (residual adds chained through h, SwiGLU
    and softmax writing shared outputs): stacking must keep every
    read-after-write, write-after-read and write-after-write order."""
    import torch
    from device_bytecode_vm_amd import composites as CP
    say("stacked_op_stream", "temporal" if temporal else "spatial")
    T, TKV, motifs = W.stream_step(5, 300, tmax=300, tkv_max=700)
    H, F = 512, 1536
    bf = dict(dtype="bf16")

    def run(stacking):
        hs = [W.device_normal((T, H), seed=20, **bf), torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")]
        rs = [W.device_normal((T, H), seed=21 + j, **bf) for j in range(4)]
        w = W.device_normal((H,), seed=25, mu=1.0, sd=0.1)
        gs = [W.device_normal((T, F), seed=26 + j, **bf) for j in range(2)]
        us = [W.device_normal((T, F), seed=28 + j, **bf) for j in range(2)]
        ss = [W.device_normal((4, T, TKV), seed=30 + j, **bf) for j in range(2)]
        n_out = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
        o_out = torch.zeros((T, F), dtype=torch.bfloat16, device="cuda")
        p_out = torch.zeros((4, T, TKV), dtype=torch.bfloat16, device="cuda")
        g = dvm.Graph(ctx)
        g.set_stacking(stacking, temporal and stacking > 1)
        cur = 0
        vh = g.input(hs[0])
        snaps = []
        for k, (kind, j) in enumerate(motifs):
            if kind == "add":
                nxt = 1 - cur
                vh = g.op("add", vh, g.input(rs[j]), out=hs[nxt])
                cur = nxt
            elif kind == "rmsnorm":
                CP.rms_norm(g, vh, g.input(w), W.RMS_EPS, out=n_out)
            elif kind == "swiglu":
                CP.swiglu(g, g.input(gs[j]), g.input(us[j]), out=o_out)
            else:
                CP.softmax(g, g.input(ss[j]), out=p_out)
            if k % 97 == 96:
                g.sync()
                snaps.append([t.clone() for t in (hs[0], hs[1], n_out, o_out, p_out)])
        g.sync()
        snaps.append([t.clone() for t in (hs[0], hs[1], n_out, o_out, p_out)])
        return snaps, g.stats()

    a, sa = run(7)
    b, sb = run(1)
    assert sa["stacked"] > 0 and sa["launches"] < sb["launches"]
    for sa_, sb_ in zip(a, b):
        for x, y in zip(sa_, sb_):
            assert torch.equal(x, y)


@pytest.mark.parametrize("temporal", [False, True])
def test_program_stack_abi(dvm, ctx, temporal):
    import torch
    say("program_stack_abi", "temporal" if temporal else "spatial")
    xs = [W.device_normal((300 + 100 * i, 777), seed=60 + i) for i in range(5)]
    outs = [torch.empty_like(x) for x in xs]
    refs = [torch.empty_like(x) for x in xs]
    progs, singles = [], []
    for x, o, r in zip(xs, outs, refs):
        for dst, lst in ((o, progs), (r, singles)):
            g = dvm.Graph(ctx)
            t = g.op("mul", g.input(x), g.input(x))
            g.op("sqrt", t, out=dst, live=True)
            g.release(t)
            lst.append(g.flush())
    q = dvm.stack_programs(progs, temporal)
    assert q.header()["segments"] == 5
    q.launch()
    for p in singles:
        p.launch()
    torch.cuda.synchronize()
    for o, r, x in zip(outs, refs, xs):
        assert torch.equal(o, r)
        assert torch.equal(o, torch.abs(x))       # sqrt(x * x) = |x| for these magnitudes


@pytest.mark.parametrize("rows", [[3000, 17, 5000, 9000], [5, 9, 40]])
def test_temporal_tilemap_bit_exact(dvm, ctx, rows):
    """Tile maps of a temporally stacked launch: every segment's element ->
    tile map is its own program's, and tile t of segment s runs on the
    workgroup the oracle's temporal order names (reported as that
    workgroup's place in the segment's strided order)."""
    import torch
    say("temporal_tilemap", rows)
    dbgs, maps = [], []
    for r in rows:
        x = torch.zeros((r, 777), dtype=torch.float32, device="cuda")
        g = dvm.Graph(ctx)
        g.op("exp", g.input(x), out=empty_dev((r, 777), "f32"), live=True)
        p = g.flush()
        h = p.header()
        tiles = empty_dev((h["R"], h["C"]), "f32")
        wgs = empty_dev((h["R"], h["C"]), "f32")
        dbgs.append(p.debug_tilemap(tiles, wgs))
        maps.append((h, tiles, wgs))
    assert len({d.header()["kernel_type"] for d in dbgs}) == 1
    q = dvm.stack_programs(dbgs, temporal=True)
    G = q.header()["grid"]
    bds = [h["block_dim"] for h, _, _ in maps]
    assert G == min(512, sum(bds))
    q.launch()
    torch.cuda.synchronize()
    # expected: from the oracle's temporal order
    base = [sum(bds[:i]) for i in range(len(bds))]
    for s, (h, tiles, wgs) in enumerate(maps):
        et = np.full((h["R"], h["C"]), -1.0)
        ew = np.full((h["R"], h["C"]), -1.0)
        n_c = -(-h["C"] // h["tc"])
        for b in range(G):
            for seg, t in TL.temporal_stack_tiles(b, G, bds):
                if seg != s:
                    continue
                (r0, r1), (c0, c1) = TL.tile_box(t, h["tr"], h["tc"], h["R"], h["C"], n_c)
                assert (et[r0:r1, c0:c1] == -1).all()
                et[r0:r1, c0:c1] = t
                ew[r0:r1, c0:c1] = (b - base[s]) % G
        assert (et >= 0).all()
        assert np.array_equal(host64(tiles), et)
        assert np.array_equal(host64(wgs), ew)

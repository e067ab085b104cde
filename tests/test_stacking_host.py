"""Host tests (no GPU) of stacking: independent encoded graphs packed into one
launch (the stacking-based fusion of the DVM review page, section 5.1,
Figure 9).  An encode-only context holds what it would launch, so the
stacking decisions show in the programs dvm_graph_take_program hands out.

Directory offsets are the bytecode format of csrc/bytecode.h, restated here
to read stacked programs.
"""
import pytest

import device_bytecode_vm_amd as dvm
from device_bytecode_vm_amd import TensorDesc as TD
from device_bytecode_vm_amd import _lib as L
from device_bytecode_vm_amd import composites as CP

STACK_MAGIC, S_NSEG, S_DIR = 0x4B545344, 1, 2
H_GRID = 6


@pytest.fixture(scope="module")
def ectx():
    return dvm.Context(-1)


def addr():
    addr.k += 1
    return addr.k << 36


addr.k = 0


def layer_norm(g, rows, h=5120, out=None, x=None):
    x = g.input(x or TD(addr(), "bf16", (rows, h)))
    gam = g.input(TD(addr(), "f32", (h,)))
    bet = g.input(TD(addr(), "f32", (h,)))
    y = out or TD(addr(), "bf16", (rows, h))
    CP.layer_norm(g, x, gam, bet, 1e-6, out=y)
    return y


def drain(g):
    out = []
    while True:
        p = g.take_program()
        if p is None:
            return out
        out.append(p)


def test_independent_graphs_stack(ectx):
    g = dvm.Graph(ectx)
    g.set_stacking(4)
    for r in (3000, 5000, 7000, 9000, 11000, 13000):
        layer_norm(g, r)
    g.flush_launch()                            # the last graph, then the stack
    progs = drain(g)
    assert [p.header()["segments"] for p in progs] == [4, 2]
    w = progs[0].words()
    assert w[0] == STACK_MAGIC and w[S_NSEG] == 4
    firsts = [w[S_DIR + 2 * i + 1] for i in range(4)]
    grids = [w[w[S_DIR + 2 * i] + H_GRID] for i in range(4)]
    assert firsts == [0, grids[0], grids[0] + grids[1], sum(grids[:3])]   # disjoint workgroup ranges
    assert progs[0].header()["grid"] == sum(grids)
    assert all(w[S_DIR + 2 * i] % 2 == 0 for i in range(4))             # even segment offsets
    st = g.stats()
    assert st["stacked"] == 6 and st["graphs"] == 6


def test_dependent_graph_breaks_the_stack(ectx):
    g = dvm.Graph(ectx)
    g.set_stacking(7)
    y1 = layer_norm(g, 3000)
    layer_norm(g, 5000)
    # reads y1, written by the first stacked graph: the stack launches first
    layer_norm(g, 3000, x=y1)
    layer_norm(g, 7000)
    g.flush_launch()
    assert [p.header()["segments"] for p in drain(g)] == [2, 2]
    # a graph writing what a stacked one reads (WAR) or writes (WAW) also does
    g2 = dvm.Graph(ectx)
    g2.set_stacking(7)
    y = layer_norm(g2, 3000)
    layer_norm(g2, 4000)
    layer_norm(g2, 3000, out=y)                 # WAW on y
    g2.flush_launch()
    assert [p.header()["segments"] for p in drain(g2)] == [2, 1]


def test_unstackable_programs_run_after_the_stack(ectx):
    g = dvm.Graph(ectx)
    g.set_stacking(7)
    layer_norm(g, 3000)
    layer_norm(g, 5000)
    x = g.input(TD(addr(), "f32", (1000, 4096)))
    g.op("reduce_sum", x, out=TD(addr(), "f32", ()), live=True, axis=L.AXIS_ALL)
    progs = drain(g)
    assert [(p.header()["segments"], p.header()["tmpl"]) for p in progs] == [(2, 1), (1, 2)]
    # programs of the two VM builds do not share a launch
    g2 = dvm.Graph(ectx)
    g2.set_stacking(7)
    layer_norm(g2, 3000)                        # wide build
    a = g2.input(TD(addr(), "f32", (64, 1000)))
    g2.op("exp", a, out=TD(addr(), "f32", (64, 1000)), live=True)   # standard build
    g2.flush_launch()
    hs = [p.header() for p in drain(g2)]
    assert [h["segments"] for h in hs] == [1, 1] and hs[0]["kernel_type"] != hs[1]["kernel_type"]


def test_program_stack_abi(ectx):
    g = dvm.Graph(ectx)
    ps = []
    for r in (100, 200, 300):
        layer_norm(g, r)
        ps.append(g.flush())
    q = dvm.stack_programs(ps)
    assert q.header()["segments"] == 3
    assert q.header()["grid"] == sum(p.header()["grid"] for p in ps)
    with pytest.raises(dvm.DvmError):
        dvm.stack_programs(ps[:1])
    with pytest.raises(dvm.DvmError):
        g.set_stacking(8)


TSTACK_MAGIC, H_BLOCK_DIM = 0x4B535454, 4


def test_temporal_stack_directory(ectx):
    """Temporal stacking: the directory lists each segment's first tile in
    one tile space (the running sum of block_dim), and the launch has
    min(512, total tiles) workgroups."""
    g = dvm.Graph(ectx)
    g.set_stacking(4, temporal=True)
    for r in (3000, 5000, 7000, 9000):
        layer_norm(g, r)
    g.flush_launch()
    (p,) = drain(g)
    w = p.words()
    assert w[0] == TSTACK_MAGIC and w[S_NSEG] == 4
    bds = [w[w[S_DIR + 2 * i] + H_BLOCK_DIM] for i in range(4)]
    assert [w[S_DIR + 2 * i + 1] for i in range(4)] == [0, bds[0], bds[0] + bds[1], sum(bds[:3])]
    assert p.header()["segments"] == 4 and p.header()["grid"] == min(512, sum(bds))
    assert p.verify() is None


def test_temporal_stack_of_small_graphs(ectx):
    """Few tiles in all: one workgroup per tile of the whole stack."""
    g = dvm.Graph(ectx)
    g.set_stacking(3, temporal=True)
    for r in (8, 16, 24):
        layer_norm(g, r)
    g.flush_launch()
    (p,) = drain(g)
    w = p.words()
    total = sum(w[w[S_DIR + 2 * i] + H_BLOCK_DIM] for i in range(3))
    assert total < 512 and p.header()["grid"] == total


def test_program_stack_temporal_abi(ectx):
    progs = []
    for r in (2000, 3000, 4000):                    # all on the wide build
        g = dvm.Graph(ectx)
        layer_norm(g, r)
        progs.append(g.flush())
    q = dvm.stack_programs(progs, temporal=True)
    w = q.words()
    assert w[0] == TSTACK_MAGIC and q.header()["segments"] == 3 and q.verify() is None
    s = dvm.stack_programs(progs)
    assert s.words()[0] == STACK_MAGIC


def test_stack_order_is_checked(ectx):
    g = dvm.Graph(ectx)
    assert L.lib.dvm_graph_set_stack_order(g.h, 2) == L.ERR_INVALID_ARG
    assert L.lib.dvm_graph_set_stack_order(g.h, 1) == 0


def test_spatial_stack_orders_segments_by_work_per_workgroup(ectx):
    """A spatial stack launches the segments with the most work per workgroup
    first (bytes per tile times tiles per workgroup), so the launch ends on
    its shortest workgroups; equal keys keep the program order."""
    H_BLOCK_DIM, H_BODY_TILE, H_R_LO = 4, 5, 18
    g = dvm.Graph(ectx)
    g.set_stacking(7)
    rows = (3000, 90000, 12000, 20000, 40000)   # all on the wide build
    for r in rows:
        layer_norm(g, r)
    g.flush_launch()
    (p,) = drain(g)
    w = p.words()
    assert w[S_NSEG] == len(rows)
    segs = [w[S_DIR + 2 * i] for i in range(len(rows))]
    got_rows = [w[o + H_R_LO] for o in segs]
    assert sorted(got_rows) == sorted(rows)
    # per-workgroup work of each segment, in launch order, never increases
    work = [w[o + H_BODY_TILE] * (w[o + H_R_LO] * 5120 * 4 + 2 * 5120 * 4) / w[o + H_BLOCK_DIM] for o in segs]
    assert all(a >= b for a, b in zip(work, work[1:])), list(zip(got_rows, work))
    firsts = [w[S_DIR + 2 * i + 1] for i in range(len(rows))]
    assert firsts == sorted(firsts) and firsts[0] == 0

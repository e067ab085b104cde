"""Host tests (no GPU) of static-graph symbolic fusion (templates): an op
graph recorded once over symbolic dims, its fusion partition decided once
(DVM review page, section 5.2, static-graph fusion), then bound to concrete
shapes that only get tiled and encoded.

* The partition decided on symbols equals the partition the streaming fuser
  makes for concrete bindings of the same graph.
* A run encodes, per graph, the program the dynamic path encodes for the same
  binding (same header words and body).
* Bindings that break the template are refused: a symbol bound to two sizes,
  a wrong concrete dim, an output aliasing an input, and a value crossing
  fused graphs without being an output.
"""
import pytest

import device_bytecode_vm_amd as dvm
from device_bytecode_vm_amd import TensorDesc as TD
from device_bytecode_vm_amd import _lib as L
from device_bytecode_vm_amd import composites as CP

H, F, NH = 5120, 17408, 40


@pytest.fixture(scope="module")
def ectx():
    return dvm.Context(-1)


def block(g, h, r, w, ga, up, sc, outs):
    """A transformer-block slice: residual add, RMSNorm, SwiGLU, softmax."""
    h1 = g.op("add", h, r, out=outs[0], live=True)
    CP.rms_norm(g, h1, w, 1e-6, out=outs[1])
    CP.swiglu(g, ga, up, out=outs[2])
    CP.softmax(g, sc, out=outs[3])


def build_template(ctx):
    t = dvm.Template(ctx)
    h = t.input("bf16", ("T", H))
    r = t.input("bf16", ("T", H))
    w = t.input("f32", (H,))
    ga = t.input("bf16", ("T", F))
    up = t.input("bf16", ("T", F))
    sc = t.input("bf16", (NH, "T", "TKV"))
    block(t, h, r, w, ga, up, sc, [t.output("bf16") for _ in range(4)])
    return t


def tensors(T, TKV, base=1):
    k = [base]

    def td(dt, shape):
        k[0] += 1
        return TD(k[0] << 40, dt, shape)
    ins = [td("bf16", (T, H)), td("bf16", (T, H)), td("f32", (H,)), td("bf16", (T, F)), td("bf16", (T, F)),
           td("bf16", (NH, T, TKV))]
    outs = [td("bf16", (T, H)), td("bf16", (T, H)), td("bf16", (T, F)), td("bf16", (NH, T, TKV))]
    return ins, outs


def dynamic(ctx, T, TKV):
    g = dvm.Graph(ctx)
    ins, outs = tensors(T, TKV)
    vs = [g.input(x) for x in ins]
    block(g, *vs, outs)
    g.flush_launch()
    progs = []
    while True:
        p = g.take_program()
        if p is None:
            break
        progs.append(p)
    return g.flush_log(), progs


def test_partition_equals_streaming_fuser(ectx):
    t = build_template(ectx)
    n = t.finalize()
    part, us = t.partition()
    assert n == 3 and us > 0
    sizes = [part.count(i) for i in range(n)]
    for T, TKV in [(100, 300), (3487, 6484), (16, 8192)]:
        log, _ = dynamic(ectx, T, TKV)
        assert [k for k, _ in log] == sizes, (T, TKV)


def test_run_encodes_the_dynamic_programs(ectx):
    t = build_template(ectx)
    t.finalize()
    for T, TKV in [(3487, 6484), (600, 1031)]:
        ins, outs = tensors(T, TKV)
        t.run(ins, outs)
        tg = t.graph
        tg.flush_launch()
        got = []
        while True:
            p = tg.take_program()
            if p is None:
                break
            got.append(p)
        _, want = dynamic(ectx, T, TKV)
        assert [p.words() for p in got] == [p.words() for p in want]


def test_template_refusals(ectx):
    t = build_template(ectx)
    t.finalize()
    ins, outs = tensors(100, 300)
    bad = list(ins)
    bad[3] = TD(99 << 40, "bf16", (101, F))          # T bound to 100 and 101
    with pytest.raises(dvm.DvmError) as e:
        t.run(bad, outs)
    assert e.value.status == L.ERR_SHAPE
    bad = list(ins)
    bad[2] = TD(99 << 40, "f32", (H + 1,))           # a concrete dim
    with pytest.raises(dvm.DvmError) as e:
        t.run(bad, outs)
    assert e.value.status == L.ERR_SHAPE
    alias = list(outs)
    alias[0] = ins[0]                                # output on top of an input
    with pytest.raises(dvm.DvmError) as e:
        t.run(ins, alias)
    assert e.value.status == L.ERR_INVALID_ARG
    # an internal value read by a later fused graph needs storage
    t2 = dvm.Template(ectx)
    x = t2.input("f32", ("N", 64))
    y = t2.input("f32", ("M", 64))
    a = t2.op("exp", x)                               # internal
    t2.op("add", y, 1.0, out=t2.output("f32"))        # another shape: a new graph
    t2.op("mul", a, 2.0, out=t2.output("f32"))        # reads a from the first graph
    with pytest.raises(dvm.DvmError) as e:
        t2.finalize()
    assert e.value.status == L.ERR_RESOURCE

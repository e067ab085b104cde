"""Encoder clean-up before tiling (constant propagation and dead-instruction
elimination, which the DVM paper review page, section 5.2, names as encoder
work), checked on the encoded program alone (no device).

Rewrites that keep every stored value bit-identical (x * 1, 1 * x, x / 1,
x - (+0), x + (-0), (-0) + x, a same-dtype cast nobody stores, ops nobody
reads) must leave exactly the program of the graph written without them;
the inexact look-alikes (x + (+0), x - (-0)) must stay.
"""
import pytest

import device_bytecode_vm_amd as dvm
from device_bytecode_vm_amd import TensorDesc as TD

X, Y, Z = 1 << 32, 2 << 32, 3 << 32
SH = (300, 1000)


@pytest.fixture(scope="module")
def ectx():
    return dvm.Context(-1)


def encode(ectx, body, dt="f32"):
    g = dvm.Graph(ectx)
    with g.group():
        body(g, g.input(TD(X, dt, SH)))
    return g.flush()


def same_program(a, b):
    return a.header() == b.header() and a.words() == b.words()


def exp_of_x(g, x):
    g.op("exp", x, out=TD(Y, "f32", SH), live=True)


def test_exact_identities_fold_away(ectx):
    def body(g, x):
        t1 = g.op("mul", x, 1.0)
        t2 = g.op("mul", 1.0, t1)
        t3 = g.op("div", t2, 1.0)
        t4 = g.op("sub", t3, 0.0)
        t5 = g.op("add", t4, -0.0)
        t6 = g.op("add", -0.0, t5)
        t7 = g.op("cast", t6, dtype="f32")
        g.op("exp", t7, out=TD(Y, "f32", SH), live=True)
        g.release(t1, t2, t3, t4, t5, t6, t7)
    assert same_program(encode(ectx, body), encode(ectx, exp_of_x))


def test_dead_ops_dropped(ectx):
    def body(g, x):
        s = g.op("reduce_sum", x)          # would make the graph a row reduction
        n = g.op("neg", x)
        m = g.op("mul", n, s)               # reads both: dead in turn
        g.op("exp", x, out=TD(Y, "f32", SH), live=True)
        g.release(s, n, m)
    p = encode(ectx, body)
    assert same_program(p, encode(ectx, exp_of_x))
    assert p.header()["tmpl"] == encode(ectx, exp_of_x).header()["tmpl"]


@pytest.mark.parametrize("op,c", [("add", 0.0), ("sub", -0.0), ("mul", 2.0), ("div", -1.0), ("sub", 0.0)])
def test_inexact_lookalikes_stay(ectx, op, c):
    def body(g, x):
        # sub with the scalar on the left (0 - x) is not x either
        t = g.op(op, 0.0, x) if (op, c) == ("sub", 0.0) else g.op(op, x, c)
        g.op("exp", t, out=TD(Y, "f32", SH), live=True)
        g.release(t)
    assert encode(ectx, body).header()["n_instr"] > encode(ectx, exp_of_x).header()["n_instr"]


def test_stored_identity_becomes_a_copy(ectx):
    def body(g, x):
        t = g.op("mul", x, 1.0, out=TD(Z, "f32", SH), live=True)
        g.op("exp", t, out=TD(Y, "f32", SH), live=True)

    def explicit(g, x):
        t = g.op("cast", x, out=TD(Z, "f32", SH), dtype="f32", live=True)
        g.op("exp", t, out=TD(Y, "f32", SH), live=True)
    assert same_program(encode(ectx, body), encode(ectx, explicit))


def test_identity_across_dtypes_is_a_cast(ectx):
    def body(g, x):
        t = g.op("div", x, 1.0, dtype="f32")      # bf16 x to an fp32 value
        g.op("exp", t, out=TD(Y, "f32", SH), live=True)
        g.release(t)

    def explicit(g, x):
        t = g.op("cast", x, dtype="f32")
        g.op("exp", t, out=TD(Y, "f32", SH), live=True)
        g.release(t)
    assert same_program(encode(ectx, body, "bf16"), encode(ectx, explicit, "bf16"))


def test_all_dead_graph_encodes_nothing(ectx):
    g = dvm.Graph(ectx)
    with g.group():
        x = g.input(TD(X, "f32", SH))
        e = g.op("exp", x)
        g.release(e)
    assert g.flush() is None
    # the graph stays usable
    with g.group():
        exp_of_x(g, g.input(TD(X, "f32", SH)))
    assert same_program(g.flush(), encode(ectx, exp_of_x))

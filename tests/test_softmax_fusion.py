"""Host tests (no GPU) of the softmax fusion: the encoded chain row max,
subtract, exp, row sum, reciprocal, multiply becomes one softmax instruction
when its row registers die with it (rows across waves then exchange each
wave's max and sum once, behind one barrier; rows inside a wave run the
chain's own steps), and stays unfused when a value of the chain is stored.

Handler ids and header words are the bytecode format of csrc/bytecode.h,
restated here to read encoded programs.
"""
import pytest

import device_bytecode_vm_amd as dvm
from device_bytecode_vm_amd import TensorDesc as TD
from device_bytecode_vm_amd import composites as CP

H_FLAGS, H_BODY_BEGIN, H_BODY_END = 26, 16, 17
HD_SOFTMAX, HD_REDX, HD_RED, HD_SYNC = 160, 127, 118, 149
HF_RED_ALT = 8


@pytest.fixture(scope="module")
def ectx():
    return dvm.Context(-1)


def handlers(p):
    w = p.words()
    return [w[i] & 0xFF for i in range(w[H_BODY_BEGIN], w[H_BODY_END], 2)]


@pytest.mark.parametrize("shape,across", [((139480, 6484), True), ((4096, 12000), True), ((3000, 5120), False),
                                          ((4096, 2000), False)])
def test_softmax_chain_fuses(ectx, shape, across):
    g = dvm.Graph(ectx)
    CP.softmax(g, g.input(TD(1 << 36, "bf16", shape)), out=TD(2 << 36, "bf16", shape))
    p = g.flush()
    hs = handlers(p)
    assert hs.count(HD_SOFTMAX) == 1 and not any(HD_RED <= h < HD_REDX + 9 for h in hs), hs
    assert (p.header()["g"] > 64) == across
    # one softmax per tile across waves: its buffer pair alternates with the
    # tile parity instead of an end-of-body barrier
    assert bool(p.words()[H_FLAGS] & HF_RED_ALT) == across and HD_SYNC not in hs
    assert p.verify() is None


def test_softmax_with_a_stored_max_stays_unfused(ectx):
    g = dvm.Graph(ectx)
    shape = (4096, 6484)
    x = g.input(TD(1 << 36, "f32", shape))
    with g.group():
        m = g.op("reduce_max", x, out=TD(3 << 36, "f32", (4096, 1)), live=True)
        d = g.op("sub", x, m)
        e = g.op("exp", d)
        s = g.op("reduce_sum", e)
        g.op("div", e, s, out=TD(2 << 36, "f32", shape), live=True)
        g.release(d, e, s)
    p = g.flush()
    hs = handlers(p)
    assert HD_SOFTMAX not in hs and sum(HD_REDX <= h < HD_REDX + 9 for h in hs) == 2
    assert p.verify() is None


@pytest.mark.parametrize("n_after", [1, 6, 7])
def test_softmax_then_row_sums_fences_buffers(ectx, n_after):
    """A fused softmax (buffer pair 0, 1) followed by n_after row sums of its
    output (buffers 2, 3, ...): the last reduction shares a buffer with the
    next tile's softmax only when the buffers wrap round (n_after = 7 ends in
    buffer 0: a closing barrier); otherwise no barrier and no alternation."""
    g = dvm.Graph(ectx)
    shape = (4096, 6484)
    x = g.input(TD(1 << 36, "f32", shape))
    y = CP.softmax(g, x)
    v = y
    for k in range(n_after):
        s = g.op("reduce_sum", v)
        last = k == n_after - 1
        nv = g.op("sub", v, s, out=TD(2 << 36, "f32", shape) if last else None, live=last)
        g.release(s)
        if k:
            g.release(v)
        v = nv
    g.release(y)
    p = g.flush()
    hs = handlers(p)
    assert hs.count(HD_SOFTMAX) == 1
    assert sum(HD_REDX <= h < HD_REDX + 9 for h in hs) == n_after
    assert not (p.words()[H_FLAGS] & HF_RED_ALT)
    assert (hs[-1] == HD_SYNC) == (n_after == 7)
    assert p.verify() is None

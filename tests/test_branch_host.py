"""Host tests (no GPU) of branch programs: device-side if-else, where the VM
reads the condition and picks one of two bodies (the dynamic control-flow
workload of the DVM review page, section 6.2).

Header offsets, flag bits and handler ids are the bytecode format of
csrc/bytecode.h, restated here to read encoded programs.
"""
import struct

import pytest

import device_bytecode_vm_amd as dvm
from device_bytecode_vm_amd import TensorDesc as TD
from device_bytecode_vm_amd import _lib as L

H_NARGS, H_PRO_BEGIN, H_PRO_END, H_BODY_BEGIN, H_BODY_END, H_FLAGS = 13, 14, 15, 16, 17, 26
H_COND_ARG, H_COND_THR, H_ALT_BEGIN, H_ALT_END = 40, 41, 42, 43
ARG_BASE, ARG_WORDS, HF_BRANCH = 44, 8, 2
HD_BIN_MEM = 156   # ACC <- ACC (op) memory operand; the ALU op in bits [23:20] (add 0, sub 1)


@pytest.fixture(scope="module")
def ectx():
    return dvm.Context(-1)


def if_else(ectx, shape=(4096, 4096), then_op="add", else_op="sub", else_out=None, thr=0.0):
    g = dvm.Graph(ectx)
    x = g.input(TD(1 << 34, "f32", shape))
    y = g.input(TD(2 << 34, "f32", shape))
    s = g.op("reduce_sum", x, out=TD(3 << 34, "f32", ()), live=True, axis=L.AXIS_ALL)
    g.begin_branch(s, thr)
    g.op(then_op, x, y, out=TD(4 << 34, "f32", shape), live=True)
    g.else_branch()
    g.op(else_op, x, y, out=else_out or TD(4 << 34, "f32", shape), live=True)
    g.end_branch()
    return g


def test_branch_program_layout(ectx):
    g = if_else(ectx, thr=0.5)
    red = g.take_program()
    assert red.header()["tmpl"] == 2          # the reduce-all ran first
    p = g.take_program()
    assert g.take_program() is None
    w = p.words()
    assert w[H_FLAGS] & HF_BRANCH
    n = w[H_NARGS]
    assert w[H_COND_ARG] == n - 1
    c = ARG_BASE + (n - 1) * ARG_WORDS
    assert (w[c] | w[c + 1] << 32) == 3 << 34   # the condition operand is the reduce-all's output
    assert struct.unpack("<f", struct.pack("<I", w[H_COND_THR]))[0] == 0.5
    assert w[H_PRO_END] == w[H_BODY_BEGIN] and w[H_BODY_END] == w[H_ALT_BEGIN] and w[H_ALT_END] > w[H_ALT_BEGIN]
    then_ops = [(w[i] & 0xFF, (w[i] >> 20) & 0xF) for i in range(w[H_BODY_BEGIN], w[H_BODY_END], 2)]
    else_ops = [(w[i] & 0xFF, (w[i] >> 20) & 0xF) for i in range(w[H_ALT_BEGIN], w[H_ALT_END], 2)]
    assert (HD_BIN_MEM, 0) in then_ops and (HD_BIN_MEM, 1) in else_ops   # x + y, x - y
    assert [h for h, _ in then_ops] == [h for h, _ in else_ops]
    log = g.flush_log()
    assert log[-1] == (2, "branch")


def test_branch_refusals(ectx):
    # bodies that write different tensors do not share one operand table
    g = dvm.Graph(ectx)
    x = g.input(TD(1 << 34, "f32", (64, 64)))
    y = g.input(TD(2 << 34, "f32", (64, 64)))
    s = g.op("reduce_sum", x, out=TD(3 << 34, "f32", ()), live=True, axis=L.AXIS_ALL)
    g.begin_branch(s)
    t = g.op("add", x, y, out=TD(4 << 34, "f32", (64, 64)), live=True)
    g.else_branch()
    u = g.op("sub", x, y, out=TD(5 << 34, "f32", (64, 64)), live=True)
    with pytest.raises(dvm.DvmError) as e:
        g.end_branch()
    assert e.value.status == L.ERR_UNSUPPORTED
    with pytest.raises(dvm.DvmError):
        g.op("neg", t, out=TD(6 << 34, "f32", (64, 64)))      # lost with the refused branch
    # an empty else-body
    g.begin_branch(s)
    g.op("add", x, y, out=TD(4 << 34, "f32", (64, 64)), live=True)
    g.else_branch()
    with pytest.raises(dvm.DvmError) as e:
        g.end_branch()
    assert e.value.status == L.ERR_UNSUPPORTED
    # the condition must be one fp32 value
    with pytest.raises(dvm.DvmError) as e:
        g.begin_branch(x)
    assert e.value.status == L.ERR_INVALID_ARG
    # no flush or group while a branch is open
    g.begin_branch(s)
    with pytest.raises(dvm.DvmError):
        g.flush()
    with pytest.raises(dvm.DvmError):
        with g.group():
            pass
    g.op("add", x, y, out=TD(4 << 34, "f32", (64, 64)), live=True)
    g.else_branch()
    g.op("sub", x, y, out=TD(4 << 34, "f32", (64, 64)), live=True)
    g.end_branch()


def test_branch_on_its_own_reduce_all(ectx):
    """begin_branch_reduce adds the reduce-all and opens the branch on it: the
    same two programs as a reduce_sum op followed by begin_branch (an
    encode-only context launches nothing, so no combine is held and the branch
    reads the condition from memory)."""
    shape = (4096, 4096)
    g = dvm.Graph(ectx)
    x = g.input(TD(1 << 34, "f32", shape))
    y = g.input(TD(2 << 34, "f32", shape))
    s = g.begin_branch_reduce(x, TD(3 << 34, "f32", ()), 0.5)
    assert s.shape == () and s.dtype == "f32"
    g.op("add", x, y, out=TD(4 << 34, "f32", shape), live=True)
    g.else_branch()
    g.op("sub", x, y, out=TD(4 << 34, "f32", shape), live=True)
    g.end_branch()
    red, br = g.take_program(), g.take_program()
    ref = if_else(ectx, thr=0.5)
    assert red.words() == ref.take_program().words()
    assert br.words() == ref.take_program().words()
    assert not br.words()[H_FLAGS] & 16        # HF_COND_FOLD: only on a device


def test_branch_on_its_own_reduce_all_refusals(ectx):
    g = dvm.Graph(ectx)
    x = g.input(TD(1 << 34, "f32", (64, 64)))
    y = g.input(TD(2 << 34, "f32", (64, 64)))
    for out, kind in [(TD(3 << 34, "f32", (1,)), "sum"), (TD(3 << 34, "bf16", ()), "sum")]:
        with pytest.raises(dvm.DvmError) as e:
            g.begin_branch_reduce(x, out, 0.0, kind)
        assert e.value.status == L.ERR_INVALID_ARG
    # after a refusal no branch is open; a max reduce-all works
    s = g.begin_branch_reduce(x, TD(3 << 34, "f32", ()), 0.0, "max")
    with pytest.raises(dvm.DvmError):
        g.begin_branch_reduce(x, TD(5 << 34, "f32", ()), 0.0)   # a branch is open
    g.op("add", x, y, out=TD(4 << 34, "f32", (64, 64)), live=True)
    g.else_branch()
    g.op("sub", x, y, out=TD(4 << 34, "f32", (64, 64)), live=True)
    g.end_branch()
    red = g.take_program()
    assert red.header()["tmpl"] == 2
    assert g.take_program().words()[H_FLAGS] & HF_BRANCH

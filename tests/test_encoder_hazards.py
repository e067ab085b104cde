"""Host tests (no GPU) of two encoder/fuser guarantees:

* the barrier that keeps a tile's cross-wave reduction buffers from being
  overwritten by the next tile while a wave still reads them (the syncs the
  encoder inserts, DVM review page, section 4.3);
* a failed flush drops the group that triggered it: its values are lost, not
  pending, and cannot feed later ops.

The handler ids and header word offsets below are the bytecode format of
csrc/bytecode.h, restated here to read encoded programs.
"""
import pytest

import device_bytecode_vm_amd as dvm
from device_bytecode_vm_amd import TensorDesc as TD
from device_bytecode_vm_amd import _lib as L

H_BODY_BEGIN, H_BODY_END, H_FLAGS = 16, 17, 26
HD_REDX, HD_SYNC = 127, 149
HF_RED_ALT = 8
N_LDSBUF = 8


@pytest.fixture(scope="module")
def ectx():
    return dvm.Context(-1)


def body(p):
    w = p.words()
    b0, b1 = w[H_BODY_BEGIN], w[H_BODY_END]
    return [(w[i] & 0xFF, (w[i] >> 16) & 0xF) for i in range(b0, b1, 2)]


def chained_reductions(ectx, n_red, shape):
    """x -> (x - rowsum(x)) repeated n_red times: n_red reductions whose rows
    span several waves (one REDX each)."""
    g = dvm.Graph(ectx)
    addr = 1 << 30
    v = g.input(TD(addr, "f32", shape))
    for k in range(n_red):
        s = g.op("reduce_sum", v)
        last = k == n_red - 1
        nv = g.op("sub", v, s, out=TD(addr * 2, "f32", shape) if last else None, live=last)
        g.release(s)
        if k:
            g.release(v)
        v = nv
    return g.flush()


def fenced(instrs, n_tiles=3, alt=False):
    """Simulates n_tiles copies of the body and checks every write of a
    cross-wave buffer against the reads of the same buffer since the last
    barrier: a write may only follow reads that a barrier separates from it.
    REDX = write, barrier, read (reduce-alls keep their partials in registers).
    alt: the workgroup's odd tiles use buffer b ^ 2 (HF_RED_ALT)."""
    reads_since_barrier = set()
    for t in range(n_tiles):
        for h, b in instrs:
            b = b ^ (2 * (t & 1)) if alt else b
            if HD_REDX <= h < HD_REDX + 9:
                if b in reads_since_barrier:
                    return False
                reads_since_barrier = {b}          # its own barrier, then its read
            elif h == HD_SYNC:
                reads_since_barrier = set()
    return True


@pytest.mark.parametrize("n_red", [1, 2, 8, 9, 10, 16, 17])
@pytest.mark.parametrize("shape", [(4096, 6000), (4096, 16384)])
def test_trailing_sync_fences_buffer_reuse(ectx, n_red, shape):
    p = chained_reductions(ectx, n_red, shape)
    h = p.header()
    assert h["body_tile"] > 1 and h["g"] > 64, h   # several tiles per workgroup, rows across waves
    ins = body(p)
    redx = [b for op, b in ins if HD_REDX <= op < HD_REDX + 9]
    assert redx == [k % N_LDSBUF for k in range(n_red)]
    alt = bool(p.words()[H_FLAGS] & HF_RED_ALT)
    assert alt == (n_red == 1)
    assert fenced(ins, alt=alt)
    trailing = ins[-1][0] == HD_SYNC
    # one reduction per tile: buffers alternate instead of a trailing barrier
    assert trailing == ((n_red - 1) % N_LDSBUF == 0 and n_red > 1)
    if n_red == 1:
        assert not fenced(ins, alt=False)    # without the alternation the body would race


def test_failed_flush_drops_the_new_group(ectx):
    g = dvm.Graph(ectx)
    a = g.input(TD(1 << 20, "f32", (4, 5)))
    g.op("exp", a)                                  # no storage and never released: its flush fails
    b = g.input(TD(2 << 20, "f32", (3, 7)))
    held = {}
    with pytest.raises(dvm.DvmError) as e:
        with g.group():                             # another shape: flushes the first graph first
            held["c"] = g.op("neg", b, out=TD(3 << 20, "f32", (3, 7)))
    assert e.value.status == L.ERR_INVALID_ARG
    # the group that triggered the failing flush was dropped with it: the
    # value it would have produced holds nothing and cannot be read
    with pytest.raises(dvm.DvmError) as e:
        g.op("mul", held["c"], 2.0, out=TD(4 << 20, "f32", (3, 7)), live=True)
    assert e.value.status == L.ERR_INVALID_ARG
    assert g.flush() is None                        # nothing pending


def test_reduce_all_program_has_no_scratch_address(ectx):
    """The reduce-all closes its graph; the encode-only context holds the
    program.  Its scratch operand has no address: each launch supplies its
    stream's own area, so programs on different streams never share it."""
    ARG_BASE, ARG_WORDS, H_ALL_SCRATCH = 44, 8, 24
    g = dvm.Graph(ectx)
    x = g.input(TD(1 << 30, "f32", (16384, 4096)))
    g.op("reduce_sum", x, out=TD(2 << 30, "f32", ()), live=True, axis=L.AXIS_ALL)
    assert g.flush() is None                         # the reduce-all flushed its own graph
    p = g.take_program()
    assert g.take_program() is None
    w = p.words()
    h = p.header()
    assert h["tmpl"] == 2 and h["body_tile"] > 1
    a = ARG_BASE + w[H_ALL_SCRATCH] * ARG_WORDS
    assert w[a] == 0 and w[a + 1] == 0               # supplied per stream at launch
    assert w[a + 7] == 256 + 4 * h["grid"]           # the bytes the program needs: one partial per workgroup


HD_LD_PF16 = 10


def ld_pf_waits(p):
    """(handler, wait count) of every prefetch read in the body: the count
    sits in the a (low 4 bits) and sub (high 4 bits) fields."""
    w = p.words()
    out = []
    for i in range(w[H_BODY_BEGIN], w[H_BODY_END], 2):
        h = w[i] & 0xFF
        if HD_LD_PF16 <= h < HD_LD_PF16 + 6:
            out.append((h, ((w[i] >> 12) & 0xF) | (((w[i] >> 20) & 0xF) << 4)))
    return out


@pytest.mark.parametrize("kind", ["softmax", "layernorm"])
def test_prefetch_wait_counts(ectx, kind):
    """The wait before a prefetch read counts the vector-memory instructions
    issued after that prefetch: the previous tile's instructions after its
    refill plus this tile's before the read (a workgroup's first tile waits
    for the whole prologue instead).  Softmax over rows of 6484 bf16 (wide
    build, nv = 7): the body is prefetch read (its refill issues 7), softmax,
    store (7 chunks), so the count is the 7 stores.  LayerNorm over 5120
    (nv = 10): read, reductions, scale-and-shift, store (10), count 10.  A
    larger count would let the read overtake its data."""
    from device_bytecode_vm_amd import composites as CP
    g = dvm.Graph(ectx)
    if kind == "softmax":
        CP.softmax(g, g.input(TD(1 << 36, "bf16", (139480, 6484))), out=TD(2 << 36, "bf16", (139480, 6484)))
        want = 7
    else:
        CP.layer_norm(g, g.input(TD(1 << 36, "bf16", (16384, 5120))), g.input(TD(3 << 36, "f32", (5120,))),
                      g.input(TD(4 << 36, "f32", (5120,))), 1e-6, out=TD(2 << 36, "bf16", (16384, 5120)))
        want = 10
    p = g.flush()
    assert p.header()["body_tile"] > 1
    assert [n for _, n in ld_pf_waits(p)] == [want]

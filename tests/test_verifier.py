"""The bytecode verifier (dvm_program_verify), on the host.

* Seeded random graphs -- elementwise chains, row reductions, reduce-alls,
  broadcast and transposed operands, bf16 / fp32 / u8, ragged shapes, both VM
  builds, branch programs and stacked programs -- encode to programs the
  verifier accepts.
* Defects planted in copies of valid programs' words (on the CPU; such
  programs are never launched) are each reported: a removed end-of-body
  barrier, a read of an unwritten register, a prefetch slot never refilled,
  an operand index outside the table, a wrong tile count, a wide program
  naming a second tile register, a bad stack directory.

Word offsets and handler ids are the bytecode format of csrc/bytecode.h,
restated here to plant the defects.
"""
import numpy as np
import pytest

import device_bytecode_vm_amd as dvm
from device_bytecode_vm_amd import TensorDesc as TD
from device_bytecode_vm_amd import _lib as L
from device_bytecode_vm_amd import composites as CP

H_KTYPE, H_BLOCK_DIM, H_BODY_BEGIN, H_BODY_END = 2, 4, 16, 17
HD_COPY, HD_SYNC, HD_LD_PF16 = 28, 149, 10
FL_ISSUE = 4
S_DIR = 2


@pytest.fixture(scope="module")
def ectx():
    return dvm.Context(-1)


class Addr:
    k = 0

    def __call__(self):
        Addr.k += 1
        return Addr.k << 38


A = Addr()


def drain(g):
    out = []
    while True:
        p = g.take_program()
        if p is None:
            return out
        out.append(p)


def random_graph(g, rg):
    """One random fused group on g (encode-only tensors)."""
    kind = int(rg.integers(0, 6))
    R = int(rg.choice([1, 3, 17, 300, 1025, 4096, 20000]))
    Cc = int(rg.choice([1, 7, 64, 513, 1031, 5120, 6484, 17408]))
    dt = str(rg.choice(["f32", "bf16"]))
    odt = str(rg.choice(["f32", "bf16"]))
    if kind == 0:       # elementwise chain with a broadcast row and a scalar
        x = g.input(TD(A(), dt, (R, Cc)))
        b = g.input(TD(A(), "f32", (Cc,)))
        t = g.op(str(rg.choice(["add", "mul", "max", "sub"])), x, b)
        u = g.op(str(rg.choice(["exp", "sqrt", "abs", "neg"])), t)
        v = g.op("mul", u, float(rg.normal()), out=TD(A(), odt, (R, Cc)), live=True)
        g.release(t, u)
    elif kind == 1:     # LayerNorm / RMSNorm / softmax composites
        x = g.input(TD(A(), dt, (R, Cc)))
        c = int(rg.integers(0, 3))
        if c == 0:
            CP.layer_norm(g, x, g.input(TD(A(), "f32", (Cc,))), g.input(TD(A(), "f32", (Cc,))), 1e-6,
                          out=TD(A(), odt, (R, Cc)))
        elif c == 1:
            CP.rms_norm(g, x, g.input(TD(A(), "f32", (Cc,))), 1e-6, out=TD(A(), odt, (R, Cc)))
        else:
            CP.softmax(g, x, out=TD(A(), odt, (R, Cc)))
    elif kind == 2:     # reduce-all
        x = g.input(TD(A(), dt, (R, Cc)))
        g.op(str(rg.choice(["reduce_sum", "reduce_max"])), x, out=TD(A(), "f32", ()), live=True, axis=L.AXIS_ALL)
    elif kind == 3:     # a transposed (strided) input
        x = g.input(TD(A(), "f32", (R, Cc), (1, R)))
        g.op("exp", x, out=TD(A(), "f32", (R, Cc)), live=True)
    elif kind == 4:     # chained row reductions (cross-wave buffers reused)
        v = g.input(TD(A(), "f32", (R, Cc)))
        n = int(rg.integers(1, 12))
        for k in range(n):
            s = g.op("reduce_sum", v)
            last = k == n - 1
            nv = g.op("sub", v, s, out=TD(A(), "f32", (R, Cc)) if last else None, live=last)
            g.release(s)
            if k:
                g.release(v)
            v = nv
    else:               # SwiGLU (fused SiLU) with a u8 side output
        a = g.input(TD(A(), "bf16", (R, Cc)))
        b = g.input(TD(A(), "bf16", (R, Cc)))
        y = CP.swiglu(g, a, b, out=TD(A(), "bf16", (R, Cc)))
        g.op("isfinite", y, out=TD(A(), "u8", (R, Cc)), live=True)


def test_random_programs_verify(ectx):
    rg = np.random.default_rng(2026)
    n_prog = 0
    for trial in range(30):
        g = dvm.Graph(ectx)
        g.set_stacking(int(rg.choice([1, 3, 7])))
        for _ in range(int(rg.integers(1, 8))):
            try:
                random_graph(g, rg)
            except dvm.DvmError as e:
                assert e.status in (L.ERR_UNSUPPORTED, L.ERR_RESOURCE), e
        g.flush_launch()
        for p in drain(g):
            msg = p.verify()
            assert msg is None, f"trial {trial}: {msg} (header {p.header()})"
            n_prog += 1
    assert n_prog > 60


def test_branch_and_matmul_programs_verify(ectx):
    g = dvm.Graph(ectx)
    x = g.input(TD(A(), "f32", (3000, 4096)))
    y = g.input(TD(A(), "f32", (3000, 4096)))
    s = g.op("reduce_sum", x, out=TD(A(), "f32", ()), live=True, axis=L.AXIS_ALL)
    out = TD(A(), "f32", (3000, 4096))
    g.begin_branch(s)
    g.op("add", x, y, out=out, live=True)
    g.else_branch()
    g.op("sub", x, y, out=out, live=True)
    g.end_branch()
    progs = drain(g)
    assert len(progs) == 2 and all(p.verify() is None for p in progs)
    g2 = dvm.Graph(ectx)
    CP.matmul_bias_silu(g2, g2.input(TD(A(), "bf16", (1000, 5120))), g2.input(TD(A(), "bf16", (5120, 17408))),
                        g2.input(TD(A(), "f32", (17408,))), out=TD(A(), "bf16", (1000, 17408)))
    assert g2.flush().verify() is None


def planted(p, edit):
    w = p.words()
    edit(w)
    return dvm.Program.from_words(w)


def layernorm_prog(ectx, rows=20000):
    g = dvm.Graph(ectx)
    CP.layer_norm(g, g.input(TD(A(), "bf16", (rows, 5120))), g.input(TD(A(), "f32", (5120,))),
                  g.input(TD(A(), "f32", (5120,))), 1e-6, out=TD(A(), "bf16", (rows, 5120)))
    return g.flush()


def test_planted_defects_are_reported(ectx):
    # a removed end-of-body barrier after 9 cross-wave reductions
    g = dvm.Graph(ectx)
    v = g.input(TD(A(), "f32", (4096, 6000)))
    for k in range(9):
        s = g.op("reduce_sum", v)
        last = k == 8
        nv = g.op("sub", v, s, out=TD(A(), "f32", (4096, 6000)) if last else None, live=last)
        g.release(s)
        if k:
            g.release(v)
        v = nv
    p = g.flush()
    assert p.verify() is None
    w = p.words()
    assert w[w[H_BODY_END] - 2] & 0xFF == HD_SYNC

    def drop_sync(w):
        w[H_BODY_END] -= 2
    msg = planted(p, drop_sync).verify()
    assert msg and "barrier" in msg

    # a read of a register no instruction of the tile wrote
    q = layernorm_prog(ectx, 300)
    assert q.verify() is None

    def read_unwritten(w):
        b = w[H_BODY_BEGIN]
        w[b] = (w[b] & ~0xFF) | (HD_COPY + 3 * 0 + 2)   # ACC <- register 2 before anything wrote it
    msg = planted(q, read_unwritten).verify()
    assert msg and "not written" in msg

    # a prefetch slot the body never refills
    ln = layernorm_prog(ectx)
    ww = ln.words()
    pf = [i for i in range(ww[H_BODY_BEGIN], ww[H_BODY_END], 2) if (ww[i] >> 28) & FL_ISSUE]
    assert pf, "the LayerNorm body refills a prefetch slot"

    def no_refill(w):
        w[pf[0]] &= ~(FL_ISSUE << 28)
    msg = planted(ln, no_refill).verify()
    assert msg and "refill" in msg

    # an operand index outside the table
    def bad_operand(w):
        for i in range(w[H_BODY_BEGIN], w[H_BODY_END], 2):
            if (w[i] & 0xFF) in (22, 23):          # the store
                w[i + 1] = 31
    msg = planted(ln, bad_operand).verify()
    assert msg and "outside the table" in msg

    # a tile count that does not follow from the shape
    def bad_count(w):
        w[H_BLOCK_DIM] += 1
    msg = planted(ln, bad_count).verify()
    assert msg and "block_dim" in msg

    # a wide program naming tile register 1
    assert ln.header()["kernel_type"] == 2

    def second_register(w):
        b = w[H_BODY_BEGIN]
        w[b] = (w[b] & ~0xFF) | (HD_LD_PF16 + 1)
    msg = planted(ln, second_register).verify()
    assert msg and "outside the build" in msg


def test_planted_stack_directory_defect(ectx):
    g = dvm.Graph(ectx)
    g.set_stacking(3)
    for r in (3000, 5000, 7000):
        CP.layer_norm(g, g.input(TD(A(), "bf16", (r, 5120))), g.input(TD(A(), "f32", (5120,))),
                      g.input(TD(A(), "f32", (5120,))), 1e-6, out=TD(A(), "bf16", (r, 5120)))
    g.flush_launch()
    (p,) = drain(g)
    assert p.header()["segments"] == 3 and p.verify() is None

    def bad_first(w):
        w[S_DIR + 3] += 1                            # segment 1's first workgroup
    msg = planted(p, bad_first).verify()
    assert msg and "directory" in msg


def test_planted_temporal_directory_defect(ectx):
    g = dvm.Graph(ectx)
    g.set_stacking(3, temporal=True)
    for r in (3000, 5000, 7000):
        CP.layer_norm(g, g.input(TD(A(), "bf16", (r, 5120))), g.input(TD(A(), "f32", (5120,))),
                      g.input(TD(A(), "f32", (5120,))), 1e-6, out=TD(A(), "bf16", (r, 5120)))
    g.flush_launch()
    (p,) = drain(g)
    assert p.header()["segments"] == 3 and p.verify() is None

    def bad_base(w):
        w[S_DIR + 5] += 1                            # segment 2's first tile
    msg = planted(p, bad_base).verify()
    assert msg and "first tile" in msg


def test_operand_reuse_fuzz_verifies(ectx):
    """Random fused groups whose ops reuse operands and intermediates (the
    case where one staged operand is read several times per tile)."""
    rg = np.random.default_rng(7)
    n_prog = 0
    for trial in range(900):
        g = dvm.Graph(ectx)
        R = int(rg.choice([5, 300, 4096, 20000]))
        Cc = int(rg.choice([512, 1031, 5120]))
        vals = [g.input(TD(A(), str(rg.choice(["f32", "bf16"])), (R, Cc))) for _ in range(int(rg.integers(1, 4)))]
        n_in, rows = len(vals), []
        try:
            with g.group():
                for _ in range(int(rg.integers(2, 14))):
                    r = rg.random()
                    pick = lambda: vals[int(rg.integers(0, len(vals)))]   # noqa: E731
                    if r < 0.55:
                        v = g.op(str(rg.choice(["add", "mul", "sub", "max", "div"])), pick(), pick())
                    elif r < 0.7:
                        v = g.op(str(rg.choice(["exp", "neg", "abs"])), pick())
                    elif r < 0.85:
                        s = g.op(str(rg.choice(["reduce_sum", "reduce_max"])), pick())
                        rows.append(s)
                        v = g.op("sub", pick(), s)
                    else:
                        v = g.op("mul", pick(), float(rg.normal()))
                    vals.append(v)
                g.op("add", vals[-1], vals[int(rg.integers(0, len(vals)))], out=TD(A(), "f32", (R, Cc)), live=True)
                for v in vals[n_in:] + rows:
                    g.release(v)
            p = g.flush()
        except dvm.DvmError as e:
            assert e.status in (L.ERR_UNSUPPORTED, L.ERR_RESOURCE, L.ERR_SHAPE), e
            continue
        if p is None:
            continue
        msg = p.verify()
        assert msg is None, f"trial {trial}: {msg}"
        n_prog += 1
    assert n_prog > 120


def test_planted_missing_buffer_alternation(ectx):
    """A row sum whose rows span waves has one cross-wave reduction per
    tile: its buffers alternate by tile parity (HF_RED_ALT) instead of an
    end-of-body barrier.  With the flag cleared the next tile's write races
    the last reads."""
    H_FLAGS, HF_RED_ALT = 26, 8
    g = dvm.Graph(ectx)
    shape = (4096, 6000)
    x = g.input(TD(A(), "f32", shape))
    s = g.op("reduce_sum", x)
    g.op("sub", x, s, out=TD(A(), "f32", shape), live=True)
    g.release(s)
    p = g.flush()
    assert p.header()["g"] > 64 and p.header()["body_tile"] > 1
    w = p.words()
    assert w[H_FLAGS] & HF_RED_ALT and w[w[H_BODY_END] - 2] & 0xFF != HD_SYNC
    assert p.verify() is None

    def clear_alt(w):
        w[H_FLAGS] &= ~HF_RED_ALT
    msg = planted(p, clear_alt).verify()
    assert msg and "before every wave read it" in msg


def test_reduce_all_body_and_planted_second_all(ectx):
    """A reduce-all body folds its operand into the lanes' running partials:
    one ALL instruction, no cross-wave buffer and no barrier per tile (the
    workgroup's partial and the final combine are the VM's epilogue).  A
    second ALL, or one of the other kind, is rejected."""
    H_FLAGS, H_ALL_KIND = 26, 22
    HD_ALL = 136
    g = dvm.Graph(ectx)
    g.op("reduce_sum", g.input(TD(A(), "f32", (16384, 4096))), out=TD(A(), "f32", ()), live=True, axis=L.AXIS_ALL)
    (p,) = drain(g)
    w = p.words()
    hs = [w[i] & 0xFF for i in range(w[H_BODY_BEGIN], w[H_BODY_END], 2)]
    assert sum(HD_ALL <= h < HD_ALL + 6 for h in hs) == 1 and HD_SYNC not in hs
    assert not (w[H_FLAGS] & 8)
    assert p.verify() is None

    def other_kind(w):
        w[H_ALL_KIND] = 1
    msg = planted(p, other_kind).verify()
    assert msg and "reduce-all instructions" in msg


def test_planted_lds_area_overlap(ectx):
    """Staging areas must be disjoint: a prefetch slot moved onto the
    cross-wave reduction buffers, or reduction buffers past the dynamic LDS,
    are rejected."""
    H_LDS_BYTES, H_PF_OFF0, H_RED_OFF = 27, 28, 39
    g = dvm.Graph(ectx)
    shape = (4096, 6000)
    x = g.input(TD(A(), "f32", shape))
    s = g.op("reduce_sum", x)
    g.op("sub", x, s, out=TD(A(), "f32", shape), live=True)
    g.release(s)
    p = g.flush()
    w = p.words()
    hs = [w[i] & 0xFF for i in range(w[14], w[15], 2)]
    assert 154 in hs and w[H_RED_OFF] > 0           # a prefetch slot and the reduction area
    assert p.verify() is None

    def onto_red(w):
        w[H_PF_OFF0] = w[H_RED_OFF]
    msg = planted(p, onto_red).verify()
    assert msg and ("overlap" in msg or "outside the dynamic LDS" in msg), msg

    def red_past_end(w):
        w[H_RED_OFF] = w[H_LDS_BYTES] - 8
    msg = planted(p, red_past_end).verify()
    assert msg and "reduction buffers outside the dynamic LDS" in msg, msg

"""Host-side tests of the C ABI (no GPU): the library loads and exports every
function include/dvm.h declares; errors come back as status codes; the
encoder's tiling equals the oracle's; the fuser's partition equals the
oracle's on seeded op streams."""
import ctypes
import os
import re

import numpy as np
import pytest

import device_bytecode_vm_amd as dvm
from device_bytecode_vm_amd import TensorDesc as TD
from device_bytecode_vm_amd import _lib as L
from device_bytecode_vm_amd import composites as CP
from oracle import tiling as TL
from oracle.fusion import Stream

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dvm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dvm_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 20
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)


@pytest.fixture(scope="module")
def ectx():
    return dvm.Context(-1)


def test_error_paths(ectx):
    g = dvm.Graph(ectx)
    a = g.input(TD(1 << 20, "f32", (4, 5)))
    b = g.input(TD(2 << 20, "f32", (3, 5)))
    with pytest.raises(dvm.DvmError) as e:
        g.op("add", a, b)                       # shapes do not broadcast
    assert e.value.status == L.ERR_SHAPE
    with pytest.raises(dvm.DvmError) as e:
        g.op("add", a, a, out=TD(3 << 20, "f32", (4, 4)))
    assert e.value.status == L.ERR_SHAPE
    with pytest.raises(dvm.DvmError) as e:
        g.op("isfinite", a, dtype="f32")
    assert e.value.status == L.ERR_UNSUPPORTED
    v = g.op("exp", a)                           # no storage, not released
    with pytest.raises(dvm.DvmError) as e:
        g.flush()
    assert e.value.status == L.ERR_INVALID_ARG
    with pytest.raises(dvm.DvmError) as e:
        g.op("neg", v)                           # its graph was flushed without storing it
    assert e.value.status == L.ERR_INVALID_ARG
    p = None
    g2 = dvm.Graph(ectx)
    x = g2.input(TD(1 << 20, "f32", (4, 5)))
    g2.op("exp", x, out=TD(2 << 20, "f32", (4, 5)), live=True)
    p = g2.flush()
    with pytest.raises(dvm.DvmError) as e:
        p.launch()                               # encode-only context
    assert e.value.status == L.ERR_DEVICE
    # an infeasible row reduce (rows wider than even a wide tile can hold:
    # 256 lanes x 10 chunks x 8 = 20480 columns) is unsupported
    g3 = dvm.Graph(ectx)
    y = g3.input(TD(1 << 20, "f32", (2, 20481)))
    with pytest.raises(dvm.DvmError) as e:
        g3.op("reduce_sum", y, out=TD(2 << 20, "f32", (2, 1)), live=True)
    assert e.value.status == L.ERR_UNSUPPORTED
    # rows up to that width run on the wide VM
    g4 = dvm.Graph(ectx)
    y = g4.input(TD(1 << 20, "f32", (2, 20480)))
    g4.op("reduce_sum", y, out=TD(2 << 20, "f32", (2, 1)), live=True)
    h = g4.flush().header()
    assert h["kernel_type"] == 2 and h["nv"] == 10 and h["g"] == 256


# ---------------------------------------------------------------------------
# encoder tiling vs oracle tiling
# ---------------------------------------------------------------------------
def dense(shape):
    st, acc = [], 1
    for d in reversed(shape):
        st.append(acc)
        acc *= d
    return tuple(reversed(st))


ESZ = {"f32": 4, "bf16": 2, "u8": 1}


def oracle_plan(tmpl, shape, operands, nv_max=TL.NV_MAX):
    """operands: list of (shape, strides, dtype, addr) over the dominant shape."""
    sts = []
    for sh, st, _, _ in operands:
        full = [0] * len(shape)
        off = len(shape) - len(sh)
        for i, (d, s) in enumerate(zip(sh, st)):
            full[off + i] = 0 if (d == 1 and shape[off + i] != 1) else s
        sts.append(full)
    R, C, col = TL.collapse(tmpl, shape, sts)
    ops = [TL.Operand(ESZ[dt], sr, sc, addr % 16) for (_, _, dt, addr), (sr, sc) in zip(operands, col)]
    return TL.plan(tmpl, R, C, ops, nv_max)


def check_header(p, plan):
    h = p.header()
    assert (h["R"], h["C"], h["tr"], h["tc"], h["block_dim"], h["body_tile"], h["grid"], h["g"], h["nv"],
            h["p"], h["pad"]) == (plan.R, plan.C, plan.tr, plan.tc, plan.block_dim, plan.body_tile,
                                  plan.grid, plan.g, plan.nv, plan.P, plan.pad)


def test_encoder_tiling_equals_oracle_elementwise(ectx):
    rg = np.random.default_rng(11)
    for trial in range(150):
        nd = int(rg.integers(1, 4))
        shape = tuple(int(rg.integers(1, 300 if nd > 1 else 3_000_000)) for _ in range(nd))
        dt_in = ["f32", "bf16"][int(rg.integers(0, 2))]
        dt_out = ["f32", "bf16"][int(rg.integers(0, 2))]
        a_addr = (1 << 30) + int(rg.integers(0, 4)) * 2 * (int(rg.integers(0, 2)))
        bcast = int(rg.integers(0, 3))  # 0: same shape, 1: row-broadcast [C], 2: scalar
        b_shape = shape if bcast == 0 else (shape[-1:] if bcast == 1 else ())
        g = dvm.Graph(ectx)
        a = g.input(TD(a_addr, dt_in, shape))
        b = g.input(TD(2 << 30, "f32", b_shape))
        t = g.op("mul", a, b)
        g.op("exp", t, out=TD(3 << 30, dt_out, shape), live=True)
        g.release(t)
        p = g.flush()
        plan = oracle_plan(TL.ELEMWISE, shape, [(shape, dense(shape), dt_in, a_addr),
                                                (b_shape, dense(b_shape), "f32", 2 << 30),
                                                (shape, dense(shape), dt_out, 3 << 30)])
        check_header(p, plan)


def test_encoder_tiling_equals_oracle_rowreduce(ectx):
    rg = np.random.default_rng(12)
    for trial in range(150):
        rows = int(rg.integers(1, 200000))
        cols = int(rg.integers(1, 8193))
        lead = int(rg.integers(1, 5)) if rg.random() < 0.3 else None
        shape = (lead, rows, cols) if lead else (rows, cols)
        dt = ["f32", "bf16"][int(rg.integers(0, 2))]
        base = (1 << 32) + (int(rg.integers(0, 8)) * 2 if rg.random() < 0.3 else 0)
        g = dvm.Graph(ectx)
        x = g.input(TD(base, dt, shape))
        opnds = [(shape, dense(shape), dt, base), (shape, dense(shape), dt, 5 << 32)]
        plans = {}
        for nvm in (TL.NV_MAX, TL.NV_WIDE):
            try:
                plans[nvm] = oracle_plan(TL.ROWREDUCE, shape, opnds, nvm)
            except ValueError:
                plans[nvm] = None
        try:
            CP.softmax(g, x, out=TD(5 << 32, dt, shape))
        except dvm.DvmError as e:
            assert e.status == L.ERR_UNSUPPORTED
            assert plans[TL.NV_MAX] is None and plans[TL.NV_WIDE] is None
            continue
        p = g.flush()
        # softmax keeps its one tile value in the accumulator: the wide VM
        # whenever the standard plan is infeasible, or the wide plan holds
        # more rows per tile with the same staging of x or in one round
        p5, p10 = plans[TL.NV_MAX], plans[TL.NV_WIDE]
        esz = ESZ[dt]
        al = 2 if esz == 2 else 4   # vector accesses: bf16 element-aligned, fp32 dword-aligned
        vec = base % al == 0 and (len(shape) == 1 or (cols * esz) % al == 0)

        def staged(pl, budget, nvk):
            # a prefetch slot holds the tile's nv chunks per lane
            return pl.body_tile >= 2 and vec and pl.nv * 256 * 16 * (esz // 2) <= budget

        # the wide build's LDS budget is 80 KiB less its cross-wave reduction
        # buffers (144 bytes) when rows span waves; staging counts only where
        # a workgroup runs more than one tile
        wide = p5 is None or (p5.n_c == 1 and p10.tr > p5.tr and
                              (p10.body_tile == 1 or
                               staged(p10, 80 * 1024 - (144 if p10.g > 64 else 0), TL.NV_WIDE) >=
                               staged(p5, 76 * 1024, TL.NV_MAX)))
        assert p.header()["kernel_type"] == (2 if wide else 0), (shape, dt)
        check_header(p, p10 if wide else p5)


def test_encoder_layernorm_workload_headers(ectx):
    import workloads as W
    for r, h in W.layernorm_shapes(0, 64):
        g = dvm.Graph(ectx)
        x = g.input(TD(1 << 34, "bf16", (r, h)))
        gm = g.input(TD(2 << 34, "f32", (h,)))
        bt = g.input(TD(3 << 34, "f32", (h,)))
        CP.layer_norm(g, x, gm, bt, W.LN_EPS, out=TD(4 << 34, "bf16", (r, h)))
        p = g.flush()
        opnds = [((r, h), dense((r, h)), "bf16", 1 << 34), ((h,), (1,), "f32", 2 << 34),
                 ((h,), (1,), "f32", 3 << 34), ((r, h), dense((r, h)), "bf16", 4 << 34)]
        p5 = oracle_plan(TL.ROWREDUCE, (r, h), opnds)
        p10 = oracle_plan(TL.ROWREDUCE, (r, h), opnds, TL.NV_WIDE)

        def staged(pl, budget, nvk):
            # x prefetched (bf16), then gamma and beta held as one shared fp32
            # row; a prefetch slot holds the tile's nv chunks per lane, an
            # invariant slot the VM build's nvk
            if pl.body_tile < 2:
                return 0, 0
            off, pf, inv = 0, 0, 0
            for sz, kind in ((pl.nv * 256 * 16, "pf"), (nvk * pl.g * 32, "inv"), (nvk * pl.g * 32, "inv")):
                if off + sz <= budget:
                    off += sz
                    pf, inv = (pf + 1, inv) if kind == "pf" else (pf, inv + 1)
            return pf, inv

        s5 = staged(p5, 76 * 1024, TL.NV_MAX)
        s10 = staged(p10, 80 * 1024 - (144 if p10.g > 64 else 0), TL.NV_WIDE)
        wide = p5.n_c == 1 and p10.tr > p5.tr and (p10.body_tile == 1 or (s10[0] >= s5[0] and s10[1] >= s5[1]))
        assert p.header()["kernel_type"] == (2 if wide else 0), (r, h)
        check_header(p, p10 if wide else p5)


# ---------------------------------------------------------------------------
# fuser partition vs oracle partition
# ---------------------------------------------------------------------------
class Twin:
    """Drives the C++ fuser (encode-only) and the oracle simulator with the
    same stream of groups."""

    def __init__(self, ectx):
        self.g = dvm.Graph(ectx)
        self.events = []
        self.vals = {}      # name -> dvm Value
        self.shape = {}
        self.n = 0
        self.addr = 1 << 40

    def alloc(self, shape, dt):
        n = int(np.prod(shape)) if len(shape) else 1
        a = self.addr
        self.addr += ((n * ESZ[dt] + 4095) // 4096 + 1) * 4096
        return a

    def input(self, shape, dt):
        name = f"i{self.n}"
        self.n += 1
        a = self.alloc(shape, dt)
        self.vals[name] = self.g.input(TD(a, dt, shape))
        self.shape[name] = tuple(shape)
        self.events.append(("input", name, tuple(shape), dense(shape), dt, a))
        return name

    def group(self, ops, releases=()):
        """ops: list of (op, ins, out_name, shape, dtype, live, has_storage, axis)."""
        recs = []
        try:
            self._group(ops, releases, recs)
        except dvm.DvmError as e:
            if e.status != L.ERR_UNSUPPORTED:
                raise
        self.events.append(("group", recs))
        for r in releases:
            self.events.append(("release", r))

    def _group(self, ops, releases, recs):
        with self.g.group():
            for op, ins, out, shape, dt, live, store, axis in ops:
                args = [self.vals[x] if isinstance(x, str) else x for x in ins]
                addr = self.alloc(shape, dt) if store else None
                o = TD(addr, dt, shape) if store else None
                v = self.g.op(op, *args, out=o, dtype=dt, live=live, axis=axis)
                self.vals[out] = v
                self.shape[out] = tuple(shape)
                n = int(np.prod(shape)) if len(shape) else 1
                recs.append({"op": op, "in": list(ins), "out": out, "shape": tuple(shape), "dtype": dt,
                             "axis": None if axis == L.AXIS_ALL else -1, "live": live, "addr": addr,
                             "nbytes": n * ESZ[dt]})
            for r in releases:
                self.g.release(self.vals[r])

    def release(self, name):
        self.g.release(self.vals[name])
        self.events.append(("release", name))

    def flush(self):
        self.g.flush_launch()
        self.events.append(("flush",))


def random_stream(tw, rg, n_groups):
    shapes = [(int(rg.integers(1, 64)), int(rg.choice([64, 512, 5120, 3001])))]
    shapes.append((shapes[0][0], int(rg.choice([96, 17408]))))
    cur = {}
    for s in shapes:
        cur[s] = tw.input(s, "bf16")
    w = {s: tw.input((s[1],), "f32") for s in shapes}
    for k in range(n_groups):
        s = shapes[int(rg.integers(0, len(shapes)))]
        kind = int(rg.integers(0, 6))
        h = cur[s]
        t = f"t{k}"
        if kind == 0:     # residual add, output stored (h chain)
            r = tw.input(s, "bf16")
            tw.group([("add", [h, r], t, s, "bf16", False, True, -1)])
            tw.release(h)
            cur[s] = t
        elif kind == 1:   # rmsnorm group
            ops = [("mul", [h, h], t + "a", s, "f32", False, False, -1),
                   ("reduce_sum", [t + "a"], t + "b", s[:-1] + (1,), "f32", False, False, -1),
                   ("div", [t + "b", float(s[1])], t + "c", s[:-1] + (1,), "f32", False, False, -1),
                   ("sqrt", [t + "c"], t + "d", s[:-1] + (1,), "f32", False, False, -1),
                   ("div", [h, t + "d"], t + "e", s, "f32", False, False, -1),
                   ("mul", [t + "e", w[s]], t, s, "bf16", True, True, -1)]
            tw.group(ops, releases=[t + x for x in "abcde"])
        elif kind == 2:   # softmax group
            ops = [("reduce_max", [h], t + "a", s[:-1] + (1,), "f32", False, False, -1),
                   ("sub", [h, t + "a"], t + "b", s, "f32", False, False, -1),
                   ("exp", [t + "b"], t + "c", s, "f32", False, False, -1),
                   ("reduce_sum", [t + "c"], t + "d", s[:-1] + (1,), "f32", False, False, -1),
                   ("div", [t + "c", t + "d"], t, s, "bf16", True, True, -1)]
            tw.group(ops, releases=[t + x for x in "abcd"])
        elif kind == 3:   # elementwise chain on a stored value
            tw.group([("exp", [h], t, s, "f32", bool(rg.integers(0, 2)), True, -1)])
        elif kind == 4:   # reduce-all
            tw.group([("reduce_sum", [h], t, (), "f32", True, True, L.AXIS_ALL)])
        else:
            tw.flush()


def test_fuser_partition_equals_oracle(ectx):
    rg = np.random.default_rng(2024)
    for trial in range(25):
        tw = Twin(ectx)
        random_stream(tw, rg, int(rg.integers(5, 60)))
        tw.flush()
        sim = Stream()
        sim.run(tw.events)
        got = tw.g.flush_log()
        want = [(len(outs), why) for outs, why, _ in sim.graphs]
        assert got == want, f"trial {trial}"
        assert tw.g.stats()["unsupported"] == len(sim.unsupported)


def test_fuser_resource_split_matches_oracle(ectx):
    tw = Twin(ectx)
    x = tw.input((4, 512), "f32")
    prev = x
    for k in range(70):
        tw.group([("add", [prev, 1.0], f"v{k}", (4, 512), "f32", False, True, -1)])
        if prev != x:
            tw.release(prev)
        prev = f"v{k}"
    tw.flush()
    sim = Stream()
    sim.run(tw.events)
    assert tw.g.flush_log() == [(len(o), w) for o, w, _ in sim.graphs] == [(64, "resource"), (6, "explicit")]


def test_single_hip_runtime_in_process():
    """Importing the binding before torch must still leave one HIP runtime
    mapped in the process (libdvm.so binds to the one torch loads)."""
    import subprocess
    import sys
    code = ("import device_bytecode_vm_amd, torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "paths = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
            "print(len(paths)); print(paths)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr
    assert r.stdout.split("\n")[0] == "1", r.stdout


def test_matmul_header_matches_oracle_plan(dvm_lib):
    """Encode-only MatMul+bias+SiLU graphs: the MIX header equals the oracle's
    MATMUL plan (tile, tile counts, body_tile, grid)."""
    from device_bytecode_vm_amd import composites as CP
    from oracle import tiling as TL
    dvm = dvm_lib
    ctx = dvm.Context(-1)
    for (m, k, n) in [(1, 5120, 17408), (300, 136, 1000), (8192, 5120, 17408), (129, 64, 8)]:
        g = dvm.Graph(ctx)
        a = g.input(dvm.TensorDesc(0x10000000, "bf16", (m, k)))
        b = g.input(dvm.TensorDesc(0x20000000, "bf16", (k, n)))
        bias = g.input(dvm.TensorDesc(0x30000000, "f32", (n,)))
        CP.matmul_bias_silu(g, a, b, bias, out=dvm.TensorDesc(0x40000000, "bf16", (m, n)))
        h = g.flush().header()
        p = TL.plan_matmul(m, n, k, 2, 2, [TL.Operand(4, 0, 1), TL.Operand(2, n, 1)])
        assert h["kernel_type"] == 1 and h["tmpl"] == 3
        assert (h["tr"], h["tc"], h["block_dim"], h["body_tile"], h["grid"]) == \
            (p.tr, p.tc, p.block_dim, p.body_tile, p.grid), (m, k, n)


def test_matmul_unsupported_forms(dvm_lib):
    """Operands outside the MIX kernel's forms are refused at add time."""
    dvm = dvm_lib
    ctx = dvm.Context(-1)
    cases = [((4, 7), (7, 16), "bf16"),      # K not a multiple of 8
             ((4, 16), (16, 12), "bf16"),    # N not a multiple of 8
             ((4, 16), (16, 16), "f32")]     # fp32 inputs
    for sa, sb, dt in cases:
        g = dvm.Graph(ctx)
        a = g.input(dvm.TensorDesc(0x10000000, dt, sa))
        b = g.input(dvm.TensorDesc(0x20000000, dt, sb))
        with pytest.raises(dvm.DvmError) as ei:
            g.op("matmul", a, b, dtype="f32")
        assert ei.value.status == 2, (sa, sb, dt)

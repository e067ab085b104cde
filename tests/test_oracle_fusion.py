"""Pins for oracle/fusion.py: hand-built op streams whose partitions follow
from the rules by hand (no GPU)."""
import numpy as np

from oracle.fusion import Stream
from oracle.graph import evaluate

MB = 1 << 20


def dense(shape):
    st, acc = [], 1
    for d in reversed(shape):
        st.append(acc)
        acc *= d
    return tuple(reversed(st))


def inp(name, shape, dtype, addr):
    return ("input", name, tuple(shape), dense(shape), dtype, addr)


def op(o, ins, out, shape, dtype="f32", live=False, addr=None, axis=-1, esize=4):
    n = 1
    for d in shape:
        n *= d
    return {"op": o, "in": ins, "out": out, "shape": tuple(shape), "dtype": dtype, "axis": axis,
            "live": live, "addr": addr, "nbytes": n * esize}


def rms_group(x, w, out, shape, addr, tag):
    R, H = shape
    t = lambda n: f"{tag}_{n}"
    return [
        op("mul", [x, x], t("sq"), shape),
        op("reduce_sum", [t("sq")], t("s"), (R, 1)),
        op("mul", [t("s"), 1.0 / H], t("ms"), (R, 1)),
        op("add", [t("ms"), 1e-6], t("mse"), (R, 1)),
        op("sqrt", [t("mse")], t("r"), (R, 1)),
        op("div", [x, t("r")], t("xn"), shape),
        op("mul", [t("xn"), w], out, shape, "bf16", live=True, addr=addr, esize=2),
    ]


def releases(grp, keep):
    return [("release", o["out"]) for o in grp if o["out"] not in keep]


def test_add_chain_then_rmsnorm_fuse_and_other_shape_flushes():
    sh = (8, 64)
    ev = [inp("h0", sh, "bf16", 0), inp("r0", sh, "bf16", 1 * MB), inp("w", (64,), "f32", 2 * MB),
          inp("g0", (8, 96), "bf16", 3 * MB)]
    a1 = op("add", ["h0", "r0"], "h1", sh, "bf16", addr=4 * MB, esize=2)
    a2 = op("add", ["h1", "r0"], "h2", sh, "bf16", addr=5 * MB, esize=2)
    rg = rms_group("h2", "w", "n", sh, 6 * MB, "rms")
    sw = [op("exp", ["g0"], "e", (8, 96), "bf16", live=True, addr=7 * MB, esize=2)]
    ev += [("group", [a1]), ("release", "h0"), ("group", [a2]), ("release", "h1"),
           ("group", rg)] + releases(rg, {"n"}) + [("group", sw), ("flush",)]
    s = Stream()
    graphs = s.run(ev)
    assert len(graphs) == 2
    outs, why, stored = graphs[0]
    assert outs[:2] == ["h1", "h2"] and outs[-1] == "n" and why == "shape"
    # h1 released before the flush -> not stored; h2 still held -> stored; n live
    assert stored == ["h2", "n"]
    assert graphs[1] == (["e"], "explicit", ["e"])


def test_reduce_all_closes_graph():
    sh = (4, 4096)
    ev = [inp("x", sh, "f32", 0), inp("y", sh, "f32", 1 * MB),
          ("group", [op("reduce_sum", ["x"], "s", (), axis=None, live=True, addr=2 * MB)]),
          ("group", [op("add", ["x", "y"], "o", sh, live=True, addr=3 * MB)]),
          ("sync",)]
    graphs = Stream().run(ev)
    assert [g[1] for g in graphs] == ["reduce_all", "sync"]


def test_war_and_waw_dependences_flush():
    sh = (4, 512)
    ev = [inp("x", sh, "f32", 0), inp("y", sh, "f32", 1 * MB),
          ("group", [op("add", ["x", "y"], "o1", sh, live=True, addr=2 * MB)]),
          # writes x's storage while the buffered graph still reads x -> WAR
          ("group", [op("mul", ["o1", 2.0], "o2", sh, live=True, addr=0)]),
          ("flush",)]
    graphs = Stream().run(ev)
    assert [g[1] for g in graphs] == ["dependence", "explicit"]
    ev = [inp("x", sh, "f32", 0),
          ("group", [op("neg", ["x"], "o1", sh, live=True, addr=2 * MB)]),
          ("group", [op("abs", ["x"], "o2", sh, live=True, addr=2 * MB + 64)]),   # WAW overlap
          ("flush",)]
    assert [g[1] for g in Stream().run(ev)] == ["dependence", "explicit"]
    # reading the produced value by name fuses; reading its storage as a tensor does not
    ev = [inp("x", sh, "f32", 0), inp("o1mem", sh, "f32", 2 * MB),
          ("group", [op("neg", ["x"], "o1", sh, live=True, addr=2 * MB)]),
          ("group", [op("abs", ["o1mem"], "o2", sh, live=True, addr=3 * MB)]),
          ("flush",)]
    assert [g[1] for g in Stream().run(ev)] == ["dependence", "explicit"]


def test_resource_limits():
    sh = (2, 512)
    ev = [inp("x", sh, "f32", 0)]
    prev = "x"
    for i in range(65):
        ev.append(("group", [op("add", [prev, 1.0], f"v{i}", sh, addr=(i + 1) * MB)]))
        if prev != "x":
            ev.append(("release", prev))
        prev = f"v{i}"
    ev.append(("flush",))
    graphs = Stream().run(ev)
    assert [len(g[0]) for g in graphs] == [64, 1]
    assert graphs[0][1] == "resource"
    # more than three tile values in flight exceed the device's tile registers
    ev = [inp(f"x{i}", sh, "f32", i * MB) for i in range(5)]
    s = Stream()
    s.run(ev)
    chain = [op("add", ["x0", "x1"], "a", sh), op("mul", ["a", "x2"], "b", sh),
             op("add", ["b", 1.0], "c", sh, live=True, addr=9 * MB)]
    # op 0: x0, x1 live + a = 3; op 1: a, x2 + b = 3; op 2: b + c = 2
    assert s.demand(chain, sh)["tile"] == 3
    grp = [op("add", ["x0", "x1"], "a", sh), op("add", ["x2", "x3"], "b", sh),
           op("add", ["a", "b"], "d", sh, live=True, addr=9 * MB)]
    # at op 1: a, x2, x3 live + output b = 4
    assert s.demand(grp, sh)["tile"] == 4
    s2 = Stream()
    s2.run(ev + [("group", grp)])
    assert s2.unsupported and s2.unsupported[0][1] == "resource"
    s3 = Stream()
    s3.run(ev + [("group", chain), ("release", "a"), ("release", "b"), ("flush",)])
    assert len(s3.graphs) == 1 and not s3.unsupported


def test_matmul_only_first_and_epilogue_fuses():
    ev = [inp("A", (16, 32), "bf16", 0), inp("B", (32, 64), "bf16", MB), inp("bias", (64,), "f32", 2 * MB)]
    mm = op("matmul", ["A", "B"], "z", (16, 64))
    ad = op("add", ["z", "bias"], "zb", (16, 64))
    ev += [("group", [mm]), ("group", [ad]), ("release", "z"),
           ("group", [op("cast", ["zb"], "y", (16, 64), "bf16", live=True, addr=3 * MB, esize=2)]),
           ("release", "zb"),
           ("group", [op("matmul", ["A", "B"], "z2", (16, 64), live=True, addr=4 * MB)]),
           ("flush",)]
    graphs = Stream().run(ev)
    assert graphs[0] == (["z", "zb", "y"], "pattern", ["y"])
    assert graphs[1][0] == ["z2"]


def test_fused_semantics_equal_unfused():
    # evaluating the fused op list equals evaluating op by op with stores
    g = np.random.default_rng(0)
    x = g.normal(size=(3, 8))
    ops = [{"op": "add", "in": ["x", 1.0], "out": "a", "dtype": "f32"},
           {"op": "exp", "in": ["a"], "out": "b", "dtype": "bf16"},
           {"op": "mul", "in": ["b", "x"], "out": "c", "dtype": "f32"}]
    fused, _ = evaluate(ops, {"x": x})
    env = {"x": x}
    for o in ops:
        v, _ = evaluate([o], env)
        env[o["out"]] = v[o["out"]]
    assert np.array_equal(fused["c"], env["c"])

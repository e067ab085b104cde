"""Seeded random fused graphs on the GPU against the oracle.

Each case draws a ragged [R, C] shape, a few inputs (fp32 and bf16 tiles, a
row-broadcast [C] and a column-broadcast [R, 1] operand) and a chain of
well-conditioned moves: binary ops between tiles, broadcasts and scalars;
|.|-guarded division, sqrt and exp; row reductions applied back to the
tile.  The same op list goes through the C ABI (capture, streaming fusion,
tiling, encoding, the VM) and through the oracle's fp64 evaluator, and the
final value is compared within the stated tolerances (fp32 1e-5 of max|ref|,
bf16 2 ulp).  Every intermediate has storage, so a flush anywhere in the
chain stays legal; the fusion decisions themselves are exercised as they
fall.
"""
import numpy as np
import pytest

import workloads as W
from oracle import numerics as N
from oracle.graph import evaluate
from tests.dvm_helpers import empty_dev, host64, torch_dev

pytestmark = pytest.mark.gpu

BIN = ["add", "sub", "mul", "max", "min"]


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


class Chain:
    """Builds one op list twice: DVM graph ops and oracle op dicts."""

    def __init__(self, dvm, ctx, R, C):
        self.g = dvm.Graph(ctx)
        self.R, self.C = R, C
        self.ops, self.inputs, self.dev, self.tmp = [], {}, {}, []
        self.n = 0

    def input(self, name, arr, dtype):
        self.inputs[name] = arr
        t = torch_dev(arr, dtype)
        self.dev[name] = self.g.input(t)
        self.tmp.append(t)
        return name

    def op(self, op, ins, shape, dtype="f32", axis=-1):
        self.n += 1
        name = f"v{self.n}"
        out = empty_dev(shape, dtype)
        args = [self.dev[x] if isinstance(x, str) else x for x in ins]
        self.dev[name] = self.g.op(op, *args, out=out, axis=axis)
        self.tmp.append(out)
        d = {"op": op, "in": list(ins), "out": name, "dtype": dtype}
        if op.startswith("reduce"):
            d["axis"] = -1
        self.ops.append(d)
        return name, out


def build_case(dvm, ctx, seed):
    rg = np.random.default_rng(seed)
    R = int(rg.integers(1, 260))
    C = int(rg.integers(1, 2600))
    ch = Chain(dvm, ctx, R, C)
    tiles = [ch.input("x0", W.normal(rg, (R, C), 0, 1), "f32"),
             ch.input("x1", W.normal(rg, (R, C), 0, 1, "bf16"), "bf16")]
    bcast = [ch.input("b", W.normal(rg, (C,), 0, 1), "f32"),
             ch.input("c", W.normal(rg, (R, 1), 0, 1), "f32")]
    outs = {}
    cur = tiles[0]
    for _ in range(int(rg.integers(2, 8))):
        move = int(rg.integers(0, 7))
        if move == 0:      # tile (op) tile
            other = tiles[int(rg.integers(0, len(tiles)))]
            a, b = (cur, other) if rg.random() < 0.5 else (other, cur)
            cur, outs[cur] = ch.op(BIN[int(rg.integers(0, 5))], [a, b], (R, C))
        elif move == 1:    # tile (op) broadcast
            other = bcast[int(rg.integers(0, 2))]
            a, b = (cur, other) if rg.random() < 0.5 else (other, cur)
            cur, outs[cur] = ch.op(BIN[int(rg.integers(0, 5))], [a, b], (R, C))
        elif move == 2:    # tile (op) scalar
            s = float(np.round(rg.normal(0, 2), 3))
            ins = [cur, s] if rg.random() < 0.5 else [s, cur]
            cur, outs[cur] = ch.op(BIN[int(rg.integers(0, 5))], ins, (R, C))
        elif move == 3:    # x / (|y| + 1)
            y = tiles[int(rg.integers(0, len(tiles)))]
            t, _ = ch.op("abs", [y], (R, C))
            u, _ = ch.op("add", [t, 1.0], (R, C))
            cur, outs[cur] = ch.op("div", [cur, u], (R, C))
        elif move == 4:    # sqrt(|x|) or exp(-|x|)
            t, _ = ch.op("abs", [cur], (R, C))
            if rg.random() < 0.5:
                cur, outs[cur] = ch.op("sqrt", [t], (R, C))
            else:
                u, _ = ch.op("neg", [t], (R, C))
                cur, outs[cur] = ch.op("exp", [u], (R, C))
        else:              # row statistic applied back: x - max(x), x - mean(x), x * sum(|x|)^-1
            kind = int(rg.integers(0, 3))
            if kind == 0:
                m, _ = ch.op("reduce_max", [cur], (R, 1))
                cur, outs[cur] = ch.op("sub", [cur, m], (R, C))
            elif kind == 1:
                s, _ = ch.op("reduce_sum", [cur], (R, 1))
                m, _ = ch.op("div", [s, float(C)], (R, 1))
                cur, outs[cur] = ch.op("sub", [cur, m], (R, C))
            else:
                t, _ = ch.op("abs", [cur], (R, C))
                s, _ = ch.op("reduce_sum", [t], (R, 1))
                u, _ = ch.op("add", [s, 1.0], (R, 1))
                cur, outs[cur] = ch.op("div", [cur, u], (R, C))
        tiles.append(cur)
    final_dtype = "bf16" if rg.random() < 0.5 else "f32"
    y, yout = ch.op("copy" if final_dtype == "f32" else "cast", [cur], (R, C), dtype=final_dtype)
    return ch, y, yout, final_dtype


@pytest.mark.parametrize("seed", list(range(24)))
def test_random_fused_graph(dvm, ctx, seed):
    import torch
    ch, y, yout, dt = build_case(dvm, ctx, seed)
    print("CASE fuzz", seed, ch.R, ch.C, [o["op"] for o in ch.ops], dt, flush=True)
    g = ch.g
    g.release(*[ch.dev[o["out"]] for o in ch.ops if o["out"] != y])
    g.sync()
    torch.cuda.synchronize()
    ref, exact = evaluate(ch.ops, ch.inputs)
    got = host64(yout)
    if dt == "bf16":
        ok, d = N.check_bf16(got, exact[y])
        assert ok, f"max ulp {d}"
    else:
        r = ref[y]
        scale = max(np.max(np.abs(r)), 1e-30)
        err = np.max(np.abs(got - r)) / scale
        assert err <= 1e-5, f"max rel err {err:.3g}"


def build_mix_case(dvm, ctx, seed):
    """A MatMul followed by a random elementwise epilogue (bias row, residual
    tile, scalars, guarded division, exp, max/min)."""
    rg = np.random.default_rng(1000 + seed)
    M = int(rg.integers(1, 700))
    K = 8 * int(rg.integers(1, 96))
    N = 8 * int(rg.integers(1, 160))
    ch = Chain(dvm, ctx, M, N)
    a = ch.input("a", W.normal(rg, (M, K), 0, 0.1, "bf16"), "bf16")
    b = ch.input("b", W.normal(rg, (K, N), 0, 0.1, "bf16"), "bf16")
    others = [ch.input("bias", W.normal(rg, (N,), 0, 0.5), "f32"),
              ch.input("res", W.normal(rg, (M, N), 0, 0.5, "bf16"), "bf16")]
    cur, _ = ch.op("matmul", [a, b], (M, N))
    for _ in range(int(rg.integers(1, 6))):
        move = int(rg.integers(0, 4))
        if move == 0:
            other = others[int(rg.integers(0, 2))]
            ins = [cur, other] if rg.random() < 0.5 else [other, cur]
            cur, _ = ch.op(BIN[int(rg.integers(0, 5))], ins, (M, N))
        elif move == 1:
            s = float(np.round(rg.normal(0, 2), 3))
            ins = [cur, s] if rg.random() < 0.5 else [s, cur]
            cur, _ = ch.op(BIN[int(rg.integers(0, 5))], ins, (M, N))
        elif move == 2:
            t, _ = ch.op("abs", [cur], (M, N))
            u, _ = ch.op("add", [t, 1.0], (M, N))
            cur, _ = ch.op("div", [cur, u], (M, N))
        else:
            t, _ = ch.op("abs", [cur], (M, N))
            u, _ = ch.op("neg", [t], (M, N))
            cur, _ = ch.op("exp", [u], (M, N))
    final_dtype = "bf16" if rg.random() < 0.5 else "f32"
    y, yout = ch.op("copy" if final_dtype == "f32" else "cast", [cur], (M, N), dtype=final_dtype)
    return ch, y, yout, final_dtype


@pytest.mark.parametrize("seed", list(range(16)))
def test_random_matmul_epilogue(dvm, ctx, seed):
    import torch
    ch, y, yout, dt = build_mix_case(dvm, ctx, seed)
    print("CASE mix fuzz", seed, ch.R, ch.C, [o["op"] for o in ch.ops], dt, flush=True)
    g = ch.g
    g.release(*[ch.dev[o["out"]] for o in ch.ops if o["out"] != y])
    g.sync()
    torch.cuda.synchronize()
    ref, _ = evaluate(ch.ops, ch.inputs)
    ok, e = N.check_matmul(host64(yout), ref[y])
    assert ok, f"max rel err {e:.3g}"

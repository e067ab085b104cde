"""Pins for oracle/graph.py (the fused-graph evaluator).

* With fp32 emulation, c = sqrt(a + b) must equal numpy's float32
  computation bit for bit (both + and sqrt are correctly rounded, and rounding
  an fp64 result of + or sqrt to fp32 equals the fp32 operation: 53 >= 2*24+2).
* A LayerNorm written as primitive ops must agree with torch's fp64
  layer_norm; an RMSNorm and a softmax op list likewise.
* A bf16 cast must equal torch's float32 -> bfloat16 conversion.
"""
import numpy as np
import torch
import torch.nn.functional as F

from oracle.graph import evaluate, out_shape
from oracle.numerics import round_bf16
import workloads as W


def test_sqrt_add_fp32_emulation_is_bit_exact_vs_torch():
    a, b = W.vv_sqrt_add(0, (37, 53))
    ops = [{"op": "add", "in": ["a", "b"], "out": "t", "dtype": "f32"},
           {"op": "sqrt", "in": ["t"], "out": "c", "dtype": "f32"}]
    vals, _ = evaluate(ops, {"a": a, "b": b}, emulate_f32=True)
    # numpy's float32 add and sqrt are IEEE correctly rounded (torch's CPU
    # float32 sqrt is a vectorised approximation and may be 1 ulp off)
    ref = np.sqrt(a.astype(np.float32) + b.astype(np.float32)).astype(np.float64)
    assert np.array_equal(vals["c"], ref)


def ln_ops(h, eps):
    return [
        {"op": "cast", "in": ["x"], "out": "xf", "dtype": "f32"},
        {"op": "reduce_sum", "in": ["xf"], "out": "s1", "dtype": "f32", "axis": -1},
        {"op": "mul", "in": ["s1", 1.0 / h], "out": "mu", "dtype": "f32"},
        {"op": "sub", "in": ["xf", "mu"], "out": "xc", "dtype": "f32"},
        {"op": "mul", "in": ["xc", "xc"], "out": "sq", "dtype": "f32"},
        {"op": "reduce_sum", "in": ["sq"], "out": "s2", "dtype": "f32", "axis": -1},
        {"op": "mul", "in": ["s2", 1.0 / h], "out": "var", "dtype": "f32"},
        {"op": "add", "in": ["var", eps], "out": "ve", "dtype": "f32"},
        {"op": "sqrt", "in": ["ve"], "out": "sd", "dtype": "f32"},
        {"op": "recip", "in": ["sd"], "out": "rs", "dtype": "f32"},
        {"op": "mul", "in": ["xc", "rs"], "out": "xn", "dtype": "f32"},
        {"op": "mul", "in": ["xn", "gamma"], "out": "yg", "dtype": "f32"},
        {"op": "add", "in": ["yg", "beta"], "out": "yb", "dtype": "f32"},
        {"op": "cast", "in": ["yb"], "out": "y", "dtype": "bf16"},
    ]


def test_layernorm_op_list_vs_torch():
    h = 96
    x = W.normal(np.random.default_rng(1), (11, h), 0, 1, "bf16")
    gam, bet = W.layernorm_params(h)
    vals, exact = evaluate(ln_ops(h, 1e-6), {"x": x, "gamma": gam, "beta": bet})
    ref = F.layer_norm(torch.from_numpy(x.astype(np.float64)), (h,),
                       torch.from_numpy(gam.astype(np.float64)),
                       torch.from_numpy(bet.astype(np.float64)), eps=1e-6).numpy()
    assert np.allclose(exact["y"], ref, rtol=0, atol=1e-12)
    assert np.array_equal(vals["y"], round_bf16(exact["y"]))


def test_rmsnorm_and_softmax_op_lists_vs_torch():
    x = np.random.default_rng(2).normal(size=(5, 24))
    w = np.random.default_rng(3).normal(1, 0.1, 24)
    rms = [
        {"op": "mul", "in": ["x", "x"], "out": "sq", "dtype": "f32"},
        {"op": "reduce_sum", "in": ["sq"], "out": "s", "dtype": "f32", "axis": -1},
        {"op": "mul", "in": ["s", 1.0 / 24], "out": "ms", "dtype": "f32"},
        {"op": "add", "in": ["ms", 1e-6], "out": "mse", "dtype": "f32"},
        {"op": "sqrt", "in": ["mse"], "out": "r", "dtype": "f32"},
        {"op": "div", "in": ["x", "r"], "out": "xn", "dtype": "f32"},
        {"op": "mul", "in": ["xn", "w"], "out": "y", "dtype": "f32"},
    ]
    vals, _ = evaluate(rms, {"x": x, "w": w})
    ref = F.rms_norm(torch.from_numpy(x), (24,), torch.from_numpy(w), eps=1e-6).numpy()
    assert np.allclose(vals["y"], ref, rtol=0, atol=1e-13)
    sm = [
        {"op": "reduce_max", "in": ["x"], "out": "m", "dtype": "f32", "axis": -1},
        {"op": "sub", "in": ["x", "m"], "out": "d", "dtype": "f32"},
        {"op": "exp", "in": ["d"], "out": "e", "dtype": "f32"},
        {"op": "reduce_sum", "in": ["e"], "out": "s", "dtype": "f32", "axis": -1},
        {"op": "div", "in": ["e", "s"], "out": "p", "dtype": "f32"},
    ]
    vals, _ = evaluate(sm, {"x": x})
    assert np.allclose(vals["p"], torch.softmax(torch.from_numpy(x), -1).numpy(), rtol=0, atol=1e-15)


def test_cast_bf16_matches_torch():
    x = np.random.default_rng(4).normal(size=1000).astype(np.float32)
    vals, _ = evaluate([{"op": "cast", "in": ["x"], "out": "y", "dtype": "bf16"}], {"x": x})
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(vals["y"], ref)


def test_reduce_all_and_isfinite_shapes():
    x = np.array([[1.0, np.inf], [np.nan, -2.0]])
    ops = [{"op": "isfinite", "in": ["x"], "out": "f", "dtype": "u8"},
           {"op": "reduce_sum", "in": ["f"], "out": "n", "dtype": "f32", "axis": None}]
    vals, _ = evaluate(ops, {"x": x})
    assert vals["n"] == 2.0
    shapes = {"x": (2, 2)}
    assert out_shape(ops[1], {**shapes, "f": (2, 2)}) == ()
    assert out_shape({"op": "reduce_sum", "in": ["x"], "axis": -1}, shapes) == (2, 1)
    assert out_shape({"op": "add", "in": ["x", 1.0]}, shapes) == (2, 2)

"""fp64 evaluator of a fused op graph given as a primitive op list
(test infrastructure).

A graph is what the streaming fuser buffers (DVM paper review page, section
5.2, dynamic-graph fusion: ops are appended in order and fused): a list of
primitive ops, each naming its inputs (external tensors, earlier op outputs or
python-float scalars), its output name and the output's storage dtype.

Semantics (the reading taken, since the pages define no numeric model): each
op is evaluated in fp64 from its inputs' values; the result is then rounded to
the op's output dtype (bf16 values are rounded; u8 holds 0/1).  fp32 results
are kept in fp64 ("exact" mode) unless ``emulate_f32`` is set, in which case
they are rounded to fp32 after every op -- the model of a device that stores
every fp32 intermediate, used for the bit-exact predictions of chains made of
correctly rounded +, -, *, / and sqrt.

Op list format::

    {"op": "add", "in": ["a", "b"], "out": "c", "dtype": "f32"}
    {"op": "mul", "in": ["s", 0.5], "out": "m", "dtype": "f32"}
    {"op": "reduce_sum", "in": ["x"], "out": "s", "dtype": "f32", "axis": -1}
    {"op": "reduce_sum", "in": ["x"], "out": "t", "dtype": "f32", "axis": None}
"""
from __future__ import annotations

import numpy as np

from . import ops as O
from .numerics import round_to, round_f32

BINARY = {
    "add": O.add, "sub": O.sub, "mul": O.mul, "div": O.div,
    "max": O.maximum, "min": O.minimum, "pow": O.power,
}
UNARY = {
    "sqrt": O.sqrt, "abs": O.absolute, "log": O.log, "exp": O.exp,
    "round": O.round_half_even, "floor": O.floor, "isfinite": O.isfinite,
    "neg": O.neg, "recip": O.reciprocal, "cast": O.copy, "copy": O.copy,
}
REDUCE = {"reduce_sum": O.reduce_sum, "reduce_max": O.reduce_max}


def evaluate(ops, inputs, emulate_f32=False):
    """Evaluate ``ops`` over ``inputs`` (name -> array of stored values).

    Returns ``(values, exact)``: ``values[name]`` is each value as the graph
    defines it (rounded to its dtype), ``exact[name]`` the fp64 result of the
    op before that rounding (for the floored-ulp bf16 comparison).
    """
    vals = {k: np.asarray(v, dtype=np.float64) for k, v in inputs.items()}
    exact = {}

    def get(x):
        if isinstance(x, (int, float)):
            return np.float64(x)
        return vals[x]

    for op in ops:
        name = op["op"]
        args = [get(x) for x in op["in"]]
        if name in BINARY:
            r = BINARY[name](args[0], args[1])
        elif name in UNARY:
            r = UNARY[name](args[0])
        elif name in REDUCE:
            r = REDUCE[name](args[0], op.get("axis", -1))
        elif name == "matmul":
            r = O.matmul(args[0], args[1])
        else:
            raise ValueError(f"unknown op {name}")
        r = np.asarray(r, dtype=np.float64)
        exact[op["out"]] = r
        dt = op["dtype"]
        if dt == "f32":
            vals[op["out"]] = round_f32(r) if emulate_f32 else r
        else:
            vals[op["out"]] = round_to(r, dt)
    return vals, exact


def out_shape(op, shapes):
    """Shape of an op's output from its input shapes (numpy broadcasting)."""
    name = op["op"]
    ins = [shapes[x] if not isinstance(x, (int, float)) else () for x in op["in"]]
    if name in REDUCE:
        if op.get("axis", -1) is None:
            return ()
        return tuple(ins[0][:-1]) + (1,)
    if name == "matmul":
        return (ins[0][0], ins[1][1])
    return tuple(np.broadcast_shapes(*ins))

"""Composite operators written as groups of primitive ops.

Each composite is one fusion group: its primitive ops are appended between
begin/end group and its internal values are released before the group ends,
so they never need storage (the fuser keeps them on chip).  The textbook
forms are used:

* LayerNorm over the last axis: mu = sum(x)/H; xc = x - mu;
  var = sum(xc^2)/H; y = xc * (1/sqrt(var + eps)) * gamma + beta.
* RMSNorm: y = x / sqrt(sum(x^2)/H + eps) * w.
* Row softmax: e = exp(x - max(x)); y = e / sum(e).
* SiLU(z) = z / (1 + exp(-z)); SwiGLU = SiLU(g) * u.
* MatMul + bias + SiLU: a matmul first, its epilogue after it (one MIX graph).

Reductions and normalisations compute in fp32; the result is rounded to the
output's dtype.
"""
from __future__ import annotations


def _cast_in(g, x, temps):
    if x.dtype == "f32":
        return x
    xf = g.op("cast", x, dtype="f32")
    temps.append(xf)
    return xf


def layer_norm(g, x, gamma, beta, eps, out=None, dtype=None):
    h = x.shape[-1]
    t = []
    with g.group():
        xf = _cast_in(g, x, t)
        s1 = g.op("reduce_sum", xf); t.append(s1)
        mu = g.op("div", s1, float(h)); t.append(mu)
        xc = g.op("sub", xf, mu); t.append(xc)
        sq = g.op("mul", xc, xc); t.append(sq)
        s2 = g.op("reduce_sum", sq); t.append(s2)
        var = g.op("div", s2, float(h)); t.append(var)
        ve = g.op("add", var, float(eps)); t.append(ve)
        sd = g.op("sqrt", ve); t.append(sd)
        rs = g.op("recip", sd); t.append(rs)
        xn = g.op("mul", xc, rs); t.append(xn)
        yg = g.op("mul", xn, gamma); t.append(yg)
        yb = g.op("add", yg, beta); t.append(yb)
        y = g.op("cast", yb, out=out, dtype=dtype or x.dtype, live=out is not None)
        g.release(*t)
    return y


def rms_norm(g, x, w, eps, out=None, dtype=None):
    h = x.shape[-1]
    t = []
    with g.group():
        xf = _cast_in(g, x, t)
        sq = g.op("mul", xf, xf); t.append(sq)
        s = g.op("reduce_sum", sq); t.append(s)
        ms = g.op("div", s, float(h)); t.append(ms)
        mse = g.op("add", ms, float(eps)); t.append(mse)
        r = g.op("sqrt", mse); t.append(r)
        xn = g.op("div", xf, r); t.append(xn)
        y = g.op("mul", xn, w, out=out, dtype=dtype or x.dtype, live=out is not None)
        g.release(*t)
    return y


def softmax(g, x, out=None, dtype=None):
    t = []
    with g.group():
        xf = _cast_in(g, x, t)
        m = g.op("reduce_max", xf); t.append(m)
        d = g.op("sub", xf, m); t.append(d)
        e = g.op("exp", d); t.append(e)
        s = g.op("reduce_sum", e); t.append(s)
        y = g.op("div", e, s, out=out, dtype=dtype or x.dtype, live=out is not None)
        g.release(*t)
    return y


def silu(g, z, out=None, dtype=None):
    t = []
    with g.group():
        zf = _cast_in(g, z, t)
        nz = g.op("neg", zf); t.append(nz)
        e = g.op("exp", nz); t.append(e)
        d = g.op("add", e, 1.0); t.append(d)
        y = g.op("div", zf, d, out=out, dtype=dtype or z.dtype, live=out is not None)
        g.release(*t)
    return y


def swiglu(g, gate, up, out=None, dtype=None):
    t = []
    with g.group():
        gf = _cast_in(g, gate, t)
        nz = g.op("neg", gf); t.append(nz)
        e = g.op("exp", nz); t.append(e)
        d = g.op("add", e, 1.0); t.append(d)
        s = g.op("div", gf, d); t.append(s)
        y = g.op("mul", s, up, out=out, dtype=dtype or gate.dtype, live=out is not None)
        g.release(*t)
    return y


def matmul_bias_silu(g, a, b, bias, out=None, dtype=None):
    """y = SiLU(a @ b + bias): a matmul (fp32 result, never rounded) and its
    elementwise epilogue, one MIX graph."""
    t = []
    with g.group():
        z = g.op("matmul", a, b, dtype="f32"); t.append(z)
        zb = g.op("add", z, bias); t.append(zb)
        n = g.op("mul", zb, -1.0); t.append(n)
        e = g.op("exp", n); t.append(e)
        d = g.op("add", e, 1.0); t.append(d)
        s = g.op("div", zb, d); t.append(s)
        y = g.op("cast", s, out=out, dtype=dtype or "bf16", live=out is not None)
        g.release(*t)
    return y

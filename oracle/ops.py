"""fp64 definitions of the operations and workload graphs (test infrastructure).

Each function states the plain mathematical definition, in float64, with no
blocking, fusion or reordering.  Rounding to a storage dtype happens only where
the definition has a stored result (the caller applies ``numerics.round_to``).

Sources
-------
* Table 1 of the DVM paper review page (section 4.1) names the tile-level
  virtual instructions: Load/ViewLoad/Store/ViewStore, Copy, Broadcast, Sqrt
  and the other elementwise ops Abs/Log/Exp/Pow/Round/Floor/IsFinite.
* Section 5.1 of that page gives the vector-vector fusion example c = a + b,
  c = sqrt(c), and cube-vector fusion (a matrix product followed by vector ops).
* Section 6.2 (Figures 12-14, Table 3) names the operator workloads LayerNorm,
  if-else-add and addmm; the MindSpore summary page (section 3.3) names the
  fusion patterns elemwise-elemwise, reduce forward fusion, MatMul+elemwise.
* The pages define none of these operators' formulas; the textbook ones are
  used and stated per function.
"""
from __future__ import annotations

import numpy as np

f64 = np.float64


def _a(x):
    return np.asarray(x, dtype=f64)


# ---------------------------------------------------------------------------
# Elementwise (Table 1 plus the binary ops the fusion examples need)
# ---------------------------------------------------------------------------
def add(a, b):
    return _a(a) + _a(b)


def sub(a, b):
    return _a(a) - _a(b)


def mul(a, b):
    return _a(a) * _a(b)


def div(a, b):
    with np.errstate(divide="ignore", invalid="ignore"):
        return _a(a) / _a(b)


def maximum(a, b):
    """NaN-propagating maximum (a NaN operand gives NaN)."""
    return np.maximum(_a(a), _a(b))


def minimum(a, b):
    return np.minimum(_a(a), _a(b))


def power(a, b):
    """C99 pow: a negative base with a non-integer exponent gives NaN."""
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        return np.power(_a(a), _a(b))


def sqrt(a):
    with np.errstate(invalid="ignore"):
        return np.sqrt(_a(a))


def absolute(a):
    return np.abs(_a(a))


def log(a):
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.log(_a(a))


def exp(a):
    with np.errstate(over="ignore"):
        return np.exp(_a(a))


def round_half_even(a):
    """Round: the pages do not fix the tie rule; ties go to even (as torch.round)."""
    return np.rint(_a(a))


def floor(a):
    return np.floor(_a(a))


def isfinite(a):
    """IsFinite: 1 where the value is neither infinite nor NaN, else 0 (stored as u8)."""
    return np.isfinite(_a(a)).astype(f64)


def neg(a):
    return -_a(a)


def reciprocal(a):
    with np.errstate(divide="ignore"):
        return 1.0 / _a(a)


def copy(a):
    return _a(a).copy()


def broadcast(xn, m, size, n):
    """Broadcast(xd, xn, M, size, N) of Table 1, read as: for m < M, n < N,
    k < size: xd[(m*N + n)*size + k] = xn[m*size + k].

    M = 1 repeats one row N times (a bias row); size = 1 spreads one scalar
    per row across N columns (a row mean).
    """
    xn = _a(xn).reshape(m, 1, size)
    return np.broadcast_to(xn, (m, n, size)).reshape(m * n * size).copy()


def reduce_sum(a, axis=-1):
    """Sum over the innermost axis (keepdims) or over all axes (axis=None)."""
    a = _a(a)
    if axis is None:
        return np.sum(a, dtype=f64).reshape(())
    return np.sum(a, axis=axis, keepdims=True, dtype=f64)


def reduce_max(a, axis=-1):
    a = _a(a)
    if axis is None:
        return np.max(a).reshape(())
    return np.max(a, axis=axis, keepdims=True)


def matmul(a, b):
    """z[m, n] = sum_k a[m, k] b[k, n] in fp64."""
    return _a(a) @ _a(b)


# ---------------------------------------------------------------------------
# Composite definitions used by the workloads (textbook forms)
# ---------------------------------------------------------------------------
def silu(z):
    """SiLU(z) = z / (1 + exp(-z))."""
    z = _a(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def layer_norm(x, gamma, beta, eps):
    """LayerNorm over the last axis: mu = mean(x); var = mean((x - mu)^2)
    (biased, two-pass); y = (x - mu) / sqrt(var + eps) * gamma + beta."""
    x = _a(x)
    mu = np.mean(x, axis=-1, keepdims=True)
    xc = x - mu
    var = np.mean(xc * xc, axis=-1, keepdims=True)
    return xc / np.sqrt(var + eps) * _a(gamma) + _a(beta)


def rms_norm(x, w, eps):
    """RMSNorm over the last axis: y = x / sqrt(mean(x^2) + eps) * w."""
    x = _a(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _a(w)


def softmax(x):
    """Row softmax over the last axis: y = exp(x - max) / sum(exp(x - max))."""
    x = _a(x)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def swiglu(g, u):
    """SwiGLU elementwise: SiLU(g) * u."""
    return silu(g) * _a(u)


def matmul_bias_silu(a, b, bias):
    """Cube-vector fusion workload: y = SiLU(a @ b + bias)."""
    return silu(matmul(a, b) + _a(bias))


def if_else_add(x, y):
    """if sum(x) > 0: x + y else x - y.  The comparison is strict: a sum of
    exactly zero takes the else branch.  Returns (out, branch_taken, S)."""
    s = float(np.sum(_a(x), dtype=f64))
    if s > 0.0:
        return _a(x) + _a(y), True, s
    return _a(x) - _a(y), False, s


def sum_guard_band(x) -> float:
    """Error bound for a blocked/pairwise fp32 sum of n terms (Higham,
    Accuracy and Stability of Numerical Algorithms, ch. 4):
    |S_fp32 - S| <= 4 (ceil(log2 n) + 1) u sum|x|, u = 2^-24.  A branch
    decided by sign(S) is well defined only when |S| exceeds it."""
    x = _a(x)
    n = max(int(x.size), 1)
    return 4.0 * (int(np.ceil(np.log2(n))) + 1) * 2.0 ** -24 * float(np.sum(np.abs(x)))

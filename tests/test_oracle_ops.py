"""Pins for oracle/ops.py against library routines, closed forms, invariants
and brute force on tiny inputs (no GPU)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ops as O

g = np.random.default_rng(2024)


def t64(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64))


def test_elementwise_specials():
    assert np.isnan(O.power(-2.0, 0.5))
    assert O.power(-2.0, 3.0) == -8.0
    assert O.power(0.0, 0.0) == 1.0
    r = O.round_half_even(np.array([0.5, 1.5, 2.5, -0.5, -1.5, 2.4999]))
    assert np.array_equal(r, [0.0, 2.0, 2.0, -0.0, -2.0, 2.0])
    assert np.signbit(r[3])
    assert np.array_equal(O.floor(np.array([-1.5, -0.0, 2.7])), [-2.0, -0.0, 2.0])
    assert np.array_equal(O.isfinite(np.array([1.0, np.inf, -np.inf, np.nan])), [1, 0, 0, 0])
    assert np.isnan(O.maximum(np.nan, 1.0)) and np.isnan(O.minimum(1.0, np.nan))
    assert O.sqrt(4.0) == 2.0 and np.isnan(O.sqrt(-1.0))
    assert O.log(np.e) == pytest.approx(1.0, abs=1e-15)


def test_broadcast_reading():
    # M = 1: one row repeated N times
    assert np.array_equal(O.broadcast([1, 2, 3], 1, 3, 2), [1, 2, 3, 1, 2, 3])
    # size = 1: one scalar per row spread over N columns
    assert np.array_equal(O.broadcast([5, 7], 2, 1, 3), [5, 5, 5, 7, 7, 7])
    # general: M = 2 rows of size 2, N = 2 copies each
    assert np.array_equal(O.broadcast([1, 2, 3, 4], 2, 2, 2), [1, 2, 1, 2, 3, 4, 3, 4])


def test_reduce():
    x = g.normal(size=(3, 7))
    s = O.reduce_sum(x)
    assert s.shape == (3, 1)
    assert np.allclose(s[:, 0], [sum(r) for r in x], rtol=0, atol=1e-14)
    assert O.reduce_sum(x, axis=None).shape == ()
    assert O.reduce_max(x)[1, 0] == max(x[1])


def test_layer_norm_vs_torch():
    x = g.normal(size=(9, 37))
    gam = g.normal(1, 0.1, 37)
    bet = g.normal(0, 0.1, 37)
    ref = F.layer_norm(t64(x), (37,), t64(gam), t64(bet), eps=1e-6).numpy()
    assert np.allclose(O.layer_norm(x, gam, bet, 1e-6), ref, rtol=0, atol=1e-13)


def test_layer_norm_invariants():
    x = g.normal(3.0, 2.0, size=(5, 64))
    eps = 1e-6
    z = O.layer_norm(x, np.ones(64), np.zeros(64), eps)
    assert np.all(np.abs(z.mean(-1)) < 1e-12)
    var = x.var(-1)
    assert np.allclose(z.var(-1), var / (var + eps), rtol=1e-12, atol=0)
    beta = g.normal(size=64)
    const = np.full((2, 64), 3.25)
    assert np.array_equal(O.layer_norm(const, g.normal(size=64), beta, eps), np.broadcast_to(beta, (2, 64)))
    one = g.normal(size=(4, 1))
    assert np.array_equal(O.layer_norm(one, [2.0], [0.5], eps), np.full((4, 1), 0.5))


def test_rms_norm_vs_torch_and_invariants():
    x = g.normal(size=(6, 40))
    w = g.normal(1, 0.1, 40)
    ref = F.rms_norm(t64(x), (40,), t64(w), eps=1e-6).numpy()
    y = O.rms_norm(x, w, 1e-6)
    assert np.allclose(y, ref, rtol=0, atol=1e-13)
    ms = (x * x).mean(-1)
    assert np.allclose(((y / w) ** 2).mean(-1), ms / (ms + 1e-6), rtol=1e-12)
    # scaling x by c > 0 changes y only through eps: with eps = 0 it is invariant
    assert np.allclose(O.rms_norm(3.5 * x, w, 0.0), O.rms_norm(x, w, 0.0), rtol=1e-13)


def test_softmax_vs_torch_and_invariants():
    x = g.normal(size=(7, 33)) * 4
    y = O.softmax(x)
    assert np.allclose(y, torch.softmax(t64(x), -1).numpy(), rtol=0, atol=1e-15)
    assert np.allclose(y.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(O.softmax(x + g.normal(size=(7, 1)) * 10), y, rtol=1e-12)
    assert np.array_equal(O.softmax(g.normal(size=(3, 1))), np.ones((3, 1)))


def test_silu_and_swiglu():
    z = g.normal(size=200) * 5
    assert np.allclose(O.silu(z), F.silu(t64(z)).numpy(), rtol=1e-14, atol=1e-15)
    assert O.silu(0.0) == 0.0
    assert np.allclose(O.silu(z) - O.silu(-z), z, rtol=1e-13, atol=1e-14)
    u = g.normal(size=200)
    assert np.allclose(O.swiglu(z, u), F.silu(t64(z)).numpy() * u, rtol=1e-14, atol=1e-15)


def test_matmul_bias_silu_brute_force():
    # M = K = 1
    a = np.array([[0.5]])
    b = np.array([[2.0, -1.0, 3.0]])
    bias = np.array([0.25, 0.0, -3.0])
    z = np.array([0.5 * 2.0 + 0.25, -0.5, 1.5 - 3.0])
    assert np.allclose(O.matmul_bias_silu(a, b, bias)[0], z / (1 + np.exp(-z)), rtol=1e-15)
    # B = identity: y = SiLU(A + bias)
    A = g.normal(size=(5, 8))
    bias = g.normal(size=8)
    assert np.allclose(O.matmul_bias_silu(A, np.eye(8), bias), O.silu(A + bias), rtol=1e-14)
    # triple-loop brute force on a small random case
    A = g.normal(size=(3, 4))
    B = g.normal(size=(4, 5))
    ref = np.zeros((3, 5))
    for m in range(3):
        for n in range(5):
            acc = 0.0
            for k in range(4):
                acc += A[m, k] * B[k, n]
            ref[m, n] = acc
    assert np.allclose(O.matmul(A, B), ref, rtol=1e-14)


def test_if_else_add_branches():
    y = np.array([10.0, 20.0])
    out, br, s = O.if_else_add(np.array([1.0, 2.0]), y)
    assert br and np.array_equal(out, [11.0, 22.0])
    out, br, s = O.if_else_add(np.array([-1.0, -2.0]), y)
    assert not br and np.array_equal(out, [-11.0, -22.0])
    out, br, s = O.if_else_add(np.array([1.0, -1.0]), y)          # S == 0 -> else
    assert not br and s == 0.0 and np.array_equal(out, [-9.0, -21.0])


def test_sum_guard_band_bounds_fp32_sums():
    for n in (1, 7, 4096, 300000):
        x = g.normal(size=n).astype(np.float32)
        s64 = float(np.sum(x.astype(np.float64)))
        s32 = float(np.sum(x, dtype=np.float32))              # numpy: pairwise fp32
        seq = np.float32(0)
        for v in x[:4096]:
            seq = np.float32(seq + v)
        s64_head = float(np.sum(x[:4096].astype(np.float64)))
        band = O.sum_guard_band(x)
        assert abs(s32 - s64) <= band
        assert abs(float(seq) - s64_head) <= 4096 * 2.0 ** -24 * float(np.sum(np.abs(x[:4096]))) + 1e-30

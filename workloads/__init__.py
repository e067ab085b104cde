"""Seeded synthetic inputs for the DVM hot path.

This module only draws random numbers and builds shape/op sequences. It holds
none of the method's arithmetic, so both the oracle (``oracle/``) and the HIP
path (``device_bytecode_vm_amd``) may consume what it produces without sharing
any computation.

Conventions
-----------
* Host draws use ``numpy.random.default_rng(seed)`` (PCG64), in float64, then
  converted to the stated storage dtype.  bf16 values are produced by torch's
  float32 -> bfloat16 conversion (round to nearest even) and returned as the
  exactly representable float32 values, so a host array can be copied to the
  device as bf16 without any further rounding.
* A stream's shape sequence is drawn first from ``default_rng(seed)``; call
  ``i``'s tensors then come from ``default_rng(seed * 1000 + i)``.
* "N(mu, s)" means mean ``mu`` and standard deviation ``s``.
"""
from __future__ import annotations

import numpy as np

H_LN = 5120          # LayerNorm / RMSNorm hidden size of the LLM-layer workloads
N_FFN = 17408        # MatMul output width / SwiGLU width
K_MM = 5120          # MatMul reduction size
HEADS = 40           # softmax heads


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def to_bf16_exact(a: np.ndarray) -> np.ndarray:
    """float -> nearest bfloat16 (RNE, via torch), returned as float32 values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def normal(g: np.random.Generator, shape, mu=0.0, sd=1.0, dtype="f32") -> np.ndarray:
    x = g.normal(mu, sd, size=shape)
    if dtype == "bf16":
        return to_bf16_exact(x.astype(np.float32))
    return x.astype(np.float32)


def uniform01(g: np.random.Generator, shape) -> np.ndarray:
    return g.random(size=shape).astype(np.float32)


# ----------------------------------------------------------------------------
# Workload 1: c = sqrt(a + b), a, b fp32 (513, 1031) ~ U[0, 1), seed 0
# ----------------------------------------------------------------------------
def vv_sqrt_add(seed: int = 0, shape=(513, 1031)):
    g = rng(seed)
    a = uniform01(g, shape)
    b = uniform01(g, shape)
    return a, b


# ----------------------------------------------------------------------------
# Workload 2: LayerNorm stream over [R, 5120] bf16, R = B*S
# ----------------------------------------------------------------------------
def layernorm_shapes(seed: int = 0, calls: int = 64, h: int = H_LN):
    g = rng(seed)
    b = g.integers(1, 33, size=calls)
    s = g.integers(1, 4097, size=calls)
    return [(int(bb) * int(ss), h) for bb, ss in zip(b, s)]


def layernorm_params(h: int = H_LN, seed: int = 1):
    g = rng(seed)
    gamma = normal(g, (h,), 1.0, 0.1)
    beta = normal(g, (h,), 0.0, 0.1)
    return gamma, beta


def layernorm_x(seed: int, i: int, rows: int, h: int = H_LN):
    return normal(rng(seed * 1000 + i), (rows, h), 0.0, 1.0, "bf16")


LN_EPS = 1e-6


# ----------------------------------------------------------------------------
# Workload 3: if sum(x) > 0: x + y else x - y, x, y fp32 [N, 4096]
# ----------------------------------------------------------------------------
def ifelse_shapes(seed: int = 0, calls: int = 256, cols: int = 4096, nmax: int = 16384):
    g = rng(seed)
    n = g.integers(1, nmax + 1, size=calls)
    return [(int(v), cols) for v in n]


def ifelse_inputs(seed: int, i: int, shape):
    """x ~ N(s*8/sqrt(n), 1), y ~ N(0, 1); s = +-1 from a coin of call i.

    The mean shift puts sum(x) about 8 standard deviations away from zero on
    the side the coin picked, so both branches occur about equally often and
    the branch is well defined (far outside fp32 summation error).
    """
    g = rng(seed * 1000 + i)
    sign = 1.0 if g.random() < 0.5 else -1.0
    n = shape[0] * shape[1]
    x = g.normal(sign * 8.0 / np.sqrt(n), 1.0, size=shape).astype(np.float32)
    y = g.normal(0.0, 1.0, size=shape).astype(np.float32)
    return x, y, sign


# ----------------------------------------------------------------------------
# Workload 4: MatMul + bias + SiLU, A [M, 5120] bf16, B [5120, 17408] bf16
# ----------------------------------------------------------------------------
def matmul_ms(seed: int = 0, calls: int = 32, mmax: int = 8192):
    g = rng(seed)
    out, seen = [], set()
    while len(out) < calls:
        m = int(g.integers(1, mmax + 1))
        if m not in seen:
            seen.add(m)
            out.append(m)
    return out


def matmul_weights(k: int = K_MM, n: int = N_FFN, seed: int = 1):
    g = rng(seed)
    b = normal(g, (k, n), 0.0, 0.02, "bf16")
    bias = normal(g, (n,), 0.0, 0.02)
    return b, bias


def matmul_a(seed: int, i: int, m: int, k: int = K_MM):
    return normal(rng(seed * 1000 + i), (m, k), 0.0, 0.02, "bf16")


# ----------------------------------------------------------------------------
# Workload 5: transformer-layer op stream (motif sequence only)
# ----------------------------------------------------------------------------
MOTIFS = ("add", "rmsnorm", "swiglu", "softmax")
RMS_EPS = 1e-6


def stream_step(seed: int, n_motifs: int = 10000, tmin: int = 16, tmax: int = 4096, tkv_max: int = 8192):
    """Returns (T, T_kv, motif list); each motif is (kind, pool index)."""
    g = rng(seed)
    t = int(g.integers(tmin, tmax + 1))
    tkv = int(g.integers(t, tkv_max + 1))
    kinds = g.integers(0, 4, size=n_motifs)
    pool = g.integers(0, 4, size=n_motifs)
    motifs = []
    for k, p in zip(kinds, pool):
        kind = MOTIFS[int(k)]
        npool = 4 if kind == "add" else (1 if kind == "rmsnorm" else 2)
        motifs.append((kind, int(p) % npool))
    return t, tkv, motifs


# ----------------------------------------------------------------------------
# Device-side draws for large performance inputs (torch generator on the GPU).
# ----------------------------------------------------------------------------
def device_normal(shape, seed: int, mu=0.0, sd=1.0, dtype="f32", device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if sd != 1.0:
        t.mul_(sd)
    if mu != 0.0:
        t.add_(mu)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    return t


def device_uniform(shape, seed: int, device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.rand(shape, generator=gen, device=device, dtype=torch.float32)

"""The encoder's SiLU fusion: the chain n = -z, e = exp(n), d = e + 1,
s = z / d becomes one instruction when n, e and d are private fp32 values.

Host tests check where the fusion applies (handler ids and opcodes of the
bytecode format of csrc/bytecode.h, restated here); GPU tests check that a
fused chain stores, bit for bit, what the unfused chain stores (the fused
instruction computes the chain's own four operations).
"""
import numpy as np
import pytest

import device_bytecode_vm_amd as dvm
from device_bytecode_vm_amd import TensorDesc as TD
from device_bytecode_vm_amd import composites as CP

H_BODY_BEGIN, H_BODY_END = 16, 17
HD_SILU, OP_UN, UN_SILU = 159, 7, 11


def ops_of(p):
    w = p.words()
    return [(w[i] & 0xFF, (w[i] >> 20) & 0xF) for i in range(w[H_BODY_BEGIN], w[H_BODY_END], 2)]


def silu_chain(g, z, keep_d=None, out=None, neg_by_mul=False):
    n = g.op("mul", z, -1.0) if neg_by_mul else g.op("neg", z)
    e = g.op("exp", n)
    d = g.op("add", e, 1.0, out=keep_d, live=keep_d is not None)
    s = g.op("div", z, d, out=out, live=True)
    g.release(n, e, d)
    return s


def test_fusion_applies_to_private_chains():
    ctx = dvm.Context(-1)
    for neg_by_mul in (False, True):
        g = dvm.Graph(ctx)
        z = g.input(TD(1 << 34, "f32", (300, 4000)))
        silu_chain(g, z, out=TD(2 << 34, "f32", (300, 4000)), neg_by_mul=neg_by_mul)
        assert (HD_SILU, UN_SILU) in ops_of(g.flush())
    # d is stored: the chain stays as it is
    g = dvm.Graph(ctx)
    z = g.input(TD(1 << 34, "f32", (300, 4000)))
    silu_chain(g, z, keep_d=TD(3 << 34, "f32", (300, 4000)), out=TD(2 << 34, "f32", (300, 4000)))
    assert all(h != HD_SILU for h, _ in ops_of(g.flush()))
    # the MIX epilogue of MatMul+bias+SiLU: bias add, SiLU, store
    g = dvm.Graph(ctx)
    CP.matmul_bias_silu(g, g.input(TD(1 << 34, "bf16", (256, 64))), g.input(TD(2 << 34, "bf16", (64, 512))),
                        g.input(TD(3 << 34, "f32", (512,))), out=TD(4 << 34, "bf16", (256, 512)))
    assert (OP_UN, UN_SILU) in ops_of(g.flush())


@pytest.mark.gpu
def test_fused_silu_bit_identical_on_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("CASE silu_fusion", flush=True)
    ctx = dvm.Context(0)
    rg = np.random.default_rng(11)
    x = torch.from_numpy((rg.normal(0, 3, (777, 3001))).astype(np.float32)).cuda()
    x[0, :5] = torch.tensor([float("inf"), -float("inf"), 0.0, -0.0, 88.0])
    fused, plain = torch.empty_like(x), torch.empty_like(x)
    d_keep = torch.empty_like(x)
    g = dvm.Graph(ctx)
    silu_chain(g, g.input(x), out=fused)
    p = g.flush()
    assert (HD_SILU, UN_SILU) in ops_of(p)
    p.launch()
    g2 = dvm.Graph(ctx)
    silu_chain(g2, g2.input(x), keep_d=d_keep, out=plain)
    p2 = g2.flush()
    assert all(h != HD_SILU for h, _ in ops_of(p2))
    p2.launch()
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int32), plain.view(torch.int32))
    # the MIX epilogue, fused against unfused (the chain's d stored)
    K, N, M = 256, 1024, 300
    a = (torch.randn(M, K, device="cuda") * 0.5).to(torch.bfloat16)
    b = (torch.randn(K, N, device="cuda") * 0.5).to(torch.bfloat16)
    bias = torch.randn(N, device="cuda")
    outs = []
    for keep in (False, True):
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        dk = torch.empty((M, N), dtype=torch.float32, device="cuda")
        gm = dvm.Graph(ctx)
        with gm.group():
            z = gm.op("matmul", gm.input(a), gm.input(b), dtype="f32")
            zb = gm.op("add", z, gm.input(bias))
            silu_chain(gm, zb, keep_d=dk if keep else None, out=y)
            gm.release(z, zb)
        pm = gm.flush()
        assert ((OP_UN, UN_SILU) in ops_of(pm)) == (not keep)
        pm.launch()
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))

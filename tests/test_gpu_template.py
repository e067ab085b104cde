"""GPU runs of a static-graph template (symbolic fusion decided once): a
transformer-block slice recorded over symbols T and TKV, run at three
bindings; every output equals, bit for bit, what the streaming fuser's
graphs store for the same binding, and sampled rows match the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import numerics as N
from oracle import ops as O
from tests.dvm_helpers import host64

pytestmark = pytest.mark.gpu
H, F, NH = 512, 1536, 4


@pytest.fixture(scope="module")
def dvm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import device_bytecode_vm_amd as m
    return m


def block(g, h, r, w, ga, up, sc, outs):
    from device_bytecode_vm_amd import composites as CP
    h1 = g.op("add", h, r, out=outs[0], live=True)
    CP.rms_norm(g, h1, w, W.RMS_EPS, out=outs[1])
    CP.swiglu(g, ga, up, out=outs[2])
    CP.softmax(g, sc, out=outs[3])


def test_template_runs_match_dynamic_graphs(dvm):
    import torch
    ctx = dvm.Context(0)
    t = dvm.Template(ctx)
    ins_t = [t.input("bf16", ("T", H)), t.input("bf16", ("T", H)), t.input("f32", (H,)),
             t.input("bf16", ("T", F)), t.input("bf16", ("T", F)), t.input("bf16", (NH, "T", "TKV"))]
    block(t, *ins_t, [t.output("bf16") for _ in range(4)])
    assert t.finalize() == 3
    for T, TKV in [(37, 100), (1000, 2500), (3, 7)]:
        print("CASE template", T, TKV, flush=True)
        bf = dict(dtype="bf16")
        ins = [W.device_normal((T, H), seed=T, **bf), W.device_normal((T, H), seed=T + 1, **bf),
               W.device_normal((H,), seed=3, mu=1.0, sd=0.1), W.device_normal((T, F), seed=T + 2, **bf),
               W.device_normal((T, F), seed=T + 3, **bf), W.device_normal((NH, T, TKV), seed=T + 4, **bf)]
        shapes = [(T, H), (T, H), (T, F), (NH, T, TKV)]
        outs = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
        ref = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
        t.run(ins, outs)
        t.graph.sync()
        g = dvm.Graph(ctx)
        block(g, *[g.input(x) for x in ins], ref)
        g.sync()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b)
        h1 = N.round_bf16(host64(ins[0]) + host64(ins[1]))
        assert np.array_equal(host64(outs[0]), h1)
        ok, d = N.check_bf16(host64(outs[1]), O.rms_norm(h1, host64(ins[2]), W.RMS_EPS))
        assert ok, d
        ok, d = N.check_bf16(host64(outs[2]), O.swiglu(host64(ins[3]), host64(ins[4])))
        assert ok, d
        ok, d = N.check_bf16(host64(outs[3]), O.softmax(host64(ins[5])))
        assert ok, d

"""GPU parity of a short transformer op stream (residual add, RMSNorm, SwiGLU,
softmax motifs in a seeded order) captured through one streaming-fusion
buffer, against the oracle applied motif by motif.

The stream runs at the real hidden sizes (H = 5120, F = 17408, 40 heads) and
ragged T and T_kv, so the fuser flushes on shape changes between motifs and
fuses residual adds into the following RMSNorm.  Every output buffer is
checked after the stream: the residual chain bit for bit (each add is exact in
fp32, then rounded once to bf16), the rest within 2 bf16 ulp.
"""
import numpy as np
import pytest

import workloads as W
from oracle import numerics as N
from oracle import ops as O
from tests.dvm_helpers import empty_dev, host64, torch_dev

pytestmark = pytest.mark.gpu

HEADS = 40


@pytest.fixture(scope="module")
def dvm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import device_bytecode_vm_amd as m
    return m


@pytest.mark.parametrize("seed,n_motifs", [(3, 48), (4, 80)])
def test_op_stream_parity(dvm, seed, n_motifs):
    import torch
    from device_bytecode_vm_amd import composites as CP
    T, TKV, motifs = W.stream_step(seed, n_motifs, tmin=17, tmax=45, tkv_max=90)
    print("CASE op_stream", seed, n_motifs, T, TKV, flush=True)
    H, F = W.H_LN, W.N_FFN
    g = W.rng(1000 + seed)
    h0 = W.normal(g, (T, H), 0, 1, "bf16")
    res = [W.normal(g, (T, H), 0, 1, "bf16") for _ in range(4)]
    w = W.normal(g, (H,), 1, 0.1)
    gates = [W.normal(g, (T, F), 0, 1, "bf16") for _ in range(2)]
    ups = [W.normal(g, (T, F), 0, 1, "bf16") for _ in range(2)]
    scores = [W.normal(g, (HEADS, T, TKV), 0, 1, "bf16") for _ in range(2)]

    hs = [torch_dev(h0, "bf16"), empty_dev((T, H), "bf16")]
    d_res = [torch_dev(r, "bf16") for r in res]
    d_w = torch_dev(w, "f32")
    d_g = [torch_dev(x, "bf16") for x in gates]
    d_u = [torch_dev(x, "bf16") for x in ups]
    d_s = [torch_dev(x, "bf16") for x in scores]
    n_out = empty_dev((T, H), "bf16")
    o_out = empty_dev((T, F), "bf16")
    p_out = empty_dev((HEADS, T, TKV), "bf16")

    ctx = dvm.Context(0)
    gr = dvm.Graph(ctx)
    cur = 0
    vh = gr.input(hs[0])
    # oracle state, motif by motif
    h_ref = h0.astype(np.float64)
    n_ref = o_ref = p_ref = None
    for kind, j in motifs:
        if kind == "add":
            nxt = 1 - cur
            vh = gr.op("add", vh, gr.input(d_res[j]), out=hs[nxt])
            cur = nxt
            h_ref = N.round_bf16(h_ref + res[j])
        elif kind == "rmsnorm":
            CP.rms_norm(gr, vh, gr.input(d_w), W.RMS_EPS, out=n_out)
            n_ref = O.rms_norm(h_ref, w, W.RMS_EPS)
        elif kind == "swiglu":
            CP.swiglu(gr, gr.input(d_g[j]), gr.input(d_u[j]), out=o_out)
            o_ref = O.swiglu(gates[j], ups[j])
        else:
            CP.softmax(gr, gr.input(d_s[j]), out=p_out)
            p_ref = O.softmax(scores[j])
    gr.sync()
    torch.cuda.synchronize()
    st = gr.stats()
    kinds = {k for k, _ in motifs}
    assert st["graphs"] < len(motifs), st           # some motifs fused
    assert st["flush_reason"]["shape"] > 0, st      # shape changes split graphs

    assert np.array_equal(host64(hs[cur]), h_ref)
    if n_ref is not None:
        ok, d = N.check_bf16(host64(n_out), n_ref)
        assert ok, f"rmsnorm max ulp {d}"
    if o_ref is not None:
        ok, d = N.check_bf16(host64(o_out), o_ref)
        assert ok, f"swiglu max ulp {d}"
    if p_ref is not None:
        ok, d = N.check_bf16(host64(p_out), p_ref)
        assert ok, f"softmax max ulp {d}"
    assert kinds == {"add", "rmsnorm", "swiglu", "softmax"}

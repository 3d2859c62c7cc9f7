"""GPU parity at full size for the further prefill workloads that `bench.py --workloads`
times (Gated DeltaNet, DeltaNet, gates from pre-activations, and q/k from
pre-activations): the whole batch (B=8, T=8192, H=32, d=128, bf16, chunk 64: the fused
pass) through the C ABI, the fp64 oracle on every (sequence, head) pair over its full
length. The inputs come from the same kda_synth generators as the bench's; the oracle
forms the gates and q, k with oracle.gate_prologue and oracle.qk_prologue.

Bar: relative L2 error of o and of hT <= 2e-2 (bf16 I/O) over the whole batch and for
every (sequence, head), every row of o within kda_testlib.ROW_TOL.
"""
import numpy as np
import pytest

import kda_synth
import oracle
from kda_testlib import assert_parity, say, workload_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["batched_gdn", "batched_deltanet", "batched_preact", "batched_preact_qk"])
def test_further_workload_full(name):
    import torch
    import gated_delta_rule_48_amd as kda
    w = kda_synth.WORKLOADS[name]
    B, T, H, d = len(w.seqlens), w.seqlens[0], w.H, w.dk
    say(f"[{name}] B={B} T={T} H={H} d={d} {w.io} chunk {w.chunk} gate={w.gate}")
    x = workload_inputs(w)
    if w.gate == "preact_qk":
        r = kda_synth.gen_qk_preact(B * T, H, d, w.io, w.seed)
        x["q"], x["k"] = r["q"], r["k"]
    p = kda_synth.gen_preact(B * T, H, d, w.io, w.seed) if w.gate.startswith("preact") else None
    dev = torch.device("cuda:0")
    bf = lambda a, *s: torch.from_numpy(a).to(dev).to(torch.bfloat16).reshape((B, T) + s)  # noqa: E731
    q, k, v = bf(x["q"], H, d), bf(x["k"], H, d), bf(x["v"], H, d)
    if p is not None:
        o, hT = kda.chunk_fwd_preact(q, k, v, bf(p["a"], H, d), torch.from_numpy(p["A_log"]).to(dev),
                                     torch.from_numpy(p["dt_bias"]).to(dev),
                                     torch.from_numpy(p["b"]).to(dev).reshape(B, T, H), scale=w.scale,
                                     chunk=w.chunk, qk_norm=w.gate == "preact_qk")
    else:
        la = torch.from_numpy(x["log_alpha"]).to(dev).reshape(B, T, H, d)
        la = la[..., 0].contiguous() if w.gate == "head" else None
        o, hT = kda.chunk_fwd(q, k, v, la, torch.from_numpy(x["beta"]).to(dev).reshape(B, T, H), scale=w.scale,
                              chunk=w.chunk)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().reshape(B * T, H, d)
    hT = hT.cpu().numpy()
    qs, ks = x["q"], x["k"]
    if p is not None:
        la, beta = oracle.gate_prologue(p["a"], p["A_log"], p["dt_bias"], p["b"])
        if w.gate == "preact_qk":
            qs, ks = oracle.qk_prologue(qs), oracle.qk_prologue(ks)
    else:
        beta = x["beta"]
        if w.gate == "head":
            la = np.repeat(x["log_alpha"][..., :1], d, axis=-1)
        else:
            la = np.zeros_like(x["log_alpha"])
    cu = x["cu_seqlens"]
    o_ref, h_ref = oracle.kda_reference(qs, ks, x["v"], la, beta, w.scale, cu_seqlens=cu)
    del la, beta, qs, ks
    assert_parity(o, o_ref, hT, h_ref, "bf16", name, cu=cu)

"""GPU parity of the backward pass (kda_chunk_bwd, through its C ABI) against the fp64
oracle (autograd of the token loop, itself pinned by finite differences of the C forward
oracle).

Bar: relative L2 error of every gradient (dq, dk, dv, dlog_alpha, dbeta, dh0), each over
its whole tensor, <= 1e-4 with fp32 I/O and <= 2e-2 with bf16 I/O (the library's bars). Inputs are seeded synthetic draws
(kda_synth): the forward workload recipe, and N(0,1) loss gradients.
"""
import numpy as np
import pytest

import kda_synth
import oracle
from kda_testlib import TOL, rel_l2, say

pytestmark = pytest.mark.gpu
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0")


def _inputs(B, T, H, dk, dv, gates, seed, h0=True, dhT=True, io="f32"):
    x = kda_synth.gen_sequences((T,) * B, H, dk, dv, io, gates, "normal" if h0 else "zero", seed)
    shp = lambda a: a.reshape((B, T) + a.shape[1:])  # noqa: E731
    d = {n: shp(x[n]) for n in ("q", "k", "v", "log_alpha", "beta")}
    d["h0"] = x["h0"] if h0 else None
    g = kda_synth.gen_grad_outputs(B, T, H, dk, dv, seed)
    d["dout"] = kda_synth.round_bf16(g["dout"]) if io == "bf16" else g["dout"]
    d["dhT"] = g["dhT"] if dhT else None
    return d


def _run(d, scale, io="f32"):
    import torch
    import gated_delta_rule_48_amd as kda
    t = {n: (None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()) for n, x in d.items()}
    if io == "bf16":  # the values are bf16-representable already
        for n in ("q", "k", "v", "dout"):
            t[n] = t[n].to(torch.bfloat16)
    out = kda.chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["dout"], scale=scale, h0=t["h0"],
                        dhT=t["dhT"])
    torch.cuda.synchronize()
    return {n: (None if x is None else x.float().cpu().numpy()) for n, x in zip(NAMES, out)}


def _check(name, B, T, H, dk, dv, gates="main", seed=0, h0=True, dhT=True, io="f32"):
    say(f"[{name}] B={B} T={T} H={H} dk={dk} dv={dv} gates={gates} h0={h0} dhT={dhT} io={io}")
    d = _inputs(B, T, H, dk, dv, gates, seed, h0, dhT, io)
    scale = dk ** -0.5
    got = _run(d, scale, io)
    ref = oracle.kda_backward_reference(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], scale, d["dout"],
                                        dhT=d["dhT"], h0=d["h0"])
    errs = {}
    for n in NAMES:
        if n == "dh0" and not h0:
            assert got[n] is None
            continue
        assert np.all(np.isfinite(got[n])), n
        errs[n] = rel_l2(got[n], ref[n])
    say(f"[{name}] rel_l2 " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[io], (n, e)


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 128)])
def test_bwd_bf16(dk, dv):
    # bf16 q, k, v, dout and dq, dk, dv; fp32 gates, states and arithmetic
    _check("bwd-bf16", 2, 150, 2, dk, dv, seed=31 + dk + dv, io="bf16")


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("T", [64, 100, 200])
def test_bwd_shapes(dk, dv, T):
    _check("bwd", 2, T, 2, dk, dv, seed=T + dk + dv)


def test_bwd_strong_gates_and_short_sequences():
    _check("strong", 2, 130, 2, 128, 128, gates="strong", seed=3)
    _check("short", 3, 1, 2, 64, 64, seed=4)
    _check("weak", 1, 65, 3, 64, 64, gates="weak", seed=5)


def test_bwd_without_h0_or_dhT():
    _check("no-h0", 2, 90, 2, 64, 64, seed=6, h0=False)
    _check("no-dhT", 2, 90, 2, 64, 64, seed=7, dhT=False)


def test_bwd_empty_sequence():
    # T = 0: every gradient is empty and dh0 = dhT
    import torch
    import gated_delta_rule_48_amd as kda
    B, H, d = 2, 3, 64
    z = lambda *s: torch.zeros(s, device="cuda")  # noqa: E731
    dhT = torch.randn(B, H, d, d, device="cuda")
    out = kda.chunk_bwd(z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H), z(B, 0, H, d),
                        h0=torch.randn(B, H, d, d, device="cuda"), dhT=dhT)
    torch.cuda.synchronize()
    assert torch.equal(out[5], dhT)
    assert all(x.numel() == 0 for x in out[:5])


def test_bwd_full_size_sampled():
    """The backward at the batched workload's shape (B=8, T=8192, H=32, d=128, fp32, weak
    gates, as `bench.py --bwd` times it): the whole batch on the GPU, the oracle on two
    sampled (sequence, head) pairs over their full length."""
    import torch
    import gated_delta_rule_48_amd as kda
    w = kda_synth.WORKLOADS["batched"]
    B, T, H, d = len(w.seqlens), w.seqlens[0], w.H, w.dk
    say(f"[bwd-full] B={B} T={T} H={H} d={d} fp32 gates={w.gates}")
    x = kda_synth.gen_sequences(w.seqlens, H, d, d, "f32", w.gates, "zero", w.seed)
    gr = kda_synth.gen_grad_outputs(B, T, H, d, d, w.seed)
    t = {n: torch.from_numpy(x[n].reshape((B, T) + x[n].shape[1:])).cuda()
         for n in ("q", "k", "v", "log_alpha", "beta")}
    dout, dhT = torch.from_numpy(gr["dout"]).cuda(), torch.from_numpy(gr["dhT"]).cuda()
    out = kda.chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], dout, scale=d ** -0.5, dhT=dhT)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1)):
        sl = lambda a: a[b:b + 1, :, h:h + 1].cpu().numpy()  # noqa: E731
        ref = oracle.kda_backward_reference(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["log_alpha"]),
                                            sl(t["beta"]), d ** -0.5, gr["dout"][b:b + 1, :, h:h + 1],
                                            dhT=gr["dhT"][b:b + 1, h:h + 1])
        errs = {n: rel_l2(sl(out[i]), ref[n]) for i, n in enumerate(NAMES[:5])}
        say(f"[bwd-full] (b={b}, h={h}) rel_l2 " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
        for n, e in errs.items():
            assert e <= TOL["f32"], (n, e)

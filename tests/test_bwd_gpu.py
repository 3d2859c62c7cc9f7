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


# bf16 I/O with d_k = d_v = 128 runs the matrix-core pass (bf16 products, kda_bwd_bf16.hip):
# ragged and exact chunk ends, one token, several heads and sequences
@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (2, 64, 2), (1, 65, 3), (3, 200, 2), (2, 333, 1)])
def test_bwd_bf16_matrix_core_shapes(B, T, H):
    _check("bwd-bf16-mc", B, T, H, 128, 128, seed=7 * T + B + H, io="bf16")


def test_bwd_bf16_matrix_core_options():
    _check("bwd-bf16-mc no-h0", 2, 130, 2, 128, 128, seed=11, h0=False, io="bf16")
    _check("bwd-bf16-mc no-dhT", 2, 130, 2, 128, 128, seed=12, dhT=False, io="bf16")
    _check("bwd-bf16-mc strong", 2, 130, 2, 128, 128, gates="strong", seed=13, io="bf16")
    _check("bwd-bf16-mc weak", 1, 190, 2, 128, 128, gates="weak", seed=14, io="bf16")


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


def test_bwd_full_size_sampled_bf16():
    """The matrix-core backward at the batched workload's shape (B=8, T=8192, H=32, d=128,
    bf16 I/O, weak gates, as the bench times it): the whole batch on the GPU, the oracle on
    two sampled (sequence, head) pairs over their full length."""
    import torch
    import gated_delta_rule_48_amd as kda
    w = kda_synth.WORKLOADS["batched"]
    B, T, H, d = len(w.seqlens), w.seqlens[0], w.H, w.dk
    say(f"[bwd-full-bf16] B={B} T={T} H={H} d={d} bf16 gates={w.gates}")
    x = kda_synth.gen_sequences(w.seqlens, H, d, d, "bf16", w.gates, "zero", w.seed)
    gr = kda_synth.gen_grad_outputs(B, T, H, d, d, w.seed)
    dout_np = kda_synth.round_bf16(gr["dout"])
    t = {n: torch.from_numpy(x[n].reshape((B, T) + x[n].shape[1:])).cuda()
         for n in ("q", "k", "v", "log_alpha", "beta")}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(torch.bfloat16)
    dout, dhT = torch.from_numpy(dout_np).cuda().to(torch.bfloat16), torch.from_numpy(gr["dhT"]).cuda()
    out = kda.chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], dout, scale=d ** -0.5, dhT=dhT)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1)):
        sl = lambda a: a[b:b + 1, :, h:h + 1].float().cpu().numpy()  # noqa: E731
        ref = oracle.kda_backward_reference(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["log_alpha"]),
                                            sl(t["beta"]), d ** -0.5, dout_np[b:b + 1, :, h:h + 1],
                                            dhT=gr["dhT"][b:b + 1, h:h + 1])
        errs = {n: rel_l2(sl(out[i]), ref[n]) for i, n in enumerate(NAMES[:5])}
        say(f"[bwd-full-bf16] (b={b}, h={h}) rel_l2 " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
        for n, e in errs.items():
            assert e <= TOL["bf16"], (n, e)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_bitwise_deterministic(io):
    """Every reduction in the backward runs in a fixed order (no atomics), so two calls on
    the same inputs give the same bits, also when the second call's workspace starts out
    holding other values."""
    import torch
    import gated_delta_rule_48_amd as kda
    B, T, H, d = 2, 333, 4, 128
    say(f"[bwd-det] B={B} T={T} H={H} d={d} io={io}")
    x = _inputs(B, T, H, d, d, "main", 41, io=io)
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).cuda() for n, a in x.items()}
    if io == "bf16":
        for n in ("q", "k", "v", "dout"):
            t[n] = t[n].to(torch.bfloat16)
    need = kda.chunk_bwd_workspace_bytes(B, T, H, d, d, io=kda.KDA_BF16 if io == "bf16" else kda.KDA_F32)
    runs = []
    for fill in (0, 0x7F):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        runs.append(kda.chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["dout"], h0=t["h0"],
                                  dhT=t["dhT"], workspace=ws))
    torch.cuda.synchronize()
    for n, a, b in zip(NAMES, *runs):
        assert torch.equal(a, b), n


def _varlen_case(seqlens, H, seed, h0=True, dhT=True, mutate=None):
    """Packed bf16 sequences at d = 128 through kda_chunk_bwd_varlen, and the oracle run on
    each sequence on its own (sequences are independent). mutate(x) may change the drawn
    inputs first."""
    import torch
    import gated_delta_rule_48_amd as kda
    d, n = 128, len(seqlens)
    x = kda_synth.gen_sequences(seqlens, H, d, d, "bf16", "main", "normal" if h0 else "zero", seed)
    if mutate is not None:
        mutate(x)
    T = int(sum(seqlens))
    do = kda_synth.round_bf16(kda_synth.gen_grad_outputs(1, T, H, d, d, seed)["dout"][0])
    dh = kda_synth.gen_grad_outputs(n, 0, H, d, d, seed + 1)["dhT"] if dhT else None
    cu = x["cu_seqlens"]
    t = {m: torch.from_numpy(np.ascontiguousarray(x[m])).cuda() for m in ("q", "k", "v", "log_alpha", "beta")}
    for m in ("q", "k", "v"):
        t[m] = t[m].to(torch.bfloat16)
    got = kda.chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"],
                        torch.from_numpy(do).cuda().to(torch.bfloat16), scale=d ** -0.5,
                        h0=None if x["h0"] is None else torch.from_numpy(x["h0"]).cuda(),
                        dhT=None if dh is None else torch.from_numpy(dh).cuda(),
                        cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    got = {nm: (None if a is None else a.float().cpu().numpy()) for nm, a in zip(NAMES, got)}
    refs = []
    for s in range(n):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda z: z[a:b][None]  # noqa: E731
        refs.append(oracle.kda_backward_reference(
            sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["log_alpha"]), sl(x["beta"]), d ** -0.5, sl(do),
            dhT=None if dh is None else dh[s:s + 1], h0=None if x["h0"] is None else x["h0"][s:s + 1]))
    return got, refs


def _check_varlen(name, got, refs):
    errs = {}
    for nm in NAMES[:5]:
        ref = np.concatenate([r[nm][0] for r in refs], axis=0)
        assert np.all(np.isfinite(got[nm])), nm
        errs[nm] = rel_l2(got[nm], ref)
    errs["dh0"] = rel_l2(got["dh0"], np.concatenate([r["dh0"] for r in refs], axis=0))
    say(f"[{name}] rel_l2 " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    for nm, e in errs.items():
        assert e <= TOL["bf16"], (nm, e)


@pytest.mark.parametrize("seqlens,H", [((0, 1, 63, 64, 65, 130, 0, 200), 3), ((300, 5), 2)])
def test_bwd_varlen_packed_ragged(seqlens, H):
    say(f"[bwd-varlen] seqlens={seqlens} H={H} bf16 d=128")
    got, refs = _varlen_case(seqlens, H, seed=51 + H)
    _check_varlen("bwd-varlen", got, refs)


def test_bwd_varlen_equals_batched():
    """Equal lengths given packed with cu_seqlens and given as [B, T, H, d]: the same chunks,
    the same kernels, the same bits."""
    import torch
    import gated_delta_rule_48_amd as kda
    B, T, H, d = 2, 150, 3, 128
    x = _inputs(B, T, H, d, d, "main", 61, io="bf16")
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).cuda() for n, a in x.items()}
    for n in ("q", "k", "v", "dout"):
        t[n] = t[n].to(torch.bfloat16)
    a = kda.chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["dout"], h0=t["h0"], dhT=t["dhT"])
    flat = lambda z: z.reshape((B * T,) + tuple(z.shape[2:]))  # noqa: E731
    cu = torch.tensor([0, T, 2 * T], dtype=torch.int32, device="cuda")
    b = kda.chunk_bwd(flat(t["q"]), flat(t["k"]), flat(t["v"]), flat(t["log_alpha"]), flat(t["beta"]),
                      flat(t["dout"]), h0=t["h0"], dhT=t["dhT"], cu_seqlens=cu)
    torch.cuda.synchronize()
    for n, x1, x2 in zip(NAMES, a, b):
        assert torch.equal(flat(x1) if n != "dh0" else x1, x2), n


# Chunks whose summed log alpha falls below -160 on some key channel leave the range of the
# chunked passes' midpoint factors: their (sequence, head) pairs are recomputed token by
# token (kda_bwd_tok.hip) after either pass. Chunk sums near -500 and -2000 per channel on
# every chunk, and on one chunk of one pair among ordinary ones.
@pytest.mark.parametrize("gates", ["sum500", "sum2000"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 128)])
def test_bwd_strong_chunks_direct(gates, dk, dv):
    _check("bwd-tok " + gates, 2, 150, 2, dk, dv, gates=gates, seed=71 + dk + dv)


@pytest.mark.parametrize("gates", ["sum500", "sum2000"])
def test_bwd_strong_chunks_matrix_core(gates):
    _check("bwd-tok-mc " + gates, 2, 150, 2, 128, 128, gates=gates, seed=73, io="bf16")


def _one_strong_chunk(B, T, H, dk, dv, seed, io):
    """Ordinary gates, except chunk 1 (rows 64 .. 127) of sequence B - 1, head 0, whose log
    alpha is -8 on every channel (a chunk sum of -512)."""
    name = f"bwd-tok one-chunk {io} dk={dk} dv={dv}"
    say(f"[{name}] B={B} T={T} H={H}")
    d = _inputs(B, T, H, dk, dv, "main", seed, io=io)
    d["log_alpha"][B - 1, 64:128, 0, :] = -8.0
    scale = dk ** -0.5
    got = _run(d, scale, io)
    ref = oracle.kda_backward_reference(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], scale, d["dout"],
                                        dhT=d["dhT"], h0=d["h0"])
    errs = {}
    for n in NAMES:
        assert np.all(np.isfinite(got[n])), n
        errs[n] = rel_l2(got[n], ref[n])
        # the recomputed pair on its own, and one pair the chunked pass kept
        if n == "dbeta":
            a, b = got[n][B - 1, :, 0], ref[n][B - 1, :, 0]
            c, e = got[n][0, :, H - 1], ref[n][0, :, H - 1]
        elif n == "dh0":
            a, b = got[n][B - 1, 0], ref[n][B - 1, 0]
            c, e = got[n][0, H - 1], ref[n][0, H - 1]
        else:
            a, b = got[n][B - 1, :, 0], ref[n][B - 1, :, 0]
            c, e = got[n][0, :, H - 1], ref[n][0, :, H - 1]
        errs[n + "[strong pair]"] = rel_l2(a, b)
        errs[n + "[other pair]"] = rel_l2(c, e)
    say(f"[{name}] rel_l2 " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[io], (n, e)


@pytest.mark.parametrize("io,dk,dv", [("f32", 64, 64), ("f32", 128, 128), ("bf16", 128, 128), ("bf16", 64, 128)])
def test_bwd_one_strong_chunk(io, dk, dv):
    _one_strong_chunk(2, 200, 3, dk, dv, 81 + dk, io)


def test_bwd_varlen_strong_sequence():
    """Packed sequences, the third of which has a chunk of summed log alpha -512 on head 1."""
    seqlens, H = (70, 0, 200, 1, 129), 2

    def mutate(x):
        a = int(x["cu_seqlens"][2])
        x["log_alpha"][a + 64:a + 128, 1, :] = -8.0

    say(f"[bwd-tok varlen] seqlens={seqlens} H={H} bf16 d=128")
    got, refs = _varlen_case(seqlens, H, seed=91, mutate=mutate)
    _check_varlen("bwd-tok varlen", got, refs)

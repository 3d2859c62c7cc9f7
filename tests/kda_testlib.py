"""Helpers shared by the GPU parity tests: device transfer, calls through the
binding (which calls the C ABI), oracle runs on sampled heads, and the
relative-L2 metric."""
from __future__ import annotations

import sys

import numpy as np

import kda_synth
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}  # relative L2 bounds of the fp32 and bf16-input paths


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def to_dev(x, io, dev="cuda"):
    """numpy inputs (fp32 arrays, q/k/v already bf16-representable) -> torch tensors."""
    import torch
    t = {}
    iod = torch.bfloat16 if io == "bf16" else torch.float32
    for n in ("q", "k", "v"):
        t[n] = torch.from_numpy(np.ascontiguousarray(x[n])).to(dev).to(iod)
    for n in ("log_alpha", "beta"):
        t[n] = torch.from_numpy(np.ascontiguousarray(x[n])).to(dev)
    t["h0"] = None if x.get("h0") is None else torch.from_numpy(np.ascontiguousarray(x["h0"])).to(dev)
    t["cu_seqlens"] = torch.from_numpy(np.ascontiguousarray(x["cu_seqlens"])).to(dev)
    return t


def gate_view(log_alpha, gate):
    """The decays the library is given for a gate kind: all of them ("channel"),
    channel 0's for every channel ("head": one per token and head), or none."""
    if gate == "channel":
        return log_alpha
    if gate == "head":
        return log_alpha[..., 0].contiguous()
    return None


def with_gate(x, gate):
    """Generator output with its per-channel decays replaced by what a gate kind
    means on every channel (the oracle's input): channel 0's decay broadcast
    ("head"), or zero ("none")."""
    y = dict(x)
    if gate == "head":
        y["log_alpha"] = np.repeat(x["log_alpha"][..., :1], x["log_alpha"].shape[-1], axis=-1).copy()
    elif gate == "none":
        y["log_alpha"] = np.zeros_like(x["log_alpha"])
    return y


def run_packed(x, io, chunk, varlen=True, B=None, T=None, h0=True, hT=True, dev="cuda", gate="channel"):
    """Run kda_chunk_fwd_gated on generator output. varlen=True passes cu_seqlens; else
    the sequences must have equal length and are passed as [B, T, H, d]. `gate`
    selects which decays the library is given (gate_view)."""
    import torch
    import gated_delta_rule_48_amd as kda
    t = to_dev(x, io, dev)
    if varlen:
        o, hT_ = kda.chunk_fwd(t["q"], t["k"], t["v"], gate_view(t["log_alpha"], gate), t["beta"],
                               h0=t["h0"] if h0 else None, cu_seqlens=t["cu_seqlens"], chunk=chunk,
                               output_final_state=hT)
    else:
        Tt, H, dk = t["q"].shape
        dv = t["v"].shape[-1]
        r = lambda a, d: a.reshape(B, T, H, d)  # noqa: E731
        la = gate_view(r(t["log_alpha"], dk), gate)
        o, hT_ = kda.chunk_fwd(r(t["q"], dk), r(t["k"], dk), r(t["v"], dv), la,
                               t["beta"].reshape(B, T, H), h0=t["h0"] if h0 else None, chunk=chunk,
                               output_final_state=hT)
        o = o.reshape(Tt, H, dv)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), (None if hT_ is None else hT_.cpu().numpy())


def oracle_run(x, heads=None, seqs=None, h0=True):
    """fp64 oracle on all heads/sequences, or on the listed ones only (heads are
    independent, so a subset is exact). Returns (o [T, len(heads), dv] restricted
    to the listed sequences' tokens, hT [len(seqs), len(heads), dk, dv], token index)."""
    cu = np.asarray(x["cu_seqlens"], dtype=np.int64)
    n = len(cu) - 1
    seqs = list(range(n)) if seqs is None else list(seqs)
    H = x["q"].shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]).astype(np.int64)
    sub_cu = np.concatenate([[0], np.cumsum([cu[s + 1] - cu[s] for s in seqs])]).astype(np.int64)
    pick = lambda a: np.ascontiguousarray(a[idx][:, heads])  # noqa: E731
    h0a = None
    if h0 and x.get("h0") is not None:
        h0a = np.ascontiguousarray(x["h0"][seqs][:, heads])
    dk = x["q"].shape[2]
    o, hT = oracle.kda_reference(pick(x["q"]), pick(x["k"]), pick(x["v"]), pick(x["log_alpha"]),
                                 pick(x["beta"]), dk ** -0.5, h0=h0a, cu_seqlens=sub_cu)
    return o, hT, idx


def gen(seqlens, H, dk, dv, io, gates="main", h0="normal", seed=0):
    return kda_synth.gen_sequences(tuple(seqlens), H, dk, dv, io, gates, h0, seed)

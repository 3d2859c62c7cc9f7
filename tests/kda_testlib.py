"""Helpers shared by the GPU parity tests: device transfer, calls through the
binding (which calls the C ABI), oracle runs on sampled heads, and the
relative-L2 metric."""
from __future__ import annotations

import sys

import numpy as np

import kda_synth
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}  # relative L2 bounds of the fp32 and bf16-input paths
# Per-row bound: the error of one (token, head) row of o, over the larger of that row's
# norm and the RMS row norm of its (sequence, head). On the bf16 path every product
# reads operands rounded once to bf16 (unit roundoff u = 2^-8) and o itself is rounded
# once, so a row's error is a sum of a few terms of order u times the row's scale; the
# bound is 16 u. On the fp32 path u = 2^-24 and the bound is 2^-10, far above rounding
# but far below the O(1) error of a row computed from wrong data.
ROW_TOL = {"f32": 2.0 ** -10, "bf16": 16 * 2.0 ** -8}
# The per-head bar (TOL) applies to (sequence, head) pairs of at least one chunk of rows.
# A shorter pair's relative L2 is that of a few rows, and one row's relative error can
# reach about 9 u on the bf16 path where a small dot product cancels (q . k of two random
# unit vectors at d = 128 is about 0.09 while sum |q_c k_c| is about 0.8, and each term
# carries a rounding of order u); such pairs are held to ROW_TOL, row by row.
HEAD_MIN_ROWS = 64
PARITY_LOG = []  # every assert_parity line of this process, printed in pytest's summary


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def parity_stats(o, o_ref, cu=None):
    """Errors of o [T, H, d] against o_ref: (whole-tensor relative L2, worst relative L2 of
    one (sequence, head) of at least HEAD_MIN_ROWS rows, where it is, worst per-row ratio,
    where it is). Sequences are
    the cu_seqlens ranges (one sequence if None); per-row ratios are each (token, head)
    row's error over max(its reference norm, the RMS row norm of its (sequence, head))."""
    T = o.shape[0]
    cu = [0, T] if cu is None else [int(c) for c in cu]
    num = den = 0.0
    worst_h, at_h, worst_r, at_r = 0.0, None, 0.0, None
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b <= a:
            continue
        x = np.asarray(o[a:b], dtype=np.float64)
        r = np.asarray(o_ref[a:b], dtype=np.float64)
        d2 = np.sum((x - r) ** 2, axis=-1)          # [len, H]
        r2 = np.sum(r * r, axis=-1)
        num += float(d2.sum())
        den += float(r2.sum())
        hn, hd = d2.sum(axis=0), r2.sum(axis=0)     # per head
        if b - a >= HEAD_MIN_ROWS:
            with np.errstate(divide="ignore", invalid="ignore"):
                rel_h = np.where(hd > 0, np.sqrt(hn / np.where(hd > 0, hd, 1)), np.sqrt(hn))
            h = int(np.argmax(rel_h))
            if rel_h[h] > worst_h:
                worst_h, at_h = float(rel_h[h]), (s, h)
        rms = np.sqrt(hd / (b - a))                 # [H]
        scl = np.maximum(np.sqrt(r2), rms[None, :])
        ratio = np.sqrt(d2) / np.maximum(scl, 1e-30)
        t, hh = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        if ratio[t, hh] > worst_r:
            worst_r, at_r = float(ratio[t, hh]), (a + int(t), int(hh))
    whole = float(np.sqrt(num / den)) if den > 0 else float(np.sqrt(num))
    return whole, worst_h, at_h, worst_r, at_r


def state_stats(hT, h_ref):
    """(whole relative L2, worst relative L2 of one (sequence, head) state, where) of
    states [n, H, dk, dv]."""
    x = np.asarray(hT, dtype=np.float64)
    r = np.asarray(h_ref, dtype=np.float64)
    d2 = np.sum((x - r) ** 2, axis=(2, 3))
    r2 = np.sum(r * r, axis=(2, 3))
    whole = float(np.sqrt(d2.sum() / r2.sum())) if r2.sum() > 0 else float(np.sqrt(d2.sum()))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(r2 > 0, np.sqrt(d2 / np.where(r2 > 0, r2, 1)), np.sqrt(d2))
    i = np.unravel_index(int(np.argmax(rel)), rel.shape)
    return whole, float(rel[i]), tuple(int(v) for v in i)


def assert_parity(o, o_ref, hT, h_ref, io, name, cu=None, tol=None, row_tol=None):
    """The parity bar: o and the final states, each as a whole tensor and for every (sequence,
    head) on its own (o: pairs of at least HEAD_MIN_ROWS rows), within the relative L2
    bound of the io path; every row of o within the per-row bound. Logs the worst head and
    row."""
    tol = TOL[io] if tol is None else tol
    row_tol = ROW_TOL[io] if row_tol is None else row_tol
    assert np.all(np.isfinite(o)), f"{name}: non-finite o"
    eo, eho, at_h, er, at_r = parity_stats(o, o_ref, cu)
    msg = f"[{name}] rel_l2 o={eo:.2e} worst head {eho:.2e} at (seq, head) {at_h}, worst row {er:.2e} at {at_r}"
    if hT is not None:
        assert np.all(np.isfinite(hT)), f"{name}: non-finite hT"
        eh, ehh, at_s = state_stats(hT, h_ref)
        msg += f"; hT={eh:.2e} worst state {ehh:.2e} at {at_s}"
    say(msg)
    PARITY_LOG.append(msg)
    assert eo <= tol and eho <= tol, msg
    assert er <= row_tol, msg
    if hT is not None:
        assert eh <= tol and ehh <= tol, msg
    return eo


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


_WORKLOAD_DRAWS = {}


def workload_inputs(w):
    """kda_synth.gen_workload(w), drawn once per process for each distinct draw (the
    batched workload and its gate-kind variants share one); a new dict each call, whose
    arrays must not be written."""
    key = (w.seqlens, w.H, w.dk, w.dv, w.io, w.gates, w.h0, w.seed)
    if key not in _WORKLOAD_DRAWS:
        _WORKLOAD_DRAWS[key] = kda_synth.gen_workload(w)
    return dict(_WORKLOAD_DRAWS[key])


def gen(seqlens, H, dk, dv, io, gates="main", h0="normal", seed=0):
    return kda_synth.gen_sequences(tuple(seqlens), H, dk, dv, io, gates, h0, seed)

"""ctypes wrapper and build step for the fp64 KDA oracle (test infrastructure).

The oracle itself is plain C in kda_oracle.c: a token-by-token fp64 loop of
the KDA gated delta rule. This wrapper only converts arrays to contiguous fp64
and calls it. It is "parity pinned": tests/test_oracle_pins.py ties it to the
worked 2x2 examples of the "ten questions" page and to closed forms, brute
force and invariants. The prologue functions and the softmax-attention decode
step (the comparator of the KDA decode step) are numpy in fp64 here, each
pinned the same way.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_libs = {}


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile kda_oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load(path: Optional[str] = None):
    """Load the oracle library (or, for the mutation tests, another build of it)."""
    path = path or _LIB
    if path not in _libs:
        if path == _LIB and (not os.path.exists(_LIB)
                             or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.kda_oracle_fwd.argtypes = [ctypes.c_int64, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       P, P, P, P, P, ctypes.c_double, ctypes.c_int, P, P, P,
                                       ctypes.c_int]
        lib.kda_oracle_fwd.restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def kda_reference(q, k, v, log_alpha, beta, scale: float, h0=None, cu_seqlens=None,
                  delta_rule: bool = True, threads: Optional[int] = None,
                  lib: Optional[str] = None):
    """fp64 oracle over packed sequences.

    q, k [T, H, dk]; v [T, H, dv]; log_alpha [T, H, dk]; beta [T, H];
    h0 [n_seqs, H, dk, dv] or None; cu_seqlens [n_seqs + 1] or None (one sequence).
    Returns (o [T, H, dv], hT [n_seqs, H, dk, dv]) as fp64 arrays.
    """
    q, k, v, log_alpha, beta = map(_f64, (q, k, v, log_alpha, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and v.shape == (T, H, dv)
    assert log_alpha.shape == (T, H, dk) and beta.shape == (T, H)
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], dtype=np.int64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    n_seqs = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T
    if h0 is not None:
        h0 = _f64(h0)
        assert h0.shape == (n_seqs, H, dk, dv)
    o = np.zeros((T, H, dv), dtype=np.float64)
    hT = np.zeros((n_seqs, H, dk, dv), dtype=np.float64)
    if threads is None:
        threads = max(1, min(os.cpu_count() or 1, n_seqs * H))
    rc = _load(lib).kda_oracle_fwd(n_seqs, _ptr(cu), H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(log_alpha), _ptr(beta), float(scale), int(bool(delta_rule)),
                                _ptr(h0), _ptr(o), _ptr(hT), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed with code {rc}")
    return o, hT


def gate_prologue(a, A_log, dt_bias, b):
    """The gates formed from their pre-activations, in fp64, as the gate line of KDA's
    open-source layer that the "ten questions" page quotes (Q9: g = -exp(A_log)
    softplus(f(x) + dt_bias), alpha = e^g; beta through a sigmoid):

        log_alpha[t, h, c] = -exp(A_log[h]) * softplus(a[t, h, c] + dt_bias[h, c])
        beta[t, h]         = sigmoid(b[t, h])

    softplus(x) = log(1 + e^x) (np.logaddexp(0, x)), sigmoid(x) = 1 / (1 + e^-x).
    a [..., H, dk]; A_log [H]; dt_bias [H, dk]; b [..., H]. Returns (log_alpha, beta)."""
    a, A_log, dt_bias, b = map(_f64, (a, A_log, dt_bias, b))
    log_alpha = -np.exp(A_log)[:, None] * np.logaddexp(0.0, a + dt_bias)
    beta = 1.0 / (1.0 + np.exp(-b))
    return log_alpha, beta


def qk_prologue(x, eps: float = 1e-12):
    """q or k from its pre-activation, in fp64, as the delta-rule layer of the essay
    "22,580: from GPT-2 to Kimi K3" (section 5.2's forward: normalize(silu(.)) over the
    head dimension, so that a key read back with itself returns its value):

        silu(x) = x / (1 + e^-x),   result = silu(x) / max(||silu(x)||_2, eps)

    over the last axis (eps as torch's normalize)."""
    x = _f64(x)
    s = x / (1.0 + np.exp(-x))
    n = np.sqrt(np.sum(s * s, axis=-1, keepdims=True))
    return s / np.maximum(n, eps)


def attn_decode_reference(q, k_cache, v_cache, seq_lens=None, scale: float = None):
    """Softmax attention of one new token per sequence over a KV cache, in fp64: the
    causal softmax attention of the essay "22,580: from GPT-2 to Kimi K3" (section 2.2)
    for the newest position, against the keys and values kept for all positions so far
    (its section 2.3, the KV cache). For each sequence b and query head h, with cached
    head j = h // (H // H_kv) and len = seq_lens[b] (all T_max rows if None):

        s_t = scale * q[b, h] . k_cache[b, j, t]          (t < len)
        o[b, h] = sum_t exp(s_t) v_cache[b, j, t] / sum_t exp(s_t)

    computed with the largest s_t subtracted first (the same value, without overflow).
    An empty cache (len = 0) gives o = 0. q [B, H, d]; caches [B, H_kv, T_max, d];
    scale defaults to d^-1/2. Returns o [B, H, d] fp64."""
    q, K, V = _f64(q), _f64(k_cache), _f64(v_cache)
    B, H, d = q.shape
    H_kv, T_max = K.shape[1], K.shape[2]
    G = H // H_kv
    if scale is None:
        scale = d ** -0.5
    o = np.zeros((B, H, d))
    for b in range(B):
        n = T_max if seq_lens is None else min(max(int(seq_lens[b]), 0), T_max)
        if n == 0:
            continue
        for h in range(H):
            j = h // G
            s = scale * (K[b, j, :n] @ q[b, h])
            w = np.exp(s - s.max())
            o[b, h] = (w @ V[b, j, :n]) / w.sum()
    return o


def kda_backward_reference(q, k, v, log_alpha, beta, scale: float, do, dhT=None, h0=None):
    """Gradients of the KDA recurrence, in fp64: reverse-mode differentiation (torch.autograd
    on the CPU) of the plain token loop of the "ten questions" page's update (its closing
    symbol-by-symbol reading) in the order of the bra-ket derivation page's state-update
    equations, for equal-length sequences:

        S~ = Diag(exp(log_alpha_t)) S;  e = beta_t (v_t - S~^T k_t);  S = S~ + k_t e^T;
        o_t = scale S^T q_t

    The pages derive no gradient; this is the derivative of that loop and nothing else.
    q, k [B, T, H, dk]; v, do [B, T, H, dv]; log_alpha [B, T, H, dk]; beta [B, T, H];
    h0, dhT [B, H, dk, dv] or None (zero). The differentiated loss is
    sum(o * do) + sum(hT * dhT). Returns a dict of fp64 numpy arrays: dq, dk, dv,
    dlog_alpha, dbeta, dh0."""
    import torch
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    t64 = lambda a: torch.tensor(_f64(a), dtype=torch.float64)  # noqa: E731
    xs = [t64(a).requires_grad_(True) for a in (q, k, v, log_alpha, beta)]
    S0 = t64(h0) if h0 is not None else torch.zeros((B, H, dk, dv), dtype=torch.float64)
    S0.requires_grad_(True)
    qq, kk, vv, la, bb = xs
    S = S0
    outs = []
    for t in range(T):
        St = torch.exp(la[:, t])[..., None] * S
        e = bb[:, t][..., None] * (vv[:, t] - torch.einsum("bhkv,bhk->bhv", St, kk[:, t]))
        S = St + kk[:, t][..., None] * e[..., None, :]
        outs.append(scale * torch.einsum("bhkv,bhk->bhv", S, qq[:, t]))
    loss = (torch.stack(outs, dim=1) * t64(do)).sum() if T > 0 else torch.zeros((), dtype=torch.float64)
    if dhT is not None:
        loss = loss + (S * t64(dhT)).sum()
    grads = torch.autograd.grad(loss, xs + [S0], allow_unused=True)
    names = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0")
    refs = xs + [S0]
    return {n: (g if g is not None else torch.zeros_like(r)).detach().numpy() for n, g, r in zip(names, grads, refs)}
"""Pins of the fp64 oracle: checks that tie it to something other than itself.

Every check takes `fwd`, a callable with the signature of
oracle.kda_reference, and raises AssertionError when the oracle disagrees with
  * the worked examples printed on the "ten questions" page
    (jokeuncle.github.io, Kimi K3 KDA math for beginners; tests/golden/),
  * closed forms (linear attention, gated linear attention, decay only),
  * brute force (the unrolled product of the update matrices on tiny inputs),
  * invariants (exact recall with unit keys, one gradient step, packing),
  * independent re-expressions of the chunked algorithms (the WY form of
    DeltaNet in the GPT-2 -> Kimi K3 essay, section 6.3, and its per-channel
    gated extension derived from the recurrence).
None of these re-types the oracle's loop; each computes its expectation a
different way. tests/test_oracle_mutants.py plants mistakes in copies of the
oracle and checks that these pins catch every one.
"""
from __future__ import annotations

import json
import os

import numpy as np
import scipy.linalg

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "ten_questions_2x2.json")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.all(np.isfinite(a)) and err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------- golden

def golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def check_golden_case(fwd, case):
    steps = case["steps"] * case.get("repeat", 1)
    q = np.array([[s["q"]] for s in steps], dtype=np.float64)
    k = np.array([[s["k"]] for s in steps], dtype=np.float64)
    v = np.array([[s["v"]] for s in steps], dtype=np.float64)
    la = np.log(np.array([[s["alpha"]] for s in steps], dtype=np.float64))
    b = np.array([[s["beta"]] for s in steps], dtype=np.float64)
    h0 = None if case["h0"] is None else np.array(case["h0"], dtype=np.float64)[None, None]
    for mode in case["modes"]:
        o, hT = fwd(q, k, v, la, b, 1.0, h0=h0, delta_rule=(mode == "delta"))
        tag = f"{case['name']}[{mode}]"
        if case["expect_o"] is not None:
            for t, row in enumerate(case["expect_o"]):
                if row is not None:
                    _close(o[t, 0], row, case["tol"], f"{tag} o[{t}]")
        if case["expect_hT"] is not None:
            _close(hT[0, 0], case["expect_hT"], case["tol"], f"{tag} hT")


def check_golden(fwd):
    for case in golden_cases():
        check_golden_case(fwd, case)


# ----------------------------------------------------------------------------- inputs

def rand_inputs(seed, seqlens, H, dk, dv, gate="main", unit_keys=True, h0=True):
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    else:
        k *= 0.6
    v = rng.standard_normal((T, H, dv))
    if gate == "main":
        la = -np.logaddexp(0.0, rng.standard_normal((T, H, dk)) - 2.0)
    elif gate == "scalar":  # one decay for all key channels (Gated DeltaNet)
        la = np.repeat(-np.logaddexp(0.0, rng.standard_normal((T, H, 1)) - 2.0), dk, axis=2)
    elif gate == "none":
        la = np.zeros((T, H, dk))
    else:
        raise ValueError(gate)
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((len(seqlens), H, dk, dv)) * 0.5 if h0 else None
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    return q, k, v, la, b, S0, cu


def _heads(cu, H):
    for s in range(len(cu) - 1):
        for h in range(H):
            yield s, h, int(cu[s]), int(cu[s + 1])


# ----------------------------------------------------------------------------- brute force

def check_bruteforce_unrolled(fwd):
    """S_t = prod_{j<=t} M_j S_0 + sum_{i<=t} (prod_{i<j<=t} M_j) beta_i k_i v_i^T with
    M_j = (I - beta_j k_j k_j^T) Diag(alpha_j), built as explicit matrices."""
    for seed, (T, dk, dv) in enumerate([(1, 1, 1), (5, 3, 2), (8, 4, 4), (7, 2, 3), (6, 4, 1)]):
        q, k, v, la, b, S0, cu = rand_inputs(100 + seed, [T], 1, dk, dv, unit_keys=False)
        scale = 0.7
        o, hT = fwd(q, k, v, la, b, scale, h0=S0)
        M = [(np.eye(dk) - b[j, 0] * np.outer(k[j, 0], k[j, 0])) @ np.diag(np.exp(la[j, 0]))
             for j in range(T)]

        def prod(lo, hi):  # M_hi ... M_lo (identity when lo > hi)
            P = np.eye(dk)
            for j in range(lo, hi + 1):
                P = M[j] @ P
            return P

        for t in range(T):
            St = prod(0, t) @ S0[0, 0]
            for i in range(t + 1):
                St = St + prod(i + 1, t) @ (b[i, 0] * np.outer(k[i, 0], v[i, 0]))
            _close(o[t, 0], scale * St.T @ q[t, 0], 1e-12, f"bruteforce T={T} o[{t}]")
        _close(hT[0, 0], St, 1e-12, f"bruteforce T={T} hT")


# ----------------------------------------------------------------------------- closed forms

def check_linear_attention(fwd):
    """alpha = beta = 1 without the delta term: o = scale (tril(Q K^T) V + Q S0), hT = S0 + K^T V
    (bra-ket page, section 1.1: the state is the running sum of v k^T)."""
    q, k, v, la, b, S0, cu = rand_inputs(3, [19, 6], 2, 5, 3, gate="none")
    b = np.ones_like(b)
    scale = 0.45
    o, hT = fwd(q, k, v, la, b, scale, h0=S0, cu_seqlens=cu, delta_rule=False)
    for s, h, t0, t1 in _heads(cu, 2):
        Q, K, V = q[t0:t1, h], k[t0:t1, h], v[t0:t1, h]
        _close(o[t0:t1, h], scale * (np.tril(Q @ K.T) @ V + Q @ S0[s, h]), 1e-12, "linear o")
        _close(hT[s, h], S0[s, h] + K.T @ V, 1e-12, "linear hT")


def check_gated_linear_attention(fwd):
    """Without the delta term, a write at step i reaches step t >= i decayed by
    exp(g_t - g_i), g the inclusive running sum of log alpha (the cumulative-decay
    remark of the aidehub summary, Gated DeltaNet section):
    o_t = scale [ sum_{i<=t} <q_t * exp(g_t - g_i), k_i> beta_i v_i + (q_t * exp(g_t))^T S0 ]."""
    q, k, v, la, b, S0, cu = rand_inputs(4, [9, 14], 2, 4, 3)
    scale = 0.8
    o, hT = fwd(q, k, v, la, b, scale, h0=S0, cu_seqlens=cu, delta_rule=False)
    for s, h, t0, t1 in _heads(cu, 2):
        Q, K, V, B = q[t0:t1, h], k[t0:t1, h], v[t0:t1, h], b[t0:t1, h]
        g = np.cumsum(la[t0:t1, h], axis=0)
        for t in range(t1 - t0):
            acc = (Q[t] * np.exp(g[t])) @ S0[s, h]
            for i in range(t + 1):
                acc = acc + np.dot(Q[t] * np.exp(g[t] - g[i]), K[i]) * B[i] * V[i]
            _close(o[t0 + t, h], scale * acc, 1e-12, f"gla o[{t}]")
        ST = np.exp(g[-1])[:, None] * S0[s, h]
        for i in range(t1 - t0):
            ST = ST + np.outer(K[i] * np.exp(g[-1] - g[i]), B[i] * V[i])
        _close(hT[s, h], ST, 1e-12, "gla hT")


def check_decay_only(fwd):
    """beta = 0: nothing is written, S_T = Diag(exp(sum_t log alpha_t)) S0, and with
    log alpha = 0 the state is unchanged."""
    for gate in ("main", "none"):
        q, k, v, la, b, S0, cu = rand_inputs(5, [11], 3, 4, 5, gate=gate)
        b = np.zeros_like(b)
        scale = 1.3
        o, hT = fwd(q, k, v, la, b, scale, h0=S0)
        g = np.cumsum(la, axis=0)
        for h in range(3):
            _close(hT[0, h], np.exp(g[-1, h])[:, None] * S0[0, h], 1e-13, f"decay-only[{gate}] hT")
            _close(o[:, h], scale * (q[:, h] * np.exp(g[:, h])) @ S0[0, h], 1e-13,
                   f"decay-only[{gate}] o")
            if gate == "none":
                _close(hT[0, h], S0[0, h], 0.0, "beta=0, alpha=1 leaves the state unchanged")


# ----------------------------------------------------------------------------- invariants

def check_exact_recall(fwd):
    """beta = 1 and a unit key: after the write the key reads back exactly its value,
    S_t^T k_t = v_t, whatever alpha and the earlier state (GPT-2 -> Kimi K3 essay,
    section 5.1: unit keys retrieve losslessly; ten-questions page, Q6 at beta = 1).
    Feeding tokens one call at a time through h0 -> hT must also equal one call."""
    q, k, v, la, b, S0, cu = rand_inputs(6, [12], 2, 6, 4)
    b = np.ones_like(b)
    S = S0
    for t in range(12):
        sl = slice(t, t + 1)
        _, S = fwd(q[sl], k[sl], v[sl], la[sl], b[sl], 1.0, h0=S)
        for h in range(2):
            _close(S[0, h].T @ k[t, h], v[t, h], 1e-12, f"exact recall t={t}")
    _, hT = fwd(q, k, v, la, b, 1.0, h0=S0)
    _close(hT, S, 1e-12, "split into single-token calls")


def check_gradient_step(fwd):
    """One delta step is one gradient step of L(S) = 1/2 |S^T k - v|^2 taken at the
    decayed state with learning rate beta (ten-questions page, Q7); the gradient is
    taken by torch autograd in fp64."""
    import torch
    q, k, v, la, b, S0, cu = rand_inputs(8, [1], 1, 4, 3, unit_keys=False)
    _, hT = fwd(q, k, v, la, b, 1.0, h0=S0)
    Sd = torch.tensor(np.exp(la[0, 0])[:, None] * S0[0, 0], dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k[0, 0], dtype=torch.float64)
    vt = torch.tensor(v[0, 0], dtype=torch.float64)
    loss = 0.5 * torch.sum((Sd.T @ kt - vt) ** 2)
    loss.backward()
    expect = (Sd - float(b[0, 0]) * Sd.grad).detach().numpy()
    _close(hT[0, 0], expect, 1e-13, "gradient step")


def check_packing(fwd):
    """Sequences and heads are independent: one packed call equals separate calls
    per sequence and per head, bit for bit."""
    q, k, v, la, b, S0, cu = rand_inputs(9, [7, 1, 13], 3, 4, 2)
    o, hT = fwd(q, k, v, la, b, 0.5, h0=S0, cu_seqlens=cu)
    for s, h, t0, t1 in _heads(cu, 3):
        sl = slice(t0, t1)
        hs = slice(h, h + 1)
        o1, h1 = fwd(q[sl, hs], k[sl, hs], v[sl, hs], la[sl, hs], b[sl, hs], 0.5,
                     h0=S0[s:s + 1, hs])
        _close(o[sl, hs], o1, 0.0, f"packing o s={s} h={h}")
        _close(hT[s:s + 1, hs], h1, 0.0, f"packing hT s={s} h={h}")


# ----------------------------------------------------------------------------- chunked forms

def _unit_lower_inverse(N):
    """(I + N)^{-1} for strictly lower N, by a library triangular solve."""
    n = N.shape[0]
    return scipy.linalg.solve_triangular(np.eye(n) + N, np.eye(n), lower=True, unit_diagonal=True)


def deltanet_wy_chunked(Q, K, V, B, scale, C, S0):
    """The WY-chunked DeltaNet of the GPT-2 -> Kimi K3 essay, section 6.3, for one
    head: per chunk T = (I + strictLower(diag(beta) K K^T))^{-1}, W = T (beta K),
    U = T (beta V); then across chunks u = U - W S, o = Q S + tril(Q K^T) u,
    S += K^T u. Scale multiplies q."""
    S = S0.copy()
    out = np.zeros((Q.shape[0], V.shape[1]))
    for c0 in range(0, Q.shape[0], C):
        q_, k_, v_, b_ = Q[c0:c0 + C], K[c0:c0 + C], V[c0:c0 + C], B[c0:c0 + C]
        Tm = _unit_lower_inverse(np.tril(b_[:, None] * (k_ @ k_.T), -1))
        W = Tm @ (b_[:, None] * k_)
        U = Tm @ (b_[:, None] * v_)
        u = U - W @ S
        out[c0:c0 + C] = scale * (q_ @ S + np.tril(q_ @ k_.T) @ u)
        S = S + k_.T @ u
    return out, S


def kda_chunked(Q, K, V, LA, B, scale, C, S0):
    """Chunked KDA for one head, derived from the recurrence (the per-channel gated
    extension of the essay's WY step). Within a chunk, g = inclusive running sum of
    log alpha; A[r,i] = sum_c K[r,c] K[i,c] exp(g[r,c] - g[i,c]) for i < r;
    T = (I + diag(beta) strictLower(A))^{-1}; W = T (beta K exp(g)); U~ = T (beta V);
    U = U~ - W S; O = scale [(Q exp(g)) S + tril_incl(Aqk) U] with
    Aqk[r,i] = sum_c Q[r,c] K[i,c] exp(g[r,c] - g[i,c]); S <- exp(g_last) S +
    (K exp(g_last - g))^T U."""
    S = S0.copy()
    out = np.zeros((Q.shape[0], V.shape[1]))
    for c0 in range(0, Q.shape[0], C):
        q_, k_, v_, b_ = Q[c0:c0 + C], K[c0:c0 + C], V[c0:c0 + C], B[c0:c0 + C]
        g = np.cumsum(LA[c0:c0 + C], axis=0)
        n = q_.shape[0]
        lower = np.tril(np.ones((n, n), dtype=bool), -1)
        D = g[:, None, :] - g[None, :, :]              # [r, i, c]
        D = np.where(np.tril(np.ones((n, n), dtype=bool))[:, :, None], D, 0.0)
        A = np.einsum("rc,ic,ric->ri", k_, k_, np.exp(D))
        Aqk = np.tril(np.einsum("rc,ic,ric->ri", q_, k_, np.exp(D)))
        Tm = _unit_lower_inverse(np.where(lower, b_[:, None] * A, 0.0))
        W = Tm @ (b_[:, None] * k_ * np.exp(g))
        U = Tm @ (b_[:, None] * v_) - W @ S
        out[c0:c0 + C] = scale * ((q_ * np.exp(g)) @ S + Aqk @ U)
        S = np.exp(g[-1])[:, None] * S + (k_ * np.exp(g[-1] - g)).T @ U
    return out, S


def check_deltanet_wy(fwd):
    """log alpha = 0 reduces KDA to DeltaNet; the oracle must equal the WY-chunked
    form for any chunk size (chunking is an exact refactoring)."""
    q, k, v, la, b, S0, cu = rand_inputs(10, [37], 2, 6, 5, gate="none")
    scale = 0.6
    o, hT = fwd(q, k, v, la, b, scale, h0=S0)
    for C in (1, 3, 8, 16, 64):
        for h in range(2):
            oc, Sc = deltanet_wy_chunked(q[:, h], k[:, h], v[:, h], b[:, h], scale, C, S0[0, h])
            _close(o[:, h], oc, 1e-12, f"deltanet WY C={C} o")
            _close(hT[0, h], Sc, 1e-12, f"deltanet WY C={C} hT")


def check_kda_chunked(fwd):
    """Per-channel (KDA) and channel-constant (Gated DeltaNet) gates: the oracle
    equals the chunked form for chunk sizes from 1 (the recurrence) to beyond T
    (masked attention over the whole sequence), including a ragged tail."""
    for gate in ("main", "scalar"):
        q, k, v, la, b, S0, cu = rand_inputs(11, [37], 2, 8, 5, gate=gate)
        scale = 0.9
        o, hT = fwd(q, k, v, la, b, scale, h0=S0)
        for C in (1, 4, 16, 64):
            for h in range(2):
                oc, Sc = kda_chunked(q[:, h], k[:, h], v[:, h], la[:, h], b[:, h], scale, C,
                                     S0[0, h])
                _close(o[:, h], oc, 1e-12, f"kda chunked[{gate}] C={C} o")
                _close(hT[0, h], Sc, 1e-12, f"kda chunked[{gate}] C={C} hT")


ALL_CHECKS = [check_golden, check_bruteforce_unrolled, check_linear_attention,
              check_gated_linear_attention, check_decay_only, check_exact_recall,
              check_gradient_step, check_packing, check_deltanet_wy, check_kda_chunked]

"""CPU tests: the fp64 oracle against its pins (worked examples, closed forms,
brute force, invariants, chunked re-expressions). See tests/oracle_pins.py."""
import numpy as np
import pytest

import kda_synth
import oracle
import oracle_pins as P


@pytest.mark.parametrize("case", P.golden_cases(), ids=lambda c: c["name"])
def test_golden_worked_example(ref, case):
    P.check_golden_case(ref, case)


@pytest.mark.parametrize("check", [c for c in P.ALL_CHECKS if c is not P.check_golden],
                         ids=lambda c: c.__name__)
def test_pin(ref, check):
    check(ref)


def test_scalar_decay_closed_form(ref):
    """0.9^20 exactly, beyond the page's two printed digits (ten-questions page, Q8)."""
    T = 20
    o, hT = ref(np.ones((T, 1, 1)), np.ones((T, 1, 1)), np.zeros((T, 1, 1)),
                np.full((T, 1, 1), np.log(0.9)), np.zeros((T, 1)), 1.0,
                h0=np.ones((1, 1, 1, 1)))
    assert abs(hT[0, 0, 0, 0] - 0.9 ** 20) < 1e-15
    assert abs(0.9 ** 20 - 0.12) < 0.005


def test_generator_squashing_matches_page_values():
    """The gate squashing used by the input recipes, against the values the
    ten-questions page prints in Q9 (to its printed precision)."""
    assert kda_synth.sigmoid(0.0) == 0.5
    assert abs(kda_synth.sigmoid(4.0) - 0.98) < 0.005
    assert abs(kda_synth.sigmoid(-4.0) - 0.02) < 0.005
    assert abs(kda_synth.softplus(-5.0) - 0.007) < 0.0005
    assert abs(kda_synth.softplus(5.0) - 5.007) < 0.0005


def test_generator_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # ties go to even
    ours = kda_synth.round_bf16(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), theirs.view(np.uint32))


def test_generator_is_seeded_and_normalised():
    a = kda_synth.gen_sequences((33, 7), 2, 8, 4, "bf16", "main", "normal", 5)
    b = kda_synth.gen_sequences((33, 7), 2, 8, 4, "bf16", "main", "normal", 5)
    for key in ("q", "k", "v", "log_alpha", "beta", "h0"):
        assert np.array_equal(a[key], b[key])
    assert list(a["cu_seqlens"]) == [0, 33, 40]
    assert np.allclose(np.linalg.norm(a["k"], axis=-1), 1.0, atol=1e-2)  # bf16-rounded unit keys
    assert np.all(a["log_alpha"] < 0) and np.all((a["beta"] > 0) & (a["beta"] < 1))


# ----------------------------------------------------------------------------- gate prologue

def _prologue_scalar(a, A_log, dt_bias, b):
    la, be = oracle.gate_prologue(np.array([[[a]]]), np.array([A_log]), np.array([[dt_bias]]), np.array([[b]]))
    return float(la[0, 0, 0]), float(be[0, 0])


def test_gate_prologue_page_values():
    """Q9 of the ten-questions page prints the squashing functions' values: sigmoid(0) = 0.5,
    sigmoid(4) ~ 0.98, sigmoid(-4) ~ 0.02, softplus(-5) ~ 0.007, softplus(5) ~ 5.007. With
    A_log = 0 (a rate scale of 1) the formed log alpha is -softplus(a + dt_bias)."""
    for bb, want in ((0.0, 0.5), (4.0, 0.98), (-4.0, 0.02)):
        assert abs(_prologue_scalar(0.0, 0.0, 0.0, bb)[1] - want) < 0.005
    assert abs(-_prologue_scalar(-5.0, 0.0, 0.0, 0.0)[0] - 0.007) < 0.0005
    assert abs(-_prologue_scalar(5.0, 0.0, 0.0, 0.0)[0] - 5.007) < 0.0005


def test_gate_prologue_closed_forms():
    # softplus(0) = ln 2; the rate scale multiplies; dt_bias shifts the pre-activation
    assert abs(_prologue_scalar(0.0, 0.0, 0.0, 0.0)[0] + np.log(2.0)) < 1e-15
    assert abs(_prologue_scalar(0.0, np.log(3.0), 0.0, 0.0)[0] + 3.0 * np.log(2.0)) < 1e-14
    assert _prologue_scalar(1.5, 0.2, -0.5, 0.0)[0] == _prologue_scalar(0.5, 0.2, 0.5, 0.0)[0]
    # far from zero softplus is its asymptote: x for large x, e^x for very negative x
    assert abs(_prologue_scalar(40.0, 0.0, 0.0, 0.0)[0] + 40.0) < 1e-12
    assert abs(_prologue_scalar(-40.0, 0.0, 0.0, 0.0)[0] + np.exp(-40.0)) < 1e-30
    # sigmoid(x) + sigmoid(-x) = 1
    assert abs(_prologue_scalar(0.0, 0.0, 0.0, 1.7)[1] + _prologue_scalar(0.0, 0.0, 0.0, -1.7)[1] - 1.0) < 1e-15


def test_gate_prologue_ranges_and_broadcast():
    """alpha = e^log_alpha lies in (0, 1) and beta in (0, 1) whatever the inputs; A_log is
    per head and dt_bias per (head, channel)."""
    rng = np.random.default_rng(5)
    T, H, dk = 7, 3, 4
    a = rng.standard_normal((T, H, dk)) * 10
    A_log = rng.standard_normal(H)
    dt_bias = rng.standard_normal((H, dk))
    b = rng.standard_normal((T, H)) * 10
    la, be = oracle.gate_prologue(a, A_log, dt_bias, b)
    assert la.shape == (T, H, dk) and be.shape == (T, H)
    assert np.all(la < 0) and np.all(np.exp(la) > 0) and np.all((be > 0) & (be < 1))
    for t, h, c in ((0, 0, 0), (6, 2, 3), (3, 1, 2)):
        want = -np.exp(A_log[h]) * np.log1p(np.exp(a[t, h, c] + dt_bias[h, c]))
        assert abs(la[t, h, c] - want) <= 1e-12 * abs(want) + 1e-300


def test_qk_prologue():
    """normalize(silu(x)): unit length along the head dimension; silu(0) = 0, silu(x) ~ x
    for large x and ~ 0 for very negative x; a zero vector stays zero (the eps floor);
    and the page's reason for it: a key of unit length reads back exactly the value it
    wrote (beta = 1, no decay, empty state)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 3, 16)) * 3
    y = oracle.qk_prologue(x)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-14)
    big = np.array([[30.0, 40.0]])  # silu(x) = x (to e^-30): direction (0.6, 0.8)
    assert np.allclose(oracle.qk_prologue(big), [[0.6, 0.8]], atol=1e-12)
    mixed = np.array([[50.0, -50.0, 0.0]])  # silu = (50, ~0, 0)
    assert np.allclose(oracle.qk_prologue(mixed), [[1.0, 0.0, 0.0]], atol=1e-12)
    assert np.all(oracle.qk_prologue(np.zeros((2, 4))) == 0.0)
    k = oracle.qk_prologue(rng.standard_normal((1, 1, 8)))
    v = rng.standard_normal((1, 1, 5))
    o, _ = oracle.kda_reference(k, k, v, np.zeros((1, 1, 8)), np.ones((1, 1)), 1.0)
    assert np.allclose(o, v, atol=1e-14)


# ---- softmax-attention decode over a KV cache (the comparator of the decode step):
# pins of oracle.attn_decode_reference against hand-worked values and closed forms

def test_attn_decode_worked_example():
    # scores scale * q . k = 0.5 * [0, 2 ln 3] = [0, ln 3] -> weights [1/4, 3/4]
    q = np.array([[[1.0, 0.0]]])
    K = np.array([[[[0.0, 0.0], [2 * np.log(3.0), 7.0]]]])
    V = np.array([[[[4.0, 0.0], [0.0, 8.0]]]])
    o = oracle.attn_decode_reference(q, K, V, scale=0.5)
    np.testing.assert_allclose(o, [[[1.0, 6.0]]], rtol=0, atol=1e-14)
    # scale defaults to d^-1/2
    o2 = oracle.attn_decode_reference(q, K * (0.5 * np.sqrt(2.0)), V)  # d = 2: scale 2^-1/2
    np.testing.assert_allclose(o2, [[[1.0, 6.0]]], rtol=0, atol=1e-14)


def test_attn_decode_grouped_heads_and_lengths():
    # query head h reads cached head h // (H / H_kv); constant value rows make o that constant
    rng = np.random.default_rng(5)
    B, H, H_kv, T, d = 2, 4, 2, 9, 8
    q = rng.standard_normal((B, H, d))
    K = rng.standard_normal((B, H_kv, T, d))
    V = np.empty((B, H_kv, T, d))
    for b in range(B):
        for j in range(H_kv):
            V[b, j] = 10 * b + j + 1
    o = oracle.attn_decode_reference(q, K, V, seq_lens=[T, 3])
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(o[b, h], 10 * b + h // 2 + 1, rtol=1e-14)
    # rows at and past the length never matter, lengths are clamped to [0, T], none gives 0
    K2, V2 = K.copy(), V.copy()
    K2[1, :, 3:] = 1e3
    V2[1, :, 3:] = 1e6
    np.testing.assert_array_equal(oracle.attn_decode_reference(q, K2, V2, seq_lens=[T, 3]), o)
    np.testing.assert_array_equal(oracle.attn_decode_reference(q, K, V, seq_lens=[T + 5, 3]), o)
    z = oracle.attn_decode_reference(q, K, V, seq_lens=[0, -2])
    np.testing.assert_array_equal(z, np.zeros((B, H, d)))


def test_attn_decode_closed_forms():
    rng = np.random.default_rng(6)
    d, T = 16, 12
    q = rng.standard_normal((1, 1, d))
    V = rng.standard_normal((1, 1, T, d))
    # identical keys: the mean of the value rows
    K = np.repeat(rng.standard_normal((1, 1, 1, d)), T, axis=2)
    np.testing.assert_allclose(oracle.attn_decode_reference(q, K, V), V.mean(axis=2), rtol=1e-12, atol=1e-14)
    # one row: that value row
    np.testing.assert_allclose(oracle.attn_decode_reference(q, K[:, :, :1], V[:, :, :1]), V[:, :, 0],
                               rtol=1e-14)
    # scores near 1000 (exp would overflow): two rows 1000 and 1000 - ln 2 -> weights 2/3, 1/3
    e = np.zeros((1, 1, d))
    e[0, 0, 0] = 1.0
    K2 = np.zeros((1, 1, 2, d))
    K2[0, 0, :, 0] = [1000.0, 1000.0 - np.log(2.0)]
    o = oracle.attn_decode_reference(e, K2, V[:, :, :2], scale=1.0)
    np.testing.assert_allclose(o[0, 0], (2 * V[0, 0, 0] + V[0, 0, 1]) / 3, rtol=1e-12)


def test_attn_decode_matches_library_softmax_and_is_order_free():
    from scipy.special import softmax
    rng = np.random.default_rng(7)
    B, H, H_kv, T, d = 2, 4, 1, 37, 32
    q = rng.standard_normal((B, H, d))
    K = rng.standard_normal((B, H_kv, T, d))
    V = rng.standard_normal((B, H_kv, T, d))
    o = oracle.attn_decode_reference(q, K, V, scale=0.3)
    for b in range(B):
        for h in range(H):
            w = softmax(0.3 * K[b, 0] @ q[b, h])
            np.testing.assert_allclose(o[b, h], w @ V[b, 0], rtol=1e-12, atol=1e-14)
    # permuting the cache rows (keys and values together) leaves o unchanged
    perm = rng.permutation(T)
    np.testing.assert_allclose(oracle.attn_decode_reference(q, K[:, :, perm], V[:, :, perm], scale=0.3), o,
                               rtol=1e-12, atol=1e-14)


# ---- gradients of the recurrence (oracle.kda_backward_reference, autograd of the token loop):
# pinned by central differences of the independent C forward oracle and by closed forms

def _loss_c(q, k, v, la, beta, scale, h0, do, dhT):
    """sum(o * do) + sum(hT * dhT) through the C oracle, for [B=1, T, H, d] inputs (h0, dhT
    [1, H, dk, dv])."""
    o, hT = oracle.kda_reference(q[0], k[0], v[0], la[0], beta[0], scale, h0=h0)
    return float((o * do[0]).sum() + (hT * dhT).sum())


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(8)
    B, T, H, dk, dv, scale = 1, 7, 2, 3, 2, 0.6
    q, k = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    la = -0.5 * np.log1p(np.exp(rng.standard_normal((B, T, H, dk))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    h0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    do, dhT = rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, H, dk, dv))
    g = oracle.kda_backward_reference(q, k, v, la, beta, scale, do, dhT=dhT, h0=h0)
    args = dict(q=q, k=k, v=v, la=la, beta=beta, h0=h0)
    names = dict(q="dq", k="dk", v="dv", la="dlog_alpha", beta="dbeta", h0="dh0")
    eps = 1e-6
    for n, key in names.items():
        x = args[n]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = dict(args, **{n: xp}), dict(args, **{n: xm})
            lp = _loss_c(ap["q"], ap["k"], ap["v"], ap["la"], ap["beta"], scale, ap["h0"], do, dhT)
            lm = _loss_c(am["q"], am["k"], am["v"], am["la"], am["beta"], scale, am["h0"], do, dhT)
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[key], fd, rtol=1e-6, atol=1e-8, err_msg=key)


def test_backward_closed_forms():
    rng = np.random.default_rng(9)
    B, T, H, dk, dv, s = 1, 6, 1, 4, 3, 0.8
    q, k = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    v, do = rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, T, H, dv))
    h0, dhT = rng.standard_normal((B, H, dk, dv)), rng.standard_normal((B, H, dk, dv))
    zero_b = np.zeros((B, T, H))
    # beta = 0, alpha = 1: S_t = h0, o_t = s h0^T q_t
    g = oracle.kda_backward_reference(q, k, v, np.zeros((B, T, H, dk)), zero_b, s, do, dhT=dhT, h0=h0)
    H0 = h0[0, 0]
    for t in range(T):
        np.testing.assert_allclose(g["dq"][0, t, 0], s * H0 @ do[0, t, 0], rtol=1e-12)
        # dL/dS_t after step t: the later outputs' s q do^T plus dhT; the delta's residual v - h0^T k
        dS = dhT[0, 0] + sum(s * np.outer(q[0, u, 0], do[0, u, 0]) for u in range(t, T))
        np.testing.assert_allclose(g["dbeta"][0, t, 0], (dS.T @ k[0, t, 0]) @ (v[0, t, 0] - H0.T @ k[0, t, 0]),
                                   rtol=1e-10)
    np.testing.assert_allclose(g["dh0"][0, 0], dhT[0, 0] + s * sum(np.outer(q[0, t, 0], do[0, t, 0]) for t in range(T)),
                               rtol=1e-12)
    np.testing.assert_array_equal(g["dv"], 0)
    np.testing.assert_array_equal(g["dk"], 0)
    # beta = 0 with decays: S_t = Diag(exp(g_t)) h0, g_t = the prefix sum of log alpha
    la = -0.4 * np.log1p(np.exp(rng.standard_normal((B, T, H, dk))))
    g = oracle.kda_backward_reference(q, k, v, la, zero_b, s, do, dhT=dhT, h0=h0)
    gt = np.cumsum(la[0, :, 0], axis=0)
    dg = np.stack([s * q[0, t, 0] * np.exp(gt[t]) * (H0 @ do[0, t, 0]) for t in range(T)])
    dg[-1] += np.exp(gt[-1]) * (H0 * dhT[0, 0]).sum(axis=1)
    np.testing.assert_allclose(g["dlog_alpha"][0, :, 0], np.cumsum(dg[::-1], axis=0)[::-1], rtol=1e-10)

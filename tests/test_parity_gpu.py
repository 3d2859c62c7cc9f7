"""GPU parity of libkda (through its C ABI) against the fp64 oracle.

Bar: relative L2 error of o and of hT <= 1e-4 on the fp32 path and <= 2e-2 on the
bf16-input path (q, k, v, o in bf16; gates and states fp32), over the whole tensor
and for every (sequence, head) on its own; and every (token, head) row of o within
the per-row bound of kda_testlib.ROW_TOL. Inputs are seeded synthetic draws
(kda_synth); the oracle reads exactly the values the GPU receives.
"""
import numpy as np
import pytest

import kda_synth
import oracle
from kda_testlib import (TOL, assert_parity, gate_view, gen, oracle_run, rel_l2, run_packed, say, to_dev,
                         with_gate, workload_inputs)

pytestmark = pytest.mark.gpu


def _check(x, io, chunk, name, varlen=True, B=None, T=None, h0=True, tol=None, gate="channel"):
    tol = TOL[io] if tol is None else tol
    say(f"[{name}] io={io} C={chunk} gate={gate} seqs={np.diff(x['cu_seqlens']).tolist()[:6]} "
        f"H={x['q'].shape[1]} dk={x['q'].shape[2]} dv={x['v'].shape[2]}")
    o, hT = run_packed(x, io, chunk, varlen=varlen, B=B, T=T, h0=h0, gate=gate)
    o_ref, h_ref, _ = oracle_run(x, h0=h0)
    assert_parity(o, o_ref, hT, h_ref, io, name, cu=x["cu_seqlens"], tol=tol)
    return o, hT


def test_tiny_config():
    """The tiny fp32 workload: B=1, H=2, T=256, d=64, C=64, weak gates, h0 = 0."""
    w = kda_synth.WORKLOADS["tiny"]
    x = kda_synth.gen_workload(w)
    _check(x, "f32", w.chunk, "tiny")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_shapes(io, chunk, dk, dv):
    """Several chunks with a ragged tail, two sequences, nonzero h0."""
    x = gen([3 * chunk + 17, 2 * chunk], 2, dk, dv, io, seed=dk + dv + chunk)
    _check(x, io, chunk, "shapes")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 15, 63, 64, 65, 127, 129])
def test_short_and_ragged_lengths(io, T):
    x = gen([T, T], 3, 128, 128, io, seed=T)
    _check(x, io, 64, f"T={T}", varlen=False, B=2, T=T)


def test_batched_layout_equals_packed():
    """[B, T, H, d] without cu_seqlens is the same computation as B packed
    sequences of length T, bit for bit."""
    x = gen([200, 200, 200], 4, 128, 128, "bf16", seed=5)
    o1, h1 = run_packed(x, "bf16", 64, varlen=False, B=3, T=200)
    o2, h2 = run_packed(x, "bf16", 64, varlen=True)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


def test_no_h0_no_hT():
    x = gen([150, 90], 2, 128, 128, "f32", h0="zero", seed=9)
    o, hT = run_packed(x, "f32", 64, h0=False, hT=False)
    assert hT is None
    o_ref, _, _ = oracle_run(x, h0=False)
    assert_parity(o, o_ref, None, None, "f32", "no h0, no hT", cu=x["cu_seqlens"])


def test_empty_input_copies_state():
    """T = 0: no token, hT = h0 (and zeros without h0)."""
    import torch
    import gated_delta_rule_48_amd as kda
    H, d = 3, 64
    q = torch.empty((2, 0, H, d), device="cuda")
    la = torch.empty((2, 0, H, d), device="cuda")
    beta = torch.empty((2, 0, H), device="cuda")
    h0 = torch.randn((2, H, d, d), device="cuda")
    _, hT = kda.chunk_fwd(q, q, q, la, beta, h0=h0)
    assert torch.equal(hT, h0)
    _, hT = kda.chunk_fwd(q, q, q, la, beta)
    assert torch.count_nonzero(hT).item() == 0


def test_varlen_with_empty_and_tiny_sequences():
    x = gen([0, 130, 1, 0, 64, 257], 2, 128, 128, "bf16", seed=13)
    _check(x, "bf16", 64, "varlen-edge")
    _check(x, "bf16", 128, "varlen-edge-C128")


def test_varlen_equals_separate_calls():
    """Packed sequences give exactly (bitwise) what separate calls give."""
    x = gen([77, 300, 64], 2, 128, 128, "bf16", seed=21)
    o, hT = run_packed(x, "bf16", 64)
    cu = x["cu_seqlens"]
    for s in range(3):
        sl = slice(cu[s], cu[s + 1])
        xs = {n: x[n][sl] for n in ("q", "k", "v", "log_alpha", "beta")}
        xs["h0"] = x["h0"][s:s + 1]
        xs["cu_seqlens"] = np.array([0, cu[s + 1] - cu[s]], dtype=np.int32)
        os_, hs = run_packed(xs, "bf16", 64)
        assert np.array_equal(o[sl], os_), s
        assert np.array_equal(hT[s:s + 1], hs), s


def test_chunk_size_invariance():
    """C = 64 and C = 128 are two blockings of the same recurrence."""
    x = gen([500], 2, 128, 128, "f32", seed=31)
    o64, h64 = _check(x, "f32", 64, "C64")
    o128, h128 = _check(x, "f32", 128, "C128")
    assert rel_l2(o64, o128) <= 1e-4 and rel_l2(h64, h128) <= 1e-4


def test_split_invariance():
    """One call over T tokens equals two calls that carry hT -> h0."""
    x = gen([300], 2, 128, 128, "f32", seed=41)
    o, hT = run_packed(x, "f32", 64)
    t1 = 130
    a = {n: x[n][:t1] for n in ("q", "k", "v", "log_alpha", "beta")}
    a["h0"], a["cu_seqlens"] = x["h0"], np.array([0, t1], dtype=np.int32)
    oa, ha = run_packed(a, "f32", 64)
    b = {n: x[n][t1:] for n in ("q", "k", "v", "log_alpha", "beta")}
    b["h0"], b["cu_seqlens"] = ha, np.array([0, 300 - t1], dtype=np.int32)
    ob, hb = run_packed(b, "f32", 64)
    assert rel_l2(np.concatenate([oa, ob]), o) <= 1e-5
    assert rel_l2(hb, hT) <= 1e-5


def test_h0_aliases_hT():
    import torch
    import gated_delta_rule_48_amd as kda
    x = gen([200], 2, 128, 128, "f32", seed=43)
    t = to_dev(x, "f32")
    args = [t[n] for n in ("q", "k", "v", "log_alpha", "beta")]
    _, ref = kda.chunk_fwd(*args, h0=t["h0"], cu_seqlens=t["cu_seqlens"])
    st = t["h0"].clone()
    kda.chunk_fwd(*args, h0=st, hT=st, cu_seqlens=t["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(st, ref)


@pytest.mark.parametrize("gate", ["deltanet", "gdn"])
def test_reductions(gate):
    """log alpha = 0 (DeltaNet) and one decay for all key channels (Gated DeltaNet)."""
    x = gen([260], 2, 128, 128, "f32", seed=51)
    if gate == "deltanet":
        x["log_alpha"] = np.zeros_like(x["log_alpha"])
    else:
        x["log_alpha"] = np.repeat(x["log_alpha"][:, :, :1], 128, axis=2).copy()
    _check(x, "f32", 64, gate)


def test_beta_zero_keeps_state():
    """beta = 0 and alpha = 1: the state is unchanged and o = scale q^T S0."""
    x = gen([100], 2, 64, 64, "f32", seed=53)
    x["beta"] = np.zeros_like(x["beta"])
    x["log_alpha"] = np.zeros_like(x["log_alpha"])
    o, hT = run_packed(x, "f32", 64)
    assert rel_l2(hT, x["h0"]) <= 1e-6
    _check(x, "f32", 64, "beta0")


def test_deterministic():
    x = gen([1000, 333], 4, 128, 128, "bf16", seed=61)
    o1, h1 = run_packed(x, "bf16", 64)
    o2, h2 = run_packed(x, "bf16", 64)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


# ----------------------------------------------------------------------------- decode

def _decode_steps(N, H, dk, dv, io, steps, seed, sample=None, gate="channel"):
    """Run `steps` decode steps on the GPU; return per-step o of the sampled
    (n, h) pairs, their final states, and the oracle's values for them. `gate`
    selects which decays the library is given (gate_view); the oracle reads what
    they mean on every channel (with_gate)."""
    import torch
    import gated_delta_rule_48_amd as kda
    st0 = kda_synth.gen_decode_state(N, H, dk, dv, seed)
    state = torch.from_numpy(st0).cuda()
    sample = [(n, h) for n in range(N) for h in range(H)] if sample is None else sample
    ns = np.array([p[0] for p in sample])
    hs = np.array([p[1] for p in sample])
    got, toks = [], []
    for step in range(steps):
        y = with_gate(kda_synth.gen_decode_step(N, H, dk, dv, io, "main", seed, step), gate)
        t = to_dev(dict(y, cu_seqlens=np.zeros(1, np.int32)), io)
        o = kda.recurrent_step(t["q"], t["k"], t["v"], gate_view(t["log_alpha"], gate), t["beta"], state)
        got.append(o.float().cpu().numpy()[ns, hs])
        toks.append({n: y[n][ns, hs] for n in ("q", "k", "v", "log_alpha", "beta")})
    torch.cuda.synchronize()
    st_got = state.cpu().numpy()[ns, hs]
    # oracle: the sampled pairs as independent heads of one sequence of `steps` tokens
    seq = {n: np.stack([tk[n] for tk in toks]) for n in toks[0]}
    o_ref, h_ref = oracle.kda_reference(
        seq["q"], seq["k"], seq["v"], seq["log_alpha"], seq["beta"], dk ** -0.5,
        h0=st0[ns, hs][None])
    return np.stack(got), st_got, o_ref, h_ref[0]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_decode_small(io, dk, dv):
    o, st, o_ref, h_ref = _decode_steps(3, 2, dk, dv, io, 5, seed=dk + dv)
    assert_parity(o, o_ref, st[None], h_ref[None], io, f"decode {io} {dk}x{dv}")


def test_decode_matches_chunked():
    """T decode steps equal one chunked call over the same T tokens."""
    import torch
    import gated_delta_rule_48_amd as kda
    x = gen([90], 2, 128, 128, "f32", seed=71)
    o_c, h_c = run_packed(x, "f32", 64)
    t = to_dev(x, "f32")
    state = t["h0"].clone()
    outs = []
    for i in range(90):
        outs.append(kda.recurrent_step(t["q"][i:i + 1], t["k"][i:i + 1], t["v"][i:i + 1],
                                       t["log_alpha"][i:i + 1], t["beta"][i:i + 1], state))
    torch.cuda.synchronize()
    o_d = torch.cat(outs).cpu().numpy()
    assert rel_l2(o_d, o_c) <= 1e-4 and rel_l2(state.cpu().numpy(), h_c) <= 1e-4


# ----------------------------------------------------------------------------- full-size workloads

def test_prefill_workload_full():
    """B=1, H=16, T=4096, d=128, bf16, C=64, main gates, h0 ~ N(0, 0.02): every head."""
    w = kda_synth.WORKLOADS["prefill"]
    x = kda_synth.gen_workload(w)
    _check(x, "bf16", w.chunk, "prefill-4096")


def test_batched_workload_full():
    """B=8, H=32, T=8192, bf16, C=64 (the benchmark's prefill launch, fused pass): every
    (sequence, head) pair against the oracle over its full length."""
    w = kda_synth.WORKLOADS["batched"]
    x = workload_inputs(w)
    say("[batched] generated")
    _check(x, "bf16", w.chunk, "batched", varlen=False, B=8, T=8192, h0=False)


def test_varlen_workload_full():
    """Packed 32768/16384/12288/4096 tokens, H=32, bf16, C=128, per-sequence h0: every
    (sequence, head) pair against the oracle."""
    w = kda_synth.WORKLOADS["varlen"]
    x = kda_synth.gen_workload(w)
    say("[varlen] generated")
    _check(x, "bf16", w.chunk, "varlen")


def test_decode_workload_1024_steps():
    """256 sequences x 32 heads, d=128, bf16, main gates, h0 ~ N(0, 0.02): all 1024 steps
    of the full batch (the benchmark's decode launch, distinct inputs every step, drawn on
    the GPU by torch's seeded generator), the oracle on 64 (sequence, head) pairs spread
    over the batch, every step's o and the final states."""
    import torch
    import gated_delta_rule_48_amd as kda
    d = kda_synth.DECODE
    N, H, dk, dv, steps = d["N"], d["H"], d["dk"], d["dv"], d["steps"]
    st0 = kda_synth.gen_decode_state(N, H, dk, dv, d["seed"])
    state = torch.from_numpy(st0).cuda()
    ns = torch.tensor([(4 * i + i // 16) % N for i in range(64)], device="cuda")
    hs = torch.tensor([(7 * i + 3) % H for i in range(64)], device="cuda")
    got = {n: [] for n in ("q", "k", "v", "log_alpha", "beta", "o")}
    for step in range(steps):
        y = kda_synth.gen_decode_step_device(N, H, dk, dv, torch.bfloat16, d["seed"], step, "cuda")
        o = kda.recurrent_step(y["q"], y["k"], y["v"], y["log_alpha"], y["beta"], state)
        for n in ("q", "k", "v", "log_alpha", "beta"):
            got[n].append(y[n][ns, hs].float())
        got["o"].append(o[ns, hs].float())
        if step % 256 == 255:
            say(f"[decode-1024] step {step + 1}")
    torch.cuda.synchronize()
    seq = {n: torch.stack(v).cpu().numpy() for n, v in got.items()}
    st_got = state[ns, hs].cpu().numpy()
    nsl, hsl = ns.cpu().numpy(), hs.cpu().numpy()
    o_ref, h_ref = oracle.kda_reference(seq["q"], seq["k"], seq["v"], seq["log_alpha"], seq["beta"], dk ** -0.5,
                                        h0=st0[nsl, hsl][None])
    assert_parity(seq["o"], o_ref, st_got[None], h_ref, "bf16", "decode-1024")


# ----------------------------------------------------------------------------- 256-pair batches
# Uniform batches of B * H = 256 (sequence, head) pairs: bf16 with d_k = d_v = 128 takes the
# fused pass (one workgroup per pair), every other dtype and size the split pass.

def _pass(io, dk, dv):
    return "fused" if io == "bf16" and dk == dv == 128 else "split"


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [200, 1, 64])
def test_uniform_batch_256_pairs(io, dk, dv, T):
    x = gen([T, T], 128, dk, dv, io, seed=7 * T + dk + dv)
    _check(x, io, 64, f"{_pass(io, dk, dv)} T={T}", varlen=False, B=2, T=T)


@pytest.mark.parametrize("io,path", [("f32", "split"), ("bf16", "split"), ("bf16", "fused"), ("bf16", "few-pairs")])
def test_strong_decay(io, path):
    """Fast-forgetting gates ("strong": chunk sums of log alpha near -117 on average and
    down to about -150). The in-chunk decay factors then span up to e^(+-75) and the state
    factors reach e^(-75) per chunk: products of such factors must be formed in an order
    that stays inside the fp32 range. Passes: split (fp32 at d = 128, bf16 at d = 64), fused
    (256 pairs) and fused with few pairs (16, one workgroup each)."""
    if path == "fused":
        x = gen([200, 200], 128, 128, 128, io, gates="strong", seed=91)
        _check(x, io, 64, "strong fused", varlen=False, B=2, T=200)
    else:
        d = 64 if (io == "bf16" and path == "split") else 128
        x = gen([200, 130], 8, d, d, io, gates="strong", seed=92)
        _check(x, io, 64, f"strong {path}")


def test_fused_path_no_h0():
    x = gen([129, 129], 128, 128, 128, "bf16", h0="zero", seed=77)
    o, hT = run_packed(x, "bf16", 64, varlen=False, B=2, T=129, h0=False)
    o_ref, h_ref, _ = oracle_run(x, h0=False)
    assert_parity(o, o_ref, hT, h_ref, "bf16", "fused no h0", cu=x["cu_seqlens"])


def test_fused_matches_segmented():
    """The same sequence through the fused pass in one workgroup per (sequence, head) (as
    part of a 256-pair batch) and alone, 128 pairs, where the pass cuts its 600 tokens into
    segments (maps, their composition, then the segments): two schedules of the same
    arithmetic, both within tolerance of the oracle and close to each other."""
    x = gen([600, 600], 128, 128, 128, "bf16", seed=79)
    of, hf = run_packed(x, "bf16", 64, varlen=False, B=2, T=600)
    one = dict(x, q=x["q"][:600], k=x["k"][:600], v=x["v"][:600], log_alpha=x["log_alpha"][:600],
               beta=x["beta"][:600], h0=None if x["h0"] is None else x["h0"][:1],
               cu_seqlens=np.array([0, 600], np.int32))
    og, hg = run_packed(one, "bf16", 64, varlen=False, B=1, T=600)
    o_ref, h_ref, _ = oracle_run(x)
    assert_parity(of, o_ref, hf, h_ref, "bf16", "fused vs segmented: fused", cu=x["cu_seqlens"])
    assert_parity(og, o_ref[:600], hg, h_ref[:1], "bf16", "fused vs segmented: segmented", cu=one["cu_seqlens"])
    assert rel_l2(of[:600], og) <= 1e-2 and rel_l2(hf[:1], hg) <= 1e-2


# ----------------------------------------------------------------------------- gate kinds

@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("io,path,chunk", [("f32", "split", 64), ("bf16", "split", 64), ("bf16", "split", 128),
                                           ("bf16", "fused", 64), ("bf16", "few-pairs", 128)])
def test_gate_kinds(gate, io, path, chunk):
    """kda_chunk_fwd_gated with one decay per token and head (Gated DeltaNet) and with
    none (DeltaNet): the oracle runs the same recurrence with that decay on every key
    channel, or with log alpha = 0. Passes: split (fp32 at d = 128, bf16 at d = 64), fused
    (256 pairs) and fused with few pairs (12)."""
    seed = {"head": 101, "none": 102}[gate] + chunk
    if path == "fused":
        x = with_gate(gen([200, 200], 128, 128, 128, io, seed=seed), gate)
        _check(x, io, chunk, f"{gate} fused", varlen=False, B=2, T=200, gate=gate)
    else:
        d = 64 if (io == "bf16" and path == "split") else 128
        x = with_gate(gen([200, 130, 1], 4, d, d, io, seed=seed), gate)
        _check(x, io, chunk, f"{gate} {path}", gate=gate)


@pytest.mark.parametrize("path", ["split", "fused"])
def test_head_gate_equals_broadcast_channel_gate(path):
    """A per-head decay and the same decay given for every key channel: one arithmetic
    (split pass: bf16 at d = 64; fused pass: d = 128)."""
    d = 64 if path == "split" else 128
    x = with_gate(gen([150, 150], 128, d, d, "bf16", seed=111), "head")
    kw = dict(varlen=False, B=2, T=150) if path == "fused" else dict(varlen=True)
    oh, hh = run_packed(x, "bf16", 64, gate="head", **kw)
    oc, hc = run_packed(x, "bf16", 64, gate="channel", **kw)
    assert np.array_equal(oh, oc) and np.array_equal(hh, hc)


@pytest.mark.parametrize("gate", ["head", "none"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_gate_kinds(gate, io):
    o, st, o_ref, h_ref = _decode_steps(3, 4, 128, 128, io, 5, seed=7 + len(gate), gate=gate)
    assert_parity(o, o_ref, st[None], h_ref[None], io, f"decode {gate} {io}")


# ----------------------------------------------------------------------------- gates from pre-activations

def _preact_case(x, io, seed):
    """Pre-activations for x's tokens, and x with the gates they form (fp64, oracle) in place
    of its own: the oracle's input."""
    T, H, dk = x["q"].shape
    p = kda_synth.gen_preact(T, H, dk, io, seed)
    la, be = oracle.gate_prologue(p["a"], p["A_log"], p["dt_bias"], p["b"])
    return p, dict(x, log_alpha=la, beta=be)


@pytest.mark.parametrize("qk_norm", [False, True])
@pytest.mark.parametrize("io,path,chunk", [("f32", "split", 64), ("bf16", "split", 64), ("bf16", "split", 128),
                                           ("f32", "split", 128), ("bf16", "fused", 64), ("bf16", "few-pairs", 64)])
def test_preact_gates(io, path, chunk, qk_norm):
    """kda_chunk_fwd_preact: log alpha = -exp(A_log) softplus(a + dt_bias) and beta =
    sigmoid(b) formed in the kernels, and with qk_norm q, k = silu(.) / ||silu(.)|| per
    row too; the oracle runs the recurrence on the same gates (and q, k) formed in fp64.
    Passes: split (fp32 at d = 128, bf16 at d = 64), fused (256 pairs), fused with few
    pairs (12)."""
    import torch
    import gated_delta_rule_48_amd as kda
    if path == "fused":
        x = gen([200, 200], 128, 128, 128, io, seed=121)
    else:
        d = 64 if (io == "bf16" and path == "split") else 128
        x = gen([200, 130, 1], 4, d, d, io, seed=122 + chunk)
    p, y = _preact_case(x, io, seed=123 + chunk)
    if qk_norm:
        T, H, dk = x["q"].shape
        r = kda_synth.gen_qk_preact(T, H, dk, io, seed=124 + chunk)
        x = dict(x, q=r["q"], k=r["k"])
        y = dict(y, q=oracle.qk_prologue(r["q"]), k=oracle.qk_prologue(r["k"]))
    say(f"[preact {path}] io={io} C={chunk} qk_norm={qk_norm}")
    t = to_dev(x, io)
    iod = torch.bfloat16 if io == "bf16" else torch.float32
    a = torch.from_numpy(p["a"]).cuda().to(iod)
    A_log, dt_bias, b = (torch.from_numpy(p[n]).cuda() for n in ("A_log", "dt_bias", "b"))
    if path == "fused":
        B, T = 2, 200
        r = lambda z: z.reshape((B, T) + tuple(z.shape[1:]))  # noqa: E731
        o, hT = kda.chunk_fwd_preact(r(t["q"]), r(t["k"]), r(t["v"]), r(a), A_log, dt_bias, r(b), h0=t["h0"],
                                     chunk=chunk, qk_norm=qk_norm)
        o = o.reshape(t["v"].shape)
    else:
        o, hT = kda.chunk_fwd_preact(t["q"], t["k"], t["v"], a, A_log, dt_bias, b, h0=t["h0"],
                                     cu_seqlens=t["cu_seqlens"], chunk=chunk, qk_norm=qk_norm)
    torch.cuda.synchronize()
    o_ref, h_ref, _ = oracle_run(y)
    assert_parity(o.float().cpu().numpy(), o_ref, hT.cpu().numpy(), h_ref, io, f"preact {path}",
                  cu=x["cu_seqlens"])


@pytest.mark.parametrize("qk_norm", [False, True])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_preact_gates(io, qk_norm):
    """Five decode steps of kda_recurrent_step_preact against the oracle on the same gates
    (and, with qk_norm, the same normalised q and k)."""
    import torch
    import gated_delta_rule_48_amd as kda
    N, H, dk, dv, steps = 3, 4, 128, 128, 5
    st0 = kda_synth.gen_decode_state(N, H, dk, dv, 131)
    state = torch.from_numpy(st0).cuda()
    iod = torch.bfloat16 if io == "bf16" else torch.float32
    got, toks = [], []
    for step in range(steps):
        y = kda_synth.gen_decode_step(N, H, dk, dv, io, "main", 131, step)
        qk_ref = None
        if qk_norm:
            r = kda_synth.gen_qk_preact(N, H, dk, io, 2000 + step)
            y = dict(y, q=r["q"], k=r["k"])
            qk_ref = (oracle.qk_prologue(r["q"]), oracle.qk_prologue(r["k"]))
        p = kda_synth.gen_preact(N, H, dk, io, 1000 + step)
        la, be = oracle.gate_prologue(p["a"], p["A_log"], p["dt_bias"], p["b"])
        t = to_dev(dict(y, cu_seqlens=np.zeros(1, np.int32)), io)
        a = torch.from_numpy(p["a"]).cuda().to(iod)
        A_log, dt_bias, b = (torch.from_numpy(p[n]).cuda() for n in ("A_log", "dt_bias", "b"))
        o = kda.recurrent_step_preact(t["q"], t["k"], t["v"], a, A_log, dt_bias, b, state, qk_norm=qk_norm)
        got.append(o.float().cpu().numpy())
        qv, kv = qk_ref if qk_norm else (y["q"], y["k"])
        toks.append(dict(q=qv, k=kv, v=y["v"], log_alpha=la, beta=be))
    torch.cuda.synchronize()
    # the (n, h) pairs as independent heads of one sequence of `steps` tokens
    seq = {n: np.stack([tk[n].reshape((N * H,) + tk[n].shape[2:]) for tk in toks]) for n in toks[0]}
    o_ref, h_ref = oracle.kda_reference(seq["q"], seq["k"], seq["v"], seq["log_alpha"], seq["beta"], dk ** -0.5,
                                        h0=st0.reshape(1, N * H, dk, dv))
    assert_parity(np.stack(got).reshape(steps, N * H, dv), o_ref, state.cpu().numpy().reshape(1, N * H, dk, dv),
                  h_ref, io, f"decode preact {io}")


@pytest.mark.parametrize("gate", ["channel", "head", "none"])
def test_fused_packed_sequences(gate):
    """Packed sequences through the fused pass (bf16, d = 128, chunk 64, n_seqs x H >= 256):
    empty, one-token, ragged and chunk-aligned sequences, with per-sequence h0."""
    x = gen((0, 1, 63, 64, 65, 130, 0, 200), 32, 128, 128, "bf16", "main", "normal", seed=71)
    _check(with_gate(x, gate), "bf16", 64, f"fused-packed-{gate}", varlen=True, gate=gate)


def test_fused_packed_workload():
    """varlen_many: 16 packed sequences of mixed lengths (1 to 8192, 65,536 tokens), H=32,
    the whole batch against the oracle."""
    w = kda_synth.WORKLOADS["varlen_many"]
    x = kda_synth.gen_workload(w)
    _check(x, "bf16", w.chunk, "varlen_many", varlen=True)
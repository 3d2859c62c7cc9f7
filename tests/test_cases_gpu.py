"""GPU cases of the method's own regimes, through the C ABI: the worked 2x2 (and 1x1)
memory examples of the "ten questions" page run through the chunked passes and the
decode step, and colliding keys at beta = 1 (the delta rule's overwrite regime).

Worked examples (tests/golden/ten_questions_2x2.json, its delta-rule cases): each
example's q, k, v are zero-padded to d = 64 (split pass, fp32, one head) and to d = 128
over 256 (sequence, head) pairs (fused pass, bf16); the padded decay channels keep
alpha = 1 and h0 is padded with zeros. The page's printed o and final S must appear in
the leading entries and zeros elsewhere: to 1e-5 on the fp32 pass and to 2e-2 on the
bf16 pass (or the example's own tolerance where the page rounds, as "0.9^20 = 0.12"), whose inputs (0.6, 0.8, sqrt 2, ...) are rounded to bf16 first; the bf16 run
is also held to the usual parity bar against the oracle on the rounded inputs.

Colliding keys: kda_synth.gen_key_repeats, exact repeats among three keys per head and
near-duplicates (cosine about 0.99), beta = 1, on the fused pass (one workgroup per
(sequence, head), and with segments), the split pass (bf16 at d = 64, fp32 at d = 128,
chunks 64 and 128) and the decode step, against the oracle with the per-head and per-row
bounds of kda_testlib.
"""
import json
import os

import numpy as np
import pytest

import kda_synth
import oracle
from kda_testlib import assert_parity, oracle_run, run_packed, say, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ten_questions_2x2.json")


def _delta_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    return [c for c in cases if "delta" in c["modes"]]


def _padded(case, d):
    """The example's steps as one sequence of T tokens and one head, zero-padded to d:
    (x [T, 1, d] arrays, h0 [1, 1, d, d], T, the example's own width n)."""
    steps = case["steps"] * case.get("repeat", 1)
    T, n = len(steps), len(steps[0]["k"])
    x = {n_: np.zeros((T, 1, d), np.float32) for n_ in ("q", "k", "v")}
    x["log_alpha"] = np.zeros((T, 1, d), np.float32)
    x["beta"] = np.zeros((T, 1), np.float32)
    for t, s in enumerate(steps):
        x["q"][t, 0, :n] = s["q"]
        x["k"][t, 0, :n] = s["k"]
        x["v"][t, 0, :n] = s["v"]
        x["log_alpha"][t, 0, :n] = np.log(np.asarray(s["alpha"], np.float64))
        x["beta"][t, 0] = s["beta"]
    h0 = np.zeros((1, 1, d, d), np.float32)
    if case["h0"] is not None:
        h0[0, 0, :n, :n] = case["h0"]
    return x, h0, T, n


def _expect(case, o, hT, n, tol, tag):
    """o [T, d], hT [d, d]: the printed values in the leading entries, zeros elsewhere."""
    d = o.shape[-1]
    if case["expect_o"] is not None:
        for t, row in enumerate(case["expect_o"]):
            if row is not None:
                assert np.max(np.abs(o[t, :n] - np.asarray(row))) <= tol, (tag, t, o[t, :n], row)
    assert np.max(np.abs(o[:, n:])) <= tol, (tag, "padding of o")
    if case["expect_hT"] is not None:
        want = np.zeros((d, d))
        want[:n, :n] = case["expect_hT"]
        assert np.max(np.abs(hT - want)) <= tol, (tag, hT[:n, :n], case["expect_hT"])


@pytest.mark.parametrize("case", _delta_cases(), ids=lambda c: c["name"])
def test_worked_example_split_fp32(case):
    import torch
    import gated_delta_rule_48_amd as kda
    x, h0, T, n = _padded(case, 64)
    say(f"[worked {case['name']}] split pass, fp32, d=64, T={T}")
    t = {k_: torch.from_numpy(v_).cuda() for k_, v_ in x.items()}
    o, hT = kda.chunk_fwd(t["q"][None], t["k"][None], t["v"][None], t["log_alpha"][None], t["beta"][None],
                          scale=1.0, h0=torch.from_numpy(h0).cuda(), chunk=64)
    torch.cuda.synchronize()
    _expect(case, o[0, :, 0].cpu().numpy(), hT[0, 0].cpu().numpy(), n, max(case["tol"], 1e-5), case["name"])


@pytest.mark.parametrize("case", _delta_cases(), ids=lambda c: c["name"])
def test_worked_example_decode(case):
    import torch
    import gated_delta_rule_48_amd as kda
    x, h0, T, n = _padded(case, 64)
    t = {k_: torch.from_numpy(v_).cuda() for k_, v_ in x.items()}
    state = torch.from_numpy(h0).cuda()
    outs = []
    for i in range(T):
        outs.append(kda.recurrent_step(t["q"][i:i + 1], t["k"][i:i + 1], t["v"][i:i + 1], t["log_alpha"][i:i + 1],
                                       t["beta"][i:i + 1], state, scale=1.0))
    torch.cuda.synchronize()
    o = torch.cat(outs)[:, 0].cpu().numpy()
    _expect(case, o, state[0, 0].cpu().numpy(), n, max(case["tol"], 1e-5), case["name"])


@pytest.mark.parametrize("case", _delta_cases(), ids=lambda c: c["name"])
def test_worked_example_fused_bf16(case):
    """The example in all 256 (sequence, head) pairs (B = 2, H = 128) of a fused-pass call."""
    import torch
    import gated_delta_rule_48_amd as kda
    x, h0, T, n = _padded(case, 128)
    B, H = 2, 128
    say(f"[worked {case['name']}] fused pass, bf16, d=128, B={B} H={H} T={T}")
    rep = lambda a: np.ascontiguousarray(np.broadcast_to(a[None], (B,) + a.shape[:1] + (H,) + a.shape[2:]))  # noqa
    xb = {k_: rep(v_) for k_, v_ in x.items()}
    for k_ in ("q", "k", "v"):
        xb[k_] = kda_synth.round_bf16(xb[k_])
    h0b = np.ascontiguousarray(np.broadcast_to(h0[0, 0], (B, H) + h0.shape[2:]))
    dv = lambda a, dt=None: torch.from_numpy(a).cuda() if dt is None else torch.from_numpy(a).cuda().to(dt)  # noqa
    o, hT = kda.chunk_fwd(dv(xb["q"], torch.bfloat16), dv(xb["k"], torch.bfloat16), dv(xb["v"], torch.bfloat16),
                          dv(xb["log_alpha"]), dv(xb["beta"]), scale=1.0, h0=dv(h0b), chunk=64)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    hT = hT.cpu().numpy()
    for b, h in ((0, 0), (1, 127), (1, 64)):
        _expect(case, o[b, :, h], hT[b, h], n, max(case["tol"], 2e-2), f"{case['name']} ({b}, {h})")
    # and the parity bar against the oracle on the rounded inputs, every pair
    packed = {k_: xb[k_].reshape((B * T,) + xb[k_].shape[2:]) for k_ in xb}
    packed["cu_seqlens"] = np.array([0, T, 2 * T], np.int32)
    o_ref1, h_ref1 = oracle.kda_reference(packed["q"], packed["k"], packed["v"], packed["log_alpha"],
                                          packed["beta"], 1.0, h0=h0b, cu_seqlens=packed["cu_seqlens"])
    assert_parity(o.reshape(B * T, H, 128), o_ref1, hT, h_ref1, "bf16", f"worked {case['name']} fused",
                  cu=packed["cu_seqlens"])


# ----------------------------------------------------------------------------- colliding keys

KINDS = ["repeat", "near"]


@pytest.mark.parametrize("kind", KINDS)
def test_colliding_keys_fused(kind):
    x = kda_synth.gen_key_repeats([200, 200], 128, 128, 128, "bf16", kind, seed=301)
    say(f"[keys {kind}] fused pass, bf16, B=2 H=128 T=200, beta=1")
    o, hT = run_packed(x, "bf16", 64, varlen=False, B=2, T=200)
    o_ref, h_ref, _ = oracle_run(x)
    assert_parity(o, o_ref, hT, h_ref, "bf16", f"keys {kind} fused", cu=x["cu_seqlens"])


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("io,chunk,d", [("bf16", 64, 64), ("bf16", 128, 64), ("f32", 64, 128), ("f32", 128, 128)])
def test_colliding_keys_split(kind, io, chunk, d):
    """The split pass: fp32 at d = 128, and bf16 at d = 64 (bf16 at d = 128 takes the fused pass)."""
    x = kda_synth.gen_key_repeats([300, 129, 64], 4, d, d, io, kind, seed=302 + chunk)
    say(f"[keys {kind}] split pass, {io}, d={d}, C={chunk}, beta=1")
    o, hT = run_packed(x, io, chunk)
    o_ref, h_ref, _ = oracle_run(x)
    assert_parity(o, o_ref, hT, h_ref, io, f"keys {kind} split {io} d{d} C{chunk}", cu=x["cu_seqlens"])


@pytest.mark.parametrize("kind", KINDS)
def test_colliding_keys_segmented(kind):
    """bf16, d = 128, 12 (sequence, head) pairs: the fused pass with segments (the 300-token
    sequence is longer than one segment)."""
    x = kda_synth.gen_key_repeats([300, 129, 64], 4, 128, 128, "bf16", kind, seed=304)
    say(f"[keys {kind}] fused pass with segments, bf16, beta=1")
    o, hT = run_packed(x, "bf16", 64)
    o_ref, h_ref, _ = oracle_run(x)
    assert_parity(o, o_ref, hT, h_ref, "bf16", f"keys {kind} segmented", cu=x["cu_seqlens"])


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_colliding_keys_decode(kind, io):
    """The same tokens through T decode steps: o of every step and the final states."""
    import torch
    import gated_delta_rule_48_amd as kda
    T, H = 150, 4
    x = kda_synth.gen_key_repeats([T], H, 128, 128, io, kind, seed=303)
    t = to_dev(x, io)
    state = t["h0"].clone()
    outs = []
    for i in range(T):
        outs.append(kda.recurrent_step(t["q"][i:i + 1], t["k"][i:i + 1], t["v"][i:i + 1], t["log_alpha"][i:i + 1],
                                       t["beta"][i:i + 1], state))
    torch.cuda.synchronize()
    o = torch.cat(outs).float().cpu().numpy()
    o_ref, h_ref, _ = oracle_run(x)
    assert_parity(o, o_ref, state.cpu().numpy(), h_ref, io, f"keys {kind} decode {io}")

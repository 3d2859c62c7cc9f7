"""The fused pass with segments (bf16, d = 128, fewer than 256 (sequence, head) pairs):
long sequences cut into segments, each segment's map S_out = M S_in + N formed in
parallel, the maps composed in order, then every segment run from its entering state.
Against the fp64 oracle with the usual parity bar, for equal-length and packed
sequences (empty, one-token and ragged ones among them), with and without h0 and hT,
for every gate kind, and with chunks of strong decay inside one segment of a pair (the
pair then runs again on the strong instance)."""
import numpy as np
import pytest

import kda_synth
import oracle
from kda_testlib import assert_parity, gen, oracle_run, run_packed, say, to_dev, with_gate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H", [(3000, 4), (4096, 16), (10000, 2)])
def test_segments_equal_length(T, H):
    x = gen([T], H, 128, 128, "bf16", seed=601 + H)
    say(f"[segments] B=1 T={T} H={H}")
    o, hT = run_packed(x, "bf16", 64, varlen=False, B=1, T=T)
    o_ref, h_ref, _ = oracle_run(x)
    assert_parity(o, o_ref, hT, h_ref, "bf16", f"segments T={T} H={H}", cu=x["cu_seqlens"])


@pytest.mark.parametrize("chunk", [64, 128])
def test_segments_packed(chunk):
    x = gen([0, 1000, 7, 2049, 0, 300, 1, 4097], 3, 128, 128, "bf16", seed=611)
    say(f"[segments] packed {np.diff(x['cu_seqlens']).tolist()}, H=3, chunk {chunk}")
    o, hT = run_packed(x, "bf16", chunk)
    o_ref, h_ref, _ = oracle_run(x)
    assert_parity(o, o_ref, hT, h_ref, "bf16", f"segments packed C{chunk}", cu=x["cu_seqlens"])


def test_segments_no_h0_no_hT():
    x = gen([2500, 1800], 2, 128, 128, "bf16", h0="zero", seed=612)
    o, hT = run_packed(x, "bf16", 64, h0=False, hT=False)
    assert hT is None
    o_ref, _, _ = oracle_run(x, h0=False)
    assert_parity(o, o_ref, None, None, "bf16", "segments no h0/hT", cu=x["cu_seqlens"])


@pytest.mark.parametrize("gate", ["head", "none"])
def test_segments_gate_kinds(gate):
    x = with_gate(gen([3100, 900], 4, 128, 128, "bf16", seed=613), gate)
    o, hT = run_packed(x, "bf16", 64, gate=gate)
    o_ref, h_ref, _ = oracle_run(x)
    assert_parity(o, o_ref, hT, h_ref, "bf16", f"segments {gate}", cu=x["cu_seqlens"])


@pytest.mark.parametrize("qk_norm", [False, True])
def test_segments_preact(qk_norm):
    import torch
    import gated_delta_rule_48_amd as kda
    x = gen([2600, 700], 3, 128, 128, "bf16", seed=614)
    T, H, dk = x["q"].shape
    p = kda_synth.gen_preact(T, H, dk, "bf16", seed=615)
    la, be = oracle.gate_prologue(p["a"], p["A_log"], p["dt_bias"], p["b"])
    y = dict(x, log_alpha=la, beta=be)
    if qk_norm:
        r = kda_synth.gen_qk_preact(T, H, dk, "bf16", seed=616)
        x = dict(x, q=r["q"], k=r["k"])
        y = dict(y, q=oracle.qk_prologue(r["q"]), k=oracle.qk_prologue(r["k"]))
    t = to_dev(x, "bf16")
    a = torch.from_numpy(p["a"]).cuda().to(torch.bfloat16)
    A_log, dt_bias, b = (torch.from_numpy(p[n]).cuda() for n in ("A_log", "dt_bias", "b"))
    o, hT = kda.chunk_fwd_preact(t["q"], t["k"], t["v"], a, A_log, dt_bias, b, h0=t["h0"],
                                 cu_seqlens=t["cu_seqlens"], qk_norm=qk_norm)
    torch.cuda.synchronize()
    o_ref, h_ref, _ = oracle_run(y)
    assert_parity(o.float().cpu().numpy(), o_ref, hT.cpu().numpy(), h_ref, "bf16", f"segments preact qk={qk_norm}",
                  cu=x["cu_seqlens"])


def test_segments_strong_decay_in_one_segment():
    """Head 1 of the long sequence decays strongly (chunk sums near -2000) in tokens 1100 ..
    1300 only (inside one segment); head 0 never: the pair of head 1 runs again on the strong
    instance, head 0 keeps its segments."""
    x = gen([3000, 400], 2, 128, 128, "bf16", seed=617)
    strong = kda_synth.gen_sequences((200,), 2, 128, 128, "bf16", "sum2000", "zero", 618)["log_alpha"]
    x["log_alpha"][1100:1300, 1] = strong[:, 1]
    o, hT = run_packed(x, "bf16", 64)
    o_ref, h_ref, _ = oracle_run(x)
    assert_parity(o, o_ref, hT, h_ref, "bf16", "segments strong in one segment", cu=x["cu_seqlens"])


def test_segments_deterministic():
    x = gen([5000, 1234], 3, 128, 128, "bf16", seed=619)
    o1, h1 = run_packed(x, "bf16", 64)
    o2, h2 = run_packed(x, "bf16", 64)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)

"""GPU parity of the softmax-attention decode step over a KV cache (kda_attn_decode,
the comparator of the KDA decode step) against the fp64 oracle.

Bar: relative L2 error of o <= 1e-4 with fp32 I/O and <= 2e-2 with bf16 I/O (the
library's bars). Small cases draw their inputs on the host (kda_synth.gen_attn_decode)
and compare every output; the two full-size workloads draw their caches on the GPU
(kda_synth.gen_attn_decode_device, torch's seeded generator) and compare sampled
(sequence, head) outputs, the oracle reading host copies of exactly those cache rows.
"""
import numpy as np
import pytest

import kda_synth
import oracle
from kda_testlib import TOL, rel_l2, say

pytestmark = pytest.mark.gpu


def _run(x, io, seq_lens, scale=None):
    import torch
    import gated_delta_rule_48_amd as kda
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    q = torch.from_numpy(x["q"]).cuda().to(dt)
    k = torch.from_numpy(x["k_cache"]).cuda().to(dt)
    v = torch.from_numpy(x["v_cache"]).cuda().to(dt)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    o = kda.attn_decode(q, k, v, seq_lens=sl, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


def _check(name, B, H, H_kv, T_max, d, io, seq_lens, seed, scale=None):
    say(f"[{name}] B={B} H={H} H_kv={H_kv} T_max={T_max} d={d} io={io} seq_lens={seq_lens}")
    x = kda_synth.gen_attn_decode(B, H, H_kv, T_max, d, io, seed)
    o = _run(x, io, seq_lens, scale)
    ref = oracle.attn_decode_reference(x["q"], x["k_cache"], x["v_cache"], seq_lens, scale)
    err = rel_l2(o, ref)
    say(f"[{name}] rel_l2 o={err:.2e}")
    assert np.all(np.isfinite(o))
    assert err <= TOL[io], err
    return o, ref


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_attn_decode_ragged_lengths(io, d, G):
    # one split per (sequence, cached head); lengths that end mid-iteration, a single row
    _check("ragged", 3, 2 * G, 2, 300, d, io, [300, 1, 173], seed=11 + G)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 8])
def test_attn_decode_split_cache(io, d, G):
    # 5000 rows over 4 splits of 1280: a sequence ending inside the second split (the
    # others empty), and one with no rows at all (o = 0); groups of 1 and of 8 query heads
    # per cached head (the split partials and the combine kernel at H = 8 H_kv)
    o, _ = _check("splits", 3, 2 * G, 2, 5000, d, io, [5000, 2049, 0], seed=21 + G, scale=0.11)
    assert np.all(o[2] == 0)


def test_attn_decode_many_splits():
    # one cached head of 300,000 rows: 261 splits of 1,152 rows (more splits than the
    # combine kernel has threads), the last one partly filled
    _check("many-splits", 1, 2, 1, 300000, 64, "f32", [299999], seed=41)


def test_attn_decode_all_rows_and_empty_cache():
    import torch
    import gated_delta_rule_48_amd as kda
    _check("all-rows", 2, 8, 4, 700, 128, "bf16", None, seed=31)
    # no cached rows at all: o = 0
    q = torch.randn(2, 4, 128, device="cuda", dtype=torch.bfloat16)
    empty = torch.empty((2, 4, 0, 128), device="cuda", dtype=torch.bfloat16)
    o = kda.attn_decode(q, empty, empty)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0


@pytest.mark.parametrize("name", sorted(kda_synth.ATTN_WORKLOADS))
def test_attn_decode_full_size_sampled(name):
    import torch
    import gated_delta_rule_48_amd as kda
    B, H, H_kv, T_max, d, io, seed = kda_synth.ATTN_WORKLOADS[name]
    say(f"[full {name}] B={B} H={H} H_kv={H_kv} T_max={T_max} d={d} io={io} seed={seed}")
    x = kda_synth.gen_attn_decode_device(B, H, H_kv, T_max, d, torch.bfloat16, seed, "cuda")
    n_ws = kda.attn_decode_workspace_bytes(B, H, H_kv, d, T_max, kda.KDA_BF16)
    say(f"[full {name}] workspace {n_ws} bytes")
    o = kda.attn_decode(x["q"], x["k_cache"], x["v_cache"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    picks = sorted({(int(rng.integers(B)), int(rng.integers(H))) for _ in range(6)} | {(B - 1, H - 1)})
    got, want = [], []
    for b, h in picks:
        j = h // (H // H_kv)
        q = x["q"][b:b + 1, h:h + 1].float().cpu().numpy()
        K = x["k_cache"][b:b + 1, j:j + 1].float().cpu().numpy()
        V = x["v_cache"][b:b + 1, j:j + 1].float().cpu().numpy()
        want.append(oracle.attn_decode_reference(q, K, V, scale=d ** -0.5)[0, 0])
        got.append(o[b, h].float().cpu().numpy())
    err = rel_l2(np.array(got), np.array(want))
    say(f"[full {name}] sampled {picks} rel_l2 o={err:.2e}")
    del x, o
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(got))
    assert err <= TOL[io], err

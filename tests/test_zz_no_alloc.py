"""kda_chunk_fwd_noalloc (the prefill entry point that allocates nothing: its workspace
is a fixed device array inside the library) against kda_chunk_fwd_gated with a caller
workspace: the same kernels, so the same bits. Two calls in a row on each pass, the
second smaller than the first (the array keeps the first call's contents, which no call
may read), and a size whose workspace exceeds the array's, which is refused before
anything runs."""
import numpy as np
import pytest

from kda_testlib import gen, say, to_dev

pytestmark = pytest.mark.gpu


def _both(x, io, chunk, varlen, B=None, T=None):
    import torch
    import gated_delta_rule_48_amd as kda
    t = to_dev(x, io)
    if varlen:
        args = (t["q"], t["k"], t["v"], t["log_alpha"], t["beta"])
        kw = dict(h0=t["h0"], cu_seqlens=t["cu_seqlens"], chunk=chunk)
    else:
        r = lambda a: a.reshape((B, T) + tuple(a.shape[1:]))  # noqa: E731
        args = (r(t["q"]), r(t["k"]), r(t["v"]), r(t["log_alpha"]), r(t["beta"]))
        kw = dict(h0=t["h0"], chunk=chunk)
    o1, h1 = kda.chunk_fwd(*args, **kw)
    o2 = torch.full_like(o1, float("nan"))
    h2 = torch.full_like(h1, float("nan"))
    kda.chunk_fwd_noalloc(*args, o=o2, hT=h2, **kw)
    torch.cuda.synchronize()
    return o1.float().cpu().numpy(), h1.cpu().numpy(), o2.float().cpu().numpy(), h2.cpu().numpy()


def _same(name, got):
    o1, h1, o2, h2 = got
    say(f"[noalloc {name}] o {o1.shape}: identical={np.array_equal(o1, o2)}, hT identical={np.array_equal(h1, h2)}")
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(h2))
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


def test_noalloc_fused_pass_two_calls():
    """The one-launch pass (bf16, d = 128, chunk 64, 256 pairs): 2 x 300 tokens, then 2 x 70."""
    x = gen([300, 300], 128, 128, 128, "bf16", seed=401)
    _same("fused 2x300", _both(x, "bf16", 64, False, B=2, T=300))
    x = gen([70, 70], 128, 128, 128, "bf16", seed=402)
    _same("fused 2x70", _both(x, "bf16", 64, False, B=2, T=70))


def test_noalloc_split_pass_two_calls():
    """The split pass (chunk table, per-chunk operands and the discard slot in the array):
    packed sequences at chunk 128, then a smaller packed batch at chunk 64, then fp32."""
    x = gen([500, 0, 129, 300], 4, 128, 128, "bf16", seed=403)
    _same("split varlen C128", _both(x, "bf16", 128, True))
    x = gen([65, 1, 200], 2, 128, 128, "bf16", seed=404)
    _same("split varlen C64", _both(x, "bf16", 64, True))
    x = gen([100, 100], 2, 64, 64, "f32", seed=405)
    _same("split f32 2x100", _both(x, "f32", 64, False, B=2, T=100))


def test_noalloc_refuses_oversized_workspace():
    """A split-pass call whose workspace exceeds the array: KDA_ERR_WORKSPACE, o untouched."""
    import torch
    import gated_delta_rule_48_amd as kda
    B, T, H, d = 1, 8192, 16, 128
    need = kda.workspace_bytes(B, T, H, d, d, 64, 0, kda.KDA_BF16)
    assert need > kda.binding.NOALLOC_MAX_WORKSPACE
    q = torch.zeros((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    la = torch.zeros((B, T, H, d), device="cuda")
    beta = torch.zeros((B, T, H), device="cuda")
    o = torch.full((B, T, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_fwd_noalloc(q, q, q, la, beta, o=o)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())

"""CPU tests of the C ABI: the library loads, exports exactly what include/kda.h
declares, and rejects bad arguments with the documented status before anything
is launched (every call below returns during host-side validation, so the fake
device addresses are never touched)."""
import os
import re
import subprocess

import pytest

import gated_delta_rule_48_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1
A = 0x10000  # fake, 256-byte aligned "device" addresses, never dereferenced


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return kda.load()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(kda.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, name
        getattr(lib, name)
    assert {n for n in exported if n.startswith("kda_")} == set(declared_functions())


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 6
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (3, b"workspace missing, misaligned or too small")]:
        assert lib.kda_status_string(code) == text
    assert lib.kda_status_string(99) == b"unknown status"


def _ws_expect(B, T, H, dk, dv, C, n_seqs, esz):
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    n_seq = n_seqs if n_seqs else B
    pairs = n_seq * H
    if esz == 2 and dk == dv == 128 and T > 0:
        # fused pass (equal-length or packed sequences, any chunk size asked): the 256-byte
        # discard slot and a flag byte per unit for the strong-decay instance. From 256 pairs
        # on, one unit per pair. Below, the plan: two launches of at most u = 256 // H units per
        # head (2 u flag bytes per head), the plan table of packed sequences, and per segment
        # slot an entering state and a map. Slots per head: packed, min(u, c + n_seqs) (launch
        # C's units hold a chunk each at least); equal lengths, B (P - 1) with P = ceil(c / T)
        # segments for the budget T: from the smallest t with B max(ceil(c / t) - 1, 1) <= u,
        # the lowest 8 T + max(P - 2, 0) (no cut, P = 1, below 8 chunks).
        if pairs >= 256:
            return 256 + r(n_seq * H)
        u, c = 256 // H, (T + 63) // 64
        total = 256 + r(2 * u * H)
        if n_seqs:
            slots = min(u, c + n_seqs)
            total += r((4 * n_seqs + 3) * 4)
        else:
            ua = lambda t: max(-(-c // t) - 1, 1) if c > t else 1  # noqa: E731
            t = c if c < 8 else next(t for t in range(1, c + 1) if B * ua(t) <= u)
            cost = lambda t: 8 * t + max(-(-c // t) - 2, 0)  # noqa: E731
            tb, t2 = t, t + 1  # the budget: the lowest cost from t on (8 T + composition steps)
            while t2 <= c and 8 * t2 <= cost(tb):
                tb = t2 if cost(t2) < cost(tb) else tb
                t2 += 1
            slots = B * (-(-c // tb) - 1)
        total += r(slots * H * dk * dv * 4) + r(slots * H * 2 * dk * dv * 4)
        return total
    per = (T + C - 1) // C
    nch = (per + n_seqs if n_seqs else B * per) * H
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    total = 0
    for nbytes in (nch * C * dk * esz, nch * C * dv * esz, nch * C * dk * esz, nch * dk * C * esz,
                   nch * C * C * esz, nch * dk * 4, nch, 256):
        total += r(nbytes)
    if n_seqs:
        total += r((3 * n_seqs + 1) * 4)
    return total


@pytest.mark.parametrize("args", [(8, 8192, 32, 128, 128, 64, 0, BF16), (1, 65536, 32, 128, 128, 128, 4, BF16),
                                  (1, 65536, 32, 128, 128, 64, 16, BF16), (1, 65536, 32, 128, 128, 64, 4, BF16),
                                  (1, 256, 2, 64, 64, 64, 0, F32), (3, 77, 5, 64, 128, 128, 0, F32)])
def test_workspace_size(lib, args):
    B, T, H, dk, dv, C, ns, io = args
    got = lib.kda_chunk_fwd_workspace_bytes(*args)
    assert got == _ws_expect(B, T, H, dk, dv, C, ns, 2 if io == BF16 else 4)


def test_workspace_size_degenerate(lib):
    assert lib.kda_chunk_fwd_workspace_bytes(2, 0, 4, 128, 128, 64, 0, BF16) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(2, 10, 4, 96, 128, 64, 0, BF16) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(2, 10, 4, 128, 128, 32, 0, BF16) == 0


def fwd(lib, **kw):
    a = dict(B=2, T=100, H=4, dk=128, dv=128, chunk=64, io=BF16, q=A, k=A, v=A, la=A, beta=A,
             scale=0.088, h0=None, cu=None, n_seqs=0, o=0x4000000, hT=None, ws=A, ws_bytes=1 << 40,
             stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd(a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["io"], a["q"],
                             a["k"], a["v"], a["la"], a["beta"], a["scale"], a["h0"], a["cu"],
                             a["n_seqs"], a["o"], a["hT"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dk=96), UNSUPPORTED), (dict(dv=256), UNSUPPORTED), (dict(chunk=32), UNSUPPORTED),
    (dict(io=7), UNSUPPORTED), (dict(H=70000), UNSUPPORTED),
    (dict(B=0), INVALID), (dict(T=-1), INVALID), (dict(H=0), INVALID),
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(beta=None), INVALID),
    (dict(q=A + 8), INVALID), (dict(la=A + 4), INVALID), (dict(h0=A + 4), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(o=A), INVALID),                           # o aliases the inputs
    (dict(cu=A, n_seqs=2), INVALID),                # varlen needs B == 1
    (dict(B=1, cu=A, n_seqs=0), INVALID),
    (dict(cu=A + 2, B=1, n_seqs=2), INVALID),
    (dict(ws=None), WORKSPACE), (dict(ws=A + 16), WORKSPACE), (dict(ws_bytes=300), WORKSPACE),
])
def test_chunk_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


def step(lib, **kw):
    a = dict(N=4, H=2, dk=128, dv=128, io=BF16, q=A, k=A, v=A, la=A, beta=A, scale=0.088,
             state=0x4000000, o=0x8000000, stream=None)
    a.update(kw)
    return lib.kda_recurrent_step(a["N"], a["H"], a["dk"], a["dv"], a["io"], a["q"], a["k"], a["v"],
                                  a["la"], a["beta"], a["scale"], a["state"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), OK),  # nothing to do, nothing launched
    (dict(dk=32), UNSUPPORTED), (dict(io=2), UNSUPPORTED), (dict(N=-1), INVALID), (dict(H=0), INVALID),
    (dict(state=None), INVALID), (dict(q=A + 2), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(o=0x4000000 + 1024), INVALID),            # o inside the state
])
def test_recurrent_step_rejects(lib, kw, code):
    assert step(lib, **kw) == code


def fwd_gated(lib, gate, **kw):
    a = dict(B=2, T=100, H=4, dk=128, dv=128, chunk=64, io=BF16, q=A, k=A, v=A, la=A, beta=A,
             scale=0.088, h0=None, cu=None, n_seqs=0, o=0x4000000, hT=None, ws=A, ws_bytes=1 << 40,
             stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_gated(gate, a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["io"], a["q"],
                                   a["k"], a["v"], a["la"], a["beta"], a["scale"], a["h0"], a["cu"],
                                   a["n_seqs"], a["o"], a["hT"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("gate,kw,code", [
    (3, {}, INVALID), (-1, {}, INVALID),              # not a kda_gate value
    (0, dict(la=None), INVALID), (1, dict(la=None), INVALID),
    (0, dict(la=A + 4), INVALID),                     # per-channel decays: 16-byte aligned
    (1, dict(la=A + 2), INVALID),                     # per-head decays: 4-byte aligned
    (1, dict(la=A + 4, ws=None), WORKSPACE),          # ... which A + 4 is: validation goes on to the workspace
    (2, dict(la=None, ws=None), WORKSPACE),           # no decay: log_alpha is not needed
    (2, dict(la=None, dk=96), UNSUPPORTED),
])
def test_chunk_fwd_gated_validation(lib, gate, kw, code):
    assert fwd_gated(lib, gate, **kw) == code


def fwd_noalloc(lib, gate=0, **kw):
    a = dict(B=2, T=100, H=4, dk=128, dv=128, chunk=64, io=BF16, q=A, k=A, v=A, la=A, beta=A,
             scale=0.088, h0=None, cu=None, n_seqs=0, o=0x4000000, hT=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_noalloc(gate, a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["io"], a["q"],
                                     a["k"], a["v"], a["la"], a["beta"], a["scale"], a["h0"], a["cu"],
                                     a["n_seqs"], a["o"], a["hT"], a["stream"])


@pytest.mark.parametrize("gate,kw,code", [
    (3, {}, INVALID), (0, dict(dk=96), UNSUPPORTED), (0, dict(q=None), INVALID), (0, dict(o=A), INVALID),
    (0, dict(la=A + 4), INVALID), (2, dict(la=None, chunk=32), UNSUPPORTED), (0, dict(scale=float("nan")), INVALID),
    # split-pass sizes whose workspace exceeds the library's fixed array (32 MiB)
    (0, dict(B=1, T=8192, H=16, o=1 << 36), WORKSPACE), (0, dict(B=1, T=100000, H=4, io=F32, o=1 << 36), WORKSPACE),
])
def test_chunk_fwd_noalloc_validation(lib, gate, kw, code):
    """Everything is checked before the fixed workspace's address is looked up (which would
    need a GPU): these calls return during validation."""
    assert fwd_noalloc(lib, gate, **kw) == code


def test_noalloc_limit_matches_header(lib):
    text = open(HEADER).read()
    assert "#define KDA_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)" in text
    assert kda.binding.NOALLOC_MAX_WORKSPACE == 32 << 20
    # the one-launch pass needs its 256-byte discard slot and a byte per pair, at any length
    assert lib.kda_chunk_fwd_workspace_bytes(8, 1 << 20, 32, 128, 128, 64, 0, BF16) == 512


def test_chunk_fwd_is_the_per_channel_gated_call(lib):
    for kw in (dict(dk=96), dict(la=A + 4), dict(ws=None), dict(la=None)):
        assert fwd(lib, **kw) == fwd_gated(lib, 0, **kw)


@pytest.mark.parametrize("gate,kw,code", [
    (7, {}, INVALID), (0, dict(la=None), INVALID), (1, dict(la=None), INVALID), (1, dict(la=A + 2), INVALID),
    (2, dict(la=None, dk=32), UNSUPPORTED), (2, dict(la=None, N=0), OK),
])
def test_recurrent_step_gated_validation(lib, gate, kw, code):
    a = dict(N=4, H=2, dk=128, dv=128, io=BF16, q=A, k=A, v=A, la=A, beta=A, scale=0.088,
             state=0x4000000, o=0x8000000, stream=None)
    a.update(kw)
    assert lib.kda_recurrent_step_gated(gate, a["N"], a["H"], a["dk"], a["dv"], a["io"], a["q"], a["k"], a["v"],
                                        a["la"], a["beta"], a["scale"], a["state"], a["o"], a["stream"]) == code


def fwd_preact(lib, **kw):
    a = dict(B=2, T=100, H=4, dk=128, dv=128, chunk=64, io=BF16, q=A, k=A, v=A, pa=A, A_log=A, dt_bias=A, b=A,
             scale=0.088, h0=None, cu=None, n_seqs=0, o=0x4000000, hT=None, ws=A, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_preact(a.get("flags", 0), a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["io"], a["q"], a["k"],
                                    a["v"], a["pa"], a["A_log"], a["dt_bias"], a["b"], a["scale"], a["h0"], a["cu"],
                                    a["n_seqs"], a["o"], a["hT"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(pa=None), INVALID), (dict(A_log=None), INVALID), (dict(dt_bias=None), INVALID), (dict(b=None), INVALID),
    (dict(pa=A + 8), INVALID), (dict(dt_bias=A + 4), INVALID), (dict(A_log=A + 2), INVALID),
    (dict(o=A), INVALID), (dict(dk=96), UNSUPPORTED),
    (dict(A_log=A + 4, ws=None), WORKSPACE),        # A_log needs 4-byte alignment only: validation goes on
    (dict(flags=2), INVALID), (dict(flags=1, ws=None), WORKSPACE),
])
def test_chunk_fwd_preact_validation(lib, kw, code):
    assert fwd_preact(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(pa=None), INVALID), (dict(A_log=None), INVALID), (dict(dt_bias=A + 4), INVALID), (dict(N=0), OK),
    (dict(flags=4), INVALID), (dict(flags=1, N=0), OK),
])
def test_recurrent_step_preact_validation(lib, kw, code):
    a = dict(N=4, H=2, dk=128, dv=128, io=BF16, q=A, k=A, v=A, pa=A, A_log=A, dt_bias=A, b=A, scale=0.088,
             state=0x4000000, o=0x8000000, stream=None)
    a.update(kw)
    assert lib.kda_recurrent_step_preact(a.get("flags", 0), a["N"], a["H"], a["dk"], a["dv"], a["io"], a["q"], a["k"], a["v"], a["pa"],
                                         a["A_log"], a["dt_bias"], a["b"], a["scale"], a["state"], a["o"],
                                         a["stream"]) == code


# ---- softmax-attention decode over a KV cache (kda_attn_decode)

def attn(lib, **kw):
    a = dict(B=2, H=4, H_kv=2, d=128, T_max=100, io=BF16, q=A, k=0x4000000, v=0x8000000, lens=None, scale=0.088,
             o=0xC000000, ws=A, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.kda_attn_decode(a["B"], a["H"], a["H_kv"], a["d"], a["T_max"], a["io"], a["q"], a["k"], a["v"],
                               a["lens"], a["scale"], a["o"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), OK),                                       # nothing to do, nothing launched
    (dict(B=-1), INVALID), (dict(H=0), INVALID), (dict(H_kv=0), INVALID), (dict(T_max=-1), INVALID),
    (dict(H=6, H_kv=4), INVALID),                          # H % H_kv != 0
    (dict(H=32, H_kv=2), UNSUPPORTED),                     # groups of 16 query heads
    (dict(H=6, H_kv=2), UNSUPPORTED),                      # groups of 3
    (dict(d=96), UNSUPPORTED), (dict(io=2), UNSUPPORTED),
    (dict(B=65536, H=2, H_kv=2, T_max=1), UNSUPPORTED),    # grid limit
    (dict(T_max=1 << 24), UNSUPPORTED),                    # T_max * d >= 2^31
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(q=A + 8), INVALID), (dict(k=0x4000000 + 4), INVALID), (dict(lens=A + 2), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(o=0x4000000 + 4096), INVALID),                   # o inside the key cache
    (dict(o=A), INVALID),                                  # o is q
])
def test_attn_decode_rejects(lib, kw, code):
    assert attn(lib, **kw) == code


def test_attn_decode_workspace(lib):
    ws = lib.kda_attn_decode_workspace_bytes
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # one million rows of 32 heads: 4096 / 32 = 128 splits of 8192 rows
    assert ws(1, 32, 32, 128, 1 << 20, BF16) == r(32 * 128 * 128 * 4) + r(32 * 128 * 2 * 4)
    # 256 x 32 heads fill the chip alone (one split each): no workspace
    assert ws(256, 32, 32, 128, 4096, BF16) == 0
    # short caches are not split below 1024 rows
    assert ws(1, 4, 4, 64, 1023, F32) == 0
    # 5000 rows of 2 x 2 cached heads (4 query heads each): 4 splits of 1280 rows
    assert ws(2, 4, 2, 128, 5000, BF16) == r(2 * 4 * 4 * 128 * 4) + r(2 * 4 * 4 * 2 * 4)
    assert ws(0, 4, 2, 128, 5000, BF16) == 0 and ws(2, 4, 3, 128, 5000, BF16) == 0
    # the workspace is checked only when one is needed
    assert attn(lib, T_max=5000, ws=None) == WORKSPACE
    assert attn(lib, T_max=5000, ws=A + 16) == WORKSPACE
    assert attn(lib, T_max=5000, ws_bytes=1000) == WORKSPACE


# ---- backward pass (kda_chunk_bwd)

def bwd(lib, **kw):
    a = dict(B=2, T=100, H=4, dk=64, dv=64, chunk=64, io=F32, q=A, k=A, v=A, la=A, beta=A, scale=0.125, h0=None,
             dout=A, dhT=None, dq=0x4000000, dk_=0x5000000, dv_=0x6000000, dla=0x7000000, dbeta=0x8000000,
             dh0=None, ws=0x10000000, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.kda_chunk_bwd(a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["io"], a["q"], a["k"], a["v"],
                             a["la"], a["beta"], a["scale"], a["h0"], a["dout"], a["dhT"], a["dq"], a["dk_"],
                             a["dv_"], a["dla"], a["dbeta"], a["dh0"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), OK), (dict(T=0), OK),                      # nothing to do (no dh0 asked for)
    (dict(B=-1), INVALID), (dict(T=-1), INVALID), (dict(H=0), INVALID),
    (dict(io=BF16, ws=None), WORKSPACE),                   # bf16 is served: validation goes on
    (dict(io=5), UNSUPPORTED), (dict(chunk=128), UNSUPPORTED),
    (dict(dk=96), UNSUPPORTED), (dict(B=65536, T=1, H=1), UNSUPPORTED),
    (dict(q=None), INVALID), (dict(dout=None), INVALID), (dict(dq=None), INVALID), (dict(dbeta=None), INVALID),
    (dict(q=A + 8), INVALID), (dict(beta=A + 2), INVALID), (dict(dh0=0x9000000 + 4), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(dq=A), INVALID),                                 # an output on an input
    (dict(dk_=0x4000000 + 64), INVALID),                   # two outputs overlapping
    (dict(ws=None), WORKSPACE), (dict(ws=0x10000000 + 64), WORKSPACE), (dict(ws_bytes=4096), WORKSPACE),
    (dict(ws=A), INVALID),                                 # the workspace on an input
])
def test_chunk_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_chunk_bwd_workspace(lib):
    ws = lib.kda_chunk_bwd_workspace_bytes
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    C = 64

    def expect(B, T, H, dk, dv):
        per = 2 * C * C + 3 * C * dk + C * dv + dk + 2 * dk * dv
        scr = 15 * C * dk + 6 * C * dv + 5 * C * C + C + 2 * dk
        units = B * ((T + C - 1) // C) * H
        return (r(units * per * 4) + r(min(units, 1024) * scr * 4) + r(units) +
                _tok_expect(B * H, (T + C - 1) // C, dk, dv)) if units else 0

    for args in ((2, 100, 4, 64, 64), (8, 8192, 32, 128, 128), (1, 1, 1, 64, 128), (3, 0, 2, 128, 64)):
        assert ws(*args, 64, F32) == expect(*args), args
    assert ws(2, 100, 4, 64, 64, 64, BF16) == expect(2, 100, 4, 64, 64)  # fp32 buffers whatever the io dtype
    assert ws(2, 100, 4, 64, 64, 128, F32) == 0
    # bf16 at d = 128: the matrix-core pass, about 170 KB of bf16 buffers per (chunk, head)
    assert ws(8, 8192, 32, 128, 128, 64, BF16) == _bwd_fast_expect(8 * 128, 32, 0, 8 * 32, 128)
    assert ws(2, 100, 4, 128, 128, 64, BF16) == _bwd_fast_expect(2 * 2, 4, 0, 2 * 4, 2)
    assert ws(2, 0, 4, 128, 128, 64, BF16) == 0


def _tok_expect(n_pairs, n_blk, dk, dv):
    """The token pass's checkpoints: a state per 64-token block of the longest sequence and
    per 4-token group, for as many workgroups as 512 MiB holds (at least one, at most one per
    pair and 1024)."""
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    if n_pairs <= 0 or n_blk <= 0:
        return 0
    slot = (n_blk + 16) * dk * dv * 4
    return r(max(1, min((512 << 20) // slot, n_pairs, 1024)) * slot)


def _bwd_fast_expect(chunks, H, n_seqs_varlen, n_pairs, n_blk, C=64, d=128):
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    u = chunks * H
    parts = [u * C * d * 2, u * C * d * 2, u * C * d * 2, u * d * C * 2, u * C * C * 2, u * d * 4, u,
             u * d * d * 2, u * d * C * 2, u * d * d * 2, u * d * C * 2, 256]
    if n_seqs_varlen:
        parts.append((3 * n_seqs_varlen + 1) * 4)
    return sum(r(x) for x in parts) + _tok_expect(n_pairs, n_blk, d, d)


def bwd_varlen(lib, **kw):
    a = dict(T=300, H=4, dk=128, dv=128, chunk=64, io=BF16, q=A, k=A, v=A, la=A, beta=A, scale=0.125, h0=None,
             cu=0x3000000, n=3, dout=A, dhT=None, dq=0x4000000, dk_=0x5000000, dv_=0x6000000, dla=0x7000000,
             dbeta=0x8000000, dh0=None, ws=0x10000000, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.kda_chunk_bwd_varlen(a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["io"], a["q"], a["k"], a["v"],
                                    a["la"], a["beta"], a["scale"], a["h0"], a["cu"], a["n"], a["dout"], a["dhT"],
                                    a["dq"], a["dk_"], a["dv_"], a["dla"], a["dbeta"], a["dh0"], a["ws"],
                                    a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(io=F32), UNSUPPORTED), (dict(dk=64), UNSUPPORTED), (dict(dv=64), UNSUPPORTED), (dict(chunk=128), UNSUPPORTED),
    (dict(io=5), UNSUPPORTED), (dict(n=0), INVALID), (dict(T=-1), INVALID), (dict(H=0), INVALID),
    (dict(cu=None), INVALID), (dict(cu=0x3000000 + 2), INVALID), (dict(q=None), INVALID), (dict(q=A + 8), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(dq=A), INVALID), (dict(dq=0x3000000), INVALID),  # dq on cu_seqlens
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=4096), WORKSPACE), (dict(ws=0x10000000 + 16), WORKSPACE),
])
def test_chunk_bwd_varlen_rejects(lib, kw, code):
    assert bwd_varlen(lib, **kw) == code


def test_chunk_bwd_varlen_workspace(lib):
    ws = lib.kda_chunk_bwd_varlen_workspace_bytes
    # sized for ceil(T / 64) + n_seqs chunks, plus the chunk-offset table
    assert ws(300, 4, 128, 128, 64, 3, BF16) == _bwd_fast_expect(5 + 3, 4, 3, 3 * 4, 5)
    assert ws(0, 4, 128, 128, 64, 2, BF16) == _bwd_fast_expect(0 + 2, 4, 2, 2 * 4, 0)
    assert ws(300, 4, 128, 128, 64, 3, F32) == 0 and ws(300, 4, 64, 64, 64, 3, BF16) == 0
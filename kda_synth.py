"""Seeded synthetic inputs for the KDA gated delta-rule workloads.

This module is shared by the tests, the benchmark and the smoke check. It holds
none of the method's arithmetic: only random draws, the per-token L2
normalisation of q and k and the sigmoid / softplus squashing that the workload
recipes prescribe for the *inputs*, and round-to-nearest-even to bfloat16.

Workloads (sizes from the five benchmark configurations of this library):

  tiny     B=1  H=2  T=256   d=64   fp32 I/O  C=64   gates "weak"  h0 = 0
  prefill  B=1  H=16 T=4096  d=128  bf16 I/O  C=64   gates "main"  h0 ~ N(0, 0.02)
  batched  B=8  H=32 T=8192  d=128  bf16 I/O  C=64   gates "weak"  h0 = 0
  varlen   seqs 32768/16384/12288/4096 packed, H=32 d=128 bf16 C=128, gates "weak",
           per-sequence h0 ~ N(0, 0.02)
  decode   N=256 sequences, H=32, d=128, one bf16 token per step, gates "main",
           h0 ~ N(0, 0.02)
  batched_gdn, batched_deltanet: the batched workload with the decay given per token
           and head (the first key channel's draw) or not at all (`gate`)
  varlen_many: 16 packed sequences of mixed lengths (1 to 8192, 65,536 tokens), H=32, d=128,
           bf16, chunk 64, per-sequence h0 ~ N(0, 0.02)
  batched_preact: the batched workload with gate pre-activations (gen_preact) instead
           of log alpha and beta; batched_preact_qk: also q and k before silu and
           normalisation (gen_qk_preact)

Gate families (log alpha is drawn per token, per head and per key channel):
  weak:  log alpha = -0.1 * softplus(N(0,1)),  beta = sigmoid(N(0,1))
  main:  log alpha = -softplus(N(-2,1)),       beta = sigmoid(N(0,1))
  strong: log alpha = -1.3 softplus(N(1,1)),   beta = sigmoid(N(0,1))   (a test family: fast
          forgetting, chunk sums of log alpha near -110 on average)
  sum500, sum2000: log alpha = -(S/64) U(0.5, 1.5) with S = 500, 2000 (test families: chunk sums
          near -S per channel, where the chunked form's midpoint factors leave the fp32 range)
q and k are N(0,1) vectors L2-normalised per (token, head); v ~ N(0,1).
"N(mu, s)" means standard deviation s.

Attention-decode comparator (a softmax-attention layer's decode step over a KV
cache, weighed against the KDA decode step; ATTN_WORKLOADS):
  attn_batched  B=256 sequences, H = H_kv = 32, d=128, T_max=4096 cached rows, bf16:
                the decode workload's 256 x 32 (sequence, head) pairs at a 4K context
  attn_1m       B=1, H = H_kv = 32, d=128, T_max=1,048,576 (a one-million-token context)
q ~ N(0,1), keys ~ N(0, 2^2) (scores of standard deviation 2 at scale d^-1/2, so the
softmax is neither flat nor one-hot), values ~ N(0,1). gen_attn_decode draws them on
the host (numpy) for the sizes an fp64 check covers; gen_attn_decode_device draws the
full-size caches on the GPU with torch's seeded generator.

Layout of every array: token-major and packed, [T_total, H, d]; gates
[T_total, H, d_k] and [T_total, H]; states [n_seqs, H, d_k, d_v] row-major
(row = key channel). Batched workloads are packed sequences of equal length.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple          # lengths of the packed sequences
    H: int
    dk: int
    dv: int
    chunk: int
    io: str                 # "f32" or "bf16": dtype of q, k, v and o
    gates: str              # "weak", "main" (or "strong" in tests)
    h0: str                 # "zero" or "normal"
    seed: int
    gate: str = "channel"   # decays given to the library: "channel", "head", "none", "preact"
                            # (formed in the kernels from gen_preact's pre-activations) or
                            # "preact_qk" (q and k from gen_qk_preact too)

    @property
    def T_total(self) -> int:
        return int(sum(self.seqlens))

    @property
    def n_seqs(self) -> int:
        return len(self.seqlens)

    @property
    def scale(self) -> float:
        return float(self.dk) ** -0.5

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)


WORKLOADS = {
    "tiny": Workload("tiny", (256,), 2, 64, 64, 64, "f32", "weak", "zero", 1000),
    "prefill": Workload("prefill", (4096,), 16, 128, 128, 64, "bf16", "main", "normal", 1001),
    "batched": Workload("batched", (8192,) * 8, 32, 128, 128, 64, "bf16", "weak", "zero", 1002),
    "varlen": Workload("varlen", (32768, 16384, 12288, 4096), 32, 128, 128, 128, "bf16", "weak",
                       "normal", 1003),
    # the batched workload with one decay per token and head (Gated DeltaNet) and with none (DeltaNet)
    "batched_gdn": Workload("batched_gdn", (8192,) * 8, 32, 128, 128, 64, "bf16", "weak", "zero", 1002, "head"),
    "batched_deltanet": Workload("batched_deltanet", (8192,) * 8, 32, 128, 128, 64, "bf16", "weak", "zero", 1002,
                                 "none"),
    # the batched workload with its gates formed in the kernels from pre-activations (gen_preact)
    "batched_preact": Workload("batched_preact", (8192,) * 8, 32, 128, 128, 64, "bf16", "weak", "zero", 1002,
                               "preact"),
    # 16 packed sequences of mixed lengths (65,536 tokens, 512 (sequence, head) pairs: the fused pass)
    "varlen_many": Workload("varlen_many", (8192, 2048, 6144, 4096, 4096, 1000, 7192, 4096, 3000, 5192, 4096, 4096,
                                            2048, 6144, 1, 4095), 32, 128, 128, 64, "bf16", "weak", "normal", 1008),
    # ... and q, k given before silu and per-row L2 normalisation too (gen_qk_preact)
    "batched_preact_qk": Workload("batched_preact_qk", (8192,) * 8, 32, 128, 128, 64, "bf16", "weak", "zero",
                                  1002, "preact_qk"),
}

# Decode: N sequences x H heads, one token per step.
DECODE = dict(name="decode", N=256, H=32, dk=128, dv=128, io="bf16", gates="main", steps=1024,
              seed=1004)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); returns fp32 values
    that are exactly representable in bfloat16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    return np.logaddexp(0.0, x)


def _unit_gaussian(rng, shape, d):
    x = rng.standard_normal(shape + (d,), dtype=np.float32).astype(np.float64)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x.astype(np.float32)


def _gates(rng, family, shape, dk):
    if family == "weak":
        la = -0.1 * softplus(rng.standard_normal(shape + (dk,), dtype=np.float32).astype(np.float64))
    elif family == "main":
        la = -softplus(rng.standard_normal(shape + (dk,), dtype=np.float32).astype(np.float64) - 2.0)
    elif family == "strong":
        la = -1.3 * softplus(rng.standard_normal(shape + (dk,), dtype=np.float32).astype(np.float64) + 1.0)
    elif family in ("sum500", "sum2000"):
        # log alpha = -(S / 64) U(0.5, 1.5): chunk sums of about -S per channel over 64 tokens
        S = 500.0 if family == "sum500" else 2000.0
        la = -(S / 64.0) * rng.uniform(0.5, 1.5, shape + (dk,))
    else:
        raise ValueError(family)
    beta = sigmoid(rng.standard_normal(shape, dtype=np.float32).astype(np.float64))
    return la.astype(np.float32), beta.astype(np.float32)


def _io(x, io):
    return round_bf16(x) if io == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def gen_sequences(seqlens, H, dk, dv, io, gates, h0, seed):
    """Draw one packed batch of sequences. Returns a dict of fp32 numpy arrays
    (q, k, v rounded to bf16 when io == "bf16"), the int32 cu_seqlens, and h0
    (None when it is zero)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q_l, k_l, v_l, la_l, b_l = [], [], [], [], []
    for L in seqlens:  # draw sequence by sequence to bound temporary memory
        q_l.append(_io(_unit_gaussian(rng, (L, H), dk), io))
        k_l.append(_io(_unit_gaussian(rng, (L, H), dk), io))
        v_l.append(_io(rng.standard_normal((L, H, dv), dtype=np.float32), io))
        la, b = _gates(rng, gates, (L, H), dk)
        la_l.append(la)
        b_l.append(b)
    out = dict(
        q=np.concatenate(q_l), k=np.concatenate(k_l), v=np.concatenate(v_l),
        log_alpha=np.concatenate(la_l), beta=np.concatenate(b_l),
        cu_seqlens=np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32),
    )
    if h0 == "normal":
        out["h0"] = (0.02 * rng.standard_normal((len(seqlens), H, dk, dv), dtype=np.float32)
                     ).astype(np.float32)
    else:
        out["h0"] = None
    return out


def gen_key_repeats(seqlens, H, dk, dv, io, kind, seed, gates="weak"):
    """A batch of gen_sequences with keys that collide inside a chunk and beta = 1 (the
    regime where the delta rule overwrites what a key stored). kind "repeat": every
    token's key is one of three fixed unit vectors of its head, drawn at random per
    token (exact repeats, also after rounding); kind "near": every key is its head's
    fixed unit vector plus a random direction of length 0.1, normalised (cosine
    about 0.99 between any two keys of a head)."""
    x = gen_sequences(seqlens, H, dk, dv, io, gates, "normal", seed)
    rng = np.random.Generator(np.random.PCG64([seed, 0xC3]))
    T = int(sum(seqlens))
    if kind == "repeat":
        pool = _unit_gaussian(rng, (3, H), dk)                   # [3, H, dk]
        pick = rng.integers(0, 3, size=(T, H))
        k = pool[pick, np.arange(H)[None, :]]
    elif kind == "near":
        base = _unit_gaussian(rng, (H,), dk).astype(np.float64)  # [H, dk]
        u = _unit_gaussian(rng, (T, H), dk).astype(np.float64)
        k = base[None] + 0.1 * u
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    else:
        raise ValueError(kind)
    x["k"] = _io(k.astype(np.float32), io)
    x["beta"] = np.ones((T, H), dtype=np.float32)
    return x


def gen_preact(T_total, H, dk, io, seed):
    """Gate pre-activations for the kernels that form the gates themselves: a ~ N(0,1)
    [T, H, dk] (rounded to the io dtype), A_log = log U(1, 16) per head, dt_bias =
    softplus^-1(dt) per (head, channel) with dt log-uniform in [1e-3, 1e-2], b ~ N(0,1)
    [T, H]. The decays these give average about -0.26 per token at the largest rate
    scale (chunk sums near -17), inside the chunked form's limit."""
    rng = np.random.Generator(np.random.PCG64([seed, 0xA7]))
    a = _io(rng.standard_normal((T_total, H, dk), dtype=np.float32), io)
    A_log = np.log(rng.uniform(1.0, 16.0, H)).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-2), (H, dk)))
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    b = rng.standard_normal((T_total, H), dtype=np.float32)
    return dict(a=a, A_log=A_log, dt_bias=dt_bias, b=b)


def gen_preact_strong(T_total, H, dk, io, seed):
    """Gate pre-activations whose decays sum to about -2000 per 64-token chunk: A_log = log 16
    for every head and a ~ N(8, 1), so that with gen_preact's dt_bias (about -5 to -7)
    log alpha = -16 softplus(a + dt_bias) is about -30 per token."""
    p = gen_preact(T_total, H, dk, io, seed)
    rng = np.random.Generator(np.random.PCG64([seed, 0xA9]))
    p["a"] = _io(rng.standard_normal((T_total, H, dk), dtype=np.float32) + 8.0, io)
    p["A_log"] = np.full(H, np.log(16.0), dtype=np.float32)
    return p


def gen_qk_preact(T_total, H, dk, io, seed):
    """q and k before their activation and normalisation: N(0,1) [T, H, dk] each, rounded
    to the io dtype."""
    rng = np.random.Generator(np.random.PCG64([seed, 0xB1]))
    return dict(q=_io(rng.standard_normal((T_total, H, dk), dtype=np.float32), io),
                k=_io(rng.standard_normal((T_total, H, dk), dtype=np.float32), io))


ATTN_WORKLOADS = {
    # name: (B, H, H_kv, T_max, d, io, seed)
    "attn_batched": (256, 32, 32, 4096, 128, "bf16", 1005),
    "attn_1m": (1, 32, 32, 1 << 20, 128, "bf16", 1006),
}


def gen_attn_decode(B, H, H_kv, T_max, d, io, seed):
    """q [B, H, d] ~ N(0,1), k_cache ~ N(0, 2^2) and v_cache ~ N(0,1) [B, H_kv, T_max, d],
    rounded to the io dtype (numpy; fp32 arrays holding bf16 values for "bf16")."""
    rng = np.random.Generator(np.random.PCG64([seed, 0xA1]))
    q = _io(rng.standard_normal((B, H, d), dtype=np.float32), io)
    k = _io(2.0 * rng.standard_normal((B, H_kv, T_max, d), dtype=np.float32), io)
    v = _io(rng.standard_normal((B, H_kv, T_max, d), dtype=np.float32), io)
    return dict(q=q, k_cache=k, v_cache=v)


def gen_attn_decode_device(B, H, H_kv, T_max, d, dtype, seed, device):
    """The same distributions drawn on the GPU (torch's seeded generator), for caches too
    large to draw on the host: q [B, H, d], k_cache, v_cache [B, H_kv, T_max, d] in dtype."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.randn((B, H, d), generator=g, device=device, dtype=torch.float32).to(dtype)
    k = torch.empty((B, H_kv, T_max, d), device=device, dtype=dtype)
    v = torch.empty((B, H_kv, T_max, d), device=device, dtype=dtype)
    k.normal_(0.0, 2.0, generator=g)
    v.normal_(0.0, 1.0, generator=g)
    return dict(q=q, k_cache=k, v_cache=v)


def gen_grad_outputs(B, T, H, dk, dv, seed):
    """Loss gradients for the backward pass: dout [B, T, H, dv] and dhT [B, H, dk, dv], both
    N(0,1) fp32."""
    rng = np.random.Generator(np.random.PCG64([seed, 0xB2]))
    return dict(dout=rng.standard_normal((B, T, H, dv), dtype=np.float32),
                dhT=rng.standard_normal((B, H, dk, dv), dtype=np.float32))


def gen_decode_step_device(N, H, dk, dv, dtype, seed, step, device):
    """Inputs of decode step `step` drawn on the GPU with torch's seeded generator (seed
    mixed with the step): the decode recipe with "main" gates. q, k [N, H, dk] N(0,1)
    L2-normalised per (sequence, head), v [N, H, dv] N(0,1), all in dtype; log_alpha
    [N, H, dk] = -softplus(N(-2, 1)) and beta [N, H] = sigmoid(N(0, 1)) in fp32. For long
    runs over the full batch, where drawing every step on the host would dominate."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(step))
    rn = lambda *s: torch.randn(s, generator=g, device=device, dtype=torch.float32)  # noqa: E731
    q = torch.nn.functional.normalize(rn(N, H, dk), dim=-1).to(dtype)
    k = torch.nn.functional.normalize(rn(N, H, dk), dim=-1).to(dtype)
    v = rn(N, H, dv).to(dtype)
    la = -torch.nn.functional.softplus(rn(N, H, dk) - 2.0)
    beta = torch.sigmoid(rn(N, H))
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta)


def gen_workload(w: Workload, seed: Optional[int] = None):
    return gen_sequences(w.seqlens, w.H, w.dk, w.dv, w.io, w.gates, w.h0,
                         w.seed if seed is None else seed)


def gen_decode_state(N, H, dk, dv, seed):
    """Initial decode state h0 ~ N(0, 0.02), [N, H, dk, dv] fp32."""
    rng = np.random.Generator(np.random.PCG64([seed, 0xD0]))
    return (0.02 * rng.standard_normal((N, H, dk, dv), dtype=np.float32)).astype(np.float32)


def gen_decode_step(N, H, dk, dv, io, gates, seed, step):
    """Inputs of decode step `step` for N sequences: q, k, v [N, H, d], log_alpha
    [N, H, dk], beta [N, H]. Each step has its own stream (seed, step), so any
    step can be regenerated on its own."""
    rng = np.random.Generator(np.random.PCG64([seed, step]))
    q = _io(_unit_gaussian(rng, (N, H), dk), io)
    k = _io(_unit_gaussian(rng, (N, H), dk), io)
    v = _io(rng.standard_normal((N, H, dv), dtype=np.float32), io)
    la, b = _gates(rng, gates, (N, H), dk)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=b)

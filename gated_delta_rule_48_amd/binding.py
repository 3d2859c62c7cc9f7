"""ctypes binding of libkda (include/kda.h).

Argument marshalling only: shape/dtype checks, output and workspace
allocation through torch (device memory is torch's), and the call into the C
ABI on torch's current HIP stream. Every step of the computation runs in
libkda's HIP kernels; there is no other code path. If libkda.so has not been
built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_CHANNEL, KDA_GATE_HEAD, KDA_GATE_NONE = 0, 1, 2
KDA_PREACT_QK_NORM = 1
STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_WORKSPACE",
          4: "KDA_ERR_HIP"}
EXPORTS = ("kda_abi_version", "kda_status_string", "kda_chunk_fwd_workspace_bytes",
           "kda_chunk_fwd", "kda_chunk_fwd_gated", "kda_chunk_fwd_preact", "kda_recurrent_step",
           "kda_recurrent_step_gated", "kda_recurrent_step_preact", "kda_attn_decode_workspace_bytes",
           "kda_attn_decode", "kda_chunk_bwd_workspace_bytes", "kda_chunk_bwd", "kda_chunk_fwd_noalloc",
           "kda_chunk_bwd_varlen_workspace_bytes", "kda_chunk_bwd_varlen")
ABI_VERSION = 6
NOALLOC_MAX_WORKSPACE = 32 << 20  # KDA_NOALLOC_MAX_WORKSPACE


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {STATUS.get(status, status)}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libkda.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libkda.so is missing at {LIB_PATH}; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = I
    lib.kda_status_string.argtypes = [I]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.kda_chunk_fwd_workspace_bytes.restype = Z
    lib.kda_chunk_fwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, F, P, P, I, P, P, P, Z, P]
    lib.kda_chunk_fwd.restype = I
    lib.kda_chunk_fwd_gated.argtypes = [I] + lib.kda_chunk_fwd.argtypes
    lib.kda_chunk_fwd_gated.restype = I
    lib.kda_chunk_fwd_preact.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, F, P, P, I, P, P, P, Z, P]
    lib.kda_chunk_fwd_preact.restype = I
    lib.kda_recurrent_step.argtypes = [I, I, I, I, I, P, P, P, P, P, F, P, P, P]
    lib.kda_recurrent_step.restype = I
    lib.kda_recurrent_step_gated.argtypes = [I] + lib.kda_recurrent_step.argtypes
    lib.kda_recurrent_step_gated.restype = I
    lib.kda_recurrent_step_preact.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, F, P, P, P]
    lib.kda_recurrent_step_preact.restype = I
    lib.kda_attn_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.kda_attn_decode_workspace_bytes.restype = Z
    lib.kda_attn_decode.argtypes = [I, I, I, I, I, I, P, P, P, P, F, P, P, Z, P]
    lib.kda_attn_decode.restype = I
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.kda_chunk_bwd_workspace_bytes.restype = Z
    lib.kda_chunk_bwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, F, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.kda_chunk_bwd.restype = I
    lib.kda_chunk_bwd_varlen_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.kda_chunk_bwd_varlen_workspace_bytes.restype = Z
    lib.kda_chunk_bwd_varlen.argtypes = [I, I, I, I, I, I, P, P, P, P, P, F, P, P, I, P, P, P, P, P, P, P, P, P, Z, P]
    lib.kda_chunk_bwd_varlen.restype = I
    lib.kda_chunk_fwd_noalloc.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, P, F, P, P, I, P, P, P]
    lib.kda_chunk_fwd_noalloc.restype = I
    if lib.kda_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libkda.so has ABI {lib.kda_abi_version()}, this binding expects {ABI_VERSION}; "
                           "rebuild it")
    _lib = lib
    return lib


def abi_version() -> int:
    return load().kda_abi_version()


def _io_code(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return KDA_BF16
    if dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q, k, v must be bfloat16 or float32, got {dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t, name, dtype, shape, device):
    if t.device.type != "cuda":
        raise ValueError(f"{name} is on {t.device}: libkda's kernels read device memory only")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gate(log_alpha, lead, H, dk, dev) -> int:
    """The decay granularity that log_alpha's shape selects (kda_gate), after checking it:
    [.., H, dk] one decay per key channel, [.., H] one per token and head, None no decay."""
    import torch
    if log_alpha is None:
        return KDA_GATE_NONE
    if log_alpha.dim() == len(lead) + 2:
        _check(log_alpha, "log_alpha", torch.float32, lead + (H, dk), dev)
        return KDA_GATE_CHANNEL
    _check(log_alpha, "log_alpha", torch.float32, lead + (H,), dev)
    return KDA_GATE_HEAD


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def workspace_bytes(B, T, H, dk, dv, chunk, n_seqs, io) -> int:
    return int(load().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, n_seqs, io))


def _chunk_fwd_call(noalloc, q, k, v, log_alpha, beta, scale, h0, cu_seqlens, chunk, output_final_state, o, hT,
                    workspace, stream):
    import torch
    lib = load()
    dev = q.device
    io = _io_code(q.dtype)
    if cu_seqlens is not None:
        if q.dim() != 3:
            raise ValueError("with cu_seqlens, q must be packed [T, H, dk]")
        B, (T, H, dk) = 1, q.shape
        n_seqs = cu_seqlens.numel() - 1
        _check(cu_seqlens, "cu_seqlens", torch.int32, (n_seqs + 1,), dev)
        lead = (T,)
    else:
        if q.dim() != 4:
            raise ValueError("q must be [B, T, H, dk]")
        B, T, H, dk = q.shape
        n_seqs = B
        lead = (B, T)
    dv = v.shape[-1]
    _check(q, "q", q.dtype, lead + (H, dk), dev)
    _check(k, "k", q.dtype, lead + (H, dk), dev)
    _check(v, "v", q.dtype, lead + (H, dv), dev)
    gate = _gate(log_alpha, lead, H, dk, dev)
    _check(beta, "beta", torch.float32, lead + (H,), dev)
    if h0 is not None:
        _check(h0, "h0", torch.float32, (n_seqs, H, dk, dv), dev)
    if o is None:
        o = torch.empty(lead + (H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", q.dtype, lead + (H, dv), dev)
    if output_final_state and hT is None:
        hT = torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=dev)
    if hT is not None:
        _check(hT, "hT", torch.float32, (n_seqs, H, dk, dv), dev)
    if scale is None:
        scale = dk ** -0.5
    ns_arg = n_seqs if cu_seqlens is not None else 0
    if noalloc:
        st = lib.kda_chunk_fwd_noalloc(gate, B, T, H, dk, dv, chunk, io, _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(log_alpha), _ptr(beta), float(scale), _ptr(h0), _ptr(cu_seqlens),
                                       ns_arg, _ptr(o), _ptr(hT), _stream(stream))
        if st != 0:
            raise KdaError(st, "kda_chunk_fwd_noalloc")
        return o, hT
    need = int(lib.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, ns_arg, io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_fwd_gated(gate, B, T, H, dk, dv, chunk, io, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                 _ptr(beta), float(scale), _ptr(h0), _ptr(cu_seqlens), ns_arg, _ptr(o), _ptr(hT),
                                 _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_gated")
    return o, hT


def chunk_fwd(q, k, v, log_alpha, beta, scale: Optional[float] = None, h0=None, cu_seqlens=None,
              chunk: int = 64, output_final_state: bool = True, o=None, hT=None, workspace=None,
              stream=None):
    """Chunked KDA forward (kda_chunk_fwd_gated).

    q, k [B, T, H, dk] (or packed [T, H, dk] with cu_seqlens); v [.., H, dv];
    log_alpha fp32 [.., H, dk] (a decay per key channel), [.., H] (one per token and
    head, Gated DeltaNet) or None (no decay, DeltaNet); beta [.., H] fp32;
    h0 [n_seq, H, dk, dv] fp32 or None;
    cu_seqlens int32 [n_seqs + 1] on the device, or None. Returns (o, hT); hT is
    None when output_final_state is False.
    """
    return _chunk_fwd_call(False, q, k, v, log_alpha, beta, scale, h0, cu_seqlens, chunk, output_final_state, o,
                           hT, workspace, stream)


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, scale: Optional[float] = None, h0=None, cu_seqlens=None,
                      chunk: int = 64, output_final_state: bool = True, o=None, hT=None, stream=None):
    """chunk_fwd through kda_chunk_fwd_noalloc: the library's own fixed workspace (at most
    NOALLOC_MAX_WORKSPACE bytes; calls overlapping on one GPU race). Pass o (and hT) to
    allocate nothing; otherwise they are allocated here as in chunk_fwd."""
    return _chunk_fwd_call(True, q, k, v, log_alpha, beta, scale, h0, cu_seqlens, chunk, output_final_state, o,
                           hT, None, stream)


def recurrent_step(q, k, v, log_alpha, beta, state, scale: Optional[float] = None, o=None,
                   stream=None):
    """One decode step (kda_recurrent_step_gated): q, k [N, H, dk]; v [N, H, dv];
    log_alpha fp32 [N, H, dk], [N, H] or None (as in chunk_fwd); beta [N, H] fp32;
    state [N, H, dk, dv] fp32, updated in place. Returns o [N, H, dv]."""
    import torch
    lib = load()
    dev = q.device
    io = _io_code(q.dtype)
    if q.dim() != 3:
        raise ValueError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _check(q, "q", q.dtype, (N, H, dk), dev)
    _check(k, "k", q.dtype, (N, H, dk), dev)
    _check(v, "v", q.dtype, (N, H, dv), dev)
    gate = _gate(log_alpha, (N,), H, dk, dev)
    _check(beta, "beta", torch.float32, (N, H), dev)
    _check(state, "state", torch.float32, (N, H, dk, dv), dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", q.dtype, (N, H, dv), dev)
    if scale is None:
        scale = dk ** -0.5
    st = lib.kda_recurrent_step_gated(gate, N, H, dk, dv, io, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                      _ptr(beta), float(scale), _ptr(state), _ptr(o), _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_recurrent_step_gated")
    return o


def chunk_fwd_preact(q, k, v, a, A_log, dt_bias, b, scale: Optional[float] = None, h0=None, cu_seqlens=None,
                     chunk: int = 64, output_final_state: bool = True, o=None, hT=None, workspace=None,
                     stream=None, qk_norm: bool = False):
    """Chunked forward with the gates formed in the kernels (kda_chunk_fwd_preact):
    log_alpha = -exp(A_log[h]) softplus(a + dt_bias[h]), beta = sigmoid(b); with qk_norm,
    q and k are given before silu and per-row L2 normalisation, which the kernels apply.

    a [.., H, dk] in q's dtype; A_log [H] fp32; dt_bias [H, dk] fp32; b [.., H] fp32;
    the rest as in chunk_fwd. Returns (o, hT)."""
    import torch
    lib = load()
    dev = q.device
    io = _io_code(q.dtype)
    if cu_seqlens is not None:
        if q.dim() != 3:
            raise ValueError("with cu_seqlens, q must be packed [T, H, dk]")
        B, (T, H, dk) = 1, q.shape
        n_seqs = cu_seqlens.numel() - 1
        _check(cu_seqlens, "cu_seqlens", torch.int32, (n_seqs + 1,), dev)
        lead = (T,)
    else:
        if q.dim() != 4:
            raise ValueError("q must be [B, T, H, dk]")
        B, T, H, dk = q.shape
        n_seqs = B
        lead = (B, T)
    dv = v.shape[-1]
    _check(q, "q", q.dtype, lead + (H, dk), dev)
    _check(k, "k", q.dtype, lead + (H, dk), dev)
    _check(v, "v", q.dtype, lead + (H, dv), dev)
    _check(a, "a", q.dtype, lead + (H, dk), dev)
    _check(A_log, "A_log", torch.float32, (H,), dev)
    _check(dt_bias, "dt_bias", torch.float32, (H, dk), dev)
    _check(b, "b", torch.float32, lead + (H,), dev)
    if h0 is not None:
        _check(h0, "h0", torch.float32, (n_seqs, H, dk, dv), dev)
    if o is None:
        o = torch.empty(lead + (H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", q.dtype, lead + (H, dv), dev)
    if output_final_state and hT is None:
        hT = torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=dev)
    if hT is not None:
        _check(hT, "hT", torch.float32, (n_seqs, H, dk, dv), dev)
    need = int(lib.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk,
                                                 n_seqs if cu_seqlens is not None else 0, io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scale is None:
        scale = dk ** -0.5
    st = lib.kda_chunk_fwd_preact(KDA_PREACT_QK_NORM if qk_norm else 0, B, T, H, dk, dv, chunk, io, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(A_log),
                                  _ptr(dt_bias), _ptr(b), float(scale), _ptr(h0), _ptr(cu_seqlens),
                                  n_seqs if cu_seqlens is not None else 0, _ptr(o), _ptr(hT),
                                  _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_preact")
    return o, hT


def recurrent_step_preact(q, k, v, a, A_log, dt_bias, b, state, scale: Optional[float] = None, o=None,
                          stream=None, qk_norm: bool = False):
    """One decode step with the gates formed in the kernel (kda_recurrent_step_preact):
    a [N, H, dk] in q's dtype; A_log [H]; dt_bias [H, dk]; b [N, H] fp32; qk_norm as in
    chunk_fwd_preact; state updated in place. Returns o [N, H, dv]."""
    import torch
    lib = load()
    dev = q.device
    io = _io_code(q.dtype)
    if q.dim() != 3:
        raise ValueError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _check(q, "q", q.dtype, (N, H, dk), dev)
    _check(k, "k", q.dtype, (N, H, dk), dev)
    _check(v, "v", q.dtype, (N, H, dv), dev)
    _check(a, "a", q.dtype, (N, H, dk), dev)
    _check(A_log, "A_log", torch.float32, (H,), dev)
    _check(dt_bias, "dt_bias", torch.float32, (H, dk), dev)
    _check(b, "b", torch.float32, (N, H), dev)
    _check(state, "state", torch.float32, (N, H, dk, dv), dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    _check(o, "o", q.dtype, (N, H, dv), dev)
    if scale is None:
        scale = dk ** -0.5
    st = lib.kda_recurrent_step_preact(KDA_PREACT_QK_NORM if qk_norm else 0, N, H, dk, dv, io, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(A_log),
                                       _ptr(dt_bias), _ptr(b), float(scale), _ptr(state), _ptr(o),
                                       _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_recurrent_step_preact")
    return o


def attn_decode_workspace_bytes(B, H, H_kv, d, T_max, io) -> int:
    return int(load().kda_attn_decode_workspace_bytes(B, H, H_kv, d, T_max, io))


def attn_decode(q, k_cache, v_cache, seq_lens=None, scale: Optional[float] = None, o=None, workspace=None,
                stream=None):
    """Softmax attention of one new token per sequence over a KV cache (kda_attn_decode):
    q [B, H, d]; k_cache, v_cache [B, H_kv, T_max, d] in q's dtype (the new token's key and
    value already in row seq_lens[b] - 1); seq_lens [B] int32 or None (all T_max rows).
    Query head h reads cached head h // (H // H_kv). Returns o [B, H, d]."""
    import torch
    lib = load()
    dev = q.device
    io = _io_code(q.dtype)
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, H, d] and the caches [B, H_kv, T_max, d]")
    B, H, d = q.shape
    H_kv, T_max = k_cache.shape[1], k_cache.shape[2]
    _check(q, "q", q.dtype, (B, H, d), dev)
    _check(k_cache, "k_cache", q.dtype, (B, H_kv, T_max, d), dev)
    _check(v_cache, "v_cache", q.dtype, (B, H_kv, T_max, d), dev)
    if seq_lens is not None:
        _check(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if o is None:
        o = torch.empty((B, H, d), dtype=q.dtype, device=dev)
    _check(o, "o", q.dtype, (B, H, d), dev)
    need = int(lib.kda_attn_decode_workspace_bytes(B, H, H_kv, d, T_max, io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scale is None:
        scale = d ** -0.5
    st = lib.kda_attn_decode(B, H, H_kv, d, T_max, io, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                             float(scale), _ptr(o), _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_attn_decode")
    return o


def chunk_bwd_workspace_bytes(B, T, H, dk, dv, chunk=64, io=KDA_F32) -> int:
    return int(load().kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, chunk, io))


def chunk_bwd_varlen_workspace_bytes(T, H, dk, dv, n_seqs, chunk=64, io=KDA_BF16) -> int:
    return int(load().kda_chunk_bwd_varlen_workspace_bytes(T, H, dk, dv, chunk, n_seqs, io))


def chunk_bwd(q, k, v, log_alpha, beta, dout, scale: Optional[float] = None, h0=None, dhT=None,
              chunk: int = 64, workspace=None, stream=None, cu_seqlens=None):
    """Backward pass of chunk_fwd (kda_chunk_bwd) for equal-length sequences: q, k
    [B, T, H, dk]; v, dout [B, T, H, dv] (fp32 or bf16); log_alpha [B, T, H, dk]; beta
    [B, T, H]; h0, dhT [B, H, dk, dv] or None (fp32). Returns (dq, dk, dv in q's dtype,
    dlog_alpha, dbeta, dh0 in fp32), dh0 None when h0 is None.
    With cu_seqlens (int32 [n_seqs + 1], on the device), packed sequences
    (kda_chunk_bwd_varlen, bf16 with dk = dv = 128): q, k [T, H, dk], v, dout [T, H, dv],
    log_alpha [T, H, dk], beta [T, H], h0 and dhT [n_seqs, H, dk, dv]."""
    import torch
    lib = load()
    dev = q.device
    io = _io_code(q.dtype)
    if cu_seqlens is not None:
        return _chunk_bwd_varlen(lib, q, k, v, log_alpha, beta, dout, scale, h0, dhT, chunk, workspace, stream,
                                 cu_seqlens, io)
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    f32 = torch.float32
    _check(q, "q", q.dtype, (B, T, H, dk), dev)
    _check(k, "k", q.dtype, (B, T, H, dk), dev)
    _check(v, "v", q.dtype, (B, T, H, dv), dev)
    _check(log_alpha, "log_alpha", f32, (B, T, H, dk), dev)
    _check(beta, "beta", f32, (B, T, H), dev)
    _check(dout, "dout", q.dtype, (B, T, H, dv), dev)
    for t, n in ((h0, "h0"), (dhT, "dhT")):
        if t is not None:
            _check(t, n, f32, (B, H, dk, dv), dev)
    dq, dk_ = (torch.empty((B, T, H, dk), dtype=q.dtype, device=dev) for _ in range(2))
    dlog_alpha = torch.empty((B, T, H, dk), dtype=f32, device=dev)
    dv_ = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    dbeta = torch.empty((B, T, H), dtype=f32, device=dev)
    dh0 = torch.empty((B, H, dk, dv), dtype=f32, device=dev) if h0 is not None else None
    need = int(lib.kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, chunk, io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scale is None:
        scale = dk ** -0.5
    st = lib.kda_chunk_bwd(B, T, H, dk, dv, chunk, io, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                           float(scale), _ptr(h0), _ptr(dout), _ptr(dhT), _ptr(dq), _ptr(dk_), _ptr(dv_),
                           _ptr(dlog_alpha), _ptr(dbeta), _ptr(dh0), _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_bwd")
    return dq, dk_, dv_, dlog_alpha, dbeta, dh0


def _chunk_bwd_varlen(lib, q, k, v, log_alpha, beta, dout, scale, h0, dhT, chunk, workspace, stream, cu_seqlens, io):
    import torch
    dev = q.device
    if q.dim() != 3:
        raise ValueError("with cu_seqlens q must be [T, H, dk]")
    T, H, dk = q.shape
    dv = v.shape[-1]
    f32 = torch.float32
    _check(cu_seqlens, "cu_seqlens", torch.int32, (cu_seqlens.numel(),), dev)
    n = cu_seqlens.numel() - 1
    _check(q, "q", q.dtype, (T, H, dk), dev)
    _check(k, "k", q.dtype, (T, H, dk), dev)
    _check(v, "v", q.dtype, (T, H, dv), dev)
    _check(log_alpha, "log_alpha", f32, (T, H, dk), dev)
    _check(beta, "beta", f32, (T, H), dev)
    _check(dout, "dout", q.dtype, (T, H, dv), dev)
    for t, nm in ((h0, "h0"), (dhT, "dhT")):
        if t is not None:
            _check(t, nm, f32, (n, H, dk, dv), dev)
    dq, dk_ = (torch.empty((T, H, dk), dtype=q.dtype, device=dev) for _ in range(2))
    dlog_alpha = torch.empty((T, H, dk), dtype=f32, device=dev)
    dv_ = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    dbeta = torch.empty((T, H), dtype=f32, device=dev)
    dh0 = torch.empty((n, H, dk, dv), dtype=f32, device=dev) if h0 is not None else None
    need = int(lib.kda_chunk_bwd_varlen_workspace_bytes(T, H, dk, dv, chunk, n, io))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if scale is None:
        scale = dk ** -0.5
    st = lib.kda_chunk_bwd_varlen(T, H, dk, dv, chunk, io, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                  float(scale), _ptr(h0), _ptr(cu_seqlens), n, _ptr(dout), _ptr(dhT), _ptr(dq),
                                  _ptr(dk_), _ptr(dv_), _ptr(dlog_alpha), _ptr(dbeta), _ptr(dh0), _ptr(workspace),
                                  ws_bytes, _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_bwd_varlen")
    return dq, dk_, dv_, dlog_alpha, dbeta, dh0

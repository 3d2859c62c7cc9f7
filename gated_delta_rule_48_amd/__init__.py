"""libkda: the KDA (Kimi Delta Attention) gated delta rule on AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI
(include/kda.h, built into libkda.so in this directory); this package is the
thin Python binding over it. It also holds the softmax-attention decode step
over a KV cache that the KDA decode step is compared with.
"""
from .binding import (KdaError, abi_version, attn_decode, attn_decode_workspace_bytes,  # noqa: F401
                      chunk_bwd, chunk_bwd_workspace_bytes, chunk_bwd_varlen_workspace_bytes, chunk_fwd, chunk_fwd_noalloc, chunk_fwd_preact, load, recurrent_step, recurrent_step_preact,
                      workspace_bytes, LIB_PATH, EXPORTS, KDA_F32, KDA_BF16, KDA_GATE_CHANNEL,
                      KDA_GATE_HEAD, KDA_GATE_NONE)

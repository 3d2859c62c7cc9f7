"""libkda: the KDA (Kimi Delta Attention) gated delta rule on AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI
(include/kda.h, built into libkda.so in this directory); this package is the
thin Python binding over it.
"""
from .binding import (KdaError, abi_version, chunk_fwd, chunk_fwd_preact, load, recurrent_step,  # noqa: F401
                      recurrent_step_preact,
                      workspace_bytes, LIB_PATH, EXPORTS, KDA_F32, KDA_BF16, KDA_GATE_CHANNEL,
                      KDA_GATE_HEAD, KDA_GATE_NONE)

"""Plain fp64 CPU oracle of the KDA gated delta rule (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The GPU library never calls it and shares no code with it.
"""
from .oracle import (attn_decode_reference, build, gate_prologue, kda_backward_reference,  # noqa: F401
                     kda_reference, library_path, qk_prologue)

"""Compile-time resource checks of the gfx950 kernels (no GPU needed).

The kernels keep their working set in registers and LDS. A kernel that spills
VGPRs or places an array in scratch (private memory) still computes the right
values, but every scratch access is a memory round trip, and a scratch reload in
the fused pass waits, in order, behind the outstanding prefetch loads. The fused
pass also relies on two waves per SIMD (eight waves per workgroup). These checks
read the compiler's own resource report for each kernel.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_48_amd", "csrc")
SOURCES = ["kda_fused.hip", "kda_prep.hip", "kda_state.hip", "kda_segment.hip", "kda_decode.hip", "kda_attn.hip",
           "kda_bwd.hip", "kda_bwd_bf16.hip", "kda_bwd_tok.hip"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _report(src, outdir):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-c", os.path.join(CSRC, src),
           "-o", os.path.join(outdir, src + ".o"), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: +(.+?) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        key, _, val = m.group(1).partition(":")
        if key == "Function Name":
            cur = val.strip()
            kernels[cur] = {}
        elif cur is not None:
            kernels[cur][key.strip()] = val.strip()
    return kernels


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d, ThreadPoolExecutor(len(SOURCES)) as ex:
        reports = list(ex.map(lambda s: _report(s, d), SOURCES))
    out = {}
    for r in reports:
        out.update(r)
    return out


def test_every_kernel_is_reported(resources):
    names = " ".join(resources)
    for k in ("kda_fused_kernel", "kda_prep_kernel", "kda_state_kernel", "kda_segment_chain_kernel", "kda_seg_plan_kernel",
              "kda_decode_kernel",
              "kda_chunk_offsets_kernel", "kda_attn_decode_kernel", "kda_attn_combine_kernel",
              "kda_bwd_chunk_fwd_kernel", "kda_bwd_states_kernel", "kda_bwd_state_grads_kernel",
              "kda_bwd_chunk_grads_kernel", "kda_bwd_rev_kernel", "kda_bwd_chunk_kernel", "kda_bwd_tok_kernel",
              "kda_bwd_tok_detect_kernel"):
        assert k in names, k


def _strong_fused(name):
    """The strong-decay instances of the fused kernel (kda_fused_kernel<G, 1>): they run only
    for (sequence, head) pairs with a chunk of strong decay, and their per-pair Gram work
    spills; the usual instance (mode 0) and the two launches with segments (modes 3 and 4,
    mode 3 holding the usual and the segment-map bodies) must not."""
    return "kda_fused_kernel" in name and "ELi1EEEv" in name


def test_no_scratch_and_no_spills(resources):
    for name, r in resources.items():
        if _strong_fused(name):
            continue
        assert r["ScratchSize [bytes/lane]"] == "0", (name, r)
        assert r["Dynamic Stack"] == "False", (name, r)
        if "kda_bwd_chunk_fwd" in name or "kda_bwd_chunk_grads" in name:
            # the direct backward's chunk-local kernels run one workgroup per CU (their LDS), so
            # the compiler may park a value in an accumulation register: no memory is involved
            continue
        assert r["VGPRs Spill"] == "0", (name, r)


def test_fused_kernel_runs_two_waves_per_simd(resources):
    fused = {n: r for n, r in resources.items() if "kda_fused_kernel" in n}
    # the usual instance and the two launches with segments: per channel, per head, none, from
    # pre-activations (with q, k normalised or not); the strong-decay instances of all but "none"
    assert sum(not _strong_fused(n) for n in fused) == 15 and sum(_strong_fused(n) for n in fused) == 4
    for n, r in fused.items():
        assert int(r["Occupancy [waves/SIMD]"]) >= 2, (n, r)
        assert int(r["VGPRs"]) <= 256, (n, r)
        if not _strong_fused(n):
            assert r["VGPRs Spill"] == "0", (n, r)


def test_attn_decode_keeps_loads_in_flight(resources):
    # a streaming kernel: at least three waves per SIMD for the instances of 1, 2 and 4 query
    # heads per cached head (2 dtypes x 2 head dimensions), so that enough cache rows are
    # requested at once; groups of 8 hold 64 query values and 64 sums per lane, at least two
    attn = {n: r for n, r in resources.items() if "kda_attn_decode_kernel" in n}
    assert len(attn) == 16
    for n, r in attn.items():
        assert int(r["Occupancy [waves/SIMD]"]) >= (2 if "ELi8E" in n else 3), (n, r)

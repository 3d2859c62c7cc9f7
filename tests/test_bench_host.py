"""Host-side checks of bench.py (no GPU needed).

bench.py reports a stored HBM-traffic figure only while the sources of the
measured kernels are byte-identical to when the counters were taken; the digest
must therefore cover exactly the files each pass is compiled from. The dispatch
rule bench.py uses to name the pass must agree with the library's.
"""
import importlib.util
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_48_amd", "csrc")


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _local_includes(name, seen=None):
    """The in-tree files `name` includes, transitively, itself included."""
    seen = set() if seen is None else seen
    if name in seen:
        return seen
    seen.add(name)
    for inc in re.findall(r'#include\s+"([^"]+)"', open(os.path.join(CSRC, name)).read()):
        _local_includes(inc, seen)
    return seen


def test_digest_covers_the_compiled_sources():
    bench = _bench()
    fused = _local_includes("kda_fused.hip")
    assert set(bench.PATHS["fused"]["sources"]) == fused
    assert set(bench.PATHS["segmented"]["sources"]) == fused | _local_includes("kda_segment.hip")
    split = _local_includes("kda_prep.hip") | _local_includes("kda_state.hip")
    assert set(bench.PATHS["split"]["sources"]) == split


def test_pass_rule_matches_the_library():
    # the library's rule, read from its source and its workspace sizes: bf16 and d_k = d_v = 128
    # take the fused pass (any chunk size asked), with segments below 256 (sequence, head)
    # pairs when a sequence may have 8 chunks or more
    src = open(os.path.join(CSRC, "kda_api.hip")).read()
    assert "kFusedMinPairs = 256" in src
    bench = _bench()
    assert bench.prefill_path(8, 8192, 32, 128, 128, 64, False, True) == "fused"
    assert bench.prefill_path(1, 4096, 16, 128, 128, 64, False, True) == "segmented"    # 16 pairs
    assert bench.prefill_path(1, 65536, 32, 128, 128, 128, True, True, 4) == "segmented"  # varlen, 128 pairs
    assert bench.prefill_path(1, 65536, 32, 128, 128, 64, True, True, 16) == "fused"     # varlen, 512 pairs
    assert bench.prefill_path(1, 200, 4, 128, 128, 64, False, True) == "fused"          # one segment: no maps
    assert bench.prefill_path(8, 8192, 32, 128, 128, 64, False, False) == "split"       # fp32
    assert bench.prefill_path(8, 8192, 32, 64, 64, 64, False, True) == "split"          # d = 64
    # the workspace says the same: 256 bytes of discard slot and a flag byte per unit on the
    # fused pass (two launches of 256 // H units per head below 256 pairs), with segments
    # 192 KB per slot (entering state and map; 15 slots per head for 1 x 4096 tokens x 16
    # heads), per chunk on the split pass
    import gated_delta_rule_48_amd as kda
    ws = lambda *a: kda.workspace_bytes(*a)  # noqa: E731
    assert ws(8, 8192, 32, 128, 128, 64, 0, kda.KDA_BF16) == 512
    assert ws(1, 200, 4, 128, 128, 64, 0, kda.KDA_BF16) == 256 + 2 * 64 * 4  # planned, no slot
    assert ws(1, 4096, 16, 128, 128, 64, 0, kda.KDA_BF16) > 15 * 16 * 3 * 65536


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_algorithmic_flops_of_the_batched_workload():
    # per chunk of 64 rows and head at d = 128: 3 C^2 dk + 2 C^2 dv + 3 C dk dv multiply-adds
    bench = _bench()
    macs = 3 * 64 * 64 * 128 + 2 * 64 * 64 * 128 + 3 * 64 * 128 * 128
    assert macs == 5_767_168
    assert bench.prefill_algorithmic_flops((8192,) * 8, 32, 128, 128, 64) == 2 * macs * 128 * 8 * 32
    # a ragged sequence counts its last partial chunk whole
    assert bench.prefill_algorithmic_flops((65, 1), 1, 128, 128, 64) == 2 * macs * 3


def test_stored_counters_follow_the_sources(tmp_path):
    bench = _bench()
    info = bench.PATHS["segmented"]
    (tmp_path / "profiles").mkdir()
    f = tmp_path / "profiles" / info["counters"]
    digest = bench.sources_digest(info["sources"])
    f.write_text(f"traffic_bytes_per_launch[varlen]: 123456\nmfma_busy_frac[varlen]: 0.25\n"
                 f"sources_sha256: {digest}\n")
    bench.ROOT = str(tmp_path)
    assert bench.stored_traffic("segmented", "varlen") == 123456
    assert bench.stored_counter("segmented", "varlen", "mfma_busy_frac") == 0.25
    assert bench.stored_traffic("segmented", "prefill") is None   # no line for it
    f.write_text(f"traffic_bytes_per_launch[varlen]: 123456\nsources_sha256: {'0' * 64}\n")
    assert bench.stored_traffic("segmented", "varlen") is None    # sources changed since

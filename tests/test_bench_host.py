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
    split = _local_includes("kda_prep.hip") | _local_includes("kda_state.hip")
    assert set(bench.PATHS["split"]["sources"]) == split


def test_pass_rule_matches_the_library():
    # the library's rule, read from its source: varlen off, chunk 64, bf16, d_k = d_v = 128, B*H >= 256
    src = open(os.path.join(CSRC, "kda_api.hip")).read()
    assert "kFusedMinPairs = 256" in src
    bench = _bench()
    assert bench.prefill_path(8, 8192, 32, 128, 128, 64, False, True) == "fused"
    assert bench.prefill_path(1, 4096, 16, 128, 128, 64, False, True) == "split"      # 16 pairs
    assert bench.prefill_path(1, 65536, 32, 128, 128, 128, True, True) == "split"     # varlen, chunk 128
    assert bench.prefill_path(1, 65536, 32, 128, 128, 64, True, True, 4) == "split"   # varlen, 128 pairs
    assert bench.prefill_path(1, 65536, 32, 128, 128, 64, True, True, 16) == "fused"  # varlen, 512 pairs
    assert bench.prefill_path(8, 8192, 32, 128, 128, 64, False, False) == "split"     # fp32
    assert bench.prefill_path(8, 8192, 32, 64, 64, 64, False, True) == "split"        # d = 64


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr

"""bench.py's command line on the CPU: more than one GPU is refused with a
message before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr


def test_bench_names_the_kernels_the_library_defaults_run():
    """bench.py labels its roofline with the kernel the default exchange runs;
    its thresholds must be the library's (csrc/halo_api.hip)."""
    import re
    from pathlib import Path
    import bench
    src = (Path(__file__).resolve().parents[1] / "domain_decomposition_halo_fusedpackx_amd" /
           "csrc" / "halo_api.hip").read_text()

    def const(name):
        m = re.search(rf"constexpr \w+ {name} = ([^;]+);", src)
        assert m, name
        return eval(m.group(1), {})  # "1 << 20" and the like

    assert const("kTransposedCoordMinEntries") == bench.TRANSPOSED_X_MIN_ENTRIES
    assert const("kTransposedForceMinEntries") == bench.TRANSPOSED_F_MIN_ENTRIES
    assert const("kTransposedForceMaxPulses") == bench.TRANSPOSED_F_MAX_PULSES


def test_traffic_counters_follow_the_compiled_code():
    """The measured HBM bytes in profiles/ are reported only while the kernel
    code they were taken on is unchanged: the hash covers the exchange
    kernels' sources and the build script that holds their compile flags
    (a flag such as the kernel-argument preloading changes the code too)."""
    import bench
    from domain_decomposition_halo_fusedpackx_amd import build
    srcs = set(bench.KERNEL_SOURCES)
    pkg = "domain_decomposition_halo_fusedpackx_amd"
    assert {f"{pkg}/csrc/exchange_kernels.hpp", f"{pkg}/csrc/sync.hpp", f"{pkg}/build.py"} <= srcs
    assert "-amdgpu-kernarg-preload-count=16" in build.HIP_FLAGS
    assert bench.read_traffic("no_such_workload", "pull_f", bench.kernel_source_sha()) is None
    assert bench.read_traffic("grid8x8x8", "pull_f", "0" * 16) is None
    got = bench.read_traffic("grid8x8x8", "pull_f", bench.kernel_source_sha())
    assert got is not None and 0.9 < got / (40 * 2090133) < 1.1

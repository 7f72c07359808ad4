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

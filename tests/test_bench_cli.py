"""bench.py's command-line contract on the CPU: one GPU only, and the option
parser accepts what the measurement docs name (no GPU is touched)."""
import os
import subprocess
import sys

from tests.conftest import ROOT

BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=120,
                          cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line for a run that did not happen


def test_help_lists_the_kernels_and_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--no-cpu-baseline", "--center",
                "--groups", "--kernel", "--copy-calibration", "--preroll-ms"):
        assert opt in r.stdout, opt
    for kernel in ("attention", "pre_attention", "chain"):
        assert kernel in r.stdout, kernel


def test_traffic_is_reported_only_for_the_profiled_kernel_source(tmp_path):
    """roofline.traffic comes from the committed counter passes only while the
    kernel's code (comments aside) is the one they were taken on."""
    import bench
    here = bench.measured_traffic("fsa_attention", "sr720")
    assert here is not None and here > 0         # the committed profile matches the committed kernel
    src = open(bench.KERNEL_SOURCE, "rb").read()
    commented = tmp_path / "commented.hip"
    commented.write_bytes(src + b"\n// a new comment\n\n")
    assert bench.measured_traffic("fsa_attention", "sr720", str(commented)) == here
    edited = tmp_path / "kernel.hip"
    edited.write_bytes(src + b"\nstatic int edited;\n")
    assert bench.measured_traffic("fsa_attention", "sr720", str(edited)) is None
    assert bench.measured_traffic("fsa_attention", "no_such_workload") is None


def test_dpm_clock_line_parsing():
    """The sampler reads the current level of the driver's pp_dpm_sclk table."""
    import bench
    assert bench.parse_dpm_mhz("1: 1989Mhz *") == 1989.0
    assert bench.parse_dpm_mhz("S: 95Mhz *") == 95.0
    assert bench.parse_dpm_mhz("0: 500Mhz") == 500.0
    assert bench.parse_dpm_mhz("no clock here") is None


def test_output_check_bars():
    """The bench line's check: every element within the oracle's element bar
    (1e-2, raised to half a bf16 spacing plus the arithmetic's error only where
    that is larger) and rel-L2 5e-3."""
    import numpy as np

    import bench

    def check(got, ref, spread=0.0):
        m2 = ref * ref + spread ** 2
        sb = np.full(ref.shape[:-1], 20.0)
        nk = np.full(ref.shape[:-1], 4800)
        return bench.output_check(got, ref, m2, sb, nk, 128, "x")["within_bars"]

    ref = np.linspace(-0.9, 0.9, 1024).reshape(8, 128)
    assert check(ref.copy(), ref)
    off = ref.copy()
    off[0, 3] += 1.5e-2                               # |ref| < 2: the 1e-2 bar applies
    assert not check(off, ref)
    big = np.full((8, 128), 4.3)
    assert check(big + 1.5e-2, big)                   # within half a bf16 spacing (2^-6) at 4.3
    assert not check(big + 2.0e-2, big)               # more than half a spacing: off by a rounding step
    noisy = ref + 0.009 * np.sign(ref)                # every element within 1e-2, rel-L2 ~1.7e-2
    assert not check(noisy, ref)

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
                "--groups", "--kernel", "--copy-calibration"):
        assert opt in r.stdout, opt
    for kernel in ("attention", "pre_attention", "chain"):
        assert kernel in r.stdout, kernel


def test_traffic_is_reported_only_for_the_profiled_kernel_source(tmp_path):
    """roofline.traffic comes from the committed counter passes only while the
    kernel source is byte-identical to the one they were taken on."""
    import bench
    here = bench.measured_traffic("fsa_attention", "sr720")
    assert here is not None and here > 0         # the committed profile matches the committed kernel
    edited = tmp_path / "kernel.hip"
    edited.write_bytes(open(bench.KERNEL_SOURCE, "rb").read() + b"\n// edited\n")
    assert bench.measured_traffic("fsa_attention", "sr720", str(edited)) is None
    assert bench.measured_traffic("fsa_attention", "no_such_workload") is None


def test_output_check_bars():
    """The bench line's check: max-abs per element 1e-2, or one bf16 step of the
    reference where that is larger; rel-L2 5e-3."""
    import numpy as np

    import bench
    ref = np.linspace(-0.9, 0.9, 1000)
    assert bench.output_check(ref.copy(), ref, "x")["within_bars"]
    off = ref.copy()
    off[3] += 1.5e-2                                  # |ref| < 2: the 1e-2 bar applies
    assert not bench.output_check(off, ref, "x")["within_bars"]
    big = np.full(1000, 4.3)
    assert bench.output_check(big + 2.0e-2, big, "x")["within_bars"]       # < one bf16 step (2^-5) at 4.3
    assert not bench.output_check(big + 4.0e-2, big, "x")["within_bars"]   # > one bf16 step
    noisy = ref + 0.009 * np.sign(ref)                # every element within 1e-2, rel-L2 ~1.7e-2
    assert not bench.output_check(noisy, ref, "x")["within_bars"]

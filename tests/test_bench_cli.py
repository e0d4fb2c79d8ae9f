"""bench.py's command-line contract, checked without a GPU: more than one
GPU is refused with a message and exit status 2 before anything touches a
device, and the algorithmic byte model counts what the kernels must move."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_expert_launch():
    sys.path.insert(0, ROOT)
    import bench
    from block_discrete_diffusion_dg_amd import synth
    kinds, per_step = bench.algorithmic_model(synth.FULL, 2048, 256, 64.0)
    # 64 touched experts x 8.65 MB (gate, up, down: 704 x 2048 bf16 each)
    # + the shared expert's 25.2 MB (three 2048 x 2048 bf16 matrices)
    assert kinds["experts"][0] == 553_648_128 + 25_165_824
    assert per_step["lmhead"][0] == 1_073_741_824  # the tied embedding, read once
    # FP8: 64 x (4,325,376 code bytes + 13,824 scale bytes) + 12,582,912 + 24,576
    assert bench.fp8_expert_bytes(synth.FULL, 64.0) == 64 * (4_325_376 + 13_824) + 12_582_912 + 24_576


def test_clock_record_parses_rocm_smi_json():
    sys.path.insert(0, ROOT)
    import bench
    text = ('{"card0": {"dcefclk clock speed:": "(0Mhz)", "fclk clock speed:": "(1900Mhz)", '
            '"mclk clock speed:": "(1900Mhz)", "mclk clock level:": "0", "sclk clock speed:": "(2400Mhz)", '
            '"sclk clock level:": "1"}, "system": {"driver": "x"}}')
    assert bench.parse_clocks(text) == {"card0": {"dcefclk": 0.0, "fclk": 1900.0, "mclk": 1900.0, "sclk": 2400.0}}
    assert bench.parse_clocks("not json") is None
    assert bench.parse_clocks('{"card0": {"Card series:": "x"}}') is None


def test_fp8_profile_needs_profile():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--fp8-profile"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--profile" in r.stderr and r.stdout == ""

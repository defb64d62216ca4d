"""CPU check of the division the one-launch linear layer uses inside the GEMM
(tests/native/fused_division_check.c, built here with gcc): the reciprocal-and-correction
quotient, with x's sign, equals the correctly rounded x / s after the +-448 clamp for every
bf16 and fp16 input and group scale, up to quotients below 2^-10 that round to the same zero
code. By default every 16th group amax is taken (all inputs x for each); BFP8_FULL_DIVISION_CHECK=1
takes all of them (about a minute of CPU time per format)."""

import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "fused_division_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path_factory.mktemp("divcheck") / "fused_division_check")
    subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, SRC, "-lm"], check=True)
    return exe


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_reciprocal_correction_matches_the_division(checker, fmt):
    step = "1" if os.environ.get("BFP8_FULL_DIVISION_CHECK") == "1" else "16"
    res = subprocess.run([checker, fmt, step], capture_output=True, text=True, timeout=600)
    m = re.match(r"(\w+) pairs=(\d+) differ=(\d+) code_mismatch=(\d+)", res.stdout)
    assert m, res.stdout + res.stderr
    pairs, mismatch = int(m.group(2)), int(m.group(4))
    assert pairs > (60_000_000 if step == "16" else 1_000_000_000)
    assert mismatch == 0, res.stdout
    assert res.returncode == 0

"""Exhaustive CPU check of the division-free quotient inside the GPU per-token quantiser.

The quantiser encodes E4M3(fl32(x / s)) per token (Lernex/Metis-1.6-Logos-FP8, "What is in FP8":
activations quantized per token at run time). The kernel obtains fl32(x / s) from x * fl32(1 / s)
with one fused residual correction; ``quotient_correction.c`` checks that this gives the same E4M3
code as the correctly rounded quotient for every BF16 (row maximum, value) pair, and that it catches
three planted mistakes in the formula. The GPU parity tests of the quantiser compare the kernel itself
with the oracle.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("quotient") / "quotient_correction")
    subprocess.run([gcc, "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-o", exe,
                    os.path.join(HERE, "quotient_correction.c"), "-lm"], check=True)
    return exe


def _run(exe, mode):
    res = subprocess.run([exe, str(mode)], capture_output=True, text=True, timeout=600)
    fields = res.stdout.split()
    return res.returncode, int(fields[fields.index("failures") + 1]), res.stdout


def test_corrected_quotient_matches_division_for_all_bf16_pairs(checker):
    rc, failures, out = _run(checker, 0)
    assert rc == 0 and failures == 0, out
    assert "pairs 1065402240" in out  # every amax in [0, 0x7F7F] times every |x| <= amax, both signs


@pytest.mark.parametrize("mode", [1, 2, 3], ids=["no_copysign", "no_scale_threshold", "no_correction"])
def test_check_catches_planted_mistakes(checker, mode):
    rc, failures, out = _run(checker, mode)
    assert rc != 0 and failures > 0, out

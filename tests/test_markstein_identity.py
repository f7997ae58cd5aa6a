"""CPU check of the arithmetic identities the HIP quantizers rely on to
replace Eq. 2's per-element division (Mix-Quant Section 3.3, Eq. 2) by a
reciprocal product with Markstein's correction: the E2M1 codes equal those of
the IEEE quotient for every finite BF16 numerator over a spread of divisors,
the corrected quotient equals the IEEE quotient for random FP32 numerators,
and signed zeros keep their sign.  The kernels themselves are compared with the oracle bit for bit
in the GPU tests; this pins the identity those kernels use, over far more
cases than any GPU test covers."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("markstein") / "markstein_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "markstein_check.c"), "-lm"], check=True)
    return exe


@pytest.mark.parametrize("mode,n", [("codes", 4096), ("quot", 50_000_000), ("zeros", 100_000)])
def test_markstein_identity(checker, mode, n):
    r = subprocess.run([checker, mode, str(n)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 mismatches" in r.stdout

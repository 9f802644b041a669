"""The activation quantizers of the HIP library replace the correctly rounded
division x / S by two FMAs from r = RN(1/S) for 16-bit inputs.  This test
compiles tests/native/div_sequence_check.c and checks, exhaustively over every
bf16 / fp16 input x with |x| <= alpha and every scale S = max(RN(alpha/qmax),
1e-8) derived from a bf16 / fp16 row absmax alpha, that the int8 codes
(qmax 127) and the e4m3 codes (qmax 448) are identical.  CPU only."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "div_sequence_check.c")


@pytest.fixture(scope="module")
def checker():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "divcheck")
    subprocess.run([gcc, "-O2", "-ffp-contract=off", "-fopenmp", "-o", exe, SRC, "-lm"], check=True)
    yield exe
    shutil.rmtree(d)


@pytest.mark.parametrize("dtype,mode", [("bf16", "i8"), ("f16", "i8"), ("bf16", "e4m3"), ("f16", "e4m3")])
def test_fma_division_gives_identical_codes(checker, dtype, mode):
    r = subprocess.run([checker, dtype, mode], capture_output=True, text=True, timeout=900)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "mismatches=0" in r.stdout
    checked = int(r.stdout.split("checked=")[1].split()[0])
    assert checked > 10**9

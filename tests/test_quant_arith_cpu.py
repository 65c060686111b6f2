"""The GPU quantizer's fp32 arithmetic, emulated on the host and checked
against the plain Eq.(4) definitions ("paper_specification.yaml",
lq1_quantization): the step base fl32(absmax / qmax) over every finite fp32
absmax (qmax 7 and 127), and the reciprocal fast path of the codes against
the correctly rounded division on random and near-tie inputs.  The emulation
is ``quant_arith_check.c`` (gcc, one IEEE fp32 rounding per operation)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "quant_arith_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("arith") / "quant_arith_check")
    flags = ["-O2", "-ffp-contract=off", "-fopenmp"]
    try:  # hardware FMA (the same single rounding as libm's fmaf, much faster)
        if " fma " in open("/proc/cpuinfo").read().replace("\n", " "):
            flags.append("-mfma")
    except OSError:
        pass
    subprocess.run([cc, *flags, "-o", exe, SRC, "-lm"], check=True)
    return exe


def run(exe, mode):
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([exe, mode], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout.strip())
    return r.returncode, r.stdout


def test_step_base_is_the_correctly_rounded_quotient_for_every_fp32(checker):
    rc, out = run(checker, "step")
    assert rc == 0, out
    assert "mismatches qmax7 0 qmax127 0" in out


def test_step_check_detects_a_missing_correction(checker):
    # without the FMA correction fl32(absmax * fl32(1/qmax)) is often off by
    # one ulp: the exhaustive check must see that
    rc, out = run(checker, "step_nocorr")
    assert rc == 1, out


def test_reciprocal_fast_path_never_decides_a_wrong_code(checker):
    rc, out = run(checker, "codes")
    assert rc == 0, out
    accepted = int(out.split(" of ")[1].split()[0])
    # 3 reciprocals x 2 forms per case; three quarters of the cases are drawn
    # at or near a rounding boundary, where the fast path must often decline
    assert accepted > 0.3 * 6 * 20_000_000


def test_codes_check_detects_a_missing_margin(checker):
    # accepting rint(fl32(x * r)) everywhere gives wrong codes next to ties
    rc, out = run(checker, "codes_loose")
    assert rc == 1, out

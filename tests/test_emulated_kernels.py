"""The library's compiled gfx950 kernels, executed on the CPU by the checking
emulator in tests/isa_emu, against the fp64 oracle.

The real host code of libqkmla.so runs over a stand-in for the HIP runtime
whose launches execute the device assembly the build keeps next to the
library.  Besides oracle parity (same tolerances as the GPU tests) every run
checks memory bounds, wait counts, LDS races and inline-asm wait states; see
tests/isa_emu/__init__.py.  The cases run in a child process, because the
stand-in must be the only HIP runtime in it.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mla_latent_decode_amd", "libqkmla.so")
ASM = glob.glob(os.path.join(ROOT, "mla_latent_decode_amd", "_build", "*-gfx950.s"))

pytestmark = pytest.mark.skipif(
    not (os.path.exists(LIB) and ASM and shutil.which("gcc")),
    reason="needs the built library with its device assembly (python -m "
           "mla_latent_decode_amd.build) and gcc")


@pytest.fixture(scope="module")
def runtime(tmp_path_factory):
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from isa_emu.device import build_runtime
    return build_runtime(str(tmp_path_factory.mktemp("hip_stand_in")))


@pytest.mark.parametrize("case", ["hazard_checker", "fp32_tiny", "bf16_split", "bf16_plain_hold",
                                  "bf16_long_segments", "bf16_plain_overflow", "bf16_append_caches",
                                  "bf16_64_heads", "multi_query", "paged_caches",
                                  "train_fwd_bwd"])
def test_kernels_on_the_emulator(runtime, case):
    env = {k: v for k, v in os.environ.items() if k != "QKMLA_NUM_WG"}
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "isa_emu", "cases.py"),
                        runtime, case], capture_output=True, text=True, timeout=900, env=env,
                       cwd=ROOT)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "RuntimeWarning" not in l)
    print(out)
    assert r.returncode == 0, out[-4000:]

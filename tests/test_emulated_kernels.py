"""The library's compiled gfx950 kernels, executed on the CPU by the checking
emulator in tests/isa_emu, against the fp64 oracle.

The real host code of libqkmla.so runs over a stand-in for the HIP runtime
whose launches execute the device assembly the build keeps next to the
library.  Besides oracle parity (same tolerances as the GPU tests) every run
checks memory bounds, wait counts, LDS races and inline-asm wait states; see
tests/isa_emu/__init__.py.  The cases run in a child process, because the
stand-in must be the only HIP runtime in it.
"""
import concurrent.futures
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


# longest first; all start together (at most _WORKERS at a time) when the
# first case is asked for, so the module takes about as long as its longest case
CASES = ["train_mfma", "train_varlen", "train_fwd_bwd", "paged_caches", "bf16_long_segments",
         "bf16_max_batch", "bf16_many_splits", "multi_query",
         "bf16_split", "bf16_append_caches", "bf16_64_heads", "bf16_plain_overflow",
         "bf16_plain_hold", "fp32_tiny", "hazard_checker", "isa_semantics"]
_WORKERS = max(1, min(6, (os.cpu_count() or 2) - 1))
_futures = {}


def _run_case(runtime, case):
    env = {k: v for k, v in os.environ.items() if k != "QKMLA_NUM_WG"}
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "isa_emu", "cases.py"),
                        runtime, case], capture_output=True, text=True, timeout=1500, env=env,
                       cwd=ROOT)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "RuntimeWarning" not in l)
    return r.returncode, out


def _result(runtime, case):
    if os.environ.get("PYTEST_XDIST_WORKER"):  # under xdist each worker runs its own cases
        return _run_case(runtime, case)
    if not _futures:
        pool = concurrent.futures.ThreadPoolExecutor(max_workers=_WORKERS)
        for c in CASES:
            _futures[c] = pool.submit(_run_case, runtime, c)
    return _futures[case].result()


@pytest.mark.parametrize("case", CASES)
def test_kernels_on_the_emulator(runtime, case):
    rc, out = _result(runtime, case)
    print(out)
    assert rc == 0, out[-4000:]

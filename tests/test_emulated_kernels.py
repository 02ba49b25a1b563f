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


# longest first; the selected cases all start together (at most _WORKERS at a
# time) when the first one is asked for, so the module takes about as long as
# its longest case
CASES = ["train_mfma", "train_varlen", "train_fwd_bwd", "paged_caches", "bf16_long_segments",
         "bf16_max_batch", "bf16_ragged_full", "bf16_32k_step", "bf16_long_context", "bf16_headline_sequence", "bf16_many_splits", "multi_query",
         "bf16_split", "bf16_append_caches", "bf16_bulk_append_wide", "bf16_64_heads", "bf16_32_heads", "bf16_plain_overflow",
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


def _selected_cases(session):
    """The emulator cases this session will run (after -k / -m selection)."""
    names = []
    for item in session.items:
        cs = getattr(item, "callspec", None)
        if item.originalname == "test_kernels_on_the_emulator" and cs is not None:
            names.append(cs.params["case"])
    return [c for c in CASES if c in names] or CASES


def _result(runtime, case, session):
    if os.environ.get("PYTEST_XDIST_WORKER"):  # under xdist each worker runs its own cases
        return _run_case(runtime, case)
    if not _futures:
        pool = concurrent.futures.ThreadPoolExecutor(max_workers=_WORKERS)
        for c in _selected_cases(session):
            _futures[c] = pool.submit(_run_case, runtime, c)
    if case not in _futures:
        return _run_case(runtime, case)
    return _futures[case].result()


@pytest.mark.parametrize("case", CASES)
def test_kernels_on_the_emulator(runtime, case, request):
    rc, out = _result(runtime, case, request.session)
    print(out)
    assert rc == 0, out[-4000:]


def test_launch_limit_check_refuses_what_the_device_would():
    """The emulator refuses launches the device would reject, so every case
    above also checks its launch configurations."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from isa_emu.device import check_launch_fits
    from isa_emu.machine import EmuError
    md = {".max_flat_workgroup_size": 256, ".vgpr_count": 512}
    check_launch_fits("k", md, 153088, (256, 1, 1), (256, 1, 1), 0)
    bad = [((1, 1, 1), (512, 1, 1), 0, 0),        # above the compiled block size
           ((1, 1, 1), (256, 1, 1), 160000, 4096),  # LDS over 160 KiB
           ((0, 1, 1), (64, 1, 1), 0, 0),          # empty grid
           ((1, 70000, 1), (64, 1, 1), 0, 0)]      # grid y out of range
    for grid, block, lds, dyn in bad:
        with pytest.raises(EmuError):
            check_launch_fits("k", md, lds, grid, block, dyn)
    with pytest.raises(EmuError):  # 8 waves of 512 registers need two waves per SIMD
        check_launch_fits("k", {".max_flat_workgroup_size": 1024, ".vgpr_count": 512}, 0,
                          (1, 1, 1), (512, 1, 1), 0)


def test_every_compiled_kernel_fits_a_gfx950_cu():
    """Static LDS and registers of every kernel in the library, at its compiled
    maximum workgroup size, fit one gfx950 compute unit."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from isa_emu.asm import load_kernels
    from isa_emu.device import GFX950_LDS_BYTES, check_launch_fits
    n = 0
    for f in ASM:
        for name, k in load_kernels(f).items():
            maxw = k.md.get(".max_flat_workgroup_size", 1024)
            check_launch_fits(name, k.md, k.lds_bytes, (1, 1, 1), (maxw, 1, 1), 0)
            assert k.lds_bytes <= GFX950_LDS_BYTES
            n += 1
    assert n >= 20, n

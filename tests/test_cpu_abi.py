"""CPU-side checks of the C-ABI library: it loads, exports every symbol the
header declares, validates arguments and plans without touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkmla.h")
LIB = os.path.join(ROOT, "mla_latent_decode_amd", "libqkmla.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libqkmla.so not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(qkmla_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("qkmla_absorb_weights", "qkmla_append", "qkmla_decode", "qkmla_out_proj"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def _ops():
    from mla_latent_decode_amd import ops
    return ops


def test_abi_version_and_status_strings():
    ops = _ops()
    assert ops.abi_version() == 2
    assert ops._lib.qkmla_status_string(0) == b"ok"
    assert ops._lib.qkmla_status_string(3) == b"workspace too small"


def _cfg(**kw):
    ops = _ops()
    base = dict(n_heads=128, n_groups=8, latent_rank=512, head_dim=128, rope_dim=64, v_head_dim=128)
    base.update(kw)
    return ops.Config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(n_heads=6, n_groups=4), 1),          # H % G != 0
    (dict(rope_dim=63), 1),                    # odd rope dim
    (dict(n_heads=0), 1),
    (dict(latent_rank=256), 2),                # bf16 path compiled for r = 512
    (dict(n_heads=96, n_groups=6), 2),         # H not in {64, 128}
    (dict(n_heads=32, n_groups=2), 2),         # one-wavefront variant switched off
    (dict(latent_rank=2048, dtype="f32"), 2),  # above the compiled limits
    (dict(eps=-1.0), 1),
    (dict(rope_base=0.0), 1),
])
def test_invalid_configs_are_rejected(kw, status):
    ops = _ops()
    cfg = _cfg(**kw)
    nwg, tile = ctypes.c_int32(), ctypes.c_int32()
    st = ops._lib.qkmla_plan(ctypes.byref(cfg.c()), 4, 1024, 256, ctypes.byref(nwg), ctypes.byref(tile))
    assert st == status
    assert ops._lib.qkmla_last_error()


def test_plan_fills_the_chip_and_respects_the_tile_bound():
    ops = _ops()
    cfg = _cfg()
    assert ops.plan(cfg, 16, 4096, 256) == (256, 32)
    assert ops.plan(cfg, 1, 262144, 256) == (256, 32)
    assert ops.plan(cfg, 1, 64, 256) == (2, 32)      # only 2 tiles exist
    assert ops.plan(cfg, 0, 64, 256)[0] == 0


def test_batch_zero_is_a_noop_without_touching_pointers():
    ops = _ops()
    cfg = _cfg()
    lib = ops._lib
    st = lib.qkmla_decode(ctypes.byref(cfg.c()), 0, None, None, None, None, None, None, None, None,
                          16, 16, None, 0, None, None, None, None)
    assert st == 0
    st = lib.qkmla_append(ctypes.byref(cfg.c()), 0, 1, None, None, None, None, None, 16, None, None,
                          None, None, None)
    assert st == 0


def test_null_and_misaligned_pointers_are_rejected():
    ops = _ops()
    cfg = _cfg()
    lib = ops._lib
    st = lib.qkmla_decode(ctypes.byref(cfg.c()), 1, None, None, None, None, None, None, None, None,
                          16, 16, None, 0, None, None, None, None)
    assert st == 1
    fake = ctypes.c_void_p(0x1000 + 2)  # misaligned for float, never dereferenced
    st = lib.qkmla_out_proj(ctypes.byref(cfg.c()), 1, fake, fake, fake, None)
    assert st == 1 and b"aligned" in lib.qkmla_last_error()


def test_decode_rejects_bad_length_bound():
    ops = _ops()
    cfg = _cfg()
    lib = ops._lib
    p = ctypes.c_void_p(0x1000)
    st = lib.qkmla_decode(ctypes.byref(cfg.c()), 1, p, p, p, p, p, p, p, p, 16, 17, p, 1 << 20,
                          p, None, None, None)
    assert st == 1  # max_seq_len > cache_capacity


def test_decode_multi_validates_query_rows():
    """s_q < 1 is an invalid argument, batch * s_q above 4096 unsupported;
    both are rejected before any pointer is used."""
    ops = _ops()
    cfg = _cfg()
    lib = ops._lib
    p = ctypes.c_void_p(0x1000)
    st = lib.qkmla_decode_multi(ctypes.byref(cfg.c()), 2, 0, p, p, p, p, p, p, p, p, 16, 16, p,
                                1 << 20, p, None, None, None)
    assert st == 1 and b"s_q" in lib.qkmla_last_error()
    st = lib.qkmla_decode_multi(ctypes.byref(cfg.c()), 1025, 4, p, p, p, p, p, p, p, p, 16, 16, p,
                                1 << 20, p, None, None, None)
    assert st == 2
    st = lib.qkmla_decode_multi(ctypes.byref(cfg.c()), 0, 3, None, None, None, None, None, None,
                                None, None, 16, 16, None, 0, None, None, None, None)
    assert st == 0

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
    assert ops.abi_version() == 8
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
    (dict(n_heads=96, n_groups=6), 2),         # H not in {32, 64, 128}
    (dict(n_heads=16, n_groups=1), 2),         # fewer heads than one wavefront's 32
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


def test_mfma_out_proj_requires_16_byte_alignment():
    """The bf16 V up-projection of the DeepSeek-V3-like layer reads o_lat and
    W^UV as 16-byte vectors: pointers aligned to their element size but not to
    16 bytes are rejected before any launch."""
    ops = _ops()
    cfg = _cfg(dtype="bf16")
    lib = ops._lib
    ok16 = ctypes.c_void_p(0x10000)
    off4 = ctypes.c_void_p(0x10000 + 4)  # float-aligned, not 16-byte aligned; never dereferenced
    for o_lat, w_uv in ((off4, ok16), (ok16, off4)):
        st = lib.qkmla_out_proj(ctypes.byref(cfg.c()), 1, o_lat, w_uv, ok16, None)
        assert st == 1 and b"16-byte" in lib.qkmla_last_error()


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


def _pages(ops, bt=0x2000, max_blocks=4, page_size=64, num_pages=8):
    return ops._Pages(ctypes.c_void_p(bt) if bt else None, max_blocks, page_size, num_pages)


def test_paged_entry_points_validate_the_page_description():
    """Bad page descriptions are rejected on the host before any pointer is
    used: a missing table or non-positive sizes are invalid arguments, a
    capacity above int32 too, a bf16 page that does not hold whole 32-row
    tiles is unsupported, and max_seq_len above max_blocks * page_size is
    invalid."""
    ops = _ops()
    cfg = _cfg()
    lib = ops._lib
    p = ctypes.c_void_p(0x1000)

    def decode(pages, max_seq_len=64):
        return lib.qkmla_decode_paged(ctypes.byref(cfg.c()), 1, 1, p, p, p, p, p, p, p, p,
                                      ctypes.byref(pages) if pages is not None else None,
                                      max_seq_len, p, 1 << 20, p, None, None, None)

    assert decode(None) == 1
    assert decode(_pages(ops, bt=0)) == 1 and b"block table" in lib.qkmla_last_error()
    assert decode(_pages(ops, page_size=0)) == 1
    assert decode(_pages(ops, num_pages=0)) == 1
    assert decode(_pages(ops, max_blocks=1 << 16, page_size=1 << 16)) == 1
    assert decode(_pages(ops, bt=0x2002)) == 1 and b"aligned" in lib.qkmla_last_error()
    assert decode(_pages(ops, page_size=48)) == 2 and b"multiple of 32" in lib.qkmla_last_error()
    assert decode(_pages(ops), max_seq_len=257) == 1  # capacity 4 * 64 = 256
    st = lib.qkmla_decode_paged(ctypes.byref(cfg.c()), 0, 1, None, None, None, None, None, None,
                                None, None, None, 16, None, 0, None, None, None, None)
    assert st == 0  # batch 0: no-op, nothing read

    def append(pages):
        return lib.qkmla_append_paged(ctypes.byref(cfg.c()), 1, 1, p, p, p, p, p,
                                      ctypes.byref(pages) if pages is not None else None,
                                      p, p, p, None, None)

    assert append(None) == 1
    assert append(_pages(ops, page_size=-1)) == 1
    st = lib.qkmla_append_paged(ctypes.byref(cfg.c()), 0, 1, None, None, None, None, None, None,
                                None, None, None, None, None)
    assert st == 0


def test_f32_pages_of_any_size_pass_host_validation():
    """The float path reads rows one by one, so any page size passes the host
    checks (the call then fails only for want of a device)."""
    ops = _ops()
    cfg = _cfg(n_heads=4, n_groups=2, latent_rank=32, head_dim=16, rope_dim=8, v_head_dim=16,
               dtype="f32")
    lib = ops._lib
    p = ctypes.c_void_p(0x1000)
    pages = _pages(ops, page_size=3)
    st = lib.qkmla_decode_paged(ctypes.byref(cfg.c()), 1, 1, p, p, p, p, p, p, p, p,
                                ctypes.byref(pages), 12, p, 0, p, None, None, None)
    assert st in (3, 4)  # workspace too small, or no device to plan for


def test_train_entry_points_validate_on_the_host():
    """Training calls: shape limits of their own (any bf16 shape, d_c and d_v
    up to 256), NULL inputs and gradients, workspace size, batch 0 no-op;
    all checked before any device access."""
    ops = _ops()
    lib = ops._lib
    small_bf16 = _cfg(n_heads=6, n_groups=3, latent_rank=40, head_dim=16, rope_dim=8,
                      v_head_dim=12)
    assert ops.train_workspace_size(small_bf16, 2, 45) > 0  # no decode shape restriction
    big = _cfg(head_dim=512, dtype="f32")
    assert lib.qkmla_train_workspace_size(ctypes.byref(big.c()), 1, 8) == 0
    assert b"d_c and d_v" in lib.qkmla_last_error()
    cfg = _cfg(n_heads=4, n_groups=2, latent_rank=12, head_dim=6, rope_dim=4, v_head_dim=5,
               dtype="f32")
    p = 0x1000
    ins = ops._TrainInputs(*([p] * 10))
    st = lib.qkmla_train_forward(ctypes.byref(cfg.c()), 0, 7, None, None, 0, None, None, None)
    assert st == 0  # batch 0
    st = lib.qkmla_train_forward(ctypes.byref(cfg.c()), 1, 0, ctypes.byref(ins), p, 1 << 20, p, p,
                                 None)
    assert st == 1  # seq_len 0
    st = lib.qkmla_train_forward(ctypes.byref(cfg.c()), 1, 7, None, p, 1 << 20, p, p, None)
    assert st == 1 and b"inputs" in lib.qkmla_last_error()
    missing = ops._TrainInputs(*([p] * 9 + [0]))  # gamma_k_rope NULL with qk_norm
    st = lib.qkmla_train_forward(ctypes.byref(cfg.c()), 1, 7, ctypes.byref(missing), p, 1 << 20,
                                 p, p, None)
    assert st == 1
    st = lib.qkmla_train_forward(ctypes.byref(cfg.c()), 1, 7, ctypes.byref(ins), p, 16, p, p, None)
    assert st == 3  # workspace too small
    grads = ops._TrainGrads(*([p] * 9 + [0]))
    need = ops.train_workspace_size(cfg, 1, 7)
    st = lib.qkmla_train_backward(ctypes.byref(cfg.c()), 1, 7, ctypes.byref(ins), p, p, p, p, need,
                                  ctypes.byref(grads), None)
    assert st == 1 and b"gradient" in lib.qkmla_last_error()
    grads = ops._TrainGrads(*([p] * 10))
    st = lib.qkmla_train_backward(ctypes.byref(cfg.c()), 1, 7, ctypes.byref(ins), p, p, p, p,
                                  need - 256, ctypes.byref(grads), None)
    assert st == 3


def test_varlen_train_entry_points_validate_on_the_host():
    """Packed-sequence training calls: empty batches are no-ops, cu_seqlens
    must be given and aligned, max_seq_len >= 1, at most 65535 sequences and 2^24 rows,
    and the workspace is checked against the packed size."""
    ops = _ops()
    lib = ops._lib
    cfg = _cfg(n_heads=4, n_groups=2, latent_rank=12, head_dim=6, rope_dim=4, v_head_dim=5,
               dtype="f32")
    p = 0x1000
    ins = ops._TrainInputs(*([p] * 10))
    c = ctypes.byref(cfg.c())
    assert lib.qkmla_train_forward_varlen(c, 0, None, 0, 1, None, None, 0, None, None, None,
                                          None) == 0
    assert lib.qkmla_train_forward_varlen(c, 3, None, 0, 4, None, None, 0, None, None, None,
                                          None) == 0  # no tokens
    assert lib.qkmla_train_forward_varlen(c, 2, None, 9, 5, ctypes.byref(ins), p, 1 << 20, p, p,
                                          None, None) == 1
    assert b"cu_seqlens" in lib.qkmla_last_error()
    assert lib.qkmla_train_forward_varlen(c, 2, p + 2, 9, 5, ctypes.byref(ins), p, 1 << 20, p, p,
                                          None, None) == 1
    assert lib.qkmla_train_forward_varlen(c, 2, p, 9, 0, ctypes.byref(ins), p, 1 << 20, p, p,
                                          None, None) == 1
    assert lib.qkmla_train_forward_varlen(c, 70000, p, 70000, 1, ctypes.byref(ins), p, 1 << 30, p,
                                          p, None, None) == 2
    # more than 2^24 token rows: the row-per-block launches would overflow
    assert lib.qkmla_train_forward_varlen(c, 1, p, (1 << 24) + 1, 8, ctypes.byref(ins), p, 1 << 30,
                                          p, p, None, None) == 2
    assert b"2^24" in lib.qkmla_last_error()
    need = ops.train_workspace_size_varlen(cfg, 2, 9, 5)
    assert need > 0
    assert lib.qkmla_train_forward_varlen(c, 2, p, 9, 5, ctypes.byref(ins), p, 16, p, p, None,
                                          None) == 3
    grads = ops._TrainGrads(*([p] * 10))
    assert lib.qkmla_train_backward_varlen(c, 2, p, 9, 5, ctypes.byref(ins), p, p, p, p, need - 256,
                                           ctypes.byref(grads), None, None) == 3


def test_binding_refuses_host_tensors_before_any_call():
    """A host tensor's address handed to a kernel would be a device memory
    fault; the binding refuses it (and wrong shapes) with an error instead."""
    import torch
    ops = _ops()
    cfg = _cfg(n_heads=4, n_groups=2, latent_rank=32, head_dim=16, rope_dim=8, v_head_dim=16,
               dtype="f32")
    w = torch.zeros((2, 32, 16))
    g = torch.ones((16,))
    with pytest.raises(ops.QkmlaError, match="current GPU"):
        ops.absorb_weights(cfg, w, g, g, out=torch.empty((2, 32, 16)))
    with pytest.raises(ops.QkmlaError, match="current GPU"):
        ops.out_proj(cfg, torch.zeros((1, 4, 32)), torch.zeros((2, 32, 16)),
                     out=torch.empty((1, 4, 16)))

"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/jfa.h declares, sizes workspaces, and rejects invalid arguments with the
documented status codes before touching any memory."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jfa.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    from variable_length_flash_jfa_amd import _binding
    if not os.path.exists(_binding.library_path()):
        pytest.skip("libjfa.so not built")
    return _binding.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jfa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("jfa_fwd", "jfa_bwd", "jfa_fwd_workspace_size", "jfa_bwd_workspace_size",
                     "jfa_last_error"):
        assert required in names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version(lib):
    assert lib.jfa_version().decode().startswith("jfa ")


FAKE = ctypes.c_void_p(1 << 20)  # 16-byte aligned, never dereferenced on rejected calls


def fwd(lib, *, batch=4, heads=2, head_dim=128, q_len=64, total_kv=100, bq=1, causal=0, scale=0.1,
        ws=FAKE, ws_bytes=1 << 30, q=FAKE, o=FAKE):
    return lib.jfa_fwd(q, FAKE, FAKE, FAKE, 0, batch, heads, head_dim, q_len, total_kv, bq, causal,
                       scale, o, FAKE, ws, ws_bytes, None)


def bwd(lib, *, batch=4, heads=2, head_dim=128, q_len=64, total_kv=100, bq=1, causal=0, scale=0.1,
        ws=FAKE, ws_bytes=1 << 30, dq=FAKE):
    return lib.jfa_bwd(FAKE, FAKE, FAKE, FAKE, 0, batch, heads, head_dim, q_len, total_kv, bq, causal,
                       scale, FAKE, FAKE, FAKE, dq, FAKE, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("call", [fwd, bwd])
def test_rejections(lib, call):
    assert call(lib, head_dim=96) == UNSUPPORTED
    assert b"head_dim" in lib.jfa_last_error()
    assert call(lib, causal=1) == UNSUPPORTED                 # broadcast + causal
    assert call(lib, bq=0, q_len=5) == INVALID                # self mode needs q_len == 0
    assert call(lib, bq=1, q_len=0) == INVALID                # broadcast needs q_len >= 1
    assert call(lib, heads=0) == INVALID
    assert call(lib, batch=-1) == INVALID
    assert call(lib, total_kv=-3) == INVALID
    assert call(lib, scale=0.0) == INVALID
    assert call(lib, scale=float("nan")) == INVALID
    assert call(lib, scale=float("inf")) == INVALID
    assert call(lib, ws=None) == INVALID
    assert call(lib, ws=ctypes.c_void_p((1 << 20) + 8)) == INVALID   # misaligned
    assert call(lib, ws_bytes=16) == WS_SMALL
    assert b"workspace" in lib.jfa_last_error()


def test_null_and_noop(lib):
    assert fwd(lib, q=None) == INVALID
    assert fwd(lib, o=None) == INVALID
    assert bwd(lib, dq=None) == INVALID
    # empty problems are OK no-ops and touch nothing
    assert fwd(lib, batch=0, q=None, o=None, ws=None) == OK
    assert bwd(lib, batch=0, dq=None, ws=None) == OK
    assert fwd(lib, bq=0, q_len=0, total_kv=0, q=None, o=None, ws=None) == OK


def test_workspace_sizes(lib):
    f = lib.jfa_fwd_workspace_size
    b = lib.jfa_bwd_workspace_size
    assert f(4, 2, 128, 64, 100, 1, 0) > 0
    assert b(4, 2, 128, 64, 100, 1, 0) >= 8 * 64 * 2 * 128 * 4      # 8 fp32 dQ stripes
    assert b(3, 2, 64, 0, 500, 0, 1) >= 500 * 2 * 64 * 4              # self-mode fp32 dQ
    assert f(4, 2, 96, 64, 100, 1, 0) == 0                              # invalid -> 0
    assert b(4, 2, 128, 64, 100, 1, 1) == 0
    # monotone in the sizes
    assert f(1000, 4, 128, 256, 10 ** 6, 1, 0) >= f(10, 4, 128, 256, 10 ** 4, 1, 0)


def test_schedule_selector(lib):
    from variable_length_flash_jfa_amd import _binding
    old = _binding.get_schedule()
    try:
        for s in (_binding.SCHED_IDENTITY, _binding.SCHED_DYNAMIC, _binding.SCHED_SORTED_ZIGZAG):
            _binding.set_schedule(s)
            assert _binding.get_schedule() == s
        with pytest.raises(_binding.JfaError):
            _binding.set_schedule(7)
    finally:
        _binding.set_schedule(old)


def bwd_rope(lib, *, batch=4, heads=2, head_dim=128, q_len=64, total_kv=100, bq=1, causal=0, scale=0.1,
             cos=FAKE, sin=FAKE, pos_q=FAKE, pos_k=FAKE, max_pos=300, ws=FAKE, ws_bytes=1 << 30):
    return lib.jfa_bwd_rope(FAKE, FAKE, FAKE, FAKE, 0, batch, heads, head_dim, q_len, total_kv, bq, causal,
                            scale, FAKE, FAKE, FAKE, cos, sin, pos_q, pos_k, max_pos, FAKE, FAKE, FAKE,
                            ws, ws_bytes, None)


def test_rope_rejections(lib):
    assert bwd_rope(lib, cos=None) == INVALID
    assert bwd_rope(lib, sin=None) == INVALID
    assert bwd_rope(lib, pos_q=None) == INVALID
    assert bwd_rope(lib, pos_k=None) == INVALID
    assert b"rotary" in lib.jfa_last_error()
    assert bwd_rope(lib, max_pos=0) == INVALID
    assert bwd_rope(lib, max_pos=(1 << 24) + 1) == INVALID
    assert bwd_rope(lib, cos=ctypes.c_void_p((1 << 20) + 4)) == INVALID    # tables 16-byte aligned
    assert bwd_rope(lib, pos_k=ctypes.c_void_p((1 << 20) + 2)) == INVALID  # positions 4-byte aligned
    # the plain backward's checks apply too, under this entry point's name
    assert bwd_rope(lib, head_dim=96) == UNSUPPORTED
    assert b"jfa_bwd_rope" in lib.jfa_last_error()
    assert bwd_rope(lib, ws_bytes=16) == WS_SMALL
    assert bwd_rope(lib, batch=0, ws=None) == OK                            # empty: a no-op


def fwd_sparse(lib, *, batch=4, heads=2, head_dim=128, q_len=64, total_kv=100, bq=1, scale=0.1, topk=4,
               ws=FAKE, ws_bytes=1 << 30, blocks=None):
    return lib.jfa_fwd_sparse(FAKE, FAKE, FAKE, FAKE, 0, batch, heads, head_dim, q_len, total_kv, bq, scale,
                              topk, FAKE, FAKE, blocks, ws, ws_bytes, None)


def test_sparse_rejections_and_sizes(lib):
    assert fwd_sparse(lib, topk=0) == INVALID
    assert fwd_sparse(lib, topk=65) == INVALID
    assert b"topk" in lib.jfa_last_error()
    assert fwd_sparse(lib, head_dim=96) == UNSUPPORTED
    assert fwd_sparse(lib, bq=0, q_len=5) == INVALID
    assert fwd_sparse(lib, blocks=ctypes.c_void_p((1 << 20) + 2)) == INVALID   # 4-byte aligned output
    assert fwd_sparse(lib, ws_bytes=16) == WS_SMALL
    assert fwd_sparse(lib, batch=0, ws=None) == OK
    ws = lib.jfa_fwd_sparse_workspace_size
    assert ws(4, 2, 128, 64, 100, 1, 4) > lib.jfa_fwd_workspace_size(4, 2, 128, 64, 100, 1, 0)
    assert ws(4, 2, 128, 64, 100, 1, 0) == 0 and ws(4, 2, 128, 64, 100, 1, 65) == 0
    nqb = lib.jfa_fwd_sparse_query_blocks
    assert nqb(4, 600, 1000, 1) == 4 * 3              # broadcast: B * ceil(Lq / 256)
    assert nqb(3, 0, 1000, 0) >= 1000 // 128 + 3       # self: an upper bound of sum ceil(n_b / 128)


def fwd_mx(lib, *, batch=4, heads=2, head_dim=128, q_len=64, total_kv=100, bq=1, causal=0, scale=0.1,
           ws=FAKE, ws_bytes=1 << 30, q8=FAKE, qs=FAKE):
    return lib.jfa_fwd_mxfp8(q8, qs, FAKE, FAKE, FAKE, FAKE, FAKE, 0, batch, heads, head_dim, q_len, total_kv,
                             bq, causal, scale, FAKE, FAKE, ws, ws_bytes, None)


def test_mxfp8_rejections_and_sizes(lib):
    assert fwd_mx(lib, head_dim=96) == UNSUPPORTED
    assert b"jfa_fwd_mxfp8" in lib.jfa_last_error()
    assert fwd_mx(lib, bq=1, causal=1) == UNSUPPORTED
    assert fwd_mx(lib, scale=0.0) == INVALID
    assert fwd_mx(lib, qs=None) == INVALID                                  # null scales
    assert fwd_mx(lib, q8=ctypes.c_void_p((1 << 20) + 8)) == INVALID       # 16-byte aligned values
    assert fwd_mx(lib, ws_bytes=16) == WS_SMALL
    assert fwd_mx(lib, batch=0, ws=None) == OK
    assert lib.jfa_mxfp8_v_blocks(3, 100) == 3 + 4 and lib.jfa_mxfp8_v_blocks(0, 0) == 0
    qr = lib.jfa_mxfp8_quantize_rows
    assert qr(FAKE, 10, 2, 96, FAKE, FAKE, None) == UNSUPPORTED
    assert qr(FAKE, -1, 2, 128, FAKE, FAKE, None) == INVALID
    assert qr(None, 10, 2, 128, FAKE, FAKE, None) == INVALID
    assert qr(None, 0, 2, 128, None, None, None) == OK                       # empty: a no-op
    qv = lib.jfa_mxfp8_quantize_v
    assert qv(FAKE, FAKE, 0, 4, 2, 64, 100, None, FAKE, None) == INVALID
    assert qv(FAKE, FAKE, 0, 4, 2, 48, 100, FAKE, FAKE, None) == UNSUPPORTED
    assert qv(None, None, 0, 0, 2, 64, 0, None, None, None) == OK

"""The C-ABI library loads, exports every declared symbol and validates on the host.

CPU only: every call here returns its status before any HIP call is made.
"""
import ctypes
import subprocess

import pytest

from query_union_paged_amd import pageweaver as pw

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: each call below fails validation first


def test_every_declared_symbol_is_exported():
    names = pw.header_functions()
    assert {"pw_group", "pw_union_attention", "pw_dense_union_ref"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", pw.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert pw._lib.pw_abi_version() == 1


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5):
        assert pw._lib.pw_status_string(st).decode()
    assert pw._lib.pw_status_string(42) == b"unknown status"


def _shape(**kw):
    base = dict(T=1024, H_q=4, H_kv=1, D=64, P=16, N_pages=64, S=8)
    base.update(kw)
    return pw.PWShape(*[base[k] for k in ("T", "H_q", "H_kv", "D", "P", "N_pages", "S")])


def _group(shp, W=32, g=8, sel=FAKE, ids=FAKE):
    return pw._lib.pw_group(ctypes.byref(shp), sel, W, g, ids, None, 0, None)


def _attn(shp, g=8, ptrs=None):
    p = ptrs or [FAKE] * 7
    return pw._lib.pw_union_attention(ctypes.byref(shp), p[0], p[1], p[2], p[3], p[4], p[5], g,
                                      p[6], None, 0, None)


def test_group_validation():
    assert pw._lib.pw_group(None, FAKE, 32, 8, FAKE, None, 0, None) == pw.PW_ERR_NULL
    assert _group(_shape(T=0)) == pw.PW_ERR_DIMS
    assert _group(_shape(T=1000)) == pw.PW_ERR_DIMS                 # T != N_pages * P
    assert _group(_shape(H_q=6, H_kv=4)) == pw.PW_ERR_DIMS
    assert _group(_shape(), sel=None) == pw.PW_ERR_NULL
    assert _group(_shape(), ids=None) == pw.PW_ERR_NULL
    assert _group(_shape(), W=0) == pw.PW_ERR_UNSUPPORTED
    assert _group(_shape(), W=1025) == pw.PW_ERR_UNSUPPORTED
    assert _group(_shape(), g=17) == pw.PW_ERR_UNSUPPORTED
    assert _group(_shape(T=2048 * 16, N_pages=2048)) == pw.PW_ERR_UNSUPPORTED
    assert b"W = 1025" in (_group(_shape(), W=1025) and pw._lib.pw_last_error())
    assert pw._lib.pw_group_workspace_bytes(ctypes.byref(_shape()), 32, 8) == 0


def test_attention_validation():
    assert _attn(_shape(), ptrs=[FAKE, None] + [FAKE] * 5) == pw.PW_ERR_NULL
    assert _attn(_shape(), ptrs=[FAKE] * 6 + [None]) == pw.PW_ERR_NULL
    assert _attn(_shape(D=96)) == pw.PW_ERR_UNSUPPORTED
    assert _attn(_shape(P=8, N_pages=128)) == pw.PW_ERR_UNSUPPORTED
    assert _attn(_shape(), g=0) == pw.PW_ERR_UNSUPPORTED
    assert _attn(_shape(), g=17) == pw.PW_ERR_UNSUPPORTED
    assert _attn(_shape(H_q=8, H_kv=1), g=16) == pw.PW_ERR_UNSUPPORTED     # 128 query rows
    assert _attn(_shape(H_q=16, H_kv=1), g=8) == pw.PW_ERR_UNSUPPORTED   # 128 query rows
    assert _attn(_shape(S=200), g=8) == pw.PW_ERR_UNSUPPORTED           # g * S > 1024
    assert _attn(_shape(N_pages=65536, T=65536 * 16)) == pw.PW_ERR_UNSUPPORTED
    assert _attn(_shape(N_pages=32769, T=32769 * 16)) == pw.PW_ERR_UNSUPPORTED
    assert _attn(_shape(S=-1)) == pw.PW_ERR_DIMS
    shp = _shape()
    need = pw._lib.pw_union_attention_workspace_bytes(ctypes.byref(shp), 8)
    assert need == 2 * 64 * 1 * 64 * 64 + 1024     # K and V tiles, then 16 bytes per page
    f = pw._lib.pw_union_attention
    assert f(ctypes.byref(shp), *[FAKE] * 6, 8, FAKE, None, need, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(shp), *[FAKE] * 6, 8, FAKE, FAKE, need - 1, None) == pw.PW_ERR_WORKSPACE
    assert f(ctypes.byref(shp), *[FAKE] * 6, 8, FAKE, ctypes.c_void_p(0x1010), need, None) == pw.PW_ERR_DIMS


def test_head_range_validation():
    f = pw._lib.pw_union_attention_heads
    shp = _shape(H_kv=2, H_q=8)
    need = pw._lib.pw_union_attention_workspace_bytes(ctypes.byref(shp), 8)
    ws = ctypes.c_void_p(0x100000)
    for h0, hc in [(-1, 1), (0, 0), (1, 2), (2, 1)]:
        assert f(ctypes.byref(shp), *[FAKE] * 6, 8, h0, hc, FAKE, ws, need, None) == pw.PW_ERR_DIMS
    assert f(ctypes.byref(shp), *[FAKE] * 6, 8, 0, 1, FAKE, ws, need - 1, None) == pw.PW_ERR_WORKSPACE
    assert f(ctypes.byref(shp), *[FAKE] * 5, None, 8, 0, 1, FAKE, ws, need, None) == pw.PW_ERR_NULL


def test_dense_union_validation():
    shp = _shape()
    f = pw._lib.pw_dense_union_ref
    assert f(ctypes.byref(shp), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(_shape(D=80)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == pw.PW_ERR_UNSUPPORTED
    need = pw._lib.pw_dense_union_ref_workspace_bytes(ctypes.byref(shp))
    if need > 0:
        assert f(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == pw.PW_ERR_WORKSPACE
        assert f(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None) == pw.PW_ERR_NULL


def test_page_pairs_validation():
    f = pw._lib.pw_page_pairs
    shp = _shape()
    need = pw._lib.pw_page_pairs_workspace_bytes(ctypes.byref(shp))
    assert need >= shp.H_kv * shp.N_pages * shp.N_pages * 4       # the co-selection counts
    assert f(ctypes.byref(shp), None, FAKE, FAKE, need, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(shp), FAKE, None, FAKE, need, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(shp), FAKE, FAKE, None, need, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(shp), FAKE, FAKE, FAKE, need - 1, None) == pw.PW_ERR_WORKSPACE
    assert f(ctypes.byref(shp), FAKE, FAKE, ctypes.c_void_p(0x1010), need, None) == pw.PW_ERR_DIMS
    big = _shape(T=4096 * 16, N_pages=4096)
    assert f(ctypes.byref(big), FAKE, FAKE, FAKE, 1 << 40, None) == pw.PW_ERR_UNSUPPORTED
    g = pw._lib.pw_dense_union_paired
    need = pw._lib.pw_dense_union_ref_workspace_bytes(ctypes.byref(shp))
    assert g(ctypes.byref(shp), *[FAKE] * 5, None, FAKE, FAKE, need, None) == pw.PW_ERR_NULL
    assert g(ctypes.byref(shp), *[FAKE] * 7, FAKE, need - 1, None) == pw.PW_ERR_WORKSPACE
    assert g(ctypes.byref(big), *[FAKE] * 7, FAKE, 1 << 40, None) == pw.PW_ERR_UNSUPPORTED


def test_select_validation():
    f = pw._lib.pw_select
    shp = _shape(S=8)
    need = pw._lib.pw_select_workspace_bytes(ctypes.byref(shp))
    assert need == 2 * (1024 * 64 * 2) + 2 * (64 * 64 * 2) + 1024 * 64 * 4   # bf16 hi/lo qs, C; fp32 scores
    assert f(ctypes.byref(shp), None, FAKE, FAKE, 2, FAKE, FAKE, need, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(shp), FAKE, FAKE, FAKE, 0, FAKE, FAKE, need, None) == pw.PW_ERR_UNSUPPORTED
    assert f(ctypes.byref(shp), FAKE, FAKE, FAKE, 8, FAKE, FAKE, need, None) == pw.PW_ERR_UNSUPPORTED
    assert f(ctypes.byref(_shape(D=96)), FAKE, FAKE, FAKE, 2, FAKE, FAKE, need, None) == pw.PW_ERR_UNSUPPORTED
    big = _shape(T=2048 * 16, N_pages=2048)
    assert f(ctypes.byref(big), FAKE, FAKE, FAKE, 2, FAKE, FAKE, 1 << 40, None) == pw.PW_ERR_UNSUPPORTED
    assert f(ctypes.byref(shp), FAKE, FAKE, FAKE, 2, FAKE, FAKE, need - 1, None) == pw.PW_ERR_WORKSPACE
    assert f(ctypes.byref(shp), FAKE, FAKE, FAKE, 2, FAKE, None, need, None) == pw.PW_ERR_NULL


def test_check_ids_validation():
    f = pw._lib.pw_check_ids
    shp = _shape(H_kv=2, H_q=4)
    need = pw._lib.pw_check_ids_workspace_bytes(ctypes.byref(shp))
    assert need == (2 * 1024 + 31) // 32 * 4
    assert f(ctypes.byref(shp), None, FAKE, FAKE, need, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(shp), FAKE, FAKE, None, need, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(shp), FAKE, FAKE, FAKE, need - 1, None) == pw.PW_ERR_WORKSPACE


def test_binding_refuses_host_tensors():
    import torch
    shp = _shape()
    with pytest.raises(TypeError):
        pw.pw_group(shp, torch.zeros((1, 1024, 8), dtype=torch.int32), 32, 8)

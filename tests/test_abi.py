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
    assert pw._lib.pw_abi_version() == 4


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
    assert _group(_shape(), W=36, g=8) == pw.PW_ERR_UNSUPPORTED      # W % g != 0
    assert b"multiple of g" in pw._lib.pw_last_error()
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


def test_tiled_validation():
    shp = _shape()
    need = pw._lib.pw_union_attention_workspace_bytes(ctypes.byref(shp), 8)
    ws = ctypes.c_void_p(0x100000)
    t = pw._lib.pw_tile_kv
    assert t(None, FAKE, FAKE, FAKE, ws, need, None) == pw.PW_ERR_NULL
    assert t(ctypes.byref(shp), None, FAKE, FAKE, ws, need, None) == pw.PW_ERR_NULL
    assert t(ctypes.byref(shp), FAKE, FAKE, FAKE, None, need, None) == pw.PW_ERR_NULL
    assert t(ctypes.byref(shp), FAKE, FAKE, FAKE, ws, need - 1, None) == pw.PW_ERR_WORKSPACE
    assert t(ctypes.byref(shp), FAKE, FAKE, FAKE, ctypes.c_void_p(0x100010), need, None) == pw.PW_ERR_DIMS
    assert t(ctypes.byref(_shape(D=96)), FAKE, FAKE, FAKE, ws, need, None) == pw.PW_ERR_UNSUPPORTED
    a = pw._lib.pw_union_attention_tiled
    assert a(ctypes.byref(shp), None, FAKE, FAKE, 8, FAKE, ws, need, None) == pw.PW_ERR_NULL
    assert a(ctypes.byref(shp), FAKE, FAKE, FAKE, 8, None, ws, need, None) == pw.PW_ERR_NULL
    assert a(ctypes.byref(shp), FAKE, FAKE, FAKE, 17, FAKE, ws, need, None) == pw.PW_ERR_UNSUPPORTED
    assert a(ctypes.byref(shp), FAKE, FAKE, FAKE, 8, FAKE, ws, need - 1, None) == pw.PW_ERR_WORKSPACE
    # a tiled copy beyond the 2^31-byte reach of the kernels' 32-bit page offsets
    big = _shape(T=4096 * 16, N_pages=4096, H_q=64, H_kv=64, D=128)
    assert t(ctypes.byref(big), FAKE, FAKE, FAKE, ws, 1 << 40, None) == pw.PW_ERR_UNSUPPORTED
    assert b"2 GiB" in pw._lib.pw_last_error()


def test_ordered_validation():
    # pw_group_ordered: the pw_group checks, then the order output and the union-size workspace
    shp = _shape()
    need = pw._lib.pw_group_ordered_workspace_bytes(ctypes.byref(shp), 32, 8)
    assert need == 1 * (1024 // 8) * 4
    ws = ctypes.c_void_p(0x100000)
    go = pw._lib.pw_group_ordered
    assert go(None, FAKE, 32, 8, FAKE, FAKE, ws, need, None) == pw.PW_ERR_NULL
    assert go(ctypes.byref(shp), FAKE, 36, 8, FAKE, FAKE, ws, need, None) == pw.PW_ERR_UNSUPPORTED
    assert go(ctypes.byref(shp), FAKE, 32, 8, FAKE, None, ws, need, None) == pw.PW_ERR_NULL
    assert go(ctypes.byref(shp), FAKE, 32, 8, FAKE, FAKE, None, need, None) == pw.PW_ERR_NULL
    assert go(ctypes.byref(shp), FAKE, 32, 8, FAKE, FAKE, ws, need - 1, None) == pw.PW_ERR_WORKSPACE
    assert go(ctypes.byref(shp), FAKE, 32, 8, FAKE, FAKE, ctypes.c_void_p(0x100002), need, None) == pw.PW_ERR_DIMS
    assert go(ctypes.byref(shp), FAKE, 32, 8, FAKE, ctypes.c_void_p(0x1001), ws, need, None) == pw.PW_ERR_DIMS
    # pw_union_attention_tiled_ordered: the tiled checks plus a required order
    wneed = pw._lib.pw_union_attention_workspace_bytes(ctypes.byref(shp), 8)
    a = pw._lib.pw_union_attention_tiled_ordered
    assert a(ctypes.byref(shp), FAKE, FAKE, FAKE, None, 8, FAKE, ws, wneed, None) == pw.PW_ERR_NULL
    assert a(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, 17, FAKE, ws, wneed, None) == pw.PW_ERR_UNSUPPORTED
    assert a(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, 8, FAKE, ws, wneed - 1, None) == pw.PW_ERR_WORKSPACE


def test_noalloc_validation():
    # host-side checks of the no-alloc entry point, before any HIP call: required pointers,
    # the support set, and shapes whose re-tiled K/V exceeds the fixed scratch
    f = pw._lib.pw_union_attention_noalloc
    shp = _shape()
    assert f(ctypes.byref(shp), None, *[FAKE] * 5, 8, FAKE, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(shp), *[FAKE] * 6, 8, None, None) == pw.PW_ERR_NULL
    assert f(ctypes.byref(shp), *[FAKE] * 6, 17, FAKE, None) == pw.PW_ERR_UNSUPPORTED
    big = _shape(T=2048 * 64, N_pages=2048, P=64, H_q=32, H_kv=8, D=128)   # 268 MB re-tiled
    assert pw._lib.pw_union_attention_workspace_bytes(ctypes.byref(big), 8) > pw.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), *[FAKE] * 6, 8, FAKE, None) == pw.PW_ERR_UNSUPPORTED
    assert b"no-alloc scratch" in pw._lib.pw_last_error()
    fits = _shape(T=1024 * 64, N_pages=1024, P=64, H_q=32, H_kv=8, D=128)  # the 64K layer: 134 MB
    assert pw._lib.pw_union_attention_workspace_bytes(ctypes.byref(fits), 8) <= pw.NOALLOC_SCRATCH_BYTES


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
    # the pair-mode kernel reads the same re-tiled copy: rejected beyond 2^31 bytes
    big = _shape(T=4096 * 16, N_pages=4096, H_q=64, H_kv=64, D=128)
    assert f(ctypes.byref(big), *[FAKE] * 7, 1 << 40, None) == pw.PW_ERR_UNSUPPORTED
    assert b"2 GiB" in pw._lib.pw_last_error()
    big2 = _shape(T=2048 * 16, N_pages=2048, H_q=128, H_kv=128, D=128)
    assert pw._lib.pw_dense_union_paired(ctypes.byref(big2), *[FAKE] * 8, 1 << 40, None) == pw.PW_ERR_UNSUPPORTED
    assert b"2 GiB" in pw._lib.pw_last_error()
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


def test_alignment_validation():
    # misaligned pointers are refused before any HIP call, naming the argument
    odd16, odd4 = ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1002)
    shp = _shape()                                      # S = 8: selection rows read 16 B at a time
    for i, name in [(0, b"Q"), (1, b"K_fp8"), (2, b"V_fp8"), (6, b"O")]:
        ptrs = [FAKE] * 7
        ptrs[i] = odd16
        assert _attn(shp, ptrs=ptrs) == pw.PW_ERR_DIMS
        assert name in pw._lib.pw_last_error()
    for i, name in [(3, b"scales"), (5, b"query_ids")]:
        ptrs = [FAKE] * 7
        ptrs[i] = odd4
        assert _attn(shp, ptrs=ptrs) == pw.PW_ERR_DIMS
        assert name in pw._lib.pw_last_error()
    ptrs = [FAKE] * 7
    ptrs[4] = odd16
    assert _attn(shp, ptrs=ptrs) == pw.PW_ERR_DIMS          # sel_pages, S a multiple of 4
    assert _group(shp, sel=odd16) == pw.PW_ERR_DIMS
    # S = 6: 4-byte alignment suffices (pw_group_ordered then stops at the missing group_order)
    assert pw._lib.pw_group_ordered(ctypes.byref(_shape(S=6)), odd16, 32, 8, FAKE, None, FAKE,
                                    1 << 20, None) == pw.PW_ERR_NULL
    assert _group(_shape(S=6), sel=odd4) == pw.PW_ERR_DIMS
    assert _group(shp, ids=odd4) == pw.PW_ERR_DIMS
    assert pw._lib.pw_tile_kv(ctypes.byref(shp), FAKE, odd16, FAKE, FAKE, 1 << 30, None) == pw.PW_ERR_DIMS
    assert pw._lib.pw_union_attention_tiled_fp8qp(ctypes.byref(shp), FAKE, FAKE, FAKE, odd4, 8,
                                                  FAKE, FAKE, 1 << 30, None) == pw.PW_ERR_DIMS
    assert b"group_order" in pw._lib.pw_last_error()
    assert pw._lib.pw_page_pairs(ctypes.byref(shp), FAKE, odd4, FAKE, 1 << 30, None) == pw.PW_ERR_DIMS
    assert b"pairs" in pw._lib.pw_last_error()


def test_header_is_plain_c_and_links(tmp_path):
    # the boundary needs nothing but C: the header compiles as C99 and as C++, and a C program
    # links the library and gets statuses back (validation only; no HIP call is made)
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    inc = os.path.join(root, "include")
    src = tmp_path / "use.c"
    src.write_text(
        '#include <stdio.h>\n#include "pageweaver.h"\n'
        "int main(void) {\n"
        "  pw_shape s = {1024, 4, 1, 64, 16, 64, 8};\n"
        "  int32_t ids[1];\n"
        "  if (pw_abi_version() != PW_ABI_VERSION) return 1;\n"
        "  if (pw_group(NULL, NULL, 32, 8, ids, NULL, 0, NULL) != PW_ERR_NULL) return 2;\n"
        "  if (pw_group(&s, NULL, 32, 8, ids, NULL, 0, NULL) != PW_ERR_NULL) return 3;\n"
        "  if (pw_union_attention_workspace_bytes(&s, 8) == 0) return 4;\n"
        '  printf("%s\\n", pw_status_string(PW_ERR_DIMS));\n'
        "  return 0;\n}\n")
    for cmd in (["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-x", "c",
                 "-I", inc, os.path.join(inc, "pageweaver.h")],
                ["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-x", "c++",
                 "-I", inc, os.path.join(inc, "pageweaver.h")]):
        subprocess.run(cmd, check=True, capture_output=True, text=True)
    exe = tmp_path / "use"
    libdir = os.path.dirname(pw.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", inc, str(src), "-o", str(exe),
                    "-L", libdir, "-l:" + os.path.basename(pw.LIB_PATH),
                    "-Wl,-rpath," + libdir], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.strip() == "invalid dimensions"

"""Thin ctypes binding of libpageweaver (argument marshalling only).

Every step of the path runs in the HIP kernels behind the C ABI declared in
include/pageweaver.h; this module only checks tensor dtypes, shapes and
devices, passes raw device pointers and the current HIP stream, and turns a
non-OK status into an exception.  Importing it fails loudly when the library
has not been built: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAGEWEAVER_LIB may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("PAGEWEAVER_LIB") or os.path.join(_HERE, "libpageweaver.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "pageweaver.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m query_union_paged_amd.build` "
        "(hipcc, gfx950). The path has no CPU or PyTorch fallback.")

_lib = ctypes.CDLL(LIB_PATH)

PW_OK, PW_ERR_NULL, PW_ERR_DIMS, PW_ERR_UNSUPPORTED, PW_ERR_WORKSPACE, PW_ERR_HIP = 0, -1, -2, -3, -4, -5


class PWShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H_q", "H_kv", "D", "P", "N_pages", "S")]


class PWError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.pw_last_error().decode()
        super().__init__(f"{where}: {_lib.pw_status_string(status).decode()} ({status}): {detail}")


_vp, _sz, _i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
_SHP = ctypes.POINTER(PWShape)
_SIGS = {
    "pw_group_workspace_bytes": (_sz, [_SHP, _i32, _i32]),
    "pw_group": (_i32, [_SHP, _vp, _i32, _i32, _vp, _vp, _sz, _vp]),
    "pw_group_ordered_workspace_bytes": (_sz, [_SHP, _i32, _i32]),
    "pw_group_ordered": (_i32, [_SHP, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "pw_union_attention_workspace_bytes": (_sz, [_SHP, _i32]),
    "pw_union_attention": (_i32, [_SHP, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "pw_union_attention_heads": (_i32, [_SHP, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp,
                                        _vp, _sz, _vp]),
    "pw_union_attention_noalloc": (_i32, [_SHP, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp]),
    "pw_tile_kv": (_i32, [_SHP, _vp, _vp, _vp, _vp, _sz, _vp]),
    "pw_union_attention_tiled": (_i32, [_SHP, _vp, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "pw_union_attention_tiled_ordered": (_i32, [_SHP, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _sz,
                                                _vp]),
    "pw_union_attention_tiled_fp8qp": (_i32, [_SHP, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _sz,
                                              _vp]),
    "pw_check_ids_workspace_bytes": (_sz, [_SHP]),
    "pw_check_ids": (_i32, [_SHP, _vp, _vp, _vp, _sz, _vp]),
    "pw_select_workspace_bytes": (_sz, [_SHP]),
    "pw_select": (_i32, [_SHP, _vp, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "pw_dense_union_ref_workspace_bytes": (_sz, [_SHP]),
    "pw_dense_union_ref": (_i32, [_SHP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "pw_dense_union_paired": (_i32, [_SHP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "pw_page_pairs_workspace_bytes": (_sz, [_SHP]),
    "pw_page_pairs": (_i32, [_SHP, _vp, _vp, _vp, _sz, _vp]),
    "pw_status_string": (ctypes.c_char_p, [_i32]),
    "pw_last_error": (ctypes.c_char_p, []),
    "pw_abi_version": (_i32, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype, _fn.argtypes = _res, _args


def header_functions():
    """Names of the functions include/pageweaver.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(pw_\w+)\s*\(", text, re.M)))


def shape(T, H_q, H_kv, D, P, N_pages, S) -> PWShape:
    return PWShape(T, H_q, H_kv, D, P, N_pages, S)


def shape_of(q: torch.Tensor, k_fp8: torch.Tensor, sel_pages: torch.Tensor) -> PWShape:
    T, H_q, D = q.shape
    N, H_kv, P, _ = k_fp8.shape
    return PWShape(T, H_q, H_kv, D, P, N, sel_pages.shape[2])


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, name: str, dtypes, shape_=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape_ is not None and tuple(t.shape) != tuple(shape_):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape_)}")
    return t.data_ptr()


_U8 = (torch.uint8, torch.float8_e4m3fn)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _check(status: int, where: str):
    if status != PW_OK:
        raise PWError(status, where)


def pw_group(shp: PWShape, sel_pages: torch.Tensor, W: int, g: int,
             query_ids: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    sel = _dev(sel_pages, "sel_pages", (torch.int32,), (shp.H_kv, shp.T, shp.S))
    if query_ids is None:
        query_ids = torch.empty((shp.H_kv, shp.T), dtype=torch.int32, device=sel_pages.device)
    ids = _dev(query_ids, "query_ids", (torch.int32,), (shp.H_kv, shp.T))
    _check(_lib.pw_group(ctypes.byref(shp), sel, W, g, ids, None, 0, _stream(stream)), "pw_group")
    return query_ids


def pw_group_ordered_workspace_bytes(shp: PWShape, W: int, g: int) -> int:
    return int(_lib.pw_group_ordered_workspace_bytes(ctypes.byref(shp), W, g))


def pw_group_ordered(shp: PWShape, sel_pages: torch.Tensor, W: int, g: int,
                     query_ids: Optional[torch.Tensor] = None,
                     group_order: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None):
    """pw_group plus an execution order of each KV head's groups (blocks of the groups one XCD
    runs at once, each block by ascending union size); returns (query_ids, group_order)."""
    sel = _dev(sel_pages, "sel_pages", (torch.int32,), (shp.H_kv, shp.T, shp.S))
    ng = (shp.T + g - 1) // g if g > 0 else 0
    if query_ids is None:
        query_ids = torch.empty((shp.H_kv, shp.T), dtype=torch.int32, device=sel_pages.device)
    if group_order is None:
        group_order = torch.empty((shp.H_kv, ng), dtype=torch.int32, device=sel_pages.device)
    if workspace is None:
        workspace = torch.empty(max(1, int(_lib.pw_group_ordered_workspace_bytes(
            ctypes.byref(shp), W, g))), dtype=torch.uint8, device=sel_pages.device)
    ids = _dev(query_ids, "query_ids", (torch.int32,), (shp.H_kv, shp.T))
    order = _dev(group_order, "group_order", (torch.int32,), (shp.H_kv, ng))
    ws = _dev(workspace, "workspace", (torch.uint8,))
    _check(_lib.pw_group_ordered(ctypes.byref(shp), sel, W, g, ids, order, ws, workspace.numel(),
                                 _stream(stream)), "pw_group_ordered")
    return query_ids, group_order


def pw_union_attention_workspace_bytes(shp: PWShape, g: int = 8) -> int:
    return int(_lib.pw_union_attention_workspace_bytes(ctypes.byref(shp), g))


def pw_union_attention(shp: PWShape, Q, K_fp8, V_fp8, scales, sel_pages, query_ids, g: int,
                       O: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None, heads: Optional[tuple] = None) -> torch.Tensor:
    """Query-union attention; `heads` = (h_begin, h_count) restricts the call to those KV heads
    (pw_union_attention_heads; the other rows of O are left untouched)."""
    T, Hq, Hkv, D, P, N, S = shp.T, shp.H_q, shp.H_kv, shp.D, shp.P, shp.N_pages, shp.S
    q = _dev(Q, "Q", _BF16, (T, Hq, D))
    k = _dev(K_fp8, "K_fp8", _U8, (N, Hkv, P, D))
    v = _dev(V_fp8, "V_fp8", _U8, (N, Hkv, P, D))
    sc = _dev(scales, "scales", (torch.float32,), (2, N, Hkv))
    sel = _dev(sel_pages, "sel_pages", (torch.int32,), (Hkv, T, S))
    ids = _dev(query_ids, "query_ids", (torch.int32,), (Hkv, T))
    if O is None:
        O = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=Q.device)
    o = _dev(O, "O", _BF16, (T, Hq, D))
    if workspace is None:
        workspace = torch.empty(pw_union_attention_workspace_bytes(shp, g), dtype=torch.uint8,
                                device=Q.device)
    ws = _dev(workspace, "workspace", (torch.uint8,))
    if heads is None:
        _check(_lib.pw_union_attention(ctypes.byref(shp), q, k, v, sc, sel, ids, g, o, ws,
                                       workspace.numel(), _stream(stream)), "pw_union_attention")
    else:
        _check(_lib.pw_union_attention_heads(ctypes.byref(shp), q, k, v, sc, sel, ids, g,
                                             int(heads[0]), int(heads[1]), o, ws,
                                             workspace.numel(), _stream(stream)),
               "pw_union_attention_heads")
    return O


NOALLOC_SCRATCH_BYTES = 160 << 20


def pw_union_attention_noalloc(shp: PWShape, Q, K_fp8, V_fp8, scales, sel_pages, query_ids,
                               g: int, O: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """pw_union_attention with the library's own device scratch instead of a workspace (for
    callers that cannot allocate: calls on one device share that scratch)."""
    T, Hq, Hkv, D, P, N, S = shp.T, shp.H_q, shp.H_kv, shp.D, shp.P, shp.N_pages, shp.S
    q = _dev(Q, "Q", _BF16, (T, Hq, D))
    k = _dev(K_fp8, "K_fp8", _U8, (N, Hkv, P, D))
    v = _dev(V_fp8, "V_fp8", _U8, (N, Hkv, P, D))
    sc = _dev(scales, "scales", (torch.float32,), (2, N, Hkv))
    sel = _dev(sel_pages, "sel_pages", (torch.int32,), (Hkv, T, S))
    ids = _dev(query_ids, "query_ids", (torch.int32,), (Hkv, T))
    if O is None:
        O = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=Q.device)
    o = _dev(O, "O", _BF16, (T, Hq, D))
    _check(_lib.pw_union_attention_noalloc(ctypes.byref(shp), q, k, v, sc, sel, ids, g, o,
                                           _stream(stream)), "pw_union_attention_noalloc")
    return O


def pw_tile_kv(shp: PWShape, K_fp8, V_fp8, scales, workspace: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Re-tile the FP8 K/V pages (and the per-page softmax factors) into a workspace for
    pw_union_attention_tiled."""
    N, Hkv, P, D = shp.N_pages, shp.H_kv, shp.P, shp.D
    k = _dev(K_fp8, "K_fp8", _U8, (N, Hkv, P, D))
    v = _dev(V_fp8, "V_fp8", _U8, (N, Hkv, P, D))
    sc = _dev(scales, "scales", (torch.float32,), (2, N, Hkv))
    if workspace is None:
        workspace = torch.empty(pw_union_attention_workspace_bytes(shp), dtype=torch.uint8,
                                device=K_fp8.device)
    ws = _dev(workspace, "workspace", (torch.uint8,))
    _check(_lib.pw_tile_kv(ctypes.byref(shp), k, v, sc, ws, workspace.numel(), _stream(stream)),
           "pw_tile_kv")
    return workspace


def pw_union_attention_tiled(shp: PWShape, Q, sel_pages, query_ids, g: int,
                             workspace: torch.Tensor, O: Optional[torch.Tensor] = None,
                             stream=None, group_order: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Union attention on a workspace that pw_tile_kv filled for the same K/V; with
    `group_order` (from pw_group_ordered) the groups run in that order
    (pw_union_attention_tiled_ordered)."""
    T, Hq, Hkv, D, S = shp.T, shp.H_q, shp.H_kv, shp.D, shp.S
    q = _dev(Q, "Q", _BF16, (T, Hq, D))
    sel = _dev(sel_pages, "sel_pages", (torch.int32,), (Hkv, T, S))
    ids = _dev(query_ids, "query_ids", (torch.int32,), (Hkv, T))
    if O is None:
        O = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=Q.device)
    o = _dev(O, "O", _BF16, (T, Hq, D))
    ws = _dev(workspace, "workspace", (torch.uint8,))
    if group_order is None:
        _check(_lib.pw_union_attention_tiled(ctypes.byref(shp), q, sel, ids, g, o, ws,
                                             workspace.numel(), _stream(stream)),
               "pw_union_attention_tiled")
    else:
        order = _dev(group_order, "group_order", (torch.int32,), (Hkv, (T + g - 1) // g))
        _check(_lib.pw_union_attention_tiled_ordered(ctypes.byref(shp), q, sel, ids, order, g, o,
                                                     ws, workspace.numel(), _stream(stream)),
               "pw_union_attention_tiled_ordered")
    return O


def pw_union_attention_tiled_fp8qp(shp: PWShape, Q, sel_pages, query_ids, g: int,
                                   workspace: torch.Tensor, O: Optional[torch.Tensor] = None,
                                   stream=None,
                                   group_order: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The lower-precision variant of pw_union_attention_tiled: Q and P rounded to e4m3fn per
    row, both products on the FP8 matrix cores (not within the exact path's tolerance)."""
    T, Hq, Hkv, D, S = shp.T, shp.H_q, shp.H_kv, shp.D, shp.S
    q = _dev(Q, "Q", _BF16, (T, Hq, D))
    sel = _dev(sel_pages, "sel_pages", (torch.int32,), (Hkv, T, S))
    ids = _dev(query_ids, "query_ids", (torch.int32,), (Hkv, T))
    if O is None:
        O = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=Q.device)
    o = _dev(O, "O", _BF16, (T, Hq, D))
    ws = _dev(workspace, "workspace", (torch.uint8,))
    order = (None if group_order is None else
             _dev(group_order, "group_order", (torch.int32,), (Hkv, (T + g - 1) // g)))
    _check(_lib.pw_union_attention_tiled_fp8qp(ctypes.byref(shp), q, sel, ids, order, g, o, ws,
                                               workspace.numel(), _stream(stream)),
           "pw_union_attention_tiled_fp8qp")
    return O


class HeadPipeline:
    """The complete call (search, then attention) with the search of later KV heads
    overlapping the attention of earlier ones: pw_group runs per chunk of `chunk` KV heads on
    an auxiliary stream, and pw_union_attention_heads of each chunk waits for its search on
    the caller's stream.  Only call ordering lives here (streams and events); every step is a
    library call.  Streams keep the default priority."""

    def __init__(self, shp: PWShape, chunk: int):
        if shp.H_kv % chunk:
            raise ValueError(f"chunk {chunk} does not divide H_kv = {shp.H_kv}")
        self.shp, self.chunk = shp, chunk
        G = shp.H_q // shp.H_kv
        self.sub = PWShape(shp.T, G * chunk, chunk, shp.D, shp.P, shp.N_pages, shp.S)
        self.aux = torch.cuda.Stream()
        self.done = [torch.cuda.Event() for _ in range(shp.H_kv // chunk)]

    def __call__(self, Q, K_fp8, V_fp8, scales, sel_pages, W: int, g: int,
                 query_ids: torch.Tensor, O: torch.Tensor, workspace: torch.Tensor):
        main = torch.cuda.current_stream()
        self.aux.wait_stream(main)              # inputs are written on the caller's stream
        c = self.chunk
        for k, h0 in enumerate(range(0, self.shp.H_kv, c)):
            pw_group(self.sub, sel_pages[h0:h0 + c], W, g, query_ids=query_ids[h0:h0 + c],
                     stream=self.aux)
            self.done[k].record(self.aux)
        for k, h0 in enumerate(range(0, self.shp.H_kv, c)):
            main.wait_event(self.done[k])
            pw_union_attention(self.shp, Q, K_fp8, V_fp8, scales, sel_pages, query_ids, g, O=O,
                               workspace=workspace, stream=main, heads=(h0, c))
        return O


def pw_check_ids(shp: PWShape, query_ids: torch.Tensor, stream=None) -> torch.Tensor:
    """Per KV head, the number of out-of-range or repeated IDs (all zero: permutations)."""
    ids = _dev(query_ids, "query_ids", (torch.int32,), (shp.H_kv, shp.T))
    bad = torch.empty((shp.H_kv,), dtype=torch.int32, device=query_ids.device)
    ws = torch.empty(int(_lib.pw_check_ids_workspace_bytes(ctypes.byref(shp))), dtype=torch.uint8,
                     device=query_ids.device)
    _check(_lib.pw_check_ids(ctypes.byref(shp), ids, bad.data_ptr(), ws.data_ptr(), ws.numel(),
                             _stream(stream)), "pw_check_ids")
    return bad


def pw_select_workspace_bytes(shp: PWShape) -> int:
    return int(_lib.pw_select_workspace_bytes(ctypes.byref(shp)))


def pw_select(shp: PWShape, Q, K_fp8, scales, n_local: int,
              sel_pages: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """Synthetic page selection (sink, n_local local pages, top pages by block key sums)."""
    N = shp.N_pages
    q = _dev(Q, "Q", _BF16, (shp.T, shp.H_q, shp.D))
    k = _dev(K_fp8, "K_fp8", _U8, (N, shp.H_kv, shp.P, shp.D))
    sc = _dev(scales, "scales", (torch.float32,), (2, N, shp.H_kv))
    if sel_pages is None:
        sel_pages = torch.empty((shp.H_kv, shp.T, shp.S), dtype=torch.int32, device=Q.device)
    sel = _dev(sel_pages, "sel_pages", (torch.int32,), (shp.H_kv, shp.T, shp.S))
    if workspace is None:
        workspace = torch.empty(pw_select_workspace_bytes(shp), dtype=torch.uint8, device=Q.device)
    ws = _dev(workspace, "workspace", (torch.uint8,))
    _check(_lib.pw_select(ctypes.byref(shp), q, k, sc, n_local, sel, ws, workspace.numel(),
                          _stream(stream)), "pw_select")
    return sel_pages


def pw_dense_union_ref_workspace_bytes(shp: PWShape) -> int:
    return int(_lib.pw_dense_union_ref_workspace_bytes(ctypes.byref(shp)))


def pw_dense_union_ref(shp: PWShape, Q, K_fp8, V_fp8, scales, sel_pages,
                       O: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None, pairs: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Direct KV-page union; adjacent pairs (2k, 2k+1), or `pairs` (int32 [H_kv][N][2], e.g.
    from pw_page_pairs) through pw_dense_union_paired."""
    T, Hq, Hkv, D, P, N, S = shp.T, shp.H_q, shp.H_kv, shp.D, shp.P, shp.N_pages, shp.S
    q = _dev(Q, "Q", _BF16, (T, Hq, D))
    k = _dev(K_fp8, "K_fp8", _U8, (N, Hkv, P, D))
    v = _dev(V_fp8, "V_fp8", _U8, (N, Hkv, P, D))
    sc = _dev(scales, "scales", (torch.float32,), (2, N, Hkv))
    sel = _dev(sel_pages, "sel_pages", (torch.int32,), (Hkv, T, S))
    if O is None:
        O = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=Q.device)
    o = _dev(O, "O", _BF16, (T, Hq, D))
    need = pw_dense_union_ref_workspace_bytes(shp)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    ws, nbytes = (0, 0) if workspace is None else (_dev(workspace, "workspace", (torch.uint8,)), workspace.numel())
    if pairs is None:
        _check(_lib.pw_dense_union_ref(ctypes.byref(shp), q, k, v, sc, sel, o, ws or None, nbytes,
                                       _stream(stream)), "pw_dense_union_ref")
    else:
        pr = _dev(pairs, "pairs", (torch.int32,), (Hkv, N, 2))
        _check(_lib.pw_dense_union_paired(ctypes.byref(shp), q, k, v, sc, sel, pr, o, ws or None,
                                          nbytes, _stream(stream)), "pw_dense_union_paired")
    return O


def pw_page_pairs_workspace_bytes(shp: PWShape) -> int:
    return int(_lib.pw_page_pairs_workspace_bytes(ctypes.byref(shp)))


def pw_page_pairs(shp: PWShape, sel_pages, pairs: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Affinity page pairs (greedy co-selection matching): int32 [H_kv][N_pages][2]."""
    sel = _dev(sel_pages, "sel_pages", (torch.int32,), (shp.H_kv, shp.T, shp.S))
    if pairs is None:
        pairs = torch.empty((shp.H_kv, shp.N_pages, 2), dtype=torch.int32, device=sel_pages.device)
    pr = _dev(pairs, "pairs", (torch.int32,), (shp.H_kv, shp.N_pages, 2))
    if workspace is None:
        workspace = torch.empty(pw_page_pairs_workspace_bytes(shp), dtype=torch.uint8,
                                device=sel_pages.device)
    ws = _dev(workspace, "workspace", (torch.uint8,))
    _check(_lib.pw_page_pairs(ctypes.byref(shp), sel, pr, ws, workspace.numel(), _stream(stream)),
           "pw_page_pairs")
    return pairs


def to_device(inputs: dict, device="cuda") -> dict:
    """Upload generator output (numpy, C-ABI layouts) as device tensors."""
    out = {}
    for key, arr in inputs.items():
        if key == "q_bits":
            t = torch.from_numpy(arr.view("int16")).view(torch.bfloat16)
        else:
            t = torch.from_numpy(arr)
        out[key] = t.to(device).contiguous()
    return out

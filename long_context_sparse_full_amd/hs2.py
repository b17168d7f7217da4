"""Python binding of libhs2.so (C ABI in include/hs2.h).

Argument marshalling only: every step of the hot path runs in the library's
gfx950 kernels.  Tensors are torch CUDA (HIP) tensors; each call passes
``tensor.data_ptr()`` and the current torch stream.  Importing this module
loads the library and raises ImportError when it has not been built (run
``python -m long_context_sparse_full_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhs2.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libhs2.so not found at {LIB_PATH}: build it with "
                      "`python -m long_context_sparse_full_amd.build` (no fallback exists)")
_lib = ctypes.CDLL(LIB_PATH)

F32, BF16, FP8_E4M3FN = 0, 1, 2
SEL_WINDOW_COMPETES = 1
SCALE_KEEP, SCALE_GROW = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4


class KVDesc(ctypes.Structure):
    """hs2_kv_desc (read-only cache view); hs2_kv_out_desc has the same layout."""
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
    ]


class KVOutDesc(KVDesc):
    """hs2_kv_out_desc: the writable view the bridge takes (same fields)."""


class PageTable(ctypes.Structure):
    """hs2_page_table: a paged cache's map from logical to pool pages."""
    _fields_ = [("table", ctypes.c_void_p), ("page_rows", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32),
                ("pool_pages", ctypes.c_int32)]


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_KVP = ctypes.POINTER(KVDesc)


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_abi_version = _sig("hs2_abi_version", ctypes.c_int, [])
_status_string = _sig("hs2_status_string", ctypes.c_char_p, [ctypes.c_int])
_last_error = _sig("hs2_last_error", ctypes.c_char_p, [])
_full_ws = _sig("hs2_full_attn_scores_workspace", _sz, [_KVP, _i32, _i32])
_full = _sig("hs2_full_attn_scores", ctypes.c_int,
             [_KVP, _vp, _i32, _i32, _i32, _i32, _vp, _f32, _vp, _vp, _vp, _vp, _sz, _vp])
_topk_ws = _sig("hs2_full_attn_topk_workspace", _sz, [_KVP, _i32, _i32])
_topk = _sig("hs2_full_attn_topk", ctypes.c_int,
             [_KVP, _vp, _i32, _i32, _i32, _i32, _vp, _f32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _sz,
              _vp])
_sel_ws = _sig("hs2_select_workspace", _sz, [_i32, _i32, _i32, _i32])
_sel_ws_for = _sig("hs2_select_workspace_for", _sz, [_i32, _i32, _i32, _i32, _i32])
_select = _sig("hs2_select_topk_window", ctypes.c_int,
               [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _sz, _vp])
_sparse = _sig("hs2_sparse_attn_gather", ctypes.c_int,
               [_KVP, _vp, _i32, _i32, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _vp])
_sparse_ws_size = _sig("hs2_sparse_attn_workspace", _sz, [_i32, _i32, _i32, _i32, _i32])
_sparse_ws = _sig("hs2_sparse_attn_gather_ws", ctypes.c_int,
                  [_KVP, _vp, _i32, _i32, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp])
_PTP = ctypes.POINTER(PageTable)
_topk_paged = _sig("hs2_full_attn_topk_paged", ctypes.c_int,
                   [_KVP, _PTP, _vp, _i32, _i32, _i32, _i32, _vp, _f32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                    _i32, _vp, _sz, _vp])
_sparse_paged = _sig("hs2_sparse_attn_gather_paged", ctypes.c_int,
                     [_KVP, _PTP, _vp, _i32, _i32, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp])
_sparse_static_limit = _sig("hs2_sparse_attn_static_limit", _sz, [])
_sparse_static = _sig("hs2_sparse_attn_gather_static", ctypes.c_int,
                      [_KVP, _vp, _i32, _i32, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _vp])
_bridge_layers_ws = _sig("hs2_kv_bridge_layers_workspace", _sz, [_i32, _i32, _i32, _i32])
_bridge_layers = _sig("hs2_kv_bridge_layers", ctypes.c_int,
                      [_vp, _i32, _i32, _vp, _i32, ctypes.POINTER(KVOutDesc), _i32, _i32, _i32, _vp, _sz, _vp])
_swa = _sig("hs2_swa_attn", ctypes.c_int, [_KVP, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _f32, _vp, _vp, _vp])
_bridge = _sig("hs2_kv_bridge", ctypes.c_int, [_vp, _i32, _i32, _vp, ctypes.POINTER(KVOutDesc), _i32, _i32, _vp])
_dbg_e4m3 = _sig("hs2_debug_e4m3fn_to_f32", ctypes.c_int, [_vp, _vp, _i32, _vp])
_dbg_stream = _sig("hs2_debug_stream_read", ctypes.c_int, [_vp, _sz, _vp, _i32, _vp])
_dbg_scanprobe = _sig("hs2_debug_scan_read_probe", ctypes.c_int, [_vp, _i32, _i32, _vp, _sz, _vp])
_t_enable = _sig("hs2_timing_enable", ctypes.c_int, [ctypes.c_int])
_t_reset = _sig("hs2_timing_reset", ctypes.c_int, [])
_t_collect = _sig("hs2_timing_collect", ctypes.c_int,
                  [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)])
_t_name = _sig("hs2_timing_kernel_name", ctypes.c_char_p, [_i32])

EXPORTED = [
    "hs2_abi_version", "hs2_status_string", "hs2_last_error", "hs2_full_attn_scores_workspace",
    "hs2_full_attn_scores", "hs2_full_attn_topk_workspace", "hs2_full_attn_topk", "hs2_select_workspace", "hs2_select_workspace_for", "hs2_select_topk_window",
    "hs2_sparse_attn_gather", "hs2_sparse_attn_workspace", "hs2_sparse_attn_gather_ws",
    "hs2_sparse_attn_static_limit", "hs2_sparse_attn_gather_static", "hs2_full_attn_topk_paged",
    "hs2_sparse_attn_gather_paged", "hs2_swa_attn", "hs2_kv_bridge",
    "hs2_kv_bridge_layers_workspace", "hs2_kv_bridge_layers", "hs2_debug_e4m3fn_to_f32", "hs2_debug_stream_read",
    "hs2_debug_scan_read_probe",
    "hs2_timing_enable",
    "hs2_timing_reset", "hs2_timing_collect", "hs2_timing_kernel_name",
]


class HS2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _last_error().decode(errors="replace")
        super().__init__(f"{where}: {_status_string(status).decode()} ({status}): {msg}")


def _check(status: int, where: str):
    if status != OK:
        raise HS2Error(status, where)


def abi_version() -> int:
    return int(_abi_version())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3FN
    raise TypeError(f"unsupported element type {t.dtype}")


def _dense(*tensors):
    """The C ABI takes dense row-major q/out/lse/scores/idx/count buffers."""
    for t in tensors:
        if t is not None and not t.is_contiguous():
            raise ValueError("q, out, lse, scores, idx, count and workspace tensors must be contiguous")


def kv_desc(k: torch.Tensor, v: torch.Tensor, k_scale=None, v_scale=None, cls=KVDesc) -> KVDesc:
    """Descriptor of a [B, Hkv, N, D] cache (uint8/float8_e4m3fn caches need scales)."""
    if k.shape != v.shape or k.dim() != 4 or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must be [B, Hkv, N, D] tensors of one dtype and layout")
    if k.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    B, H, N, D = k.shape
    code = _dtype_code(k)
    ks = vs = None
    if code == FP8_E4M3FN:
        if k_scale is None or v_scale is None:
            ks = vs = None
        else:
            _dense(k_scale, v_scale)
            ks = k_scale.data_ptr()
            vs = v_scale.data_ptr()
    return cls(k.data_ptr(), v.data_ptr(), code, k.stride(0), k.stride(1), k.stride(2), ks, vs, B, H, N, D)


def pool_desc(k_pool: torch.Tensor, v_pool: torch.Tensor, B: int, N: int, k_scale=None, v_scale=None) -> KVDesc:
    """Descriptor of a paged pool [Hkv, pool_rows, D] shared by B sequences of
    logical length N (stride_b 0; FP8 pools need per-(sequence, head) scales)."""
    if k_pool.shape != v_pool.shape or k_pool.dim() != 3 or k_pool.stride() != v_pool.stride() \
            or k_pool.dtype != v_pool.dtype:
        raise ValueError("k and v pools must be [Hkv, pool_rows, D] tensors of one dtype and layout")
    if k_pool.stride(2) != 1:
        raise ValueError("head_dim must be contiguous")
    H, _, D = k_pool.shape
    code = _dtype_code(k_pool)
    ks = vs = None
    if code == FP8_E4M3FN and k_scale is not None and v_scale is not None:
        _dense(k_scale, v_scale)
        ks, vs = k_scale.data_ptr(), v_scale.data_ptr()
    return KVDesc(k_pool.data_ptr(), v_pool.data_ptr(), code, 0, k_pool.stride(0), k_pool.stride(1), ks, vs, B, H,
                  N, D)


def page_table(table: torch.Tensor, page_rows: int, pool_pages: int) -> PageTable:
    """hs2_page_table over an int32 [B, pages_per_seq] device tensor."""
    if table.dtype != torch.int32 or table.dim() != 2 or not table.is_contiguous():
        raise ValueError("the page table must be a contiguous int32 [B, pages_per_seq] tensor")
    return PageTable(table.data_ptr(), int(page_rows), table.shape[1], int(pool_pages))


def full_attn_topk_paged(k_pool, v_pool, table, page_rows: int, N: int, q, q_pos0: int, topk: int, window: int,
                         max_sel: int | None = None, softmax_scale: float | None = None, k_scale=None, v_scale=None,
                         out=None, lse=None, scores=None, idx=None, count=None, workspace=None, want_lse: bool = True,
                         window_competes: bool = False, q_pos0_b=None):
    """full_attn_topk over a paged pool [Hkv, pool_rows, D]: `table` [B, pages_per_seq] int32 maps each
    sequence's pages of `page_rows` rows to pool pages.  Returns (out, lse, scores, idx, count)."""
    B, Tq, Hq, D = q.shape
    d = pool_desc(k_pool, v_pool, B, N, k_scale, v_scale)
    pt = page_table(table, page_rows, k_pool.shape[1] // page_rows)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if max_sel is None:
        max_sel = min(N, topk + window)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=dev)
    if scores is None:
        scores = torch.empty((B, Tq, d.Hkv, N), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((B, Tq, d.Hkv, max_sel), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B, Tq, d.Hkv), dtype=torch.int32, device=dev)
    need = int(_topk_ws(ctypes.byref(d), Tq, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dense(q, out, lse, scores, idx, count, workspace)
    st = _topk_paged(ctypes.byref(d), ctypes.byref(pt), q.data_ptr(), _dtype_code(q), Tq, Hq, int(q_pos0),
                     _qpos(q_pos0_b), float(softmax_scale), out.data_ptr(), None if lse is None else lse.data_ptr(),
                     scores.data_ptr(), int(topk), int(window), SEL_WINDOW_COMPETES if window_competes else 0,
                     idx.data_ptr(), count.data_ptr(), int(max_sel), workspace.data_ptr(), workspace.numel(),
                     _stream())
    _check(st, "hs2_full_attn_topk_paged")
    return out, lse, scores, idx, count


def sparse_attn_gather_paged(k_pool, v_pool, table, page_rows: int, N: int, q, idx, count, workspace,
                             softmax_scale: float | None = None, k_scale=None, v_scale=None, out=None, lse=None,
                             want_lse: bool = True):
    """sparse_attn_gather_ws over a paged pool (idx holds logical positions); `workspace` as there."""
    B, Tq, Hq, D = q.shape
    d = pool_desc(k_pool, v_pool, B, N, k_scale, v_scale)
    pt = page_table(table, page_rows, k_pool.shape[1] // page_rows)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    _dense(q, idx, count, out, lse, workspace)
    st = _sparse_paged(ctypes.byref(d), ctypes.byref(pt), q.data_ptr(), _dtype_code(q), Tq, Hq, float(softmax_scale),
                       idx.data_ptr(), count.data_ptr(), idx.shape[-1], out.data_ptr(),
                       None if lse is None else lse.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "hs2_sparse_attn_gather_paged")
    return out, lse


def full_attn_scores_workspace(k, v, Tq: int, Hq: int) -> int:
    d = kv_desc(k, v)
    return int(_full_ws(ctypes.byref(d), Tq, Hq))


def _qpos(q_pos0_b):
    if q_pos0_b is None:
        return None
    _dense(q_pos0_b)
    if q_pos0_b.dtype != torch.int32:
        raise TypeError("q_pos0_b must be an int32 device tensor [B]")
    return q_pos0_b.data_ptr()


def full_attn_scores(k, v, q, q_pos0: int, softmax_scale: float | None = None, k_scale=None, v_scale=None,
                     out=None, lse=None, scores=None, workspace=None, want_lse: bool = True, q_pos0_b=None):
    """Full-attention layer: returns (out [B,Tq,Hq,D], lse [B,Tq,Hq] or None, scores [B,Tq,Hkv,N])."""
    d = kv_desc(k, v, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=dev)
    if scores is None:
        scores = torch.empty((B, Tq, d.Hkv, d.N), dtype=torch.float32, device=dev)
    need = int(_full_ws(ctypes.byref(d), Tq, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dense(q, out, lse, scores, workspace)
    st = _full(ctypes.byref(d), q.data_ptr(), _dtype_code(q), Tq, Hq, int(q_pos0), _qpos(q_pos0_b), float(softmax_scale),
               out.data_ptr(), None if lse is None else lse.data_ptr(), scores.data_ptr(),
               workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "hs2_full_attn_scores")
    return out, lse, scores


def full_attn_topk_workspace(k, v, Tq: int, Hq: int) -> int:
    d = kv_desc(k, v)
    return int(_topk_ws(ctypes.byref(d), Tq, Hq))


def full_attn_topk(k, v, q, q_pos0: int, topk: int, window: int, max_sel: int | None = None,
                   softmax_scale: float | None = None, k_scale=None, v_scale=None, out=None, lse=None, scores=None,
                   idx=None, count=None, workspace=None, want_lse: bool = True, window_competes: bool = False,
                   q_pos0_b=None):
    """Full layer + token top-k with forced window in one call (window_competes:
    the window takes no budget of its own; see hs2.h).
    Returns (out, lse, scores, idx [B,Tq,Hkv,max_sel] int32, count [B,Tq,Hkv] int32)."""
    d = kv_desc(k, v, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if max_sel is None:
        max_sel = min(d.N, topk + window)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=dev)
    if scores is None:
        scores = torch.empty((B, Tq, d.Hkv, d.N), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((B, Tq, d.Hkv, max_sel), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B, Tq, d.Hkv), dtype=torch.int32, device=dev)
    need = int(_topk_ws(ctypes.byref(d), Tq, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dense(q, out, lse, scores, idx, count, workspace)
    st = _topk(ctypes.byref(d), q.data_ptr(), _dtype_code(q), Tq, Hq, int(q_pos0), _qpos(q_pos0_b), float(softmax_scale),
               out.data_ptr(), None if lse is None else lse.data_ptr(), scores.data_ptr(), int(topk), int(window),
               SEL_WINDOW_COMPETES if window_competes else 0, idx.data_ptr(), count.data_ptr(), int(max_sel), workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "hs2_full_attn_topk")
    return out, lse, scores, idx, count


def select_workspace(B, Tq, Hkv, N, block_size: int | None = None) -> int:
    if block_size is None:
        return int(_sel_ws(B, Tq, Hkv, N))
    return int(_sel_ws_for(B, Tq, Hkv, N, block_size))


def select_topk_window(scores, q_pos0: int, k: int, window: int, block_size: int = 1, max_sel: int | None = None,
                       idx=None, count=None, workspace=None, window_competes: bool = False, q_pos0_b=None):
    """Top-k (token or block) + forced window: returns (idx int32, count int32)."""
    B, Tq, Hkv, N = scores.shape
    if max_sel is None:
        max_sel = min(N, k * block_size + window)
    dev = scores.device
    if idx is None:
        idx = torch.empty((B, Tq, Hkv, max_sel), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B, Tq, Hkv), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(select_workspace(B, Tq, Hkv, N, block_size), 256), dtype=torch.uint8, device=dev)
    _dense(scores, idx, count, workspace)
    st = _select(scores.data_ptr(), B, Tq, Hkv, N, int(q_pos0), _qpos(q_pos0_b), int(k), int(window), int(block_size),
                 SEL_WINDOW_COMPETES if window_competes else 0, idx.data_ptr(), count.data_ptr(), int(max_sel), workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "hs2_select_topk_window")
    return idx, count


def sparse_attn_gather(k, v, q, idx, count, softmax_scale: float | None = None, k_scale=None, v_scale=None,
                       out=None, lse=None, want_lse: bool = True):
    """Sparse layer over the shared index list: returns (out, lse or None)."""
    d = kv_desc(k, v, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    _dense(q, idx, count, out, lse)
    st = _sparse(ctypes.byref(d), q.data_ptr(), _dtype_code(q), Tq, Hq, float(softmax_scale), idx.data_ptr(),
                 count.data_ptr(), idx.shape[-1], out.data_ptr(), None if lse is None else lse.data_ptr(), _stream())
    _check(st, "hs2_sparse_attn_gather")
    return out, lse


def sparse_attn_workspace(B, Tq, Hkv, D, max_sel) -> int:
    return int(_sparse_ws_size(B, Tq, Hkv, D, max_sel))


def sparse_attn_gather_ws(k, v, q, idx, count, workspace, softmax_scale: float | None = None, k_scale=None,
                          v_scale=None, out=None, lse=None, want_lse: bool = True):
    """Sparse layer, split over list slices; `workspace` must start zero-filled (calls keep it so)."""
    d = kv_desc(k, v, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    _dense(q, idx, count, out, lse, workspace)
    st = _sparse_ws(ctypes.byref(d), q.data_ptr(), _dtype_code(q), Tq, Hq, float(softmax_scale), idx.data_ptr(),
                    count.data_ptr(), idx.shape[-1], out.data_ptr(), None if lse is None else lse.data_ptr(),
                    workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "hs2_sparse_attn_gather_ws")
    return out, lse


def sparse_attn_static_limit() -> int:
    return int(_sparse_static_limit())


def sparse_attn_gather_static(k, v, q, idx, count, softmax_scale: float | None = None, k_scale=None, v_scale=None,
                              out=None, lse=None, want_lse: bool = True):
    """Sparse layer, split over list slices, with the library's static scratch
    (the call allocates nothing; calls on one GPU must not overlap)."""
    d = kv_desc(k, v, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    _dense(q, idx, count, out, lse)
    st = _sparse_static(ctypes.byref(d), q.data_ptr(), _dtype_code(q), Tq, Hq, float(softmax_scale), idx.data_ptr(),
                        count.data_ptr(), idx.shape[-1], out.data_ptr(), None if lse is None else lse.data_ptr(),
                        _stream())
    _check(st, "hs2_sparse_attn_gather_static")
    return out, lse


def swa_attn(k, v, q, q_pos0: int, window: int, softmax_scale: float | None = None, k_scale=None, v_scale=None,
             out=None, lse=None, want_lse: bool = True, q_pos0_b=None):
    """Sliding-window attention: query t attends to [q_pos0 + t - window + 1, q_pos0 + t]."""
    d = kv_desc(k, v, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    _dense(q, out, lse)
    st = _swa(ctypes.byref(d), q.data_ptr(), _dtype_code(q), Tq, Hq, int(q_pos0), _qpos(q_pos0_b), int(window),
              float(softmax_scale),
              out.data_ptr(), None if lse is None else lse.data_ptr(), _stream())
    _check(st, "hs2_swa_attn")
    return out, lse


def kv_bridge(hidden, w_kv, k_cache, v_cache, batch_index: int, pos0: int, k_scale=None, v_scale=None):
    """Project bf16 hidden states [T, d_model] with w_kv [d_model, 2*Hkv*D] into the cache rows
    (bf16 cache, or E4M3FN cache with its per-(b, head) scales)."""
    d = kv_desc(k_cache, v_cache, k_scale, v_scale, cls=KVOutDesc)
    T, dm = hidden.shape
    _dense(hidden, w_kv)
    st = _bridge(hidden.data_ptr(), T, dm, w_kv.data_ptr(), ctypes.byref(d), int(batch_index), int(pos0), _stream())
    _check(st, "hs2_kv_bridge")


def kv_bridge_layers(hidden, w_kv, caches, batch_index: int, pos0: int, grow: bool = False, workspace=None):
    """Bridge of L layers from one hidden state [T, d_model]: w_kv [L, d_model, 2*Hkv*D] (bf16, contiguous),
    caches a list of L tuples (k, v) or (k, v, k_scale, v_scale); grow=True maintains FP8 scales."""
    L = len(caches)
    descs = (KVOutDesc * L)(*[kv_desc(*c, cls=KVOutDesc) if len(c) == 4 else kv_desc(c[0], c[1], cls=KVOutDesc)
                              for c in caches])
    T, dm = hidden.shape
    _dense(hidden, w_kv)
    d0 = descs[0]
    if workspace is None:
        need = int(_bridge_layers_ws(L, T, d0.Hkv, d0.D))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=hidden.device)
    st = _bridge_layers(hidden.data_ptr(), T, dm, w_kv.data_ptr(), L, descs, int(batch_index), int(pos0),
                        SCALE_GROW if grow else SCALE_KEEP, workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "hs2_kv_bridge_layers")


def debug_e4m3fn_to_f32(codes: torch.Tensor) -> torch.Tensor:
    out = torch.empty(codes.numel(), dtype=torch.float32, device=codes.device)
    _check(_dbg_e4m3(codes.data_ptr(), out.data_ptr(), codes.numel(), _stream()), "hs2_debug_e4m3fn_to_f32")
    return out


def debug_stream_read(buf: torch.Tensor, blocks: int = 2048) -> torch.Tensor:
    """Read every byte of buf once (streaming probe); returns the per-thread xor words."""
    out = torch.empty(blocks * 256, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(_dbg_stream(buf.data_ptr(), nbytes - nbytes % 16, out.data_ptr(), blocks, _stream()),
           "hs2_debug_stream_read")
    return out


def debug_scan_read_probe(k, v, Hq: int, with_codes: bool, k_scale=None, v_scale=None, workspace=None):
    """The decode scan's read pattern over the cache with its arithmetic replaced by an xor
    (with_codes: plus its code stores); returns the scratch workspace."""
    d = kv_desc(k, v, k_scale, v_scale)
    need = int(_full_ws(ctypes.byref(d), 1, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=k.device)
    _dense(workspace)
    _check(_dbg_scanprobe(ctypes.byref(d), int(Hq), int(bool(with_codes)), workspace.data_ptr(), workspace.numel(),
                          _stream()), "hs2_debug_scan_read_probe")
    return workspace


def timing_enable(on: bool = True):
    _check(_t_enable(int(bool(on))), "hs2_timing_enable")


def timing_reset():
    _check(_t_reset(), "hs2_timing_reset")


def timing_collect(name: str):
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    _check(_t_collect(name.encode(), ctypes.byref(ms), ctypes.byref(n)), "hs2_timing_collect")
    return ms.value, n.value


def timing_kernel_names():
    out, i = [], 0
    while True:
        s = _t_name(i)
        if s is None:
            return out
        out.append(s.decode())
        i += 1


def raw_call(name: str):
    """The underlying ctypes function of an exported symbol (for tests of the C ABI)."""
    return getattr(_lib, name)

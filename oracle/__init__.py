"""Plain fp64 CPU oracle for the HySparse2 cross-decoder attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library and
its Python binding never import, link or call it, and it never imports them.

The arithmetic lives in ``hs2ref.c`` (C99 + OpenMP, IEEE fp64, two-pass
softmax, plain loops); this module only builds that file with gcc and marshals
numpy arrays to it.  ``hs2ref.h`` states, per function, which passage of the
pages it follows.

Array conventions (numpy, host memory):
  * fp32 tensors are ``float32``; bf16 tensors are ``uint16`` bit patterns;
    E4M3FN tensors are ``uint8`` codes with fp32 per-(batch, kv-head) scales.
  * q ``[B, Tq, Hq, D]``; k, v ``[B, Hkv, N, D]`` (any strides with d
    contiguous); scores ``[B, Tq, Hkv, N]``; idx ``[B, Tq, Hkv, max_sel]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hs2ref.c")
_HDR = os.path.join(_HERE, "hs2ref.h")

F32, BF16, E4M3FN = 0, 1, 2


def lib_path(mutant: int = 0) -> str:
    name = "libhs2ref.so" if mutant == 0 else f"libhs2ref_mutant{mutant}.so"
    return os.path.join(_HERE, name)


def build(mutant: int = 0, out: str | None = None) -> str:
    """Compile hs2ref.c with gcc (-O2, OpenMP, IEEE semantics: no fast-math)."""
    out = out or lib_path(mutant)
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", f"-DHS2REF_MUTANT={int(mutant)}",
           _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _KV(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
    ]


_LIBS: dict[int, ctypes.CDLL] = {}


def load(mutant: int = 0) -> ctypes.CDLL:
    if mutant in _LIBS:
        return _LIBS[mutant]
    path = lib_path(mutant)
    newest_src = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if not os.path.exists(path) or os.path.getmtime(path) < newest_src:
        build(mutant)
    lib = ctypes.CDLL(path)
    vp, i32, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
    lib.hs2ref_e4m3fn_decode.restype = f64
    lib.hs2ref_e4m3fn_decode.argtypes = [ctypes.c_uint32]
    lib.hs2ref_bf16_decode.restype = f64
    lib.hs2ref_bf16_decode.argtypes = [ctypes.c_uint32]
    lib.hs2ref_num_threads.restype = ctypes.c_int
    lib.hs2ref_full_attn_scores.restype = ctypes.c_int
    lib.hs2ref_full_attn_scores.argtypes = [ctypes.POINTER(_KV), vp, i32, i32, i32, i32, f64, vp, vp, vp]
    lib.hs2ref_select_topk_window.restype = ctypes.c_int
    lib.hs2ref_select_topk_window.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, i32]
    lib.hs2ref_sparse_attn.restype = ctypes.c_int
    lib.hs2ref_sparse_attn.argtypes = [ctypes.POINTER(_KV), vp, i32, i32, i32, f64, vp, vp, i32, vp, vp]
    lib.hs2ref_kv_bridge.restype = ctypes.c_int
    lib.hs2ref_kv_bridge.argtypes = [vp, i32, i32, vp, i32, i32, vp]
    _LIBS[mutant] = lib
    return lib


def num_threads() -> int:
    return int(load().hs2ref_num_threads())


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3FN
    raise TypeError(f"unsupported element type {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _kv_struct(k: np.ndarray, v: np.ndarray, k_scale, v_scale) -> _KV:
    if k.shape != v.shape or k.dtype != v.dtype or k.ndim != 4:
        raise ValueError("k and v must share a [B, Hkv, N, D] shape and element type")
    if k.strides != v.strides:
        raise ValueError("k and v must share strides")
    es = k.itemsize
    if k.strides[3] != es:
        raise ValueError("head_dim must be contiguous")
    B, Hkv, N, D = k.shape
    code = _dtype_code(k)
    if code == E4M3FN:
        if k_scale is None or v_scale is None:
            raise ValueError("E4M3FN caches need k_scale and v_scale")
        k_scale = np.ascontiguousarray(k_scale, dtype=np.float32).reshape(B * Hkv)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.float32).reshape(B * Hkv)
    kv = _KV(k.ctypes.data, v.ctypes.data, code,
             k.strides[0] // es, k.strides[1] // es, k.strides[2] // es,
             _ptr(k_scale) if code == E4M3FN else None,
             _ptr(v_scale) if code == E4M3FN else None, B, Hkv, N, D)
    kv._keep = (k, v, k_scale, v_scale)  # keep buffers alive for the call
    return kv


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def e4m3fn_decode(code: int, mutant: int = 0) -> float:
    return float(load(mutant).hs2ref_e4m3fn_decode(int(code)))


def e4m3fn_table(mutant: int = 0) -> np.ndarray:
    return np.array([e4m3fn_decode(c, mutant) for c in range(256)], dtype=np.float64)


def e4m3fn_encode(x) -> np.ndarray:
    """OCP E4M3FN code of each real x: the nearest finite value of the format
    (magnitudes above the largest, 448, saturate to it), ties to the code with
    an even mantissa, the sign from x < 0.  A nearest-value search over the
    format's positive codes 0x00..0x7E decoded by e4m3fn_decode (the definition
    of the values; 0x7F is NaN); storing an FP8 KV cache (zgeo.com.cn
    comparison table) needs this encoder."""
    vals = e4m3fn_table()[:0x7F]  # increasing with the code
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), vals[-1])
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_hi, d_lo = vals[hi] - a, a - vals[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(x < 0, code | np.uint8(0x80), code).astype(np.uint8)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    lib = load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.hs2ref_bf16_decode(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(bits))


def full_attn_scores(q, k, v, q_pos0, scale=None, k_scale=None, v_scale=None,
                     want_out=True, want_lse=True, want_scores=True, mutant: int = 0):
    """fp64 full causal attention and importance scores.  Returns (out, lse, scores)."""
    lib = load(mutant)
    q = np.ascontiguousarray(q)
    B, Tq, Hq, D = q.shape
    kv = _kv_struct(k, v, k_scale, v_scale)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Tq, Hq, D), np.float64) if want_out else None
    lse = np.zeros((B, Tq, Hq), np.float64) if want_lse else None
    sc = np.zeros((B, Tq, kv.Hkv, kv.N), np.float64) if want_scores else None
    rc = lib.hs2ref_full_attn_scores(ctypes.byref(kv), q.ctypes.data, _dtype_code(q), Tq, Hq,
                                     int(q_pos0), float(scale), _ptr(out), _ptr(lse), _ptr(sc))
    _check(rc, "full_attn_scores")
    return out, lse, sc


def select_topk_window(scores, q_pos0, k, window, block_size=1, max_sel=None,
                       window_competes=False, mutant: int = 0):
    """Top-k (token or block) + forced window.  Returns (idx int32, count int32)."""
    lib = load(mutant)
    s = np.ascontiguousarray(scores, dtype=np.float64)
    B, Tq, Hkv, N = s.shape
    if max_sel is None:
        max_sel = min(N, k * block_size + window)
    idx = np.empty((B, Tq, Hkv, max_sel), np.int32)
    cnt = np.empty((B, Tq, Hkv), np.int32)
    rc = lib.hs2ref_select_topk_window(s.ctypes.data, B, Tq, Hkv, N, int(q_pos0), int(k), int(window),
                                       int(block_size), int(bool(window_competes)),
                                       idx.ctypes.data, cnt.ctypes.data, int(max_sel))
    _check(rc, "select_topk_window")
    return idx, cnt


def sparse_attn(q, k, v, idx, count, scale=None, k_scale=None, v_scale=None, mutant: int = 0):
    """fp64 attention over each (b, t, g)'s index list.  Returns (out, lse)."""
    lib = load(mutant)
    q = np.ascontiguousarray(q)
    B, Tq, Hq, D = q.shape
    kv = _kv_struct(k, v, k_scale, v_scale)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    count = np.ascontiguousarray(count, dtype=np.int32)
    max_sel = idx.shape[-1]
    out = np.zeros((B, Tq, Hq, D), np.float64)
    lse = np.zeros((B, Tq, Hq), np.float64)
    rc = lib.hs2ref_sparse_attn(ctypes.byref(kv), q.ctypes.data, _dtype_code(q), Tq, Hq, float(scale),
                                idx.ctypes.data, count.ctypes.data, int(max_sel),
                                out.ctypes.data, lse.ctypes.data)
    _check(rc, "sparse_attn")
    return out, lse


def kv_bridge(hidden_bits, w_bits, Hkv, D, mutant: int = 0):
    """fp64 K/V projection of bf16 hidden states.  Returns (K [T,Hkv,D], V [T,Hkv,D])."""
    lib = load(mutant)
    h = np.ascontiguousarray(hidden_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    T, dm = h.shape
    if w.shape != (dm, 2 * Hkv * D):
        raise ValueError("w must be [d_model, 2*Hkv*D]")
    y = np.zeros((T, 2 * Hkv * D), np.float64)
    rc = lib.hs2ref_kv_bridge(h.ctypes.data, T, dm, w.ctypes.data, Hkv, D, y.ctypes.data)
    _check(rc, "kv_bridge")
    return y[:, : Hkv * D].reshape(T, Hkv, D), y[:, Hkv * D:].reshape(T, Hkv, D)


def swa_attn(q, k, v, q_pos0, window, scale=None, k_scale=None, v_scale=None, mutant: int = 0):
    """fp64 sliding-window attention: query token t at position p = q_pos0 + t
    attends to positions [max(0, p - window + 1), p] (javabetter.cn,
    MiMo-V2.6-Flash paragraph: a sliding-window layer looks at each token's
    nearest 128; the current token included, as in reading o4).  The sparse
    layer of hs2ref.c over each query's window as its index list.
    Returns (out, lse)."""
    B, Tq, Hq, D = np.shape(q)
    Hkv = k.shape[1]
    window = int(window)
    if window < 1:
        raise ValueError("window must be at least 1")
    idx = np.full((B, Tq, Hkv, window), -1, np.int32)
    cnt = np.zeros((B, Tq, Hkv), np.int32)
    for t in range(Tq):
        p = int(q_pos0) + t
        lo = max(0, p - window + 1)
        idx[:, t, :, : p - lo + 1] = np.arange(lo, p + 1, dtype=np.int32)
        cnt[:, t, :] = p - lo + 1
    return sparse_attn(q, k, v, idx, cnt, scale=scale, k_scale=k_scale, v_scale=v_scale, mutant=mutant)


def kv_bridge_fp8_write(hidden_bits, w_bits, k_codes, v_codes, k_scale, v_scale, batch_index, pos0, grow,
                        mutant: int = 0):
    """One layer's K/V bridge written into an FP8 (E4M3FN) cache with one fp32
    scale per (batch, kv head) for K and one for V (javabetter.cn, KV Bridging
    paragraph: the layer's own projection of the hidden state; zgeo.com.cn
    comparison table: the FP8 KV cache).  Returns new (k_codes, v_codes,
    k_scale, v_scale) arrays; the inputs are not modified.

    The pages give no quantisation rule; reading o25, per head and per part
    (K or V), with y the fp64 projection of the T new rows:
      * grow = False: the scale stays; new codes = encode(y / scale).
      * grow = True (scale maintenance): s' = max(s, fp32(max|y| / 448)); if
        s' > s, every existing row [0, pos0) of the head is re-encoded,
        code' = encode(fp32(decode(code) * s) / s') (its cache value read as
        the attention reads it, then stored at the new scale); the new rows
        are encoded at s'.  A head whose scale is 0 and whose new rows are all
        0 keeps scale 0 and gets zero codes.
    encode() rounds to nearest even and saturates at +-448."""
    K, V = kv_bridge(hidden_bits, w_bits, k_codes.shape[1], k_codes.shape[3],
                     mutant=mutant if mutant < 20 else 0)  # [T, Hkv, D] fp64
    T = K.shape[0]
    table = e4m3fn_table(mutant if mutant < 20 else 0)
    out = []
    for codes, scale, Y in ((k_codes, k_scale, K), (v_codes, v_scale, V)):
        codes = np.array(codes, copy=True)
        scale = np.array(scale, dtype=np.float32, copy=True)
        Hkv = codes.shape[1]
        for h in range(Hkv):
            s_old = np.float32(scale[batch_index, h])
            y = Y[:, h, :]
            s_new = s_old
            if grow:
                s_new = max(s_old, np.float32(np.abs(y).max() / (1.0 if mutant == 23 else 448.0)))
                if s_new > s_old and pos0 > 0 and mutant != 22:
                    vals = (table[codes[batch_index, h, :pos0]].astype(np.float32) * s_old).astype(np.float64)
                    q = vals * np.float64(s_new) / np.float64(s_old) ** 2 if mutant == 21 else vals / np.float64(s_new)
                    codes[batch_index, h, :pos0] = e4m3fn_encode(q)
            scale[batch_index, h] = s_new
            if s_new > 0:
                codes[batch_index, h, pos0:pos0 + T] = e4m3fn_encode(y / np.float64(s_new))
            else:
                codes[batch_index, h, pos0:pos0 + T] = 0
        out += [codes, scale]
    return out[0], out[2], out[1], out[3]

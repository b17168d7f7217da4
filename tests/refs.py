"""Independent references used to pin the oracle (CPU only).

Nothing here calls the oracle's arithmetic: attention comes from
torch.nn.functional.scaled_dot_product_attention in float64, element decoding
from torch's own bf16 / float8_e4m3fn casts, selection from exhaustive
enumeration with exact (integer or Fraction) arithmetic.
"""
from __future__ import annotations

import itertools

import numpy as np
import torch
import torch.nn.functional as F


def torch_decode(a: np.ndarray, scale=None) -> np.ndarray:
    """Storage array -> float64 values, decoded by torch's casts."""
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
        return t.to(torch.float32).numpy().astype(np.float64)
    if a.dtype == np.uint8:
        t = torch.from_numpy(a.copy()).view(torch.float8_e4m3fn).to(torch.float32)
        B, H = a.shape[:2]
        s = torch.from_numpy(np.asarray(scale, np.float32).reshape(B, H, 1, 1))
        return (t * s).numpy().astype(np.float64)  # float32 multiply, as the cache is read
    raise TypeError(a.dtype)


def sdpa(q, k, v, mask, scale):
    """float64 SDPA.  q [B,Tq,Hq,D]; k,v [B,Hkv,N,Dv]; mask bool [B,Tq,Hkv,N] (True = attend)."""
    q = torch.from_numpy(np.asarray(q, np.float64)).permute(0, 2, 1, 3)  # B,Hq,Tq,D
    k = torch.from_numpy(np.asarray(k, np.float64))
    v = torch.from_numpy(np.array(v, np.float64))
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    k = k.repeat_interleave(G, dim=1).contiguous()
    v = v.repeat_interleave(G, dim=1).contiguous()
    m = torch.from_numpy(np.asarray(mask)).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)  # B,Hq,Tq,N
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=float(scale))
    return o.permute(0, 2, 1, 3).numpy()


def sdpa_probs(q, k, mask, scale):
    """Attention probabilities from SDPA itself: values = identity rows, so out = P."""
    B, Hkv, N, _ = k.shape
    eye = np.broadcast_to(np.eye(N, dtype=np.float64), (B, Hkv, N, N))
    return sdpa(q, k, eye, mask, scale)  # [B,Tq,Hq,N]


def causal_mask(B, Tq, Hkv, N, q_pos0):
    j = np.arange(N)[None, None, None, :]
    p = (q_pos0 + np.arange(Tq))[None, :, None, None]
    return np.broadcast_to(j <= p, (B, Tq, Hkv, N)).copy()


def band_mask(B, Tq, Hkv, N, q_pos0, W):
    j = np.arange(N)[None, None, None, :]
    p = (q_pos0 + np.arange(Tq))[None, :, None, None]
    return np.broadcast_to((j <= p) & (j > p - W), (B, Tq, Hkv, N)).copy()


def index_mask(idx, count, N):
    B, Tq, Hkv, _ = idx.shape
    m = np.zeros((B, Tq, Hkv, N), bool)
    for u in np.ndindex(B, Tq, Hkv):
        m[u][idx[u][: count[u]]] = True
    return m


def brute_select(scores, p, k, window, block_size=1):
    """Exhaustive top-k over exact scores (ints or Fractions).

    Among all subsets T of the candidate units with |T| = min(k, #units) take
    the one of largest total mass; among equal masses the lexicographically
    smallest ascending list of units.  Units are positions (block_size 1) or
    aligned blocks of block_size positions clipped to C = [0, p - window].
    Returns the ascending list T union [p-window+1, p]."""
    clast = p - window
    if block_size == 1:
        units = [(j, [j]) for j in range(clast + 1)]
    else:
        nb = clast // block_size + 1 if clast >= 0 else 0
        units = [(b, list(range(b * block_size, min(b * block_size + block_size - 1, clast) + 1)))
                 for b in range(nb)]
    mass = {u: sum(scores[j] for j in members) for u, members in units}
    members = dict(units)
    take = min(k, len(units))
    best_key, best = None, ()
    for combo in itertools.combinations([u for u, _ in units], take):
        tot = sum(mass[u] for u in combo)
        key = (-tot, combo)
        if best_key is None or key < best_key:
            best_key, best = key, combo
    chosen = set(j for u in best for j in members[u])
    chosen |= set(range(max(0, p - window + 1), p + 1))
    return sorted(chosen)

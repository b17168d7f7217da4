"""Helpers shared by the GPU parity tests, smoke() and bench.py: moving the
generator's host arrays to the device, running the hot path through the C ABI,
and the parity criteria (tolerances are stated here, once)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

# ---- tolerances --------------------------------------------------------------
# Outputs of the full and sparse layers, max-abs against the fp64 oracle on the
# same (dequantised) inputs: 1e-5 for fp32, 1e-2 for bf16 / FP8 caches.
O_TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}
# LSE (natural log): |dLSE| <= LSE_TOL + LSE_REL * |LSE|.  Every path forms
# its logits in fp32, so the maximum logit that LSE carries is itself rounded
# to a few fp32 ulps of its size (2^-20 = 8 ulps); at the workloads' logits
# (|LSE| up to about 14) the absolute term dominates.
LSE_TOL = {"f32": 1e-5, "bf16": 1e-4, "fp8": 1e-4}
LSE_REL = 2.0 ** -20
# Relative output gate, per (b, t, h) row: max_d |dO| <= O_REL * max_d |O_oracle|
# + O_FLOOR.  The absolute bounds above check little at long context, where
# the outputs are of order 1e-3; this one scales with them.  bf16/FP8: the
# probabilities enter the PV products rounded to bf16 (2^-9 relative each)
# and the output is rounded to bf16 once more, so 2^-7 leaves a factor 2 over
# their sum.  fp32: every step in fp32.
O_REL = {"f32": 1e-4, "bf16": 2.0 ** -7, "fp8": 2.0 ** -7}
O_FLOOR = {"f32": 1e-7, "bf16": 1e-6, "fp8": 1e-6}
# Scores: |dS_j| <= S_ABS + S_REL * S_j.  The full layer keeps each head's
# log2-domain logit as a 16-bit code below that head's maximum over the
# aligned 32-position tile, step 2^-12, so a probability term carries a
# relative error <= 2^-13 ln 2 (8.5e-5) plus fp32 rounding; a code that
# saturates (16+ log2 units below the tile maximum) is recomputed exactly from
# the cache unless the tile maximum's probability is below 2^-24, where the
# term is below 2^-40 and G of them stay below S_ABS.  S_ABS is stricter than
# the 1e-7 absolute term of the stated score gate.
S_REL, S_ABS = 1e-4, 1e-9
# Selection: bit-exact indices where the oracle's score gap at the k-th
# boundary exceeds GAP; elsewhere the selected score mass must agree to MASS.
GAP, MASS = 1e-4, 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


class DeviceBlock:
    """One hybrid block's inputs on the device."""

    def __init__(self, inp):
        self.inp = inp
        self.k = dev(inp.k)
        self.v = dev(inp.v)
        self.ks = dev(inp.k_scale) if inp.k_scale is not None else None
        self.vs = dev(inp.v_scale) if inp.v_scale is not None else None
        self.q = dev(inp.q_full)
        self.qs = [dev(x) for x in inp.q_sparse]


def run_block(hs2, blk: DeviceBlock, spec, k=None, window=None, block_size=1, layers=None, split_gather=False,
              topk_call=False):
    """full -> select -> sparse layers on the GPU; topk_call=True runs the full
    layer and the token selection as one hs2_full_attn_topk call, and
    split_gather=True the split gather with a zero-filled workspace (together:
    the launch configuration bench.py times); returns host arrays."""
    k = spec.k if k is None else k
    window = spec.window if window is None else window
    max_sel = min(spec.N, k * block_size + window)
    if topk_call:
        assert block_size == 1
        out, lse, sc, idx, cnt = hs2.full_attn_topk(blk.k, blk.v, blk.q, spec.q_pos0, k, window, max_sel=max_sel,
                                                    k_scale=blk.ks, v_scale=blk.vs)
    else:
        out, lse, sc = hs2.full_attn_scores(blk.k, blk.v, blk.q, spec.q_pos0, k_scale=blk.ks, v_scale=blk.vs)
        idx, cnt = hs2.select_topk_window(sc, spec.q_pos0, k, window, block_size=block_size, max_sel=max_sel)
    ws = torch.zeros(max(hs2.sparse_attn_workspace(spec.B, spec.Tq, spec.Hkv, spec.D, max_sel), 256),
                     dtype=torch.uint8, device="cuda")
    sp = []
    for q in (blk.qs if layers is None else blk.qs[:layers]):
        if split_gather:
            o, l = hs2.sparse_attn_gather_ws(blk.k, blk.v, q, idx, cnt, ws, k_scale=blk.ks, v_scale=blk.vs)
        else:
            o, l = hs2.sparse_attn_gather(blk.k, blk.v, q, idx, cnt, k_scale=blk.ks, v_scale=blk.vs)
        sp.append((host(o), host(l)))
    torch.cuda.synchronize()
    return dict(out=host(out), lse=host(lse), scores=host(sc), idx=host(idx), count=host(cnt), sparse=sp)


def max_abs(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def assert_close(got, want, tol, what):
    err = max_abs(got, want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"
    return err


def assert_lse(got, want, kv, what="lse"):
    """|dLSE| <= LSE_TOL + LSE_REL * |LSE| element by element (infinite
    entries, of empty lists, must match exactly)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(got[~fin], want[~fin]), f"{what}: infinite entries differ"
    err = np.abs(got[fin] - want[fin])
    bound = LSE_TOL[kv] + LSE_REL * np.abs(want[fin])
    assert np.all(err <= bound), f"{what}: |dLSE| up to {float(err.max()):.3e} beyond {LSE_TOL[kv]:g} + 2^-20 |LSE|"
    return float(err.max()) if err.size else 0.0


def assert_scores(got, want, what="scores", G=None):
    """Scores within |dS| <= S_ABS + S_REL * S of the oracle's, element by
    element (G is accepted for call compatibility; the bound does not use it)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    bound = S_ABS + S_REL * np.abs(want)
    bad = np.abs(got - want) > bound
    if bad.any():
        i = np.unravel_index(np.argmax(np.abs(got - want) - bound), got.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} entries outside |dS| <= {S_ABS:g} + {S_REL:g}*S; "
                             f"worst at {i}: got {got[i]:.9e} want {want[i]:.9e}")
    rel = np.max(np.abs(got - want) / (S_ABS + np.abs(want)))
    return float(rel)


def assert_rows_rel(got, want, kv, what="out"):
    """Per (b, t, h) row: max_d |dO| <= O_REL * max_d |O_oracle| + O_FLOOR.
    Returns the worst ratio of a row's error to its scale max_d |O_oracle|."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want).max(-1)
    scale = np.abs(want).max(-1)
    bound = O_REL[kv] * scale + O_FLOOR[kv]
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} rows outside max|dO| <= {O_REL[kv]:.3g}*max|O| + "
                             f"{O_FLOOR[kv]:g}; worst row {i}: err {err[i]:.3e}, max|O| {scale[i]:.3e}")
    return float(np.max(err / np.maximum(scale, 1e-30)))


def check_structure(idx, count, q_pos0, k, window, N, block_size=1):
    """Window always in, ascending, unique, causal, exact count, -1 padding."""
    B, Tq, Hkv, max_sel = idx.shape
    for u in np.ndindex(B, Tq, Hkv):
        p = q_pos0 + u[1]
        n = int(count[u])
        sel = idx[u][:n]
        ncand = max(0, p - window + 1)
        if block_size == 1:
            want_n = min(k, ncand) + min(window, p + 1)
            assert n == want_n, f"count {n} != {want_n} at {u}"
        assert np.all(idx[u][n:] == -1), f"padding at {u}"
        assert np.all(np.diff(sel) > 0), f"not ascending/unique at {u}"
        assert n == 0 or (sel[0] >= 0 and sel[-1] <= p), f"not causal at {u}"
        wlo = max(0, p - window + 1)
        nw = p - wlo + 1
        assert np.array_equal(sel[n - nw:] if nw else sel[:0], np.arange(wlo, p + 1)), f"window missing at {u}"


def check_selection_vs_oracle(idx, count, idx_or, count_or, scores_or, q_pos0, k, window):
    """North-star criterion per (b, t, g): bit-exact where the oracle's gap at the
    k-th boundary exceeds GAP, else equal selected mass within MASS.  Returns
    (units checked bit-exact, units checked by mass, worst mass difference)."""
    B, Tq, Hkv, _ = idx.shape
    exact = by_mass = 0
    worst = 0.0
    for u in np.ndindex(B, Tq, Hkv):
        p = q_pos0 + u[1]
        ncand = max(0, p - window + 1)
        s = scores_or[u][:ncand]
        if k <= 0 or k >= ncand:
            gap = math.inf
        else:
            top = np.sort(s)[::-1]
            gap = top[k - 1] - top[k]
        g_sel = idx[u][: count[u]]
        o_sel = idx_or[u][: count_or[u]]
        if gap > GAP:
            assert np.array_equal(g_sel, o_sel), f"index set differs at {u} although gap {gap:.2e} > {GAP}"
            exact += 1
        else:
            gm = s[g_sel[g_sel < ncand]].sum()
            om = s[o_sel[o_sel < ncand]].sum()
            d = abs(gm - om)
            worst = max(worst, d)
            assert d <= MASS, f"selected mass differs by {d:.2e} at {u} (gap {gap:.2e})"
            by_mass += 1
    return exact, by_mass, worst

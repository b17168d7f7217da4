"""Variable-length batches through the C ABI: each batch entry's queries at
their own position (q_pos0_b, a device array), against the fp64 oracle run on
that batch entry alone at its position -- full layer, token top-k + window,
sparse layers, the multi-query chunk path and sliding-window attention; and
out-of-range positions clamped on the device."""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_full_amd import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs2():
    from long_context_sparse_full_amd import hs2 as mod
    assert torch.cuda.is_available()
    return mod


def spec_for(kv, B, N, Tq, k=256, window=32, Hkv=2, G=8, D=128):
    return synth.Spec("varlen", 93, B=B, N=N, Tq=Tq, Hq=G * Hkv, Hkv=Hkv, D=D, kv_dtype=kv, q_dtype="bf16", k=k,
                      window=window, n_sparse=2, needles=8, needle_mode="uniform", q_std=1.0 / math.sqrt(D))


def entry(a, b):
    return None if a is None else np.ascontiguousarray(a[b:b + 1])


@pytest.mark.parametrize("kv,Tq", [("bf16", 1), ("fp8", 1), ("bf16", 40)], ids=["bf16-decode", "fp8-decode", "bf16-chunk"])
def test_varlen_block(hs2, kv, Tq):
    """Full layer + top-k in one call, then split-gather sparse layers, with a
    different context length per batch entry; per entry, everything equals the
    oracle at that entry's position, scores past it are 0."""
    N, B = 12000, 4
    pos = [N - Tq, 7000, 900 - Tq, 3] if Tq == 1 else [N - Tq, 5000, 1500, 200]
    spec = spec_for(kv, B, N, Tq)
    inp = synth.make_inputs(spec, seed=808 + Tq)
    blk = gu.DeviceBlock(inp)
    qb = torch.tensor(pos, dtype=torch.int32, device="cuda")
    gu.log(f"varlen {kv} Tq={Tq} positions {pos}")
    out, lse, sc, idx, cnt = hs2.full_attn_topk(blk.k, blk.v, blk.q, spec.q_pos0, spec.k, spec.window,
                                                max_sel=spec.max_sel, k_scale=blk.ks, v_scale=blk.vs, q_pos0_b=qb)
    ws = torch.zeros(max(hs2.sparse_attn_workspace(B, Tq, spec.Hkv, spec.D, spec.max_sel), 256), dtype=torch.uint8,
                     device="cuda")
    sp = [hs2.sparse_attn_gather_ws(blk.k, blk.v, q, idx, cnt, ws, k_scale=blk.ks, v_scale=blk.vs) for q in blk.qs]
    torch.cuda.synchronize()
    out, lse, sc, idx, cnt = (gu.host(x) for x in (out, lse, sc, idx, cnt))
    for b, p0 in enumerate(pos):
        ks, vs = entry(inp.k_scale, b), entry(inp.v_scale, b)
        kb, vb = inp.k[b:b + 1], inp.v[b:b + 1]
        o_or, l_or, s_or = oracle.full_attn_scores(entry(inp.q_full, b), kb, vb, p0, k_scale=ks, v_scale=vs)
        gu.assert_close(out[b:b + 1], o_or, gu.O_TOL[kv], f"entry {b} out")
        gu.assert_rows_rel(out[b:b + 1], o_or, kv, f"entry {b} out (per row)")
        gu.assert_lse(lse[b:b + 1], l_or, kv, f"entry {b} lse")
        gu.assert_scores(sc[b:b + 1], s_or, f"entry {b} scores")
        for t in range(Tq):
            assert np.all(sc[b, t, :, p0 + t + 1:] == 0.0), f"entry {b}: scores past the position"
        i_g, c_g = oracle.select_topk_window(sc[b:b + 1].astype(np.float64), p0, spec.k, spec.window,
                                             max_sel=spec.max_sel)
        assert np.array_equal(idx[b:b + 1], i_g) and np.array_equal(cnt[b:b + 1], c_g), f"entry {b}: selection"
        gu.check_structure(idx[b:b + 1], cnt[b:b + 1], p0, spec.k, spec.window, N)
        for layer, (o, l) in enumerate(sp):
            o2, l2 = oracle.sparse_attn(entry(inp.q_sparse[layer], b), kb, vb, idx[b:b + 1], cnt[b:b + 1],
                                        k_scale=ks, v_scale=vs)
            gu.assert_close(gu.host(o)[b:b + 1], o2, gu.O_TOL[kv], f"entry {b} sparse {layer}")


def test_varlen_swa_and_clamping(hs2):
    """Sliding-window attention at per-entry positions (gather and banded
    paths), and positions outside [0, N - Tq] clamped into it."""
    N, B = 5000, 3
    for Tq in (1, 64):
        spec = spec_for("bf16", B, N, Tq)
        inp = synth.make_inputs(spec, seed=909 + Tq)
        blk = gu.DeviceBlock(inp)
        pos = [N - Tq, 1234, 0]
        o, l = hs2.swa_attn(blk.k, blk.v, blk.q, spec.q_pos0, 128, q_pos0_b=torch.tensor(pos, dtype=torch.int32,
                                                                                            device="cuda"))
        raw = [N + 50, 1234, -7]  # clamps to the positions above
        o2, _ = hs2.swa_attn(blk.k, blk.v, blk.q, spec.q_pos0, 128, q_pos0_b=torch.tensor(raw, dtype=torch.int32,
                                                                                            device="cuda"))
        torch.cuda.synchronize()
        o, l, o2 = gu.host(o), gu.host(l), gu.host(o2)
        assert np.array_equal(o, o2), "clamped positions differ from the in-range ones"
        for b, p0 in enumerate(pos):
            o_or, l_or = oracle.swa_attn(entry(inp.q_full, b), inp.k[b:b + 1], inp.v[b:b + 1], p0, 128)
            gu.assert_close(o[b:b + 1], o_or, gu.O_TOL["bf16"], f"swa Tq={Tq} entry {b}")
            gu.assert_lse(l[b:b + 1], l_or, "bf16", f"swa Tq={Tq} entry {b} lse")
    # the full layer with clamped positions
    spec = spec_for("bf16", B, N, 1)
    inp = synth.make_inputs(spec, seed=911)
    blk = gu.DeviceBlock(inp)
    a = hs2.full_attn_scores(blk.k, blk.v, blk.q, spec.q_pos0, q_pos0_b=torch.tensor([N - 1, 10, 0], dtype=torch.int32,
                                                                                       device="cuda"))
    c = hs2.full_attn_scores(blk.k, blk.v, blk.q, spec.q_pos0, q_pos0_b=torch.tensor([N + 9, 10, -3], dtype=torch.int32,
                                                                                       device="cuda"))
    torch.cuda.synchronize()
    for x, y in zip(a, c):
        assert np.array_equal(gu.host(x), gu.host(y)), "full layer: clamped positions differ"


@pytest.mark.parametrize("competes", [False, True], ids=["window", "competes"])
def test_varlen_select_large_grid(hs2, competes):
    """Per-batch query positions on a grid of 2048 rows x 3 chunks (the
    bracketed selection): long rows whose bracket comes from a sample, rows
    sampled whole, rows that take every candidate and rows that take none,
    in one call; bit for bit against the oracle run per batch entry at its
    position."""
    B, Tq, Hkv, N, k, W = 4, 128, 4, 40000, 1024, 128
    pos = [N - Tq, 12000, 100, 1200]
    gu.log(f"varlen select, 2048 rows, positions {pos}, window competes: {competes}")
    rng = np.random.default_rng(78 + competes)
    sc = (rng.integers(0, 20000, (B, Tq, Hkv, N)) / 20000.0 * 1e-3).astype(np.float32)
    max_sel = min(N, k + W)
    qb = torch.tensor(pos, dtype=torch.int32, device="cuda")
    idx, cnt = hs2.select_topk_window(torch.from_numpy(sc).cuda(), N - Tq, k, W, max_sel=max_sel, q_pos0_b=qb,
                                      window_competes=competes)
    torch.cuda.synchronize()
    idx, cnt = gu.host(idx), gu.host(cnt)
    for b in range(B):
        i_or, c_or = oracle.select_topk_window(sc[b:b + 1].astype(np.float64), pos[b], k, W, max_sel=max_sel,
                                               window_competes=competes)
        assert np.array_equal(cnt[b:b + 1], c_or), f"counts differ at batch entry {b} (position {pos[b]})"
        assert np.array_equal(idx[b:b + 1], i_or), f"index lists differ at batch entry {b} (position {pos[b]})"

"""hs2_sparse_attn_gather_static -- the sparse layer for callers that cannot
allocate -- against the entry point whose kernels it shares
(hs2_sparse_attn_gather_ws), through the C ABI: two calls in a row on one
GPU, the second with a smaller input (fewer lists, shorter lists, another
cache type); each result bit for bit equal to the workspace form's on the
same inputs, and within the oracle parity bars."""
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


def lists(rng, B, Tq, Hkv, N, max_sel, counts):
    idx = np.full((B, Tq, Hkv, max_sel), -1, np.int32)
    cnt = np.zeros((B, Tq, Hkv), np.int32)
    for u, n in zip(np.ndindex(B, Tq, Hkv), counts):
        idx[u][:n] = np.sort(rng.choice(N, n, replace=False))
        cnt[u] = n
    return idx, cnt


CALLS = [
    # kv, B, Tq, Hkv, N, max_sel, list lengths (one per (b, t, g))
    ("fp8", 2, 2, 4, 20000, 1152, [1152, 1152, 0, 1, 127, 128, 129, 1000, 1152, 300, 64, 1151, 777, 1152, 5, 1152]),
    ("bf16", 1, 1, 2, 3000, 300, [300, 129]),
]


def test_static_gather_two_calls_second_smaller(hs2):
    rng = np.random.default_rng(0x5747)
    for call, (kv, B, Tq, Hkv, N, max_sel, counts) in enumerate(CALLS):
        gu.log(f"static gather call {call}: {kv} B={B} Tq={Tq} Hkv={Hkv} N={N} max_sel={max_sel}")
        spec = synth.Spec(f"static{call}", 92, B=B, N=N, Tq=Tq, Hq=8 * Hkv, Hkv=Hkv, D=128, kv_dtype=kv,
                          q_dtype="bf16", k=64, window=16, n_sparse=1, needles=4, needle_mode="uniform",
                          q_std=1.0 / math.sqrt(128))
        inp = synth.make_inputs(spec, seed=300 + call)
        blk = gu.DeviceBlock(inp)
        idx, cnt = lists(rng, B, Tq, Hkv, N, max_sel, counts)
        di, dc = gu.dev(idx), gu.dev(cnt)
        o_s, l_s = hs2.sparse_attn_gather_static(blk.k, blk.v, blk.qs[0], di, dc, k_scale=blk.ks, v_scale=blk.vs)
        ws = torch.zeros(hs2.sparse_attn_workspace(B, Tq, Hkv, spec.D, max_sel), dtype=torch.uint8, device="cuda")
        o_w, l_w = hs2.sparse_attn_gather_ws(blk.k, blk.v, blk.qs[0], di, dc, ws, k_scale=blk.ks, v_scale=blk.vs)
        torch.cuda.synchronize()
        o_s, l_s, o_w, l_w = gu.host(o_s), gu.host(l_s), gu.host(o_w), gu.host(l_w)
        assert np.array_equal(o_s, o_w), f"call {call}: output differs from the workspace form"
        assert np.array_equal(l_s, l_w, equal_nan=True), f"call {call}: lse differs from the workspace form"
        o_or, l_or = oracle.sparse_attn(inp.q_sparse[0], inp.k, inp.v, idx, cnt, k_scale=inp.k_scale,
                                        v_scale=inp.v_scale)
        gu.assert_close(o_s, o_or, gu.O_TOL[kv], f"call {call} out")
        gu.assert_rows_rel(o_s, o_or, kv, f"call {call} out (per row)")
        fin = ~np.isinf(l_or)
        gu.assert_lse(l_s[fin], l_or[fin], kv, f"call {call} lse")
        assert np.all(np.isneginf(l_s[~fin])) and np.all(o_s[np.broadcast_to(~fin[..., None], o_s.shape)] == 0)

"""The five workloads at their full sizes, in the launch configuration bench.py
times: full layer, selection and sparse layers against the fp64 oracle.

Full-layer outputs and scores are compared on every (b, t, g) unit; the GPU
selection is compared bit for bit with the oracle's selection on the GPU's own
scores, and with the oracle's selection on the oracle's scores under the
gap/mass rule; sparse layers are compared with the oracle on the GPU's index
lists."""
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


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny", "decode32k", "decode256k", "decode1m_fp8"])
def test_decode_config_end_to_end(hs2, name):
    spec = synth.config(name)
    gu.log(f"[{name}] generating inputs")
    inp = synth.make_inputs(spec)
    blk = gu.DeviceBlock(inp)
    runs = {}
    # the launch configuration bench.py times (kernel-sequence full layer and
    # top-k in one call, split gather), the separate calls with the
    # one-workgroup gather, and the one call with the cooperative kernel
    for label, mode, one_call in (("bench", 0, True), ("separate calls", 0, False), ("cooperative", 1, True)):
        gu.log(f"[{name}] GPU block: {label}")
        hs2.full_attn_set_mode(mode)
        try:
            runs[label] = gu.run_block(hs2, blk, spec, split_gather=one_call, topk_call=one_call)
        finally:
            hs2.full_attn_set_mode(0)
    del blk
    torch.cuda.empty_cache()

    gu.log(f"[{name}] oracle full layer ({spec.B * spec.Tq * spec.Hkv} units)")
    o_or, l_or, s_or = oracle.full_attn_scores(inp.q_full, inp.k, inp.v, spec.q_pos0, k_scale=inp.k_scale,
                                               v_scale=inp.v_scale)
    for label, res in runs.items():
        gu.log(f"[{name}] checking: {label}")
        check_run(name, spec, inp, res, o_or, l_or, s_or)


def check_run(name, spec, inp, res, o_or, l_or, s_or):
    kv = spec.kv_dtype
    e_o = gu.assert_close(res["out"], o_or, gu.O_TOL[kv], "full out")
    e_l = gu.assert_close(res["lse"], l_or, gu.LSE_TOL[kv], "full lse")
    e_s = gu.assert_scores(res["scores"], s_or, G=spec.G)
    gu.log(f"[{name}] full: max|dO|={e_o:.2e} max|dLSE|={e_l:.2e} max rel dS={e_s:.2e}")

    gu.check_structure(res["idx"], res["count"], spec.q_pos0, spec.k, spec.window, spec.N)
    idx_g, cnt_g = oracle.select_topk_window(res["scores"].astype(np.float64), spec.q_pos0, spec.k, spec.window,
                                             max_sel=spec.max_sel)
    assert np.array_equal(res["count"], cnt_g) and np.array_equal(res["idx"], idx_g), \
        "GPU selection differs from the oracle's selection on the same scores"
    idx_or, cnt_or = oracle.select_topk_window(s_or, spec.q_pos0, spec.k, spec.window, max_sel=spec.max_sel)
    exact, by_mass, worst = gu.check_selection_vs_oracle(res["idx"], res["count"], idx_or, cnt_or, s_or,
                                                         spec.q_pos0, spec.k, spec.window)
    gu.log(f"[{name}] selection: {exact} units bit-exact, {by_mass} by mass (worst {worst:.2e})")

    for layer, (o, l) in enumerate(res["sparse"]):
        o2, l2 = oracle.sparse_attn(inp.q_sparse[layer], inp.k, inp.v, res["idx"], res["count"],
                                    k_scale=inp.k_scale, v_scale=inp.v_scale)
        e1 = gu.assert_close(o, o2, gu.O_TOL[kv], f"sparse {layer} out")
        e2 = gu.assert_close(l, l2, gu.LSE_TOL[kv], f"sparse {layer} lse")
        gu.log(f"[{name}] sparse layer {layer}: max|dO|={e1:.2e} max|dLSE|={e2:.2e}")

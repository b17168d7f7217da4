"""The five workloads at their full sizes, in the launch configuration bench.py
times: full layer, selection and sparse layers against the fp64 oracle.

Full-layer outputs and scores are compared on every (b, t, g) unit, outputs
also row by row against a bound relative to the row's own size; the GPU
selection is compared bit for bit with the oracle's selection on the GPU's own
scores, and with the oracle's selection on the oracle's scores under the
gap/mass rule; sparse layers are compared with the oracle on the GPU's index
lists.  A planted-gap variant of the 1M FP8 workload (k strong needles per kv
head) puts every unit on the bit-exact branch of that rule at the size the
bench times."""
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


def run_and_check(hs2, name, spec, inp):
    blk = gu.DeviceBlock(inp)
    runs = {}
    # the launch configuration bench.py times (full layer and top-k in one
    # call, split gather), and the separate calls with the one-workgroup gather
    for label, one_call in (("bench", True), ("separate calls", False)):
        gu.log(f"[{name}] GPU block: {label}")
        runs[label] = gu.run_block(hs2, blk, spec, split_gather=one_call, topk_call=one_call)
    del blk
    torch.cuda.empty_cache()

    gu.log(f"[{name}] oracle full layer ({spec.B * spec.Tq * spec.Hkv} units)")
    o_or, l_or, s_or = oracle.full_attn_scores(inp.q_full, inp.k, inp.v, spec.q_pos0, k_scale=inp.k_scale,
                                               v_scale=inp.v_scale)
    out = {}
    for label, res in runs.items():
        gu.log(f"[{name}] checking: {label}")
        out[label] = check_run(name, spec, inp, res, o_or, l_or, s_or)
    return out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny", "decode32k", "decode256k", "decode1m_fp8"])
def test_decode_config_end_to_end(hs2, name):
    spec = synth.config(name)
    gu.log(f"[{name}] generating inputs")
    inp = synth.make_inputs(spec)
    run_and_check(hs2, name, spec, inp)


@pytest.mark.timeout(900)
def test_decode1m_fp8_planted_gap_bit_exact(hs2):
    """The 1M FP8 workload with k = 1024 strong needles per kv head (needle
    keys 8 sqrt(D) long along one of the group's query directions): the k-th
    boundary of every unit has a gap far above 1e-4, so the GPU's index list
    must equal the oracle's on the oracle's own scores, bit for bit, at the
    size and launch configuration the bench times."""
    base = synth.config("decode1m_fp8")
    spec = base.replace(name="decode1m_fp8_gap", needles=base.k, needle_mode="per_head", needle_norm=8.0)
    gu.log("[decode1m_fp8 planted gap] generating inputs")
    inp = synth.make_inputs(spec, seed=synth.default_seed(base) + 17)
    res = run_and_check(hs2, "decode1m_fp8 planted gap", spec, inp)
    for label, (exact, by_mass) in res.items():
        assert by_mass == 0 and exact == spec.B * spec.Tq * spec.Hkv, \
            f"{label}: planted gaps must put every unit on the bit-exact branch ({exact} exact, {by_mass} by mass)"


def check_run(name, spec, inp, res, o_or, l_or, s_or):
    kv = spec.kv_dtype
    e_o = gu.assert_close(res["out"], o_or, gu.O_TOL[kv], "full out")
    r_o = gu.assert_rows_rel(res["out"], o_or, kv, "full out (per row)")
    e_l = gu.assert_lse(res["lse"], l_or, kv, "full lse")
    e_s = gu.assert_scores(res["scores"], s_or)
    gu.log(f"[{name}] full: max|dO|={e_o:.2e} (worst row {r_o:.2e} of its max|O|) max|dLSE|={e_l:.2e} "
           f"max rel dS={e_s:.2e}")

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
        r1 = gu.assert_rows_rel(o, o2, kv, f"sparse {layer} out (per row)")
        e2 = gu.assert_lse(l, l2, kv, f"sparse {layer} lse")
        gu.log(f"[{name}] sparse layer {layer}: max|dO|={e1:.2e} (worst row {r1:.2e}) max|dLSE|={e2:.2e}")
    return exact, by_mass

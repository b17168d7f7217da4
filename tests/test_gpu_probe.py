"""The scan read-pattern probe (a diagnostic entry point): it runs on bf16 and
FP8 caches at both head dims and a ragged length, writes only its workspace,
and leaves a full-layer call on the same workspace bit-identical."""
import pytest
import torch

from long_context_sparse_full_amd import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hs2():
    from long_context_sparse_full_amd import hs2 as mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return mod


@pytest.mark.parametrize("kv,D", [("bf16", 128), ("fp8", 128), ("fp8", 64), ("bf16", 64)])
def test_scan_read_probe_runs_and_touches_only_its_workspace(hs2, kv, D):
    spec = synth.Spec(f"probe-{kv}", 90, B=2, N=3001, Tq=1, Hq=16, Hkv=2, D=D, kv_dtype=kv, q_dtype="bf16", k=64,
                      window=16, n_sparse=1, needles=4, needle_mode="uniform", q_std=D ** -0.5)
    gu.log(f"scan read probe {kv} D={D} N={spec.N}")
    blk = gu.DeviceBlock(synth.make_inputs(spec, seed=77))
    ws = torch.empty(hs2.full_attn_scores_workspace(blk.k, blk.v, 1, spec.Hq), dtype=torch.uint8, device="cuda")
    o1, l1, s1 = hs2.full_attn_scores(blk.k, blk.v, blk.q, spec.q_pos0, k_scale=blk.ks, v_scale=blk.vs, workspace=ws)
    torch.cuda.synchronize()
    o1, l1, s1 = o1.clone(), l1.clone(), s1.clone()
    k0, v0 = blk.k.clone(), blk.v.clone()
    for codes in (False, True):
        hs2.debug_scan_read_probe(blk.k, blk.v, spec.Hq, codes, blk.ks, blk.vs, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(blk.k, k0) and torch.equal(blk.v, v0)
    o2, l2, s2 = hs2.full_attn_scores(blk.k, blk.v, blk.q, spec.q_pos0, k_scale=blk.ks, v_scale=blk.vs, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(s1, s2)

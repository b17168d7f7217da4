"""The fp64 oracle against references other than itself (CPU only)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(0)


def test_oracle_thread_split_is_bitwise_neutral():
    """The oracle gives the same bits whether its threads take whole (b, t, g)
    units (16 units here) or the positions of one unit at a time (a call per
    query token and kv head)."""
    import numpy as np

    import oracle
    from long_context_sparse_full_amd import synth
    spec = synth.Spec("split", 98, B=1, N=3000, Tq=8, Hq=8, Hkv=2, D=64, kv_dtype="fp8", q_dtype="bf16", k=8,
                      window=4, n_sparse=1, needles=4, needle_mode="uniform", q_std=0.1)
    inp = synth.make_inputs(spec, seed=5)
    o, l, s = oracle.full_attn_scores(inp.q_full, inp.k, inp.v, spec.q_pos0, k_scale=inp.k_scale,
                                      v_scale=inp.v_scale)
    for t in range(spec.Tq):
        for g in range(spec.Hkv):
            q = np.ascontiguousarray(inp.q_full[:, t:t + 1, g * spec.G:(g + 1) * spec.G])
            o1, l1, s1 = oracle.full_attn_scores(q, inp.k[:, g:g + 1], inp.v[:, g:g + 1], spec.q_pos0 + t,
                                                 k_scale=inp.k_scale[:, g:g + 1], v_scale=inp.v_scale[:, g:g + 1])
            assert np.array_equal(o1, o[:, t:t + 1, g * spec.G:(g + 1) * spec.G])
            assert np.array_equal(l1, l[:, t:t + 1, g * spec.G:(g + 1) * spec.G])
            assert np.array_equal(s1, s[:, t:t + 1, g:g + 1])

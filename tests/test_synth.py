"""Seeded generator: determinism and the workload recipe (CPU only)."""
import hashlib

import numpy as np
import pytest

from long_context_sparse_full_amd import synth


def _digest(inp):
    h = hashlib.sha256()
    for a in [inp.q_full, inp.k, inp.v, inp.k_scale, inp.v_scale, *inp.q_sparse, inp.hidden, inp.w_kv]:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def _small(name, **kw):
    base = dict(N=2048)
    if name == "chunk512":
        base.update(Tq=16, bridge=(16, 256))
    base.update(kw)
    return synth.config(name).replace(**base)


@pytest.mark.parametrize("name", [c.name for c in synth.CONFIGS])
def test_same_seed_same_bytes(name):
    spec = _small(name)
    assert _digest(synth.make_inputs(spec, 123)) == _digest(synth.make_inputs(spec, 123))
    assert _digest(synth.make_inputs(spec, 123)) != _digest(synth.make_inputs(spec, 124))


@pytest.mark.parametrize("name", [c.name for c in synth.CONFIGS])
def test_shapes_and_storage(name):
    spec = _small(name)
    inp = synth.make_inputs(spec)
    assert inp.q_full.shape == (spec.B, spec.Tq, spec.Hq, spec.D)
    assert inp.k.shape == inp.v.shape == (spec.B, spec.Hkv, spec.N, spec.D)
    want = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[spec.kv_dtype]
    assert inp.k.dtype == want and inp.v.dtype == want
    assert len(inp.q_sparse) == spec.n_sparse
    if spec.kv_dtype == "fp8":
        import torch
        vals = torch.from_numpy(inp.k).view(torch.float8_e4m3fn).float().numpy()
        assert np.isfinite(vals).all() and np.abs(vals).max() <= 448.0
        assert inp.k_scale.shape == (spec.B, spec.Hkv)
    if spec.bridge:
        T, dm = spec.bridge
        assert inp.hidden.shape == (T, dm) and inp.w_kv.shape == (dm, 2 * spec.Hkv * spec.D)


def test_needles_outside_window_and_bursts():
    spec = _small("decode256k", N=8192)
    inp = synth.make_inputs(spec)
    pos = inp.needle_pos
    assert pos.shape == (spec.B, spec.Hkv, spec.needles)
    assert pos.max() < spec.N - spec.window
    # five bursts: the sorted positions fall into at most five 512-wide clusters
    p = np.sort(pos[0, 0])
    gaps = np.diff(p)
    assert (gaps > 512).sum() <= 4


def test_needle_is_three_times_query_direction():
    spec = _small("tiny", N=512)
    inp = synth.make_inputs(spec)
    j = int(inp.needle_pos[0, 0, 0])
    kn = inp.k[0, 0, j].astype(np.float64)
    assert abs(np.linalg.norm(kn) - 3 * np.sqrt(spec.D)) < 1e-3
    q = inp.q_full[0].astype(np.float64).reshape(-1, spec.D)
    cos = (q @ kn) / (np.linalg.norm(q, axis=1) * np.linalg.norm(kn))
    assert cos.max() > 0.9999


def test_full_size_shapes_declared():
    c = {s.name: s for s in synth.CONFIGS}
    assert (c["decode1m_fp8"].N, c["decode1m_fp8"].kv_dtype) == (1 << 20, "fp8")
    assert c["decode32k"].max_sel == 1152 and c["tiny"].max_sel == 288
    assert c["chunk512"].bridge == (512, 4096) and c["chunk512"].block_k * c["chunk512"].block_size == 1024

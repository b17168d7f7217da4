"""The cache-write side through the C ABI: the K/V bridge of several
cross-decoder layers from one hidden state in one call, FP8 caches with
their scales kept or maintained (reading o25: a head's scale grows to cover
its new rows, and its older rows are re-encoded at the new scale), and the
one-token append of decoding, against the fp64 oracle."""
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


def fp8_codes(rng, shape, lo_exp=1):
    """Random finite E4M3FN codes (normal range, exponent field >= lo_exp)."""
    e = rng.integers(max(1, lo_exp), 16, shape)
    m = rng.integers(0, 8, shape)
    m = np.where(e == 15, np.minimum(m, 6), m)
    return ((rng.integers(0, 2, shape) << 7) | (e << 3) | m).astype(np.uint8)


def fp8_view(big, Hkv, N, D):
    """A cache view into a padded buffer: extra head, rows and columns."""
    return big[:, :Hkv, :N, :D]


def check_codes(got, want, q, bound, what):
    """Codes equal, or one step apart where the quotient lies within `bound`
    of the midpoint between the two codes (rounding decided in fp32)."""
    table = oracle.e4m3fn_table()
    diff = got != want
    if diff.any():
        apart = np.abs(got[diff].astype(int) - want[diff].astype(int))
        assert np.all(apart == 1), f"{what}: codes more than one step apart"
        mid = (table[got[diff]] + table[want[diff]]) / 2
        assert np.all(np.abs(np.abs(q[diff]) - np.abs(mid)) <= bound[diff] + 1e-12), \
            f"{what}: a code differs away from a rounding midpoint"
    return int(diff.sum())


def run_layers(hs2, h, w_layers, caches_np, b, pos0, grow, pad=True):
    """Device copies of the caches (views into padded buffers), one call; returns host copies."""
    L = len(caches_np)
    dev = []
    for kc, vc, ks, vs in caches_np:
        B, Hkv, N, D = kc.shape
        ks_d = gu.dev(ks) if ks is not None else None
        vs_d = gu.dev(vs) if vs is not None else None
        if kc.dtype == np.uint8:
            bk = torch.full((B, Hkv + 1, N + 5, D + 16), 0x11, dtype=torch.uint8, device="cuda")
            bv = torch.full_like(bk, 0x22)
            k, v = fp8_view(bk, Hkv, N, D), fp8_view(bv, Hkv, N, D)
            k.copy_(torch.from_numpy(kc))
            v.copy_(torch.from_numpy(vc))
        else:
            bk = torch.full((B, Hkv + 1, N + 5, D + 8), 7.0, dtype=torch.bfloat16, device="cuda")
            bv = torch.full_like(bk, -3.0)
            k, v = fp8_view(bk, Hkv, N, D), fp8_view(bv, Hkv, N, D)
            k.copy_(gu.dev(kc))
            v.copy_(gu.dev(vc))
        dev.append((bk, bv, k, v, ks_d, vs_d))
    w = gu.dev(np.ascontiguousarray(np.stack(w_layers)))
    hs2.kv_bridge_layers(gu.dev(h), w, [(k, v, ks, vs) if ks is not None else (k, v) for _, _, k, v, ks, vs in dev],
                         b, pos0, grow=grow)
    torch.cuda.synchronize()
    res = []
    for (bk, bv, k, v, ks, vs), (kc, *_rest) in zip(dev, caches_np):
        B, Hkv, N, D = kc.shape
        if kc.dtype == np.uint8:
            res.append(dict(k=k.cpu().numpy(), v=v.cpu().numpy(), ks=gu.host(ks), vs=gu.host(vs),
                            bk=bk.cpu().numpy(), bv=bv.cpu().numpy()))
        else:
            res.append(dict(k=k.view(torch.int16).cpu().numpy().view(np.uint16),
                            v=v.view(torch.int16).cpu().numpy().view(np.uint16),
                            bk=bk.view(torch.int16).cpu().numpy().view(np.uint16),
                            bv=bv.view(torch.int16).cpu().numpy().view(np.uint16)))
    return res


def untouched_padding(r, Hkv, N, D, fill_k, fill_v):
    for name, big, fill in (("K", r["bk"], fill_k), ("V", r["bv"], fill_v)):
        mask = np.ones(big.shape, bool)
        mask[:, :Hkv, :N, :D] = False
        assert np.all(big[mask] == fill), f"{name}: wrote outside the cache view"


def test_bridge_layers_bf16(hs2):
    """Three layers, one hidden state: each layer's rows within one bf16 step
    of its own fp64 projection; rows outside [pos0, pos0 + T) and other batch
    entries untouched."""
    rng = np.random.default_rng(0xB1)
    L, T, dm, Hkv, D, B, N, pos0, b = 3, 77, 256, 2, 128, 2, 150, 40, 1
    h = synth.to_bf16_bits(rng.standard_normal((T, dm)).astype(np.float32))
    ws = [synth.to_bf16_bits((rng.standard_normal((dm, 2 * Hkv * D)) / math.sqrt(dm)).astype(np.float32))
          for _ in range(L)]
    caches = [(synth.to_bf16_bits(rng.standard_normal((B, Hkv, N, D)).astype(np.float32)),
               synth.to_bf16_bits(rng.standard_normal((B, Hkv, N, D)).astype(np.float32)), None, None)
              for _ in range(L)]
    res = run_layers(hs2, h, ws, caches, b, pos0, grow=False)
    for l, (r, (kc, vc, _, _)) in enumerate(zip(res, caches)):
        Kr, Vr = oracle.kv_bridge(h, ws[l], Hkv, D)
        for name, got, old, ref in (("K", r["k"], kc, Kr), ("V", r["v"], vc, Vr)):
            g = oracle.bf16_decode(got[b, :, pos0:pos0 + T])
            want = np.transpose(ref, (1, 0, 2))
            _, e = np.frexp(want)
            assert np.all(np.abs(g - want) <= np.ldexp(1.0, e - 8) + 1e-5), f"layer {l} {name}: beyond one bf16 step"
            mask = np.ones(old.shape, bool)
            mask[b, :, pos0:pos0 + T] = False
            assert np.array_equal(got[mask], old[mask]), f"layer {l} {name}: other rows changed"
        untouched_padding(r, Hkv, N, D, np.uint16(0x40E0), np.uint16(0xC040))


def fp8_case(rng, L, T, dm, Hkv, D, B, N, scale_k, scale_v, w_std):
    h = synth.to_bf16_bits(rng.standard_normal((T, dm)).astype(np.float32))
    ws = [synth.to_bf16_bits((rng.standard_normal((dm, 2 * Hkv * D)) * w_std).astype(np.float32))
          for _ in range(L)]
    caches = [(fp8_codes(rng, (B, Hkv, N, D)), fp8_codes(rng, (B, Hkv, N, D)),
               np.asarray(scale_k, np.float32).copy(), np.asarray(scale_v, np.float32).copy()) for _ in range(L)]
    return h, ws, caches


def check_fp8_layers(res, h, ws, caches, b, pos0, T, grow, what):
    """Against oracle.kv_bridge_fp8_write: scales to fp32 accumulation
    accuracy; codes equal or one step apart at a rounding midpoint (the
    quotients decided in fp32 with the GPU's own scale)."""
    Hkv, D = caches[0][0].shape[1], caches[0][0].shape[3]
    dm = h.shape[1]
    habs = np.abs(oracle.bf16_decode(h))
    table = oracle.e4m3fn_table()
    n_mid = grown = 0
    for l, (r, (kc, vc, ks, vs)) in enumerate(zip(res, caches)):
        k2, v2, ks2, vs2 = oracle.kv_bridge_fp8_write(h, ws[l], kc, vc, ks, vs, b, pos0, grow)
        Kr, Vr = oracle.kv_bridge(h, ws[l], Hkv, D)
        acc = dm * 2.0 ** -23 * (habs @ np.abs(oracle.bf16_decode(ws[l])))  # [T, C]: fp32 accumulation bound
        for part, (name, got, old, gs, os_, ws_, Y) in enumerate((("K", r["k"], kc, r["ks"], ks, ks2, Kr),
                                                                   ("V", r["v"], vc, r["vs"], vs, vs2, Vr))):
            rel_s = np.abs(gs[b] - ws_[b]) / np.maximum(ws_[b], 1e-30)
            ymax = np.abs(Y).max(axis=(0, 2))
            amax_bound = acc[:, part * Hkv * D:(part + 1) * Hkv * D].reshape(T, Hkv, D).max(axis=(0, 2))
            assert np.all(rel_s <= (amax_bound / np.maximum(ymax, 1e-30)) + 2.0 ** -22), f"{what} layer {l} {name}: scales"
            for hh in range(Hkv):
                s0, s1 = np.float64(os_[b, hh]), np.float64(gs[b, hh])
                grew = s1 > s0
                grown += int(grew)
                if grew and pos0 > 0:
                    vals = (table[old[b, hh, :pos0]].astype(np.float32) * np.float32(s0)).astype(np.float64)
                    q = vals / s1
                    want = oracle.e4m3fn_encode(q)
                    n_mid += check_codes(got[b, hh, :pos0], want, q, np.abs(q) * 2.0 ** -22,
                                         f"{what} layer {l} {name} head {hh} older rows")
                else:
                    assert np.array_equal(got[b, hh, :pos0], old[b, hh, :pos0]), f"{what}: older rows changed"
                yv = Y[:, hh, :]
                q = yv / s1
                bound = acc[:, part * Hkv * D + hh * D:part * Hkv * D + (hh + 1) * D] / s1 + np.abs(q) * 2.0 ** -22
                n_mid += check_codes(got[b, hh, pos0:pos0 + T], oracle.e4m3fn_encode(q), q, bound,
                                     f"{what} layer {l} {name} head {hh} new rows")
                assert np.array_equal(got[b, hh, pos0 + T:], old[b, hh, pos0 + T:]), f"{what}: rows past changed"
            other = [i for i in range(old.shape[0]) if i != b]
            assert np.array_equal(got[other], old[other]), f"{what}: other batch entries changed"
            assert np.array_equal(gs[other], os_[other]), f"{what}: other batch entries' scales changed"
        untouched_padding(r, Hkv, kc.shape[2], D, 0x11, 0x22)
    gu.log(f"  {what}: {grown} heads grew, {n_mid} codes one step apart at a midpoint")
    return grown


@pytest.mark.parametrize("grow", [False, True], ids=["keep", "grow"])
def test_bridge_layers_fp8(hs2, grow):
    """Two layers into FP8 caches; with scale maintenance some heads' scales
    are below the new rows' range (they grow, older rows re-encoded) and some
    above (unchanged)."""
    rng = np.random.default_rng(0xB2 + grow)
    L, T, dm, Hkv, D, B, N, pos0, b = 2, 130, 512, 3, 128, 2, 400, 200, 1
    sk = np.array([[1e-3, 1e-2, 2e-2], [5e-3, 1.0, 1e-3]], np.float32)
    sv = np.array([[1e-3, 1e-3, 1e-3], [1.0, 2e-3, 1.0]], np.float32)
    h, ws, caches = fp8_case(rng, L, T, dm, Hkv, D, B, N, sk, sv, 0.5 / math.sqrt(dm) * 40)
    res = run_layers(hs2, h, ws, caches, b, pos0, grow)
    grown = check_fp8_layers(res, h, ws, caches, b, pos0, T, grow, "grow" if grow else "keep")
    if grow:
        assert 0 < grown < L * 2 * Hkv, "the case should grow some heads and keep others"


def test_bridge_layers_fp8_grow_exact(hs2):
    """Projections that are exact in fp32 (identity hidden rows): the GPU's
    grown scales equal the oracle's bit for bit, and codes differ only where a
    quotient sits at a rounding midpoint."""
    rng = np.random.default_rng(0xB4)
    L, T, Hkv, D, B, N, pos0, b, dm = 2, 24, 2, 64, 1, 100, 60, 0, 64
    ys = []
    for _ in range(L):
        y = torch.from_numpy((rng.integers(-4000, 4000, (T, 2 * Hkv * D)) / 64.0).astype(np.float32))
        ys.append(y.to(torch.bfloat16).float().numpy())
    h = np.zeros((T, dm), np.float32)
    h[np.arange(T), np.arange(T)] = 1.0
    h = synth.to_bf16_bits(h)
    ws = []
    for y in ys:
        w = np.zeros((dm, 2 * Hkv * D), np.float32)
        w[:T] = y
        ws.append(synth.to_bf16_bits(w))
    sk = np.array([[0.05, 1.0]], np.float32)   # head 0 grows (|y| up to 62 > 448 * 0.05), head 1 not
    sv = np.array([[1e-3, 0.0]], np.float32)   # head 1 starts empty (scale 0)
    caches = [(fp8_codes(rng, (B, Hkv, N, D)), fp8_codes(rng, (B, Hkv, N, D)), sk.copy(), sv.copy())
              for _ in range(L)]
    res = run_layers(hs2, h, ws, caches, b, pos0, grow=True)
    for l, (r, (kc, vc, ks, vs)) in enumerate(zip(res, caches)):
        k2, v2, ks2, vs2 = oracle.kv_bridge_fp8_write(h, ws[l], kc, vc, ks, vs, b, pos0, True)
        assert np.array_equal(r["ks"], ks2) and np.array_equal(r["vs"], vs2), f"layer {l}: scales differ"
        for name, got, want_c, old, s0, s1, part in (("K", r["k"], k2, kc, ks, ks2, 0), ("V", r["v"], v2, vc, vs, vs2, 1)):
            table = oracle.e4m3fn_table()
            for hh in range(Hkv):
                a, c = np.float64(s0[b, hh]), np.float64(s1[b, hh])
                if c > a:
                    q_old = (table[old[b, hh, :pos0]].astype(np.float32) * np.float32(a)).astype(np.float64) / c
                else:
                    q_old = table[old[b, hh, :pos0]] * 0.0 + 1e9  # unchanged rows: no midpoint allowance
                yv = ys[l][:, part * Hkv * D + hh * D:part * Hkv * D + (hh + 1) * D]
                q_new = yv / c if c > 0 else np.zeros_like(yv)
                q = np.concatenate([q_old, q_new], 0)
                g = got[b, hh, :pos0 + T]
                w = want_c[b, hh, :pos0 + T]
                check_codes(g, w, q, np.abs(q) * 2.0 ** -23, f"layer {l} {name} head {hh}")


def test_kv_append_one_token(hs2):
    """Decoding's append: T = 1 at the end of a 16K-token cache, four layers,
    bf16 caches and FP8 caches with scale maintenance (one head's scale
    grows, which re-encodes its 16383 older rows)."""
    rng = np.random.default_rng(0xB5)
    L, T, dm, Hkv, D, B, N, b = 4, 1, 4096, 4, 128, 1, 16384, 0
    pos0 = N - 1
    h = synth.to_bf16_bits(rng.standard_normal((T, dm)).astype(np.float32))
    ws = [synth.to_bf16_bits((rng.standard_normal((dm, 2 * Hkv * D)) / 64.0).astype(np.float32)) for _ in range(L)]
    caches = [(synth.to_bf16_bits(rng.standard_normal((B, Hkv, N, D)).astype(np.float32)),
               synth.to_bf16_bits(rng.standard_normal((B, Hkv, N, D)).astype(np.float32)), None, None)
              for _ in range(L)]
    res = run_layers(hs2, h, ws, caches, b, pos0, grow=False)
    for l, r in enumerate(res):
        Kr, Vr = oracle.kv_bridge(h, ws[l], Hkv, D)
        for got, ref in ((r["k"], Kr), (r["v"], Vr)):
            g = oracle.bf16_decode(got[b, :, pos0])
            want = ref[0]
            _, e = np.frexp(want)
            assert np.all(np.abs(g - want) <= np.ldexp(1.0, e - 8) + 1e-5)
    sk = np.full((B, Hkv), 0.02, np.float32)
    sk[0, 2] = 1e-4  # grows
    sv = np.full((B, Hkv), 0.02, np.float32)
    caches8 = [(fp8_codes(rng, (B, Hkv, N, D)), fp8_codes(rng, (B, Hkv, N, D)), sk.copy(), sv.copy())
               for _ in range(L)]
    res8 = run_layers(hs2, h, ws, caches8, b, pos0, grow=True)
    grown = check_fp8_layers(res8, h, ws, caches8, b, pos0, T, True, "append")
    assert grown == L, "exactly one head per layer should grow"

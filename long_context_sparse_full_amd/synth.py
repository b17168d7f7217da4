"""Seeded synthetic inputs for the HySparse2 cross-decoder attention hot path.

This module only draws random tensors and encodes them into the storage
formats the path reads (fp32, bf16, OCP E4M3FN with a per-(batch, kv-head)
scale).  It holds none of the method's arithmetic: no attention, no scores,
no selection.  Both the CPU oracle's tests and the HIP path's tests and
benchmark take their inputs from here, so the two sides see identical bytes.

Workloads (the pages measure on trained models and public suites that are not
available here; planted "needle" keys stand in for retrieval targets and
clustered needle bursts stand in for multi-turn tool outputs, the agentic
workload the pages motivate the method with -- aitop.news item 35442, first
paragraph; zgeo.com.cn, "core principle" section):

  tiny      fp32, B=1, N=4096, Tq=8, 8 q / 2 kv heads, D=64, k=256, W=32,
            1 sparse layer, 16 needles per kv head.
  decode32k bf16, B=8, N=32768, Tq=1, 32 q / 4 kv heads, D=128, k=1024, W=128,
            3 sparse layers, 64 needles per sequence at uniform positions.
  decode256k bf16, B=2, N=262144, otherwise as decode32k, needles in 5 bursts.
  decode1m_fp8 B=1, N=1048576, K/V E4M3FN + fp32 scale per (b, kv head), Q bf16.
  chunk512  bf16, B=1, N=131072, Tq=512, plus a [512x4096]x[4096x1024] bridge
            and a 16 x 64-token block-selection baseline.

The selection budget (1024 global tokens + 128 forced recent) and the 64-token
block of the previous generation come from zgeo.com.cn (comparison table and
"core principle" section) and javabetter.cn (the two changes versus HySparse).

Random streams: numpy PCG64 seeded from SeedSequence(seed).spawn(9), one stream
per tensor in the fixed order Q_full, K, V, needles, Q_1, Q_2, Q_3, H, W.
Default seed = 0x48533200 + config index.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

try:  # torch supplies the bf16 and E4M3FN encoders (round-to-nearest-even)
    import torch
except ImportError:  # pragma: no cover
    torch = None

E4M3FN_MAX = 448.0


@dataclass(frozen=True)
class Spec:
    name: str
    index: int
    B: int
    N: int
    Tq: int
    Hq: int
    Hkv: int
    D: int
    kv_dtype: str          # "f32" | "bf16" | "fp8"
    q_dtype: str           # "f32" | "bf16"
    k: int                 # global top-k budget (tokens)
    window: int            # forced recent window
    n_sparse: int          # sparse layers sharing the full layer's K/V and indices
    needles: int           # planted needle keys (per kv head for "per_head", per sequence otherwise)
    needle_mode: str       # "per_head" | "uniform" | "bursts"
    q_std: float           # std of query elements
    bridge: tuple = ()     # (T, d_model) of the K/V bridge projection, or ()
    block_k: int = 0       # blocks selected by the 64-token block baseline (0 = none)
    block_size: int = 64
    needle_lo_limit: int = 0   # needles drawn from [0, N - max(window, this))
    needle_norm: float = 3.0   # needle key = needle_norm * sqrt(D) * (unit query direction)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def q_pos0(self) -> int:
        return self.N - self.Tq

    @property
    def max_sel(self) -> int:
        return min(self.N, self.k + self.window)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


CONFIGS = (
    Spec("tiny", 0, B=1, N=4096, Tq=8, Hq=8, Hkv=2, D=64, kv_dtype="f32", q_dtype="f32",
         k=256, window=32, n_sparse=1, needles=16, needle_mode="per_head", q_std=1.0),
    Spec("decode32k", 1, B=8, N=32768, Tq=1, Hq=32, Hkv=4, D=128, kv_dtype="bf16", q_dtype="bf16",
         k=1024, window=128, n_sparse=3, needles=64, needle_mode="uniform", q_std=1.0 / math.sqrt(128)),
    Spec("decode256k", 2, B=2, N=262144, Tq=1, Hq=32, Hkv=4, D=128, kv_dtype="bf16", q_dtype="bf16",
         k=1024, window=128, n_sparse=3, needles=64, needle_mode="bursts", q_std=1.0 / math.sqrt(128)),
    Spec("decode1m_fp8", 3, B=1, N=1048576, Tq=1, Hq=32, Hkv=4, D=128, kv_dtype="fp8", q_dtype="bf16",
         k=1024, window=128, n_sparse=3, needles=64, needle_mode="uniform", q_std=1.0 / math.sqrt(128)),
    Spec("chunk512", 4, B=1, N=131072, Tq=512, Hq=32, Hkv=4, D=128, kv_dtype="bf16", q_dtype="bf16",
         k=1024, window=128, n_sparse=3, needles=64, needle_mode="uniform", q_std=1.0 / math.sqrt(128),
         bridge=(512, 4096), block_k=16, needle_lo_limit=512),
)


def config(key) -> Spec:
    for c in CONFIGS:
        if key == c.name or key == c.index:
            return c
    raise KeyError(key)


def default_seed(spec: Spec) -> int:
    return 0x48533200 + spec.index


@dataclass
class Inputs:
    spec: Spec
    seed: int
    q_full: np.ndarray                  # [B, Tq, Hq, D] float32 or bf16 bits (uint16)
    k: np.ndarray                       # [B, Hkv, N, D] float32 / uint16 / uint8
    v: np.ndarray
    k_scale: np.ndarray | None          # [B, Hkv] float32 (E4M3FN only)
    v_scale: np.ndarray | None
    q_sparse: list = field(default_factory=list)   # n_sparse arrays like q_full
    hidden: np.ndarray | None = None    # [T, d_model] bf16 bits
    w_kv: np.ndarray | None = None      # [d_model, 2*Hkv*D] bf16 bits
    needle_pos: np.ndarray | None = None  # [B, Hkv, n] int64


def _streams(seed: int):
    ss = np.random.SeedSequence(int(seed))
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(9)]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch's conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3fn(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """float32 [B, H, N, D] -> E4M3FN codes of x/scale, clamped to +-448 first."""
    y = np.clip(x / scale[:, :, None, None].astype(np.float32), -E4M3FN_MAX, E4M3FN_MAX)
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _normal(rng, shape, std=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _needle_positions(rng, spec: Spec, n_pos_hi: int, count: int) -> np.ndarray:
    """Distinct needle positions in [0, n_pos_hi)."""
    count = min(count, n_pos_hi)
    if count <= 0:
        return np.zeros(0, np.int64)
    if spec.needle_mode != "bursts":
        return np.sort(rng.choice(n_pos_hi, size=count, replace=False)).astype(np.int64)
    # bursts: 5 spans of 512 tokens with uniform starts; needles split 13/13/13/13/12
    span = min(512, n_pos_hi)
    per = [count // 5 + (1 if i < count % 5 else 0) for i in range(5)]
    chosen: set[int] = set()
    for n_i in per:
        start = int(rng.integers(0, n_pos_hi - span + 1))
        while n_i > 0:
            cand = int(start + rng.integers(0, span))
            if cand not in chosen:
                chosen.add(cand)
                n_i -= 1
    return np.array(sorted(chosen), np.int64)


def make_inputs(spec: Spec, seed: int | None = None, *, with_sparse: bool = True) -> Inputs:
    """Draw every tensor of one workload.  Deterministic in (spec, seed)."""
    if torch is None and (spec.kv_dtype != "f32" or spec.q_dtype != "f32"):
        raise RuntimeError("bf16/E4M3FN encoding needs torch")
    seed = default_seed(spec) if seed is None else int(seed)
    rs = _streams(seed)
    B, N, Tq, Hq, Hkv, D, G = spec.B, spec.N, spec.Tq, spec.Hq, spec.Hkv, spec.D, spec.G

    q32 = _normal(rs[0], (B, Tq, Hq, D), spec.q_std)
    k32 = _normal(rs[1], (B, Hkv, N, D))
    v32 = _normal(rs[2], (B, Hkv, N, D))

    # needles: a key of norm needle_norm*sqrt(D) along the unit direction of one query of
    # that kv group (head and token drawn per needle); planted in every kv head.
    rn = rs[3]
    hi = max(0, N - max(spec.window, spec.needle_lo_limit))
    if spec.needle_mode == "per_head":
        pos = np.stack([np.stack([_needle_positions(rn, spec, hi, spec.needles) for _ in range(Hkv)])
                        for _ in range(B)])
    else:
        pos = np.stack([np.repeat(_needle_positions(rn, spec, hi, spec.needles)[None], Hkv, 0)
                        for _ in range(B)])
    for b in range(B):
        for g in range(Hkv):
            for j in pos[b, g]:
                h = g * G + int(rn.integers(0, G))
                t = int(rn.integers(0, Tq))
                u = q32[b, t, h].astype(np.float64)
                u = u / max(np.linalg.norm(u), 1e-30)
                k32[b, g, j] = (spec.needle_norm * math.sqrt(D) * u).astype(np.float32)

    if spec.q_dtype == "f32":
        enc_q = lambda x: np.ascontiguousarray(x, np.float32)  # noqa: E731
    else:
        enc_q = to_bf16_bits
    k_scale = v_scale = None
    if spec.kv_dtype == "f32":
        k_st, v_st = k32, v32
    elif spec.kv_dtype == "bf16":
        k_st, v_st = to_bf16_bits(k32), to_bf16_bits(v32)
    elif spec.kv_dtype == "fp8":
        k_scale = (np.abs(k32).max(axis=(2, 3)) / E4M3FN_MAX).astype(np.float32)
        v_scale = (np.abs(v32).max(axis=(2, 3)) / E4M3FN_MAX).astype(np.float32)
        k_st, v_st = to_e4m3fn(k32, k_scale), to_e4m3fn(v32, v_scale)
    else:
        raise ValueError(spec.kv_dtype)
    del k32, v32

    inp = Inputs(spec=spec, seed=seed, q_full=enc_q(q32), k=k_st, v=v_st,
                 k_scale=k_scale, v_scale=v_scale, needle_pos=pos)
    if with_sparse:
        for layer in range(spec.n_sparse):
            inp.q_sparse.append(enc_q(_normal(rs[4 + layer], (B, Tq, Hq, D), spec.q_std)))
    if spec.bridge:
        T, dm = spec.bridge
        inp.hidden = to_bf16_bits(_normal(rs[7], (T, dm)))
        inp.w_kv = to_bf16_bits(_normal(rs[8], (dm, 2 * Hkv * D), 1.0 / math.sqrt(dm)))
    return inp


def random_index_lists(rng_seed: int, units: int, n_rows: int, per_list: int) -> tuple[np.ndarray, np.ndarray]:
    """Sorted distinct random row indices: idx [units, per_list] int32, count [units].

    Used for the throughput-regime gather measurement (independent query
    streams, each with its own index list, against one cache)."""
    rng = np.random.Generator(np.random.PCG64(int(rng_seed)))
    per_list = min(per_list, n_rows)
    idx = np.empty((units, per_list), np.int32)
    for u in range(units):
        idx[u] = np.sort(rng.choice(n_rows, size=per_list, replace=False)).astype(np.int32)
    return idx, np.full(units, per_list, np.int32)


def make_dominant_inputs(spec: Spec, gaps, seed: int, dominant: float = 48.0) -> Inputs:
    """A workload whose attention is dominated by one key per (b, kv head),
    with weaker keys beside it in the same aligned 32-position tile.

    Every query head of a group points along one random unit direction u of
    that group (plus a 5% perturbation), scaled so that a key's projection on
    u, in units of |u|, is its logit in log2 units at softmax scale 1/sqrt(D)
    (q = u * sqrt(D) / log2(e)).  Keys and values are N(0, 1), so ordinary
    logits are about N(0, 1) in those units.  One key per (b, g), at a random
    position j*, is `dominant * u`; for each entry of `gaps` another key of
    the same tile is (dominant - gap) * u.  So the dominant key holds nearly
    all of every head's probability and the others sit `gap` log2 units below
    it (before the storage rounding of q and K).  Needle positions are returned
    in needle_pos[b, g] (the dominant one first).  Tq query tokens, one
    sparse layer of ordinary queries."""
    B, N, Tq, Hq, Hkv, D, G = spec.B, spec.N, spec.Tq, spec.Hq, spec.Hkv, spec.D, spec.G
    gaps = list(gaps)
    if len(gaps) > 31 or N < 32:
        raise ValueError("at most 31 gaps, N >= 32")
    rs = _streams(seed)
    k32 = _normal(rs[1], (B, Hkv, N, D))
    v32 = _normal(rs[2], (B, Hkv, N, D))
    rn = rs[3]
    q32 = np.empty((B, Tq, Hq, D), np.float32)
    qscale = math.sqrt(D) / math.log2(math.e)
    hi_tile = max(1, (N - spec.window) // 32)
    pos = np.empty((B, Hkv, 1 + len(gaps)), np.int64)
    for b in range(B):
        for g in range(Hkv):
            u = rn.standard_normal(D)
            u /= np.linalg.norm(u)
            for t in range(Tq):
                for i in range(G):
                    n = rn.standard_normal(D) / math.sqrt(D)
                    q32[b, t, g * G + i] = (qscale * (u + 0.05 * n)).astype(np.float32)
            tile = int(rn.integers(0, hi_tile))
            offs = rn.permutation(32)[: 1 + len(gaps)]
            js = [32 * tile + int(o) for o in offs]
            k32[b, g, js[0]] = (dominant * u).astype(np.float32)
            for j, gap in zip(js[1:], gaps):
                k32[b, g, j] = ((dominant - gap) * u).astype(np.float32)
            pos[b, g] = js
    enc_q = (lambda x: np.ascontiguousarray(x, np.float32)) if spec.q_dtype == "f32" else to_bf16_bits
    k_scale = v_scale = None
    if spec.kv_dtype == "f32":
        k_st, v_st = k32, v32
    elif spec.kv_dtype == "bf16":
        k_st, v_st = to_bf16_bits(k32), to_bf16_bits(v32)
    else:
        k_scale = (np.abs(k32).max(axis=(2, 3)) / E4M3FN_MAX).astype(np.float32)
        v_scale = (np.abs(v32).max(axis=(2, 3)) / E4M3FN_MAX).astype(np.float32)
        k_st, v_st = to_e4m3fn(k32, k_scale), to_e4m3fn(v32, v_scale)
    inp = Inputs(spec=spec, seed=seed, q_full=enc_q(q32), k=k_st, v=v_st, k_scale=k_scale, v_scale=v_scale,
                 needle_pos=pos)
    inp.q_sparse.append(enc_q(_normal(rs[4], (B, Tq, Hq, D), spec.q_std)))
    return inp

"""The C-ABI library without a GPU: it loads, exports every declared symbol,
the header compiles as C and C++, and argument validation returns its status
codes before any launch (CPU only; no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hs2.h")


@pytest.fixture(scope="module")
def hs2():
    from long_context_sparse_full_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    from long_context_sparse_full_amd import hs2 as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs2_[a-z0-9_]+)\s*\(", text)))


def test_header_compiles_as_c_and_cpp(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "hs2.h"\nint main(void){ return hs2_abi_version() == HS2_ABI_VERSION ? 0 : 1; }\n')
    for comp, std in (("gcc", "-std=c99"), ("g++", "-std=c++11")):
        subprocess.run([comp, std, "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                        "-x", "c" if comp == "gcc" else "c++", str(src)], check=True)


def test_header_coexists_with_hip_runtime(tmp_path):
    src = tmp_path / "use.cpp"
    src.write_text('#include <hip/hip_runtime.h>\n#include "hs2.h"\n'
                   'int f(hipStream_t s){ return hs2_sparse_attn_gather(0,0,HS2_BF16,1,8,1.f,0,0,1,0,0,s); }\n')
    subprocess.run(["/opt/rocm/bin/hipcc", "-fsyntax-only", "-I", os.path.join(ROOT, "include"), str(src)], check=True)


def test_every_declared_symbol_is_exported(hs2):
    lib = ctypes.CDLL(hs2.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), f"{n} declared in hs2.h but not exported"
    assert sorted(hs2.EXPORTED) == names


def test_version_and_status_strings(hs2):
    assert hs2.abi_version() == 3
    for st in (0, -1, -2, -3, -4):
        assert hs2._status_string(st).decode()


def test_timing_names(hs2):
    names = hs2.timing_kernel_names()
    assert "full_scan" in names and "sparse_gather" in names and "select_hist" in names
    assert "scan_read_probe" in names and "scan_read_probe_codes" in names


# --- validation, with fake (never dereferenced) device addresses -----------

FAKE = 1 << 20  # 16-byte aligned, never touched: every case fails validation first


def desc(hs2, dtype=1, B=1, H=2, N=256, D=128, sn=None, k=FAKE, scales=False, cls=None):
    sn = D if sn is None else sn
    cls = cls or hs2.KVDesc
    d = cls(k, FAKE, dtype, H * N * sn, N * sn, sn, FAKE if scales else None, FAKE if scales else None,
            B, H, N, D)
    return d


def full(hs2, d, q=FAKE, qdt=1, Tq=1, Hq=16, q_pos0=None, out=FAKE, scores=FAKE, ws=FAKE, wsb=1 << 40):
    q_pos0 = d.N - Tq if q_pos0 is None else q_pos0
    return hs2._full(ctypes.byref(d), q, qdt, Tq, Hq, q_pos0, None, 0.1, out, None, scores, ws, wsb, None)


@pytest.mark.parametrize("case,want", [
    ("ok_shape_but_small_ws", -3),
    ("null_kv", -1), ("null_q", -1), ("null_out", -1), ("hq_not_multiple", -1),
    ("qpos_past_end", -1), ("neg_qpos", -1), ("misaligned_q", -1), ("misaligned_stride", -1),
    ("head_dim_96", -2), ("group_32", -2), ("fp8_without_scales", -2), ("q_f32_kv_bf16", -2),
    ("bad_dtype", -2), ("ws_misaligned", -1), ("qpos_b_misaligned", -1),
])
def test_full_attn_validation(hs2, case, want):
    d = desc(hs2)
    kw = {}
    if case == "ok_shape_but_small_ws":
        kw["wsb"] = 16
    elif case == "null_kv":
        assert hs2._full(None, FAKE, 1, 1, 16, 0, None, 0.1, FAKE, None, FAKE, FAKE, 1 << 40, None) == want
        return
    elif case == "null_q":
        kw["q"] = None
    elif case == "null_out":
        kw["out"] = None
    elif case == "hq_not_multiple":
        kw["Hq"] = 15
    elif case == "qpos_past_end":
        kw["q_pos0"] = d.N
    elif case == "neg_qpos":
        kw["q_pos0"] = -1
    elif case == "misaligned_q":
        kw["q"] = FAKE + 2
    elif case == "misaligned_stride":
        d = desc(hs2, sn=130)  # 260-byte rows are not a multiple of 16 bytes
    elif case == "head_dim_96":
        d = desc(hs2, D=96)
    elif case == "group_32":
        d = desc(hs2, H=1)
        kw["Hq"] = 32
    elif case == "fp8_without_scales":
        d = desc(hs2, dtype=2)
    elif case == "q_f32_kv_bf16":
        kw["qdt"] = 0
    elif case == "bad_dtype":
        d = desc(hs2, dtype=7)
    elif case == "ws_misaligned":
        kw["ws"] = FAKE + 16
    elif case == "qpos_b_misaligned":
        assert hs2._full(ctypes.byref(d), FAKE, 1, 1, 16, d.N - 1, FAKE + 2, 0.1, FAKE, None, FAKE, FAKE, 1 << 40,
                         None) == want
        return
    assert full(hs2, d, **kw) == want
    assert hs2._last_error().decode()


@pytest.mark.parametrize("case,want", [
    ("small_ws", -3), ("null_kv", -1), ("f32_cache", -2), ("hq_not_multiple", -1), ("group_32", -1),
    ("fp8_without_scales", -2), ("ws_misaligned", -1),
])
def test_scan_read_probe_validation(hs2, case, want):
    d, Hq, ws, wsb = desc(hs2), 16, FAKE, 1 << 40
    if case == "small_ws":
        wsb = 16
    elif case == "null_kv":
        assert hs2._dbg_scanprobe(None, Hq, 1, ws, wsb, None) == want
        return
    elif case == "f32_cache":
        d = desc(hs2, dtype=0)
    elif case == "hq_not_multiple":
        Hq = 15
    elif case == "group_32":
        d, Hq = desc(hs2, H=1), 32
    elif case == "fp8_without_scales":
        d = desc(hs2, dtype=2)
    elif case == "ws_misaligned":
        ws = FAKE + 16
    assert hs2._dbg_scanprobe(ctypes.byref(d), Hq, 1, ws, wsb, None) == want
    assert hs2._last_error().decode()


def test_workspace_figures(hs2):
    d = desc(hs2, N=1 << 20, H=4)
    ws = hs2._full_ws(ctypes.byref(d), 1, 32)
    # logit codes: 4 kv heads x 8 rows x 2^20 positions x 2 B, tile maxima (1/16 of that), split partials
    codes = 4 * 8 * (1 << 20) * 2
    assert codes + codes // 16 <= ws < codes + codes // 16 + (32 << 20)
    assert hs2._sel_ws(1, 1, 4, 1 << 20) >= hs2._sel_ws_for(1, 1, 4, 1 << 20, 1)
    assert hs2._sel_ws_for(1, 512, 4, 131072, 64) > 0
    assert hs2._full_ws(None, 1, 32) == 0


@pytest.mark.parametrize("case,want", [
    ("small_ws", -3), ("max_sel_small", -1), ("neg_k", -1), ("neg_window", -1), ("block0", -1),
    ("qpos_past_end", -1), ("null_idx", -1), ("bad_flags", -1), ("competes_blocks", -2),
])
def test_select_validation(hs2, case, want):
    a = dict(scores=FAKE, B=1, Tq=1, Hkv=4, N=4096, q_pos0=4095, k=1024, window=128, bs=1, flags=0, idx=FAKE,
             cnt=FAKE, max_sel=1152, ws=FAKE, wsb=1 << 40)
    if case == "small_ws":
        a["wsb"] = 100
    elif case == "max_sel_small":
        a["max_sel"] = 1151
    elif case == "neg_k":
        a["k"] = -1
    elif case == "neg_window":
        a["window"] = -1
    elif case == "block0":
        a["bs"] = 0
    elif case == "qpos_past_end":
        a["q_pos0"] = 4096
    elif case == "null_idx":
        a["idx"] = None
    elif case == "bad_flags":
        a["flags"] = 2
    elif case == "competes_blocks":
        a["flags"], a["bs"], a["k"] = 1, 64, 16
    st = hs2._select(a["scores"], a["B"], a["Tq"], a["Hkv"], a["N"], a["q_pos0"], None, a["k"], a["window"], a["bs"],
                     a["flags"], a["idx"], a["cnt"], a["max_sel"], a["ws"], a["wsb"], None)
    assert st == want


def test_select_max_sel_rule_uses_context_cap(hs2):
    # N smaller than k + window: max_sel = N suffices (fails later only on the workspace)
    st = hs2._select(FAKE, 1, 1, 1, 600, 599, None, 1024, 128, 1, 0, FAKE, FAKE, 600, FAKE, 10, None)
    assert st == -3


def test_full_attn_topk_validation(hs2):
    d = desc(hs2)
    ws = int(hs2._topk_ws(ctypes.byref(d), 1, 16))
    full = int(hs2._full_ws(ctypes.byref(d), 1, 16))
    assert ws > full
    args = lambda idx=FAKE, k=8, window=4, max_sel=12, wsb=ws, flags=0: (ctypes.byref(d), FAKE, 1, 1, 16, 255, None,
                                                                          0.1, FAKE, None, FAKE, k, window, flags, idx,
                                                                          FAKE, max_sel, FAKE, wsb, None)
    assert hs2._topk(*args(idx=None)) == -1            # NULL idx
    assert hs2._topk(*args(k=-1)) == -1                # negative k
    assert hs2._topk(*args(max_sel=11)) == -1          # max_sel < k + window
    assert hs2._topk(*args(wsb=ws - 1)) == -3          # workspace too small
    assert hs2._topk(*args(flags=4)) == -1             # unknown flag


def test_sparse_and_bridge_validation(hs2):
    d = desc(hs2)
    assert hs2._sparse(ctypes.byref(d), FAKE, 1, 1, 16, 0.1, None, FAKE, 8, FAKE, None, None) == -1
    assert hs2._sparse(ctypes.byref(d), FAKE, 1, 1, 16, 0.1, FAKE, FAKE, 0, FAKE, None, None) == -1
    assert hs2._sparse(ctypes.byref(d), FAKE, 0, 1, 16, 0.1, FAKE, FAKE, 8, FAKE, None, None) == -2
    assert hs2._sparse(ctypes.byref(d), FAKE, 1, 1, 16, float("nan"), FAKE, FAKE, 8, FAKE, None, None) == -1
    out = hs2.KVOutDesc
    d32 = desc(hs2, dtype=0, cls=out)
    assert hs2._bridge(FAKE, 4, 4096, FAKE, ctypes.byref(d32), 0, 0, None) == -2  # cache bf16 or FP8
    d8n = desc(hs2, dtype=2, scales=False, cls=out)
    assert hs2._bridge(FAKE, 4, 4096, FAKE, ctypes.byref(d8n), 0, 0, None) == -2  # FP8 cache needs scales
    do = desc(hs2, cls=out)
    assert hs2._bridge(FAKE, 4, 4000, FAKE, ctypes.byref(do), 0, 0, None) == -2   # d_model % 64
    assert hs2._bridge(FAKE, 4, 4096, FAKE, ctypes.byref(do), 1, 0, None) == -1   # batch index
    assert hs2._bridge(FAKE, 4, 4096, FAKE, ctypes.byref(do), 0, 253, None) == -1  # pos0 + T > N
    assert hs2._bridge(FAKE, 4, 4096, FAKE, None, 0, 0, None) == -1                # NULL descriptor
    assert hs2._dbg_e4m3(None, FAKE, 4, None) == -1


def test_static_gather_limits(hs2):
    """The no-allocation sparse layer rejects a split larger than its static
    scratch before touching the device, and validates like the other calls."""
    assert hs2.sparse_attn_static_limit() == 4 << 20
    # 63 lists of 4096 entries at D = 128: 63 * 32 slices * 16 rows * 130 floats > 4 MiB
    d = desc(hs2, H=63, N=8192)
    st = hs2._sparse_static(ctypes.byref(d), FAKE, 1, 1, 63 * 8, 0.1, FAKE, FAKE, 4096, FAKE, None, None)
    assert st == -3 and "static scratch" in hs2._last_error().decode()
    d = desc(hs2)
    assert hs2._sparse_static(ctypes.byref(d), FAKE, 1, 1, 16, 0.1, None, FAKE, 8, FAKE, None, None) == -1
    assert hs2._sparse_static(ctypes.byref(d), FAKE, 1, 1, 16, 0.1, FAKE, FAKE, 0, FAKE, None, None) == -1
    assert hs2._sparse_static(None, FAKE, 1, 1, 16, 0.1, FAKE, FAKE, 8, FAKE, None, None) == -1


def test_bridge_layers_validation(hs2):
    out = hs2.KVOutDesc
    d = desc(hs2, cls=out)
    arr = (out * 2)(d, d)
    f = hs2._bridge_layers
    assert f(FAKE, 4, 4096, FAKE, 0, arr, 0, 0, 0, None, 0, None) == -1     # no layers
    assert f(FAKE, 4, 4096, FAKE, 17, arr, 0, 0, 0, None, 0, None) == -1    # too many layers
    assert f(FAKE, 4, 4096, FAKE, 2, arr, 0, 0, 5, None, 0, None) == -1     # unknown scale mode
    assert f(FAKE, 4, 4096, FAKE, 2, None, 0, 0, 0, None, 0, None) == -1    # NULL descriptors
    d2 = desc(hs2, cls=out, D=64)
    assert f(FAKE, 4, 4096, FAKE, 2, (out * 2)(d, d2), 0, 0, 0, None, 0, None) == -1  # caches disagree
    d8 = desc(hs2, dtype=2, scales=True, cls=out)
    ws = hs2._bridge_layers_ws(2, 4, d8.Hkv, d8.D)
    assert ws > 2 * 4 * 2 * d8.Hkv * d8.D * 4
    assert f(FAKE, 4, 4096, FAKE, 2, (out * 2)(d8, d8), 0, 0, 1, FAKE, ws - 1, None) == -3  # grow: workspace


def test_paged_validation(hs2):
    """The paged entry points check the page table and the pool descriptor
    before any launch: page rows a power of two of at least 32, the table
    covering N, a pool shared by the sequences (stride_b 0), bf16/FP8 only, and
    no multi-query chunk on a paged cache."""
    d = desc(hs2, B=2, H=2, N=256)
    d.stride_b = 0
    ws = int(hs2._topk_ws(ctypes.byref(d), 1, 16))

    def topk(pt, dd=d, Tq=1, wsb=ws):
        return hs2._topk_paged(ctypes.byref(dd), None if pt is None else ctypes.byref(pt), FAKE, 1, Tq, 16,
                               dd.N - Tq, None, 0.1, FAKE, None, FAKE, 8, 4, 0, FAKE, FAKE, 12, FAKE, wsb, None)

    def gather(pt, dd=d):
        return hs2._sparse_paged(ctypes.byref(dd), None if pt is None else ctypes.byref(pt), FAKE, 1, 1, 16, 0.1,
                                 FAKE, FAKE, 12, FAKE, None, FAKE, 1 << 30, None)

    P = hs2.PageTable
    assert topk(None) == -1                              # no table
    assert topk(P(None, 64, 4, 8)) == -1                 # NULL table pointer
    assert topk(P(FAKE, 48, 6, 8)) == -1                 # page rows not a power of two
    assert topk(P(FAKE, 16, 16, 32)) == -1               # pages below 32 rows
    assert topk(P(FAKE, 64, 3, 8)) == -1                 # 3 pages of 64 rows do not cover N = 256
    assert topk(P(FAKE, 64, 4, 0)) == -1                 # empty pool
    assert topk(P(FAKE, 1 << 20, 1, 4096)) == -1         # pool rows beyond 2^31
    assert topk(P(FAKE + 2, 64, 4, 8)) == -1             # misaligned table
    d_b = desc(hs2, B=2, H=2, N=256)
    assert topk(P(FAKE, 64, 4, 8), dd=d_b) == -1         # stride_b of a per-sequence cache
    d32 = desc(hs2, dtype=0, B=2, H=2, N=256)
    d32.stride_b = 0
    assert topk(P(FAKE, 64, 4, 8), dd=d32) == -2         # fp32 cache
    wsc = int(hs2._topk_ws(ctypes.byref(d), 64, 16))
    assert topk(P(FAKE, 64, 4, 8), Tq=64, wsb=wsc) == -2  # 64 query tokens: the chunk path
    assert topk(P(FAKE, 64, 4, 8), wsb=ws - 1) == -3     # workspace
    assert gather(None) == -1
    assert gather(P(FAKE, 64, 3, 8)) == -1
    assert gather(P(FAKE, 64, 4, 8), dd=d32) == -2

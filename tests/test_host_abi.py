"""Host-side checks of libwpa that need no GPU: exported symbols, the closed-form kept-term
count against the oracle's enumerations, the window table, and argument validation (every
rejected call returns before any HIP call)."""
import ctypes
import json
import math
import os
import re

import numpy as np
import pytest

import oracle
import rope_wavelength_sparsity_amd as wpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "wpa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wpa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = wpa.lib()
    declared = _declared_symbols()
    assert declared, "no declarations parsed"
    assert set(declared) == set(wpa.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


GRID = [(d, base, alpha) for d in (2, 8, 64, 128) for base in (10.0, 1e4, 5e5, 1e7)
        for alpha in (0.0, 0.3, 1.0, 2.0, 8.0, math.inf)]


@pytest.mark.parametrize("d,base,alpha", GRID)
def test_closed_form_count_matches_enumeration(d, base, alpha):
    for (n_q, q0, n_k) in [(1, 0, 1), (5, 0, 5), (64, 0, 64), (300, 0, 300), (1, 299, 300),
                           (1, 0, 300), (37, 250, 260), (10, 400, 300), (50, 3, 20)]:
        got = wpa.count_terms(d, base, alpha, n_q, q0, n_k)
        assert got == oracle.count_enumerate(d, base, alpha, n_q, q0, n_k), (n_q, q0, n_k)


def test_closed_form_count_matches_golden_large():
    """Workload-sized counts written by tests/golden/make_counts.py (oracle only)."""
    data = json.load(open(os.path.join(ROOT, "tests", "golden", "counts.json")))
    for c in data["cases"]:
        alpha = math.inf if c["alpha"] == "inf" else c["alpha"]
        got = wpa.count_terms(c["d"], c["base"], alpha, c["n_q"], c["q0"], c["n_k"])
        assert got == (c["kept"], c["total"]), c["name"]


@pytest.mark.parametrize("N", [1000, 4097, 65536, 1 << 20])
def test_closed_form_count_matches_distance_histogram(N):
    for d, base in ((64, 1e6), (128, 5e5), (128, 1e7)):
        for alpha in (1.0, 2.0, 0.25):
            assert wpa.count_terms(d, base, alpha, N, 0, N) == \
                oracle.count_by_distance(d, base, alpha, N, 0, N)
    assert wpa.count_terms(128, 5e5, 1.0, 1, N - 1, N) == \
        oracle.count_by_distance(128, 5e5, 1.0, 1, N - 1, N)


@pytest.mark.parametrize("d,base,alpha", [(64, 1e4, 1.0), (128, 5e5, 2.0), (128, 1e7, 0.5),
                                          (64, 1e6, math.inf), (16, 10.0, 1e12)])
def test_window_table_is_floor_of_oracle_threshold(d, base, alpha):
    W = wpa.thresholds(d, base, alpha)
    thr = oracle.thresholds(d, base, alpha)
    for w, t in zip(W, thr):
        if t >= 2 ** 31 - 1:
            assert w == 2 ** 31 - 1
        else:
            assert w == math.floor(t)
    assert all(a <= b for a, b in zip(W, W[1:]))       # non-decreasing: a suffix is active


FAKE = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced: validation fails first


def _prefill_rc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, pos=None, B=1, N=128, Hq=4, Hkv=2, d=64,
             base=1e4, alpha=1.0, scale=0.0, dtype=0, odt=0, cnt=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    L = wpa.lib()
    return L.wpa_prefill(a["q"], a["k"], a["v"], a["out"], a["lse"], a["pos"], a["B"], a["N"],
                         a["Hq"], a["Hkv"], a["d"], a["base"], a["alpha"], a["scale"], a["dtype"],
                         a["odt"], a["cnt"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), wpa.WPA_ERR_UNSUPPORTED),
    (dict(d=32), wpa.WPA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), wpa.WPA_ERR_INVALID),
    (dict(alpha=float("nan")), wpa.WPA_ERR_INVALID),
    (dict(alpha=-1.0), wpa.WPA_ERR_INVALID),
    (dict(base=1.0), wpa.WPA_ERR_INVALID),
    (dict(base=float("inf")), wpa.WPA_ERR_INVALID),
    (dict(N=0), wpa.WPA_ERR_INVALID),
    (dict(B=0), wpa.WPA_ERR_INVALID),
    (dict(dtype=7), wpa.WPA_ERR_INVALID),
    (dict(odt=2), wpa.WPA_ERR_INVALID),
    (dict(scale=float("nan")), wpa.WPA_ERR_INVALID),
    (dict(q=None), wpa.WPA_ERR_INVALID),
    (dict(ws=None), wpa.WPA_ERR_INVALID),
    (dict(k=ctypes.c_void_p((1 << 20) + 8)), wpa.WPA_ERR_INVALID),
    (dict(cnt=ctypes.c_void_p((1 << 20) + 4)), wpa.WPA_ERR_INVALID),
    (dict(ws_bytes=100), wpa.WPA_ERR_WORKSPACE),
])
def test_prefill_rejects_bad_arguments(kw, code):
    assert _prefill_rc(**kw) == code
    assert wpa.lib().wpa_last_error().decode() != ""


def _decode_rc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, qpos=None, out=FAKE, lse=None, B=2, Lmax=4096,
             Hq=8, Hkv=2, d=128, base=5e5, alpha=1.0, scale=0.0, dtype=0, odt=1, cnt=None,
             chunk=0, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return wpa.lib().wpa_decode(a["q"], a["kc"], a["vc"], a["lens"], a["qpos"], a["out"],
                                a["lse"], a["B"], a["Lmax"], a["Hq"], a["Hkv"], a["d"], a["base"],
                                a["alpha"], a["scale"], a["dtype"], a["odt"], a["cnt"], a["chunk"],
                                a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=80), wpa.WPA_ERR_UNSUPPORTED),
    (dict(Hq=34, Hkv=2), wpa.WPA_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), wpa.WPA_ERR_INVALID),
    (dict(chunk=100), wpa.WPA_ERR_INVALID),
    (dict(odt=-1), wpa.WPA_ERR_INVALID),
    (dict(chunk=-256), wpa.WPA_ERR_INVALID),
    (dict(lens=None), wpa.WPA_ERR_INVALID),
    (dict(alpha=float("nan")), wpa.WPA_ERR_INVALID),
    (dict(ws_bytes=64), wpa.WPA_ERR_WORKSPACE),
])
def test_decode_rejects_bad_arguments(kw, code):
    assert _decode_rc(**kw) == code


def _cached_rc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, out=FAKE, lse=None, B=2, Nq=64, Lmax=4096,
             Hq=8, Hkv=2, d=128, base=5e5, rope=None, alpha=1.0, scale=0.0, dtype=0, odt=1,
             cnt=None)
    a.update(kw)
    return wpa.lib().wpa_prefill_cached(a["q"], a["kc"], a["vc"], a["lens"], a["out"], a["lse"],
                                        a["B"], a["Nq"], a["Lmax"], a["Hq"], a["Hkv"], a["d"],
                                        a["base"], a["rope"], a["alpha"], a["scale"], a["dtype"],
                                        a["odt"], a["cnt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), wpa.WPA_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), wpa.WPA_ERR_INVALID),
    (dict(Nq=0), wpa.WPA_ERR_INVALID),
    (dict(Nq=5000), wpa.WPA_ERR_INVALID),
    (dict(Lmax=0), wpa.WPA_ERR_INVALID),
    (dict(lens=None), wpa.WPA_ERR_INVALID),
    (dict(kc=None), wpa.WPA_ERR_INVALID),
    (dict(lens=ctypes.c_void_p((1 << 20) + 2)), wpa.WPA_ERR_INVALID),
    (dict(vc=ctypes.c_void_p((1 << 20) + 8)), wpa.WPA_ERR_INVALID),
    (dict(odt=3), wpa.WPA_ERR_INVALID),
    (dict(alpha=-2.0), wpa.WPA_ERR_INVALID),
    (dict(scale=float("nan")), wpa.WPA_ERR_INVALID),
])
def test_prefill_cached_rejects_bad_arguments(kw, code):
    assert _cached_rc(**kw) == code
    assert wpa.lib().wpa_last_error().decode() != ""


def _cached_ex_rc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, table=None, npages=0, psize=0, cu=None, lens=FAKE,
             out=FAKE, lse=None, B=2, Nq=64, Lmax=4096, Hq=8, Hkv=2, d=128, base=5e5, rope=None,
             alpha=1.0, scale=0.0, dtype=0, odt=1, cnt=None, splits=4, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(kw)
    return wpa.lib().wpa_prefill_cached_ex(
        a["q"], a["kc"], a["vc"], a["table"], a["npages"], a["psize"], a["cu"], a["lens"],
        a["out"], a["lse"], a["B"], a["Nq"], a["Lmax"], a["Hq"], a["Hkv"], a["d"], a["base"],
        a["rope"], a["alpha"], a["scale"], a["dtype"], a["odt"], a["cnt"], a["splits"], a["ws"],
        a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(splits=-1), wpa.WPA_ERR_INVALID),
    (dict(splits=17), wpa.WPA_ERR_INVALID),
    (dict(splits=2, ws=None, ws_bytes=0), wpa.WPA_ERR_INVALID),          # splits need room
    (dict(splits=4, ws_bytes=3 * 2 * 64 * 8 * 129 * 4), wpa.WPA_ERR_INVALID),   # room for 3
    (dict(ws=ctypes.c_void_p((1 << 20) + 4)), wpa.WPA_ERR_INVALID),      # misaligned workspace
    (dict(cu=ctypes.c_void_p((1 << 20) + 2)), wpa.WPA_ERR_INVALID),      # misaligned cu_q
    (dict(table=FAKE, npages=16, psize=16), wpa.WPA_ERR_INVALID),        # pages below 32
    (dict(table=FAKE, npages=16, psize=384), wpa.WPA_ERR_INVALID),       # not a power of two
    (dict(table=FAKE, npages=16, psize=256, Lmax=4000), wpa.WPA_ERR_INVALID),
    (dict(d=96), wpa.WPA_ERR_UNSUPPORTED),
    (dict(Nq=5000), wpa.WPA_ERR_INVALID),
    (dict(rope=None, alpha=float("nan")), wpa.WPA_ERR_INVALID),
])
def test_prefill_cached_ex_rejects_bad_arguments(kw, code):
    assert _cached_ex_rc(**kw) == code
    assert wpa.lib().wpa_last_error().decode() != ""


def test_prefill_cached_workspace_bytes():
    f = wpa.lib().wpa_prefill_cached_workspace_bytes
    # explicit counts: splits * B * Nq * Hq * (d + 1) floats
    assert f(2, 64, 8, 2, 128, 4) == 4 * 2 * 64 * 8 * 129 * 4
    assert f(1, 4096, 14, 2, 64, 2) == 2 * 4096 * 14 * 65 * 4
    assert f(1, 64, 8, 2, 128, 1) == 0            # no splits, no room
    for bad in ((0, 64, 8, 2, 128, 2), (1, 64, 8, 3, 128, 2), (1, 64, 8, 2, 96, 2),
                (1, 64, 8, 2, 128, 17), (1, 64, 8, 2, 128, -1)):
        assert f(*bad) == 0
    # the launch's own choice: a multiple of one split's room, at most 16 of them
    per = 1 * 4096 * 14 * 65 * 4
    auto = f(1, 4096, 14, 2, 64, 0)
    assert auto % per == 0 and auto // per in range(0, 17)
    assert f(1, 1 << 20, 28, 4, 128, 0) == 0      # rows enough to fill the GPU: no splits


def test_kv_write_rejects_out_of_range():
    L = wpa.lib()
    rc = L.wpa_kv_write(FAKE, FAKE, 4000, 200, FAKE, FAKE, 1, 4096, 2, 64, 1e4, 0, None)
    assert rc == wpa.WPA_ERR_INVALID
    rc = L.wpa_kv_write(FAKE, FAKE, -1, 1, FAKE, FAKE, 1, 4096, 2, 64, 1e4, 0, None)
    assert rc == wpa.WPA_ERR_INVALID


def test_workspace_sizes():
    assert wpa.prefill_workspace_bytes(1, 100, 2, 64) == 2 * 1 * 2 * 128 * 64 * 2
    assert wpa.kcache_bytes(2, 1000, 4, 128) == 2 * 4 * 1000 * 128 * 2
    ws = wpa.decode_workspace_bytes(16, 131072, 24, 8, 128, 4096)
    assert ws == 16 * 8 * 32 * 3 * 130 * 4


def test_count_rejects_bad_arguments():
    kept, total = ctypes.c_int64(), ctypes.c_int64()
    L = wpa.lib()
    assert L.wpa_count_terms(3, 1e4, 1.0, 1, 0, 1, ctypes.byref(kept), ctypes.byref(total)) == -1
    assert L.wpa_count_terms(64, 0.5, 1.0, 1, 0, 1, ctypes.byref(kept), ctypes.byref(total)) == -1
    assert L.wpa_count_terms(64, 1e4, -1.0, 1, 0, 1, ctypes.byref(kept), ctypes.byref(total)) == -1


# ------------------------------------------------------------------ RoPE variants

def _llama32_table(d=128):
    return wpa.llama3_inv_freq(d, 5e5, factor=32.0, low_freq_factor=1.0, high_freq_factor=4.0,
                               original_max_position=8192)


def test_llama3_inv_freq_matches_transformers():
    """The Llama-3 frequency-scaling helper against transformers' own (fp32) computation."""
    transformers = pytest.importorskip("transformers")
    from transformers import LlamaConfig
    from transformers import modeling_rope_utils as mru
    cfg = LlamaConfig(hidden_size=3072, num_attention_heads=24, num_key_value_heads=8, head_dim=128,
                      rope_theta=500000.0, max_position_embeddings=131072,
                      rope_scaling={"rope_type": "llama3", "factor": 32.0, "low_freq_factor": 1.0,
                                    "high_freq_factor": 4.0, "original_max_position_embeddings": 8192})
    ref, _ = mru._compute_llama3_parameters(cfg, "cpu")
    got = _llama32_table()
    assert np.allclose(got, ref.double().numpy(), rtol=2e-6, atol=0)
    assert np.all(np.diff(got) <= 0)                     # non-increasing, as the kernels need


@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0, 2.0, math.inf])
def test_table_count_matches_enumeration(alpha):
    theta = _llama32_table(64)
    for (n_q, q0, n_k) in [(1, 0, 1), (300, 0, 300), (1, 9999, 10000), (37, 250, 260)]:
        ref = oracle.count_by_distance(64, 5e5, alpha, n_q, q0, n_k, inv_freq=theta)
        assert wpa.count_terms(64, 5e5, alpha, n_q, q0, n_k, inv_freq=theta) == ref
    W = wpa.thresholds(64, 5e5, alpha, inv_freq=theta)
    thr = oracle.thresholds(64, 5e5, alpha, inv_freq=theta)
    assert W == [min(int(math.floor(t)), 2**31 - 1) if math.isfinite(t) else 2**31 - 1 for t in thr]


def test_rope_description_is_validated():
    L = wpa.lib()
    W = (ctypes.c_int32 * 32)()
    up = np.linspace(0.1, 1.0, 32)                       # increasing: suffix property broken
    r = wpa.Rope(0, up.ctypes.data)
    assert L.wpa_thresholds_ex(64, 1e4, ctypes.byref(r), 1.0, W) == wpa.WPA_ERR_UNSUPPORTED
    bad = np.full(32, 0.5)
    bad[3] = float("nan")
    r = wpa.Rope(0, bad.ctypes.data)
    assert L.wpa_thresholds_ex(64, 1e4, ctypes.byref(r), 1.0, W) == wpa.WPA_ERR_UNSUPPORTED
    r = wpa.Rope(7, None)
    assert L.wpa_thresholds_ex(64, 1e4, ctypes.byref(r), 1.0, W) == wpa.WPA_ERR_INVALID
    ok = _llama32_table(64)
    r = wpa.Rope(1, ok.ctypes.data)                      # a table makes `base` irrelevant
    assert L.wpa_thresholds_ex(64, 1.0, ctypes.byref(r), 1.0, W) == wpa.WPA_OK
    # the _ex entry points check the description before anything else
    rc = L.wpa_prefill_ex(FAKE, FAKE, FAKE, FAKE, None, None, 1, 128, 4, 2, 64, 1e4,
                          ctypes.byref(wpa.Rope(0, up.ctypes.data)), 1.0, 0.0, 0, 0, None, FAKE,
                          1 << 30, None)
    assert rc == wpa.WPA_ERR_UNSUPPORTED
    rc = L.wpa_decode_ex(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 2, 4096, 8, 2, 128, 1e4,
                         ctypes.byref(wpa.Rope(3, None)), 1.0, 0.0, 0, 0, None, 0, FAKE, 1 << 30,
                         None)
    assert rc == wpa.WPA_ERR_INVALID


def _window_rows_from_oracle(d, base, Lmax, alpha):
    """Rows per (sequence, kv head) of the windowed K cache, from the oracle's thresholds:
    block j keeps floor(alpha * lambda of pair 8j+7) + 1 tokens rounded up to 32, at most
    Lmax (all Lmax once that window reaches Lmax - 1)."""
    W = oracle.thresholds(d, base, alpha)
    rows = 0
    for j in range(d // 16):
        t = W[8 * j + 7]
        cap = Lmax if t >= Lmax - 1 else min(Lmax, (int(math.floor(t)) + 1 + 31) // 32 * 32)
        rows += cap
    return rows


@pytest.mark.parametrize("d,base,Lmax,alpha", [(128, 5e5, 131072, 1.0), (128, 5e5, 131072, 2.0),
                                               (128, 1e7, 1 << 20, 1.0), (64, 1e6, 32768, 1.0),
                                               (64, 1e4, 8192, 1.0), (64, 1e4, 100, 0.0),
                                               (128, 1e4, 5000, 0.25)])
def test_window_cache_size_matches_oracle_windows(d, base, Lmax, alpha):
    got = wpa.lib().wpa_kcache_window_bytes(3, Lmax, 2, d, base, None, alpha)
    assert got == 3 * 2 * _window_rows_from_oracle(d, base, Lmax, alpha) * 32
    assert got <= wpa.kcache_bytes(3, Lmax, 2, d)


def test_window_cache_llama_shape_saving():
    """Llama-3.2-3B shape at alpha = 1: the K cache shrinks to about a third."""
    w = wpa.lib().wpa_kcache_window_bytes(16, 131072, 8, 128, 5e5, None, 1.0)
    assert 0.30 < w / wpa.kcache_bytes(16, 131072, 8, 128) < 0.40


@pytest.mark.parametrize("alpha", [math.inf, float("nan"), -1.0])
def test_window_cache_rejects_bad_cache_alpha(alpha):
    assert wpa.lib().wpa_kcache_window_bytes(1, 4096, 2, 64, 1e4, None, alpha) == 0
    rc = wpa.lib().wpa_kv_write_window(FAKE, FAKE, 0, 16, FAKE, FAKE, 1, 4096, 2, 64, 1e4, None,
                                       alpha, 0, None)
    assert rc == wpa.WPA_ERR_INVALID


def _decode_window_rc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, out=FAKE, lse=None, B=2, Lmax=4096, Hq=8,
             Hkv=2, d=128, base=5e5, rope=None, calpha=1.0, alpha=1.0, scale=0.0, dtype=0,
             odt=1, cnt=None, chunk=0, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return wpa.lib().wpa_decode_window(a["q"], a["kc"], a["vc"], a["lens"], a["out"], a["lse"],
                                       a["B"], a["Lmax"], a["Hq"], a["Hkv"], a["d"], a["base"],
                                       a["rope"], a["calpha"], a["alpha"], a["scale"], a["dtype"],
                                       a["odt"], a["cnt"], a["chunk"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(alpha=2.0), wpa.WPA_ERR_INVALID),
    (dict(alpha=math.inf), wpa.WPA_ERR_INVALID),
    (dict(calpha=math.inf), wpa.WPA_ERR_INVALID),
    (dict(calpha=-0.5), wpa.WPA_ERR_INVALID),
    (dict(d=96), wpa.WPA_ERR_UNSUPPORTED),
    (dict(lens=None), wpa.WPA_ERR_INVALID),
    (dict(ws_bytes=64), wpa.WPA_ERR_WORKSPACE),
])
def test_decode_window_rejects_bad_arguments(kw, code):
    assert _decode_window_rc(**kw) == code


def test_kv_page_bytes():
    assert wpa.lib().wpa_kv_page_bytes(8, 128, 64) == 8 * 128 * 64 * 2
    assert wpa.lib().wpa_kv_page_bytes(2, 64, 32) == 2 * 64 * 32 * 2
    for hkv, d, ps in ((8, 128, 48), (8, 128, 16), (8, 96, 64), (0, 128, 64), (8, 128, 1 << 17)):
        assert wpa.lib().wpa_kv_page_bytes(hkv, d, ps) == 0


def _decode_paged_rc(**kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, table=FAKE, npages=16, lens=FAKE, qpos=None, out=FAKE,
             lse=None, B=2, maxp=8, ps=64, Hq=8, Hkv=2, d=128, base=5e5, rope=None, alpha=1.0,
             scale=0.0, dtype=0, odt=1, cnt=None, chunk=0, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return wpa.lib().wpa_decode_paged(a["q"], a["kp"], a["vp"], a["table"], a["npages"],
                                      a["lens"], a["qpos"], a["out"], a["lse"], a["B"], a["maxp"],
                                      a["ps"], a["Hq"], a["Hkv"], a["d"], a["base"], a["rope"],
                                      a["alpha"], a["scale"], a["dtype"], a["odt"], a["cnt"],
                                      a["chunk"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ps=48), wpa.WPA_ERR_INVALID),
    (dict(ps=16), wpa.WPA_ERR_INVALID),
    (dict(table=None), wpa.WPA_ERR_INVALID),
    (dict(npages=0), wpa.WPA_ERR_INVALID),
    (dict(maxp=0), wpa.WPA_ERR_INVALID),
    (dict(maxp=1 << 20, ps=4096), wpa.WPA_ERR_INVALID),
    (dict(d=96), wpa.WPA_ERR_UNSUPPORTED),
    (dict(Hq=7), wpa.WPA_ERR_INVALID),
    (dict(lens=None), wpa.WPA_ERR_INVALID),
    (dict(ws_bytes=64), wpa.WPA_ERR_WORKSPACE),
])
def test_decode_paged_rejects_bad_arguments(kw, code):
    assert _decode_paged_rc(**kw) == code


def _kv_write_paged_rc(**kw):
    a = dict(k=FAKE, v=FAKE, start=0, n=64, kp=FAKE, vp=FAKE, table=FAKE, npages=16, B=2,
             maxp=8, ps=64, Hkv=2, d=128, base=5e5, rope=None, dtype=0)
    a.update(kw)
    return wpa.lib().wpa_kv_write_paged(a["k"], a["v"], a["start"], a["n"], a["kp"], a["vp"],
                                        a["table"], a["npages"], a["B"], a["maxp"], a["ps"],
                                        a["Hkv"], a["d"], a["base"], a["rope"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(start=480, n=64), wpa.WPA_ERR_INVALID),      # past 8 pages of 64
    (dict(n=0), wpa.WPA_ERR_INVALID),
    (dict(ps=100), wpa.WPA_ERR_INVALID),
    (dict(table=None), wpa.WPA_ERR_INVALID),
    (dict(d=80), wpa.WPA_ERR_UNSUPPORTED),
    (dict(kp=None), wpa.WPA_ERR_INVALID),
])
def test_kv_write_paged_rejects_bad_arguments(kw, code):
    assert _kv_write_paged_rc(**kw) == code


def _prefill_paged_rc(**kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, table=FAKE, npages=16, lens=FAKE, out=FAKE, lse=None, B=2,
             Nq=64, maxp=8, ps=128, Hq=8, Hkv=2, d=128, base=5e5, rope=None, alpha=1.0, scale=0.0,
             dtype=0, odt=1, cnt=None)
    a.update(kw)
    return wpa.lib().wpa_prefill_paged(a["q"], a["kp"], a["vp"], a["table"], a["npages"],
                                       a["lens"], a["out"], a["lse"], a["B"], a["Nq"], a["maxp"],
                                       a["ps"], a["Hq"], a["Hkv"], a["d"], a["base"], a["rope"],
                                       a["alpha"], a["scale"], a["dtype"], a["odt"], a["cnt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ps=16), wpa.WPA_ERR_INVALID),              # a page must hold a 32-key tile
    (dict(ps=96), wpa.WPA_ERR_INVALID),
    (dict(table=None), wpa.WPA_ERR_INVALID),
    (dict(Nq=2000), wpa.WPA_ERR_INVALID),             # more rows than the table reaches
    (dict(d=96), wpa.WPA_ERR_UNSUPPORTED),
    (dict(lens=None), wpa.WPA_ERR_INVALID),
])
def test_prefill_paged_rejects_bad_arguments(kw, code):
    assert _prefill_paged_rc(**kw) == code


def test_prefill_varlen_needs_cu_q():
    rc = wpa.lib().wpa_prefill_cached_varlen(FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 2, 64,
                                             4096, 8, 2, 128, 5e5, None, 1.0, 0.0, 0, 1, None,
                                             None)
    assert rc == wpa.WPA_ERR_INVALID
    rc = wpa.lib().wpa_prefill_paged_varlen(FAKE, FAKE, FAKE, FAKE, 16, None, FAKE, FAKE, None,
                                            2, 64, 8, 128, 8, 2, 128, 5e5, None, 1.0, 0.0, 0, 1,
                                            None, None)
    assert rc == wpa.WPA_ERR_INVALID


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libwpa.so the binding raises: there is no fallback path."""
    monkeypatch.setattr(wpa, "_lib", None)
    monkeypatch.setattr(wpa, "LIB_PATH", str(tmp_path / "libwpa.so"))
    with pytest.raises(RuntimeError, match="not built"):
        wpa.lib()
    with pytest.raises(RuntimeError, match="not built"):
        wpa.count_terms(64, 1e4, 1.0, 16, 0, 16)


# ---------------------------------------------------------------- binding argument checks
# The binding must reject a wrongly shaped or typed caller buffer before any library call.
# CPU tensors stand in for device tensors here: the device test is relaxed to contiguity.

@pytest.fixture
def cpu_as_device(monkeypatch):
    import torch

    def dev(t, name):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    monkeypatch.setattr(wpa, "_dev", dev)

    def no_call(*a, **k):
        raise AssertionError("a rejected call reached the library")
    for name in ("wpa_prefill_ex", "wpa_prefill_attend_ex", "wpa_prefill_prepare_ex", "wpa_decode_ex",
                 "wpa_prefill_cached", "wpa_prefill_sparse", "wpa_prefill_cached_ex",
                 "wpa_prefill_sparse_ex", "wpa_prefill_sparse_pos"):
        monkeypatch.setattr(wpa.lib(), name, no_call)
    return torch


def _pf(torch, B=1, N=64, Hq=4, Hkv=2, d=64):
    q = torch.zeros((B, N, Hq, d), dtype=torch.bfloat16)
    k = torch.zeros((B, N, Hkv, d), dtype=torch.bfloat16)
    return q, k, k.clone()


@pytest.mark.parametrize("case", ["out_shape", "out_dtype", "lse_shape", "lse_dtype", "count_empty",
                                  "count_dtype", "positions_dtype", "positions_size"])
def test_binding_rejects_bad_prefill_buffers(cpu_as_device, case):
    torch = cpu_as_device
    q, k, v = _pf(torch)
    kw = {}
    if case == "out_shape":
        kw["out"] = torch.empty((1, 64, 4, 32), dtype=torch.bfloat16)
    elif case == "out_dtype":
        kw["out"] = torch.empty((1, 64, 4, 64), dtype=torch.float16)
    elif case == "lse_shape":
        kw["lse"] = torch.empty((1, 64, 4), dtype=torch.float32)
    elif case == "lse_dtype":
        kw["lse"] = torch.empty((1, 4, 64), dtype=torch.bfloat16)
    elif case == "count_empty":
        kw["term_count"] = torch.empty((0,), dtype=torch.int64)
    elif case == "count_dtype":
        kw["term_count"] = torch.zeros((1,), dtype=torch.int32)
    elif case == "positions_dtype":
        kw["positions"] = torch.zeros((1, 64), dtype=torch.int64)
    elif case == "positions_size":
        kw["positions"] = torch.zeros((1, 63), dtype=torch.int32)
    with pytest.raises(ValueError):
        wpa.prefill(q, k, v, 1e4, 1.0, **kw)
    ws = torch.empty(wpa.prefill_workspace_bytes(1, 64, 2, 64), dtype=torch.uint8)
    if case.startswith(("out", "lse", "count", "positions")):
        with pytest.raises(ValueError):
            wpa.prefill_attend(q, ws, 2, 1e4, 1.0, **kw)


def test_binding_rejects_bad_decode_buffers(cpu_as_device, monkeypatch):
    torch = cpu_as_device

    class FakeCache:                      # a dense cache's attributes, host memory
        B, Lmax, Hkv, d, base, inv_freq, pairs, window_alpha = 2, 256, 2, 64, 1e4, None, "half", None
        k = torch.empty(16, dtype=torch.uint8)
        v = torch.empty(16, dtype=torch.uint8)
    q = torch.zeros((2, 4, 64), dtype=torch.bfloat16)
    lens = torch.full((2,), 100, dtype=torch.int32)
    bad = [dict(out=torch.empty((2, 4, 32), dtype=torch.bfloat16)),
           dict(lse=torch.empty((4, 2), dtype=torch.float32)),
           dict(lse=torch.empty((2, 4), dtype=torch.float64)),
           dict(term_count=torch.empty((0,), dtype=torch.int64)),
           dict(q_pos=torch.zeros((3,), dtype=torch.int32))]
    for kw in bad:
        with pytest.raises(ValueError):
            wpa.decode(q, FakeCache(), lens, 1.0, **kw)
    with pytest.raises(ValueError):                          # q of the wrong rank
        wpa.decode(q[0], FakeCache(), lens, 1.0)


def test_per_head_tables_are_validated_on_the_host():
    """The binding checks per-kv-head rows before uploading them; the C ABI refuses per-head
    tables where it does not take them, and both inv_freq and head_inv_freq at once."""
    import torch
    d, Hkv = 64, 2
    good = np.stack([wpa.default_inv_freq(d, 1e4), wpa.default_inv_freq(d, 1e6)])
    for bad in (good[:, ::-1].copy(), -good, good[:1]):
        with pytest.raises(ValueError):
            wpa.head_table(bad, d, Hkv, "cpu")
    assert wpa.head_table(good, d, Hkv, "cpu").dtype == torch.float64
    # host-only queries take one row at a time
    kept, total = wpa.count_terms_heads(d, 1.0, 300, 0, 300, good, 3)
    assert kept == 3 * (wpa.count_terms(d, 1e4, 1.0, 300, 0, 300)[0] +
                        wpa.count_terms(d, 1e6, 1.0, 300, 0, 300)[0])
    r = wpa.Rope(0, None, ctypes.c_void_p(1 << 20).value)
    W = (ctypes.c_int32 * (d // 2))()
    assert wpa.lib().wpa_thresholds_ex(d, 1e4, ctypes.byref(r), 1.0, W) == wpa.WPA_ERR_UNSUPPORTED
    r2 = wpa.Rope(0, good[0].ctypes.data, ctypes.c_void_p(1 << 20).value)
    assert _prefill_ex_rc(ctypes.byref(r2)) == wpa.WPA_ERR_INVALID
    r3 = wpa.Rope(0, None, ctypes.c_void_p((1 << 20) + 4).value)
    assert _prefill_ex_rc(ctypes.byref(r3)) == wpa.WPA_ERR_INVALID


def _prefill_ex_rc(rope):
    L = wpa.lib()
    return L.wpa_prefill_ex(FAKE, FAKE, FAKE, FAKE, None, None, 1, 128, 4, 2, 64, 1e4, rope, 1.0, 0.0,
                            0, 0, None, FAKE, 1 << 30, None)


# ---------------------------------------------------------------- debug mode (host side)

def test_debug_mode_switch():
    L = wpa.lib()
    was = L.wpa_set_debug(-1)
    try:
        assert L.wpa_set_debug(1) == was
        assert L.wpa_set_debug(-1) == 1 and wpa.set_debug(None) is True
        assert L.wpa_set_debug(0) == 1
        assert L.wpa_set_debug(-1) == 0
    finally:
        L.wpa_set_debug(was)


@pytest.mark.parametrize("value,on", [("1", 1), ("yes", 1), ("0", 0), ("", 0)])
def test_debug_mode_from_environment(value, on):
    import subprocess
    import sys
    code = "import ctypes, sys; print(ctypes.CDLL(sys.argv[1]).wpa_set_debug(-1))"
    env = dict(os.environ, WPA_DEBUG=value)
    r = subprocess.run([sys.executable, "-c", code, wpa.LIB_PATH], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == str(on)


def test_debug_mode_checks_after_argument_checks():
    """Argument errors keep their codes in debug mode; arguments that pass them meet the
    buffer checks, which reject a pointer outside every allocation before any launch."""
    L = wpa.lib()
    was = L.wpa_set_debug(1)
    try:
        assert _cached_rc(d=96) == wpa.WPA_ERR_UNSUPPORTED
        assert _cached_rc(Nq=5000) == wpa.WPA_ERR_INVALID
        assert "debug" not in L.wpa_last_error().decode()
        assert _cached_rc() == wpa.WPA_ERR_INVALID
        assert L.wpa_last_error().decode().startswith("debug: kv_len")
        assert _cached_ex_rc(splits=0) == wpa.WPA_ERR_INVALID
        assert L.wpa_last_error().decode().startswith("debug:")
    finally:
        L.wpa_set_debug(was)


def _sparse_ex_rc(block, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, cnt_l=FAKE, idx=FAKE, bmax=4, B=1, N=4096,
             Hq=4, Hkv=2, d=64, base=1e4, alpha=1.0, scale=0.0, dtype=0, odt=0, cnt=None, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(kw)
    return wpa.lib().wpa_prefill_sparse_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["cnt_l"],
                                           a["idx"], a["bmax"], block, a["B"], a["N"], a["Hq"],
                                           a["Hkv"], a["d"], a["base"], None, a["alpha"], a["scale"],
                                           a["dtype"], a["odt"], a["cnt"], a["ws"], a["ws_bytes"],
                                           None)


@pytest.mark.parametrize("block", [0, 32, 96, 100, 2048, -64])
def test_sparse_block_size_is_checked_first(block):
    """Block sizes that are not a power of two from 64 to 1024 are refused before anything
    is enqueued, with the reason in the error text."""
    assert _sparse_ex_rc(block) == wpa.WPA_ERR_INVALID
    assert "block must be" in wpa.lib().wpa_last_error().decode()


def test_sparse_lists_rejected_like_the_64_block_entry():
    """The other argument checks of the block-size entry run for every block size."""
    for block in (64, 128, 1024):
        assert _sparse_ex_rc(block, cnt_l=None) == wpa.WPA_ERR_INVALID
        assert _sparse_ex_rc(block, bmax=-1) == wpa.WPA_ERR_INVALID
        assert _sparse_ex_rc(block, Hq=3) == wpa.WPA_ERR_INVALID
        assert _sparse_ex_rc(block, N=(1 << 21) + 1) == wpa.WPA_ERR_UNSUPPORTED


def test_binding_checks_sparse_block_and_list_shapes(cpu_as_device, monkeypatch):
    torch = cpu_as_device
    monkeypatch.setattr(wpa, "_stream", lambda s: None)
    q, k, v = _pf(torch, N=512)
    for block, nblk, ok in ((128, 4, True), (128, 8, False), (256, 2, True), (96, 6, False),
                            (2048, 1, False)):
        cnt = torch.zeros((1, 4, nblk), dtype=torch.int32)
        idx = torch.zeros((1, 4, nblk, 2), dtype=torch.int32)
        if ok:                      # shapes accepted: the call reaches the (stubbed) library
            with pytest.raises(AssertionError):
                wpa.prefill(q, k, v, 1e4, 1.0, block_count=cnt, block_idx=idx, block=block)
        else:
            with pytest.raises(ValueError):
                wpa.prefill(q, k, v, 1e4, 1.0, block_count=cnt, block_idx=idx, block=block)


def _sparse_pos_rc(pos, rope=None, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, cnt_l=FAKE, idx=FAKE, bmax=4, B=1, N=4096,
             Hq=4, Hkv=2, d=64, base=1e4, alpha=1.0, scale=0.0, dtype=0, odt=0, cnt=None, ws=FAKE,
             ws_bytes=1 << 30, block=64)
    a.update(kw)
    return wpa.lib().wpa_prefill_sparse_pos(a["q"], a["k"], a["v"], a["out"], a["lse"], a["cnt_l"],
                                            a["idx"], a["bmax"], a["block"], pos, a["B"], a["N"],
                                            a["Hq"], a["Hkv"], a["d"], a["base"], rope, a["alpha"],
                                            a["scale"], a["dtype"], a["odt"], a["cnt"], a["ws"],
                                            a["ws_bytes"], None)


def test_sparse_at_positions_host_checks():
    """The positions entry refuses a null or misaligned positions pointer and every argument
    the token-index entry refuses, before anything is enqueued."""
    L = wpa.lib()
    assert _sparse_pos_rc(None) == wpa.WPA_ERR_INVALID
    assert "positions" in L.wpa_last_error().decode()
    assert _sparse_pos_rc(ctypes.c_void_p((1 << 20) + 2)) == wpa.WPA_ERR_INVALID
    assert "positions" in L.wpa_last_error().decode()
    assert _sparse_pos_rc(FAKE, block=96) == wpa.WPA_ERR_INVALID
    assert _sparse_pos_rc(FAKE, cnt_l=None) == wpa.WPA_ERR_INVALID
    assert _sparse_pos_rc(FAKE, Hq=3) == wpa.WPA_ERR_INVALID
    assert _sparse_pos_rc(FAKE, N=(1 << 21) + 1) == wpa.WPA_ERR_UNSUPPORTED

"""Guard bands and debug mode on the GPU.

Guard bands: every output, gradient, workspace and cache buffer handed to the library sits
between two 4 KiB canary regions of one allocation.  After the call both canaries must be
byte-identical, and the results must equal (bitwise) those of the same call on ordinary
buffers.  So no kernel writes outside the bytes its arguments describe.

Debug mode (wpa_set_debug): a buffer shorter than the call needs, and each device-resident
value that breaks its precondition, is reported as WPA_ERR_INVALID before anything is
enqueued; with valid arguments the results are bit-identical to normal mode."""
import ctypes
import math

import numpy as np
import pytest
import torch

import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

G = 4096              # guard bytes on each side
CANARY = 0xA5


def _padded(shape, dtype):
    """A view of `shape` inside a uint8 buffer with G canary bytes on both sides."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((G + n + G,), CANARY, dtype=torch.uint8, device="cuda")
    return buf, buf[G:G + n].view(dtype).view(*shape)


def _untouched(buf, what):
    torch.cuda.synchronize()
    assert bool((buf[:G] == CANARY).all()), "%s: the guard before it was written" % what
    assert bool((buf[-G:] == CANARY).all()), "%s: the guard after it was written" % what


def _same(a, b, what):
    assert torch.equal(a, b), "%s differs from the call on ordinary buffers" % what


@pytest.fixture
def debug_mode():
    was = wpa.set_debug(True)
    yield
    wpa.set_debug(was)


# ------------------------------------------------------------------------------ guard bands

@pytest.mark.parametrize("d,Hq,Hkv,odt", [(64, 14, 2, torch.bfloat16), (128, 24, 8, torch.float32)])
def test_guard_prefill(d, Hq, Hkv, odt):
    need_gpu()
    B, N = 2, 333
    q, k, v = (t.cuda() for t in synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=40))
    say("guard prefill", d)
    ref, ref_lse = wpa.prefill(q, k, v, 1e4, 1.0, want_lse=True, out_dtype=odt)
    ob, out = _padded((B, N, Hq, d), odt)
    lb, lse = _padded((B, Hq, N), torch.float32)
    wb, ws = _padded((wpa.prefill_workspace_bytes(B, N, Hkv, d),), torch.uint8)
    cb, cnt = _padded((1,), torch.int64)
    cnt.zero_()
    wpa.prefill(q, k, v, 1e4, 1.0, out=out, lse=lse, workspace=ws, term_count=cnt)
    for b, name in ((ob, "out"), (lb, "lse"), (wb, "workspace"), (cb, "term_count")):
        _untouched(b, name)
    _same(out, ref, "out")
    _same(lse, ref_lse, "lse")


def test_guard_prefill_positions_and_sparse():
    need_gpu()
    B, N, Hq, Hkv, d = 1, 500, 4, 2, 64
    q, k, v = (t.cuda() for t in synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=41))
    pos = (torch.arange(N, dtype=torch.int32, device="cuda") * 3).view(1, N)
    say("guard prefill positions")
    ref = wpa.prefill(q, k, v, 1e4, 1.0, positions=pos)
    ob, out = _padded((B, N, Hq, d), torch.bfloat16)
    wpa.prefill(q, k, v, 1e4, 1.0, positions=pos, out=out)
    _untouched(ob, "out (positions)")
    _same(out, ref, "out (positions)")
    nblk = (N + 63) // 64
    cnt = torch.full((B, Hq, nblk), 2, dtype=torch.int32, device="cuda")
    idx = torch.zeros((B, Hq, nblk, 2), dtype=torch.int32, device="cuda")
    idx[..., 1] = torch.arange(nblk, dtype=torch.int32, device="cuda").view(1, 1, nblk) - 2
    say("guard prefill sparse")
    ref = wpa.prefill(q, k, v, 1e4, 1.0, block_count=cnt, block_idx=idx)
    ob, out = _padded((B, N, Hq, d), torch.bfloat16)
    wpa.prefill(q, k, v, 1e4, 1.0, block_count=cnt, block_idx=idx, out=out)
    _untouched(ob, "out (sparse)")
    _same(out, ref, "out (sparse)")


def _cache_with(B, Lmax, Hkv, d, base, lens, k, v):
    cache = wpa.KVCache(B, Lmax, Hkv, d, base)
    for b, L in enumerate(lens):
        cache.write(k[b:b + 1, :L].contiguous(), v[b:b + 1, :L].contiguous(), 0, seq=b)
    return cache


@pytest.mark.parametrize("splits", [1, 0, 3])
def test_guard_chunked_prefill(splits):
    need_gpu()
    B, Nq, Hq, Hkv, d, base = 2, 300, 14, 2, 64, 1e6
    lens = [700, 1300]
    Lmax = 1400
    q, k, v = (t.cuda() for t in synth.prefill_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=42))
    cache = _cache_with(B, Lmax, Hkv, d, base, lens, k, v)
    qc = torch.stack([q[b, L - Nq:L] for b, L in enumerate(lens)]).contiguous()
    kv_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    say("guard chunked", splits)
    ref, ref_lse = wpa.prefill_cached(qc, cache, kv_len, 1.0, want_lse=True, splits=splits)
    ob, out = _padded((B, Nq, Hq, d), torch.bfloat16)
    lb, lse = _padded((B, Hq, Nq), torch.float32)
    need = wpa.prefill_cached_workspace_bytes(B, Nq, Hq, Hkv, d, splits) if splits != 1 else 0
    wb, ws = _padded((max(need, 16),), torch.uint8)
    wpa.prefill_cached(qc, cache, kv_len, 1.0, out=out, lse=lse, splits=splits,
                       workspace=ws if need else None)
    _untouched(ob, "out")
    _untouched(lb, "lse")
    _untouched(wb, "workspace")
    _same(out, ref, "out")
    _same(lse, ref_lse, "lse")


def test_guard_varlen_paged_prefill():
    need_gpu()
    Hq, Hkv, d, base, page = 14, 2, 64, 1e6, 128
    qn, kv = [5, 0, 200], [300, 50, 900]
    B = len(qn)
    max_pages = (max(kv) + page - 1) // page
    q, k, v = (t.cuda() for t in synth.prefill_inputs(B, max_pages * page, Hq, Hkv, d, "bf16", seed=43))
    table = torch.arange(B * max_pages, dtype=torch.int32, device="cuda").flip(0).view(B, max_pages).contiguous()
    paged = wpa.PagedKVCache(B * max_pages, page, Hkv, d, base, block_table=table)
    for b, L in enumerate(kv):
        paged.write(k[b:b + 1, :L].contiguous(), v[b:b + 1, :L].contiguous(), 0, block_table=table[b:b + 1])
    cu = torch.tensor(np.concatenate([[0], np.cumsum(qn)]), dtype=torch.int32, device="cuda")
    qp = torch.cat([q[b, kv[b] - qn[b]:kv[b]] for b in range(B)]).contiguous()
    kv_len = torch.tensor(kv, dtype=torch.int32, device="cuda")
    say("guard varlen paged")
    ref, ref_lse = wpa.prefill_cached(qp, paged, kv_len, 1.0, cu_q=cu, max_q=max(qn), want_lse=True)
    rows = sum(qn)
    ob, out = _padded((rows, Hq, d), torch.bfloat16)
    lb, lse = _padded((rows, Hq), torch.float32)
    wpa.prefill_cached(qp, paged, kv_len, 1.0, cu_q=cu, max_q=max(qn), out=out, lse=lse)
    _untouched(ob, "out")
    _untouched(lb, "lse")
    _same(out, ref, "out")
    _same(lse, ref_lse, "lse")


def test_guard_decode_and_cache_writes():
    """Decode (with a workspace and through the entry point that allocates nothing) and the
    cache writes, each cache buffer padded as well: a write of tokens start .. start+n-1
    stays inside the caches."""
    need_gpu()
    B, Lmax, Hq, Hkv, d, base = 2, 1000, 14, 2, 64, 1e6
    q, k, v = (t.cuda() for t in synth.prefill_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=44))
    ref_cache = wpa.KVCache(B, Lmax, Hkv, d, base)
    cache = wpa.KVCache(B, Lmax, Hkv, d, base)
    kb, cache.k = _padded(tuple(cache.k.shape), cache.k.dtype)
    vb, cache.v = _padded(tuple(cache.v.shape), cache.v.dtype)
    cache.k.zero_()
    cache.v.zero_()
    ref_cache.k.zero_()
    ref_cache.v.zero_()
    say("guard cache writes")
    for s, n in ((0, 600), (600, 123), (723, 277)):
        for c in (ref_cache, cache):
            c.write(k[:, s:s + n].contiguous(), v[:, s:s + n].contiguous(), s)
    _untouched(kb, "k_cache")
    _untouched(vb, "v_cache")
    _same(cache.k, ref_cache.k, "k_cache")
    _same(cache.v, ref_cache.v, "v_cache")
    qd = q[:, -1].contiguous()
    kv_len = torch.tensor([1000, 517], dtype=torch.int32, device="cuda")
    say("guard decode")
    ref, ref_lse = wpa.decode(qd, ref_cache, kv_len, 1.0, want_lse=True)
    ob, out = _padded((B, Hq, d), torch.bfloat16)
    lb, lse = _padded((B, Hq), torch.float32)
    wb, ws = _padded((wpa.decode_workspace_bytes(B, Lmax, Hq, Hkv, d),), torch.uint8)
    wpa.decode(qd, cache, kv_len, 1.0, out=out, lse=lse, workspace=ws)
    for b_, name in ((ob, "out"), (lb, "lse"), (wb, "workspace")):
        _untouched(b_, name)
    _same(out, ref, "decode out")
    _same(lse, ref_lse, "decode lse")
    ob2, out2 = _padded((B, Hq, d), torch.bfloat16)
    lb2, lse2 = _padded((B, Hq), torch.float32)
    wpa.decode_noalloc(qd, cache, kv_len, 1.0, out=out2, lse=lse2)
    _untouched(ob2, "noalloc out")
    _untouched(lb2, "noalloc lse")
    _same(out2, ref, "noalloc out")


def test_guard_backward():
    need_gpu()
    B, N, Hq, Hkv, d = 1, 300, 6, 2, 128
    q, k, v = (t.cuda() for t in synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=45))
    g = torch.randn(q.shape, generator=torch.Generator().manual_seed(46)).to(torch.bfloat16).cuda()
    out, lse = wpa.prefill(q, k, v, 1e4, 1.0, want_lse=True, out_dtype=torch.float32)
    say("guard backward")
    rq, rk, rv = wpa.prefill_backward(q, k, v, out, lse, g, 1e4, 1.0)
    qb, dq = _padded(tuple(q.shape), torch.float32)
    kb, dk = _padded(tuple(k.shape), torch.float32)
    vb, dv = _padded(tuple(v.shape), torch.float32)
    wb, ws = _padded((wpa.prefill_backward_workspace_bytes(B, N, Hq, Hkv, d),), torch.uint8)
    # the workspace must be 256-byte aligned: G keeps the buffer's own alignment
    wpa.prefill_backward(q, k, v, out, lse, g, 1e4, 1.0, dq=dq, dk=dk, dv=dv, workspace=ws)
    for b_, name in ((qb, "dq"), (kb, "dk"), (vb, "dv"), (wb, "workspace")):
        _untouched(b_, name)
    _same(dq, rq, "dq")
    _same(dk, rk, "dk")
    _same(dv, rv, "dv")


# ------------------------------------------------------------------------------ debug mode

def test_debug_mode_results_identical(debug_mode):
    """Valid calls in debug mode pass its checks and give the results of normal mode."""
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 700, 14, 2, 64, 1e6
    q, k, v = (t.cuda() for t in synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=47))
    pos = torch.arange(N, dtype=torch.int32, device="cuda").view(1, N)
    say("debug: prefill")
    a = wpa.prefill(q, k, v, base, 1.0, positions=pos)
    cache = _cache_with(B, N, Hkv, d, base, [N], k, v)
    kv_len = torch.tensor([N], dtype=torch.int32, device="cuda")
    c = wpa.prefill_cached(q[:, -200:].contiguous(), cache, kv_len, 1.0, splits=3)
    dec = wpa.decode(q[:, -1].contiguous(), cache, kv_len, 1.0)
    wpa.set_debug(False)
    _same(a, wpa.prefill(q, k, v, base, 1.0, positions=pos), "prefill")
    _same(c, wpa.prefill_cached(q[:, -200:].contiguous(), cache, kv_len, 1.0, splits=3), "cached")
    _same(dec, wpa.decode(q[:, -1].contiguous(), cache, kv_len, 1.0), "decode")


def _hip():
    return ctypes.CDLL("libamdhip64.so")


def test_debug_mode_rejects_short_buffer(debug_mode):
    """An output allocation 16 bytes shorter than the call writes: WPA_ERR_INVALID naming it,
    and nothing enqueued (the buffer keeps its fill)."""
    need_gpu()
    B, N, Hq, Hkv, d = 1, 256, 2, 2, 64
    q, k, v = (t.cuda() for t in synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=48))
    ws = torch.empty(wpa.prefill_workspace_bytes(B, N, Hkv, d), dtype=torch.uint8, device="cuda")
    hip = _hip()
    nbytes = B * N * Hq * d * 2
    p = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(p), ctypes.c_size_t(nbytes - 16)) == 0
    try:
        assert hip.hipMemset(p, ctypes.c_int(0x3C), ctypes.c_size_t(nbytes - 16)) == 0
        assert hip.hipDeviceSynchronize() == 0
        say("debug: short out")
        rc = wpa.lib().wpa_prefill_ex(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            p, None, None, B, N, Hq, Hkv, d, 1e4, None, 1.0, 0.0, wpa.WPA_BF16, wpa.WPA_BF16, None,
            ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()), None)
        assert rc == wpa.WPA_ERR_INVALID
        assert "out" in wpa.lib().wpa_last_error().decode()
        host = (ctypes.c_uint8 * (nbytes - 16))()
        assert hip.hipMemcpy(host, p, ctypes.c_size_t(nbytes - 16), 2) == 0   # device to host
        assert set(bytes(host)) == {0x3C}
    finally:
        hip.hipFree(p)


def test_debug_mode_rejects_broken_device_values(debug_mode):
    """Each device-resident precondition, broken: the call raises (WPA_ERR_INVALID) and the
    message names it."""
    need_gpu()
    B, N, Hq, Hkv, d, base = 2, 300, 4, 2, 64, 1e4
    q, k, v = (t.cuda() for t in synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=49))

    def rejected(fn, word):
        with pytest.raises(wpa.WpaError) as e:
            fn()
        assert e.value.code == wpa.WPA_ERR_INVALID and word in str(e.value), str(e.value)

    say("debug: positions")
    pos = torch.arange(N, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    pos[1, 100] = 5                                            # decreases at 101
    rejected(lambda: wpa.prefill(q, k, v, base, 1.0, positions=pos), "positions")
    pos[1, 100] = -1
    rejected(lambda: wpa.prefill(q, k, v, base, 1.0, positions=pos), "negative")

    say("debug: head tables")
    # (the binding checks tables it is given on the host: the C ABI is called directly)
    th = torch.tensor(np.tile(base ** (-np.arange(d // 2) * 2.0 / d), (Hkv, 1)), device="cuda")
    th[1, 7] = th[1, 6] * 2                                    # grows
    rope = wpa.Rope(0, None, th.data_ptr())
    out = torch.empty_like(q)
    ws = torch.empty(wpa.prefill_workspace_bytes(B, N, Hkv, d), dtype=torch.uint8, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = wpa.lib().wpa_prefill_ex(P(q), P(k), P(v), P(out), None, None, B, N, Hq, Hkv, d, base,
                                  ctypes.byref(rope), 1.0, 0.0, wpa.WPA_BF16, wpa.WPA_BF16, None,
                                  P(ws), ctypes.c_size_t(ws.numel()), None)
    assert rc == wpa.WPA_ERR_INVALID and "head_inv_freq" in wpa.lib().wpa_last_error().decode()

    cache = _cache_with(B, N, Hkv, d, base, [N, N], k, v)
    say("debug: kv_len")
    qc = q[:, -64:].contiguous()
    bad = torch.tensor([N, 40], dtype=torch.int32, device="cuda")          # below Nq = 64
    rejected(lambda: wpa.prefill_cached(qc, cache, bad, 1.0), "kv_len")
    bad = torch.tensor([N, N + 1], dtype=torch.int32, device="cuda")       # past Lmax
    rejected(lambda: wpa.prefill_cached(qc, cache, bad, 1.0), "kv_len")

    say("debug: cu_q")
    cu = torch.tensor([0, 40, 30], dtype=torch.int32, device="cuda")       # decreasing
    qp = q[0, :40].contiguous()
    lens = torch.tensor([N, N], dtype=torch.int32, device="cuda")
    rejected(lambda: wpa.prefill_cached(qp, cache, lens, 1.0, cu_q=cu, max_q=40), "queries")

    say("debug: block table")
    page = 128
    table = torch.tensor([[0, 1, 2], [3, 4, 5]], dtype=torch.int32, device="cuda")
    paged = wpa.PagedKVCache(6, page, Hkv, d, base, block_table=table)
    paged.write(k[:, :N].contiguous(), v[:, :N].contiguous(), 0, block_table=table)
    broken = table.clone()
    broken[1, 2] = 6                                           # past the pool, reached by N=300
    lens = torch.tensor([N, N], dtype=torch.int32, device="cuda")
    rejected(lambda: wpa.decode(q[:, -1].contiguous(), paged, lens, 1.0, block_table=broken),
             "block_table")
    short = torch.tensor([N, 200], dtype=torch.int32, device="cuda")       # page 2 unreached
    wpa.decode(q[:, -1].contiguous(), paged, short, 1.0, block_table=broken)
    torch.cuda.synchronize()

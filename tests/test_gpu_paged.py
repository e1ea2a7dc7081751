"""GPU parity of decode on paged caches (a pool of pages and a block table): bit-identical to
decode on contiguous caches holding the same tokens (the same rotation, the same layouts inside
a page, the same split of the keys), and within tolerance of the fp64 oracle; shuffled and
shared pages, per-sequence appends that end inside a page and inside an octet, ragged
sequences, the full window and explicit query positions."""
import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, check_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _table(B, max_pages, num_pages, seed):
    """A block table whose rows use distinct, shuffled pages of a larger pool."""
    rng = np.random.default_rng(seed)
    pages = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages)
    return torch.from_numpy(pages.astype(np.int32)).cuda()


def _fill_nan(*caches):
    for c in caches:
        c.k.fill_(255)                      # NaN in half / bf16: stale slots must never count
        c.v.fill_(255)


def _decode_both(q, dense, paged, table, lens, alpha, **kw):
    cd = torch.zeros(1, dtype=torch.int64, device="cuda")
    cp = torch.zeros(1, dtype=torch.int64, device="cuda")
    od, ld = wpa.decode(q, dense, lens, alpha, out_dtype=torch.float32, want_lse=True,
                        term_count=cd, **kw)
    op, lp = wpa.decode(q, paged, lens, alpha, out_dtype=torch.float32, want_lse=True,
                        term_count=cp, block_table=table, **kw)
    torch.cuda.synchronize()
    assert torch.equal(od, op) and torch.equal(ld, lp), "paged cache differs from contiguous"
    assert int(cd.item()) == int(cp.item())
    return op, lp


@pytest.mark.parametrize("d,Hq,Hkv,base,page", [(128, 24, 8, 5e5, 32), (128, 24, 8, 5e5, 256),
                                                (64, 14, 2, 1e6, 64)])
def test_paged_decode_matches_contiguous_and_oracle(d, Hq, Hkv, base, page):
    """Ragged sequences written in one piece each into shuffled pages of a pool with unused
    pages; decode at alpha 1 and inf against the contiguous caches and the oracle."""
    need_gpu()
    B, max_pages = 3, (6000 + page - 1) // page
    Lmax = max_pages * page
    q, k, v, _ = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=81)
    lens_h = [Lmax, 4001, 77]
    table = _table(B, max_pages, B * max_pages + 5, seed=page)
    dense = wpa.KVCache(B, Lmax, Hkv, d, base)
    paged = wpa.PagedKVCache(B * max_pages + 5, page, Hkv, d, base)
    _fill_nan(dense, paged)
    for b, L in enumerate(lens_h):
        kk, vv = k[b:b + 1, :L].cuda().contiguous(), v[b:b + 1, :L].cuda().contiguous()
        dense.write(kk, vv, 0, seq=b)
        paged.write(kk, vv, 0, block_table=table[b:b + 1])
    lens = torch.tensor(lens_h, dtype=torch.int32, device="cuda")
    for alpha in (1.0, float("inf")):
        say("paged decode", d, page, alpha)
        out, lse = _decode_both(q.cuda(), dense, paged, table, lens, alpha)
        ro, rl, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                     np.array(lens_h), base, alpha)
        check_close(out.cpu().numpy(), ro, "decode out")
        check_close(lse.cpu().numpy(), rl, "decode lse", LSE_MAX, LSE_MAX)


def test_paged_incremental_appends_and_chunks():
    """d=64, pages of 32: appends of 1, 5, 37, 300 and 2000 tokens (ending inside pages and
    inside octets) to all sequences at once, a decode after each, with the default and two
    fixed split sizes."""
    need_gpu()
    B, page, max_pages, Hq, Hkv, d, base = 2, 32, 80, 8, 2, 64, 1e4
    Lmax = page * max_pages
    q, k, v, _ = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=82)
    table = _table(B, max_pages, B * max_pages, seed=3)
    dense = wpa.KVCache(B, Lmax, Hkv, d, base)
    paged = wpa.PagedKVCache(B * max_pages, page, Hkv, d, base, block_table=table)
    _fill_nan(dense, paged)
    qc, t = q.cuda(), 0
    for n in (1, 5, 37, 300, 2000, 217):
        kk, vv = k[:, t:t + n].cuda().contiguous(), v[:, t:t + n].cuda().contiguous()
        dense.write(kk, vv, t)
        paged.write(kk, vv, t)
        t += n
        lens = torch.full((B,), t, dtype=torch.int32, device="cuda")
        for ch in (0, 256, 1024):
            say("paged append", t, "chunk", ch)
            out, lse = _decode_both(qc, dense, paged, table, lens, 1.0, chunk_keys=ch)
    assert t == Lmax
    ro, rl, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 np.full(B, Lmax), base, 1.0)
    check_close(out.cpu().numpy(), ro, "decode out")


def test_paged_shared_prefix_pages():
    """Two sequences share the pages of a common 1024-token prefix (written once) and then
    diverge; explicit query positions.  Each must equal its own contiguous cache."""
    need_gpu()
    page, Hq, Hkv, d, base = 128, 8, 4, 128, 1e6
    pre, tail = 1024, 700
    Lmax = pre + 1024
    q, k, v, _ = synth.decode_inputs(2, Lmax, Hq, Hkv, d, "bf16", seed=83)
    k[1, :pre] = k[0, :pre]
    v[1, :pre] = v[0, :pre]
    npp = pre // page                           # shared pages 0 .. npp-1
    mp = Lmax // page
    rows = [list(range(npp)) + [npp + i for i in range(mp - npp)],
            list(range(npp)) + [mp + i for i in range(mp - npp)]]
    table = torch.tensor(rows, dtype=torch.int32, device="cuda")
    paged = wpa.PagedKVCache(2 * mp - npp, page, Hkv, d, base)
    dense = wpa.KVCache(2, Lmax, Hkv, d, base)
    _fill_nan(dense, paged)
    paged.write(k[0:1, :pre].cuda().contiguous(), v[0:1, :pre].cuda().contiguous(), 0,
                block_table=table[0:1])
    for b in range(2):
        paged.write(k[b:b + 1, pre:pre + tail].cuda().contiguous(),
                    v[b:b + 1, pre:pre + tail].cuda().contiguous(), pre, block_table=table[b:b + 1])
        dense.write(k[b:b + 1, :pre + tail].cuda().contiguous(),
                    v[b:b + 1, :pre + tail].cuda().contiguous(), 0, seq=b)
    lens = torch.full((2,), pre + tail, dtype=torch.int32, device="cuda")
    qpos = torch.tensor([pre + tail + 5, pre + tail + 100000], dtype=torch.int32, device="cuda")
    say("paged shared prefix")
    out, lse = _decode_both(q.cuda(), dense, paged, table, lens, 1.0, q_pos=qpos)
    ro, rl, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 np.full(2, pre + tail), base, 1.0, q_pos=qpos.cpu().numpy())
    check_close(out.cpu().numpy(), ro, "decode out")


def test_paged_rejects_misuse():
    need_gpu()
    paged = wpa.PagedKVCache(4, 64, 2, 64, 1e4)
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((1,), 64, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        wpa.decode(q, paged, lens, 1.0)                # no block table
    with pytest.raises(ValueError):
        wpa.PagedKVCache(4, 48, 2, 64, 1e4)            # page size not a power of two
    table = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    kk = torch.zeros((1, 200, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        paged.write(kk, kk, 0, block_table=table)     # 200 tokens > 2 pages of 64


@pytest.mark.parametrize("d,Hq,Hkv,base,page", [(64, 14, 2, 1e6, 128), (128, 24, 8, 5e5, 256),
                                                 (64, 14, 2, 1e6, 32), (128, 24, 8, 5e5, 64)])
def test_paged_chunked_prefill_matches_contiguous_and_oracle(d, Hq, Hkv, base, page):
    """Ragged prompts whose last 300 tokens are attended as a chunk against shuffled pages
    (pages of 32 and 64 tokens: a 128-key tile spans 4 or 2 of them): bit-identical to the same
    chunk against contiguous caches, and within tolerance of the oracle's rows."""
    need_gpu()
    B, Nq = 3, 300
    lens_h = [Nq, Nq + 777, Nq + 2000]
    max_pages = (max(lens_h) + page - 1) // page + 1
    Lmax = max_pages * page
    q, k, v = synth.prefill_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=84)
    table = _table(B, max_pages, B * max_pages + 3, seed=page + 1)
    dense = wpa.KVCache(B, Lmax, Hkv, d, base)
    paged = wpa.PagedKVCache(B * max_pages + 3, page, Hkv, d, base, block_table=table)
    _fill_nan(dense, paged)
    for b, L in enumerate(lens_h):
        kk, vv = k[b:b + 1, :L].cuda().contiguous(), v[b:b + 1, :L].cuda().contiguous()
        dense.write(kk, vv, 0, seq=b)
        paged.write(kk, vv, 0, block_table=table[b:b + 1])
    qc = torch.stack([q[b, L - Nq:L] for b, L in enumerate(lens_h)]).contiguous().cuda()
    kv_len = torch.tensor(lens_h, dtype=torch.int32, device="cuda")
    cd = torch.zeros(1, dtype=torch.int64, device="cuda")
    cp = torch.zeros(1, dtype=torch.int64, device="cuda")
    say("paged chunked prefill", d, page)
    od, ld = wpa.prefill_cached(qc, dense, kv_len, 1.0, want_lse=True, term_count=cd,
                                out_dtype=torch.float32)
    op, lp = wpa.prefill_cached(qc, paged, kv_len, 1.0, want_lse=True, term_count=cp,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(od, op) and torch.equal(ld, lp), "paged chunk differs from contiguous"
    assert int(cd.item()) == int(cp.item())
    for b, L in enumerate(lens_h):
        ro, rl, kept = oracle.prefill(synth.to_oracle(q[b:b + 1, :L]), synth.to_oracle(k[b:b + 1, :L]),
                                      synth.to_oracle(v[b:b + 1, :L]), base, 1.0,
                                      rows=np.arange(L - Nq, L))
        check_close(op[b:b + 1].cpu().numpy(), ro, "out[%d]" % b)
        check_close(lp[b:b + 1].cpu().numpy(), rl, "lse[%d]" % b, LSE_MAX, LSE_MAX)

"""GPU parity of the RoPE variants (a per-pair frequency table, e.g. Llama-3 frequency
scaling, and the interleaved pair layout) against the fp64 oracle given the same
description: prefill, cache write and decode, with kept-term counts."""
import math

import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, as_bf16_for_oracle, check_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _table(kind, d, base):
    if kind == "llama3":
        return wpa.llama3_inv_freq(d, base, factor=32.0, low_freq_factor=1.0,
                                   high_freq_factor=4.0, original_max_position=8192)
    return None


VARIANTS = [("llama3", "half"), (None, "interleaved"), ("llama3", "interleaved")]


@pytest.mark.parametrize("alpha", [1.0, 2.0])
@pytest.mark.parametrize("table,pairs", VARIANTS)
@pytest.mark.parametrize("shape", [
    (1, 700, 14, 2, 64, 1e6),          # Qwen2.5-0.5B heads
    (2, 400, 24, 8, 128, 5e5),         # Llama-3.2-3B heads (the model scales its frequencies)
])
def test_prefill_variants_match_oracle(shape, table, pairs, alpha):
    need_gpu()
    B, N, Hq, Hkv, d, base = shape
    theta = _table(table, d, base)
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=50 + N)
    say("prefill variant", shape, table, pairs, alpha)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lse = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), base, alpha, want_lse=True,
                           term_count=cnt, out_dtype=torch.float32, inv_freq=theta, pairs=pairs)
    torch.cuda.synchronize()
    ro, rl, kept = oracle.prefill(as_bf16_for_oracle(q), as_bf16_for_oracle(k),
                                  as_bf16_for_oracle(v), base, alpha, inv_freq=theta, layout=pairs)
    check_close(out.cpu().numpy(), ro, "out")
    check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
    closed = wpa.count_terms(d, base, alpha, N, 0, N, inv_freq=theta, pairs=pairs)[0]
    assert int(cnt.item()) == kept == B * Hq * closed


def test_scaled_frequencies_change_the_window():
    """The table is what the kernels use: with Llama-3 scaling the far pairs' windows are 32x
    longer, so more terms are kept than with the plain frequencies of the same base."""
    need_gpu()
    d, base, N = 128, 5e5, 20000
    theta = _table("llama3", d, base)
    plain = wpa.count_terms(d, base, 1.0, N, 0, N)[0]
    scaled = wpa.count_terms(d, base, 1.0, N, 0, N, inv_freq=theta)[0]
    assert scaled > plain


@pytest.mark.parametrize("table,pairs", VARIANTS)
def test_kv_write_variant_rotation(table, pairs):
    """The K cache holds keys rotated by the description given to the cache."""
    need_gpu()
    B, L, Hkv, d, base = 2, 200, 2, 128, 5e5
    theta = _table(table, d, base)
    k, v = synth.prefill_inputs(B, L, Hkv, Hkv, d, "bf16", seed=61)[1:]
    say("kv_write variant", table, pairs)
    cache = wpa.KVCache(B, L, Hkv, d, base, inv_freq=theta, pairs=pairs)
    cache.write(k.cuda().contiguous(), v.cuda().contiguous(), 0)
    torch.cuda.synchronize()
    kb = cache.k.view(torch.float16).view(B, Hkv, d // 16, L, 16).float().cpu()
    P = d // 2
    x = kb[..., :8].permute(0, 3, 1, 2, 4).reshape(B, L, Hkv, P).numpy()      # pair i, first comp.
    y = kb[..., 8:].permute(0, 3, 1, 2, 4).reshape(B, L, Hkv, P).numpy()
    for b in range(B):
        ref = oracle.rope(synth.to_oracle(k[b]), np.arange(L), base, inv_freq=theta, layout=pairs)
        if pairs == "interleaved":
            rx, ry = ref[..., 0::2], ref[..., 1::2]
        else:
            rx, ry = ref[..., :P], ref[..., P:]
        for got, want in ((x[b], rx), (y[b], ry)):
            err = np.abs(got - want)
            assert (err <= 2 ** -11 * np.abs(want) + 4e-6 * (np.abs(want).max() + 1e-3)).all()


@pytest.mark.parametrize("alpha", [1.0, 2.0, math.inf])
@pytest.mark.parametrize("table,pairs", VARIANTS)
def test_decode_variants_match_oracle(table, pairs, alpha):
    need_gpu()
    B, Lmax, Hq, Hkv, d, base = 3, 3000, 24, 8, 128, 5e5
    theta = _table(table, d, base)
    q, k, v, lens = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=63, len_lo=500)
    say("decode variant", table, pairs, alpha, lens.tolist())
    cache = wpa.KVCache(B, Lmax, Hkv, d, base, inv_freq=theta, pairs=pairs)
    cache.write(k.cuda(), v.cuda(), 0)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = wpa.decode(q.cuda(), cache, lens.cuda(), alpha, out_dtype=torch.float32, term_count=cnt)
    torch.cuda.synchronize()
    ro, _, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                lens.numpy(), base, alpha, inv_freq=theta, layout=pairs)
    check_close(out.cpu().numpy(), ro, "decode out")
    closed = sum(wpa.count_terms(d, base, alpha, 1, int(L) - 1, int(L), inv_freq=theta)[0]
                 for L in lens.tolist())
    assert int(cnt.item()) == kept == Hq * closed


# ------------------------------------------------------------------ per-kv-head tables
# One rotation-frequency row per kv head (its q heads use the same row): the rows here are
# RoPE tables of different bases and Llama-3-style scalings, so every kv head has its own
# windows.

def _head_rows(Hkv, d):
    rows = []
    for g in range(Hkv):
        base = (1e4, 5e5, 1e6, 1e7)[g % 4]
        t = wpa.default_inv_freq(d, base)
        if g % 2:
            t = wpa.llama3_inv_freq(d, base, factor=8.0 * (g + 1), low_freq_factor=1.0,
                                    high_freq_factor=4.0, original_max_position=4096)
        rows.append(t)
    return np.stack(rows)


def _head_count(d, alpha, N, rows, G):
    return wpa.count_terms_heads(d, alpha, N, 0, N, rows, G)[0]


@pytest.mark.parametrize("alpha", [1.0, 2.0])
@pytest.mark.parametrize("pairs", ["half", "interleaved"])
@pytest.mark.parametrize("shape", [
    (1, 700, 14, 2, 64),               # Qwen2.5-0.5B heads
    (2, 400, 24, 8, 128),              # Llama-3.2-3B heads
])
def test_prefill_per_head_tables_match_oracle(shape, pairs, alpha):
    need_gpu()
    B, N, Hq, Hkv, d = shape
    rows = _head_rows(Hkv, d)
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=60 + N)
    say("prefill per-head tables", shape, pairs, alpha)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lse = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), 1e4, alpha, want_lse=True,
                           term_count=cnt, out_dtype=torch.float32, inv_freq=rows, pairs=pairs)
    torch.cuda.synchronize()
    ro, rl, kept = oracle.prefill(as_bf16_for_oracle(q), as_bf16_for_oracle(k),
                                  as_bf16_for_oracle(v), 1e4, alpha, inv_freq=rows, layout=pairs)
    check_close(out.cpu().numpy(), ro, "out")
    check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
    assert int(cnt.item()) == kept == B * _head_count(d, alpha, N, rows, Hq // Hkv)


def test_prefill_per_head_tables_with_positions():
    """Explicit (gapped) positions with per-head rows, at d = 128 and d = 64."""
    need_gpu()
    for (B, N, Hq, Hkv, d) in ((1, 600, 8, 4, 128), (2, 500, 6, 2, 64)):
        rows = _head_rows(Hkv, d)
        q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=61)
        pos = (np.cumsum(np.random.default_rng(9).integers(0, 30, (B, N)), axis=1) + 77).astype(np.int32)
        say("per-head tables, positions", d)
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        out, lse = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), 1e4, 1.0, want_lse=True,
                               term_count=cnt, out_dtype=torch.float32, inv_freq=rows,
                               positions=torch.from_numpy(pos).cuda())
        torch.cuda.synchronize()
        ro, rl, kept = oracle.prefill(as_bf16_for_oracle(q), as_bf16_for_oracle(k),
                                      as_bf16_for_oracle(v), 1e4, 1.0, pos=pos, inv_freq=rows)
        check_close(out.cpu().numpy(), ro, "out d=%d" % d)
        check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
        assert int(cnt.item()) == kept


def test_per_head_tables_equal_rows_is_bitwise_shared_table():
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 900, 24, 8, 128, 5e5
    theta = _table("llama3", d, base)
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=62)
    say("per-head rows all equal")
    a = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), base, 1.0, inv_freq=theta, out_dtype=torch.float32)
    b = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), base, 1.0, inv_freq=np.stack([theta] * Hkv),
                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_per_head_tables_match_oracle():
    """The decode step and the cache write with per-head rows (contiguous and paged caches)."""
    need_gpu()
    B, Lmax, Hq, Hkv, d = 4, 3000, 24, 8, 128
    rows = _head_rows(Hkv, d)
    q, k, v, lens = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=63, len_lo=500)
    say("decode per-head tables")
    cache = wpa.KVCache(B, Lmax, Hkv, d, 1e4, inv_freq=rows)
    cache.write(k.cuda(), v.cuda(), 0)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lse = wpa.decode(q.cuda(), cache, lens.cuda(), 1.0, want_lse=True, term_count=cnt,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 lens.numpy(), 1e4, 1.0, inv_freq=rows)
    check_close(out.cpu().numpy(), ro, "out")
    check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
    assert int(cnt.item()) == kept == sum(
        wpa.count_terms_heads(d, 1.0, 1, int(L) - 1, int(L), rows, Hq // Hkv)[0] for L in lens)
    # the same tokens in a paged pool give the same bits
    ps, maxp = 256, (Lmax + 255) // 256
    table = torch.arange(B * maxp, dtype=torch.int32).flip(0).reshape(B, maxp).contiguous().cuda()
    paged = wpa.PagedKVCache(B * maxp, ps, Hkv, d, 1e4, inv_freq=rows)
    paged.write(k.cuda(), v.cuda(), 0, block_table=table)
    op = wpa.decode(q.cuda(), paged, lens.cuda(), 1.0, out_dtype=torch.float32, block_table=table)
    torch.cuda.synchronize()
    assert torch.equal(op.cpu(), out.cpu())


def test_per_head_tables_unsupported_paths():
    need_gpu()
    rows = _head_rows(2, 64)
    with pytest.raises(ValueError):              # the windowed cache's size query refuses
        wpa.KVCache(1, 256, 2, 64, 1e4, inv_freq=rows, window_alpha=1.0)


@pytest.mark.parametrize("d,Hq,Hkv", [(64, 14, 2), (128, 24, 8)])
def test_chunked_prefill_per_head_tables(d, Hq, Hkv):
    """Chunked prefill against caches written with a distinct frequency row per kv head: the
    last 300 tokens of two ragged prompts, automatic key splits on the dense cache, the same on
    a paged pool of 64-token pages (bit-identical), no splits (rounding only), against the
    oracle's rows with the same tables (outputs, LSE, counts)."""
    need_gpu()
    rows = _head_rows(Hkv, d)
    B, Nq, page = 2, 300, 64
    lens_h = [Nq + 500, Nq + 1700]
    Lmax = 2048
    q, k, v = synth.prefill_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=71)
    max_pages = Lmax // page
    table = torch.from_numpy(np.random.default_rng(3).permutation(B * max_pages).astype(np.int32)
                             .reshape(B, max_pages)).cuda()
    cache = wpa.KVCache(B, Lmax, Hkv, d, 1e4, inv_freq=rows)
    paged = wpa.PagedKVCache(B * max_pages, page, Hkv, d, 1e4, inv_freq=rows, block_table=table)
    for b, L in enumerate(lens_h):
        kk, vv = k[b:b + 1, :L].cuda().contiguous(), v[b:b + 1, :L].cuda().contiguous()
        cache.write(kk, vv, 0, seq=b)
        paged.write(kk, vv, 0, block_table=table[b:b + 1])
    qc = torch.stack([q[b, L - Nq:L] for b, L in enumerate(lens_h)]).contiguous().cuda()
    kv_len = torch.tensor(lens_h, dtype=torch.int32, device="cuda")
    say("chunked prefill per-head tables", d)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    od, ld = wpa.prefill_cached(qc, cache, kv_len, 1.0, want_lse=True, term_count=cnt,
                                out_dtype=torch.float32)
    op, lp = wpa.prefill_cached(qc, paged, kv_len, 1.0, want_lse=True, out_dtype=torch.float32)
    o1 = wpa.prefill_cached(qc, cache, kv_len, 1.0, out_dtype=torch.float32, splits=1)
    torch.cuda.synchronize()
    assert torch.equal(od, op) and torch.equal(ld, lp), "paged chunk differs from contiguous"
    assert (od - o1).abs().max() <= 2e-3
    kept_all = 0
    for b, L in enumerate(lens_h):
        ro, rl, kept = oracle.prefill(as_bf16_for_oracle(q[b:b + 1, :L]), as_bf16_for_oracle(k[b:b + 1, :L]),
                                      as_bf16_for_oracle(v[b:b + 1, :L]), 1e4, 1.0,
                                      rows=np.arange(L - Nq, L), inv_freq=rows)
        check_close(od[b:b + 1].cpu().numpy(), ro, "out[%d]" % b)
        check_close(ld[b:b + 1].cpu().numpy(), rl, "lse[%d]" % b, LSE_MAX, LSE_MAX)
        kept_all += kept
    assert int(cnt.item()) == kept_all


def test_full_size_llama3b_per_head_tables():
    """The Llama-3.2-3B-shaped prefill at its full 131072 tokens with a distinct frequency row
    per kv head, in the bench's launch configuration: sampled rows against the oracle, exact
    count (per head, summed)."""
    need_gpu()
    w = synth.WORKLOADS["llama3b"]
    rows = _head_rows(w.Hkv, w.d)
    say("full size llama3b per-head tables")
    q, k, v = synth.workload_inputs(w, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = wpa.prefill(q, k, v, w.base, 1.0, term_count=cnt, out_dtype=torch.float32, inv_freq=rows)
    torch.cuda.synchronize()
    srows = synth.sample_rows(w.N, 24, seed=w.seed)
    got = out[:, torch.as_tensor(srows, device="cuda")].cpu().numpy()
    del out
    say("oracle rows", len(srows))
    ro, _, _ = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v), w.base, 1.0,
                              rows=srows, inv_freq=rows)
    check_close(got, ro, "llama3b per-head sampled rows")
    assert int(cnt.item()) == _head_count(w.d, 1.0, w.N, rows, w.Hq // w.Hkv)

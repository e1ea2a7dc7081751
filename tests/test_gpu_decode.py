"""GPU parity of the cache write and the windowed decode step against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, check_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _cache_from(k, v, base, Lmax=None):
    B, L, Hkv, d = k.shape
    cache = wpa.KVCache(B, Lmax or L, Hkv, d, base)
    cache.write(k.cuda(), v.cuda(), 0)
    return cache


@pytest.mark.parametrize("d,base", [(64, 1e4), (128, 5e5), (128, 1e7)])
def test_kv_write_rotation(d, base):
    """The K cache holds the keys rotated at their token index, rounded to IEEE half, in
    the pair-blocked layout [B][Hkv][d/16][Lmax][16]; the V cache holds V as bf16 (blocked
    by 8 tokens).  Two appends, the second starting inside an 8-token block."""
    need_gpu()
    B, L, Hkv = 2, 300, 3
    k, v = synth.prefill_inputs(B, L, Hkv, Hkv, d, "bf16", seed=5)[1:]
    say("kv_write", d, base)
    cache = wpa.KVCache(B, L + 17, Hkv, d, base)
    cache.write(k[:, :101].cuda().contiguous(), v[:, :101].cuda().contiguous(), 0)
    cache.write(k[:, 101:].cuda().contiguous(), v[:, 101:].cuda().contiguous(), 101)
    torch.cuda.synchronize()
    kb = cache.k.view(torch.float16).view(B, Hkv, d // 16, L + 17, 16)[:, :, :, :L].float().cpu()
    P = d // 2
    x = kb[..., :8].permute(0, 3, 1, 2, 4).reshape(B, L, Hkv, P)
    y = kb[..., 8:].permute(0, 3, 1, 2, 4).reshape(B, L, Hkv, P)
    got = torch.cat([x, y], dim=-1).numpy()
    for b in range(B):
        ref = oracle.rope(synth.to_oracle(k[b]), np.arange(L), base)
        # half rounding of the rotated value (relative 2^-11) plus fp32 sincos (~1e-6 of
        # the pair's norm)
        err = np.abs(got[b] - ref)
        assert (err <= 2 ** -11 * np.abs(ref) + 4e-6 * (np.abs(ref).max() + 1e-3)).all()
    vb = cache.v_tokens()[:, :, :L].float().cpu().permute(0, 2, 1, 3)
    assert torch.equal(vb, v.float())


@pytest.mark.parametrize("alpha", [1.0, 2.0, math.inf, 0.0])
@pytest.mark.parametrize("shape", [
    # B, Lmax, Hq, Hkv, d, base
    (3, 700, 24, 8, 128, 5e5),
    (2, 1500, 14, 2, 64, 1e6),
    (1, 300, 28, 4, 128, 1e7),
    (2, 257, 16, 1, 64, 1e4),
])
def test_decode_matches_oracle(shape, alpha):
    need_gpu()
    B, Lmax, Hq, Hkv, d, base = shape
    q, k, v, lens = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=Lmax, len_lo=1)
    lens[0] = Lmax
    lens[-1] = 1 if B > 1 else lens[-1]
    say("decode", shape, alpha, lens.tolist())
    cache = _cache_from(k, v, base)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lse = wpa.decode(q.cuda(), cache, lens.cuda(), alpha, want_lse=True, term_count=cnt,
                          out_dtype=torch.float32)
    ob = wpa.decode(q.cuda(), cache, lens.cuda(), alpha)
    assert ob.dtype == torch.bfloat16 and torch.equal(ob, out.to(torch.bfloat16))
    torch.cuda.synchronize()
    ro, rl, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 lens.numpy(), base, alpha)
    check_close(out.float().cpu().numpy(), ro, "decode out")
    check_close(lse.cpu().numpy(), rl, "decode lse", LSE_MAX, LSE_MAX)
    expect = sum(Hq * wpa.count_terms(d, base, alpha, 1, int(L) - 1, int(L))[0] for L in lens)
    assert int(cnt.item()) == kept == expect


@pytest.mark.parametrize("alpha", [0.0, 1.0, math.inf])
def test_decode_split_edges(alpha):
    """The library's split-KV items take ranges of distance from each sequence's last key
    that stream equal cache bytes, rounded to 32 keys.  Lengths below, at and just past 32
    keys, around the 256-key chunk grid and just below Lmax, against the oracle (outputs,
    LSE, counts), and against the uniform split of explicit chunk_keys (rounding only)."""
    need_gpu()
    Lmax, Hq, Hkv, d, base = 2600, 14, 2, 128, 1e4
    lens_l = [1, 5, 31, 32, 33, 63, 255, 256, 257, 511, 1025, 2047, 2599, 2600]
    B = len(lens_l)
    q, k, v, _ = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=91, len_lo=1)
    lens = torch.tensor(lens_l, dtype=torch.int32)
    say("decode split edges", alpha)
    cache = _cache_from(k, v, base)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lse = wpa.decode(q.cuda(), cache, lens.cuda(), alpha, want_lse=True, term_count=cnt,
                          out_dtype=torch.float32)
    uni = wpa.decode(q.cuda(), cache, lens.cuda(), alpha, chunk_keys=256, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 lens.numpy(), base, alpha)
    check_close(out.cpu().numpy(), ro, "decode out")
    check_close(lse.cpu().numpy(), rl, "decode lse", LSE_MAX, LSE_MAX)
    assert int(cnt.item()) == kept
    assert (out.cpu() - uni.cpu()).abs().max() <= 2e-3


def test_decode_explicit_query_position():
    need_gpu()
    B, Lmax, Hq, Hkv, d, base = 2, 400, 8, 2, 128, 1e4
    q, k, v, lens = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=3, len_lo=50)
    qpos = (lens + torch.tensor([0, 77], dtype=torch.int32)).to(torch.int32)
    say("decode q_pos")
    cache = _cache_from(k, v, base)
    out = wpa.decode(q.cuda(), cache, lens.cuda(), 1.0, q_pos=qpos.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, _, _ = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                             lens.numpy(), base, 1.0, q_pos=qpos.numpy())
    check_close(out.float().cpu().numpy(), ro, "decode q_pos")


def test_decode_equals_last_prefill_row():
    need_gpu()
    B, L, Hq, Hkv, d, base = 1, 1100, 24, 8, 128, 5e5
    q, k, v = synth.prefill_inputs(B, L, Hq, Hkv, d, "bf16", seed=21)
    say("decode vs prefill row")
    pre = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), base, 1.0, out_dtype=torch.float32).cpu()
    cache = _cache_from(k, v, base)
    lens = torch.tensor([L], dtype=torch.int32)
    dec = wpa.decode(q[:, L - 1].contiguous().cuda(), cache, lens.cuda(), 1.0,
                     out_dtype=torch.float32).cpu()
    torch.cuda.synchronize()
    check_close(dec.numpy(), pre[:, L - 1].numpy(), "decode vs prefill")


def test_decode_chunking_invariance():
    """The split of the keys into work items changes only rounding: the probabilities enter
    the P*V product as bf16 relative to each split's running max, so outputs may move by a
    few bf16 ulps of p (bound 2e-3, a fifth of the parity tolerance); LSE by fp32 rounding."""
    need_gpu()
    B, Lmax, Hq, Hkv, d, base = 2, 5000, 24, 8, 128, 5e5
    q, k, v, lens = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=11, len_lo=3000)
    say("decode chunking")
    cache = _cache_from(k, v, base)
    outs = []
    for ch in (256, 1024, 4096, 0):
        o, l = wpa.decode(q.cuda(), cache, lens.cuda(), 1.0, chunk_keys=ch, want_lse=True,
                          out_dtype=torch.float32)
        outs.append((o.cpu(), l.cpu()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert (o - outs[0][0]).abs().max() <= 2e-3
        assert (l - outs[0][1]).abs().max() <= 1e-4


def test_decode_full_size_llama_batch():
    """Llama-3.2-3B-shaped decode at full size: B=16, Lmax=131072, kv_len ~ U{8192..131072}."""
    need_gpu()
    w = synth.WORKLOADS["llama3b_decode"]
    say("decode full size", w.name)
    q, k, v, lens = synth.workload_inputs(w, device="cuda")
    cache = wpa.KVCache(w.B, w.N, w.Hkv, w.d, w.base)
    cache.write(k, v, 0)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = wpa.decode(q, cache, lens, 1.0, term_count=cnt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    lens_h = lens.cpu().numpy()
    expect = sum(w.Hq * wpa.count_terms(w.d, w.base, 1.0, 1, int(L) - 1, int(L))[0] for L in lens_h)
    assert int(cnt.item()) == expect
    say("oracle decode full size")
    ro, _, _ = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v), lens_h,
                             w.base, 1.0)
    check_close(out.float().cpu().numpy(), ro, "llama decode full size")


def test_decode_full_size_qwen7b1m():
    """The Qwen2.5-7B-1M-shaped decode step: one sequence at the full 1M-token context."""
    need_gpu()
    w = synth.WORKLOADS["qwen7b1m_decode"]
    say("decode full size", w.name)
    q, k, v, lens = synth.workload_inputs(w, device="cuda")
    assert int(lens.min()) == w.N
    cache = wpa.KVCache(w.B, w.N, w.Hkv, w.d, w.base)
    cache.write(k, v, 0)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = wpa.decode(q, cache, lens, 1.0, term_count=cnt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(cnt.item()) == w.B * w.Hq * wpa.count_terms(w.d, w.base, 1.0, 1, w.N - 1, w.N)[0]
    say("oracle decode full size")
    ro, _, _ = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                             lens.cpu().numpy(), w.base, 1.0)
    check_close(out.float().cpu().numpy(), ro, "qwen7b1m decode full size")

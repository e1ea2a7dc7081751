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

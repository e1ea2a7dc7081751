"""GPU parity of decode on the windowed K cache (pair blocks kept only for the keys inside
their window, in rows reused as a ring): bit-identical to decode on the dense cache, which
reads the same values for every key a block still serves, and within tolerance of the fp64
oracle; appends of every size relative to the ring lengths, ragged sequences, and a decode
alpha below the cache's."""
import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, check_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _pair(B, Lmax, Hkv, d, base, calpha):
    dense = wpa.KVCache(B, Lmax, Hkv, d, base)
    win = wpa.KVCache(B, Lmax, Hkv, d, base, window_alpha=calpha)
    for c in (dense, win):
        c.k.fill_(255)                      # NaN in half: unwritten rows must never count
        c.v.fill_(255)
    assert win.k.numel() < dense.k.numel()
    return dense, win


def _decode_both(q, dense, win, lens, alpha):
    cd = torch.zeros(1, dtype=torch.int64, device="cuda")
    cw = torch.zeros(1, dtype=torch.int64, device="cuda")
    od, ld = wpa.decode(q, dense, lens, alpha, out_dtype=torch.float32, want_lse=True, term_count=cd)
    ow, lw = wpa.decode(q, win, lens, alpha, out_dtype=torch.float32, want_lse=True, term_count=cw)
    torch.cuda.synchronize()
    assert torch.equal(od, ow) and torch.equal(ld, lw), "windowed cache differs from dense"
    assert int(cd.item()) == int(cw.item())
    return ow, lw


@pytest.mark.parametrize("calpha,alpha", [(1.0, 1.0), (2.0, 1.0), (1.0, 0.5)])
def test_window_cache_incremental_appends(calpha, alpha):
    """d=64, base 1e4: rings of 64, 480 and 4736 rows (alpha 1); appends of 1, 37, 500 and
    1300 tokens, so writes both fill and overrun rings; a decode after every append."""
    need_gpu()
    B, Lmax, Hq, Hkv, d, base = 2, 6000, 4, 2, 64, 1e4
    q, k, v, _ = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=71)
    dense, win = _pair(B, Lmax, Hkv, d, base, calpha)
    qc = q.cuda()
    t = 0
    for n in (1, 37, 500, 1, 1300, 64, 2000, 3, 2094):
        say("append", t, n, calpha, alpha)
        kk, vv = k[:, t:t + n].cuda().contiguous(), v[:, t:t + n].cuda().contiguous()
        dense.write(kk, vv, t)
        win.write(kk, vv, t)
        t += n
        lens = torch.full((B,), t, dtype=torch.int32, device="cuda")
        out, lse = _decode_both(qc, dense, win, lens, alpha)
    assert t == Lmax
    ro, rl, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 np.full(B, Lmax), base, alpha)
    check_close(out.cpu().numpy(), ro, "decode out")
    check_close(lse.cpu().numpy(), rl, "decode lse", LSE_MAX, LSE_MAX)


def test_window_cache_llama_shape_ragged():
    """Llama-3.2-3B heads (d=128, base 5e5, 24/8 heads), alpha 1: sequences of 9000, 30001 and
    40000 tokens written per sequence in one piece each (rings of 32 .. 18880 rows)."""
    need_gpu()
    B, Lmax, Hq, Hkv, d, base = 3, 40000, 24, 8, 128, 5e5
    q, k, v, _ = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=72)
    lens_h = [9000, 30001, 40000]
    dense, win = _pair(B, Lmax, Hkv, d, base, 1.0)
    for b, L in enumerate(lens_h):
        kk, vv = k[b:b + 1, :L].cuda().contiguous(), v[b:b + 1, :L].cuda().contiguous()
        dense.write(kk, vv, 0, seq=b)
        win.write(kk, vv, 0, seq=b)
    lens = torch.tensor(lens_h, dtype=torch.int32, device="cuda")
    say("llama ragged window decode")
    out, lse = _decode_both(q.cuda(), dense, win, lens, 1.0)
    ro, rl, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 np.array(lens_h), base, 1.0)
    check_close(out.cpu().numpy(), ro, "decode out")
    check_close(lse.cpu().numpy(), rl, "decode lse", LSE_MAX, LSE_MAX)


def test_window_cache_rejects_misuse():
    need_gpu()
    win = wpa.KVCache(1, 512, 2, 64, 1e4, window_alpha=1.0)
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((1,), 512, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        wpa.decode(q, win, lens, 2.0)                  # alpha above the cache's window
    with pytest.raises(ValueError):
        wpa.decode(q, win, lens, 1.0, q_pos=lens)      # the query must be the newest token

"""The decode entry point that allocates nothing (wpa_decode_noalloc), called through the C ABI:
its output must equal wpa_decode_ex's on the same inputs (bit for bit: the same kernels, the
same split, only the partials' buffer differs) and match the oracle to the usual bar, on two
calls in a row, the second with a smaller input (the scratch array keeps the first call's
contents)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, check_close, need_gpu, say

FAKE = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced: validation fails first


def _noalloc_rc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, qpos=None, out=FAKE, lse=None, B=2, Lmax=4096,
             Hq=8, Hkv=2, d=128, base=5e5, alpha=1.0, scale=0.0, dtype=0, odt=1, cnt=None, chunk=0)
    a.update(kw)
    return wpa.lib().wpa_decode_noalloc(a["q"], a["kc"], a["vc"], a["lens"], a["qpos"], a["out"],
                                        a["lse"], a["B"], a["Lmax"], a["Hq"], a["Hkv"], a["d"],
                                        a["base"], None, a["alpha"], a["scale"], a["dtype"],
                                        a["odt"], a["cnt"], a["chunk"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=80), wpa.WPA_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), wpa.WPA_ERR_INVALID),
    (dict(chunk=100), wpa.WPA_ERR_INVALID),
    (dict(lens=None), wpa.WPA_ERR_INVALID),
    (dict(out=None), wpa.WPA_ERR_INVALID),
    (dict(lse=ctypes.c_void_p((1 << 20) + 2)), wpa.WPA_ERR_INVALID),
    # partials beyond the 16 MiB scratch: 1 x 8 kv heads x 4096 chunks x 3 heads x 130 x 4 B
    (dict(B=1, Lmax=1 << 20, Hq=24, Hkv=8, chunk=256), wpa.WPA_ERR_UNSUPPORTED),
])
def test_noalloc_decode_rejects_bad_arguments(kw, code):
    """Host only: every rejection happens before the scratch array or the GPU is touched."""
    assert _noalloc_rc(**kw) == code
    assert wpa.lib().wpa_last_error().decode() != ""


def _case(B, Lmax, Hq, Hkv, d, base, seed, chunk_keys):
    q, k, v, lens = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=seed, len_lo=Lmax // 3)
    cache = wpa.KVCache(B, Lmax, Hkv, d, base)
    cache.write(k.cuda(), v.cuda(), 0)
    qd, ld = q.cuda(), lens.cuda()
    say("no-alloc decode", (B, Lmax, Hq, Hkv, d), "chunk", chunk_keys)
    ref, ref_lse = wpa.decode(qd, cache, ld, 1.0, want_lse=True, out_dtype=torch.float32,
                              chunk_keys=chunk_keys)
    out = torch.full((B, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    wpa.decode_noalloc(qd, cache, ld, 1.0, out=out, lse=lse, term_count=cnt, chunk_keys=chunk_keys)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
    ro, rl, kept = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 lens.numpy(), base, 1.0)
    check_close(out.cpu().numpy(), ro, "out")
    check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
    assert int(cnt.item()) == kept


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_decode_twice():
    need_gpu()
    # first call: Llama-3.2-3B heads, 8 sequences, small chunks (many partials)
    _case(8, 6000, 24, 8, 128, 5e5, seed=31, chunk_keys=256)
    # second call, smaller: Qwen2.5-0.5B heads, 2 sequences, the library's chunk
    _case(2, 1500, 14, 2, 64, 1e6, seed=32, chunk_keys=0)

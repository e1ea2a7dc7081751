"""GPU parity of chunked prefill against the decode caches (ragged batches: each sequence
has its own cached prefix) with the fp64 oracle: a chunk's rows are rows kv_len-Nq ..
kv_len-1 of a causal windowed prefill over the sequence's first kv_len tokens.  With key
splits (each row block's key tiles shared among several workgroups, their partials merged by
a second kernel) the rows are the same attention up to fp32 rounding order: the same bar."""
import math

import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, as_bf16_for_oracle as exact, check_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _poisoned_cache(B, Lmax, Hkv, d, base, **rope):
    """A cache whose every byte starts as 0xff (NaN in both half and bf16): slots a sequence
    has not written must never reach a result."""
    cache = wpa.KVCache(B, Lmax, Hkv, d, base, **rope)
    cache.k.fill_(255)
    cache.v.fill_(255)
    return cache


def _run_ragged(B, Nq, prefix, Hq, Hkv, d, base, alpha, dtype="bf16", seed=0, rope=None,
                splits=0):
    rope = rope or {}
    lens = [Nq + p for p in prefix]
    Lmax = max(lens) + 13
    q, k, v = synth.prefill_inputs(B, Lmax, Hq, Hkv, d, dtype, seed=seed)
    cache = _poisoned_cache(B, Lmax, Hkv, d, base, **rope)
    for b, L in enumerate(lens):
        cache.write(k[b:b + 1, :L].cuda().contiguous(), v[b:b + 1, :L].cuda().contiguous(), 0,
                    seq=b)
    qc = torch.stack([q[b, L - Nq:L] for b, L in enumerate(lens)]).contiguous()
    kv_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lse = wpa.prefill_cached(qc.cuda(), cache, kv_len, alpha, want_lse=True, term_count=cnt,
                                  out_dtype=torch.float32, splits=splits)
    torch.cuda.synchronize()
    kept_all = 0
    for b, L in enumerate(lens):
        ro, rl, kept = oracle.prefill(exact(q[b:b + 1, :L]), exact(k[b:b + 1, :L]),
                                      exact(v[b:b + 1, :L]), base, alpha,
                                      rows=np.arange(L - Nq, L), inv_freq=rope.get("inv_freq"),
                                      layout=rope.get("pairs", "half"))
        check_close(out[b:b + 1].cpu().numpy(), ro, "out[%d]" % b)
        check_close(lse[b:b + 1].cpu().numpy(), rl, "lse[%d]" % b, LSE_MAX, LSE_MAX)
        closed = wpa.count_terms(d, base, alpha, Nq, L - Nq, L, inv_freq=rope.get("inv_freq"))[0]
        assert kept == Hq * closed
        kept_all += kept
    assert int(cnt.item()) == kept_all


@pytest.mark.parametrize("splits", [1, 0])
@pytest.mark.parametrize("alpha", [1.0, 2.0, math.inf])
@pytest.mark.parametrize("Nq", [1, 77, 300])
@pytest.mark.parametrize("shape", [
    (14, 2, 64, 1e6),          # Qwen2.5-0.5B heads
    (24, 8, 128, 5e5),         # Llama-3.2-3B heads
])
def test_chunked_prefill_ragged_matches_oracle(shape, Nq, alpha, splits):
    """Three sequences with prefixes 0, 517 and 1290 tokens (chunk starts off the 32-token
    grid), Nq not a multiple of 32, cache slots past each length poisoned with NaN; no key
    splits (the plain entry point) and the launch's own choice (here the most: few rows)."""
    need_gpu()
    Hq, Hkv, d, base = shape
    say("chunked ragged", shape, Nq, alpha, "splits", splits)
    _run_ragged(3, Nq, [0, 517, 1290], Hq, Hkv, d, base, alpha, seed=Nq + d, splits=splits)


@pytest.mark.parametrize("splits", [2, 3, 5, 16])
@pytest.mark.parametrize("shape", [(14, 2, 64, 1e6), (24, 8, 128, 5e5), (16, 16, 64, 1e4)])
def test_key_split_counts_match_oracle(shape, splits):
    """Explicit split counts, from two to more splits than a row block has key tiles (empty
    splits), over prefixes that put row blocks across tile edges; one q head per kv head
    takes the several-row-groups-per-workgroup layout."""
    need_gpu()
    Hq, Hkv, d, base = shape
    say("key splits", shape, splits)
    _run_ragged(3, 200, [0, 400, 1700], Hq, Hkv, d, base, 1.0, seed=splits + d, splits=splits)


def test_key_splits_need_room():
    need_gpu()
    cache = wpa.KVCache(1, 512, 2, 64, 1e4)
    q = torch.zeros((1, 64, 14, 64), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((1,), 512, dtype=torch.int32, device="cuda")
    need = wpa.prefill_cached_workspace_bytes(1, 64, 14, 2, 64, 4)
    assert need == 4 * 64 * 14 * 65 * 4
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        wpa.prefill_cached(q, cache, lens, 1.0, splits=4, workspace=small)
    with pytest.raises(ValueError):
        wpa.prefill_cached(q, cache, lens, 1.0, splits=17)


def test_chunked_prefill_fp32_queries_and_variant():
    """fp32 inputs (rounded to bf16 on load) with a Llama-3 frequency table, interleaved pairs."""
    need_gpu()
    d, base = 128, 5e5
    theta = wpa.llama3_inv_freq(d, base, factor=32.0, low_freq_factor=1.0, high_freq_factor=4.0,
                                original_max_position=8192)
    say("chunked fp32 llama3 interleaved")
    _run_ragged(2, 130, [40, 1000], 24, 8, d, base, 1.0, dtype="fp32", seed=5,
                rope=dict(inv_freq=theta, pairs="interleaved"))


@pytest.mark.parametrize("d,Hq,Hkv,base", [(64, 14, 2, 1e6), (128, 24, 8, 5e5)])
def test_prompt_in_chunks_equals_one_shot_oracle(d, Hq, Hkv, base):
    """A 1000-token prompt prefilled as chunks of 300, 300 and 400 (append K/V, then attend)
    gives the rows of a one-shot prefill of the whole prompt."""
    need_gpu()
    N, alpha = 1000, 1.0
    q, k, v = synth.prefill_inputs(1, N, Hq, Hkv, d, "bf16", seed=9)
    cache = _poisoned_cache(1, N, Hkv, d, base)
    outs = []
    s = 0
    for n in (300, 300, 400):
        say("chunk", s, n)
        cache.write(k[:, s:s + n].cuda().contiguous(), v[:, s:s + n].cuda().contiguous(), s)
        kv_len = torch.tensor([s + n], dtype=torch.int32, device="cuda")
        outs.append(wpa.prefill_cached(q[:, s:s + n].cuda().contiguous(), cache, kv_len, alpha,
                                       out_dtype=torch.float32))       # (key splits: automatic)
        s += n
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=1).cpu().numpy()
    ro, _, _ = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v), base,
                              alpha)
    check_close(got, ro, "chunked vs one-shot")


def test_chunk_after_long_prefix_sampled_rows():
    """A 2048-query chunk after a 32768-token prefix at Qwen2.5-7B heads (d=128, 28 q heads,
    4 kv heads), checked on sampled rows."""
    need_gpu()
    Hq, Hkv, d, base, P, Nq = 28, 4, 128, 1e6, 32768, 2048
    L = P + Nq
    q, k, v = synth.prefill_inputs(1, L, Hq, Hkv, d, "bf16", seed=21)
    cache = wpa.KVCache(1, L, Hkv, d, base)
    cache.write(k.cuda(), v.cuda(), 0)
    kv_len = torch.tensor([L], dtype=torch.int32, device="cuda")
    say("chunk after 32K prefix")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = wpa.prefill_cached(q[:, P:].cuda().contiguous(), cache, kv_len, 1.0,
                             out_dtype=torch.float32, term_count=cnt)
    torch.cuda.synchronize()
    rows = synth.sample_rows(Nq, 12, seed=3)
    ro, _, _ = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v), base,
                              1.0, rows=rows + P)
    check_close(out[:, rows].cpu().numpy(), ro, "sampled rows")
    assert int(cnt.item()) == Hq * wpa.count_terms(d, base, 1.0, Nq, P, L)[0]


def test_qwen05b_chunk_schedule_key_splits_sampled():
    """The Qwen2.5-0.5B prompt of 32768 tokens in 8 chunks of 4096 (append K/V, then attend,
    key splits chosen by the launch), sampled rows of every chunk against the oracle, and
    the kept-term count of the whole schedule against the closed form."""
    need_gpu()
    w = synth.WORKLOADS["qwen05b"]
    q, k, v = synth.workload_inputs(w, device="cuda")
    cache = wpa.KVCache(w.B, w.N, w.Hkv, w.d, w.base)
    out = torch.empty_like(q, dtype=torch.float32)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    C = 4096
    for s in range(0, w.N, C):
        cache.write(k[:, s:s + C], v[:, s:s + C], s)
        lens = torch.full((w.B,), s + C, dtype=torch.int32, device="cuda")
        wpa.prefill_cached(q[:, s:s + C], cache, lens, 1.0, out=out[:, s:s + C], term_count=cnt)
    torch.cuda.synchronize()
    say("qwen05b chunk schedule: oracle rows")
    rows = np.unique(np.concatenate([synth.sample_rows(w.N, 12, seed=w.seed),
                                     np.arange(0, w.N, C), np.arange(C - 1, w.N, C)]))
    got = out[:, torch.as_tensor(rows, device="cuda")].cpu().numpy()
    ro, _, _ = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v), w.base,
                              1.0, rows=rows)
    check_close(got, ro, "chunk schedule sampled rows")
    assert int(cnt.item()) == w.Hq * wpa.count_terms(w.d, w.base, 1.0, w.N, 0, w.N)[0]

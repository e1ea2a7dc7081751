"""GPU parity of varlen chunked prefill (a query count per sequence, rows packed back to back):
without key splits every row bit-identical to the same row of a per-sequence chunked prefill
with that count; with or without them, paged caches bit-identical to contiguous ones and every
row within tolerance of the fp64 oracle; sequences with no rows, one row, rows not a multiple
of 32, and a whole-prompt chunk."""
import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, as_bf16_for_oracle as exact, check_close, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("splits", [1, 0, 3])
@pytest.mark.parametrize("d,Hq,Hkv,base", [(64, 14, 2, 1e6), (128, 24, 8, 5e5)])
def test_varlen_chunks_match_per_sequence_and_oracle(d, Hq, Hkv, base, splits):
    need_gpu()
    qn = [0, 1, 77, 300, 256]                       # query rows per sequence
    kv = [50, 1000, 2000, 300, 1500]                # tokens in the cache, each >= its rows
    B = len(qn)
    page = {1: 256, 0: 32, 3: 64}[splits]           # pages shorter than a 128-key tile too
    max_pages = (max(kv) + page - 1) // page
    Lmax = max_pages * page
    q, k, v = synth.prefill_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=91)
    cache = wpa.KVCache(B, Lmax, Hkv, d, base)
    rng = np.random.default_rng(5)
    table = torch.from_numpy(rng.permutation(B * max_pages).reshape(B, max_pages)
                             .astype(np.int32)).cuda()
    paged = wpa.PagedKVCache(B * max_pages, page, Hkv, d, base, block_table=table)
    for c in (cache, paged):
        c.k.fill_(255)
        c.v.fill_(255)
    for b, L in enumerate(kv):
        kk, vv = k[b:b + 1, :L].cuda().contiguous(), v[b:b + 1, :L].cuda().contiguous()
        cache.write(kk, vv, 0, seq=b)
        paged.write(kk, vv, 0, block_table=table[b:b + 1])
    cu = np.concatenate([[0], np.cumsum(qn)]).astype(np.int32)
    qp = torch.cat([q[b, kv[b] - qn[b]:kv[b]] for b in range(B)]).contiguous().cuda()
    cu_q = torch.from_numpy(cu).cuda()
    kv_len = torch.tensor(kv, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    say("varlen contiguous", d, "splits", splits)
    out, lse = wpa.prefill_cached(qp, cache, kv_len, 1.0, cu_q=cu_q, max_q=max(qn),
                                  want_lse=True, term_count=cnt, out_dtype=torch.float32,
                                  splits=splits)
    say("varlen paged", d)
    outp, lsep = wpa.prefill_cached(qp, paged, kv_len, 1.0, cu_q=cu_q, max_q=max(qn),
                                    want_lse=True, out_dtype=torch.float32, splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(out, outp) and torch.equal(lse, lsep), "paged varlen differs"
    kept_all = 0
    for b in range(B):
        if qn[b] == 0:
            continue
        r0, r1, L = cu[b], cu[b + 1], kv[b]
        if splits == 1:
            one = wpa.KVCache(1, Lmax, Hkv, d, base)
            one.write(k[b:b + 1, :L].cuda().contiguous(), v[b:b + 1, :L].cuda().contiguous(), 0)
            ro1, rl1 = wpa.prefill_cached(qp[r0:r1].unsqueeze(0).contiguous(), one,
                                          kv_len[b:b + 1].contiguous(), 1.0, want_lse=True,
                                          out_dtype=torch.float32, splits=1)
            torch.cuda.synchronize()
            assert torch.equal(out[r0:r1], ro1[0]), "varlen rows of sequence %d differ" % b
            assert torch.equal(lse[r0:r1].transpose(0, 1), rl1[0]), "varlen lse of sequence %d" % b
        ro, rl, kept = oracle.prefill(exact(q[b:b + 1, :L]), exact(k[b:b + 1, :L]),
                                      exact(v[b:b + 1, :L]), base, 1.0,
                                      rows=np.arange(L - qn[b], L))
        check_close(out[r0:r1].cpu().numpy()[None], ro, "out[%d]" % b)
        check_close(lse[r0:r1].transpose(0, 1).cpu().numpy()[None], rl, "lse[%d]" % b,
                    LSE_MAX, LSE_MAX)
        kept_all += kept
    assert int(cnt.item()) == kept_all

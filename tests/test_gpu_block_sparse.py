"""GPU parity of prefill composed with token-level block sparsity (64-token blocks, an
ascending list of key blocks per query block and head) against the fp64 oracle: output,
LSE and kept-term count; all blocks listed equals the dense prefill bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, as_bf16_for_oracle as exact, check_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _lists(B, H, N, density, seed, width=None, junk=False, blk=64):
    """MInference-like lists: the first block (attention sink), the two blocks below the
    query block (local), and random earlier blocks with the given density; ascending.
    junk adds duplicates and entries outside [0, R) (ignored by the rule)."""
    rng = np.random.default_rng(seed)
    nblk = (N + blk - 1) // blk
    lists = [[[None] * nblk for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for R in range(nblk):
                s = {0, R - 1, R - 2} | {c for c in range(R) if rng.random() < density}
                s = sorted(c for c in s if 0 <= c < R)
                if junk and s:
                    s = sorted(s + [s[0], R, R + 3, -1])
                lists[b][h][R] = s
    mx = width or max(1, max(len(x) for bl in lists for hl in bl for x in hl))
    count = np.zeros((B, H, nblk), np.int32)
    idx = np.zeros((B, H, nblk, mx), np.int32)
    for b in range(B):
        for h in range(H):
            for R in range(nblk):
                x = lists[b][h][R][:mx]
                count[b, h, R] = len(x)
                idx[b, h, R, :len(x)] = x
    return count, idx


def _run(q, k, v, base, alpha, count, idx, rows=None, blk=64):
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lse = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), base, alpha, want_lse=True, term_count=cnt,
                           out_dtype=torch.float32, block_count=torch.from_numpy(count).cuda(),
                           block_idx=torch.from_numpy(idx).cuda(), block=blk)
    torch.cuda.synchronize()
    ro, rl, kept = oracle.prefill_sparse(exact(q), exact(k), exact(v), base, alpha, count, idx,
                                         rows=rows, blk=blk)
    return out, lse, int(cnt.item()), ro, rl, kept


@pytest.mark.parametrize("alpha", [1.0, 2.0, math.inf])
@pytest.mark.parametrize("shape", [
    (1, 700, 14, 2, 64, 1e6),          # Qwen2.5-0.5B heads; N not a multiple of 64
    (2, 650, 24, 8, 128, 5e5),         # Llama-3.2-3B heads
])
def test_block_sparse_matches_oracle(shape, alpha):
    need_gpu()
    B, N, Hq, Hkv, d, base = shape
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=90 + d)
    count, idx = _lists(B, Hq, N, 0.3, seed=91)
    say("block sparse", shape, alpha)
    out, lse, cnt, ro, rl, kept = _run(q, k, v, base, alpha, count, idx)
    check_close(out.cpu().numpy(), ro, "out")
    check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept


@pytest.mark.parametrize("at_pos", [False, True])
@pytest.mark.parametrize("shape", [(1, 700, 14, 2, 64), (2, 650, 24, 8, 128)])
def test_block_sparse_per_head_tables_match_oracle(shape, at_pos):
    """Block sparsity with one frequency row per kv head (different bases, Llama-3 scaling on
    odd heads), at token indices and at gapped explicit positions: outputs, LSE and counts
    against the oracle with the same rows and positions."""
    need_gpu()
    B, N, Hq, Hkv, d = shape
    rows = []
    for g in range(Hkv):
        t = wpa.default_inv_freq(d, (1e4, 5e5, 1e6, 1e7)[g % 4])
        if g % 2:
            t = wpa.llama3_inv_freq(d, (1e4, 5e5, 1e6, 1e7)[g % 4], factor=8.0 * (g + 1),
                                    low_freq_factor=1.0, high_freq_factor=4.0,
                                    original_max_position=4096)
        rows.append(t)
    rows = np.stack(rows)
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=97 + d)
    count, idx = _lists(B, Hq, N, 0.3, seed=98)
    pos = _positions(B, N, "gapped", seed=100) if at_pos else None
    say("block sparse per-head tables", shape, "positions" if at_pos else "")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lse = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), 1e4, 1.0, want_lse=True, term_count=cnt,
                           out_dtype=torch.float32, block_count=torch.from_numpy(count).cuda(),
                           block_idx=torch.from_numpy(idx).cuda(), inv_freq=rows,
                           positions=None if pos is None else torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    ro, rl, kept = oracle.prefill_sparse(exact(q), exact(k), exact(v), 1e4, 1.0, count, idx,
                                         inv_freq=rows, pos=pos)
    check_close(out.cpu().numpy(), ro, "out")
    check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
    assert int(cnt.item()) == kept


def test_block_sparse_lists_with_junk_and_truncation():
    """Duplicates, entries at or past the query block, -1, and lists longer than the
    width (truncated by count) are absorbed as the rule says."""
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 600, 4, 2, 64, 1e4
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=95)
    count, idx = _lists(B, Hq, N, 0.5, seed=96, width=5, junk=True)
    count = np.minimum(count + 2, 7).astype(np.int32)      # counts above the width are clamped
    say("block sparse junk")
    out, lse, cnt, ro, rl, kept = _run(q, k, v, base, 1.0, count, idx)
    check_close(out.cpu().numpy(), ro, "out")
    check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept


def test_block_sparse_empty_lists_are_block_local():
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 512, 7, 1, 64, 1e6
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=97)
    nblk = N // 64
    count = np.zeros((B, Hq, nblk), np.int32)
    idx = np.zeros((B, Hq, nblk, 1), np.int32)
    say("block sparse empty")
    out, lse, cnt, ro, rl, kept = _run(q, k, v, base, 1.0, count, idx)
    check_close(out.cpu().numpy(), ro, "out")
    assert cnt == kept


@pytest.mark.parametrize("d,Hq,Hkv,base", [(64, 14, 2, 1e6), (128, 24, 8, 5e5)])
def test_block_sparse_every_block_is_dense(d, Hq, Hkv, base):
    need_gpu()
    B, N = 1, 1000
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=98)
    nblk = (N + 63) // 64
    count = np.tile(np.arange(nblk, dtype=np.int32), (B, Hq, 1))
    idx = np.tile(np.arange(nblk, dtype=np.int32), (B, Hq, nblk, 1))
    say("block sparse all blocks", d)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    sp = wpa.prefill(qc, kc, vc, base, 1.0, out_dtype=torch.float32,
                     block_count=torch.from_numpy(count).cuda(), block_idx=torch.from_numpy(idx).cuda())
    de = wpa.prefill(qc, kc, vc, base, 1.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(sp, de)


def test_block_sparse_long_sampled_rows():
    """N = 8192 at Qwen2.5-0.5B heads, 10% random density plus sink and local blocks;
    sampled rows against the oracle, the full kept-term count against the oracle's."""
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 8192, 14, 2, 64, 1e6
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=99, dim_scale=True)
    count, idx = _lists(B, Hq, N, 0.1, seed=100)
    say("block sparse long")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), base, 1.0, term_count=cnt,
                      out_dtype=torch.float32, block_count=torch.from_numpy(count).cuda(),
                      block_idx=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    rows = synth.sample_rows(N, 24, seed=7)
    ro, _, _ = oracle.prefill_sparse(exact(q), exact(k), exact(v), base, 1.0, count, idx, rows=rows)
    check_close(out[:, rows].cpu().numpy(), ro, "sampled rows")
    # exact kept-term count on one head (the count is per q head)
    q1, k1, v1 = (t[:, :, :1].contiguous() for t in (q, k, v))
    c1, i1 = np.ascontiguousarray(count[:, :1]), np.ascontiguousarray(idx[:, :1])
    cnt1 = torch.zeros(1, dtype=torch.int64, device="cuda")
    wpa.prefill(q1.cuda(), k1.cuda(), v1.cuda(), base, 1.0, term_count=cnt1,
                block_count=torch.from_numpy(c1).cuda(), block_idx=torch.from_numpy(i1).cuda())
    torch.cuda.synchronize()
    _, _, kept = oracle.prefill_sparse(exact(q1), exact(k1), exact(v1), base, 1.0, c1, i1)
    assert int(cnt1.item()) == kept


def _expand(count, idx, f, N):
    """Lists over blocks of 64*f tokens as lists of 64-token blocks: a listed block becomes
    its f 64-token blocks, and each 64-row block also lists the earlier 64-token blocks of its
    own coarse block."""
    B, H, _ = count.shape
    nf = (N + 63) // 64
    rows = [[[sorted({c * f + j for c in idx[b, h, R // f, :min(max(int(count[b, h, R // f]), 0),
                                                                 idx.shape[3])]
                      if 0 <= c < R // f for j in range(f)} | set(range((R // f) * f, R)))
              for R in range(nf)] for h in range(H)] for b in range(B)]
    m = max(1, max(len(x) for bl in rows for hl in bl for x in hl))
    cf = np.zeros((B, H, nf), np.int32)
    xf = np.zeros((B, H, nf, m), np.int32)
    for b in range(B):
        for h in range(H):
            for R in range(nf):
                cf[b, h, R] = len(rows[b][h][R])
                xf[b, h, R, :cf[b, h, R]] = rows[b][h][R]
    return cf, xf


@pytest.mark.parametrize("blk,N", [(128, 1300), (256, 1300), (1024, 2500)])
@pytest.mark.parametrize("d,Hq,Hkv,base", [(64, 14, 2, 1e6), (128, 24, 8, 5e5)])
def test_block_sparse_other_block_sizes(blk, N, d, Hq, Hkv, base):
    """Blocks of 128, 256 and 1024 tokens (N not a multiple of the block): outputs, LSE and
    counts against the oracle at that block size, and bit-identical to the 64-token call on
    the expanded lists (the same visited keys)."""
    need_gpu()
    q, k, v = synth.prefill_inputs(1, N, Hq, Hkv, d, "bf16", seed=95 + d)
    count, idx = _lists(1, Hq, N, 0.3, seed=96, junk=True, blk=blk)
    say("block sparse blocks of", blk, "d", d)
    out, lse, cnt, ro, rl, kept = _run(q, k, v, base, 1.0, count, idx, blk=blk)
    check_close(out.cpu().numpy(), ro, "out")
    check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept
    cf, xf = _expand(count, idx, blk // 64, N)
    c64 = torch.zeros(1, dtype=torch.int64, device="cuda")
    o64, l64 = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), base, 1.0, want_lse=True, term_count=c64,
                           out_dtype=torch.float32, block_count=torch.from_numpy(cf).cuda(),
                           block_idx=torch.from_numpy(xf).cuda())
    torch.cuda.synchronize()
    assert torch.equal(out, o64) and torch.equal(lse, l64) and int(c64.item()) == cnt


def _positions(B, N, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "gapped":
        pos = np.cumsum(rng.integers(0, 40, (B, N)), axis=1) + 1000
    elif kind == "repeated":
        pos = np.cumsum(rng.integers(0, 2, (B, N)), axis=1)
    else:                                   # near the top of the int32 range
        pos = (2 ** 31 - 2 - N) + np.arange(N)[None, :].repeat(B, 0)
    return np.ascontiguousarray(pos, dtype=np.int32)


@pytest.mark.parametrize("kind", ["gapped", "repeated", "high"])
@pytest.mark.parametrize("blk", [64, 256])
@pytest.mark.parametrize("d,Hq,Hkv,base", [(64, 14, 2, 1e6), (128, 24, 8, 5e5)])
def test_block_sparse_at_explicit_positions(kind, blk, d, Hq, Hkv, base):
    """Block sparsity at explicit positions (blocks by token index; rotation and window at the
    positions): outputs, LSE and kept-term counts against the oracle given the same
    positions, with junk entries in the lists and N not a multiple of the block."""
    need_gpu()
    B, N = 2, 1100
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=97 + d)
    count, idx = _lists(B, Hq, N, 0.3, seed=98, junk=True, blk=blk)
    pos = _positions(B, N, kind, seed=99)
    say("block sparse at positions", kind, "blk", blk, "d", d)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lse = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), base, 1.0, want_lse=True, term_count=cnt,
                           out_dtype=torch.float32, positions=torch.from_numpy(pos).cuda(),
                           block_count=torch.from_numpy(count).cuda(),
                           block_idx=torch.from_numpy(idx).cuda(), block=blk)
    torch.cuda.synchronize()
    ro, rl, kept = oracle.prefill_sparse(exact(q), exact(k), exact(v), base, 1.0, count, idx,
                                         blk=blk, pos=pos)
    check_close(out.cpu().numpy(), ro, "out")
    check_close(lse.cpu().numpy(), rl, "lse", LSE_MAX, LSE_MAX)
    assert int(cnt.item()) == kept


def test_block_sparse_positions_every_block_equals_dense_at_positions():
    """With every earlier block listed, the sparse call at positions visits the keys of the
    dense prefill at the same positions: the two agree within the oracle bar, with the same
    kept-term count (different kernel instances, so not bit for bit)."""
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 900, 14, 2, 64, 1e6
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=101)
    pos = torch.from_numpy(_positions(B, N, "gapped", seed=102)).cuda()
    nblk = (N + 63) // 64
    count = np.tile(np.arange(nblk, dtype=np.int32), (B, Hq, 1))
    idx = np.tile(np.arange(max(nblk, 1), dtype=np.int32), (B, Hq, nblk, 1))
    c1 = torch.zeros(1, dtype=torch.int64, device="cuda")
    c2 = torch.zeros(1, dtype=torch.int64, device="cuda")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = wpa.prefill(qd, kd, vd, base, 1.0, want_lse=True, term_count=c1, positions=pos,
                         out_dtype=torch.float32, block_count=torch.from_numpy(count).cuda(),
                         block_idx=torch.from_numpy(idx).cuda())
    o2, l2 = wpa.prefill(qd, kd, vd, base, 1.0, want_lse=True, term_count=c2, positions=pos,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_close(o1.cpu().numpy(), o2.cpu().numpy().astype(np.float64), "out")
    check_close(l1.cpu().numpy(), l2.cpu().numpy().astype(np.float64), "lse", LSE_MAX, LSE_MAX)
    assert int(c1.item()) == int(c2.item())

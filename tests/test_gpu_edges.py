"""GPU parity on the edges of the contract: explicit positions at d = 64, positions next to
the 2^31 limit, one-shot fp32 inputs at d = 128, large-magnitude q/k inside the half-precision
operand range, decode lengths the kernels clamp, and the full attention matrix of the tiny
configuration reconstructed column by column against the oracle's."""
import math

import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, as_bf16_for_oracle, check_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _prefill(q, k, v, base, alpha, positions=None):
    dev = "cuda"
    pos = None if positions is None else torch.as_tensor(positions, dtype=torch.int32).to(dev)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    out, lse = wpa.prefill(q.to(dev), k.to(dev), v.to(dev), base, alpha, positions=pos,
                           want_lse=True, term_count=cnt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), int(cnt.item())


def _oracle(q, k, v, base, alpha, positions=None):
    return oracle.prefill(as_bf16_for_oracle(q), as_bf16_for_oracle(k), as_bf16_for_oracle(v),
                          base, alpha, pos=positions)


def _gapped(B, N, rng, max_gap, start):
    return (np.cumsum(rng.integers(0, max_gap, (B, N)), axis=1) + start).astype(np.int64)


@pytest.mark.parametrize("kind", ["gapped", "repeated", "sparse_far"])
def test_d64_explicit_positions(kind):
    """The d = 64 kernel with explicit positions (its own register budget and the per-element
    straddling path), at the Qwen2.5-0.5B head shape, 1100 tokens over several tiles."""
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 1100, 14, 2, 64, 1e6
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=21, dim_scale=True)
    rng = np.random.default_rng(5)
    if kind == "gapped":
        pos = _gapped(B, N, rng, 40, 1000)
    elif kind == "repeated":
        pos = _gapped(B, N, rng, 2, 0)
    else:                       # long jumps: distances beyond most windows within one tile
        pos = _gapped(B, N, rng, 5000, 7)
    say("d64 positions", kind)
    out, lse, cnt = _prefill(q, k, v, base, 1.0, pos)
    ro, rl, kept = _oracle(q, k, v, base, 1.0, pos)
    check_close(out, ro, "out")
    check_close(lse, rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept


@pytest.mark.parametrize("d,Hq,Hkv,base", [(128, 8, 2, 5e5), (64, 4, 2, 1e4)])
def test_positions_near_int32_limit(d, Hq, Hkv, base):
    """Positions ending at 2^31 - 1 (the ABI's limit): angles of about 2^31 radians exercise
    the kernels' fp64 angle reduction; distances stay small, so the window is as usual."""
    need_gpu()
    B, N = 2, 600
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=22)
    rng = np.random.default_rng(6)
    steps = rng.integers(0, 3, (B, N))
    pos = np.cumsum(steps, axis=1)
    pos = pos - pos[:, -1:] + (2 ** 31 - 1)          # last position of each sequence is 2^31 - 1
    assert pos.min() >= 0 and pos.max() == 2 ** 31 - 1
    say("positions near 2^31", d)
    out, lse, cnt = _prefill(q, k, v, base, 1.0, pos)
    ro, rl, kept = _oracle(q, k, v, base, 1.0, pos)
    check_close(out, ro, "out")
    check_close(lse, rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept


@pytest.mark.parametrize("alpha", [1.0, math.inf])
def test_one_shot_fp32_inputs_d128(alpha):
    """One-shot prefill with fp32 q, k, v at d = 128 (rounded to bf16 on load); the oracle sees
    the same rounded values."""
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 777, 24, 8, 128, 5e5
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "fp32", seed=23)
    say("fp32 d128", alpha)
    out, lse, cnt = _prefill(q, k, v, base, alpha)
    ro, rl, kept = _oracle(q, k, v, base, alpha)
    check_close(out, ro, "out")
    check_close(lse, rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept


def _outlier_pairs(B, N, Hq, Hkv, d, seed):
    """q and k with a per-pair magnitude 10^u, u ~ U[-3, 3] on q and the reciprocal (times a
    log-uniform [0.5, 2] factor) on k: components reach several thousand, inside the half
    range the header states, while each pair's q.k term stays O(1) (outlier channels of real
    checkpoints have this spread)."""
    g = torch.Generator().manual_seed(seed)
    P = d // 2
    u = torch.rand((P,), generator=g) * 6.0 - 3.0
    a = torch.pow(10.0, u)
    f = torch.exp(math.log(0.5) + torch.rand((P,), generator=g) * math.log(4.0))
    sq = torch.cat([a, a])                       # both dims of a pair share the scale
    sk = torch.cat([f / a, f / a])
    q = (torch.randn((B, N, Hq, d), generator=g) * sq).to(torch.bfloat16)
    k = (torch.randn((B, N, Hkv, d), generator=g) * sk).to(torch.bfloat16)
    v = torch.randn((B, N, Hkv, d), generator=g).to(torch.bfloat16)
    return q, k, v


@pytest.mark.parametrize("d,Hq,Hkv,base", [(64, 14, 2, 1e6), (128, 24, 8, 5e5)])
def test_large_magnitude_pairs(d, Hq, Hkv, base):
    need_gpu()
    q, k, v = _outlier_pairs(1, 700, Hq, Hkv, d, seed=24 + d)
    mx = max(q.float().abs().max().item(), k.float().abs().max().item())
    assert 1e3 < mx < 6e4, mx                    # large, and below the half overflow bound
    say("large-magnitude pairs", d, "max |x| %.0f" % mx)
    for alpha in (1.0, math.inf):
        out, lse, cnt = _prefill(q, k, v, base, alpha)
        ro, rl, kept = _oracle(q, k, v, base, alpha)
        check_close(out, ro, "out alpha=%g" % alpha)
        check_close(lse, rl, "lse", LSE_MAX, LSE_MAX)
        assert cnt == kept


def test_decode_lengths_are_clamped():
    """kv_len above Lmax decodes as Lmax; kv_len 0 (or negative) gives out = 0, lse = -inf."""
    need_gpu()
    B, Lmax, Hq, Hkv, d, base = 4, 700, 8, 2, 128, 5e5
    q, k, v, _ = synth.decode_inputs(B, Lmax, Hq, Hkv, d, "bf16", seed=25, len_lo=1)
    cache = wpa.KVCache(B, Lmax, Hkv, d, base)
    cache.write(k.cuda(), v.cuda(), 0)
    lens = torch.tensor([Lmax + 5, 0, -3, 300], dtype=torch.int32)
    say("decode clamped lengths")
    out, lse = wpa.decode(q.cuda(), cache, lens.cuda(), 1.0, want_lse=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    eff = np.array([Lmax, 1, 1, 300])             # oracle lengths; rows 1 and 2 are checked apart
    ro, rl, _ = oracle.decode(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v), eff, base, 1.0)
    for b in (0, 3):
        check_close(out[b], ro[b], "out seq %d" % b)
        check_close(lse[b], rl[b], "lse seq %d" % b, LSE_MAX, LSE_MAX)
    for b in (1, 2):
        assert np.all(out[b] == 0.0) and np.all(np.isneginf(lse[b])), b


# ------------------------------------------------------------------ attention matrix
N1, H1, D1, BASE1 = 256, 2, 64, 1e4          # the tiny configuration


def _attention_matrix(q, k, alpha, gpu):
    """P[h][r][c], reconstructed from N/d launches whose values are one-hot columns: launch j
    has v[c][h][e] = 1 iff c = j*d + e, so out[r][h][e] = P[h][r][j*d + e]."""
    P = np.zeros((H1, N1, N1))
    for j in range(N1 // D1):
        v = torch.zeros((1, N1, H1, D1))
        for e in range(D1):
            v[0, j * D1 + e, :, e] = 1.0
        if gpu:
            o = wpa.prefill(q.cuda(), k.cuda(), v.cuda(), BASE1, alpha, out_dtype=torch.float32)
            torch.cuda.synchronize()
            o = o.cpu().numpy()
        else:
            o, _, _ = oracle.prefill(as_bf16_for_oracle(q), as_bf16_for_oracle(k),
                                     as_bf16_for_oracle(v), BASE1, alpha)
        P[:, :, j * D1:(j + 1) * D1] = o[0].transpose(1, 0, 2)
    return P


def _diagonal_mass(P):
    """Mean attention weight at each distance D = r - c (over heads and rows)."""
    return np.array([P[:, np.arange(D, N1), np.arange(0, N1 - D)].mean() for D in range(N1)])


@pytest.mark.parametrize("alpha", [1.0, math.inf])
def test_tiny_attention_matrix(alpha):
    """The whole 2 x 256 x 256 attention matrix of the tiny configuration (fp32 N(0,1)
    inputs), element by element against the oracle's; exact zeros above the diagonal."""
    need_gpu()
    q, k, _ = synth.workload_inputs(synth.WORKLOADS["tiny"])
    say("tiny attention matrix", alpha)
    Pg = _attention_matrix(q, k, alpha, gpu=True)
    Po = _attention_matrix(q, k, alpha, gpu=False)
    check_close(Pg, Po, "P alpha=%g" % alpha)
    iu = np.triu_indices(N1, 1)
    assert np.all(Pg[:, iu[0], iu[1]] == 0.0)
    assert np.abs(Pg.sum(-1) - 1.0).max() < 1e-2


def test_tiny_attention_matrix_window_changes_it():
    """On the tiny inputs the window moves attention weights by far more than the tolerance."""
    need_gpu()
    q, k, _ = synth.workload_inputs(synth.WORKLOADS["tiny"])
    say("tiny attention matrix, alpha 1 vs inf")
    P1 = _attention_matrix(q, k, 1.0, gpu=True)
    Pi = _attention_matrix(q, k, math.inf, gpu=True)
    assert np.abs(P1 - Pi).max() > 10 * 1e-2


def test_window_removes_ghost_diagonal():
    """Position aliasing (WavePrune, What the paper found): on inputs whose score depends on
    distance alone, the full window puts weight on a far sub-diagonal where the fast pairs
    come back into phase; the window (alpha = 1) drops those pairs there and the sub-diagonal
    fades.  The GPU's per-distance weights match the oracle's in both modes."""
    need_gpu()
    q, k, _ = synth.alias_inputs(N1, H1, D1, "fp32", seed=10, amp=5.0)
    W = oracle.thresholds(D1, BASE1, 1.0)
    lo = int(W[4]) + 1                       # distances past the window of the 5 fastest pairs
    say("ghost diagonal")
    M = {}
    for alpha in (1.0, math.inf):
        Pg = _attention_matrix(q, k, alpha, gpu=True)
        Po = _attention_matrix(q, k, alpha, gpu=False)
        check_close(Pg, Po, "P alpha=%g" % alpha)
        mg, mo = _diagonal_mass(Pg), _diagonal_mass(Po)
        assert np.all(np.abs(mg - mo) <= 0.02 * mo + 1e-6), alpha
        M[alpha] = (mg, mo)
    ghost = lo + int(np.argmax(M[math.inf][1][lo:]))     # the oracle's far peak, full window
    for which in (0, 1):                                 # GPU, oracle
        full, win = M[math.inf][which][ghost], M[1.0][which][ghost]
        say("  ghost distance %d: full %.2e, windowed %.2e" % (ghost, full, win))
        assert full > 10 * win

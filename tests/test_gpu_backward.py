"""GPU parity of the windowed prefill's backward (C ABI through the binding) against the fp64
oracle's backward, on the same bf16 inputs and the same dout.

Tolerance (derived from the arithmetic): the kernels recompute P from the forward's fp32 lse
with rotated q and k rounded to IEEE half (relative 2^-11), feed P to the dv product as bf16
(2^-9) and dl = P (dP - D) to the dq and dk products as half.  Every gradient is a sum of such
rounded terms weighted by softmax probabilities, so its error is a small multiple of 2^-9 of the
gradient's own scale.  The bound is max-abs <= 1e-2 * s and mean-abs <= 1e-3 * s, with s the
larger of 1 and the reference's root-mean-square (the forward's output bar, in the units of
the gradient)."""
import math

import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import check_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _bar(ref):
    s = max(1.0, float(np.sqrt(np.mean(np.square(ref)))))
    return 1e-2 * s, 1e-3 * s


def _check(got, ref, what):
    mx, mn = _bar(ref)
    check_close(got, ref, what, mx, mn)


def _gpu_grads(q, k, v, g, base, alpha, **kw):
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, g))
    out, lse = wpa.prefill(qd, kd, vd, base, alpha, want_lse=True, out_dtype=torch.float32, **kw)
    dq, dk, dv = wpa.prefill_backward(qd, kd, vd, out, lse, gd, base, alpha, **kw)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def _oracle_grads(q, k, v, g, base, alpha, rows=None, keys=None, **kw):
    return oracle.prefill_backward(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                   synth.to_oracle(g), base, alpha, rows=rows, keys=keys, **kw)


def _dout(shape, seed):
    return torch.randn(shape, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)


@pytest.mark.parametrize("alpha", [1.0, 2.0, math.inf])
def test_tiny_backward_matches_oracle(alpha):
    """The tiny configuration (B=1, 2/2 heads, d=64, N=256, base 1e4), inputs rounded to bf16."""
    need_gpu()
    w = synth.WORKLOADS["tiny"]
    q, k, v = (t.to(torch.bfloat16) for t in synth.workload_inputs(w))
    g = _dout(q.shape, 80)
    say("tiny backward", alpha)
    dq, dk, dv = _gpu_grads(q, k, v, g, w.base, alpha)
    rq, rk, rv = _oracle_grads(q, k, v, g, w.base, alpha)
    _check(dq, rq, "dq")
    _check(dk, rk, "dk")
    _check(dv, rv, "dv")


@pytest.mark.parametrize("shape", [
    # B, N, Hq, Hkv, d, base (several 32-row groups, a ragged tail, GQA ratios 7, 3, 16, 1)
    (1, 1000, 14, 2, 64, 1e6),
    (2, 500, 24, 8, 128, 5e5),
    (1, 333, 16, 1, 128, 1e4),
    (1, 130, 4, 4, 64, 1e4),
    (1, 1, 2, 1, 64, 1e4),
    (1, 31, 2, 2, 128, 1e4),
])
@pytest.mark.parametrize("alpha", [1.0, 2.0])
def test_backward_shapes_match_oracle(shape, alpha):
    need_gpu()
    B, N, Hq, Hkv, d, base = shape
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=200 + N)
    g = _dout(q.shape, 81 + N)
    say("backward", shape, alpha)
    dq, dk, dv = _gpu_grads(q, k, v, g, base, alpha)
    rq, rk, rv = _oracle_grads(q, k, v, g, base, alpha)
    _check(dq, rq, "dq %s" % (shape,))
    _check(dk, rk, "dk")
    _check(dv, rv, "dv")


@pytest.mark.parametrize("pairs", ["half", "interleaved"])
def test_backward_variants_match_oracle(pairs):
    """A Llama-3-style frequency table, half-split and interleaved pairs."""
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 400, 24, 8, 128, 5e5
    theta = wpa.llama3_inv_freq(d, base, factor=32.0, low_freq_factor=1.0, high_freq_factor=4.0,
                                original_max_position=8192)
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=83)
    g = _dout(q.shape, 84)
    say("backward variant", pairs)
    dq, dk, dv = _gpu_grads(q, k, v, g, base, 1.0, inv_freq=theta, pairs=pairs)
    rq, rk, rv = _oracle_grads(q, k, v, g, base, 1.0, inv_freq=theta, layout=pairs)
    _check(dq, rq, "dq")
    _check(dk, rk, "dk")
    _check(dv, rv, "dv")


def test_backward_window_changes_gradients():
    """On position-aliasing inputs the windowed and full-window gradients differ by far more
    than the bar, and each matches its own oracle."""
    need_gpu()
    N, H, d, base = 512, 2, 64, 1e4
    q, k, v = synth.alias_inputs(N, H, d, "bf16", seed=10, amp=3.5)
    g = _dout(q.shape, 85)
    say("backward discrimination")
    res = {}
    for alpha in (1.0, math.inf):
        dq, dk, dv = _gpu_grads(q, k, v, g, base, alpha)
        rq, rk, rv = _oracle_grads(q, k, v, g, base, alpha)
        _check(dq, rq, "dq alpha=%g" % alpha)
        _check(dk, rk, "dk")
        _check(dv, rv, "dv")
        res[alpha] = (rq, dq)
    assert np.abs(res[1.0][0] - res[math.inf][0]).max() > 10 * _bar(res[1.0][0])[0]
    assert np.abs(res[1.0][1] - res[math.inf][1]).max() > 10 * _bar(res[1.0][0])[0]


def test_backward_huge_alpha_is_bitwise_full_window():
    need_gpu()
    q, k, v = synth.prefill_inputs(1, 700, 14, 2, 64, "bf16", seed=86)
    g = _dout(q.shape, 87)
    say("backward bitwise full window")
    a = _gpu_grads(q, k, v, g, 1e6, math.inf)
    b = _gpu_grads(q, k, v, g, 1e6, 1e9)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_full_size_qwen05b_backward_sampled():
    """The Qwen2.5-0.5B-shaped layer at its full 32768 tokens: dq of sampled rows (first, last,
    random) and dk, dv of the last 64 keys against the oracle."""
    need_gpu()
    w = synth.WORKLOADS["qwen05b"]
    say("full size qwen05b backward")
    q, k, v = synth.workload_inputs(w, device="cuda")
    g = torch.randn(q.shape, generator=torch.Generator(device="cuda").manual_seed(88),
                    device="cuda").to(torch.bfloat16)
    out, lse = wpa.prefill(q, k, v, w.base, 1.0, want_lse=True, out_dtype=torch.float32)
    dq, dk, dv = wpa.prefill_backward(q, k, v, out, lse, g, w.base, 1.0)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w.N, 16, seed=w.seed)
    keys = np.arange(w.N - 64, w.N)
    gq = dq[:, torch.as_tensor(rows, device="cuda")].cpu().numpy()
    gk = dk[:, torch.as_tensor(keys, device="cuda")].cpu().numpy()
    gv = dv[:, torch.as_tensor(keys, device="cuda")].cpu().numpy()
    del dq, dk, dv, out, lse
    say("oracle rows", len(rows), "keys", len(keys))
    rq, rk, rv = oracle.prefill_backward(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                         synth.to_oracle(g), w.base, 1.0, rows=rows, keys=keys)
    _check(gq, rq, "qwen05b dq sampled rows")
    _check(gk, rk, "qwen05b dk last keys")
    _check(gv, rv, "qwen05b dv last keys")

"""GPU parity of the windowed prefill (C ABI through the Python binding) against the fp64
oracle, plus kept-term counts, full-window identity, determinism and discrimination."""
import math

import numpy as np
import pytest
import torch

import oracle
import rope_wavelength_sparsity_amd as wpa
import synth
from gpu_util import LSE_MAX, as_bf16_for_oracle, check_close, need_gpu, say

pytestmark = pytest.mark.gpu


def _run(q, k, v, base, alpha, positions=None, count=False, check_bf16_out=True):
    """fp32 output (the tolerance applies to the fp32-accumulated result); when the inputs
    are bf16, also check that the bf16 output is exactly that result rounded to nearest even."""
    dev = "cuda"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    pos = None if positions is None else torch.as_tensor(positions, dtype=torch.int32).to(dev)
    cnt = torch.zeros(1, dtype=torch.int64, device=dev) if count else None
    out, lse = wpa.prefill(qd, kd, vd, base, alpha, positions=pos, want_lse=True, term_count=cnt,
                           out_dtype=torch.float32)
    if check_bf16_out and q.dtype == torch.bfloat16:
        ob = wpa.prefill(qd, kd, vd, base, alpha, positions=pos)
        assert ob.dtype == torch.bfloat16 and torch.equal(ob, out.to(torch.bfloat16))
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), (int(cnt.item()) if count else None)


def _oracle(q, k, v, base, alpha, positions=None, rows=None):
    return oracle.prefill(as_bf16_for_oracle(q), as_bf16_for_oracle(k), as_bf16_for_oracle(v),
                          base, alpha, pos=positions, rows=rows)


@pytest.mark.parametrize("alpha", [1.0, 2.0, math.inf, 0.0, 0.3])
def test_tiny_prefill_matches_oracle(alpha):
    """B=1, 2/2 heads, d=64, N=256, base 1e4, fp32 N(0,1)."""
    need_gpu()
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.workload_inputs(w)
    say("tiny prefill alpha", alpha)
    out, lse, cnt = _run(q, k, v, w.base, alpha, count=True)
    ro, rl, kept = _oracle(q, k, v, w.base, alpha)
    check_close(out, ro, "out")
    check_close(lse, rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept == w.Hq * wpa.count_terms(w.d, w.base, alpha, w.N, 0, w.N)[0]


@pytest.mark.parametrize("shape", [
    # B, N, Hq, Hkv, d, base, dim_scale  (several tiles and a ragged tail)
    (1, 1000, 14, 2, 64, 1e6, False),       # Qwen2.5-0.5B heads
    (2, 777, 24, 8, 128, 5e5, False),       # Llama-3.2-3B heads
    (1, 600, 28, 4, 128, 1e7, False),       # Qwen2.5-7B-1M heads
    (1, 130, 4, 4, 64, 1e4, False),         # G = 1: 8 row groups per workgroup
    (1, 333, 16, 1, 128, 1e4, False),       # G = 16: two head chunks
    (2, 65, 6, 2, 64, 1e4, False),          # G = 3
    (1, 1, 2, 1, 64, 1e4, False),           # one token
    (1, 31, 2, 2, 128, 1e4, False),
])
@pytest.mark.parametrize("alpha", [1.0, 2.0])
def test_prefill_shapes_match_oracle(shape, alpha):
    need_gpu()
    B, N, Hq, Hkv, d, base, ds = shape
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=100 + N, dim_scale=ds)
    say("prefill", shape, alpha)
    out, lse, cnt = _run(q, k, v, base, alpha, count=True)
    ro, rl, kept = _oracle(q, k, v, base, alpha)
    check_close(out, ro, "out %s" % (shape,))
    check_close(lse, rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept == B * Hq * wpa.count_terms(d, base, alpha, N, 0, N)[0]


@pytest.mark.parametrize("alpha", [1.0, 2.0])
def test_prefill_scaled_inputs(alpha):
    """Qwen2.5-0.5B-shaped inputs with the per-dim log-uniform [0.5, 2] scale on q and k at a
    short length (1000 tokens, where rows see few keys and attention is peaked): the input
    most sensitive to the rounding of the rotated q and k.  Rounded to bf16 they would by
    themselves cost 1.02e-2 max-abs here (emulated in fp64 on the CPU); the kernels round
    them to IEEE half (11 significant bits), which keeps this case inside the standard
    bounds."""
    need_gpu()
    B, N, Hq, Hkv, d, base = 1, 1000, 14, 2, 64, 1e6
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=100 + N, dim_scale=True)
    say("prefill scaled inputs", alpha)
    out, lse, cnt = _run(q, k, v, base, alpha, count=True)
    ro, rl, kept = _oracle(q, k, v, base, alpha)
    check_close(out, ro, "out")
    check_close(lse, rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept


@pytest.mark.parametrize("kind", ["gapped", "repeated"])
def test_prefill_explicit_positions(kind):
    need_gpu()
    B, N, Hq, Hkv, d, base = 2, 500, 8, 2, 128, 1e4
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=7)
    rng = np.random.default_rng(3)
    if kind == "gapped":
        pos = np.cumsum(rng.integers(0, 40, (B, N)), axis=1) + 1000
    else:
        pos = np.cumsum(rng.integers(0, 2, (B, N)), axis=1)
    pos = pos.astype(np.int32)
    say("prefill positions", kind)
    out, lse, cnt = _run(q, k, v, base, 1.0, positions=pos, count=True)
    ro, rl, kept = _oracle(q, k, v, base, 1.0, positions=pos)
    check_close(out, ro, "out")
    check_close(lse, rl, "lse", LSE_MAX, LSE_MAX)
    assert cnt == kept


def test_huge_alpha_is_bitwise_full_window():
    need_gpu()
    q, k, v = synth.prefill_inputs(1, 700, 14, 2, 64, "bf16", seed=8)
    say("bitwise full window")
    a, la, _ = _run(q, k, v, 1e6, math.inf)
    b, lb, _ = _run(q, k, v, 1e6, 1e9)     # every threshold beyond any distance
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_deterministic():
    need_gpu()
    q, k, v = synth.prefill_inputs(1, 900, 24, 8, 128, "bf16", seed=9)
    say("determinism")
    a, la, _ = _run(q, k, v, 5e5, 1.0)
    b, lb, _ = _run(q, k, v, 5e5, 1.0)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_window_changes_the_output():
    """On position-aliasing inputs the windowed and full-window outputs differ by far more
    than the tolerance, and each matches its own oracle."""
    need_gpu()
    N, H, d, base = 512, 2, 64, 1e4
    q, k, v = synth.alias_inputs(N, H, d, "bf16", seed=10, amp=3.5)
    say("discrimination")
    o1, _, _ = _run(q, k, v, base, 1.0)
    oi, _, _ = _run(q, k, v, base, math.inf)
    r1, _, _ = _oracle(q, k, v, base, 1.0)
    ri, _, _ = _oracle(q, k, v, base, math.inf)
    check_close(o1, r1, "windowed")
    check_close(oi, ri, "full")
    assert np.abs(r1 - ri).max() > 10 * 1e-2
    assert np.abs(o1 - oi).max() > 10 * 1e-2


@pytest.mark.parametrize("name,alpha", [("qwen05b", 1.0), ("llama3b", 1.0), ("llama3b", 2.0)])
def test_full_size_sampled_rows(name, alpha):
    """Full workload sizes, in the launch configuration the bench times; sampled query rows
    (first, last and random) against the oracle; exact kept-term count."""
    need_gpu()
    w = synth.WORKLOADS[name]
    say("full size", name, alpha)
    q, k, v = synth.workload_inputs(w, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = wpa.prefill(q, k, v, w.base, alpha, term_count=cnt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w.N, 48, seed=w.seed)
    got = out[:, torch.as_tensor(rows, device="cuda")].float().cpu().numpy()
    say("oracle rows", len(rows))
    ro, _, _ = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                              w.base, alpha, rows=rows)
    check_close(got, ro, "%s sampled rows" % name)
    assert int(cnt.item()) == w.Hq * wpa.count_terms(w.d, w.base, alpha, w.N, 0, w.N)[0]


def test_full_size_qwen7b1m_sampled_rows():
    """The Qwen2.5-7B-1M-shaped prefill at its full 1M tokens, in the launch configuration the
    sweep times: sampled query rows (first, last and random) against the oracle; exact
    kept-term count (about 3.4e14 at this size)."""
    need_gpu()
    w = synth.WORKLOADS["qwen7b1m"]
    say("full size", w.name, 1.0)
    q, k, v = synth.workload_inputs(w, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = wpa.prefill(q, k, v, w.base, 1.0, term_count=cnt)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w.N, 16, seed=w.seed)
    got = out[:, torch.as_tensor(rows, device="cuda")].float().cpu().numpy()
    del out
    say("oracle rows", len(rows))
    ro, _, _ = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                              w.base, 1.0, rows=rows)
    check_close(got, ro, "qwen7b1m sampled rows")
    assert int(cnt.item()) == w.Hq * wpa.count_terms(w.d, w.base, 1.0, w.N, 0, w.N)[0]

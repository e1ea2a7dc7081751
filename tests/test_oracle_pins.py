"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

None of these re-types the oracle's own loop: each compares it with an independent
formulation (complex-number rotation, library softmax attention, closed forms,
invariants, hand-derived tiny cases, three separate count enumerations).

Sources:
  ATFlash abstract ("Per-RoPE-Wavelength Attention Windows for Compute/Memory-Efficient
  LLM Inference"): exact decomposition over 2-D rotation pairs; pruning beyond a
  wavelength-proportional distance; every key reachable through low-frequency pairs;
  a dropped share fixed by the shapes alone that grows like log N; online softmax untouched.
  WavePrune original abstract ("One period is often enough for RoPE"): alpha=1 is the
  first rotation period.
  "The Heterogeneous Feature of RoPE-based Attention", Explanation: the critical
  dimension (pairs completing a full period inside the context).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import synth


def _complex_rope(x, pos, base):
    """Independent rotation: pair i of a half-split vector as the complex number
    x_i + 1j*x_{i+P}, multiplied by exp(1j*pos*theta_i)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    P = d // 2
    theta = np.power(float(base), -np.arange(P) * 2.0 / d)
    z = x[..., :P] + 1j * x[..., P:]
    ang = np.asarray(pos, dtype=np.float64).reshape((-1,) + (1,) * (x.ndim - 1)) * theta
    zr = z * np.exp(1j * ang)
    return np.concatenate([zr.real, zr.imag], axis=-1)


def _f64(t):
    return t.double().numpy()


def test_rope_is_complex_multiplication():
    q, _, _ = synth.prefill_inputs(1, 37, 3, 3, 16, "fp32", seed=11)
    pos = np.arange(37) * 101 + 5
    got = oracle.rope(synth.to_oracle(q[0]), pos, 1e4)
    ref = _complex_rope(_f64(q[0]), pos, 1e4)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_full_window_equals_library_sdpa(dtype):
    """alpha = inf is ordinary causal RoPE attention."""
    B, N, Hq, Hkv, d, base = 2, 45, 4, 2, 16, 1e4
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, dtype, seed=3)
    out, lse, kept = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                    base, math.inf)
    pos = np.arange(N)
    qr = torch.from_numpy(np.stack([_complex_rope(_f64(q[b]), pos, base) for b in range(B)]))
    kr = torch.from_numpy(np.stack([_complex_rope(_f64(k[b]), pos, base) for b in range(B)]))
    vv = v.double()
    G = Hq // Hkv
    kr = kr.repeat_interleave(G, dim=2)
    vv = vv.repeat_interleave(G, dim=2)
    ref = F.scaled_dot_product_attention(qr.transpose(1, 2), kr.transpose(1, 2),
                                         vv.transpose(1, 2), is_causal=True)
    np.testing.assert_allclose(out, ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    s = (qr.transpose(1, 2) @ kr.transpose(1, 2).transpose(-1, -2)) / math.sqrt(d)
    s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)
    assert kept == B * Hq * (d // 2) * N * (N + 1) // 2


def test_huge_alpha_is_bitwise_full_window():
    q, k, v = synth.prefill_inputs(1, 60, 2, 1, 32, "bf16", seed=4)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    o1, l1, _ = oracle.prefill(*a, 1e4, math.inf)
    o2, l2, _ = oracle.prefill(*a, 1e4, 1e9)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def _relative_form(q, k, v, qpos, kpos, base, alpha, scale, visible=None):
    """Windowed attention written with the relative (complex) form of each pair's term:
    Term_i = Re( zq_i * conj(zk_i) * exp(1j*(tq - tk)*theta_i) ), computed on pre-RoPE
    vectors; softmax from scipy.  q [Nq][d], k, v [Nk][d]; causal by token index; an
    optional boolean visible [Nq][Nk] removes keys from the softmax."""
    d = q.shape[-1]
    P = d // 2
    theta = np.power(float(base), -np.arange(P) * 2.0 / d)
    lam = 2.0 * np.pi * np.power(float(base), np.arange(P) * 2.0 / d)
    zq = q[:, :P] + 1j * q[:, P:]
    zk = k[:, :P] + 1j * k[:, P:]
    dt = (np.asarray(qpos, np.float64)[:, None] - np.asarray(kpos, np.float64)[None, :])
    terms = np.real(zq[:, None, :] * np.conj(zk[None, :, :]) * np.exp(1j * dt[..., None] * theta))
    keep = np.abs(dt)[..., None] <= alpha * lam
    logits = scale * np.where(keep, terms, 0.0).sum(-1)
    Nq, Nk = logits.shape
    causal = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]
    if visible is not None:
        causal = causal & visible
    logits = np.where(causal, logits, -np.inf)
    p = scipy.special.softmax(logits, axis=-1)
    return p @ v, scipy.special.logsumexp(logits, axis=-1)


@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0, 2.0, 8.0])
@pytest.mark.parametrize("positions", ["default", "gapped", "nonmonotone"])
def test_windowed_equals_relative_form(alpha, positions):
    N, H, d, base = 40, 1, 16, 100.0
    q, k, v = synth.prefill_inputs(1, N, H, H, d, "fp32", seed=7)
    rng = np.random.default_rng(5)
    if positions == "default":
        pos = np.arange(N)
    elif positions == "gapped":
        pos = np.cumsum(rng.integers(0, 9, N))
    else:
        pos = rng.integers(0, 200, N)
    out, lse, _ = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 base, alpha, pos=pos)
    ref_o, ref_l = _relative_form(_f64(q[0, :, 0]), _f64(k[0, :, 0]), _f64(v[0, :, 0]),
                                  pos, pos, base, alpha, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(out[0, :, 0], ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], ref_l, rtol=0, atol=1e-12)


def test_alpha_zero_closed_form():
    """alpha = 0 keeps terms only at distance 0: row r has logit s*q_r.k_r on the diagonal
    (rotation by the same angle preserves the dot product) and 0 elsewhere, so
    out_r = (e^l v_r + sum_{c<r} v_c) / (e^l + r),  lse_r = log(e^l + r)."""
    N, d = 50, 32
    q, k, v = synth.prefill_inputs(1, N, 1, 1, d, "fp32", seed=9)
    out, lse, kept = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                    1e4, 0.0)
    qq, kk, vv = _f64(q[0, :, 0]), _f64(k[0, :, 0]), _f64(v[0, :, 0])
    ell = (qq * kk).sum(-1) / math.sqrt(d)
    csum = np.cumsum(vv, axis=0) - vv
    r = np.arange(N)[:, None]
    ref = (np.exp(ell)[:, None] * vv + csum) / (np.exp(ell)[:, None] + r)
    np.testing.assert_allclose(out[0, :, 0], ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.log(np.exp(ell) + np.arange(N)), rtol=0, atol=1e-12)
    assert kept == N * d // 2


@pytest.mark.parametrize("tk, alpha_steps, kept_far", [(6, 0, True), (7, 0, False),
                                                       (7, +7, True), (7, -1, False)])
def test_two_token_window_edge(tk, alpha_steps, kept_far):
    """Hand-derived d=2 case (one pair, theta_0 = 1, lambda_0 = 2*pi).  q = k = (1, 0) for
    both tokens, v_0 = (1, 0), v_1 = (0, 1).  Row 1 sees key 1 at distance 0 (term 1) and
    key 0 at distance tk (term cos(tk) if tk <= alpha*2*pi, else 0)."""
    alpha = 1.0
    if alpha_steps:
        alpha = 7.0 / (2.0 * math.pi)          # alpha*2*pi lands within an ulp of 7
        for _ in range(abs(alpha_steps)):
            alpha = float(np.nextafter(alpha, np.inf if alpha_steps > 0 else -np.inf))
    thr = oracle.thresholds(2, 1e4, alpha)[0]
    assert (tk <= thr) == kept_far
    q = np.array([[[[1.0, 0.0]], [[1.0, 0.0]]]], dtype=np.float32)
    v = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]], dtype=np.float32)
    out, lse, _ = oracle.prefill(q, q, v, 1e4, alpha, pos=np.array([0, tk]))
    s = 1.0 / math.sqrt(2.0)
    l0 = s * math.cos(tk) if kept_far else 0.0
    l1 = s * 1.0
    w0 = math.exp(l0) / (math.exp(l0) + math.exp(l1))
    np.testing.assert_allclose(out[0, 1, 0], [w0, 1.0 - w0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 0, 0], [1.0, 0.0], rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 1] - math.log(math.exp(l0) + math.exp(l1))) < 1e-15


def test_shift_invariance():
    """RoPE scores depend on positions only through their difference (WavePrune, original
    abstract); the window, a test on that difference, keeps this property."""
    N = 64
    q, k, v = synth.prefill_inputs(1, N, 2, 2, 32, "fp32", seed=12)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    pos = np.cumsum(np.random.default_rng(1).integers(0, 5, N))
    o1, l1, c1 = oracle.prefill(*a, 1e4, 1.0, pos=pos)
    o2, l2, c2 = oracle.prefill(*a, 1e4, 1.0, pos=pos + 123457)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-9)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-9)
    assert c1 == c2


def test_gqa_equals_repeated_kv():
    q, k, v = synth.prefill_inputs(1, 33, 6, 2, 16, "fp32", seed=13)
    a = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v), 1e4, 1.0)
    kr = k.repeat_interleave(3, dim=2)
    vr = v.repeat_interleave(3, dim=2)
    b = oracle.prefill(synth.to_oracle(q), synth.to_oracle(kr), synth.to_oracle(vr), 1e4, 1.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_sampled_rows_equal_full():
    q, k, v = synth.prefill_inputs(2, 70, 4, 2, 16, "bf16", seed=14)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    full_o, full_l, _ = oracle.prefill(*a, 1e4, 1.0)
    rows = np.array([0, 3, 31, 32, 69])
    o, l, _ = oracle.prefill(*a, 1e4, 1.0, rows=rows)
    assert np.array_equal(o, full_o[:, rows]) and np.array_equal(l, full_l[:, :, rows])


def test_decode_equals_last_prefill_row():
    B, L, Hq, Hkv, d = 3, 57, 4, 2, 32
    q, k, v = synth.prefill_inputs(B, L, Hq, Hkv, d, "bf16", seed=15)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    po, pl, _ = oracle.prefill(*a, 1e4, 1.0)
    lens = np.array([L, 20, 1], dtype=np.int32)
    for b in range(B):
        n = int(lens[b])
        qd = synth.to_oracle(q[:, n - 1])                  # [B][Hq][d]
        o, l, kept = oracle.decode(qd, a[1], a[2], lens, 1e4, 1.0)
        if n == L:
            np.testing.assert_allclose(o[b], po[b, L - 1], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l[b], pl[b, :, L - 1], rtol=0, atol=1e-13)
        pb, plb, _ = oracle.prefill(a[0][b:b + 1, :n], a[1][b:b + 1, :n], a[2][b:b + 1, :n],
                                    1e4, 1.0)
        np.testing.assert_allclose(o[b], pb[0, n - 1], rtol=0, atol=1e-13)


def test_decode_explicit_query_position():
    """q_pos = kv_len-1 is the default; an explicit q_pos shifts every distance."""
    B, L, H, d = 1, 40, 2, 16
    q, k, v, _ = synth.decode_inputs(B, L, H, H, d, "fp32", seed=16, len_lo=L)
    lens = np.array([L], np.int32)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    o1, _, _ = oracle.decode(*a, lens, 100.0, 1.0)
    o2, _, _ = oracle.decode(*a, lens, 100.0, 1.0, q_pos=np.array([L - 1], np.int32))
    assert np.array_equal(o1, o2)
    o3, l3, _ = oracle.decode(*a, lens, 100.0, 1.0, q_pos=np.array([L + 30], np.int32))
    # a query past its keys sees all of them: all-visible softmax of the relative form
    d2 = d // 2
    theta = np.power(100.0, -np.arange(d2) * 2.0 / d)
    lam = 2.0 * np.pi * np.power(100.0, np.arange(d2) * 2.0 / d)
    qq, kk, vv = _f64(q[0, 0]), _f64(k[0, :, 0]), _f64(v[0, :, 0])
    zq = qq[:d2] + 1j * qq[d2:]
    zk = kk[:, :d2] + 1j * kk[:, d2:]
    dt = (L + 30) - np.arange(L, dtype=np.float64)
    terms = np.real(zq[None] * np.conj(zk) * np.exp(1j * dt[:, None] * theta))
    logit = np.where(np.abs(dt)[:, None] <= lam, terms, 0.0).sum(-1) / math.sqrt(d)
    p = scipy.special.softmax(logit)
    np.testing.assert_allclose(o3[0, 0], p @ vv, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3[0, 0], scipy.special.logsumexp(logit), rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------- counts

GRID = [(d, base, alpha) for d in (2, 4, 16, 64, 128) for base in (10.0, 1e4, 1e6)
        for alpha in (0.0, 0.5, 1.0, 2.0, 8.0, math.inf)]


@pytest.mark.parametrize("d,base,alpha", GRID)
def test_count_three_enumerations_agree(d, base, alpha):
    for N in (1, 2, 7, 64, 300):
        a = oracle.count_enumerate(d, base, alpha, N, 0, N)
        b = oracle.count_bruteforce(d, base, alpha, N, 0, N)
        c = oracle.count_by_distance(d, base, alpha, N, 0, N)
        assert a == b == c
        assert a[1] == (d // 2) * N * (N + 1) // 2
    for L in (1, 5, 300):                                  # decode: one query at L-1
        a = oracle.count_enumerate(d, base, alpha, 1, L - 1, L)
        assert a == oracle.count_bruteforce(d, base, alpha, 1, L - 1, L)
        assert a == oracle.count_by_distance(d, base, alpha, 1, L - 1, L)
    a = oracle.count_enumerate(d, base, alpha, 37, 250, 260)   # chunk of queries
    assert a == oracle.count_bruteforce(d, base, alpha, 37, 250, 260)
    assert a == oracle.count_by_distance(d, base, alpha, 37, 250, 260)


def test_count_matches_attention_tally():
    """The kept-term tally of the attention oracle equals the enumerated count."""
    q, k, v = synth.prefill_inputs(1, 256, 2, 2, 64, "fp32", seed=1)
    _, _, kept = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                1e4, 1.0)
    assert kept == 2 * oracle.count_enumerate(64, 1e4, 1.0, 256, 0, 256)[0]


@pytest.mark.parametrize("d,base", [(128, 5e5), (64, 1e6), (128, 1e7)])
def test_pruned_fraction_grows_logarithmically(d, base):
    """ATFlash abstract: the dropped share of terms depends on the shapes alone and grows
    like log N.  Once
    every short-wavelength pair is well inside N, doubling N adds ln 2 / ln base to the
    pruned fraction (pairs are spaced ln(base)*2/d apart in ln(lambda))."""
    slope = math.log(2.0) / math.log(base)
    frac = {}
    for k in range(12, 21):
        N = 1 << k
        kept, total = oracle.count_by_distance(d, base, 1.0, N, 0, N)
        frac[k] = 1.0 - kept / total
    diffs = [frac[k + 1] - frac[k] for k in range(12, 20)]
    assert all(dd > 0 for dd in diffs)
    # the per-doubling increment oscillates around the slope with the pair spacing
    assert abs(np.mean(diffs) - slope) < 0.1 * slope
    assert all(abs(dd - slope) < 0.45 * slope for dd in diffs)


@pytest.mark.parametrize("N,alpha", [(256, 1.0), (300, 0.001), (300, 0.0), (1000, 0.01)])
def test_reachability(N, alpha):
    """ATFlash abstract: every key remains reachable through the low-frequency pairs.
    A (query, key) pair has no active term iff its distance exceeds the largest
    threshold; there are C(N - W, 2) such pairs, W = min(floor(alpha*lambda_max), N-1),
    which is zero whenever alpha*lambda_max >= N-1."""
    d, base = 64, 1e4
    thr = oracle.thresholds(d, base, alpha)
    r = np.arange(N)[:, None]
    c = np.arange(N)[None, :]
    dist = (r - c).astype(np.float64)
    visible = c <= r
    zero_terms = int(np.count_nonzero(visible & ~(dist[..., None] <= thr).any(-1)))
    W = min(math.floor(thr[-1]), N - 1)
    assert zero_terms == (N - W) * (N - W - 1) // 2
    if thr[-1] >= N - 1:
        assert zero_terms == 0


@pytest.mark.parametrize("d,base,N", [(64, 1e4, 256), (64, 1e6, 32768), (128, 5e5, 131072),
                                      (128, 1e7, 1 << 20)])
def test_critical_dimension(d, base, N):
    """'Heterogeneous Feature' talk, Explanation: the critical dimension counts the dims
    whose RoPE period completes inside the context.  At alpha = 1 those are exactly the
    pairs that ever lose a term inside N (a pair loses a term iff some visible distance
    exceeds its period)."""
    thr = oracle.thresholds(d, base, 1.0)
    ever_pruned = 0
    for t in thr:
        kept_i = int(np.sum((N - np.arange(N))[np.arange(N) <= t]))
        ever_pruned += kept_i < N * (N + 1) // 2
    periods = 2.0 * np.pi * np.power(base, np.arange(d // 2) * 2.0 / d)
    assert ever_pruned == int(np.count_nonzero(periods < N - 1))


# ------------------------------------------------------------------ RoPE variants
# A frequency table theta_i (frequency-scaled RoPE) gives pair i the wavelength
# 2*pi/theta_i; the interleaved layout pairs dims (2i, 2i+1).  Pins: complex rotation,
# library attention at alpha = inf, the relative complex form, a layout permutation, and
# hand values of the window table.

def _dims(d, layout):
    P = d // 2
    if layout == "interleaved":
        return np.arange(P) * 2, np.arange(P) * 2 + 1
    return np.arange(P), np.arange(P) + P


def _complex_rope_table(x, pos, theta, layout):
    """Pair i as the complex number x[dx_i] + 1j*x[dy_i], times exp(1j*pos*theta_i)."""
    x = np.asarray(x, dtype=np.float64)
    dx, dy = _dims(x.shape[-1], layout)
    z = x[..., dx] + 1j * x[..., dy]
    ang = np.asarray(pos, dtype=np.float64).reshape((-1,) + (1,) * (x.ndim - 1)) * theta
    zr = z * np.exp(1j * ang)
    out = np.empty_like(x)
    out[..., dx] = zr.real
    out[..., dy] = zr.imag
    return out


def _llama3_table(d, base):
    """Llama-3.2 style frequency scaling (factor 32, bands 1..4 of an 8192-token context),
    written out here independently of the package helper."""
    theta = base ** (-np.arange(d // 2) * 2.0 / d)
    lam = 2 * np.pi / theta
    out = theta.copy()
    for i, l in enumerate(lam):
        if l > 8192 / 1.0:
            out[i] = theta[i] / 32.0
        elif l >= 8192 / 4.0:
            s = (8192 / l - 1.0) / (4.0 - 1.0)
            out[i] = (1 - s) * theta[i] / 32.0 + s * theta[i]
    return out


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_rope_variants_are_complex_multiplication(layout):
    q, _, _ = synth.prefill_inputs(1, 29, 3, 3, 16, "fp32", seed=31)
    pos = np.arange(29) * 97 + 3
    theta = np.sort(np.random.default_rng(2).uniform(1e-4, 2.0, 8))[::-1].copy()
    got = oracle.rope(synth.to_oracle(q[0]), pos, 1e4, inv_freq=theta, layout=layout)
    np.testing.assert_allclose(got, _complex_rope_table(_f64(q[0]), pos, theta, layout), rtol=0,
                               atol=1e-12)


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_full_window_variant_equals_library_sdpa(layout):
    B, N, Hq, Hkv, d, base = 1, 41, 4, 2, 32, 5e5
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=33)
    theta = _llama3_table(d, base)
    out, lse, kept = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                    base, math.inf, inv_freq=theta, layout=layout)
    pos = np.arange(N)
    qr = torch.from_numpy(_complex_rope_table(_f64(q[0]), pos, theta, layout))[None]
    kr = torch.from_numpy(_complex_rope_table(_f64(k[0]), pos, theta, layout))[None]
    G = Hq // Hkv
    kr = kr.repeat_interleave(G, dim=2)
    vv = v.double().repeat_interleave(G, dim=2)
    ref = F.scaled_dot_product_attention(qr.transpose(1, 2), kr.transpose(1, 2),
                                         vv.transpose(1, 2), is_causal=True)
    np.testing.assert_allclose(out, ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    assert kept == B * Hq * (d // 2) * N * (N + 1) // 2


def _relative_form_table(q, k, v, qpos, kpos, theta, layout, alpha, scale, visible=None):
    """The relative complex form with a frequency table: Term_i = Re(zq_i conj(zk_i)
    exp(1j*(tq - tk)*theta_i)), kept iff |tq - tk| <= alpha*2*pi/theta_i; an optional boolean
    visible [Nq][Nk] removes keys from the softmax."""
    dx, dy = _dims(q.shape[-1], layout)
    zq = q[:, dx] + 1j * q[:, dy]
    zk = k[:, dx] + 1j * k[:, dy]
    dt = (np.asarray(qpos, np.float64)[:, None] - np.asarray(kpos, np.float64)[None, :])
    terms = np.real(zq[:, None, :] * np.conj(zk[None, :, :]) * np.exp(1j * dt[..., None] * theta))
    keep = np.abs(dt)[..., None] <= alpha * (2.0 * np.pi / theta)
    logits = scale * np.where(keep, terms, 0.0).sum(-1)
    Nq, Nk = logits.shape
    causal = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]
    if visible is not None:
        causal = causal & visible
    logits = np.where(causal, logits, -np.inf)
    return scipy.special.softmax(logits, axis=-1) @ v, scipy.special.logsumexp(logits, axis=-1)


@pytest.mark.parametrize("alpha", [0.5, 1.0, 2.0])
@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_windowed_variant_equals_relative_form(alpha, layout):
    N, H, d = 40, 1, 16
    q, k, v = synth.prefill_inputs(1, N, H, H, d, "fp32", seed=35)
    pos = np.cumsum(np.random.default_rng(7).integers(0, 6, N))
    theta = np.array([1.3, 0.9, 0.5, 0.31, 0.2, 0.11, 0.05, 0.02])     # decreasing
    out, lse, _ = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                 1e4, alpha, pos=pos, inv_freq=theta, layout=layout)
    ref_o, ref_l = _relative_form_table(_f64(q[0, :, 0]), _f64(k[0, :, 0]), _f64(v[0, :, 0]),
                                        pos, pos, theta, layout, alpha, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(out[0, :, 0], ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], ref_l, rtol=0, atol=1e-12)


def test_interleaved_is_half_split_of_permuted_dims():
    """Moving dims (2i, 2i+1) to (i, i+d/2) in q and k maps the interleaved layout onto the
    half-split one with identical outputs (v is untouched)."""
    B, N, Hq, Hkv, d = 1, 33, 2, 1, 16
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "fp32", seed=37)
    perm = np.concatenate([np.arange(d // 2) * 2, np.arange(d // 2) * 2 + 1])
    a = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v), 100.0, 1.0,
                       layout="interleaved")
    b = oracle.prefill(synth.to_oracle(q[..., perm].contiguous()),
                       synth.to_oracle(k[..., perm].contiguous()), synth.to_oracle(v), 100.0, 1.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    assert a[2] == b[2]


def test_table_thresholds_and_counts():
    """alpha * 2*pi / theta_i by hand, and the three count enumerations agree on a table."""
    theta = np.array([1.0, 0.5, 0.25, 0.001])
    np.testing.assert_array_equal(oracle.thresholds(8, 1e4, 1.5, inv_freq=theta),
                                  1.5 * (2.0 * math.pi / theta))
    d, theta = 64, _llama3_table(64, 5e5)
    for n_q, q0, n_k in [(300, 0, 300), (1, 4999, 5000), (70, 200, 250)]:
        a = oracle.count_enumerate(d, 5e5, 1.0, n_q, q0, n_k, inv_freq=theta)
        b = oracle.count_bruteforce(d, 5e5, 1.0, n_q, q0, n_k, inv_freq=theta)
        c = oracle.count_by_distance(d, 5e5, 1.0, n_q, q0, n_k, inv_freq=theta)
        assert a == b == c


# ---------------------------------------------------------------------------------------
# Composition with token-level block sparsity: key blocks listed per query block


def _random_lists(B, H, nblk, maxb, seed):
    """Block lists with the quirks the rule must absorb: unsorted, duplicates, entries
    above the query block or negative, the query block itself listed or not, counts above
    max_blocks."""
    rng = np.random.default_rng(seed)
    count = rng.integers(0, maxb + 3, (B, H, nblk)).astype(np.int32)
    idx = rng.integers(-2, nblk + 2, (B, H, nblk, maxb)).astype(np.int32)
    return count, idx


def _visible(N, blk, count, idx):
    """[B][H][N][N] boolean, written from the rule: c <= r and (c//blk == r//blk or c//blk
    among the first count entries of r//blk's list)."""
    B, H, nblk = count.shape
    vis = np.zeros((B, H, N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            for r in range(N):
                R = r // blk
                listed = set(int(x) for x in idx[b, h, R, :min(int(count[b, h, R]), idx.shape[3])])
                for c in range(r + 1):
                    vis[b, h, r, c] = (c // blk == R) or (c // blk in listed)
    return vis


@pytest.mark.parametrize("alpha", [0.5, 1.0, math.inf])
def test_block_sparse_equals_relative_form_with_mask(alpha):
    B, N, Hq, Hkv, d, base, blk = 2, 45, 4, 2, 16, 100.0, 8
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "fp32", seed=81)
    nblk = (N + blk - 1) // blk
    count, idx = _random_lists(B, Hq, nblk, 4, seed=82)
    out, lse, kept = oracle.prefill_sparse(synth.to_oracle(q), synth.to_oracle(k),
                                           synth.to_oracle(v), base, alpha, count, idx, blk=blk)
    vis = _visible(N, blk, count, idx)
    pos = np.arange(N)
    G = Hq // Hkv
    P = d // 2
    lam = 2.0 * np.pi * np.power(base, np.arange(P) * 2.0 / d)
    tally = 0
    for b in range(B):
        for h in range(Hq):
            ro, rl = _relative_form(_f64(q[b, :, h]), _f64(k[b, :, h // G]), _f64(v[b, :, h // G]),
                                    pos, pos, base, alpha, 1.0 / math.sqrt(d), visible=vis[b, h])
            np.testing.assert_allclose(out[b, :, h], ro, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], rl, rtol=0, atol=1e-12)
            dist = pos[:, None] - pos[None, :]
            tally += int(((np.abs(dist)[..., None] <= alpha * lam) & vis[b, h][..., None]).sum())
    assert kept == tally


@pytest.mark.parametrize("positions", ["gapped", "nonmonotone"])
def test_block_sparse_with_positions_equals_relative_form_with_mask(positions):
    """Blocks by token index, rotation and window at explicit positions: each head against
    the complex relative form at those positions with the block mask, and a brute-force
    tally of the kept terms."""
    B, N, Hq, Hkv, d, base, blk, alpha = 1, 45, 2, 1, 16, 100.0, 8, 1.0
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "fp32", seed=87)
    rng = np.random.default_rng(88)
    if positions == "gapped":
        pos = np.cumsum(rng.integers(1, 9, N)) + 3
    else:
        pos = rng.integers(0, 200, N)
    nblk = (N + blk - 1) // blk
    count, idx = _random_lists(B, Hq, nblk, 4, seed=89)
    out, lse, kept = oracle.prefill_sparse(synth.to_oracle(q), synth.to_oracle(k),
                                           synth.to_oracle(v), base, alpha, count, idx, blk=blk,
                                           pos=pos[None])
    vis = _visible(N, blk, count, idx)
    lam = 2.0 * np.pi * np.power(base, np.arange(d // 2) * 2.0 / d)
    tally = 0
    for h in range(Hq):
        ro, rl = _relative_form(_f64(q[0, :, h]), _f64(k[0, :, 0]), _f64(v[0, :, 0]), pos, pos,
                                base, alpha, 1.0 / math.sqrt(d), visible=vis[0, h])
        np.testing.assert_allclose(out[0, :, h], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], rl, rtol=0, atol=1e-12)
        dist = pos[:, None] - pos[None, :]
        tally += int(((np.abs(dist)[..., None] <= alpha * lam) & vis[0, h][..., None]
                      & np.tri(N, dtype=bool)[..., None]).sum())
    assert kept == tally


def test_block_sparse_with_positions_and_every_block_is_the_dense_prefill():
    """Listing every block at explicit positions is the plain prefill at those positions,
    bit for bit (and differs from the same call at token indices)."""
    B, N, Hq, Hkv, d, base, blk = 2, 70, 2, 1, 32, 1e4, 16
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=90)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    pos = np.cumsum(np.random.default_rng(91).integers(1, 40, (B, N)), axis=1).astype(np.int32)
    nblk = (N + blk - 1) // blk
    count = np.full((B, Hq, nblk), nblk, np.int32)
    idx = np.broadcast_to(np.arange(nblk, dtype=np.int32), (B, Hq, nblk, nblk)).copy()
    o1, l1, k1 = oracle.prefill(*a, base, 1.0, pos=pos)
    o2, l2, k2 = oracle.prefill_sparse(*a, base, 1.0, count, idx, blk=blk, pos=pos)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and k1 == k2
    o3, _, k3 = oracle.prefill_sparse(*a, base, 1.0, count, idx, blk=blk)
    assert not np.array_equal(o1, o3) and k3 != k1


def test_block_sparse_with_every_block_is_dense():
    """Listing every block is the plain causal prefill, bit for bit."""
    B, N, Hq, Hkv, d, base, blk = 1, 70, 3, 1, 32, 1e4, 16
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=83)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    nblk = (N + blk - 1) // blk
    count = np.full((B, Hq, nblk), nblk, np.int32)
    idx = np.broadcast_to(np.arange(nblk, dtype=np.int32), (B, Hq, nblk, nblk)).copy()
    o1, l1, k1 = oracle.prefill(*a, base, 1.0)
    o2, l2, k2 = oracle.prefill_sparse(*a, base, 1.0, count, idx, blk=blk)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and k1 == k2


def _expand_lists(count, idx, f, N, fine):
    """Lists over blocks of f*fine tokens as lists over blocks of `fine`: each listed coarse
    block becomes its f fine blocks, and each fine query block also lists the earlier fine
    blocks of its own coarse block."""
    B, H, nc = count.shape
    nf = (N + fine - 1) // fine
    cf = np.zeros((B, H, nf), np.int32)
    rows = [[[[] for _ in range(nf)] for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for Rf in range(nf):
                R = Rf // f
                got = [int(x) for x in idx[b, h, R, :max(0, min(int(count[b, h, R]), idx.shape[3]))]]
                lst = [c * f + j for c in got if 0 <= c < R for j in range(f)]
                lst += list(range(R * f, Rf))
                rows[b][h][Rf] = lst
                cf[b, h, Rf] = len(lst)
    m = max(1, int(cf.max()))
    xf = np.zeros((B, H, nf, m), np.int32)
    for b in range(B):
        for h in range(H):
            for Rf in range(nf):
                xf[b, h, Rf, :cf[b, h, Rf]] = rows[b][h][Rf]
    return cf, xf


@pytest.mark.parametrize("f", [2, 4])
def test_block_sparse_coarse_blocks_equal_expanded_fine_lists(f):
    """A list over blocks of f*8 tokens is the same attention as the list of their 8-token
    blocks (plus the earlier 8-token blocks of the row's own coarse block), bit for bit."""
    B, N, Hq, Hkv, d, base, fine = 1, 77, 2, 1, 16, 100.0, 8
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=85)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    nc = (N + f * fine - 1) // (f * fine)
    count, idx = _random_lists(B, Hq, nc, 3, seed=86)
    cf, xf = _expand_lists(count, idx, f, N, fine)
    o1, l1, k1 = oracle.prefill_sparse(*a, base, 1.0, count, idx, blk=f * fine)
    o2, l2, k2 = oracle.prefill_sparse(*a, base, 1.0, cf, xf, blk=fine)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and k1 == k2
    # dropping one coarse block's expansion changes the result (the pin sees the lists)
    R = next(R for R in range(nc) for e in range(min(int(count[0, 0, R]), 3))
             if 0 <= idx[0, 0, R, e] < R)
    cf2 = cf.copy()
    cf2[0, 0, R * f:(R + 1) * f] = 0
    o4, _, _ = oracle.prefill_sparse(*a, base, 1.0, cf2, xf, blk=fine)
    assert not np.array_equal(o1, o4)


def test_block_sparse_empty_lists_are_block_local():
    """With no listed blocks every row sees only its own block: the same rows as a plain
    prefill of that block alone (positions shifted, which RoPE attention does not see)."""
    N, d, base, blk = 48, 16, 1e4, 16
    q, k, v = synth.prefill_inputs(1, N, 1, 1, d, "fp32", seed=84)
    count = np.zeros((1, 1, N // blk), np.int32)
    idx = np.zeros((1, 1, N // blk, 1), np.int32)
    out, _, _ = oracle.prefill_sparse(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                      base, 1.0, count, idx, blk=blk)
    for R in range(N // blk):
        sl = slice(R * blk, (R + 1) * blk)
        ref, _, _ = oracle.prefill(synth.to_oracle(q[:, sl]), synth.to_oracle(k[:, sl]),
                                   synth.to_oracle(v[:, sl]), base, 1.0)
        np.testing.assert_allclose(out[:, sl], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------
# Per-head frequency tables (AdaRoPE abstract, on the cards page: each head gets its own
# rotation frequencies).  One row per kv head; its q heads use the same row.  Pins: the
# relative complex form per head, the shared-table oracle when all rows are equal, and the
# count as a sum of single-table enumerations.

def _head_tables(Hkv, d, seed):
    rng = np.random.default_rng(seed)
    rows = [np.sort(rng.uniform(0.01, 1.5, d // 2))[::-1] for _ in range(Hkv)]
    return np.ascontiguousarray(np.stack(rows))


@pytest.mark.parametrize("alpha", [0.5, 1.0, math.inf])
@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_per_head_tables_equal_relative_form(alpha, layout):
    N, Hq, Hkv, d = 37, 6, 2, 16
    q, k, v = synth.prefill_inputs(1, N, Hq, Hkv, d, "fp32", seed=41)
    pos = np.cumsum(np.random.default_rng(8).integers(0, 4, N))
    tabs = _head_tables(Hkv, d, 9)
    out, lse, kept = oracle.prefill(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                    1e4, alpha, pos=pos, inv_freq=tabs, layout=layout)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        ro, rl = _relative_form_table(_f64(q[0, :, h]), _f64(k[0, :, g]), _f64(v[0, :, g]), pos,
                                      pos, tabs[g], layout, alpha, 1.0 / math.sqrt(d))
        np.testing.assert_allclose(out[0, :, h], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], rl, rtol=0, atol=1e-12)


def test_per_head_tables_all_equal_is_shared_table():
    B, N, Hq, Hkv, d = 2, 45, 4, 2, 32
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=42)
    theta = _llama3_table(d, 5e5)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    shared = oracle.prefill(*a, 5e5, 1.0, inv_freq=theta)
    heads = oracle.prefill(*a, 5e5, 1.0, inv_freq=np.stack([theta, theta]))
    np.testing.assert_array_equal(shared[0], heads[0])
    np.testing.assert_array_equal(shared[1], heads[1])
    assert shared[2] == heads[2]


@pytest.mark.parametrize("alpha", [0.5, 1.0, math.inf])
def test_block_sparse_per_head_tables_equal_relative_form_with_mask(alpha):
    """Block sparsity with one frequency row per kv head: each q head against the relative
    complex form with its kv head's row and the list mask written from the rule; the kept
    count as a tally over visible pairs with each head's windows."""
    B, N, Hq, Hkv, d, blk = 2, 45, 4, 2, 16, 8
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "fp32", seed=91)
    tabs = _head_tables(Hkv, d, 92)
    nblk = (N + blk - 1) // blk
    count, idx = _random_lists(B, Hq, nblk, 4, seed=93)
    out, lse, kept = oracle.prefill_sparse(synth.to_oracle(q), synth.to_oracle(k),
                                           synth.to_oracle(v), 1e4, alpha, count, idx, blk=blk,
                                           inv_freq=tabs)
    vis = _visible(N, blk, count, idx)
    pos = np.arange(N)
    G = Hq // Hkv
    tally = 0
    for b in range(B):
        for h in range(Hq):
            g = h // G
            ro, rl = _relative_form_table(_f64(q[b, :, h]), _f64(k[b, :, g]), _f64(v[b, :, g]), pos,
                                          pos, tabs[g], "half", alpha, 1.0 / math.sqrt(d),
                                          visible=vis[b, h])
            np.testing.assert_allclose(out[b, :, h], ro, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], rl, rtol=0, atol=1e-12)
            dist = pos[:, None] - pos[None, :]
            lam = 2.0 * np.pi / tabs[g]
            tally += int(((np.abs(dist)[..., None] <= alpha * lam) & vis[b, h][..., None]).sum())
    assert kept == tally


def test_block_sparse_per_head_tables_every_block_is_dense():
    """With every block listed, per-head block sparsity is the per-head causal prefill, bit for
    bit; with all rows equal it is the shared-table block sparsity, bit for bit."""
    B, N, Hq, Hkv, d, blk = 1, 70, 4, 2, 32, 16
    q, k, v = synth.prefill_inputs(B, N, Hq, Hkv, d, "bf16", seed=94)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    tabs = _head_tables(Hkv, d, 95)
    nblk = (N + blk - 1) // blk
    count = np.full((B, Hq, nblk), nblk, np.int32)
    idx = np.broadcast_to(np.arange(nblk, dtype=np.int32), (B, Hq, nblk, nblk)).copy()
    o1, l1, k1 = oracle.prefill(*a, 1e4, 1.0, inv_freq=tabs)
    o2, l2, k2 = oracle.prefill_sparse(*a, 1e4, 1.0, count, idx, blk=blk, inv_freq=tabs)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and k1 == k2
    c2, i2 = _random_lists(B, Hq, nblk, 3, seed=96)
    eq = np.stack([tabs[0], tabs[0]])
    s1 = oracle.prefill_sparse(*a, 1e4, 1.0, c2, i2, blk=blk, inv_freq=tabs[0])
    s2 = oracle.prefill_sparse(*a, 1e4, 1.0, c2, i2, blk=blk, inv_freq=eq)
    assert np.array_equal(s1[0], s2[0]) and np.array_equal(s1[1], s2[1]) and s1[2] == s2[2]


def test_per_head_tables_count_and_decode():
    """Kept terms: the sum over kv heads of (q heads per kv head) x that row's enumeration.
    Decode with per-head rows equals the last prefill row."""
    N, Hq, Hkv, d = 50, 6, 3, 16
    tabs = _head_tables(Hkv, d, 10)
    q, k, v = synth.prefill_inputs(1, N, Hq, Hkv, d, "fp32", seed=43)
    a = [synth.to_oracle(t) for t in (q, k, v)]
    _, _, kept = oracle.prefill(*a, 1e4, 1.0, inv_freq=tabs)
    G = Hq // Hkv
    assert kept == sum(G * oracle.count_enumerate(d, 1e4, 1.0, N, 0, N, inv_freq=tabs[g])[0]
                       for g in range(Hkv))
    po, pl, _ = oracle.prefill(*a, 1e4, 1.0, inv_freq=tabs, rows=[N - 1])
    do, dl, _ = oracle.decode(synth.to_oracle(q[:, N - 1]), a[1], a[2], np.array([N]), 1e4, 1.0,
                              inv_freq=tabs)
    np.testing.assert_allclose(do, po[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dl, pl[:, :, 0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------
# Backward (WavePrune, What the paper found: training with the window).  Pins: torch
# autograd, in fp64 on the CPU, through the relative complex form (no rotation of q or k, no
# back-rotation: an independent route to the pre-RoPE gradients), and central finite
# differences of the pinned forward.

def _torch_relative_loss(q, k, v, dout, pos, theta, alpha, scale, layout="half"):
    """sum(out * dout) of windowed attention written with the relative form of each pair's
    term, q [N][Hq][d], k, v [N][Hkv][d] (torch fp64, requires_grad on q, k, v)."""
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dx, dy = _dims(d, layout)
    th = torch.as_tensor(theta, dtype=torch.float64)
    tpos = torch.as_tensor(np.asarray(pos), dtype=torch.float64)
    dt = tpos[:, None] - tpos[None, :]
    keep = (dt.abs()[..., None] <= alpha * (2.0 * math.pi / th)).to(torch.float64)
    rot = torch.exp(1j * dt[..., None] * th)
    causal = torch.arange(N)[None, :] <= torch.arange(N)[:, None]
    loss = 0.0
    for h in range(Hq):
        g = h // G
        zq = torch.complex(q[:, h, dx], q[:, h, dy])
        zk = torch.complex(k[:, g, dx], k[:, g, dy])
        terms = torch.real(zq[:, None, :] * torch.conj(zk[None, :, :]) * rot)
        logits = scale * (terms * keep).sum(-1)
        logits = logits.masked_fill(~causal, float("-inf"))
        out = torch.softmax(logits, dim=-1) @ v[:, g]
        loss = loss + (out * dout[:, h]).sum()
    return loss


@pytest.mark.parametrize("alpha", [0.5, 1.0, 2.0, math.inf])
@pytest.mark.parametrize("positions", ["default", "gapped"])
def test_backward_equals_autograd_of_relative_form(alpha, positions):
    N, Hq, Hkv, d, base = 33, 4, 2, 16, 100.0
    q, k, v = synth.prefill_inputs(1, N, Hq, Hkv, d, "fp32", seed=71)
    g = torch.randn((1, N, Hq, d), generator=torch.Generator().manual_seed(72))
    pos = np.arange(N) if positions == "default" else \
        np.cumsum(np.random.default_rng(11).integers(0, 7, N))
    dq, dk, dv = oracle.prefill_backward(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                         synth.to_oracle(g), base, alpha, pos=pos)
    theta = base ** (-np.arange(d // 2) * 2.0 / d)
    tq, tk, tv = (torch.from_numpy(_f64(t[0])).requires_grad_() for t in (q, k, v))
    loss = _torch_relative_loss(tq, tk, tv, torch.from_numpy(_f64(g[0])), pos, theta, alpha,
                                1.0 / math.sqrt(d))
    loss.backward()
    np.testing.assert_allclose(dq[0], tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk[0], tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv[0], tv.grad.numpy(), rtol=0, atol=1e-11)


def test_backward_equals_autograd_per_head_tables_interleaved():
    N, Hq, Hkv, d = 25, 4, 2, 16
    q, k, v = synth.prefill_inputs(1, N, Hq, Hkv, d, "fp32", seed=73)
    g = torch.randn((1, N, Hq, d), generator=torch.Generator().manual_seed(74))
    tabs = _head_tables(Hkv, d, 12)
    pos = np.arange(N)
    dq, dk, dv = oracle.prefill_backward(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                         synth.to_oracle(g), 1e4, 1.0, inv_freq=tabs,
                                         layout="interleaved")
    G = Hq // Hkv
    for gg in range(Hkv):
        hs = slice(gg * G, (gg + 1) * G)
        tq = torch.from_numpy(_f64(q[0, :, hs])).requires_grad_()
        tk = torch.from_numpy(_f64(k[0, :, gg:gg + 1])).requires_grad_()
        tv = torch.from_numpy(_f64(v[0, :, gg:gg + 1])).requires_grad_()
        loss = _torch_relative_loss(tq, tk, tv, torch.from_numpy(_f64(g[0, :, hs])), pos, tabs[gg],
                                    1.0, 1.0 / math.sqrt(d), layout="interleaved")
        loss.backward()
        np.testing.assert_allclose(dq[0, :, hs], tq.grad.numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk[0, :, gg:gg + 1], tk.grad.numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv[0, :, gg:gg + 1], tv.grad.numpy(), rtol=0, atol=1e-11)


def test_backward_equals_finite_differences_of_forward():
    """Central differences of sum(out * dout) through the (pinned) forward, on fp32 inputs: the
    step applied is the exact fp32 difference, so the quotient is accurate to O(eps^2)."""
    N, Hq, Hkv, d, base, alpha = 14, 2, 1, 8, 30.0, 1.0
    q, k, v = synth.prefill_inputs(1, N, Hq, Hkv, d, "fp32", seed=75)
    g = torch.randn((1, N, Hq, d), generator=torch.Generator().manual_seed(76))
    ga = synth.to_oracle(g).astype(np.float64)
    dq, dk, dv = oracle.prefill_backward(synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v),
                                         synth.to_oracle(g), base, alpha)
    arrs = [synth.to_oracle(t).copy() for t in (q, k, v)]

    def loss(a):
        out, _, _ = oracle.prefill(*a, base, alpha)
        return float((out * ga).sum())

    rng = np.random.default_rng(13)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arrs[which].shape)
            x0 = arrs[which][idx]
            hi, lo = np.float32(x0 + 1e-2), np.float32(x0 - 1e-2)
            arrs[which][idx] = hi
            lp = loss(arrs)
            arrs[which][idx] = lo
            lm = loss(arrs)
            arrs[which][idx] = x0
            fd = (lp - lm) / (float(hi) - float(lo))
            assert abs(fd - grad[idx]) <= 2e-5 * max(1.0, abs(grad[idx])), (which, idx, fd, grad[idx])


def test_backward_row_and_key_subsets_equal_full():
    N, Hq, Hkv, d = 40, 6, 2, 32
    q, k, v = synth.prefill_inputs(2, N, Hq, Hkv, d, "bf16", seed=77)
    g = synth.prefill_inputs(2, N, Hq, Hkv, d, "bf16", seed=78)[0]
    a = [synth.to_oracle(t) for t in (q, k, v, g)]
    full = oracle.prefill_backward(*a, 1e4, 1.0)
    rows, keys = np.array([0, 7, 39]), np.array([3, 38, 39])
    part = oracle.prefill_backward(*a, 1e4, 1.0, rows=rows, keys=keys)
    np.testing.assert_array_equal(part[0], full[0][:, rows])
    np.testing.assert_array_equal(part[1], full[1][:, keys])
    np.testing.assert_array_equal(part[2], full[2][:, keys])

"""fp64 CPU oracle for per-RoPE-wavelength windowed causal attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``; never by the product package.  It shares no code
with the HIP library (its C part is ``wpa_oracle.c``; the counting helpers below are
numpy).

Method (ATFlash abstract, "Per-RoPE-Wavelength Attention Windows"): the RoPE score is
an exact sum over frequency pairs; pair i (wavelength lambda_i = 2*pi*base^(2i/d), one
rotation period: WavePrune original abstract) keeps its q.k term only while
the query-key distance is <= alpha*lambda_i.  Online softmax and P.V are unchanged.

Parity status of each function (what pins it is listed in the design notes and in
``tests/test_oracle_pins.py``):
  prefill / prefill_rows / decode -- pinned (full-window library SDPA, complex relative
      form, alpha=0 closed form, hand-derived two-token cases, shift invariance, GQA);
      with a frequency table or the interleaved layout: full-window SDPA on complex-rotated
      inputs, the complex relative form with the table, and the layout permutation identity
  count_enumerate / count_bruteforce / count_by_distance -- pinned against each other
      (three independent enumerations) and against closed-form asymptotics.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wpa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16 = 0
FP32 = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile wpa_oracle.c with gcc (OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-D_GNU_SOURCE", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.orc_prefill_ex.argtypes = [P, P, P, I, P, I, I64, I, I, I, D, P, I, I, D, D, P, I64, P,
                                       P, P, I]
        lib.orc_prefill_ex.restype = I
        lib.orc_prefill_sparse.argtypes = [P, P, P, I, P, I, I64, I, I, I, D, P, I, I, D, D, P, P, I, I,
                                           P, I64, P, P, P, I]
        lib.orc_prefill_sparse.restype = I
        lib.orc_prefill_backward_ex.argtypes = [P, P, P, P, I, P, I, I64, I, I, I, D, P, I, I, D, D,
                                                P, I64, P, I64, P, P, P, I]
        lib.orc_prefill_backward_ex.restype = I
        lib.orc_decode_ex.argtypes = [P, P, P, I, P, P, I, I64, I, I, I, D, P, I, I, D, D, P, P, P,
                                      I]
        lib.orc_decode_ex.restype = I
        lib.orc_rope_ex.argtypes = [P, I, I64, I, I, P, D, P, I, P]
        lib.orc_rope_ex.restype = None
        lib.orc_thresholds_ex.argtypes = [I, D, P, D, P]
        lib.orc_thresholds_ex.restype = None
        lib.orc_count_enumerate_ex.argtypes = [I, D, P, D, I64, I64, I64, P, P]
        lib.orc_count_enumerate_ex.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x):
    """Accept float32 arrays (fp32) or uint16 arrays holding bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, FP32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle inputs are float32 or uint16 (bf16 bits), got %s" % x.dtype)


LAYOUTS = {"half": 0, "interleaved": 1}


def _freq(inv_freq, d):
    """Optional per-pair rotation frequencies th_i (a d/2 float64 table), else None."""
    if inv_freq is None:
        return None
    f = np.ascontiguousarray(inv_freq, dtype=np.float64)
    assert f.shape == (d // 2,)
    return f


def _freq_heads(inv_freq, d, Hkv):
    """(table, number of tables): None; one shared d/2 table; or one row per kv head,
    [Hkv][d/2] (per-head frequencies)."""
    if inv_freq is None:
        return None, 0
    f = np.ascontiguousarray(inv_freq, dtype=np.float64)
    if f.ndim == 1:
        assert f.shape == (d // 2,)
        return f, 1
    assert f.shape == (Hkv, d // 2), f.shape
    return f, Hkv


def thresholds(d: int, base: float, alpha: float, inv_freq=None) -> np.ndarray:
    """alpha*lambda_i for i < d/2, in double (may be +inf); lambda_i = 2*pi*base^(2i/d), or
    2*pi/th_i for a given frequency table."""
    out = np.empty(d // 2, dtype=np.float64)
    _load().orc_thresholds_ex(d, float(base), _ptr(_freq(inv_freq, d)), float(alpha), _ptr(out))
    return out


def rope(x, pos, base: float, inv_freq=None, layout: str = "half") -> np.ndarray:
    """Rotate x [T][H][d] (fp32 or bf16 bits) at positions pos[T]; returns fp64."""
    x, dt = _as_input(x)
    T, H, d = x.shape
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    out = np.empty((T, H, d), dtype=np.float64)
    _load().orc_rope_ex(_ptr(x), dt, T, H, d, _ptr(pos), float(base), _ptr(_freq(inv_freq, d)),
                        LAYOUTS[layout], _ptr(out))
    return out


def prefill(q, k, v, base: float, alpha: float, scale: float | None = None, pos=None,
            rows=None, nthreads: int = 0, inv_freq=None, layout: str = "half"):
    """Causal windowed prefill.  q [B][N][Hq][d], k/v [B][N][Hkv][d] (same dtype).
    inv_freq: optional d/2 rotation frequencies (else base^(-2i/d)), or [Hkv][d/2], one row
    per kv head (its q heads use the same row); layout: "half" (pair i = dims i, i+d/2) or
    "interleaved" (dims 2i, 2i+1).

    Returns (out [B][R][Hq][d], lse [B][Hq][R], kept) in fp64, R = len(rows) or N.
    """
    q, dt = _as_input(q)
    k, dk = _as_input(k)
    v, dv = _as_input(v)
    assert dt == dk == dv
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if pos is not None:
        pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(B, N)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        R = rows.shape[0]
    else:
        R = N
    out = np.empty((B, R, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)
    kept = ctypes.c_int64(0)
    tab, ntab = _freq_heads(inv_freq, d, Hkv)
    rc = _load().orc_prefill_ex(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(pos), B, N, Hq, Hkv, d,
                                float(base), _ptr(tab), ntab, LAYOUTS[layout],
                                float(alpha), float(scale), _ptr(rows), R,
                                _ptr(out), _ptr(lse), ctypes.byref(kept), int(nthreads))
    if rc != 0:
        raise ValueError("orc_prefill rejected its arguments")
    return out, lse, kept.value


def prefill_backward(q, k, v, dout, base: float, alpha: float, scale: float | None = None,
                     pos=None, rows=None, keys=None, nthreads: int = 0, inv_freq=None,
                     layout: str = "half"):
    """Gradients of the windowed causal prefill for dout = dL/dout [B][N][Hq][d] (same dtype as
    q, k, v): dq at query rows `rows`, dk and dv at key rows `keys` (None: all).  Returns
    (dq [B][R][Hq][d], dk [B][K][Hkv][d], dv [B][K][Hkv][d]) in fp64, with respect to the
    pre-RoPE q and k."""
    q, dt = _as_input(q)
    k, dk_ = _as_input(k)
    v, dv_ = _as_input(v)
    g, dg = _as_input(dout)
    assert dt == dk_ == dv_ == dg
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    assert g.shape == q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if pos is not None:
        pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(B, N)
    R, K = N, N
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        R = rows.shape[0]
    if keys is not None:
        keys = np.ascontiguousarray(keys, dtype=np.int64)
        K = keys.shape[0]
    dq = np.empty((B, R, Hq, d), dtype=np.float64)
    dk = np.empty((B, K, Hkv, d), dtype=np.float64)
    dv = np.empty((B, K, Hkv, d), dtype=np.float64)
    tab, ntab = _freq_heads(inv_freq, d, Hkv)
    rc = _load().orc_prefill_backward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), dt, _ptr(pos), B, N,
                                         Hq, Hkv, d, float(base), _ptr(tab), ntab, LAYOUTS[layout],
                                         float(alpha), float(scale), _ptr(rows), R, _ptr(keys), K,
                                         _ptr(dq), _ptr(dk), _ptr(dv), int(nthreads))
    if rc != 0:
        raise ValueError("orc_prefill_backward rejected its arguments")
    return dq, dk, dv


def prefill_sparse(q, k, v, base: float, alpha: float, count, idx, blk: int = 64,
                   scale: float | None = None, rows=None, nthreads: int = 0, inv_freq=None,
                   layout: str = "half", pos=None):
    """Causal windowed prefill restricted to listed key blocks: with R = r // blk, row r of
    head h attends key c <= r iff c // blk == R or c // blk is among the first
    count[b][h][R] entries of idx[b][h][R]; other keys leave the softmax.  Blocks are by
    token index; pos ([B][N] int, default token indices) are the RoPE positions, as in
    prefill().  count int32 [B][Hq][nblk], idx int32 [B][Hq][nblk][max_blocks].
    Returns (out [B][R][Hq][d], lse [B][Hq][R], kept) in fp64 like prefill()."""
    q, dt = _as_input(q)
    k, dk = _as_input(k)
    v, dv = _as_input(v)
    assert dt == dk == dv
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    nblk = (N + blk - 1) // blk
    count = np.ascontiguousarray(count, dtype=np.int32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    assert count.shape == (B, Hq, nblk) and idx.shape[:3] == (B, Hq, nblk)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        R = rows.shape[0]
    else:
        R = N
    out = np.empty((B, R, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)
    kept = ctypes.c_int64(0)
    tabs, ntab = _freq_heads(inv_freq, d, Hkv)
    if pos is not None:
        pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(B, N)
    rc = _load().orc_prefill_sparse(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(pos), B, N, Hq, Hkv, d,
                                    float(base),
                                    _ptr(tabs), ntab, LAYOUTS[layout], float(alpha),
                                    float(scale), _ptr(count), _ptr(idx), idx.shape[3], blk,
                                    _ptr(rows), R, _ptr(out), _ptr(lse), ctypes.byref(kept),
                                    int(nthreads))
    if rc != 0:
        raise ValueError("orc_prefill_sparse rejected its arguments")
    return out, lse, kept.value


def decode(q, k, v, kv_len, base: float, alpha: float, scale: float | None = None,
           q_pos=None, nthreads: int = 0, inv_freq=None, layout: str = "half"):
    """One decode step.  q [B][Hq][d]; k/v pre-RoPE cache [B][Lmax][Hkv][d]; kv_len [B];
    inv_freq and layout as for prefill."""
    q, dt = _as_input(q)
    k, _ = _as_input(k)
    v, _ = _as_input(v)
    B, Hq, d = q.shape
    Lmax, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kv_len = np.ascontiguousarray(kv_len, dtype=np.int32)
    if q_pos is not None:
        q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    out = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    kept = ctypes.c_int64(0)
    tab, ntab = _freq_heads(inv_freq, d, Hkv)
    rc = _load().orc_decode_ex(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(kv_len), _ptr(q_pos), B, Lmax,
                               Hq, Hkv, d, float(base), _ptr(tab), ntab, LAYOUTS[layout],
                               float(alpha), float(scale), _ptr(out), _ptr(lse),
                               ctypes.byref(kept), int(nthreads))
    if rc != 0:
        raise ValueError("orc_decode rejected its arguments")
    return out, lse, kept.value


# --------------------------------------------------------------------------------------
# Kept-term counts.  A "term" is one frequency pair's contribution to one (query, key)
# score.  Queries sit at token indices q0..q0+n_q-1, keys at 0..n_k-1, positions equal
# indices, key c visible to query r iff c <= r.  Three independent enumerations.
# --------------------------------------------------------------------------------------

def count_enumerate(d, base, alpha, n_q, q0, n_k, inv_freq=None):
    """C loop over every (r, c, i).  Returns (kept, total)."""
    kept, total = ctypes.c_int64(0), ctypes.c_int64(0)
    _load().orc_count_enumerate_ex(int(d), float(base), _ptr(_freq(inv_freq, d)), float(alpha),
                                   int(n_q), int(q0), int(n_k), ctypes.byref(kept),
                                   ctypes.byref(total))
    return kept.value, total.value


def count_bruteforce(d, base, alpha, n_q, q0, n_k, inv_freq=None):
    """numpy: materialise the (r, c) distance matrix and test every pair.  O(n_q*n_k*d/2)."""
    thr = thresholds(d, base, alpha, inv_freq)
    r = np.arange(q0, q0 + n_q, dtype=np.int64)[:, None]
    c = np.arange(n_k, dtype=np.int64)[None, :]
    visible = c <= r
    dist = (r - c).astype(np.float64)
    kept = 0
    for t in thr:
        kept += int(np.count_nonzero(visible & (dist <= t)))
    return kept, int(np.count_nonzero(visible)) * (d // 2)


def count_by_distance(d, base, alpha, n_q, q0, n_k, inv_freq=None):
    """numpy: histogram of distances.  For each distance D, the number of visible (r, c)
    with r - c = D is the size of r in [max(q0, D), min(q0+n_q-1, n_k-1+D)].
    O((q0+n_q) * d/2), exact in int64."""
    thr = thresholds(d, base, alpha, inv_freq)
    D = np.arange(0, q0 + n_q, dtype=np.int64)
    lo = np.maximum(q0, D)
    hi = np.minimum(q0 + n_q - 1, n_k - 1 + D)
    mult = np.maximum(hi - lo + 1, 0)
    kept = 0
    Df = D.astype(np.float64)
    for t in thr:
        kept += int(mult[Df <= t].sum())
    return kept, int(mult.sum()) * (d // 2)

"""Per-RoPE-wavelength windowed causal attention on MI355X (gfx950).

Thin ctypes binding over ``libwpa.so`` (C ABI in ``include/wpa.h``).  This module only
marshals arguments: it checks the shape, dtype, device and contiguity of every tensor it
is given (inputs and caller-supplied out, lse, workspace, counters, positions), allocates
outputs and workspace with torch when the caller does not pass them, and forwards raw
device pointers and the current HIP stream.  Every step of the computation runs in the HIP
kernels behind the C ABI; there is no CPU or PyTorch fallback.  If the library is not
built, every entry point raises.

Method (ATFlash abstract, "Per-RoPE-Wavelength Attention Windows"; WavePrune original
abstract): pair i of the half-split head vector, with wavelength 2*pi*base^(2i/d),
contributes its q.k term only while the query-key distance is <= alpha*wavelength;
alpha = 1 is the first rotation period, alpha = inf is full causal RoPE attention.

RoPE variants: every op takes ``inv_freq`` (the d/2 per-pair rotation frequencies of a
frequency-scaled RoPE, e.g. ``llama3_inv_freq(...)``; wavelength 2*pi/theta_i) and
``pairs`` ("half": dims i, i+d/2; "interleaved": dims 2i, 2i+1).
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwpa.so")

WPA_OK, WPA_ERR_INVALID, WPA_ERR_UNSUPPORTED, WPA_ERR_WORKSPACE, WPA_ERR_HIP = 0, -1, -2, -3, -4
WPA_BF16, WPA_FP32 = 0, 1

WPA_PAIRS = {"half": 0, "interleaved": 1}

# every symbol include/wpa.h declares
EXPORTS = ("wpa_count_terms", "wpa_thresholds", "wpa_prefill_workspace_bytes", "wpa_prefill",
           "wpa_prefill_prepare", "wpa_prefill_attend", "wpa_kcache_bytes", "wpa_vcache_bytes",
           "wpa_kv_write", "wpa_decode_workspace_bytes", "wpa_decode", "wpa_count_terms_ex",
           "wpa_thresholds_ex", "wpa_prefill_ex", "wpa_prefill_prepare_ex", "wpa_prefill_attend_ex",
           "wpa_kv_write_ex", "wpa_decode_ex", "wpa_prefill_cached", "wpa_kcache_window_bytes",
           "wpa_kv_write_window", "wpa_decode_window", "wpa_prefill_sparse", "wpa_kv_page_bytes",
           "wpa_kv_write_paged", "wpa_decode_paged", "wpa_prefill_paged",
           "wpa_prefill_cached_varlen", "wpa_prefill_paged_varlen", "wpa_decode_noalloc",
           "wpa_prefill_backward_workspace_bytes", "wpa_prefill_backward",
           "wpa_prefill_cached_workspace_bytes", "wpa_prefill_cached_ex", "wpa_set_debug",
           "wpa_last_error", "wpa_prefill_sparse_ex", "wpa_prefill_sparse_pos")


class Rope(ctypes.Structure):
    """wpa_rope_t: pair layout, optional host table of rotation frequencies, optional device
    tables of one row per kv head."""
    _fields_ = [("pairs", ctypes.c_int32), ("inv_freq", ctypes.c_void_p),
                ("head_inv_freq", ctypes.c_void_p)]


def _ndim(x):
    return x.dim() if isinstance(x, torch.Tensor) else np.ndim(x)


def head_table(tab, d: int, Hkv: int, device):
    """Per-kv-head rotation frequencies [Hkv][d/2] as a float64 tensor on `device`, checked on
    the host (each row finite, > 0 and non-increasing, as the kernels require)."""
    t = torch.as_tensor(tab, dtype=torch.float64)
    host = t.detach().cpu().numpy()
    if host.shape != (Hkv, d // 2):
        raise ValueError("per-head frequency tables must be [Hkv][d/2] = [%d][%d], got %s"
                         % (Hkv, d // 2, host.shape))
    if not (np.all(np.isfinite(host)) and np.all(host > 0) and np.all(np.diff(host, axis=1) <= 0)):
        raise ValueError("each per-head frequency row must be finite, > 0 and non-increasing")
    return t.to(device).contiguous()


def _rope(d, inv_freq, pairs, Hkv=None, device=None):
    """(pointer to a wpa_rope_t or None, objects that must outlive the call).  inv_freq: None,
    d/2 shared frequencies, or [Hkv][d/2] per-kv-head rows (uploaded to `device`)."""
    if inv_freq is None and pairs == "half":
        return None, ()
    if pairs not in WPA_PAIRS:
        raise ValueError("pairs must be 'half' or 'interleaved'")
    tab, heads = None, None
    if inv_freq is not None and _ndim(inv_freq) == 2:
        if Hkv is None or device is None:
            raise ValueError("per-head frequency tables are not taken here")
        heads = head_table(inv_freq, d, Hkv, device)
    elif inv_freq is not None:
        tab = np.ascontiguousarray(np.asarray(inv_freq, dtype=np.float64))
        if tab.shape != (d // 2,):
            raise ValueError("inv_freq must hold d/2 = %d frequencies" % (d // 2))
    r = Rope(WPA_PAIRS[pairs], None if tab is None else tab.ctypes.data,
             None if heads is None else heads.data_ptr())
    return ctypes.byref(r), (r, tab, heads)


def default_inv_freq(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d), i < d/2 (float64)."""
    return np.power(float(base), -np.arange(d // 2, dtype=np.float64) * 2.0 / d)


def llama3_inv_freq(d: int, base: float, factor: float, low_freq_factor: float,
                    high_freq_factor: float, original_max_position: int) -> np.ndarray:
    """Rotation frequencies of Llama-3-style frequency-scaled RoPE (float64): pairs whose
    wavelength is shorter than original_max_position/high_freq_factor keep theta_i, pairs
    longer than original_max_position/low_freq_factor are slowed by `factor`, and the band
    in between blends the two linearly in original_max_position/wavelength.  The result is
    non-increasing in i, as the kernels require."""
    theta = default_inv_freq(d, base)
    wavelen = 2.0 * math.pi / theta
    ratio = original_max_position / wavelen                    # periods within the old context
    blend = np.clip((ratio - low_freq_factor) / (high_freq_factor - low_freq_factor), 0.0, 1.0)
    return theta * (blend + (1.0 - blend) / factor)


class WpaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("wpa error %d: %s" % (code, msg))
        self.code = code


_lib = None


def lib():
    """Load libwpa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libwpa.so is not built: run `python -m rope_wavelength_sparsity_amd.build` "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, D, F, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                             ctypes.c_float, ctypes.c_size_t)
    L.wpa_count_terms.argtypes = [I32, D, D, I64, I64, I64, P, P]
    L.wpa_count_terms.restype = ctypes.c_int
    L.wpa_thresholds.argtypes = [I32, D, D, P]
    L.wpa_thresholds.restype = ctypes.c_int
    L.wpa_prefill_workspace_bytes.argtypes = [I32, I64, I32, I32]
    L.wpa_prefill_workspace_bytes.restype = SZ
    L.wpa_prefill.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, I32, D, D, F, I32, I32, P, P, SZ,
                              P]
    L.wpa_prefill.restype = ctypes.c_int
    L.wpa_prefill_prepare.argtypes = [P, P, P, I32, I64, I32, I32, D, I32, P, SZ, P]
    L.wpa_prefill_prepare.restype = ctypes.c_int
    L.wpa_prefill_attend.argtypes = [P, P, P, P, I32, I64, I32, I32, I32, D, D, F, I32, I32, P, P,
                                     SZ, P]
    L.wpa_prefill_attend.restype = ctypes.c_int
    L.wpa_kcache_bytes.argtypes = [I32, I64, I32, I32]
    L.wpa_kcache_bytes.restype = SZ
    L.wpa_vcache_bytes.argtypes = [I32, I64, I32, I32]
    L.wpa_vcache_bytes.restype = SZ
    L.wpa_kv_write.argtypes = [P, P, I64, I64, P, P, I32, I64, I32, I32, D, I32, P]
    L.wpa_kv_write.restype = ctypes.c_int
    L.wpa_decode_workspace_bytes.argtypes = [I32, I64, I32, I32, I32, I32]
    L.wpa_decode_workspace_bytes.restype = SZ
    L.wpa_decode.argtypes = [P, P, P, P, P, P, P, I32, I64, I32, I32, I32, D, D, F, I32, I32, P,
                             I32, P, SZ, P]
    L.wpa_decode.restype = ctypes.c_int
    L.wpa_count_terms_ex.argtypes = [I32, D, P, D, I64, I64, I64, P, P]
    L.wpa_count_terms_ex.restype = ctypes.c_int
    L.wpa_thresholds_ex.argtypes = [I32, D, P, D, P]
    L.wpa_thresholds_ex.restype = ctypes.c_int
    L.wpa_prefill_ex.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, I32, D, P, D, F, I32, I32, P,
                                 P, SZ, P]
    L.wpa_prefill_ex.restype = ctypes.c_int
    L.wpa_prefill_prepare_ex.argtypes = [P, P, P, I32, I64, I32, I32, D, P, I32, P, SZ, P]
    L.wpa_prefill_prepare_ex.restype = ctypes.c_int
    L.wpa_prefill_attend_ex.argtypes = [P, P, P, P, I32, I64, I32, I32, I32, D, P, D, F, I32, I32, P,
                                        P, SZ, P]
    L.wpa_prefill_attend_ex.restype = ctypes.c_int
    L.wpa_kv_write_ex.argtypes = [P, P, I64, I64, P, P, I32, I64, I32, I32, D, P, I32, P]
    L.wpa_kv_write_ex.restype = ctypes.c_int
    L.wpa_decode_ex.argtypes = [P, P, P, P, P, P, P, I32, I64, I32, I32, I32, D, P, D, F, I32, I32,
                                P, I32, P, SZ, P]
    L.wpa_decode_ex.restype = ctypes.c_int
    L.wpa_prefill_cached.argtypes = [P, P, P, P, P, P, I32, I32, I64, I32, I32, I32, D, P, D, F,
                                     I32, I32, P, P]
    L.wpa_prefill_cached.restype = ctypes.c_int
    L.wpa_kcache_window_bytes.argtypes = [I32, I64, I32, I32, D, P, D]
    L.wpa_kcache_window_bytes.restype = SZ
    L.wpa_kv_write_window.argtypes = [P, P, I64, I64, P, P, I32, I64, I32, I32, D, P, D, I32, P]
    L.wpa_kv_write_window.restype = ctypes.c_int
    L.wpa_decode_window.argtypes = [P, P, P, P, P, P, I32, I64, I32, I32, I32, D, P, D, D, F, I32,
                                    I32, P, I32, P, SZ, P]
    L.wpa_decode_window.restype = ctypes.c_int
    L.wpa_prefill_sparse.argtypes = [P, P, P, P, P, P, P, I32, I32, I64, I32, I32, I32, D, P, D, F,
                                     I32, I32, P, P, SZ, P]
    L.wpa_prefill_sparse.restype = ctypes.c_int
    L.wpa_prefill_sparse_ex.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I64, I32, I32, I32, D,
                                        P, D, F, I32, I32, P, P, SZ, P]
    L.wpa_prefill_sparse_ex.restype = ctypes.c_int
    L.wpa_prefill_sparse_pos.argtypes = [P, P, P, P, P, P, P, I32, I32, P, I32, I64, I32, I32, I32,
                                         D, P, D, F, I32, I32, P, P, ctypes.c_size_t, P]
    L.wpa_prefill_sparse_pos.restype = ctypes.c_int
    L.wpa_kv_page_bytes.argtypes = [I32, I32, I32]
    L.wpa_kv_page_bytes.restype = SZ
    L.wpa_kv_write_paged.argtypes = [P, P, I64, I64, P, P, P, I32, I32, I32, I32, I32, I32, D, P,
                                     I32, P]
    L.wpa_kv_write_paged.restype = ctypes.c_int
    L.wpa_decode_paged.argtypes = [P, P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, I32, D, P,
                                   D, F, I32, I32, P, I32, P, SZ, P]
    L.wpa_decode_paged.restype = ctypes.c_int
    L.wpa_prefill_paged.argtypes = [P, P, P, P, I32, P, P, P, I32, I32, I32, I32, I32, I32, I32, D,
                                    P, D, F, I32, I32, P, P]
    L.wpa_prefill_paged.restype = ctypes.c_int
    L.wpa_prefill_cached_varlen.argtypes = [P, P, P, P, P, P, P, I32, I32, I64, I32, I32, I32, D,
                                            P, D, F, I32, I32, P, P]
    L.wpa_prefill_cached_varlen.restype = ctypes.c_int
    L.wpa_prefill_paged_varlen.argtypes = [P, P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32,
                                           I32, I32, D, P, D, F, I32, I32, P, P]
    L.wpa_prefill_paged_varlen.restype = ctypes.c_int
    L.wpa_decode_noalloc.argtypes = [P, P, P, P, P, P, P, I32, I64, I32, I32, I32, D, P, D, F, I32,
                                     I32, P, I32, P]
    L.wpa_decode_noalloc.restype = ctypes.c_int
    L.wpa_prefill_backward_workspace_bytes.argtypes = [I32, I64, I32, I32, I32]
    L.wpa_prefill_backward_workspace_bytes.restype = SZ
    L.wpa_prefill_backward.argtypes = [P, P, P, P, P, P, P, P, P, I32, I64, I32, I32, I32, D, P, D, F,
                                       I32, I32, I32, P, SZ, P]
    L.wpa_prefill_backward.restype = ctypes.c_int
    L.wpa_prefill_cached_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    L.wpa_prefill_cached_workspace_bytes.restype = SZ
    L.wpa_prefill_cached_ex.argtypes = [P, P, P, P, I32, I32, P, P, P, P, I32, I32, I64, I32, I32,
                                        I32, D, P, D, F, I32, I32, P, I32, P, SZ, P]
    L.wpa_prefill_cached_ex.restype = ctypes.c_int
    L.wpa_set_debug.argtypes = [I32]
    L.wpa_set_debug.restype = ctypes.c_int
    L.wpa_last_error.argtypes = []
    L.wpa_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int):
    if rc != WPA_OK:
        raise WpaError(rc, lib().wpa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return WPA_BF16
    if t.dtype == torch.float32:
        return WPA_FP32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _dev(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % name)


def _same_device(t, ref, name):
    if t.device != ref.device:
        raise ValueError("%s is on %s, the inputs on %s" % (name, t.device, ref.device))


def _out(out, shape, ref, out_dtype):
    """The output buffer: given (checked: shape, dtype, device, contiguity) or allocated."""
    if out is None:
        return torch.empty(tuple(shape), device=ref.device, dtype=out_dtype or ref.dtype)
    _dev(out, "out")
    _same_device(out, ref, "out")
    if tuple(out.shape) != tuple(shape):
        raise ValueError("out must be %s, got %s" % (tuple(shape), tuple(out.shape)))
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be bfloat16 or float32")
    return out


def _lse(lse, want, shape, ref):
    """The lse buffer: None, allocated when wanted, or a checked float32 [shape] tensor."""
    if lse is None:
        return torch.empty(tuple(shape), device=ref.device, dtype=torch.float32) if want else None
    _dev(lse, "lse")
    _same_device(lse, ref, "lse")
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape):
        raise ValueError("lse must be float32 %s" % (tuple(shape),))
    return lse


def _workspace(ws, need, ref):
    """The workspace: given (a contiguous device buffer on the inputs' device, at least
    `need` bytes; the library re-checks the size) or allocated."""
    if ws is None:
        return torch.empty(max(need, 16), device=ref.device, dtype=torch.uint8)
    _dev(ws, "workspace")
    _same_device(ws, ref, "workspace")
    return ws


def _ws_bytes(ws):
    return ws.numel() * ws.element_size()


def _counter(term_count, ref):
    if term_count is None:
        return None
    _dev(term_count, "term_count")
    _same_device(term_count, ref, "term_count")
    if term_count.dtype != torch.int64 or term_count.numel() < 1:
        raise ValueError("term_count must be an int64 device tensor of at least one element")
    return term_count


def _int32_vec(t, n, ref, name):
    if t is None:
        return None
    _dev(t, name)
    _same_device(t, ref, name)
    if t.dtype != torch.int32 or t.numel() != n:
        raise ValueError("%s must be int32 with %d elements" % (name, n))
    return t


# ------------------------------------------------------------------------------ host-only

def count_terms(d: int, base: float, alpha: float, n_q: int, q_pos0: int, n_k: int, *,
                inv_freq=None, pairs: str = "half"):
    """(kept, total) (query, key, pair) terms per head; exact closed form, host only."""
    kept, total = ctypes.c_int64(), ctypes.c_int64()
    rope, keep = _rope(d, inv_freq, pairs)
    _check(lib().wpa_count_terms_ex(d, float(base), rope, float(alpha), n_q, q_pos0, n_k,
                                    ctypes.byref(kept), ctypes.byref(total)))
    return kept.value, total.value


def count_terms_heads(d: int, alpha: float, n_q: int, q_pos0: int, n_k: int, head_inv_freq,
                      q_per_kv: int):
    """(kept, total) terms summed over the q heads of one sequence with per-kv-head frequency
    rows [Hkv][d/2]: each row counted by the closed form and weighted by its q heads."""
    kept = total = 0
    for row in np.asarray(torch.as_tensor(head_inv_freq, dtype=torch.float64).cpu()):
        k, t = count_terms(d, 2.0, alpha, n_q, q_pos0, n_k, inv_freq=row)
        kept += q_per_kv * k
        total += q_per_kv * t
    return kept, total


def thresholds(d: int, base: float, alpha: float, *, inv_freq=None, pairs: str = "half"):
    """Integer window table W_i = floor(alpha * lambda_i) (INT32_MAX if unbounded), with
    lambda_i = 2*pi*base^(2i/d) or 2*pi/inv_freq[i]."""
    W = (ctypes.c_int32 * (d // 2))()
    rope, keep = _rope(d, inv_freq, pairs)
    _check(lib().wpa_thresholds_ex(d, float(base), rope, float(alpha), W))
    return list(W)


def prefill_workspace_bytes(B, N, Hkv, d) -> int:
    return lib().wpa_prefill_workspace_bytes(B, N, Hkv, d)


def kcache_bytes(B, Lmax, Hkv, d) -> int:
    return lib().wpa_kcache_bytes(B, Lmax, Hkv, d)


def vcache_bytes(B, Lmax, Hkv, d) -> int:
    return lib().wpa_vcache_bytes(B, Lmax, Hkv, d)


def decode_workspace_bytes(B, Lmax, Hq, Hkv, d, chunk_keys=0) -> int:
    return lib().wpa_decode_workspace_bytes(B, Lmax, Hq, Hkv, d, chunk_keys)


# ------------------------------------------------------------------------------ device ops

def prefill(q, k, v, base: float, alpha: float, *, scale: float | None = None, positions=None,
            out=None, out_dtype=None, lse=None, want_lse: bool = False, term_count=None,
            workspace=None, stream=None, inv_freq=None, pairs: str = "half", block_count=None,
            block_idx=None, block: int = 64):
    """Causal windowed prefill.  q [B][N][Hq][d], k/v [B][N][Hkv][d] (bf16 or fp32, pre-RoPE).

    block_count / block_idx (int32 device [B][Hq][ceil(N/block)] and [...][max]): token-level
    block sparsity on top of the window; each query block of `block` rows (a power of two,
    64 .. 1024) attends its own block and the key blocks listed for it.  Blocks are by token
    index; with positions, the rotation and the window use the positions.

    Returns out [B][N][Hq][d] (out_dtype, default q's dtype), or (out, lse [B][Hq][N] fp32)
    when want_lse or an lse buffer is passed.  term_count: optional int64 device tensor of
    one element to which the kept-term count is added.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if q.dim() != 4 or k.shape != v.shape or k.dim() != 4:
        raise ValueError("q [B][N][Hq][d], k, v [B][N][Hkv][d] expected")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape[0] != B or k.shape[1] != N or k.shape[3] != d or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v shapes/dtypes disagree")
    _same_device(k, q, "k")
    _same_device(v, q, "v")
    out = _out(out, q.shape, q, out_dtype)
    lse = _lse(lse, want_lse, (B, Hq, N), q)
    positions = _int32_vec(positions, B * N, q, "positions")
    term_count = _counter(term_count, q)
    workspace = _workspace(workspace, prefill_workspace_bytes(B, N, Hkv, d), q)
    rope, keep = _rope(d, inv_freq, pairs, Hkv, q.device)
    if block_count is not None:
        # token-level block sparsity on top of the window (blocks of `block` tokens)
        block = int(block)
        if block < 64 or block > 1024 or block & (block - 1):
            raise ValueError("block must be a power of two from 64 to 1024")
        nblk = (N + block - 1) // block
        for t, n in ((block_count, "block_count"), (block_idx, "block_idx")):
            _dev(t, n)
            if t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError("%s must be a contiguous int32 device tensor" % n)
        if tuple(block_count.shape) != (B, Hq, nblk) or block_idx.dim() != 4 \
                or tuple(block_idx.shape[:3]) != (B, Hq, nblk):
            raise ValueError("block_count [B][Hq][ceil(N/block)], block_idx [B][Hq][ceil(N/block)][max]")
        if positions is not None:
            # blocks by token index; rotation and window at the positions
            _check(lib().wpa_prefill_sparse_pos(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                                _ptr(block_count), _ptr(block_idx),
                                                block_idx.shape[3], block, _ptr(positions), B, N,
                                                Hq, Hkv, d, float(base), rope, float(alpha),
                                                float(scale) if scale is not None else 0.0,
                                                _dtype_code(q), _dtype_code(out), _ptr(term_count),
                                                _ptr(workspace), _ws_bytes(workspace),
                                                _stream(stream)))
            return (out, lse) if lse is not None else out
        _check(lib().wpa_prefill_sparse_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                           _ptr(block_count), _ptr(block_idx), block_idx.shape[3],
                                           block, B, N, Hq, Hkv, d, float(base), rope,
                                           float(alpha), float(scale) if scale is not None else 0.0,
                                           _dtype_code(q), _dtype_code(out), _ptr(term_count),
                                           _ptr(workspace), _ws_bytes(workspace), _stream(stream)))
        return (out, lse) if lse is not None else out
    _check(lib().wpa_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(positions),
                                B, N, Hq, Hkv, d, float(base), rope, float(alpha),
                                float(scale) if scale is not None else 0.0, _dtype_code(q),
                                _dtype_code(out), _ptr(term_count), _ptr(workspace),
                                _ws_bytes(workspace), _stream(stream)))
    return (out, lse) if lse is not None else out


def prefill_backward_workspace_bytes(B, N, Hq, Hkv, d) -> int:
    return lib().wpa_prefill_backward_workspace_bytes(B, N, Hq, Hkv, d)


def prefill_backward(q, k, v, out, lse, dout, base: float, alpha: float, *, scale=None,
                     grad_dtype=None, dq=None, dk=None, dv=None, workspace=None, stream=None,
                     inv_freq=None, pairs: str = "half"):
    """Gradients (dq, dk, dv) of the windowed causal prefill with respect to the pre-RoPE q, k
    and v, for dout = dL/dout.  q, k, v, dout bf16 ([B][N][Hq|Hkv][d]); out and lse are the
    forward's (prefill(..., want_lse=True)); positions are token indices.  grad_dtype:
    torch.float32 (default) or torch.bfloat16."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"), (lse, "lse")):
        _dev(t, n)
        _same_device(t, q, n)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q [B][N][Hq][d], k, v [B][N][Hkv][d] expected")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError("q, k, v shapes disagree")
    if not (q.dtype == k.dtype == v.dtype == dout.dtype == torch.bfloat16):
        raise ValueError("the backward takes bf16 q, k, v and dout")
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("out and dout must be shaped like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be float32 [B][Hq][N]")
    gdt = grad_dtype or torch.float32
    dq = _out(dq, q.shape, q, gdt)
    dk = _out(dk, k.shape, q, gdt)
    dv = _out(dv, v.shape, q, gdt)
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise ValueError("dq, dk, dv must share one dtype")
    workspace = _workspace(workspace, prefill_backward_workspace_bytes(B, N, Hq, Hkv, d), q)
    rope, keep = _rope(d, inv_freq, pairs, Hkv, q.device)
    _check(lib().wpa_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                      _ptr(dq), _ptr(dk), _ptr(dv), B, N, Hq, Hkv, d, float(base),
                                      rope, float(alpha), float(scale) if scale is not None else 0.0,
                                      WPA_BF16, _dtype_code(out), _dtype_code(dq), _ptr(workspace),
                                      _ws_bytes(workspace), _stream(stream)))
    return dq, dk, dv


def prefill_prepare(k, v, base: float, *, positions=None, workspace=None, stream=None,
                    inv_freq=None, pairs: str = "half"):
    """First half of prefill: rotate k, transpose v into a workspace (returned)."""
    _dev(k, "k")
    _dev(v, "v")
    if k.dim() != 4 or k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k, v must be [B][N][Hkv][d] of one dtype")
    B, N, Hkv, d = k.shape
    _same_device(v, k, "v")
    positions = _int32_vec(positions, B * N, k, "positions")
    workspace = _workspace(workspace, prefill_workspace_bytes(B, N, Hkv, d), k)
    rope, keep = _rope(d, inv_freq, pairs, Hkv, k.device)
    _check(lib().wpa_prefill_prepare_ex(_ptr(k), _ptr(v), _ptr(positions), B, N, Hkv, d,
                                        float(base), rope, _dtype_code(k), _ptr(workspace),
                                        _ws_bytes(workspace), _stream(stream)))
    return workspace


def prefill_attend(q, workspace, Hkv: int, base: float, alpha: float, *, scale=None,
                   positions=None, out=None, out_dtype=None, lse=None, want_lse=False,
                   term_count=None, stream=None, inv_freq=None, pairs: str = "half"):
    """Second half of prefill: windowed attention of q against a prepared workspace."""
    _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B][N][Hq][d]")
    _dev(workspace, "workspace")
    _same_device(workspace, q, "workspace")
    B, N, Hq, d = q.shape
    out = _out(out, q.shape, q, out_dtype)
    lse = _lse(lse, want_lse, (B, Hq, N), q)
    positions = _int32_vec(positions, B * N, q, "positions")
    term_count = _counter(term_count, q)
    rope, keep = _rope(d, inv_freq, pairs, Hkv, q.device)
    _check(lib().wpa_prefill_attend_ex(_ptr(q), _ptr(out), _ptr(lse), _ptr(positions), B, N, Hq,
                                       Hkv, d, float(base), rope, float(alpha),
                                       float(scale) if scale is not None else 0.0, _dtype_code(q),
                                       _dtype_code(out), _ptr(term_count), _ptr(workspace),
                                       _ws_bytes(workspace), _stream(stream)))
    return (out, lse) if lse is not None else out


def _own_table(inv_freq, d, Hkv, device):
    """A cache's copy of its frequency description: None, a host d/2 table, or the per-kv-head
    rows as a checked float64 device tensor."""
    if inv_freq is None:
        return None
    if _ndim(inv_freq) == 2:
        return head_table(inv_freq, d, Hkv, device)
    return np.asarray(inv_freq, dtype=np.float64).copy()


class KVCache:
    """Decode caches for B sequences of up to Lmax tokens (library-owned K layout).  The
    RoPE description (inv_freq, pairs) given here rotates the keys written and the queries
    of every decode step against this cache.

    window_alpha: build the windowed K cache, which keeps each 16-dim pair block only for the
    keys still inside that block's window at this alpha (decodes then take alpha <=
    window_alpha, with the query at the newest token)."""

    def __init__(self, B, Lmax, Hkv, d, base, device="cuda", *, inv_freq=None, pairs="half",
                 window_alpha=None):
        self.B, self.Lmax, self.Hkv, self.d, self.base = B, Lmax, Hkv, d, float(base)
        self.inv_freq = _own_table(inv_freq, d, Hkv, device)
        self.pairs = pairs
        self._rope = _rope(d, self.inv_freq, pairs, Hkv, device)   # validates the description
        rope = self._rope[0]
        self.window_alpha = None if window_alpha is None else float(window_alpha)
        if self.window_alpha is None:
            self.k_seq_bytes = kcache_bytes(1, Lmax, Hkv, d)
        else:
            self.k_seq_bytes = lib().wpa_kcache_window_bytes(1, Lmax, Hkv, d, self.base, rope,
                                                             self.window_alpha)
            if self.k_seq_bytes == 0:
                raise ValueError("invalid windowed cache arguments")
        self.k = torch.empty(B * self.k_seq_bytes, device=device, dtype=torch.uint8)
        self.v = torch.empty(vcache_bytes(B, Lmax, Hkv, d), device=device, dtype=torch.uint8)

    def write(self, k, v, start: int, stream=None, *, seq: int | None = None):
        """Append pre-RoPE k, v [B][n][Hkv][d] at token indices start .. start+n-1; with
        `seq`, k and v are [1][n][Hkv][d] and go to sequence `seq` alone (ragged batches)."""
        _dev(k, "k")
        _dev(v, "v")
        nb = self.B if seq is None else 1
        if k.shape != v.shape or k.dim() != 4 or k.shape[0] != nb or k.shape[2] != self.Hkv \
                or k.shape[3] != self.d or k.dtype != v.dtype:
            raise ValueError("k, v must be [%d][n][Hkv][d] of one dtype" % nb)
        kc, vc = self.k.data_ptr(), self.v.data_ptr()
        if seq is not None:
            if not 0 <= seq < self.B:
                raise ValueError("seq out of range")
            kc += seq * self.k_seq_bytes
            vc += seq * vcache_bytes(1, self.Lmax, self.Hkv, self.d)
        rope = self._rope[0]
        if self.window_alpha is None:
            _check(lib().wpa_kv_write_ex(_ptr(k), _ptr(v), int(start), k.shape[1], kc, vc, nb,
                                         self.Lmax, self.Hkv, self.d, self.base, rope,
                                         _dtype_code(k), _stream(stream)))
        else:
            _check(lib().wpa_kv_write_window(_ptr(k), _ptr(v), int(start), k.shape[1], kc, vc, nb,
                                             self.Lmax, self.Hkv, self.d, self.base, rope,
                                             self.window_alpha, _dtype_code(k), _stream(stream)))

    def v_tokens(self):
        """A copy of the V cache as bf16 [B][Hkv][Lmax][d] (the cache itself is blocked by
        8 consecutive tokens: [B][Hkv][ceil(Lmax/8)][d][8])."""
        L8 = (self.Lmax + 7) // 8
        v = self.v.view(torch.bfloat16).view(self.B, self.Hkv, L8, self.d, 8)
        return v.permute(0, 1, 2, 4, 3).reshape(self.B, self.Hkv, L8 * 8, self.d)[:, :, :self.Lmax]


class PagedKVCache:
    """Decode caches as a pool of `num_pages` pages of `page_size` tokens (all Hkv kv heads of
    a page together); a block table int32 device [B][max_pages] maps token range
    [i*page_size, (i+1)*page_size) of sequence b to page table[b][i].  The table is the
    caller's: `block_table` here is only a convenience default (set it or pass one per call)."""

    def __init__(self, num_pages, page_size, Hkv, d, base, device="cuda", *, inv_freq=None,
                 pairs="half", block_table=None):
        self.num_pages, self.page_size, self.Hkv, self.d = num_pages, page_size, Hkv, d
        self.base = float(base)
        self.inv_freq = _own_table(inv_freq, d, Hkv, device)
        self.pairs = pairs
        self._rope = _rope(d, self.inv_freq, pairs, Hkv, device)   # validates the description
        self.page_bytes = lib().wpa_kv_page_bytes(Hkv, d, page_size)
        if self.page_bytes == 0:
            raise ValueError("invalid page arguments (d 64 or 128, page_size a power of two >= 32)")
        self.k = torch.empty(num_pages * self.page_bytes, device=device, dtype=torch.uint8)
        self.v = torch.empty(num_pages * self.page_bytes, device=device, dtype=torch.uint8)
        self.window_alpha = None
        self.block_table = block_table

    def _table(self, block_table):
        t = self.block_table if block_table is None else block_table
        if t is None:
            raise ValueError("no block table")
        _dev(t, "block_table")
        if t.dtype != torch.int32 or t.dim() != 2 or not t.is_contiguous():
            raise ValueError("block_table must be a contiguous int32 [B][max_pages] tensor")
        return t

    def write(self, k, v, start: int, block_table=None, stream=None):
        """Append pre-RoPE k, v [B][n][Hkv][d] at token indices start .. start+n-1 of the B
        sequences whose block-table rows are given (one sequence: its row, as [1][max_pages])."""
        _dev(k, "k")
        _dev(v, "v")
        t = self._table(block_table)
        if k.shape != v.shape or k.dim() != 4 or k.shape[0] != t.shape[0] or \
                k.shape[2] != self.Hkv or k.shape[3] != self.d or k.dtype != v.dtype:
            raise ValueError("k, v must be [B][n][Hkv][d] of one dtype, B = block_table rows")
        rope = self._rope[0]
        _check(lib().wpa_kv_write_paged(_ptr(k), _ptr(v), int(start), k.shape[1], _ptr(self.k),
                                        _ptr(self.v), _ptr(t), self.num_pages, t.shape[0],
                                        t.shape[1], self.page_size, self.Hkv, self.d, self.base,
                                        rope, _dtype_code(k), _stream(stream)))


def decode(q, cache, kv_len, alpha: float, *, q_pos=None, scale: float | None = None,
           out=None, out_dtype=None, lse=None, want_lse: bool = False, term_count=None,
           chunk_keys: int = 0, workspace=None, stream=None, block_table=None):
    """One decode step.  q [B][Hq][d] pre-RoPE; kv_len int32 device [B]; `cache` a KVCache or
    a PagedKVCache (with `block_table` [B][max_pages], or the cache's default table)."""
    _dev(q, "q")
    _dev(kv_len, "kv_len")
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][d]")
    B, Hq, d = q.shape
    paged = isinstance(cache, PagedKVCache)
    if paged:
        table = cache._table(block_table)
        nseq, lmax = table.shape[0], table.shape[1] * cache.page_size
    else:
        nseq, lmax = cache.B, cache.Lmax
    if B != nseq or d != cache.d or kv_len.dtype != torch.int32 or kv_len.numel() != B:
        raise ValueError("q [B][Hq][d] and kv_len int32 [B] must match the cache")
    _same_device(kv_len, q, "kv_len")
    _same_device(cache.k, q, "the cache")
    q_pos = _int32_vec(q_pos, B, q, "q_pos")
    out = _out(out, q.shape, q, out_dtype)
    lse = _lse(lse, want_lse, (B, Hq), q)
    term_count = _counter(term_count, q)
    workspace = _workspace(workspace, decode_workspace_bytes(B, lmax, Hq, cache.Hkv, d, chunk_keys), q)
    rope = cache._rope[0]
    if paged:
        _check(lib().wpa_decode_paged(_ptr(q), _ptr(cache.k), _ptr(cache.v), _ptr(table),
                                      cache.num_pages, _ptr(kv_len), _ptr(q_pos), _ptr(out),
                                      _ptr(lse), B, table.shape[1], cache.page_size, Hq,
                                      cache.Hkv, d, cache.base, rope, float(alpha),
                                      float(scale) if scale is not None else 0.0,
                                      _dtype_code(q), _dtype_code(out), _ptr(term_count),
                                      int(chunk_keys), _ptr(workspace), _ws_bytes(workspace),
                                      _stream(stream)))
        return (out, lse) if lse is not None else out
    if cache.window_alpha is not None:
        if q_pos is not None:
            raise ValueError("a windowed cache decodes at the newest token (q_pos must be None)")
        _check(lib().wpa_decode_window(_ptr(q), _ptr(cache.k), _ptr(cache.v), _ptr(kv_len),
                                       _ptr(out), _ptr(lse), B, cache.Lmax, Hq, cache.Hkv, d,
                                       cache.base, rope, cache.window_alpha, float(alpha),
                                       float(scale) if scale is not None else 0.0,
                                       _dtype_code(q), _dtype_code(out), _ptr(term_count),
                                       int(chunk_keys), _ptr(workspace), _ws_bytes(workspace),
                                       _stream(stream)))
        return (out, lse) if lse is not None else out
    _check(lib().wpa_decode_ex(_ptr(q), _ptr(cache.k), _ptr(cache.v), _ptr(kv_len), _ptr(q_pos),
                               _ptr(out), _ptr(lse), B, cache.Lmax, Hq, cache.Hkv, d, cache.base,
                               rope, float(alpha), float(scale) if scale is not None else 0.0,
                               _dtype_code(q), _dtype_code(out), _ptr(term_count),
                               int(chunk_keys), _ptr(workspace), _ws_bytes(workspace),
                               _stream(stream)))
    return (out, lse) if lse is not None else out


def decode_noalloc(q, cache, kv_len, alpha: float, *, out, q_pos=None, scale: float | None = None,
                   lse=None, term_count=None, chunk_keys: int = 0, stream=None):
    """decode() on a dense KVCache through the entry point that allocates nothing: the split-KV
    partials live in the library's per-GPU scratch array (16 MiB).  `out` (and `lse`, if
    wanted) must be given; calls that may overlap on one GPU race on the scratch array."""
    _dev(q, "q")
    _dev(kv_len, "kv_len")
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][d]")
    B, Hq, d = q.shape
    if isinstance(cache, PagedKVCache) or cache.window_alpha is not None:
        raise ValueError("decode_noalloc takes a dense KVCache")
    if B != cache.B or d != cache.d or kv_len.dtype != torch.int32 or kv_len.numel() != B:
        raise ValueError("q [B][Hq][d] and kv_len int32 [B] must match the cache")
    _same_device(kv_len, q, "kv_len")
    _same_device(cache.k, q, "the cache")
    if out is None:
        raise ValueError("decode_noalloc needs a caller-supplied out")
    out = _out(out, q.shape, q, None)
    lse = _lse(lse, False, (B, Hq), q)
    q_pos = _int32_vec(q_pos, B, q, "q_pos")
    term_count = _counter(term_count, q)
    rope = cache._rope[0]
    _check(lib().wpa_decode_noalloc(_ptr(q), _ptr(cache.k), _ptr(cache.v), _ptr(kv_len), _ptr(q_pos),
                                    _ptr(out), _ptr(lse), B, cache.Lmax, Hq, cache.Hkv, d,
                                    cache.base, rope, float(alpha),
                                    float(scale) if scale is not None else 0.0, _dtype_code(q),
                                    _dtype_code(out), _ptr(term_count), int(chunk_keys),
                                    _stream(stream)))
    return (out, lse) if lse is not None else out


def set_debug(on) -> bool:
    """Switch the library's debug mode (buffer-extent and device-value checks, a wait after
    every launch); None only reports it.  Returns the previous state."""
    return bool(lib().wpa_set_debug(-1 if on is None else int(bool(on))))


def prefill_cached_workspace_bytes(B: int, Nq: int, Hq: int, Hkv: int, d: int,
                                   splits: int = 0) -> int:
    """Workspace bytes of a chunked prefill with `splits` key splits (0: the launch's own
    choice on the current device); 0 when no split is taken."""
    return int(lib().wpa_prefill_cached_workspace_bytes(int(B), int(Nq), int(Hq), int(Hkv), int(d),
                                                        int(splits)))


def prefill_cached(q, cache, kv_len, alpha: float, *, scale: float | None = None,
                   out=None, out_dtype=None, lse=None, want_lse: bool = False, term_count=None,
                   stream=None, block_table=None, cu_q=None, max_q: int | None = None,
                   splits: int = 0, workspace=None):
    """Chunked prefill: q [B][Nq][Hq][d] pre-RoPE holds the last Nq tokens of each sequence,
    whose keys and values are already in `cache` (a KVCache, or a PagedKVCache with
    `block_table` [B][max_pages] or the cache's default table; per-kv-head frequency tables
    as the cache was made with);
    kv_len int32 device [B], each >= Nq.
    Varlen: with cu_q (int32 device [B+1]) q is [rows][Hq][d], sequence b's chunk being rows
    cu_q[b] .. cu_q[b+1]-1 (its last tokens), max_q an upper bound of the per-sequence counts;
    lse is then [rows][Hq].
    splits: key splits of each row block's key tiles (0: chosen by the launch, 1: none, 2..16:
    that many); their partials live in `workspace` (uint8 device tensor, at least
    prefill_cached_workspace_bytes(...) long), allocated here when not given."""
    if cu_q is not None:
        return _prefill_varlen(q, cache, kv_len, alpha, cu_q, max_q, scale, out, out_dtype, lse,
                               want_lse, term_count, stream, block_table, splits, workspace)
    _dev(q, "q")
    _dev(kv_len, "kv_len")
    if q.dim() != 4:
        raise ValueError("q must be [B][Nq][Hq][d]")
    B, Nq, Hq, d = q.shape
    paged = isinstance(cache, PagedKVCache)
    if paged:
        table = cache._table(block_table)
        nseq = table.shape[0]
    else:
        nseq = cache.B
    if B != nseq or d != cache.d or kv_len.dtype != torch.int32 or kv_len.numel() != B:
        raise ValueError("q [B][Nq][Hq][d] and kv_len int32 [B] must match the cache")
    if cache.window_alpha is not None:
        raise ValueError("chunked prefill needs the dense cache (window_alpha=None)")
    _same_device(kv_len, q, "kv_len")
    _same_device(cache.k, q, "the cache")
    out = _out(out, q.shape, q, out_dtype)
    lse = _lse(lse, want_lse, (B, Hq, Nq), q)
    term_count = _counter(term_count, q)
    _cached_ex(q, cache, table if paged else None, None, kv_len, out, lse, B, Nq, Hq, d, alpha,
               scale, term_count, splits, workspace, stream)
    return (out, lse) if lse is not None else out


def _cached_ex(q, cache, table, cu_q, kv_len, out, lse, B, Nq, Hq, d, alpha, scale, term_count,
               splits, workspace, stream):
    """wpa_prefill_cached_ex on a dense or paged cache (table), fixed or varlen (cu_q)."""
    splits = int(splits)
    if not 0 <= splits <= 16:
        raise ValueError("splits must be in [0, 16]")
    need = prefill_cached_workspace_bytes(B, Nq, Hq, cache.Hkv, d, splits) if splits != 1 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device) if need else None
    else:
        _dev(workspace, "workspace")
        _same_device(workspace, q, "workspace")
        if splits > 1 and workspace.numel() * workspace.element_size() < need:
            raise ValueError("workspace needs %d bytes for %d splits" % (need, splits))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if table is not None:
        nt, Lmax, ps = cache.num_pages, table.shape[1] * cache.page_size, cache.page_size
    else:
        nt, Lmax, ps = 0, cache.Lmax, 0
    sc = float(scale) if scale is not None else 0.0
    if splits == 1:
        # no key splits: the four plain entry points
        args = (_ptr(out), _ptr(lse), B, Nq)
        tail = (Hq, cache.Hkv, d, cache.base, cache._rope[0], float(alpha), sc, _dtype_code(q),
                _dtype_code(out), _ptr(term_count), _stream(stream))
        kv = (_ptr(cu_q), _ptr(kv_len)) if cu_q is not None else (_ptr(kv_len),)
        fn = {(False, False): lib().wpa_prefill_cached, (False, True): lib().wpa_prefill_cached_varlen,
              (True, False): lib().wpa_prefill_paged, (True, True): lib().wpa_prefill_paged_varlen}
        f = fn[(table is not None, cu_q is not None)]
        if table is not None:
            _check(f(_ptr(q), _ptr(cache.k), _ptr(cache.v), _ptr(table), nt, *kv, *args,
                     table.shape[1], ps, *tail))
        else:
            _check(f(_ptr(q), _ptr(cache.k), _ptr(cache.v), *kv, *args, Lmax, *tail))
        return
    _check(lib().wpa_prefill_cached_ex(_ptr(q), _ptr(cache.k), _ptr(cache.v), _ptr(table), nt, ps,
                                       _ptr(cu_q), _ptr(kv_len), _ptr(out), _ptr(lse), B, Nq, Lmax,
                                       Hq, cache.Hkv, d, cache.base, cache._rope[0], float(alpha),
                                       sc, _dtype_code(q), _dtype_code(out), _ptr(term_count),
                                       splits, _ptr(workspace), ws_bytes, _stream(stream)))


def _prefill_varlen(q, cache, kv_len, alpha, cu_q, max_q, scale, out, out_dtype, lse, want_lse,
                    term_count, stream, block_table, splits, workspace):
    _dev(q, "q")
    _dev(kv_len, "kv_len")
    _dev(cu_q, "cu_q")
    if q.dim() != 3:
        raise ValueError("varlen q must be [rows][Hq][d]")
    rows, Hq, d = q.shape
    B = kv_len.numel()
    if cu_q.dtype != torch.int32 or cu_q.numel() != B + 1 or kv_len.dtype != torch.int32:
        raise ValueError("cu_q int32 [B+1] and kv_len int32 [B]")
    if max_q is None:
        raise ValueError("max_q (an upper bound of the per-sequence query counts) is needed")
    paged = isinstance(cache, PagedKVCache)
    if paged:
        table = cache._table(block_table)
        if table.shape[0] != B:
            raise ValueError("block_table must have B rows")
    elif B != cache.B:
        raise ValueError("kv_len must hold one length per cache sequence")
    if d != cache.d or cache.window_alpha is not None:
        raise ValueError("q must match the (dense) cache")
    _same_device(kv_len, q, "kv_len")
    _same_device(cu_q, q, "cu_q")
    _same_device(cache.k, q, "the cache")
    out = _out(out, q.shape, q, out_dtype)
    lse = _lse(lse, want_lse, (rows, Hq), q)
    term_count = _counter(term_count, q)
    _cached_ex(q, cache, table if paged else None, cu_q, kv_len, out, lse, B, int(max_q), Hq, d,
               alpha, scale, term_count, splits, workspace, stream)
    return (out, lse) if lse is not None else out


def full_window() -> float:
    """alpha for the full-window (dense) mode of the same kernels."""
    return math.inf

"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds workload shapes and random-number recipes only: no RoPE, no window,
no softmax.  Both the HIP path and the CPU oracle consume the exact tensors produced
here (the oracle receives the bf16 bit patterns / fp32 values, never a re-draw).

Shapes follow the attention layers of the models the pages evaluate (ATFlash abstract:
Qwen2.5-0.5B, Llama-3.2-3B, Qwen2.5-7B-1M).  No weights or datasets exist here; the
method's cost does not depend on the input values (ATFlash abstract: the pruned share is
fixed by the shapes alone), so seeded tensors at those shapes reproduce the cost profile.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    N: int               # prefill length, or decode Lmax
    Hq: int
    Hkv: int
    d: int
    base: float
    alphas: tuple
    dtype: str           # "bf16" or "fp32"
    seed: int
    dim_scale: bool = False      # per-dim log-uniform [0.5, 2] scale on q and k
    len_lo: int = 0              # decode: kv_len ~ U{len_lo .. N}


WORKLOADS = {
    # B=1, 2/2 heads, d=64, N=256, base 1e4, fp32 N(0,1)
    "tiny": Workload("tiny", "prefill", 1, 256, 2, 2, 64, 1e4, (1.0, 2.0, math.inf), "fp32", 1),
    # Qwen2.5-0.5B attention: 14 q / 2 kv heads, d=64, base 1e6, N=32768, alpha=1
    "qwen05b": Workload("qwen05b", "prefill", 1, 32768, 14, 2, 64, 1e6, (1.0,), "bf16", 2,
                        dim_scale=True),
    # Llama-3.2-3B attention: 24 q / 8 kv heads, d=128, base 5e5, N=131072, alpha 1 and 2
    "llama3b": Workload("llama3b", "prefill", 1, 131072, 24, 8, 128, 5e5, (1.0, 2.0), "bf16", 3),
    # Llama-3.2-3B decode: batch 16, Lmax 131072, kv_len ~ U{8192..131072}
    "llama3b_decode": Workload("llama3b_decode", "decode", 16, 131072, 24, 8, 128, 5e5, (1.0,),
                               "bf16", 4, len_lo=8192),
    # Qwen2.5-7B-1M attention: 28 q / 4 kv heads, d=128, base 1e7, 1M tokens
    "qwen7b1m": Workload("qwen7b1m", "prefill", 1, 1 << 20, 28, 4, 128, 1e7, (1.0,), "bf16", 5),
    "qwen7b1m_decode": Workload("qwen7b1m_decode", "decode", 1, 1 << 20, 28, 4, 128, 1e7, (1.0,),
                                "bf16", 5, len_lo=1 << 20),
}


def torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _gen(seed: int, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, dtype):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def dim_scales(d: int, g, device) -> torch.Tensor:
    """Per-dimension scale, log-uniform in [0.5, 2], shared by all heads and tokens."""
    u = torch.rand((d,), generator=g, device=device, dtype=torch.float32)
    return torch.exp(math.log(0.5) + u * (math.log(2.0) - math.log(0.5)))


def prefill_inputs(B, N, Hq, Hkv, d, dtype="bf16", seed=0, dim_scale=False, device="cpu"):
    """q [B][N][Hq][d], k, v [B][N][Hkv][d], N(0,1) (q, k optionally scaled per dim)."""
    g = _gen(seed, device)
    tdt = torch_dtype(dtype)
    if dim_scale:
        sq = dim_scales(d, g, device)
        sk = dim_scales(d, g, device)
        q = (torch.randn((B, N, Hq, d), generator=g, device=device) * sq).to(tdt)
        k = (torch.randn((B, N, Hkv, d), generator=g, device=device) * sk).to(tdt)
    else:
        q = _randn((B, N, Hq, d), g, device, tdt)
        k = _randn((B, N, Hkv, d), g, device, tdt)
    v = _randn((B, N, Hkv, d), g, device, tdt)
    return q, k, v


def decode_inputs(B, Lmax, Hq, Hkv, d, dtype="bf16", seed=0, len_lo=1, device="cpu"):
    """q [B][Hq][d]; pre-RoPE cache contents k, v [B][Lmax][Hkv][d]; kv_len [B] int32
    uniform on {len_lo .. Lmax}."""
    g = _gen(seed, device)
    tdt = torch_dtype(dtype)
    q = _randn((B, Hq, d), g, device, tdt)
    k = _randn((B, Lmax, Hkv, d), g, device, tdt)
    v = _randn((B, Lmax, Hkv, d), g, device, tdt)
    lens = torch.randint(len_lo, Lmax + 1, (B,), generator=g, device=device, dtype=torch.int64)
    return q, k, v, lens.to(torch.int32)


def workload_inputs(w: Workload, device="cpu", N=None):
    """Inputs for a named workload (optionally at a different length N)."""
    n = w.N if N is None else N
    if w.kind == "prefill":
        return prefill_inputs(w.B, n, w.Hq, w.Hkv, w.d, w.dtype, w.seed, w.dim_scale, device)
    return decode_inputs(w.B, n, w.Hq, w.Hkv, w.d, w.dtype, w.seed, min(w.len_lo, n), device)


def sample_rows(N: int, n: int, seed: int) -> np.ndarray:
    """Sorted query rows for sampled checks: first and last rows plus seeded random ones."""
    n = min(n, N)
    edge = min(n // 4, N)
    rows = set(range(edge)) | set(range(max(0, N - edge), N))
    rng = np.random.default_rng(seed)
    while len(rows) < n:
        rows.add(int(rng.integers(0, N)))
    return np.array(sorted(rows), dtype=np.int64)


def alias_inputs(N, H, d, dtype="bf16", seed=0, amp=2.5, device="cpu"):
    """Structured prefill inputs: every token's q and k is the same fixed random direction
    (times `amp`) plus small noise.  The pre-rotation product is then identical for every
    (query, key) and the score of a key depends on distance alone, through each pair's
    rotation; keys at distances where many high-frequency pairs come back into phase
    score high in the full window (the position aliasing the WavePrune abstract
    describes).  A short window removes those terms at long distance, so the outputs
    differ well beyond the parity tolerance.  Returns q, k, v [1][N][H][d]."""
    g = _gen(seed, device)
    tdt = torch_dtype(dtype)
    u = torch.randn((d,), generator=g, device=device)
    u = u / u.norm() * math.sqrt(d) / 4.0 * amp
    q = u + 0.1 * torch.randn((1, N, H, d), generator=g, device=device)
    k = u + 0.1 * torch.randn((1, N, H, d), generator=g, device=device)
    v = torch.randn((1, N, H, d), generator=g, device=device)
    return q.to(tdt), k.to(tdt), v.to(tdt)


def to_oracle(t: torch.Tensor) -> np.ndarray:
    """Exact bytes of a tensor for the oracle: float32 values, or bf16 bits as uint16."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)

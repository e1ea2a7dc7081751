#!/usr/bin/env python3
"""Benchmark of per-RoPE-wavelength windowed attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: the Qwen2.5-7B-1M-shaped attention layer (28 q / 4 kv heads, d=128,
rope base 1e7, alpha=1, bf16 synthetic N(0,1) tensors): a causal prefill of N = 1,048,576
tokens plus one batch-1 decode step at 1M context.  One step is that whole path:
key rotation/relayout (prefill_prepare) + windowed attention (prefill_attend) + the decode
step (decode_partial + decode_combine) against a resident 1M-token cache.  `value` is the
algorithmic (active-term) prefill TFLOP/s of the step, inputs resident in HBM:
    flops = B*Hq*(4*kept + 2*d*N(N+1)/2)
where kept (per head) is the exact kept-term count and P*V stays full.

Also reported on the same line:
  roofline       the attention kernel alone (HIP events around its launch on the launch
                 stream) vs the bf16 MFMA peak
  decode         the step's decode (Qwen2.5-7B-1M shape, L = 1M), algorithmic KV bytes/s
                 vs the HBM peak; decode_batch: the Llama-3.2-3B-shaped batch (B=16, 24/8
                 heads, kv_len ~ U{8192..131072}) timed in its own loop
  speedup_vs_full_window   the same kernels with alpha = inf (fewer prefill repetitions)
  cpu_baseline   the fp64 CPU oracle on a bounded sample of query rows of the same prefill,
                 with the full prefill's CPU time extrapolated from it
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("prefill active-term TFLOP/s + decode KV GB/s vs roofline; "
          "speedup over α=∞")
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen7b1m", help="prefill workload (synth.WORKLOADS)")
    ap.add_argument("--alpha", type=float, default=None, help="override the workload's alpha")
    ap.add_argument("--decode-workload", default="qwen7b1m_decode",
                    help="the decode step inside each timed step")
    ap.add_argument("--decode-batch-workload", default="llama3b_decode",
                    help="a second decode workload, timed in its own loop ('' to skip)")
    ap.add_argument("--full-window-reps", type=int, default=2,
                    help="timed prefill repetitions of the alpha = inf leg (after one warm-up)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-full-window", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line: the speedup sweep over alpha in {1, 2, inf} "
                         "at N = 32K..1M for the Llama-3.2-3B and Qwen2.5-7B-1M shapes, prefill "
                         "and decode (B=1 and B=16), printed as one JSON line")
    ap.add_argument("--sweep-max", type=int, default=1 << 20, help="largest N of the sweep")
    ap.add_argument("--extras", action="store_true",
                    help="instead of the headline line: the paths beside the core one (windowed "
                         "decode cache, chunked prefill, RoPE variants, block-sparse prefill), "
                         "printed as one JSON line")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the headline line: the prefill backward (dq, dk, dv) at the "
                         "Qwen2.5-0.5B (32K) and Llama-3.2-3B (128K) shapes, alpha 1 and inf, "
                         "printed as one JSON line")
    ap.add_argument("--cpu-table", action="store_true",
                    help="instead of the headline line: the fp64 oracle timed on this host's cores "
                         "for each workload (full runs of tiny and qwen05b, sampled rows of the "
                         "larger prefills with the full time extrapolated, full decode steps), "
                         "printed as one JSON line")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (twice), as the "
                         "reference kernel for scaling FETCH_SIZE/WRITE_SIZE counters")
    return ap.parse_args()


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _prefill_flops(w, alpha, N=None):
    import rope_wavelength_sparsity_amd as wpa
    n = w.N if N is None else N
    kept, _ = wpa.count_terms(w.d, w.base, alpha, n, 0, n)
    return w.B * w.Hq * (4 * kept + 2 * w.d * n * (n + 1) // 2), kept


def _decode_bytes(w, alpha, lens_h):
    """Algorithmic bytes of one decode step: K at 2 bf16-sized values per kept pair, full V
    rows, q in and out."""
    import rope_wavelength_sparsity_amd as wpa
    nbytes = 0
    for L in lens_h:
        kept, _ = wpa.count_terms(w.d, w.base, alpha, 1, L - 1, L)
        nbytes += w.Hkv * (4 * kept + 2 * w.d * L)
    return nbytes + 2 * 2 * w.B * w.Hq * w.d


class DecodeState:
    """A decode workload's query, lengths and resident KV cache (filled once, untimed)."""

    def __init__(self, w):
        import torch
        import rope_wavelength_sparsity_amd as wpa
        import synth
        self.w = w
        q, k, v, lens = synth.workload_inputs(w, device="cuda")
        self.cache = wpa.KVCache(w.B, w.N, w.Hkv, w.d, w.base)
        self.cache.write(k, v, 0)
        del k, v
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.q, self.lens = q, lens
        self.ws = torch.empty(max(wpa.decode_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.d), 16),
                              device="cuda", dtype=torch.uint8)
        self.out = torch.empty_like(q)
        self.lens_h = [int(x) for x in lens.cpu().tolist()]

    def step(self, alpha):
        import rope_wavelength_sparsity_amd as wpa
        wpa.decode(self.q, self.cache, self.lens, alpha, out=self.out, workspace=self.ws)


def bench_step(w, alpha, steps, warmup, dec):
    """Times `steps` steps of the whole path: prefill_prepare + prefill_attend over the
    prompt, then the decode step of `dec` (None: prefill only).  HIP events on the launch
    stream bracket each part of every timed step.  Returns a dict of timings."""
    import torch
    import rope_wavelength_sparsity_amd as wpa
    import synth
    q, k, v = synth.workload_inputs(w, device="cuda")
    ws = torch.empty(wpa.prefill_workspace_bytes(w.B, w.N, w.Hkv, w.d), device="cuda",
                     dtype=torch.uint8)
    out = torch.empty_like(q)
    ev = [_events(4) for _ in range(steps)]

    def step(e=None):
        if e is not None:
            e[0].record()
        wpa.prefill_prepare(k, v, w.base, workspace=ws)
        if e is not None:
            e[1].record()
        wpa.prefill_attend(q, ws, w.Hkv, w.base, alpha, out=out)
        if e is not None:
            e[2].record()
        if dec is not None:
            dec.step(alpha)
        if e is not None:
            e[3].record()

    slow = w.N >= (1 << 18)           # seconds per step: report progress as steps complete
    for i in range(warmup):
        step()
        if slow:
            torch.cuda.synchronize()
            _log("warm-up step %d/%d done" % (i + 1, warmup))
    torch.cuda.synchronize()
    t0, t1 = _events(2)
    w0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step(ev[i])
        if slow and i > 0:
            # step i is queued behind step i-1, so waiting for the end of step i-1 leaves the
            # GPU busy while the host prints
            ev[i - 1][3].synchronize()
            _log("step %d/%d done" % (i, steps))
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    avg = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in ev) / steps
    flops, kept = _prefill_flops(w, alpha)
    res = {"step_ms": t0.elapsed_time(t1) / steps, "prepare_ms": avg(0, 1), "attend_ms": avg(1, 2),
           "decode_ms": avg(2, 3), "wall_s": wall, "flops": flops, "kept_per_head": kept}
    del q, k, v, ws, out
    torch.cuda.empty_cache()
    return res


def bench_decode(dec, alpha, steps, warmup):
    """Mean time of `steps` back-to-back decode steps (HIP events) after `warmup`."""
    import torch
    for _ in range(warmup):
        dec.step(alpha)
    torch.cuda.synchronize()
    t0, t1 = _events(2)
    t0.record()
    for _ in range(steps):
        dec.step(alpha)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    return {"ms": ms, "bytes": _decode_bytes(dec.w, alpha, dec.lens_h),
            "kv_len_mean": sum(dec.lens_h) / len(dec.lens_h)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, alpha, target_s):
    """The unmodified fp64 oracle on a bounded sample of query rows (all heads) of the same
    prefill, on the same input values (drawn on the device, copied to the host).  The rate is
    algorithmic flops of the sampled rows per second; the full prefill's CPU time is
    extrapolated from it (labelled as such)."""
    import numpy as np
    import torch
    import oracle
    import rope_wavelength_sparsity_amd as wpa
    import synth
    q, k, v = synth.workload_inputs(w, device="cuda")
    qa, ka, va = synth.to_oracle(q), synth.to_oracle(k), synth.to_oracle(v)
    del q, k, v
    torch.cuda.empty_cache()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))

    def run(rows):
        t = time.perf_counter()
        oracle.prefill(qa, ka, va, w.base, alpha, rows=rows, nthreads=threads)
        return time.perf_counter() - t

    def row_flops(rows):
        f = 0
        for r in rows.tolist():
            kept, _ = wpa.count_terms(w.d, w.base, alpha, 1, r, r + 1)
            f += w.B * w.Hq * (4 * kept + 2 * w.d * (r + 1))
        return f

    rng = np.random.default_rng(12345)
    cal = np.sort(rng.integers(0, w.N, 8))
    tc = run(cal)
    n = int(max(8, min(4096, 8 * target_s / max(tc, 1e-3))))
    rows = np.sort(rng.integers(0, w.N, n))
    dt = run(rows)
    rate = row_flops(rows) / dt
    full, _ = _prefill_flops(w, alpha)
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": "%d random query rows x %d heads of %s (N=%d), fp64, %.1f s (%.3f s per row "
                      "on average, setup included)" % (n, w.Hq, w.name, w.N, dt, dt / n),
            "full_prefill_s_extrapolated": full / rate}


def backward_flops(w, alpha, N=None):
    """Algorithmic flops of the backward per call: per q head, the recomputed scores, dq' and
    dk' over the kept terms (4 flops each) and dP and dv over every visible (row, key) pair
    (2d flops each): 12*kept + 4*d*N(N+1)/2."""
    import rope_wavelength_sparsity_amd as wpa
    n = w.N if N is None else N
    kept, _ = wpa.count_terms(w.d, w.base, alpha, n, 0, n)
    return w.B * w.Hq * (12 * kept + 4 * w.d * n * (n + 1) // 2)


def bench_backward(names, reps):
    """wpa_prefill_backward timed with HIP events (mean of reps after one warm-up), alpha 1
    and alpha = inf, at each named prefill workload."""
    import torch
    import rope_wavelength_sparsity_amd as wpa
    import synth
    rows = []
    for name in names:
        w = synth.WORKLOADS[name]
        q, k, v = synth.workload_inputs(w, device="cuda")
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed + 100)
        dout = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
        ws = torch.empty(wpa.prefill_backward_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.d),
                         device="cuda", dtype=torch.uint8)
        dq = torch.empty(q.shape, device="cuda", dtype=torch.float32)
        dk = torch.empty(k.shape, device="cuda", dtype=torch.float32)
        dv = torch.empty(v.shape, device="cuda", dtype=torch.float32)
        r = {"workload": "%s: B=%d N=%d Hq=%d Hkv=%d d=%d base=%g" % (name, w.B, w.N, w.Hq, w.Hkv,
                                                                       w.d, w.base)}
        for alpha in (1.0, math.inf):
            out, lse = wpa.prefill(q, k, v, w.base, alpha, want_lse=True)
            run = lambda: wpa.prefill_backward(q, k, v, out, lse, dout, w.base, alpha, dq=dq, dk=dk,
                                               dv=dv, workspace=ws)
            run()
            torch.cuda.synchronize()
            a, b = _events(2)
            a.record()
            for _ in range(reps):
                run()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            fl = backward_flops(w, alpha)
            key = "alpha_1" if alpha == 1.0 else "alpha_inf"
            r[key] = {"ms": ms, "flops": fl, "tflops": fl / (ms * 1e-3) / 1e12,
                      "frac_of_bf16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
            _log("backward %s alpha=%g: %.2f ms, %.1f TFLOP/s" % (name, alpha, ms, r[key]["tflops"]))
            del out, lse
        r["speedup_vs_full_window"] = r["alpha_inf"]["ms"] / r["alpha_1"]["ms"]
        rows.append(r)
        del q, k, v, dout, ws, dq, dk, dv
        torch.cuda.empty_cache()
    return {"backward": rows, "timing": "HIP events, mean of %d calls after one warm-up; one call "
            "= prep + dq + dk/dv + reduce kernels" % reps,
            "flops": "per q head 12*kept + 4*d*N(N+1)/2 (scores, dq', dk' over kept terms; dP, dv "
                     "over visible pairs)"}


def _log(*a):
    print("#", *a, file=sys.stderr, flush=True)


def sweep_prefill(w, N, alphas, reps):
    """Prefill at length N for each alpha: prepare + attend timed per rep (HIP events), the
    attend kernel alone as well.  Returns a list of result dicts."""
    import torch
    import rope_wavelength_sparsity_amd as wpa
    import synth
    q, k, v = synth.workload_inputs(w, device="cuda", N=N)
    ws = torch.empty(wpa.prefill_workspace_bytes(w.B, N, w.Hkv, w.d), device="cuda",
                     dtype=torch.uint8)
    out = torch.empty_like(q)
    res = []
    for alpha in alphas:
        wpa.prefill_prepare(k, v, w.base, workspace=ws)          # warm-up
        wpa.prefill_attend(q, ws, w.Hkv, w.base, alpha, out=out)
        torch.cuda.synchronize()
        ev = _events(3 * reps)
        for i in range(reps):
            ev[3 * i].record()
            wpa.prefill_prepare(k, v, w.base, workspace=ws)
            ev[3 * i + 1].record()
            wpa.prefill_attend(q, ws, w.Hkv, w.base, alpha, out=out)
            ev[3 * i + 2].record()
        torch.cuda.synchronize()
        step = sorted(ev[3 * i].elapsed_time(ev[3 * i + 2]) for i in range(reps))[reps // 2]
        kern = sorted(ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(reps))[reps // 2]
        kept, total = wpa.count_terms(w.d, w.base, alpha, N, 0, N)
        flops = w.B * w.Hq * (4 * kept + 2 * w.d * N * (N + 1) // 2)
        r = {"kind": "prefill", "shape": w.name, "N": N, "alpha": alpha, "reps": reps,
             "attend_ms": kern, "step_ms": step, "flops": flops,
             "kept_fraction": kept / total, "attend_tflops": flops / (kern * 1e-3) / 1e12}
        _log("prefill %s N=%d alpha=%g: attend %.2f ms (%.0f TFLOP/s), step %.2f ms" % (
            w.name, N, alpha, kern, r["attend_tflops"], step))
        res.append(r)
    del q, k, v, ws, out
    torch.cuda.empty_cache()
    return res


def sweep_decode(w, B, L, alphas, reps):
    """One decode step of B sequences all at kv_len L, for each alpha; the 256 MB last-level
    cache is flushed by a 1 GB write before every timed call."""
    import torch
    import rope_wavelength_sparsity_amd as wpa
    import synth
    cache = wpa.KVCache(B, L, w.Hkv, w.d, w.base)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    chunk = max(1, min(L, (1 << 30) // (B * w.Hkv * w.d * 4)))
    for t0 in range(0, L, chunk):                 # fill the caches chunk by chunk
        n = min(chunk, L - t0)
        k = torch.randn((B, n, w.Hkv, w.d), generator=g, device="cuda").to(torch.bfloat16)
        v = torch.randn((B, n, w.Hkv, w.d), generator=g, device="cuda").to(torch.bfloat16)
        cache.write(k, v, t0)
        del k, v
    q = torch.randn((B, w.Hq, w.d), generator=g, device="cuda").to(torch.bfloat16)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(wpa.decode_workspace_bytes(B, L, w.Hq, w.Hkv, w.d), 16), device="cuda",
                     dtype=torch.uint8)
    out = torch.empty_like(q)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    res = []
    for alpha in alphas:
        wpa.decode(q, cache, lens, alpha, out=out, workspace=ws)
        ts = []
        for _ in range(reps):
            flush.zero_()
            a, b = _events(2)
            a.record()
            wpa.decode(q, cache, lens, alpha, out=out, workspace=ws)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ms = sorted(ts)[reps // 2]
        kept, _ = wpa.count_terms(w.d, w.base, alpha, 1, L - 1, L)
        nbytes = B * w.Hkv * (4 * kept + 2 * w.d * L) + 2 * 2 * B * w.Hq * w.d
        r = {"kind": "decode", "shape": w.name, "B": B, "L": L, "alpha": alpha, "reps": reps,
             "ms": ms, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9}
        _log("decode %s B=%d L=%d alpha=%g: %.3f ms (%.0f GB/s)" % (w.name, B, L, alpha, ms, r["gbs"]))
        res.append(r)
    del cache, q, ws, out, flush
    torch.cuda.empty_cache()
    return res


def sweep(max_n):
    """Speedup over the full window (alpha = inf) across lengths, prefill and decode."""
    import synth
    alphas = (1.0, 2.0, math.inf)
    lengths = [n for n in (1 << 15, 1 << 16, 1 << 17, 1 << 18, 1 << 19, 1 << 20) if n <= max_n]
    rows = []
    for name in ("llama3b", "qwen7b1m"):
        w = synth.WORKLOADS[name]
        for N in lengths:
            rows += sweep_prefill(w, N, alphas, 3 if N >= (1 << 19) else 5)
        for B in (1, 16):
            for L in lengths:
                rows += sweep_decode(w, B, L, alphas, 10)
    speed = []
    key = lambda r: (r["kind"], r["shape"], r.get("B", 1), r.get("N", r.get("L")))
    for r in rows:
        if math.isinf(r["alpha"]):
            continue
        full = [x for x in rows if key(x) == key(r) and math.isinf(x["alpha"])][0]
        t, tf = (r["attend_ms"], full["attend_ms"]) if r["kind"] == "prefill" else (r["ms"], full["ms"])
        speed.append({"kind": r["kind"], "shape": r["shape"], "B": r.get("B", 1),
                      "N": r.get("N", r.get("L")), "alpha": r["alpha"], "speedup": tf / t})
    return {"sweep": {"rows": rows, "speedup_vs_full_window": speed,
                      "timing": "median of reps; HIP events; decode after a 1 GB cache flush",
                      "data": "synthetic N(0,1) bf16 tensors (seeded)"}}


def _traffic(kernel_file, workload, alpha):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel source is
    unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    src = os.path.join(ROOT, "rope_wavelength_sparsity_amd", "csrc", kernel_file)
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for e in json.load(open(path)).get("entries", []):
        if e.get("source_sha256") == sha and e.get("workload") == workload and e.get("alpha") == alpha:
            return e["hbm_bytes_per_launch"]
    return None


def _time(fn, reps):
    """Mean ms of reps calls after three warm-up calls (HIP events on the current stream)."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a, b = _events(2)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _block_lists(B, H, N, density, seed, pattern="random"):
    """Block lists of 64-token blocks, ascending: the first block and the two blocks below the
    query block, plus
      random          each earlier block with probability `density`, drawn anew for every
                      (head, query block);
      vertical_slash  per head, a fixed set of key blocks ("vertical" columns, each block with
                      probability `density`) and 4 fixed diagonal offsets in [3, 64) ("slash"
                      lines), the same for every query block of the head: the shape of
                      MInference's vertical-slash index."""
    import numpy as np
    import torch
    rng = np.random.default_rng(seed)
    nblk = (N + 63) // 64
    width = max(3, int(density * nblk) + 16)
    count = np.zeros((B, H, nblk), np.int32)
    idx = np.zeros((B, H, nblk, width), np.int32)
    for b in range(B):
        for h in range(H):
            if pattern == "vertical_slash":
                vert = np.nonzero(rng.random(nblk) < density)[0]
                slash = rng.integers(3, 64, size=4)
            for R in range(nblk):
                if pattern == "random":
                    extra = np.nonzero(rng.random(R) < density)[0].tolist()
                else:
                    extra = vert[vert < R].tolist() + [R - int(o) for o in slash]
                s = sorted(c for c in {0, R - 1, R - 2} | set(extra) if 0 <= c < R)[-width:]
                count[b, h, R] = len(s)
                idx[b, h, R, :len(s)] = s
    return torch.from_numpy(count).cuda(), torch.from_numpy(idx).cuda()


def cpu_table():
    """The unmodified fp64 oracle on this host's cores for each workload, on the inputs the
    GPU runs use (drawn on the device, copied to the host): the tiny and Qwen2.5-0.5B prefills
    in full (the latter in slices of 4096 query rows, timed and summed), 128 / 64 sampled rows
    of the Llama-3.2-3B / Qwen2.5-7B-1M prefills with the full time extrapolated from them,
    and one full decode step of each decode workload."""
    import numpy as np
    import torch
    import oracle
    import rope_wavelength_sparsity_amd as wpa
    import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    res = {"cpu_model": _cpu_model(), "threads": threads, "rows": []}

    def host(w):
        ins = synth.workload_inputs(w, device="cuda")
        out = tuple(synth.to_oracle(t) if t.dtype != torch.int32 else t.cpu().numpy() for t in ins)
        del ins
        torch.cuda.empty_cache()
        return out

    def row_flops(w, alpha, rows):
        f = 0
        for r in rows.tolist():
            kept, _ = wpa.count_terms(w.d, w.base, alpha, 1, r, r + 1)
            f += w.B * w.Hq * (4 * kept + 2 * w.d * (r + 1))
        return f

    for name, sample in (("tiny", 0), ("qwen05b", 0), ("llama3b", 128), ("qwen7b1m", 64)):
        w = synth.WORKLOADS[name]
        alpha = 1.0
        qa, ka, va = host(w)
        if sample == 0:
            dt = 0.0
            for r0 in range(0, w.N, 4096):
                rows = np.arange(r0, min(w.N, r0 + 4096))
                t = time.perf_counter()
                oracle.prefill(qa, ka, va, w.base, alpha, rows=rows, nthreads=threads)
                dt += time.perf_counter() - t
                _log("cpu table: %s rows %d..%d, %.1f s so far" % (name, r0, rows[-1], dt))
            flops, _ = _prefill_flops(w, alpha)
            res["rows"].append({"workload": name, "kind": "prefill", "alpha": alpha, "run": "full",
                                "wall_s": dt, "gflops_fp64": flops / dt / 1e9})
        else:
            rows = synth.sample_rows(w.N, sample, seed=w.seed)
            t = time.perf_counter()
            oracle.prefill(qa, ka, va, w.base, alpha, rows=rows, nthreads=threads)
            dt = time.perf_counter() - t
            rate = row_flops(w, alpha, rows) / dt
            flops, _ = _prefill_flops(w, alpha)
            res["rows"].append({"workload": name, "kind": "prefill", "alpha": alpha,
                                "run": "%d sampled rows (first, last, random)" % len(rows),
                                "sample_s": dt, "s_per_row": dt / len(rows),
                                "gflops_fp64": rate / 1e9,
                                "full_s_extrapolated": flops / rate})
            _log("cpu table: %s %d rows in %.1f s" % (name, len(rows), dt))
        del qa, ka, va
    for name in ("llama3b_decode", "qwen7b1m_decode"):
        w = synth.WORKLOADS[name]
        qa, ka, va, lens = host(w)
        t = time.perf_counter()
        oracle.decode(qa, ka, va, lens, w.base, 1.0, nthreads=threads)
        dt = time.perf_counter() - t
        nbytes = _decode_bytes(w, 1.0, lens.tolist())
        res["rows"].append({"workload": name, "kind": "decode", "alpha": 1.0,
                            "run": "one full step (B=%d)" % w.B, "wall_s": dt,
                            "algorithmic_gbs": nbytes / dt / 1e9})
        _log("cpu table: %s step in %.2f s" % (name, dt))
        del qa, ka, va
    return res


def extras(reps):
    """Measurements of the paths beside the core prefill/decode, one dict per path."""
    import torch
    import rope_wavelength_sparsity_amd as wpa
    import synth
    res = {}
    w = synth.WORKLOADS["qwen05b"]
    q, k, v = synth.workload_inputs(w, device="cuda")
    ws = torch.empty(wpa.prefill_workspace_bytes(w.B, w.N, w.Hkv, w.d), device="cuda",
                     dtype=torch.uint8)
    kept_full, _ = wpa.count_terms(w.d, w.base, 1.0, w.N, 0, w.N)
    dense_flops = w.B * w.Hq * (4 * kept_full + 2 * w.d * w.N * (w.N + 1) // 2)
    # the GPU clock takes ~50 ms of work to settle: a short kernel timed right after input
    # generation runs up to 1.3x slower than once warm, so warm up for ~200 ms first
    for _ in range(100):
        wpa.prefill(q, k, v, w.base, 1.0, workspace=ws)
    t_one = _time(lambda: wpa.prefill(q, k, v, w.base, 1.0, workspace=ws), reps)

    # RoPE variants: the same prefill with a Llama-3-style frequency table, interleaved pairs
    theta = wpa.llama3_inv_freq(w.d, w.base, factor=32.0, low_freq_factor=1.0,
                                high_freq_factor=4.0, original_max_position=8192)
    var = {"workload": "qwen05b prefill (prepare + attend), alpha 1", "half_split_ms": t_one}
    for name, kw in (("llama3_table_ms", dict(inv_freq=theta)),
                     ("interleaved_ms", dict(pairs="interleaved")),
                     ("llama3_table_interleaved_ms", dict(inv_freq=theta, pairs="interleaved"))):
        var[name] = _time(lambda: wpa.prefill(q, k, v, w.base, 1.0, workspace=ws, **kw), reps)
    kept_t, _ = wpa.count_terms(w.d, w.base, 1.0, w.N, 0, w.N, inv_freq=theta)
    var["llama3_table_tflops"] = w.B * w.Hq * (4 * kept_t + 2 * w.d * w.N * (w.N + 1) // 2) / (
        var["llama3_table_ms"] * 1e-3) / 1e12
    res["rope_variants"] = var
    _log("extras: rope variants %s" % var)

    # chunked prefill: the same prompt appended and attended in chunks against the decode caches
    ch = {"workload": "qwen05b prompt of 32768 tokens, alpha 1", "one_shot_ms": t_one,
          "one_shot_tflops": dense_flops / (t_one * 1e-3) / 1e12}
    for C in (4096, 8192):
        cache = wpa.KVCache(w.B, w.N, w.Hkv, w.d, w.base)
        out = torch.empty_like(q)
        lens = [torch.full((w.B,), s + C, dtype=torch.int32, device="cuda")
                for s in range(0, w.N, C)]
        # key splits as the launch chooses them (their workspace allocated once), and none
        ns_bytes = wpa.prefill_cached_workspace_bytes(w.B, C, w.Hq, w.Hkv, w.d, 0)
        wsc = torch.empty(max(ns_bytes, 16), dtype=torch.uint8, device="cuda")
        ch["chunks_%d_key_splits" % C] = ns_bytes // (w.B * C * w.Hq * (w.d + 1) * 4) or 1
        for tag, sp in (("", 0), ("_no_key_splits", 1)):
            def run():
                for i, s in enumerate(range(0, w.N, C)):
                    cache.write(k[:, s:s + C], v[:, s:s + C], s)
                    wpa.prefill_cached(q[:, s:s + C], cache, lens[i], 1.0, out=out[:, s:s + C],
                                       splits=sp, workspace=wsc if sp != 1 else None)
            t = _time(run, reps)
            ch["chunks_%d%s_ms" % (C, tag)] = t
            ch["chunks_%d%s_tflops" % (C, tag)] = dense_flops / (t * 1e-3) / 1e12
        ch["chunks_%d_over_one_shot" % C] = ch["chunks_%d_ms" % C] / t_one
        del cache, out, wsc
    res["chunked_prefill"] = ch
    _log("extras: chunked %s" % ch)

    # block-sparse prefill on top of the window
    sp = {"workload": "qwen05b prefill (prepare + attend), alpha 1, 64-token blocks: first block, "
                      "two local blocks and earlier blocks, random per (head, query block) or "
                      "vertical-slash per head"}
    for pattern, dens in (("random", 0.3), ("random", 0.1), ("vertical_slash", 0.3),
                          ("vertical_slash", 0.1)):
        bc, bi = _block_lists(w.B, w.Hq, w.N, dens, 5, pattern)
        t = _time(lambda: wpa.prefill(q, k, v, w.base, 1.0, workspace=ws, block_count=bc,
                                      block_idx=bi), reps)
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        wpa.prefill(q, k, v, w.base, 1.0, workspace=ws, block_count=bc, block_idx=bi,
                    term_count=cnt)
        # active flops: 4 per kept term, P*V over the visited keys
        vis = 0
        cnt_h = bc.cpu().numpy()
        for R in range(cnt_h.shape[2]):
            # keys visited by the rows of block R: own block (causal) + listed blocks
            vis += int(cnt_h[:, :, R].sum()) * 64 * 64 + w.B * w.Hq * (64 * 65 // 2)
        flops = 4 * int(cnt.item()) + 2 * w.d * vis
        listed = float(bc.double().mean().item()) / ((w.N + 63) // 64 / 2)
        sp["%s_%g" % (pattern, dens)] = {"ms": t, "vs_dense_window": t / t_one,
                                         "listed_fraction": listed,
                                         "active_tflops": flops / (t * 1e-3) / 1e12}
        del bc, bi
    res["block_sparse_prefill"] = sp
    _log("extras: block sparse %s" % sp)
    del q, k, v, ws
    torch.cuda.empty_cache()

    # windowed decode cache: same step, K cache kept only inside each block's window
    wd = synth.WORKLOADS["llama3b_decode"]
    qd, kd, vd, lens = synth.workload_inputs(wd, device="cuda")
    dec = {"workload": "llama3b_decode, alpha 1"}
    nbytes = 0
    for L in lens.cpu().tolist():
        kp, _ = wpa.count_terms(wd.d, wd.base, 1.0, 1, L - 1, L)
        nbytes += wd.Hkv * (4 * kp + 2 * wd.d * L)
    for name, walpha in (("dense_cache", None), ("window_cache", 1.0)):
        cache = wpa.KVCache(wd.B, wd.N, wd.Hkv, wd.d, wd.base, window_alpha=walpha)
        for bi_, L in enumerate(lens.cpu().tolist()):        # each sequence up to its length
            cache.write(kd[bi_:bi_ + 1, :L].contiguous(), vd[bi_:bi_ + 1, :L].contiguous(), 0,
                        seq=bi_)
        wsd = torch.empty(max(wpa.decode_workspace_bytes(wd.B, wd.N, wd.Hq, wd.Hkv, wd.d), 16),
                          device="cuda", dtype=torch.uint8)
        out = torch.empty_like(qd)
        t = _time(lambda: wpa.decode(qd, cache, lens, 1.0, out=out, workspace=wsd), reps)
        dec[name] = {"ms": t, "gbs": nbytes / (t * 1e-3) / 1e9, "k_cache_bytes": cache.k.numel(),
                     "v_cache_bytes": cache.v.numel()}
        del cache, wsd, out
        torch.cuda.empty_cache()
    dec["kv_bytes_ratio"] = (dec["window_cache"]["k_cache_bytes"] + dec["window_cache"]["v_cache_bytes"]) / (
        dec["dense_cache"]["k_cache_bytes"] + dec["dense_cache"]["v_cache_bytes"])
    res["window_decode_cache"] = dec
    _log("extras: window cache %s" % dec)

    # paged decode cache: each sequence holds only the pages its length needs, shuffled
    import numpy as np
    pg = {"workload": "llama3b_decode, alpha 1, pages shuffled over the pool"}
    for ps in (64, 256):
        maxp = (wd.N + ps - 1) // ps
        need = [(L + ps - 1) // ps for L in lens.cpu().tolist()]
        order = np.random.default_rng(ps).permutation(sum(need))
        tab = np.zeros((wd.B, maxp), np.int32)
        at = 0
        for bi_, n_ in enumerate(need):
            tab[bi_, :n_] = order[at:at + n_]
            at += n_
        table = torch.from_numpy(tab).cuda()
        cache = wpa.PagedKVCache(sum(need), ps, wd.Hkv, wd.d, wd.base)
        for bi_, L in enumerate(lens.cpu().tolist()):
            cache.write(kd[bi_:bi_ + 1, :L].contiguous(), vd[bi_:bi_ + 1, :L].contiguous(), 0,
                        block_table=table[bi_:bi_ + 1])
        wsd = torch.empty(max(wpa.decode_workspace_bytes(wd.B, maxp * ps, wd.Hq, wd.Hkv, wd.d), 16),
                          device="cuda", dtype=torch.uint8)
        out = torch.empty_like(qd)
        t = _time(lambda: wpa.decode(qd, cache, lens, 1.0, out=out, workspace=wsd,
                                     block_table=table), reps)
        pg["page_%d" % ps] = {"ms": t, "gbs": nbytes / (t * 1e-3) / 1e9,
                              "kv_bytes": cache.k.numel() + cache.v.numel(),
                              "kv_bytes_vs_contiguous": (cache.k.numel() + cache.v.numel()) / (
                                  dec["dense_cache"]["k_cache_bytes"] + dec["dense_cache"]["v_cache_bytes"])}
        del cache, wsd, out, table
        torch.cuda.empty_cache()
    pg["contiguous_ms"] = dec["dense_cache"]["ms"]
    res["paged_decode_cache"] = pg
    _log("extras: paged cache %s" % pg)
    return res


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py runs on one GPU only: the windowed attention kernels here are single-GPU; "
              "the multi-GPU sharding is a design note, not an implemented path. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.sweep:
        print(json.dumps(sweep(args.sweep_max)), flush=True)
        return
    if args.extras:
        print(json.dumps({"extras": extras(max(5, args.steps // 2))}), flush=True)
        return
    if args.backward:
        print(json.dumps(bench_backward(("qwen05b", "llama3b"), max(2, args.steps // 4))), flush=True)
        return
    if args.cpu_table:
        print(json.dumps({"cpu_oracle_table": cpu_table()}), flush=True)
        return
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("# copy calibration: %d bytes per copy" % n, file=sys.stderr, flush=True)
        del src, dst
    w = synth.WORKLOADS[args.workload]
    assert w.kind == "prefill"
    alpha = args.alpha if args.alpha is not None else w.alphas[0]
    dec = None
    if not args.no_decode:
        wd = synth.WORKLOADS[args.decode_workload]
        _log("decode cache %s" % wd.name)
        dec = DecodeState(wd)
    _log("steps of %s alpha=%g%s" % (w.name, alpha, " + decode %s" % dec.w.name if dec else ""))
    st = bench_step(w, alpha, args.steps, args.warmup, dec)
    achieved = st["flops"] / (st["attend_ms"] * 1e-3) / 1e12
    step_desc = "prefill_prepare (key rotation + relayout) + prefill_attend"
    if dec is not None:
        step_desc += " + one decode step (decode_partial + decode_combine) of %s" % dec.w.name
    res = {
        "metric": METRIC,
        "value": st["flops"] / (st["step_ms"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": st["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tensors at the layer's shapes; no weights or datasets)",
        "config": {"workload": "%s prefill: B=%d N=%d Hq=%d Hkv=%d d=%d base=%g alpha=%g%s" % (
            w.name, w.B, w.N, w.Hq, w.Hkv, w.d, w.base, alpha,
            (" + decode step B=%d L=%d" % (dec.w.B, max(dec.lens_h))) if dec else ""),
            "step": step_desc,
            "value_is": "prefill algorithmic flops per step / step time (the decode step adds "
                        "%.4f ms to each step)" % st["decode_ms"],
            "algorithmic_flops_per_step": st["flops"],
            "kept_terms_per_head": st["kept_per_head"],
            "step_parts_ms": {"prefill_prepare": st["prepare_ms"], "prefill_attend": st["attend_ms"],
                              "decode": st["decode_ms"]}},
    }
    res["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                       "traffic": _traffic("prefill_kernel.hip", w.name, alpha),
                       "kernel": "prefill_kernel (attend)", "kernel_ms": st["attend_ms"]}
    _log("step %.1f ms: prepare %.2f ms, attend %.1f ms (%.1f TFLOP/s), decode %.4f ms" % (
        st["step_ms"], st["prepare_ms"], st["attend_ms"], achieved, st["decode_ms"]))
    speed = {}
    if dec is not None:
        gbs = _decode_bytes(dec.w, alpha, dec.lens_h) / (st["decode_ms"] * 1e-3) / 1e9
        res["decode"] = {"workload": "%s: B=%d L=%d Hq=%d Hkv=%d d=%d base=%g alpha=%g" % (
                             dec.w.name, dec.w.B, max(dec.lens_h), dec.w.Hq, dec.w.Hkv, dec.w.d,
                             dec.w.base, alpha),
                         "value": gbs, "unit": "GB/s", "ms_per_step": st["decode_ms"],
                         "timing": "HIP events around the decode launches inside each timed step",
                         "algorithmic_bytes": _decode_bytes(dec.w, alpha, dec.lens_h),
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                      "kernel": "decode_partial + decode_combine"}}
    if not args.no_full_window and not math.isinf(alpha):
        _log("full window: %d + 1 steps" % args.full_window_reps)
        full = bench_step(w, math.inf, args.full_window_reps, 1, dec)
        speed["prefill_attend"] = full["attend_ms"] / st["attend_ms"]
        speed["step"] = full["step_ms"] / st["step_ms"]
        speed["prefill_full_window_attend_ms"] = full["attend_ms"]
        speed["prefill_full_window_tflops_dense"] = full["flops"] / (full["attend_ms"] * 1e-3) / 1e12
        speed["prefill_full_window_reps"] = args.full_window_reps
        if dec is not None:
            speed["decode"] = full["decode_ms"] / st["decode_ms"]
            speed["decode_full_window_ms"] = full["decode_ms"]
        _log("full window attend %.1f ms: speedup %.3f" % (full["attend_ms"], speed["prefill_attend"]))
    del dec
    torch.cuda.empty_cache()
    if not args.no_decode and args.decode_batch_workload:
        wb = synth.WORKLOADS[args.decode_batch_workload]
        _log("decode batch %s" % wb.name)
        db = DecodeState(wb)
        r = bench_decode(db, alpha, args.steps, args.warmup)
        gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
        res["decode_batch"] = {"workload": "%s: B=%d Lmax=%d Hq=%d Hkv=%d d=%d base=%g alpha=%g, "
                                           "kv_len ~ U{%d..%d} (mean %.0f)" % (
                                               wb.name, wb.B, wb.N, wb.Hq, wb.Hkv, wb.d, wb.base,
                                               alpha, wb.len_lo, wb.N, r["kv_len_mean"]),
                               "value": gbs, "unit": "GB/s", "ms_per_step": r["ms"],
                               "algorithmic_bytes": r["bytes"],
                               "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                            "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                            "kernel": "decode_partial + decode_combine"}}
        _log("decode batch %.3f ms, %.0f GB/s" % (r["ms"], gbs))
        if not args.no_full_window:
            rf = bench_decode(db, math.inf, args.steps, args.warmup)
            speed["decode_batch"] = rf["ms"] / r["ms"]
            speed["decode_batch_full_window_ms"] = rf["ms"]
        del db
        torch.cuda.empty_cache()
    if speed:
        res["speedup_vs_full_window"] = speed
    if not args.no_cpu_baseline:
        _log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(w, alpha, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

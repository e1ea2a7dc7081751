"""Write tests/golden/counts.json: kept/total (query, key, pair) term counts per head at
the workload shapes, computed by the oracle's distance-histogram enumeration only.

Run from the repository root:  python tests/golden/make_counts.py
"""
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

CASES = [
    # name, d, base, alpha, n_q, q0, n_k
    ("tiny a=1", 64, 1e4, 1.0, 256, 0, 256),
    ("tiny a=2", 64, 1e4, 2.0, 256, 0, 256),
    ("tiny a=0", 64, 1e4, 0.0, 256, 0, 256),
    ("tiny a=inf", 64, 1e4, math.inf, 256, 0, 256),
    ("qwen05b prefill", 64, 1e6, 1.0, 32768, 0, 32768),
    ("llama3b prefill a=1", 128, 5e5, 1.0, 131072, 0, 131072),
    ("llama3b prefill a=2", 128, 5e5, 2.0, 131072, 0, 131072),
    ("llama3b decode L=131072", 128, 5e5, 1.0, 1, 131071, 131072),
    ("qwen7b1m prefill", 128, 1e7, 1.0, 1 << 20, 0, 1 << 20),
    ("qwen7b1m decode L=1M", 128, 1e7, 1.0, 1, (1 << 20) - 1, 1 << 20),
]


def main():
    out = []
    for name, d, base, alpha, n_q, q0, n_k in CASES:
        kept, total = oracle.count_by_distance(d, base, alpha, n_q, q0, n_k)
        out.append({"name": name, "d": d, "base": base, "alpha": "inf" if math.isinf(alpha) else alpha,
                    "n_q": n_q, "q0": q0, "n_k": n_k, "kept": kept, "total": total})
        print(name, kept, total, "pruned %.4f" % (1 - kept / total))
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "counts.json"), "w") as f:
        json.dump({"source": "oracle.count_by_distance (tests/golden/make_counts.py)",
                   "cases": out}, f, indent=1)


if __name__ == "__main__":
    main()

"""Write tests/golden/tiny_exact.json: a tiny seeded decode case and its
50-digit decimal result.  Calls only oracle.brute.exact (the high-precision
evaluation of the definition), never the GPU library.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import brute            # noqa: E402
from workloads import round_bf16    # noqa: E402


def main():
    rng = np.random.default_rng(2024)
    B, Hq, Hkv, D, P, NP = 2, 4, 2, 8, 2, 6
    lens = np.array([3, 5], dtype=np.int32)
    bt = np.array([[4, 1, -1], [0, 5, 2]], dtype=np.int32)
    q = round_bf16(rng.standard_normal((B, Hq, D)).astype(np.float32))
    k = round_bf16(rng.standard_normal((NP, P, Hkv, D)).astype(np.float32))
    v = round_bf16(rng.standard_normal((NP, P, Hkv, D)).astype(np.float32))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    expected = brute.exact(q, k, v, bt, lens, scale, Hkv)
    doc = {
        "citation": "definition of decode paged attention: page 1 of the source pages, issue "
                    "'ROCm gfx1200: PagedAttnOnline is 8.1x slower per call', section 'Where to "
                    "look' (online softmax over an NHD cache via block table and strides); "
                    "values from a 50-digit decimal evaluation (oracle/brute.py:exact)",
        "seed": 2024, "scale": scale, "num_kv_heads": Hkv,
        "q": q.tolist(), "k_cache": k.tolist(), "v_cache": v.tolist(),
        "block_tables": bt.tolist(), "context_lens": lens.tolist(),
        "expected": expected.tolist(),
    }
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_exact.json")
    with open(out, "w") as f:
        json.dump(doc, f)
    print("wrote", out)


if __name__ == "__main__":
    main()

"""Write tests/golden/tiny_fp32.json from the pure-Python brute force.

The pages print no worked numbers for this path, so the stored case is
computed here by ``oracle.brute`` alone (explicit loops, math.fsum sums,
selection by pairwise rank) on a seeded input from the shared generator:
B=2, 4 query / 2 KV heads, d=64, 40 cached tokens (second sequence 29),
W=4, fp32, keep ratio 0.25 (k = floor(0.25 n + 1/2)), one decode query per
query head over the kept rows.  Run: python tests/golden/make_golden.py
"""
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

from kv_cache_compression_score_amd import workloads as wl  # noqa: E402
from oracle import brute  # noqa: E402

CASE = dict(seed=7, B=2, Hq=4, Hkv=2, d=64, N_max=40, W=4, ctx=[40, 29], ratio=0.25)


def main():
    c = CASE
    lay = wl.random_case(c["seed"], B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], d=c["d"],
                         N_max=c["N_max"], W=c["W"], dtype=torch.float32, ctx=c["ctx"])
    G = c["Hq"] // c["Hkv"]
    scale = 1.0 / math.sqrt(c["d"])
    q, k, v = lay.q_win.double().tolist(), lay.k.double().tolist(), lay.v.double().tolist()
    qd = lay.q_dec[0].double().tolist()
    out = {"case": c, "scores": [], "lse": [], "kept": [], "dec_out": [], "dec_lse": []}
    for b in range(c["B"]):
        n = c["ctx"][b]
        kk = int(math.floor(c["ratio"] * n + 0.5))
        for h in range(c["Hkv"]):
            s, lse = brute.score([q[b][h * G + j] for j in range(G)], k[b][h], n, G, scale)
            kept = brute.top_k(s, kk)
            out["scores"].append(s)
            out["lse"].append(lse)
            out["kept"].append(kept)
            for j in range(G):
                o, l = brute.attend(qd[b][h * G + j], [k[b][h][t] for t in kept],
                                    [v[b][h][t] for t in kept], scale)
                out["dec_out"].append(o)
                out["dec_lse"].append(l)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32.json")
    with open(path, "w") as fh:
        json.dump(out, fh, separators=(",", ":"))
        fh.write("\n")
    print(path)


if __name__ == "__main__":
    main()

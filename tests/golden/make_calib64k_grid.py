"""Writes tests/golden/calib64k_grid.json: the oracle's per-KV-head NMSE grid
(8 heads x 9 learned candidates x 5 clips) and selections of the batched
calibration search at full size (65,536 tokens x 8 KV heads x 64 queries,
bf16 inputs, W_O [1024, 1024]), with a digest of the seeded inputs.

Calls nothing but the oracle (and the seeded input generator).  With G = 1
the per-head objective of KV head h is the one-head problem on head h's K,
V, queries and 128 rows of W_O (the oracle's per-head mode with one KV head
is its joint mode), so the heads run in parallel processes.

    python tests/golden/make_calib64k_grid.py [--procs 8]
"""
import argparse
import hashlib
import json
import os
import sys
import multiprocessing
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
OUT = os.path.join(HERE, "calib64k_grid.json")


def inputs():
    import synthetic
    w = synthetic.make("calib64k", "cpu")
    f = lambda t: t.float().numpy()
    return w, f(w.k), f(w.v), f(w.q), f(w.w_o)


def input_digest(k, v, q, w_o) -> str:
    h = hashlib.sha256()
    for a in (k, v, q, w_o):
        h.update(np.ascontiguousarray(a, np.float32).tobytes())
    return h.hexdigest()


def one_head(h):
    import oracle
    w, k, v, q, w_o = inputs()
    cands = [oracle.Rotation(c.kind, matrix=c.matrix.numpy()[h:h + 1]) for c in w.candidates]
    t0 = time.time()
    nm, _, best = oracle.candidate_nmse(k[:, h:h + 1], v[:, h:h + 1], q[:, h:h + 1], cands, list(w.clips),
                                        w_o[h * 128:(h + 1) * 128], oracle.SELECT_JOINT)
    print(f"head {h}: best {int(best[0])}, {time.time() - t0:.0f} s", flush=True)
    return h, nm[0].tolist(), int(best[0])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=8)
    a = ap.parse_args()
    import oracle
    oracle.build(force=False)
    w, k, v, q, w_o = inputs()
    H = w.H
    # (spawned workers: a forked copy of a process that has run torch can hang)
    with ProcessPoolExecutor(max_workers=a.procs, mp_context=multiprocessing.get_context("spawn")) as ex:
        res = sorted(ex.map(one_head, range(H)))
    out = {
        "_about": "Oracle NMSE grid of the batched calibration search at full size (written by "
                  "make_calib64k_grid.py, which calls only the oracle). Per KV head: post-W_O NMSE of each "
                  "(candidate, clip) variant, mean over the 64 calibration queries, and the first minimum.",
        "workload": "calib64k", "tokens": w.tokens, "kv_heads": H, "queries": int(q.shape[0]),
        "candidates": len(w.candidates), "clips": list(w.clips), "d_model": w.d_model,
        "input_sha256": input_digest(k, v, q, w_o),
        "nmse": [r[1] for r in res], "best": [r[2] for r in res],
    }
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {OUT}: best {out['best']}")


if __name__ == "__main__":
    main()

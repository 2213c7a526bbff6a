"""Writes tests/golden/optr_paper_settings.json: the oracle's OptR
calibration (Algorithm 1 at the paper's settings: 80 Adam steps per phase,
learning rate 0.02, held-out checks every 20 steps, lambda_K = 1, clip ratios
0.96 / 0.92, 64 sink and 256 recent BF16 tokens, the final 64 query
positions) of one synthetic layer with 8 KV heads, 32 query heads, d_model
4096, 6 calibration and 5 held-out sequences of 328-700 tokens (bf16).

Stores, per KV head and phase, the training loss of every step, the held-out
values and the selected step, the key mean, and a fixed sample of entries of
the two calibrated rotations.  Calls nothing but the oracle and the seeded
input generator; each KV head is an independent problem, so the heads run in
parallel processes.

    python tests/golden/make_optr_fixture.py [--procs 8]
"""
import argparse
import json
import multiprocessing
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
OUT = os.path.join(HERE, "optr_paper_settings.json")
SEED, H, HQ, DM = 11, 8, 32, 4096


def problem():
    import synthetic
    return synthetic.optr_problem(SEED, H=H, Hq=HQ, d_model=DM)


def sample_index():
    rng = np.random.default_rng(0)
    return rng.integers(0, 128, size=(32, 2))


def one_head(h):
    import torch
    torch.set_num_threads(1)   # (one head per process: no oversubscription)
    from oracle import optr
    pb = problem()
    G = HQ // H
    f = lambda t: t.float().numpy()
    sub = lambda ts: optr.TraceSet(np.ascontiguousarray(f(ts.k)[:, :, h:h + 1]),
                                   np.ascontiguousarray(f(ts.v)[:, :, h:h + 1]),
                                   np.ascontiguousarray(f(ts.q)[:, :, h * G:(h + 1) * G]), list(ts.lens))
    t0 = time.time()
    res = optr.calibrate(sub(pb["calib"]), sub(pb["heldout"]), G, pb["nq"],
                         f(pb["w_o"])[h * G * 128:(h + 1) * G * 128], pb["r0_k"].numpy()[h:h + 1],
                         pb["r0_v"].numpy()[h:h + 1], optr.Config())
    idx = sample_index()
    out = {"head": h, "key_mean": res["key_mean"][0].tolist(),
           "key": res["log"][0]["key"], "value": res["log"][0]["value"],
           "r_k_sample": [float(res["r_k"][0][i, j]) for i, j in idx],
           "r_v_sample": [float(res["r_v"][0][i, j]) for i, j in idx]}
    print(f"head {h}: selected {out['key']['selected_step']} / {out['value']['selected_step']}, "
          f"{time.time() - t0:.0f} s", flush=True)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=8)
    a = ap.parse_args()
    import oracle
    oracle.build(force=False)
    with ProcessPoolExecutor(max_workers=a.procs, mp_context=multiprocessing.get_context("spawn")) as ex:
        heads = list(ex.map(one_head, range(H)))
    pb = problem()
    out = {"_about": "Oracle OptR calibration of one synthetic layer at the paper's settings (written by "
                     "make_optr_fixture.py, which calls only the oracle).",
           "seed": SEED, "kv_heads": H, "q_heads": HQ, "d_model": DM, "queries": pb["nq"],
           "calib_lens": list(pb["calib"].lens), "heldout_lens": list(pb["heldout"].lens),
           "sample_index": sample_index().tolist(), "heads": heads}
    with open(OUT, "w") as f:
        json.dump(out, f)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()

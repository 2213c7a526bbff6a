"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (library defaults: automatic split count, the same entry points).

The GPU runs the whole workload; the oracle checks seeded samples it can
afford: the decode of whole sequences (all heads) read from the GPU's own
cache bytes, the cache write of sampled tokens group by group, and, for the
calibration search, one KV head's NMSE grid of one candidate rebuilt as a
single-head problem.  Bars: rel-L2 <= 1e-4 (fp32 inputs) / 2e-2 (bf16) for
out_o and out_y per (row, head); NMSE within 1e-3 relative.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from kvq_testlib import (f32np, gpu_decode, gpu_quantize, gpu_rot, oracle_decode_on_cache, oracle_rot, rel_l2,
                         sampled_quantize_check, tolerance)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_int2_amd import kvq
    kvq.load_library()
    return torch.device("cuda:0")


def _decode_check(name, w, cache, dev, seqs):
    out_o, out_y = gpu_decode(w, cache, dev)
    pages = cache.pages.cpu().numpy()
    (ref_o, ref_y), rows = oracle_decode_on_cache(w, pages, seqs)
    o, y = f32np(out_o)[rows], f32np(out_y)[rows]
    tol = tolerance(w)
    per = [rel_l2(o[r, j], ref_o[r, j]) for r in range(o.shape[0]) for j in range(o.shape[1])]
    per_y = [rel_l2(y[r], ref_y[r]) for r in range(y.shape[0])]
    print(f"{name}: sequences {list(seqs)}: out_o rel-L2 max {max(per):.2e}, out_y max {max(per_y):.2e} (tol {tol})",
          flush=True)
    assert max(per) <= tol and max(per_y) <= tol
    assert np.all(np.isfinite(f32np(out_o))) and np.all(np.isfinite(f32np(out_y)))
    return pages


@pytest.mark.parametrize("preset,seqs", [("paged16x32k", (0, 15)), ("gqa32k", (0,)), ("long131k", (2,))])
def test_fullsize_decode_and_cache_write(dev, preset, seqs):
    print(f"full-size {preset}", flush=True)
    w = synthetic.make(preset, dev)
    cache = gpu_quantize(w, dev)
    torch.cuda.synchronize()
    pages = _decode_check(preset, w, cache, dev, seqs)
    stats = sampled_quantize_check(w, pages, 384, seed=11)
    print(f"{preset}: sampled cache write {stats}", flush=True)


def test_fullsize_envelope(dev):
    """Envelope (fp32, 4,096 tokens x 4 heads): the whole cache write equals the
    oracle's byte for byte with the page-1 selected kind of rotation, and the
    10 fresh queries decode within 1e-4."""
    w = synthetic.make("envelope", dev)
    w.rot_k = w.rot_v = w.candidates[7]
    cache = gpu_quantize(w, dev)
    torch.cuda.synchronize()
    oc = oracle.Cache(w.num_pages, w.page_size, w.H)
    oracle.quantize(f32np(w.k), f32np(w.v), oc, oracle_rot(w.rot_k), oracle_rot(w.rot_v), clip_k=w.clip_k,
                    clip_v=w.clip_v, slot_mapping=w.slot_mapping.cpu().numpy())
    got = cache.pages.cpu().numpy()
    frac = float(np.mean(got != oc.pages))
    print(f"envelope: full cache byte mismatch {frac:.3e}", flush=True)
    assert frac <= 1e-4
    _decode_check("envelope", w, cache, dev, range(w.num_seqs))


def test_fullsize_calibration_search_sampled(dev):
    """Calibration search at 65,536 tokens x 8 heads x 64 queries x 9 x 5: the
    GPU's full per-head NMSE grid; the oracle recomputes head 5's row for the
    GPU-selected candidate (all 5 clips) as a one-head problem (G = 1: the
    head's query head and its 128 rows of W_O)."""
    from decode_attention_int2_amd import kvq
    w = synthetic.make("calib64k", dev)
    C, n = len(w.candidates), len(w.clips)
    T, H, Nq, Hq = w.tokens, w.H, w.q.shape[0], w.Hq
    out = torch.empty((H, C, n), dtype=torch.float32, device=dev)
    best = torch.empty((H,), dtype=torch.int32, device=dev)
    ws = torch.empty(kvq.kvq_candidate_workspace_bytes(T, H, Hq, Nq, C, n, w.d_model), dtype=torch.uint8, device=dev)
    kvq.kvq_candidate_nmse(w.k, w.v, w.q, [gpu_rot(c) for c in w.candidates], list(w.clips), w.w_o,
                           kvq.KVQ_SELECT_PER_HEAD, out, best, workspace=ws)
    torch.cuda.synchronize()
    got, best = f32np(out), best.cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(got >= 0)
    for u in range(H):   # the selection is the first argmin of the GPU's own grid
        assert best[u] == int(np.argmin(got[u].ravel()))
    h = 5
    r = int(best[h]) // n
    dm = w.d_model
    k1 = f32np(w.k)[:, h:h + 1]
    v1 = f32np(w.v)[:, h:h + 1]
    q1 = f32np(w.q)[:, h:h + 1]
    wo1 = f32np(w.w_o)[h * 128:(h + 1) * 128]
    ref, _, _ = oracle.candidate_nmse(k1, v1, q1, [oracle_rot(w.candidates[r], heads=[h])], list(w.clips), wo1,
                                      oracle.SELECT_JOINT)
    rel = np.abs(got[h, r] - ref[0, 0]) / np.abs(ref[0, 0])
    print(f"calib64k head {h} candidate {r}: GPU {got[h, r]}, oracle {ref[0, 0]}, max rel {rel.max():.2e}", flush=True)
    assert rel.max() <= 1e-3
    assert dm == 1024

"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (library defaults: automatic split count, the same entry points).

The GPU runs the whole workload; the oracle checks what it can afford: the
decode of whole sequences (all heads) read from the GPU's own cache bytes,
the cache write of sampled tokens group by group, the envelope's whole
search-then-evaluate protocol, and the calibration search's full grid (the
oracle's values stored by a script that runs only the oracle).  Bars: rel-L2
<= 1e-4 (fp32 inputs) / 2e-2 (bf16) for out_o and out_y per (row, head); NMSE
within 1e-3 relative; selections identical up to near-ties within that
tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from kvq_testlib import (check_selection, f32np, gpu_decode, gpu_quantize, gpu_rot, oracle_decode_on_cache,
                         oracle_rot, rel_l2, sampled_quantize_check, tolerance)

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


def _search(dev, k, v, q, cands, clips, w_o, mode, key_mean=None):
    from decode_attention_int2_amd import kvq
    T, H = k.shape[0], k.shape[1]
    Nq, Hq = q.shape[0], q.shape[1]
    U = 1 if mode == kvq.KVQ_SELECT_JOINT else H
    C, n = len(cands), len(clips)
    out = torch.empty((U, C, n), dtype=torch.float32, device=dev)
    outq = torch.empty((U, C, n, Nq), dtype=torch.float32, device=dev)
    best = torch.empty((U,), dtype=torch.int32, device=dev)
    ws = torch.empty(kvq.kvq_candidate_workspace_bytes(T, H, Hq, Nq, C, n, w_o.shape[1]), dtype=torch.uint8,
                     device=dev)
    kvq.kvq_candidate_nmse(k, v, q, [gpu_rot(c) for c in cands], clips, w_o, mode, out, best,
                           out_nmse_per_query=outq, key_mean=key_mean, workspace=ws)
    torch.cuda.synchronize()
    return f32np(out), f32np(outq), best.cpu().numpy()


def test_fullsize_envelope_protocol(dev):
    """The evaluation page's protocol at its size ("Output-aware INT2 KV-cache
    rotation evaluation", observed envelope and results table): the joint
    search of identity + 8 signed-Hadamard candidates x 5 clips on 1
    calibration query over 4,096 tokens x 4 KV heads (fp32), then the 10
    fresh queries at the selected (candidate, clip): per-query post-W_O NMSE,
    their mean and population sd, and the threshold quality (NMSE <= 10),
    each against the oracle (NMSE within 1e-3 relative)."""
    from decode_attention_int2_amd import kvq
    w = synthetic.make("envelope", dev)
    clips = list(w.clips)
    n = len(clips)
    q_cal, q_eval = w.q[:1].contiguous(), w.q[1:].contiguous()
    ocands = [oracle_rot(c) for c in w.candidates]
    k, v, wo = f32np(w.k), f32np(w.v), f32np(w.w_o)
    got, _, best = _search(dev, w.k, w.v, q_cal, w.candidates, clips, w.w_o, kvq.KVQ_SELECT_JOINT)
    ref, _, rbest = oracle.candidate_nmse(k, v, f32np(q_cal), ocands, clips, wo, oracle.SELECT_JOINT)
    rel = np.abs(got - ref) / ref
    print(f"envelope search: GPU best {int(best[0])}, oracle best {int(rbest[0])}, NMSE max rel {rel.max():.2e}; "
          f"identity best {ref[0, 0].min():.4g}, selected {ref[0].ravel()[int(rbest[0])]:.4g}", flush=True)
    assert rel.max() <= 1e-3
    check_selection(best, rbest, ref)
    r, i = divmod(int(rbest[0]), n)
    # the 10 fresh queries at the selected variant (C = 1, one clip, per-query output)
    _, gq, _ = _search(dev, w.k, w.v, q_eval, [w.candidates[r]], [clips[i]], w.w_o, kvq.KVQ_SELECT_JOINT)
    _, rq, _ = oracle.candidate_nmse(k, v, f32np(q_eval), [ocands[r]], [clips[i]], wo, oracle.SELECT_JOINT)
    gq, rq = gq[0, 0, 0], rq[0, 0, 0]
    relq = np.abs(gq - rq) / rq
    sg, so = oracle.evaluation_stats(gq), oracle.evaluation_stats(rq)
    print(f"envelope fresh queries: NMSE GPU {sg['nmse_mean']:.6g} +- {sg['nmse_sd']:.6g}, oracle "
          f"{so['nmse_mean']:.6g} +- {so['nmse_sd']:.6g}; quality GPU {sg['quality_mean']:.2f} +- "
          f"{sg['quality_sd']:.2f}, oracle {so['quality_mean']:.2f} +- {so['quality_sd']:.2f}; "
          f"max rel {relq.max():.2e}", flush=True)
    assert relq.max() <= 1e-3
    assert abs(sg["nmse_mean"] - so["nmse_mean"]) <= 1e-3 * so["nmse_mean"]
    assert abs(sg["nmse_sd"] - so["nmse_sd"]) <= 1e-3 * so["nmse_mean"]
    # threshold quality: identical unless a query sits within the NMSE tolerance of the threshold
    if not np.any(np.abs(rq - 10.0) <= 1e-3 * 10.0):
        assert (sg["quality_mean"], sg["quality_sd"]) == (so["quality_mean"], so["quality_sd"])


def test_fullsize_calibration_search_all_heads(dev):
    """Calibration search at full size (65,536 tokens x 8 KV heads x 64
    queries x 9 learned candidates x 5 clips, bf16): all 8 x 45 NMSE values
    within 1e-3 relative of the oracle's and every head's selection equal to
    the oracle's first minimum (tests/golden/calib64k_grid.json, written by
    make_calib64k_grid.py from the oracle; the inputs are drawn on the host
    as there, and their digest is checked first)."""
    import json
    import os
    from decode_attention_int2_amd import kvq
    with open(os.path.join(os.path.dirname(__file__), "golden", "calib64k_grid.json")) as f:
        gold = json.load(f)
    w = synthetic.make("calib64k", "cpu")
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    from make_calib64k_grid import input_digest
    assert input_digest(f32np(w.k), f32np(w.v), f32np(w.q), f32np(w.w_o)) == gold["input_sha256"], \
        "seeded inputs differ from the ones the fixture was computed on"
    to = lambda t: None if t is None else t.to(dev)
    cands = [synthetic.RotationSpec(c.kind, matrix=to(c.matrix)) for c in w.candidates]
    got, _, best = _search(dev, to(w.k), to(w.v), to(w.q), cands, list(w.clips), to(w.w_o),
                           kvq.KVQ_SELECT_PER_HEAD)
    ref = np.asarray(gold["nmse"], np.float64)
    rbest = np.asarray(gold["best"], np.int64)
    rel = np.abs(got - ref) / ref
    print(f"calib64k: GPU best {best.tolist()}, oracle best {rbest.tolist()}, NMSE max rel {rel.max():.2e}",
          flush=True)
    assert rel.max() <= 1e-3
    check_selection(best, rbest, ref)


def test_fullsize_windows_decode_sampled(dev):
    """The BF16-window decode at the paged workload's full size (16 x 32,768
    tokens x 8 KV heads, 64 sink + 256 recent tokens, the default split plan
    bench.py times): sequences 0 and 15 against the oracle, whose windows are
    written by the oracle from those sequences' own tokens and whose cache is
    the GPU's bytes; bar 1e-4 per (row, head)."""
    from decode_attention_int2_amd import kvq
    w = synthetic.make("paged16x32k", dev)
    cache = gpu_quantize(w, dev)
    B, T, H, qps = w.num_seqs, w.tokens, w.H, w.queries_per_seq
    S_w, W_w = 64, 256
    seq_idx = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(T)
    pos = torch.arange(T, dtype=torch.int32, device=dev).repeat(B)
    gw = kvq.Windows(B, H, S_w, W_w, device=dev)
    kvq.kvq_window_write(w.k, w.v, seq_idx, pos, gw, seq_lens=w.seq_lens)
    out_o = torch.full((B * qps, w.Hq, 128), 12345.0, dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.kvq_decode_workspace_bytes(B, qps, w.Hq, H, T, 0, 0), dtype=torch.uint8, device=dev)
    kvq.kvq_decode_attn_windows(w.q, B, qps, cache, w.page_table, w.page_table.shape[1], w.seq_lens, T,
                                gpu_rot(w.rot_k), gpu_rot(w.rot_v), gw, out_o, key_mean=w.key_mean, workspace=ws)
    torch.cuda.synchronize()
    seqs = [0, 15]
    oc = oracle.Cache(w.num_pages, w.page_size, H)
    oc.pages[...] = cache.pages.cpu().numpy()
    lens = w.seq_lens.cpu().numpy()[seqs]
    ow = oracle.Windows(len(seqs), H, S_w, W_w, key_mean=None if w.key_mean is None else f32np(w.key_mean))
    for i, s in enumerate(seqs):
        oracle.window_write(f32np(w.k[s * T:(s + 1) * T]), f32np(w.v[s * T:(s + 1) * T]), np.full(T, i, np.int32),
                            np.arange(T, dtype=np.int32), ow, seq_lens=lens)
    rows = np.concatenate([np.arange(s * qps, (s + 1) * qps) for s in seqs])
    pt = w.page_table.cpu().numpy()[seqs]
    ref = oracle.decode_windows(f32np(w.q)[rows], oc, lens, oracle_rot(w.rot_k), oracle_rot(w.rot_v), ow,
                                num_seqs=len(seqs), queries_per_seq=qps, page_table=pt, max_pages=pt.shape[1])
    o = f32np(out_o)[rows]
    per = max(rel_l2(o[r, j], ref[r, j]) for r in range(o.shape[0]) for j in range(o.shape[1]))
    print(f"full-size windows decode: sequences {seqs}: worst (row, head) rel-L2 {per:.2e}", flush=True)
    assert per <= 1e-4
    assert np.all(np.isfinite(f32np(out_o)))

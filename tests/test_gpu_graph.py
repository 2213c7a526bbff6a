"""The hot path under HIP graph capture: kvq_quantize and kvq_decode_attn
(with and without W_O) captured once in a torch.cuda.CUDAGraph and replayed
several times, with eager calls of the same entry points (sharing the decode
workspace, so its arrival counters see other launches in between) and
synchronizations between the replays.  Every replay must give the eager
result: cache bytes identical, decode outputs within 1e-5 rel-L2 per
(row, head) (the split partials may be formed by other waves than in the
eager call, which moves fp32 rounding only).  Nothing in these entry points
allocates, synchronizes or records a memset, so the capture holds kernel
nodes only."""
import numpy as np
import pytest
import torch

import synthetic
from kvq_testlib import f32np, gpu_rot, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_int2_amd import kvq
    kvq.load_library()
    return torch.device("cuda:0")


def _per_row_head(a, b):
    a, b = f32np(a), f32np(b)
    if a.ndim == 3:
        return max(rel_l2(a[r, j], b[r, j]) for r in range(a.shape[0]) for j in range(a.shape[1]))
    return max(rel_l2(a[r], b[r]) for r in range(a.shape[0]))


@pytest.mark.parametrize("preset,kw", [("gqa32k", dict(tokens=4096)), ("paged16x32k", dict(tokens=2048, num_seqs=4))])
def test_graph_replay_matches_eager(dev, preset, kw):
    from decode_attention_int2_amd import kvq
    print(f"graph replay: {preset} {kw}", flush=True)
    w = synthetic.make(preset, dev, **kw)
    rk, rv = gpu_rot(w.rot_k), gpu_rot(w.rot_v)
    rows, T = w.num_seqs * w.queries_per_seq, w.tokens
    max_pages = w.page_table.shape[1]
    ws = torch.empty(kvq.kvq_decode_workspace_bytes(w.num_seqs, w.queries_per_seq, w.Hq, w.H, T, w.d_model, 0),
                     dtype=torch.uint8, device=dev)

    def write(cache):
        kvq.kvq_quantize(w.k, w.v, cache, rk, rv, key_mean=w.key_mean, clip_k=w.clip_k, clip_v=w.clip_v,
                         slot_mapping=w.slot_mapping)

    def decode(cache, o, y, o2):
        kvq.kvq_decode_attn(w.q, w.num_seqs, w.queries_per_seq, cache, w.page_table, max_pages, w.seq_lens, T, rk, rv,
                            o, w_o=w.w_o, out_y=y, workspace=ws)
        kvq.kvq_decode_attn(w.q, w.num_seqs, w.queries_per_seq, cache, w.page_table, max_pages, w.seq_lens, T, rk, rv,
                            o2, workspace=ws)

    new_o = lambda: torch.full((rows, w.Hq, 128), 12345.0, dtype=torch.float32, device=dev)
    new_y = lambda: torch.full((rows, w.d_model), 12345.0, dtype=torch.float32, device=dev)
    # eager reference
    ce = kvq.Cache(w.num_pages, w.page_size, w.H, device=dev)
    ce.pages.fill_(0xA5)  # (the same filler as the graph's cache gets before each replay)
    write(ce)
    oe, ye, o2e = new_o(), new_y(), new_o()
    decode(ce, oe, ye, o2e)
    torch.cuda.synchronize()
    # capture (the graph's cache and outputs are its own buffers)
    cg = kvq.Cache(w.num_pages, w.page_size, w.H, device=dev)
    og, yg, o2g = new_o(), new_y(), new_o()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        write(cg)
        decode(cg, og, yg, o2g)
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between the replays: fresh sentinels, and eager calls on
        # another cache with the same workspace
        cg.pages.fill_(0xA5)
        for t in (og, yg, o2g):
            t.fill_(12345.0)
        cx = kvq.Cache(w.num_pages, w.page_size, w.H, device=dev)
        write(cx)
        decode(cx, new_o(), new_y(), new_o())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        mism = int((cg.pages != ce.pages).sum().item())
        eo, ey, eo2 = _per_row_head(og, oe), _per_row_head(yg, ye), _per_row_head(o2g, o2e)
        print(f"  replay {rep}: cache byte mismatches {mism}, out_o {eo:.2e}, out_y {ey:.2e}, out_o (no W_O) "
              f"{eo2:.2e}", flush=True)
        assert mism == 0
        assert eo <= 1e-5 and ey <= 1e-5 and eo2 <= 1e-5
        assert np.all(np.isfinite(f32np(og))) and np.all(np.isfinite(f32np(yg)))
    del g

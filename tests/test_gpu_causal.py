"""Causal query chunks on the GPU (kvq_decode_attn_causal) against the
oracle's causal decode on the same INT2 cache bytes: row qi of a sequence
attends its first L - (queries_per_seq - 1 - qi) tokens."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from kvq_testlib import f32np, gpu_quantize, gpu_rot, oracle_rot, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_int2_amd import kvq
    kvq.load_library()
    return torch.device("cuda:0")


CASES = {
    # name: (workload, overrides, ragged lengths, num_splits)
    "paged_sh_chunk16": ("paged16x32k", dict(tokens=1500, num_seqs=3, H=2, Hq=8, d_model=64, queries=16),
                         [1500, 700, 9], 0),
    "gqa_dense_chunk64_g1": ("gqa32k", dict(tokens=2000, H=4, Hq=4, d_model=64, queries=64), None, 0),
    "long_dense_chunk8_many_splits": ("long131k", dict(tokens=3000, num_seqs=2, H=2, Hq=4, d_model=64, queries=8),
                                      [3000, 1111], 12),
    "envelope_f32_chunk10": ("envelope", dict(tokens=900, queries=10), None, 0),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_causal_decode_matches_oracle(dev, case):
    from decode_attention_int2_amd import kvq
    name, over, lens, ns = CASES[case]
    w = synthetic.make(name, dev, **over)
    if name == "envelope":
        w.rot_k = w.rot_v = w.candidates[2]
    if lens is not None:
        w.seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    cache = gpu_quantize(w, dev)
    B, qps = w.num_seqs, w.queries_per_seq
    rows = B * qps
    out_o = torch.full((rows, w.Hq, 128), 12345.0, dtype=torch.float32, device=dev)
    out_y = torch.full((rows, w.d_model), 12345.0, dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.kvq_decode_workspace_bytes(B, qps, w.Hq, w.H, w.tokens, w.d_model, ns), dtype=torch.uint8,
                     device=dev)
    kvq.kvq_decode_attn_causal(w.q, B, qps, cache, w.page_table, w.page_table.shape[1], w.seq_lens, w.tokens,
                               gpu_rot(w.rot_k), gpu_rot(w.rot_v), out_o, w_o=w.w_o, out_y=out_y, workspace=ws,
                               num_splits=ns)
    torch.cuda.synchronize()
    oc = oracle.Cache(w.num_pages, w.page_size, w.H)
    oc.pages[...] = cache.pages.cpu().numpy()
    ref = oracle.decode_causal(f32np(w.q), oc, w.seq_lens.cpu().numpy(), oracle_rot(w.rot_k), oracle_rot(w.rot_v),
                               num_seqs=B, queries_per_seq=qps, page_table=w.page_table.cpu().numpy(),
                               max_pages=w.page_table.shape[1])
    o = f32np(out_o)
    lens_np = w.seq_lens.cpu().numpy()
    live = [r for r in range(rows) if lens_np[r // qps] - (qps - 1 - r % qps) > 0]
    for r in set(range(rows)) - set(live):
        assert np.all(o[r] == 0.0)                       # rows with no token
    eo = rel_l2(o[live], ref[live])
    per = max(rel_l2(o[r, j], ref[r, j]) for r in live for j in range(w.Hq))
    y_ref = ref.reshape(rows, -1) @ f32np(w.w_o).astype(np.float64)
    ey = rel_l2(f32np(out_y)[live], y_ref[live])
    print(f"{case}: rel-L2 out_o {eo:.2e}, worst (row, head) {per:.2e}, out_y {ey:.2e}")
    assert eo <= 1e-4 and per <= 1e-4 and ey <= 1e-4

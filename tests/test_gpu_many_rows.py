"""Decodes with 32 to 64 query rows per (sequence, KV head): the matrix-core
kernel then runs 4 to 8 pairs of 4-row groups per KV head, each pair in its
own workgroups over the head's cache.  The oracle decodes the GPU's own
cache bytes; every (query row, head) within the fp32 bar, rel-L2 <= 1e-4
([OptR] §3 Eq. (1)-(2); Appendix Eq. (21)-(22), (26)-(28)).  Cases: full and
partial groups (32, 33, 40, 48, 64 rows), ragged lengths (1 token, a page
boundary, full), a permuted page table with 16- and 64-token pages (one group
per workgroup), fp32 and bf16 inputs, identity / signed-Hadamard / dense
rotations with key centering, one split and many, the W_O projection, and a
bad page index confined to its sequence (host-forced condition)."""
import numpy as np
import pytest
import torch

import synthetic
from kvq_testlib import f32np, gpu_decode, gpu_quantize, oracle_decode_on_cache, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_int2_amd import kvq
    kvq.load_library()
    return torch.device("cuda:0")


def _per_row_head(got, ref):
    return max(rel_l2(got[r, j], ref[r, j]) for r in range(ref.shape[0]) for j in range(ref.shape[1]))


def _case(name, dev):
    splits, lens, with_wo = 0, None, False
    if name == "rows64_sh_ragged":
        w = synthetic.make("paged16x32k", dev, tokens=1500, num_seqs=3, H=2, Hq=32, queries=4, d_model=64)
        lens = synthetic.ragged_seq_lens(3, 1500, seed=31)
    elif name == "rows32_dense_centered_wo":
        w = synthetic.make("gqa32k", dev, tokens=1700, H=2, Hq=8, queries=8, d_model=96)
        with_wo = True
    elif name == "rows40_pages64":
        w = synthetic.make("paged16x32k", dev, tokens=1400, num_seqs=2, H=2, Hq=8, queries=10, d_model=64,
                           page_size=64)
        lens = synthetic.ragged_seq_lens(2, 1400, seed=32, page_size=64)
    elif name == "rows48_f32":
        w = synthetic.make("envelope", dev, tokens=1100, H=2, Hq=2, queries=48, d_model=64)
    elif name == "rows33_identity":
        w = synthetic.make("envelope", dev, tokens=800, H=1, Hq=1, queries=33, d_model=64)
        w.rot_k = w.rot_v = synthetic.RotationSpec(synthetic.ROT_IDENTITY)
    elif name == "rows64_one_split":
        w = synthetic.make("paged16x32k", dev, tokens=1200, num_seqs=2, H=2, Hq=32, queries=4, d_model=64)
        splits = 1
    else:  # rows64_many_splits
        w = synthetic.make("paged16x32k", dev, tokens=3000, num_seqs=2, H=2, Hq=32, queries=4, d_model=64)
        splits = 12
    if lens is not None:
        w.seq_lens = lens.to(dev)
    return w, splits, with_wo


@pytest.mark.parametrize("name", ["rows64_sh_ragged", "rows32_dense_centered_wo", "rows40_pages64", "rows48_f32",
                                  "rows33_identity", "rows64_one_split", "rows64_many_splits"])
def test_many_rows_parity(dev, name):
    w, splits, with_wo = _case(name, dev)
    R = w.queries_per_seq * w.Hq // w.H
    print(f"{name}: {R} rows per KV head, page size {w.page_size}, splits {splits or 'default'}", flush=True)
    assert 32 <= R <= 64
    cache = gpu_quantize(w, dev)
    out_o, out_y = gpu_decode(w, cache, dev, with_wo=with_wo, num_splits=splits)
    (ref_o, ref_y), rows = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), range(w.num_seqs), with_wo=with_wo)
    e = _per_row_head(f32np(out_o)[rows], ref_o)
    msg = f"{name}: max rel-L2 per (row, head) {e:.2e}"
    if with_wo:
        ey = rel_l2(f32np(out_y)[rows], ref_y)
        msg += f", out_y {ey:.2e}"
        assert ey <= 1e-4
    print(msg, flush=True)
    assert e <= 1e-4


def test_many_rows_bad_page_confined(dev):
    """An out-of-range page index inside sequence 1 (64 rows per KV head):
    that sequence's outputs are NaN, the others match the oracle."""
    w = synthetic.make("paged16x32k", dev, tokens=1500, num_seqs=3, H=2, Hq=32, queries=4, d_model=64)
    cache = gpu_quantize(w, dev)
    pt = w.page_table.clone()
    pt[1, 40] = w.num_pages + 3
    out_o, _ = gpu_decode(w, cache, dev, page_table=pt, with_wo=False)
    o = f32np(out_o)
    nq = w.queries_per_seq
    assert np.all(np.isnan(o[nq:2 * nq]))
    (ref_o, _), rows = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), [0, 2], with_wo=False)
    assert np.all(np.isfinite(o[rows]))
    e = _per_row_head(o[rows], ref_o)
    print(f"bad page: sequences 0 and 2 max rel-L2 per (row, head) {e:.2e}", flush=True)
    assert e <= 1e-4

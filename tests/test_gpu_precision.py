"""fp32 precision of the decode where the value weights' fixed-point floor
matters: a long single sequence with the default split plan, and one split
holding a dominant token and a long, coherent tail whose weights lie 20-24
binary orders below it ([OptR] §3 Eq. (1)-(2): every cached token keeps its
softmax weight).  The oracle decodes the same cache bytes; the bar is the
fp32 one, rel-L2 <= 1e-4 per (query row, head)."""
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


def test_fp32_long_sequence_default_plan(dev):
    """1 sequence x 131,072 tokens x 2 KV heads (8 query heads, 2 query rows),
    fp32 inputs, signed-Hadamard rotation, the default split plan."""
    w = synthetic.make("envelope", dev, tokens=131072, H=2, Hq=8, queries=2, d_model=256)
    cache = gpu_quantize(w, dev)
    out_o, out_y = gpu_decode(w, cache, dev)
    (ref_o, ref_y), _ = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), [0])
    e = _per_row_head(f32np(out_o), ref_o)
    ey = rel_l2(f32np(out_y), ref_y)
    print(f"131072 tokens: max rel-L2 per (row, head) {e:.2e}, out_y {ey:.2e}", flush=True)
    assert e <= 1e-4 and ey <= 1e-4


@pytest.mark.parametrize("gap_log2,queries", [(20.0, 1), (22.0, 1), (24.0, 1), (20.0, 8), (24.0, 8)])
def test_fp32_dominant_token_and_long_tail_in_one_split(dev, gap_log2, queries):
    """One split of 131,072 tokens: one dominant token whose logit lies about
    gap_log2 binary orders above the others, and a tail whose values share a
    direction opposite to the dominant value, so that the tail's ~3-10% of the
    softmax mass visibly moves the output.  4 query rows per KV head (one
    group per workgroup) and 32 (four pairs of groups)."""
    T, H, Hq = 131072, 1, 4
    w = synthetic.make("envelope", dev, tokens=T, H=H, Hq=Hq, queries=queries, d_model=64)
    g = torch.Generator().manual_seed(9100 + int(gap_log2))
    s = 0.5
    z = torch.randn(128, generator=g, dtype=torch.float64)
    q = (s * z).to(torch.float32)
    k = torch.randn((T, H, 128), generator=g)
    u = torch.randn(128, generator=g)
    v = u + 0.3 * torch.randn((T, H, 128), generator=g)
    pos = T // 2 + 77
    # (INT2 keeps a Gaussian key's projection on itself on average): aim the
    # dominant logit gap_log2 binary orders (natural units: * ln 2) above the tail's
    beta = gap_log2 * np.log(2.0) / (s * float(z.norm()) / np.sqrt(128.0))
    k[pos, 0] = (beta * z / z.norm()).to(torch.float32)
    v[pos, 0] = -u
    w.k, w.v = k.contiguous().to(dev), v.contiguous().to(dev)
    w.q = q.expand(queries, Hq, 128).contiguous().to(dev)
    w.rot_k = w.rot_v = synthetic.RotationSpec(synthetic.ROT_IDENTITY)
    w.clip_k = w.clip_v = 1.0
    cache = gpu_quantize(w, dev)
    out_o, out_y = gpu_decode(w, cache, dev, num_splits=1)
    (ref_o, ref_y), _ = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), [0])
    # the workload is what it claims: the dominant token's logit sits 20-24 binary orders above the tail
    from kvq_testlib import parse_cache
    pc = parse_cache(cache.pages.cpu().numpy(), w.slot_mapping.cpu().numpy(), w.page_size)
    codes, sc, zr = pc["k"]
    kh = codes[:, 0].astype(np.float64) * sc[:, 0, None] + zr[:, 0, None]
    lg = kh @ q.double().numpy() / np.sqrt(128.0) / np.log(2.0)
    gap = lg[pos] - np.delete(lg, pos)
    tail_mass = float(np.sum(2.0 ** -gap))
    print(f"gap {gap_log2}: log2 gaps {gap.min():.1f}..{gap.max():.1f}, tail mass {tail_mass:.3f}", flush=True)
    assert abs(np.median(gap) - gap_log2) < 2 and tail_mass > 5e-3
    e = _per_row_head(f32np(out_o), ref_o)
    print(f"gap {gap_log2}, {queries * Hq // H} rows: max rel-L2 per (row, head) {e:.2e}", flush=True)
    assert e <= 1e-4

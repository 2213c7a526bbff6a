"""kvq_decode_attn_noalloc (the library's per-GPU scratch array instead of a
workspace) against kvq_decode_attn with a workspace, on calls in a row whose
plans lay the scratch out differently (the later ones smaller), and the
error for shapes that need more scratch than the array holds."""
import pytest
import torch

import synthetic
from kvq_testlib import f32np, gpu_quantize, gpu_rot, rel_l2, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_int2_amd import kvq
    kvq.load_library()
    return torch.device("cuda:0")


def _both(w, cache, dev):
    from decode_attention_int2_amd import kvq
    rows = w.num_seqs * w.queries_per_seq
    max_pages = w.page_table.shape[1]
    outs = []
    for noalloc in (False, True):
        out_o = torch.full((rows, w.Hq, 128), 12345.0, dtype=torch.float32, device=dev)
        out_y = torch.full((rows, w.d_model), 12345.0, dtype=torch.float32, device=dev)
        args = (w.q, w.num_seqs, w.queries_per_seq, cache, w.page_table, max_pages, w.seq_lens, w.tokens,
                gpu_rot(w.rot_k), gpu_rot(w.rot_v), out_o)
        if noalloc:
            kvq.kvq_decode_attn_noalloc(*args, w_o=w.w_o, out_y=out_y)
        else:
            ws = torch.empty(kvq.kvq_decode_workspace_bytes(w.num_seqs, w.queries_per_seq, w.Hq, w.H, w.tokens,
                                                            w.d_model, 0), dtype=torch.uint8, device=dev)
            kvq.kvq_decode_attn(*args, w_o=w.w_o, out_y=out_y, workspace=ws)
        torch.cuda.synchronize()
        outs.append((f32np(out_o), f32np(out_y)))
    return outs


def test_noalloc_matches_workspace_decode_on_calls_in_a_row(dev):
    big = synthetic.make("paged16x32k", dev, tokens=3000, num_seqs=4, H=4, Hq=16, d_model=256)
    small = synthetic.make("envelope", dev, tokens=1000, H=2, Hq=4, d_model=128)
    smaller = synthetic.make("paged16x32k", dev, tokens=700, num_seqs=2, H=2, Hq=8, d_model=128, seed=7)
    for w in (big, small, smaller, big):
        cache = gpu_quantize(w, dev)
        (ro, ry), (no, ny) = _both(w, cache, dev)
        eo, ey = rel_l2(no, ro), rel_l2(ny, ry)
        print(f"{w.name} {w.num_seqs}x{w.tokens} H={w.H} Hq={w.Hq}: rel-L2 out_o {eo:.2e}, out_y {ey:.2e}",
              flush=True)
        assert eo <= tolerance(w) and ey <= tolerance(w)
        assert (no != 12345.0).all() and (ny != 12345.0).all()


def test_noalloc_rejects_shapes_beyond_the_scratch(dev):
    from decode_attention_int2_amd import kvq
    B, Hq, H = 256, 32, 8
    need = kvq.kvq_decode_workspace_bytes(B, 1, Hq, H, 16, 0, 0)
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    cache = kvq.Cache(B, 16, H, device=dev)
    rot = kvq.Rotation(kvq.KVQ_ROT_IDENTITY)
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    out = torch.full((B, Hq, 128), 7.0, dtype=torch.float32, device=dev)
    lens = torch.full((B,), 16, dtype=torch.int32, device=dev)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn_noalloc(q, B, 1, cache, None, 1, lens, 16, rot, rot, out)
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

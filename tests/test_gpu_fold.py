"""Value-rotation folding on the GPU against the oracle, and the decode
equivalence it exists for: decoding with an identity R_V and the folded W_O
gives the out_y of decoding with R_V and W_O (the pages' Appendix, Eq. (31))."""
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


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("kind", ["identity", "sh", "dense"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fold_matches_oracle(dev, kind, dtype):
    from decode_attention_int2_amd import kvq
    w = synthetic.make("gqa32k" if kind == "dense" else "paged16x32k", dev, tokens=16, H=2, Hq=8, d_model=200)
    rot = {"identity": synthetic.RotationSpec(synthetic.ROT_IDENTITY), "sh": w.rot_k, "dense": w.rot_k}[kind]
    wo = w.w_o.float() if dtype == "f32" else w.w_o.to(torch.bfloat16)
    out = torch.empty_like(wo)
    kvq.kvq_fold_value_rotation(wo, w.Hq // w.H, gpu_rot(rot), out)
    torch.cuda.synchronize()
    ref = oracle.fold_value_rotation(f32np(wo), w.Hq // w.H, oracle_rot(rot))
    got = f32np(out)
    if kind == "identity":
        assert np.array_equal(got, f32np(wo))
    elif dtype == "f32":
        assert np.allclose(got, ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())
    else:
        # the GPU rounds its fp32 sum (off by at most ~1e-6 of the block's scale) to bf16 (half a
        # step, 2^-8 relative): the bound where cancellation makes a value small is the absolute term
        bound = 2.0 ** -8 * np.maximum(np.abs(ref), np.abs(got)) + 1e-6 * np.abs(ref).max()
        assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("case", ["paged_sh_f32w", "gqa_dense_bf16"])
def test_decode_with_folded_wo_equals_explicit_inverse_rotation(dev, case):
    from decode_attention_int2_amd import kvq
    if case == "paged_sh_f32w":
        w = synthetic.make("paged16x32k", dev, tokens=700, num_seqs=3, H=2, Hq=8, d_model=96)
        wo = w.w_o.float().contiguous()
        tol = 1e-5
    else:
        w = synthetic.make("gqa32k", dev, tokens=900, H=2, Hq=8, d_model=128)
        wo = w.w_o
        tol = 1e-2          # the folded weights are rounded to bf16 once more
    cache = gpu_quantize(w, dev)
    wf = torch.empty_like(wo)
    kvq.kvq_fold_value_rotation(wo, w.Hq // w.H, gpu_rot(w.rot_v), wf)
    ident = kvq.Rotation(synthetic.ROT_IDENTITY)
    B, qps = w.num_seqs, w.queries_per_seq
    ys = []
    for rv, wmat in ((gpu_rot(w.rot_v), wo), (ident, wf)):
        out_o = torch.empty((B * qps, w.Hq, 128), dtype=torch.float32, device=dev)
        out_y = torch.empty((B * qps, w.d_model), dtype=torch.float32, device=dev)
        ws = torch.empty(kvq.kvq_decode_workspace_bytes(B, qps, w.Hq, w.H, w.tokens, w.d_model, 0), dtype=torch.uint8,
                         device=dev)
        q = w.q if wmat.dtype == w.q.dtype else w.q.to(wmat.dtype)
        kvq.kvq_decode_attn(q, B, qps, cache, w.page_table, w.page_table.shape[1], w.seq_lens, w.tokens,
                            gpu_rot(w.rot_k), rv, out_o, w_o=wmat, out_y=out_y, workspace=ws)
        torch.cuda.synchronize()
        ys.append(f32np(out_y))
    err = rel_l2(ys[1], ys[0])
    print(f"{case}: rel-L2 of out_y, folded vs explicit {err:.2e}")
    assert err <= tol

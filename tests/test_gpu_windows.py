"""BF16 sink and recent windows on the GPU against the oracle.

The window write is compared byte for byte (bf16 copies, fp32 rounded to
nearest even); the decode with windows is compared with the oracle's fp64
decode reading the same INT2 cache bytes and the same window buffers, at the
fp32 tolerance of the plain decode (rel-L2 <= 1e-4), per (row, head) too.
"""
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


def _windows_from_tokens(w, dev, num_sink, num_recent):
    """GPU windows written from the workload's tokens in one call (every
    position of every sequence, the sequences' lengths given, so only the
    positions that end inside a window are kept) and the oracle's windows
    written from the same tokens in order."""
    from decode_attention_int2_amd import kvq
    B, T = w.num_seqs, w.tokens
    seq_idx = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(T)
    pos = torch.arange(T, dtype=torch.int32, device=dev).repeat(B)
    gw = kvq.Windows(B, w.H, num_sink, num_recent, device=dev)
    kvq.kvq_window_write(w.k, w.v, seq_idx, pos, gw, seq_lens=w.seq_lens)
    km = None if w.key_mean is None else f32np(w.key_mean)
    ow = oracle.Windows(B, w.H, num_sink, num_recent, key_mean=km)
    oracle.window_write(f32np(w.k), f32np(w.v), seq_idx.cpu().numpy(), pos.cpu().numpy(), ow,
                        seq_lens=w.seq_lens.cpu().numpy())
    torch.cuda.synchronize()
    return gw, ow


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_write_bit_exact(dev, dtype):
    from decode_attention_int2_amd import kvq
    rng = np.random.default_rng(41)
    B, H, S, W, n = 3, 2, 16, 32, 400
    k = torch.from_numpy(rng.standard_normal((n, H, 128)).astype(np.float32)).to(dev)
    v = torch.from_numpy(rng.standard_normal((n, H, 128)).astype(np.float32)).to(dev)
    if dtype == "bf16":
        k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    seq = rng.integers(-1, B + 1, n).astype(np.int32)          # includes out-of-range sequences
    pos = rng.integers(-3, 120, n).astype(np.int32)            # includes negative positions
    keep = np.ones(n, bool)                                    # one writer per destination slot
    seen = set()
    for i in range(n):
        dst = (int(seq[i]), int(pos[i]) if pos[i] < S else S + int(pos[i]) % W)
        if dst in seen:
            keep[i] = False
        seen.add(dst)
    seq, pos = seq[keep], pos[keep]
    k, v = k[torch.from_numpy(keep).to(dev)].contiguous(), v[torch.from_numpy(keep).to(dev)].contiguous()
    gw = kvq.Windows(B, H, S, W, device=dev)
    kvq.kvq_window_write(k, v, torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev), gw)
    ow = oracle.Windows(B, H, S, W)
    oracle.window_write(f32np(k), f32np(v), seq, pos, ow)
    torch.cuda.synchronize()
    for g, o in ((gw.sink_k, ow.sink_k), (gw.sink_v, ow.sink_v), (gw.recent_k, ow.recent_k),
                 (gw.recent_v, ow.recent_v)):
        assert np.array_equal(_bits(g), o)
    # whole sequences in one call with their lengths: ring slots shared by
    # earlier positions are not written, so the result is deterministic
    T = 150
    kk = torch.from_numpy(rng.standard_normal((B * T, H, 128)).astype(np.float32)).to(dev)
    vv = torch.from_numpy(rng.standard_normal((B * T, H, 128)).astype(np.float32)).to(dev)
    if dtype == "bf16":
        kk, vv = kk.to(torch.bfloat16), vv.to(torch.bfloat16)
    seq2 = np.repeat(np.arange(B, dtype=np.int32), T)
    pos2 = np.tile(np.arange(T, dtype=np.int32), B)
    lens = np.array([150, 37, 9], np.int32)              # tokens past a length are not written
    gw2 = kvq.Windows(B, H, S, W, device=dev)
    kvq.kvq_window_write(kk, vv, torch.from_numpy(seq2).to(dev), torch.from_numpy(pos2).to(dev), gw2,
                         seq_lens=torch.from_numpy(lens).to(dev))
    ow2 = oracle.Windows(B, H, S, W)
    oracle.window_write(f32np(kk), f32np(vv), seq2, pos2, ow2, seq_lens=lens)
    torch.cuda.synchronize()
    for g, o in ((gw2.sink_k, ow2.sink_k), (gw2.sink_v, ow2.sink_v), (gw2.recent_k, ow2.recent_k),
                 (gw2.recent_v, ow2.recent_v)):
        assert np.array_equal(_bits(g), o)


CASES = {
    # name: (workload, overrides, ragged lengths, num_sink, num_recent, with W_O)
    "paged_sh_ragged": ("paged16x32k", dict(tokens=900, num_seqs=6, H=2, Hq=8, d_model=64),
                        [900, 0, 40, 64, 300, 513], 64, 256, True),
    "gqa_dense_centered": ("gqa32k", dict(tokens=1500, H=2, Hq=8, d_model=128), None, 64, 256, True),
    "long_dense_multiquery": ("long131k", dict(tokens=1100, num_seqs=2, H=2, Hq=4, d_model=96, queries=3),
                              [1100, 333], 64, 256, False),
    "envelope_f32_small_windows": ("envelope", dict(tokens=700, queries=2), None, 16, 40, True),
    # 22 splits of ~1,600 INT2 tokens: every wave of the long sequence completes
    # rounds of claims and computes its last blocks after requesting its window
    # tiles; splits 20 and 21 get no window tile (20 tiles of 16), and the
    # short sequence's waves leave their loops before a full round
    "paged_sh_22_splits": ("paged16x32k", dict(tokens=36000, num_seqs=2, H=2, Hq=8, d_model=64),
                           [36000, 20000], 64, 256, False, 22),
    # 64-token pages, 6 splits of ~2,000 tokens (the last blocks computed after
    # the window tiles' request, on the 64-token page addressing), W_O
    "pages64_6_splits": ("paged16x32k", dict(tokens=12800, num_seqs=2, H=2, Hq=8, d_model=64, page_size=64),
                         [12800, 7000], 64, 256, True, 6),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_with_windows_matches_oracle(dev, case):
    from decode_attention_int2_amd import kvq
    name, over, lens, S, W, with_wo, *splits = CASES[case]
    splits = splits[0] if splits else 0
    w = synthetic.make(name, dev, **over)
    if name == "envelope":
        w.rot_k = w.rot_v = w.candidates[3]
    if lens is not None:
        w.seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    cache = gpu_quantize(w, dev)
    gw, ow = _windows_from_tokens(w, dev, S, W)
    B, qps = w.num_seqs, w.queries_per_seq
    rows = B * qps
    out_o = torch.full((rows, w.Hq, 128), 12345.0, dtype=torch.float32, device=dev)
    out_y = torch.full((rows, w.d_model), 12345.0, dtype=torch.float32, device=dev) if with_wo else None
    ws = torch.empty(max(1, kvq.kvq_decode_workspace_bytes(B, qps, w.Hq, w.H, w.tokens, w.d_model if with_wo else 0,
                                                           splits)), dtype=torch.uint8, device=dev)
    kvq.kvq_decode_attn_windows(w.q, B, qps, cache, w.page_table, w.page_table.shape[1], w.seq_lens, w.tokens,
                                gpu_rot(w.rot_k), gpu_rot(w.rot_v), gw, out_o, key_mean=w.key_mean,
                                w_o=w.w_o if with_wo else None, out_y=out_y, workspace=ws, num_splits=splits)
    torch.cuda.synchronize()
    oc = oracle.Cache(w.num_pages, w.page_size, w.H)
    oc.pages[...] = cache.pages.cpu().numpy()
    ref = oracle.decode_windows(f32np(w.q), oc, w.seq_lens.cpu().numpy(), oracle_rot(w.rot_k), oracle_rot(w.rot_v),
                                ow, num_seqs=B, queries_per_seq=qps, page_table=w.page_table.cpu().numpy(),
                                max_pages=w.page_table.shape[1])
    o = f32np(out_o)
    lens_np = w.seq_lens.cpu().numpy()
    for r in range(rows):
        if lens_np[r // qps] == 0:
            assert np.all(o[r] == 0.0)
    eo = rel_l2(o, ref)
    per = max(rel_l2(o[r, j], ref[r, j]) for r in range(rows) for j in range(w.Hq) if lens_np[r // qps] > 0)
    print(f"{case}: rel-L2 out_o {eo:.2e}, worst (row, head) {per:.2e}")
    assert eo <= 1e-4 and per <= 1e-4
    if with_wo:
        y_ref = ref.reshape(rows, -1) @ f32np(w.w_o).astype(np.float64)
        assert rel_l2(f32np(out_y), y_ref) <= 1e-4


def test_decode_with_windows_bad_page_is_nan_for_that_sequence(dev):
    from decode_attention_int2_amd import kvq
    w = synthetic.make("paged16x32k", dev, tokens=900, num_seqs=3, H=2, Hq=8, d_model=64)
    cache = gpu_quantize(w, dev)
    gw, _ = _windows_from_tokens(w, dev, 64, 256)
    pt = w.page_table.clone()
    pt[1, 20] = w.num_pages + 5                         # an INT2 position of sequence 1 (320 .. 643)
    out_o = torch.zeros((3, w.Hq, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.kvq_decode_workspace_bytes(3, 1, w.Hq, w.H, w.tokens, 0, 0), dtype=torch.uint8, device=dev)
    kvq.kvq_decode_attn_windows(w.q, 3, 1, cache, pt, pt.shape[1], w.seq_lens, w.tokens, gpu_rot(w.rot_k),
                                gpu_rot(w.rot_v), gw, out_o, workspace=ws)
    torch.cuda.synchronize()
    o = f32np(out_o)
    assert np.all(np.isnan(o[1])) and np.all(np.isfinite(o[[0, 2]]))


def test_bits_per_element_library_matches_oracle():
    from decode_attention_int2_amd import kvq
    for L, S, W in ((65536, 64, 256), (300, 64, 256), (4096, 0, 0), (1, 64, 256), (70000, 16, 40)):
        assert kvq.kvq_bits_per_element(L, S, W) == oracle.bits_per_element(L, S, W)

"""HIP path vs CPU oracle, element by element, on seeded inputs through the C ABI.

Bars: codes and metadata bit-exact (byte work); floats within rel-L2 1e-4 for
fp32 inputs and 2e-2 for bf16 inputs; candidate NMSE within 1e-3 relative and
the selected candidate identical unless the oracle's best two are a near-tie.
Sizes span several 256-token chunks, several splits and ragged tails.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from kvq_testlib import (check_rotated_quantization, check_selection, f32np, gpu_decode, gpu_quantize, gpu_rot,
                         oracle_cache_and_decode, oracle_decode_on_cache, oracle_rot, rel_l2, tolerance)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_int2_amd import kvq
    kvq.load_library()
    return torch.device("cuda:0")


def _special_groups(n_tok, H, rng):
    """Edge groups: constant (s == 0), exact rounding ties, one huge outlier, tiny range."""
    x = rng.standard_normal((n_tok, H, 128)).astype(np.float32)
    x[0, 0, :] = 1.25                                  # degenerate: all codes 0, z = 1.25
    tie = np.zeros(128, np.float32)
    tie[:4] = [0.0, 3.0, 0.5, 2.5]                     # c = 1: s = 1, z = 0; ties 0.5 -> 0, 2.5 -> 2
    tie[4:] = 1.5                                      # tie 1.5 -> 2
    x[1, 0, :] = tie
    x[2, 0, 7] = 4000.0                                # outlier dominates the range
    x[3, 0, :] *= 1e-4                                 # tiny range, fp16 subnormal scale
    return x


@pytest.mark.parametrize("dtype,clip_k,clip_v,center", [("f32", 1.0, 1.0, False), ("f32", 0.96, 0.92, False),
                                                         ("f32", 0.8, 0.85, True), ("bf16", 1.0, 1.0, False),
                                                         ("bf16", 0.96, 0.92, False), ("bf16", 0.8, 0.85, True)])
def test_quantize_prerotated_bitexact(dev, dtype, clip_k, clip_v, center):
    """Identity rotation (pre-rotated inputs), fp32 inputs (exact kernel) and
    bf16 inputs (matrix-core kernel's identity path), with and without key
    centering: codes and metadata equal the oracle bit for bit."""
    rng = np.random.default_rng(100)
    T, H, P = 777, 4, 16
    k = _special_groups(T, H, rng)
    v = _special_groups(T, H, rng) * 3
    if dtype == "bf16":                               # both sides see the same bf16 values
        k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
        v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    mean = (rng.standard_normal((H, 128)) * 0.3).astype(np.float32) if center else None
    num_pages = (T + P - 1) // P + 5
    run_a = np.arange(64) + P * (num_pages - 5)       # 4-aligned consecutive slots (grouped V writes)
    run_b = np.arange(10) + P * (num_pages - 1) + 3   # consecutive but not 4-aligned
    others = np.setdiff1d(np.arange(num_pages * P), np.concatenate([run_a, run_b]))
    slots = rng.permutation(others)[:T].astype(np.int64)
    slots[100:164] = run_a
    slots[300:310] = run_b
    slots[5] = -1                                     # negative slot: token skipped
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    ocache = oracle.Cache(num_pages, P, H)
    oracle.quantize(k, v, ocache, ident, ident, key_mean=mean, clip_k=clip_k, clip_v=clip_v, slot_mapping=slots)
    from decode_attention_int2_amd import kvq
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = kvq.Cache(num_pages, P, H, device=dev)
    gid = kvq.Rotation(kvq.KVQ_ROT_IDENTITY)
    kvq.kvq_quantize(torch.from_numpy(k).to(dev).to(tdt), torch.from_numpy(v).to(dev).to(tdt), cache, gid, gid,
                     key_mean=None if mean is None else torch.from_numpy(mean).to(dev), clip_k=clip_k,
                     clip_v=clip_v, slot_mapping=torch.from_numpy(slots).to(dev))
    torch.cuda.synchronize()
    got = cache.pages.cpu().numpy()
    diff = np.argwhere(got != ocache.pages)
    where = [(int(p), int(h), int(o), "code" if o < 64 * P else "meta") for p, h, o in diff[:8]]
    assert diff.shape[0] == 0, f"{diff.shape[0]} bytes differ (page, head, offset, kind): {where}"


@pytest.mark.parametrize("preset,rot", [("envelope", "sh"), ("gqa32k", "dense"), ("paged16x32k", "sh"),
                                        ("long131k", "dense")])
def test_quantize_end_to_end(dev, preset, rot):
    """Rotation (+ key centering where the preset has it) then quantization:
    cache bytes vs the oracle's own cache write of the same inputs.  fp32
    inputs (exact kernel): bytes equal up to 1e-4.  bf16 inputs (matrix-core
    rotation, fp32 accumulation): every group checked against the oracle's
    rotated values (scale/zero within one fp16 step, codes on their rounding
    interval, rare boundary flips)."""
    w = synthetic.make(preset, dev, tokens=600, num_seqs=2, H=3, Hq=6, d_model=64)
    if preset == "envelope":
        w.rot_k = w.rot_v = w.candidates[3]
    cache = gpu_quantize(w, dev)
    torch.cuda.synchronize()
    ocache = oracle.Cache(w.num_pages, w.page_size, w.H)
    km = None if w.key_mean is None else f32np(w.key_mean)
    slots = w.slot_mapping.cpu().numpy()
    oracle.quantize(f32np(w.k), f32np(w.v), ocache, oracle_rot(w.rot_k), oracle_rot(w.rot_v), key_mean=km,
                    clip_k=w.clip_k, clip_v=w.clip_v, slot_mapping=slots)
    got = cache.pages.cpu().numpy()
    if w.dtype == "f32":
        frac = float(np.mean(got != ocache.pages))
        print(f"{preset}: byte mismatch fraction {frac:.3e}")
        assert frac <= 1e-4
        return
    y = {"k": oracle.rotate(f32np(w.k), oracle_rot(w.rot_k), km), "v": oracle.rotate(f32np(w.v), oracle_rot(w.rot_v))}
    stats = check_rotated_quantization(got, ocache.pages, y, slots, w.page_size)
    print(f"{preset}: (code, meta) mismatch fractions {stats}")


@pytest.mark.parametrize("case", ["envelope_f32_sh", "gqa_bf16_dense_centered", "paged_bf16_sh_ragged",
                                  "t3_bf16_dense_multiquery"])
def test_decode_parity(dev, case):
    if case == "envelope_f32_sh":
        w = synthetic.make("envelope", dev, tokens=1000, queries=3)
        w.rot_k = w.rot_v = w.candidates[5]
        seq_lens = None
    elif case == "gqa_bf16_dense_centered":
        w = synthetic.make("gqa32k", dev, tokens=1500, H=2, Hq=8, d_model=256)
        seq_lens = None
    elif case == "paged_bf16_sh_ragged":
        w = synthetic.make("paged16x32k", dev, tokens=900, num_seqs=5, H=2, Hq=8, d_model=128)
        seq_lens = synthetic.ragged_seq_lens(5, 900, seed=3).to(dev)
    else:
        w = synthetic.make("long131k", dev, tokens=1100, num_seqs=2, H=2, Hq=4, d_model=192, queries=3)
        seq_lens = synthetic.ragged_seq_lens(2, 1100, seed=4).to(dev)
    cache = gpu_quantize(w, dev)
    out_o, out_y = gpu_decode(w, cache, dev, seq_lens=seq_lens)
    _, (ref_o, ref_y) = oracle_cache_and_decode(w, seq_lens=seq_lens)
    tol = tolerance(w)
    eo, ey = rel_l2(f32np(out_o), ref_o), rel_l2(f32np(out_y), ref_y)
    print(f"{case}: rel-L2 out_o {eo:.2e} out_y {ey:.2e} (tol {tol})")
    assert eo <= tol and ey <= tol
    # per (row, head) too, so no small output hides behind a large one
    per = [rel_l2(f32np(out_o)[r, j], ref_o[r, j]) for r in range(ref_o.shape[0]) for j in range(ref_o.shape[1])]
    assert max(per) <= tol


@pytest.mark.parametrize("case", ["gqa8_pair", "odd_groups", "partial_rows", "pair_one_split", "pages64"])
def test_decode_two_row_groups_per_workgroup(dev, case):
    """Decodes with two or more groups of 4 query rows per (sequence, KV
    head).  With 16-token pages one workgroup takes two groups (each block's
    codes unpacked once for both): a full pair (GQA group of 8, one query),
    an odd number of groups (the last workgroup's second group is empty), a
    pair whose second group holds 2 rows, one split (8 rows stored per wave,
    no premerge), and 64-token pages (one group per workgroup).  The oracle
    decodes the GPU's own cache bytes; every (row, head) within 1e-4."""
    splits, seq_lens = 0, None
    if case == "gqa8_pair":
        w = synthetic.make("paged16x32k", dev, tokens=1500, num_seqs=3, H=2, Hq=16, d_model=64)
        seq_lens = synthetic.ragged_seq_lens(3, 1500, seed=21).to(dev)
    elif case == "odd_groups":
        w = synthetic.make("gqa32k", dev, tokens=1300, H=2, Hq=8, d_model=64, queries=3)
    elif case == "partial_rows":
        w = synthetic.make("long131k", dev, tokens=900, num_seqs=2, H=2, Hq=6, d_model=96, queries=2)
        seq_lens = synthetic.ragged_seq_lens(2, 900, seed=22).to(dev)
    elif case == "pair_one_split":
        w = synthetic.make("paged16x32k", dev, tokens=1200, num_seqs=2, H=2, Hq=16, d_model=64)
        splits = 1
    else:
        w = synthetic.make("paged16x32k", dev, tokens=1500, num_seqs=2, H=2, Hq=16, d_model=64, page_size=64)
    if seq_lens is not None:
        w.seq_lens = seq_lens
    print(f"{case}: rows per KV head {w.queries_per_seq * w.Hq // w.H}, page size {w.page_size}", flush=True)
    cache = gpu_quantize(w, dev)
    out_o, _ = gpu_decode(w, cache, dev, with_wo=False, num_splits=splits)
    (ref_o, _), rows = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), range(w.num_seqs), with_wo=False)
    o = f32np(out_o)[rows]
    per = [rel_l2(o[r, j], ref_o[r, j]) for r in range(ref_o.shape[0]) for j in range(ref_o.shape[1])]
    print(f"{case}: max rel-L2 per (row, head) {max(per):.2e}", flush=True)
    assert max(per) <= 1e-4


def test_decode_split_count_invariance(dev):
    """The split-K log-sum-exp merge equals a single pass (one split).

    The matrix-core kernel rounds each value weight to an integer below 2^24
    on a per-split power-of-two scale kept within 2^2 of the running bound, so
    the weights of one split carry >= 2^-20 relative resolution at the
    dominant tokens; two split counts then agree to a few 1e-6 (measured
    1e-5 worst case on these inputs), not to fp32 summation order."""
    w = synthetic.make("paged16x32k", dev, tokens=3000, num_seqs=2, H=2, Hq=8, d_model=64)
    cache = gpu_quantize(w, dev)
    base, _ = gpu_decode(w, cache, dev, with_wo=False, num_splits=1)
    for ns in (0, 3, 12):
        o, _ = gpu_decode(w, cache, dev, with_wo=False, num_splits=ns)
        assert rel_l2(f32np(o), f32np(base)) < 5e-5


def test_decode_premerged_splits_nan_and_parity(dev):
    """More than 8 splits per sequence: the workgroup merges its waves'
    partials first.  Parity with the oracle and NaN confined to the sequence
    with an out-of-range page index (host-forced condition)."""
    w = synthetic.make("paged16x32k", dev, tokens=3000, num_seqs=3, H=2, Hq=8, d_model=64)
    cache = gpu_quantize(w, dev)
    out_o, _ = gpu_decode(w, cache, dev, with_wo=False, num_splits=12)
    (ref_o, _), _ = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), range(3), with_wo=False)
    assert rel_l2(f32np(out_o), ref_o) <= 1e-4
    pt = w.page_table.clone()
    pt[1, 100] = w.num_pages + 3                        # invalid page inside sequence 1
    o2, _ = gpu_decode(w, cache, dev, with_wo=False, num_splits=12, page_table=pt)
    o2 = f32np(o2)
    assert np.all(np.isnan(o2[1]))
    assert rel_l2(o2[[0, 2]], ref_o[[0, 2]]) <= 1e-4


def test_decode_workspace_garbage_then_reuse(dev):
    """The split arrival counters need no zeroed workspace: a workspace full
    of random bytes (first call counts with the tagged compare-and-swap and
    validates the counters), then the same workspace again (fetch-add
    counting), then overwritten with random bytes again."""
    from decode_attention_int2_amd import kvq
    w = synthetic.make("paged16x32k", dev, tokens=3000, num_seqs=3, H=2, Hq=8, d_model=64)
    cache = gpu_quantize(w, dev)
    (ref_o, _), _ = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), range(3), with_wo=False)
    nbytes = kvq.kvq_decode_workspace_bytes(w.num_seqs, 1, w.Hq, w.H, w.tokens, 0, 12)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    g = torch.Generator(device="cpu").manual_seed(11)
    for garbage in (True, False, False, True):
        if garbage:
            ws.copy_(torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8))
        out_o = torch.full((w.num_seqs, w.Hq, 128), 12345.0, dtype=torch.float32, device=dev)
        kvq.kvq_decode_attn(w.q, w.num_seqs, 1, cache, w.page_table, w.page_table.shape[1], w.seq_lens, w.tokens,
                            gpu_rot(w.rot_k), gpu_rot(w.rot_v), out_o, workspace=ws, num_splits=12)
        torch.cuda.synchronize()
        assert rel_l2(f32np(out_o), ref_o) <= 1e-4


def test_decode_workspace_reuse_across_shapes(dev):
    """One workspace buffer shared by decodes of different shapes, whose split
    plans put the partials and the arrival counters at different offsets:
    every call still merges all of its splits (a counter word left by
    another shape's layout is not taken for a count)."""
    from decode_attention_int2_amd import kvq
    wa = synthetic.make("paged16x32k", dev, tokens=3000, num_seqs=3, H=2, Hq=8, d_model=64)
    wb = synthetic.make("paged16x32k", dev, tokens=1500, num_seqs=5, H=2, Hq=4, d_model=64, seed=5)
    plans = [(wa, 12), (wb, 5), (wa, 3), (wb, 20), (wa, 12), (wb, 5)]
    nbytes = max(kvq.kvq_decode_workspace_bytes(w.num_seqs, 1, w.Hq, w.H, w.tokens, 0, n) for w, n in plans)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    refs = {}
    for w in (wa, wb):
        cache = gpu_quantize(w, dev)
        (ro, _), _ = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), range(w.num_seqs), with_wo=False)
        refs[id(w)] = (cache, ro)
    for w, n in plans:
        cache, ro = refs[id(w)]
        out_o = torch.full((w.num_seqs, w.Hq, 128), 12345.0, dtype=torch.float32, device=dev)
        kvq.kvq_decode_attn(w.q, w.num_seqs, 1, cache, w.page_table, w.page_table.shape[1], w.seq_lens, w.tokens,
                            gpu_rot(w.rot_k), gpu_rot(w.rot_v), out_o, workspace=ws, num_splits=n)
        torch.cuda.synchronize()
        e = rel_l2(f32np(out_o), ro)
        print(f"{w.num_seqs} seqs, {n} splits: rel-L2 {e:.2e}", flush=True)
        assert e <= 1e-4


def test_decode_more_units_than_compute_units(dev):
    """80 sequences x 4 KV heads = 320 (sequence, head) units, more than the
    device's compute units: one split each, workgroups in a second round."""
    w = synthetic.make("paged16x32k", dev, tokens=300, num_seqs=80, H=4, Hq=16, d_model=64)
    w.seq_lens = synthetic.ragged_seq_lens(80, 300, 31).to(dev)
    cache = gpu_quantize(w, dev)
    out_o, out_y = gpu_decode(w, cache, dev)
    seqs = [0, 1, 2, 41, 79]
    (ref_o, ref_y), rows = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), seqs)
    eo = rel_l2(f32np(out_o)[rows], ref_o)
    ey = rel_l2(f32np(out_y)[rows], ref_y)
    print(f"320 units: rel-L2 out_o {eo:.2e}, out_y {ey:.2e}", flush=True)
    assert eo <= 1e-4 and ey <= 1e-4


def test_decode_edge_cases(dev):
    """Empty and one-token sequences; an out-of-range page index or seq_len
    gives NaN for that sequence only (host-forced condition)."""
    w = synthetic.make("paged16x32k", dev, tokens=200, num_seqs=4, H=2, Hq=4, d_model=32)
    cache = gpu_quantize(w, dev)
    lens = torch.tensor([0, 1, 200, 57], dtype=torch.int32, device=dev)
    out_o, out_y = gpu_decode(w, cache, dev, seq_lens=lens)
    _, (ref_o, ref_y) = oracle_cache_and_decode(w, seq_lens=lens)
    o = f32np(out_o)
    assert np.all(o[0] == 0.0)
    assert rel_l2(o[1:], ref_o[1:]) <= 2e-2
    pt = w.page_table.clone()
    pt[2, 3] = w.num_pages + 7                         # invalid page inside sequence 2
    bad_lens = lens.clone()
    bad_lens[3] = 10_000                               # beyond max_seq_len
    out_o, out_y = gpu_decode(w, cache, dev, seq_lens=bad_lens, page_table=pt)
    o, y = f32np(out_o), f32np(out_y)
    assert np.all(np.isnan(o[2])) and np.all(np.isnan(o[3])) and np.all(np.isnan(y[2]))
    assert np.all(o[0] == 0.0) and rel_l2(o[1], ref_o[1]) <= 2e-2


@pytest.mark.parametrize("page_size,splits", [(16, 0), (16, 3), (64, 0)])
def test_decode_ignores_slots_and_table_entries_past_the_length(dev, page_size, splits):
    """Positions at or past a sequence's length are never used: their cache
    slots hold 0xFF bytes (codes 3, fp16 NaN metadata) and their page-table
    entries point outside the cache, and the outputs still match the oracle
    reading the valid positions; an empty sequence with a wholly invalid
    table row gives zeros."""
    from decode_attention_int2_amd import kvq
    T = 900
    w = synthetic.make("paged16x32k", dev, tokens=T, num_seqs=4, H=2, Hq=8, d_model=64, page_size=page_size)
    cache = gpu_quantize(w, dev)
    lens = [T, 37, 0, 517]
    w.seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    P = page_size
    pages = cache.pages.cpu().numpy()
    pt = w.page_table.cpu().numpy().copy()
    for b, L in enumerate(lens):
        for p in range(L, T):
            pg, o = pt[b, p // P], p % P
            for lo, width in ((32 * o, 32), (32 * P + 32 * o, 32), (64 * P + 4 * o, 4), (68 * P + 4 * o, 4)):
                pages[pg, :, lo:lo + width] = 0xFF
        first_unused = (L + P - 1) // P
        pt[b, first_unused:] = w.num_pages + 1000 + np.arange(pt.shape[1] - first_unused)
    cache.pages.copy_(torch.from_numpy(pages))
    ptd = torch.from_numpy(pt).to(dev)
    out_o, out_y = gpu_decode(w, cache, dev, page_table=ptd, num_splits=splits)
    w.page_table = ptd
    (ref_o, ref_y), _ = oracle_decode_on_cache(w, pages, range(4))
    o, y = f32np(out_o), f32np(out_y)
    assert np.all(o[2] == 0.0) and np.all(y[2] == 0.0)
    live = [0, 1, 3]
    eo, ey = rel_l2(o[live], ref_o[live]), rel_l2(y[live], ref_y[live])
    per = max(rel_l2(o[r, j], ref_o[r, j]) for r in live for j in range(w.Hq))
    print(f"P={P} splits={splits}: rel-L2 out_o {eo:.2e} (worst head {per:.2e}), out_y {ey:.2e}")
    assert eo <= 1e-4 and per <= 1e-4 and ey <= 1e-4


def test_decode_vector_path_pages_of_48_tokens(dev):
    """A page size that is not a power of two takes the VALU split kernel and
    the separate merge launch, which also clears out_y before the W_O
    projection adds its K slices (d_model 200: two slices, ragged column
    block); out_y starts at 12345 so a row left uncleared fails."""
    w = synthetic.make("paged16x32k", dev, tokens=900, num_seqs=3, H=2, Hq=8, d_model=200, page_size=48)
    w.seq_lens = torch.tensor([900, 433, 47], dtype=torch.int32, device=dev)
    cache = gpu_quantize(w, dev)
    out_o, out_y = gpu_decode(w, cache, dev)
    (ref_o, ref_y), _ = oracle_decode_on_cache(w, cache.pages.cpu().numpy(), range(3))
    eo, ey = rel_l2(f32np(out_o), ref_o), rel_l2(f32np(out_y), ref_y)
    print(f"P=48: rel-L2 out_o {eo:.2e}, out_y {ey:.2e}")
    assert eo <= 1e-4 and ey <= 1e-4


def test_api_rejects_bad_arguments(dev):
    from decode_attention_int2_amd import kvq
    w = synthetic.make("paged16x32k", dev, tokens=64, num_seqs=1, H=2, Hq=4, d_model=32)
    cache = kvq.Cache(w.num_pages, w.page_size, w.H, device=dev)
    rot = gpu_rot(w.rot_k)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_quantize(w.k, w.v, cache, rot, rot, clip_k=1.5)
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARGUMENT
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_quantize(w.k, w.v, cache, kvq.Rotation(9), rot)
    assert e.value.status == kvq.KVQ_ERR_UNSUPPORTED
    out = torch.empty((1, 4, 128), device=dev)
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn(w.q, 1, 1, cache, w.page_table, w.page_table.shape[1], w.seq_lens, 64, rot, rot, out,
                            workspace=small)
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE
    assert torch.all(out == out)  # untouched memory is still readable


def _candidate_case(dev, preset, mode, T, H, Hq, Nq, n_cand, clips, dm, center=False):
    from decode_attention_int2_amd import kvq
    w = synthetic.make(preset, dev, tokens=T, H=H, Hq=Hq, queries=Nq, d_model=dm, num_candidates=n_cand)
    if center:  # calibration mean of the cached keys (input preparation, as the generator does)
        w.key_mean = w.k.to(torch.float64).mean(dim=0).to(torch.float32).contiguous()
    U = 1 if mode == kvq.KVQ_SELECT_JOINT else H
    C, n = len(w.candidates), len(clips)
    out = torch.empty((U, C, n), dtype=torch.float32, device=dev)
    outq = torch.empty((U, C, n, Nq), dtype=torch.float32, device=dev)
    best = torch.empty((U,), dtype=torch.int32, device=dev)
    ws = torch.empty(kvq.kvq_candidate_workspace_bytes(T, H, Hq, Nq, C, n, dm), dtype=torch.uint8, device=dev)
    kvq.kvq_candidate_nmse(w.k, w.v, w.q, [gpu_rot(c) for c in w.candidates], clips, w.w_o, mode, out, best,
                           out_nmse_per_query=outq, key_mean=w.key_mean, workspace=ws)
    torch.cuda.synchronize()
    km = None if w.key_mean is None else f32np(w.key_mean)
    ref, refq, rbest = oracle.candidate_nmse(f32np(w.k), f32np(w.v), f32np(w.q), [oracle_rot(c) for c in w.candidates],
                                             clips, f32np(w.w_o), mode, key_mean=km)
    return f32np(out), f32np(outq), best.cpu().numpy(), ref, refq, rbest




def test_candidate_nmse_joint_envelope(dev):
    from decode_attention_int2_amd import kvq
    clips = list(synthetic.CLIP_GRID)
    got, gotq, best, ref, refq, rbest = _candidate_case(dev, "envelope", kvq.KVQ_SELECT_JOINT, 1024, 4, 4, 1, 9,
                                                        clips, 128)
    rel = np.abs(got - ref) / np.abs(ref)
    print("joint envelope: max NMSE rel diff", rel.max(), "best", best, rbest)
    assert rel.max() <= 1e-3
    assert np.abs(gotq - refq).max() / np.abs(refq).max() <= 1e-3
    check_selection(best, rbest, ref)


def test_candidate_nmse_per_head_dense(dev):
    from decode_attention_int2_amd import kvq
    clips = [1.0, 0.9, 0.8]
    got, gotq, best, ref, refq, rbest = _candidate_case(dev, "calib64k", kvq.KVQ_SELECT_PER_HEAD, 800, 2, 2, 5, 3,
                                                        clips, 96)
    rel = np.abs(got - ref) / np.abs(ref)
    print("per-head dense: max NMSE rel diff", rel.max(), "best", best, rbest)
    assert rel.max() <= 1e-3
    check_selection(best, rbest, ref)


def test_candidate_nmse_per_head_gqa(dev):
    """Per-head units with G = 2 query heads per KV head and centered keys."""
    from decode_attention_int2_amd import kvq
    clips = [1.0, 0.85]
    got, gotq, best, ref, refq, rbest = _candidate_case(dev, "envelope", kvq.KVQ_SELECT_PER_HEAD, 700, 2, 4, 3, 4,
                                                        clips, 64, center=True)
    rel = np.abs(got - ref) / np.abs(ref)
    assert rel.max() <= 1e-3
    check_selection(best, rbest, ref)

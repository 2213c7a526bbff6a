"""Helpers shared by the GPU tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from decode_attention_int2_amd import kvq


def f32np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def gpu_rot(spec) -> kvq.Rotation:
    return kvq.Rotation(spec.kind, signs=spec.signs, matrix=spec.matrix)


def oracle_rot(spec, heads=None) -> oracle.Rotation:
    s = None if spec.signs is None else spec.signs.cpu().numpy()
    m = None if spec.matrix is None else spec.matrix.cpu().numpy()
    if heads is not None:
        s = None if s is None else s[heads]
        m = None if m is None else m[heads]
    return oracle.Rotation(spec.kind, signs=s, matrix=m)


def gpu_quantize(w, dev, rot_k=None, rot_v=None, key_mean="default", clip_k=None, clip_v=None, slot_mapping="default"):
    cache = kvq.Cache(w.num_pages, w.page_size, w.H, device=dev)
    kvq.kvq_quantize(w.k, w.v, cache, gpu_rot(rot_k or w.rot_k), gpu_rot(rot_v or w.rot_v),
                     key_mean=w.key_mean if isinstance(key_mean, str) else key_mean,
                     clip_k=w.clip_k if clip_k is None else clip_k, clip_v=w.clip_v if clip_v is None else clip_v,
                     slot_mapping=w.slot_mapping if isinstance(slot_mapping, str) else slot_mapping)
    return cache


def gpu_decode(w, cache, dev, seq_lens=None, page_table="default", with_wo=True, num_splits=0, max_seq_len=None):
    seq_lens = w.seq_lens if seq_lens is None else seq_lens
    pt = w.page_table if isinstance(page_table, str) else page_table
    max_pages = w.page_table.shape[1]
    msl = w.tokens if max_seq_len is None else max_seq_len
    rows = w.num_seqs * w.queries_per_seq
    out_o = torch.full((rows, w.Hq, 128), 12345.0, dtype=torch.float32, device=dev)
    out_y = torch.full((rows, w.d_model), 12345.0, dtype=torch.float32, device=dev) if with_wo else None
    ws = torch.empty(max(1, kvq.kvq_decode_workspace_bytes(w.num_seqs, w.queries_per_seq, w.Hq, w.H, msl,
                                                           w.d_model if with_wo else 0, num_splits)),
                     dtype=torch.uint8, device=dev)
    kvq.kvq_decode_attn(w.q, w.num_seqs, w.queries_per_seq, cache, pt, max_pages, seq_lens, msl, gpu_rot(w.rot_k),
                        gpu_rot(w.rot_v), out_o, w_o=w.w_o if with_wo else None, out_y=out_y, workspace=ws,
                        num_splits=num_splits)
    torch.cuda.synchronize()
    return out_o, out_y


def oracle_cache_and_decode(w, seq_lens=None, with_wo=True):
    """Oracle path on the same inputs: its own cache write, then decode."""
    seq_lens = w.seq_lens if seq_lens is None else seq_lens
    ocache = oracle.Cache(w.num_pages, w.page_size, w.H)
    ork, orv = oracle_rot(w.rot_k), oracle_rot(w.rot_v)
    km = None if w.key_mean is None else f32np(w.key_mean)
    oracle.quantize(f32np(w.k), f32np(w.v), ocache, ork, orv, key_mean=km, clip_k=w.clip_k, clip_v=w.clip_v,
                    slot_mapping=w.slot_mapping.cpu().numpy())
    res = oracle.decode(f32np(w.q), ocache, seq_lens.cpu().numpy(), ork, orv, num_seqs=w.num_seqs,
                        queries_per_seq=w.queries_per_seq, page_table=w.page_table.cpu().numpy(),
                        max_pages=w.page_table.shape[1], w_o=f32np(w.w_o) if with_wo else None,
                        d_model=w.d_model if with_wo else 0)
    return ocache, res


def tolerance(w) -> float:
    """Float tolerance on rel-L2: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs."""
    return 1e-4 if w.dtype == "f32" else 2e-2


def parse_cache(pages: np.ndarray, slots: np.ndarray, P: int):
    """Codes [T][H][128] and fp16 scale/zero [T][H] of both sides, read from a
    packed cache (uint8 [num_pages][H][72 P]) at the given slots, following
    the layout documented in include/kvq.h."""
    pages = np.asarray(pages)
    page, p = slots // P, slots % P
    blk = pages[page]                                     # [T][H][72 P]
    T, H = blk.shape[0], blk.shape[1]
    shifts = np.array([0, 2, 4, 6], np.uint8)
    kb = np.stack([blk[i, :, 32 * p[i]:32 * p[i] + 32] for i in range(T)])           # [T][H][32]
    vidx = 32 * P + 128 * (p[:, None] // 4) + 4 * np.arange(32)[None, :] + (p[:, None] % 4)
    vb = np.stack([blk[i][:, vidx[i]] for i in range(T)])                              # [T][H][32]
    out = {}
    for name, by, moff in (("k", kb, 64 * P), ("v", vb, 68 * P)):
        codes = ((by[..., None] >> shifts) & 3).reshape(T, H, 128)
        meta = np.stack([blk[i, :, moff + 4 * p[i]:moff + 4 * p[i] + 4] for i in range(T)])
        sb = meta[..., 0].astype(np.uint16) | (meta[..., 1].astype(np.uint16) << 8)
        zb = meta[..., 2].astype(np.uint16) | (meta[..., 3].astype(np.uint16) << 8)
        out[name] = (codes, sb.view(np.float16).astype(np.float64), zb.view(np.float16).astype(np.float64))
    return out


def fp16_spacing(x: np.ndarray) -> np.ndarray:
    """Distance from |x| to the next fp16 value (subnormal spacing at the bottom)."""
    a = np.abs(np.asarray(x, np.float64)).astype(np.float16)
    return np.abs(np.nextafter(a, np.float16(np.inf)).astype(np.float64) - a.astype(np.float64))


def check_rotated_quantization(got_pages, ref_pages, y_ref: dict, slots: np.ndarray, P: int,
                               max_code_mismatch=2e-3, max_meta_mismatch=1e-2):
    """Cache write with a rotation computed in a different rounding order than
    the oracle's fp64 product: fp16 scale and zero may move by one fp16 step
    and codes may differ at rounding boundaries, nothing more.

    y_ref[side]: the oracle's rotated (centered) fp32 values [T][H][128].
    Checks, per group: scale and zero within one fp16 spacing of the oracle's;
    every code is a nearest (or boundary-adjacent) rounding of the oracle's
    value under the cache's own scale and zero; mismatch fractions bounded."""
    keep = slots >= 0
    g = parse_cache(got_pages, slots[keep], P)
    r = parse_cache(ref_pages, slots[keep], P)
    stats = {}
    for side in ("k", "v"):
        cg, sg, zg = g[side]
        cr, sr, zr = r[side]
        y = np.asarray(y_ref[side], np.float64)[keep]
        assert np.all(np.abs(sg - sr) <= fp16_spacing(sr)), f"{side}: scale moved by more than one fp16 step"
        assert np.all(np.abs(zg - zr) <= fp16_spacing(zr)), f"{side}: zero moved by more than one fp16 step"
        pos = sg > 0
        t = np.where(pos[..., None], (y - zg[..., None]) / np.where(pos, sg, 1.0)[..., None], 0.0)
        t = np.clip(t, 0.0, 3.0)
        err = np.abs(t - cg)
        assert np.all(err <= 0.5 + 1e-2), f"{side}: code off its rounding interval by {err.max() - 0.5:.3e}"
        assert np.all(cg[~pos] == 0)
        stats[side] = (float(np.mean(cg != cr)), float(np.mean((sg != sr) | (zg != zr))))
        assert stats[side][0] <= max_code_mismatch, (side, stats[side])
        assert stats[side][1] <= max_meta_mismatch, (side, stats[side])
    return stats


def oracle_decode_on_cache(w, cache_pages: np.ndarray, seqs, with_wo=True):
    """The oracle's decode of the sequences `seqs` of workload w, reading the
    given cache bytes (the GPU's), with the workload's page table: returns
    (out_o [rows][Hq][128], out_y [rows][d_model] or None) for those
    sequences' query rows."""
    seqs = list(seqs)
    oc = oracle.Cache(w.num_pages, w.page_size, w.H)
    oc.pages[...] = cache_pages
    nq = w.queries_per_seq
    rows = np.concatenate([np.arange(s * nq, (s + 1) * nq) for s in seqs])
    q = f32np(w.q)[rows]
    pt = w.page_table.cpu().numpy()[seqs]
    sl = w.seq_lens.cpu().numpy()[seqs]
    res = oracle.decode(q, oc, sl, oracle_rot(w.rot_k), oracle_rot(w.rot_v), num_seqs=len(seqs),
                        queries_per_seq=nq, page_table=pt, max_pages=pt.shape[1],
                        w_o=f32np(w.w_o) if with_wo else None, d_model=w.d_model if with_wo else 0)
    return (res if with_wo else (res, None)), rows


def sampled_quantize_check(w, cache_pages: np.ndarray, n_sample: int, seed: int):
    """Cache write of n_sample seeded tokens, group by group, against the
    oracle's rotation and quantizer of the same tokens (rotated path:
    check_rotated_quantization; fp32 inputs: bytes equal)."""
    rng = np.random.default_rng(seed)
    T = w.k.shape[0]
    idx = np.sort(rng.choice(T, size=min(n_sample, T), replace=False))
    slots = w.slot_mapping.cpu().numpy()[idx]
    k = f32np(w.k[torch.from_numpy(idx).to(w.k.device)])
    v = f32np(w.v[torch.from_numpy(idx).to(w.v.device)])
    km = None if w.key_mean is None else f32np(w.key_mean)
    oc = oracle.Cache(w.num_pages, w.page_size, w.H)
    oracle.quantize(k, v, oc, oracle_rot(w.rot_k), oracle_rot(w.rot_v), key_mean=km, clip_k=w.clip_k,
                    clip_v=w.clip_v, slot_mapping=slots)
    if w.dtype == "f32":
        got = parse_cache(cache_pages, slots, w.page_size)
        ref = parse_cache(oc.pages, slots, w.page_size)
        mism = sum(float(np.mean(got[s][0] != ref[s][0])) for s in ("k", "v")) / 2
        return {"code_mismatch": mism}
    y = {"k": oracle.rotate(k, oracle_rot(w.rot_k), km), "v": oracle.rotate(v, oracle_rot(w.rot_v))}
    return check_rotated_quantization(cache_pages, oc.pages, y, slots, w.page_size)


def check_selection(best, rbest, ref, nmse_rtol: float = 1e-3) -> int:
    """The selected variant per unit equals the oracle's first minimum; a
    different pick is accepted only when the oracle's own objective of the
    GPU's pick lies within the NMSE tolerance of the oracle's minimum (the two
    are then a near-tie that fp32 rounding may order either way).  Returns the
    number of such near-ties (printed)."""
    ties = 0
    for u in range(len(rbest)):
        if int(best[u]) == int(rbest[u]):
            continue
        flat = np.asarray(ref[u], np.float64).ravel()
        gap = (flat[int(best[u])] - flat[int(rbest[u])]) / flat[int(rbest[u])]
        assert gap <= nmse_rtol, (u, int(best[u]), int(rbest[u]), gap)
        ties += 1
        print(f"unit {u}: GPU picked {int(best[u])}, oracle {int(rbest[u])}: near-tie, oracle objectives "
              f"{flat[int(rbest[u])]:.6g} vs {flat[int(best[u])]:.6g} ({gap:.1e} relative)", flush=True)
    print(f"selection: {len(rbest) - ties} of {len(rbest)} units identical, {ties} near-ties", flush=True)
    return ties

"""Seeded synthetic workloads for the rotated INT2 KV-cache hot path.

This module only draws inputs.  It holds none of the method's arithmetic (no
rotation, quantization, attention or error computation) and is shared by the
oracle-side tests, the GPU-side tests, ``bench.py`` and ``__graft_entry__``.

Shapes and value distributions follow the workloads the pages describe: the
4,096-token, 4-KV-head observed envelope of "Output-aware INT2 KV-cache
rotation evaluation" (seed 6260, identity + 8 signed-Hadamard candidates, clip
grid {1.00, 0.95, 0.90, 0.85, 0.80}), and decode shapes of the Qwen3-8B /
Phi4-14B class models of "Output-Aware Rotation for INT2 KV-Cache
Quantization" (GQA 32/8 and 40/10, head_dim 128), with the paper's Appendix
Table A clip ratios (keys 0.96, values 0.92).  No dataset, benchmark item or
model weight is used; every tensor is drawn from a seeded generator.

Conventions (stated readings):
  * N(a, b) has variance b; K, V ~ N(0, 1) per channel; per KV head 4 seeded
    outlier channels are multiplied by 10 (chosen independently for K and V),
    then per-channel key offsets ~ N(0, 2) are added to K only.
  * Student-t(3) = z / sqrt(chi2_3 / 3).
  * Learned rotations are exp(A - A^T), A ~ N(0, 0.01), evaluated in fp64 by
    scipy's scaling-and-squaring Pade expm, then rounded to fp32.
  * Signed-Hadamard candidates are given by their +/-1 sign vectors.
  * The key mean (when centering is on) is the fp64 mean of the cached keys
    of each head, rounded to fp32 (the calibration statistic, estimated from
    the synthetic trace).
  * Paged caches use a seeded permutation of all pages as the page table.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

D = 128
ROT_IDENTITY, ROT_SIGNED_HADAMARD, ROT_DENSE = 0, 1, 2
CLIP_GRID = (1.00, 0.95, 0.90, 0.85, 0.80)

# name -> preset.  "tokens" is per sequence.
PRESETS = {
    "envelope": dict(seed=6260, num_seqs=1, tokens=4096, H=4, Hq=4, d_model=128, dtype="f32", dist="normal",
                     rot="candidates_sh", center=False, page_size=16, paged=False, queries=1 + 10),
    "gqa32k": dict(seed=6261, num_seqs=1, tokens=32768, H=8, Hq=32, d_model=4096, dtype="bf16", dist="normal",
                   rot="dense", center=True, page_size=16, paged=False, queries=1),
    "paged16x32k": dict(seed=6262, num_seqs=16, tokens=32768, H=8, Hq=32, d_model=4096, dtype="bf16",
                        dist="normal", rot="sh", center=False, page_size=16, paged=True, queries=1),
    "long131k": dict(seed=6263, num_seqs=4, tokens=131072, H=10, Hq=40, d_model=5120, dtype="bf16", dist="t3",
                     rot="dense", center=False, page_size=16, paged=False, queries=1),
    "calib64k": dict(seed=6264, num_seqs=1, tokens=65536, H=8, Hq=8, d_model=1024, dtype="bf16", dist="normal",
                     rot="candidates_dense", center=False, page_size=16, paged=False, queries=64),
}
DESCRIPTIONS = {
    "envelope": "observed envelope: 4,096 tokens x 4 KV heads x d128, fp32, W_O [512,128], identity + 8 "
                "signed-Hadamard candidates x 5 clips, joint post-W_O NMSE selection on 1 query, 10 fresh queries",
    "gqa32k": "single-layer GQA decode 32/8 heads, d128, hidden 4096, batch 1 x 32,768 tokens, bf16, learned "
              "rotation per head, keys mean-centered",
    "paged16x32k": "paged batched decode: 16 x 32,768 tokens, 16-token pages, permuted page table, 32/8 heads, "
                   "bf16, signed-Hadamard rotation per head",
    "long131k": "long-context decode 40/10 heads, hidden 5120, 4 x 131,072 tokens, bf16 Student-t(3) K/V, "
                "learned rotation per head, split-K",
    "calib64k": "batched calibration search: 65,536 tokens x 8 KV heads, bf16, 9 learned candidates x 5 clips, "
                "64 queries, W_O [1024,1024], per-head selection",
}


@dataclasses.dataclass
class RotationSpec:
    kind: int
    signs: Optional[torch.Tensor] = None   # int8 [H][128]
    matrix: Optional[torch.Tensor] = None  # fp32 [H][128][128], z' = z R


@dataclasses.dataclass
class Workload:
    name: str
    num_seqs: int
    tokens: int               # per sequence
    H: int
    Hq: int
    d_model: int
    dtype: str                # "f32" or "bf16"
    page_size: int
    k: torch.Tensor           # [num_seqs * tokens][H][128]  (token-major, sequence after sequence)
    v: torch.Tensor
    q: torch.Tensor           # [num_seqs * queries][Hq][128]
    queries_per_seq: int
    w_o: torch.Tensor         # [Hq * 128][d_model]
    rot_k: RotationSpec
    rot_v: RotationSpec
    candidates: list          # list[RotationSpec] (candidate search presets)
    clips: tuple
    clip_k: float
    clip_v: float
    key_mean: Optional[torch.Tensor]  # fp32 [H][128] or None
    num_pages: int
    page_table: torch.Tensor  # int32 [num_seqs][max_pages]
    slot_mapping: torch.Tensor  # int64 [num_seqs * tokens]
    seq_lens: torch.Tensor    # int32 [num_seqs]
    seed: int


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + stream)
    return g


def _to_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == "bf16" else x.to(torch.float32)


def _draw_cache(n_tok: int, H: int, dist: str, g: torch.Generator, device, chunk: int = 1 << 16):
    """Base draws [n_tok][H][128] float32, chunked to bound temporary memory."""
    out = torch.empty((n_tok, H, D), dtype=torch.float32, device=device)
    for s in range(0, n_tok, chunk):
        e = min(n_tok, s + chunk)
        if dist == "normal":
            out[s:e] = torch.randn((e - s, H, D), generator=g, device=device)
        else:  # Student-t(3)
            z = torch.randn((e - s, H, D), generator=g, device=device)
            c = torch.randn((3, e - s, H, D), generator=g, device=device)
            chi2 = (c * c).sum(0)
            out[s:e] = z / torch.sqrt(chi2 / 3.0)
    return out


def _outlier_mask(H: int, g_cpu: torch.Generator, device) -> torch.Tensor:
    """Per-head multipliers: 4 seeded channels x10, others x1."""
    mult = torch.ones((H, D), dtype=torch.float32)
    for h in range(H):
        ch = torch.randperm(D, generator=g_cpu)[:4]
        mult[h, ch] = 10.0
    return mult.to(device)


def learned_rotation(n_heads: int, g_cpu: torch.Generator, sd: float = 0.1) -> torch.Tensor:
    """exp(A - A^T) per head, A ~ N(0, sd^2), fp64 then fp32 [n_heads][128][128]."""
    from scipy.linalg import expm

    mats = []
    for _ in range(n_heads):
        a = torch.randn((D, D), generator=g_cpu, dtype=torch.float64).numpy() * sd
        r = expm(a - a.T)
        err = np.abs(r @ r.T - np.eye(D)).max()
        if err > 1e-12:
            raise RuntimeError(f"expm rotation not orthogonal to 1e-12 (err {err})")
        mats.append(r.astype(np.float32))
    return torch.from_numpy(np.stack(mats))


def sh_signs(n_heads: int, g_cpu: torch.Generator) -> torch.Tensor:
    bits = torch.randint(0, 2, (n_heads, D), generator=g_cpu)
    return (bits * 2 - 1).to(torch.int8)


def make(name: str, device="cpu", tokens: Optional[int] = None, num_seqs: Optional[int] = None,
         H: Optional[int] = None, Hq: Optional[int] = None, d_model: Optional[int] = None,
         queries: Optional[int] = None, seed: Optional[int] = None, page_size: Optional[int] = None,
         num_candidates: Optional[int] = None) -> Workload:
    """Draw one workload.  Overrides shrink a preset for fast tests; the value
    distributions and structure stay those of the preset."""
    p = dict(PRESETS[name])
    seed = p["seed"] if seed is None else seed
    T = p["tokens"] if tokens is None else tokens
    B = p["num_seqs"] if num_seqs is None else num_seqs
    H_ = p["H"] if H is None else H
    Hq_ = p["Hq"] if Hq is None else Hq
    dm = p["d_model"] if d_model is None else d_model
    nq = p["queries"] if queries is None else queries
    P = p["page_size"] if page_size is None else page_size
    dtype = p["dtype"]
    device = torch.device(device)
    g_cpu = _gen(seed, 0, "cpu")
    g_dev = _gen(seed, 1, device)

    n_tok = B * T
    kb = _draw_cache(n_tok, H_, p["dist"], g_dev, device)
    vb = _draw_cache(n_tok, H_, p["dist"], g_dev, device)
    if p["dist"] == "normal":
        kb *= _outlier_mask(H_, g_cpu, device)
        vb *= _outlier_mask(H_, g_cpu, device)
    offsets = (torch.randn((H_, D), generator=g_cpu) * math.sqrt(2.0)).to(device)
    kb += offsets
    k = _to_dtype(kb, dtype)
    del kb
    v = _to_dtype(vb, dtype)
    del vb
    q = _to_dtype(torch.randn((B * nq, Hq_, D), generator=g_dev, device=device), dtype)
    fan_in = Hq_ * D
    w_o = _to_dtype(torch.randn((fan_in, dm), generator=g_dev, device=device) / math.sqrt(fan_in), dtype)

    ident = RotationSpec(ROT_IDENTITY)
    candidates = []
    if p["rot"] == "sh":
        s = sh_signs(H_, g_cpu).to(device)
        rot_k = rot_v = RotationSpec(ROT_SIGNED_HADAMARD, signs=s)
    elif p["rot"] == "dense":
        m = learned_rotation(H_, g_cpu).to(device)
        rot_k = rot_v = RotationSpec(ROT_DENSE, matrix=m)
    elif p["rot"] == "candidates_sh":
        nc = 9 if num_candidates is None else num_candidates
        candidates = [ident] + [RotationSpec(ROT_SIGNED_HADAMARD, signs=sh_signs(H_, g_cpu).to(device))
                                for _ in range(nc - 1)]
        rot_k = rot_v = candidates[min(1, nc - 1)]
    else:  # candidates_dense
        nc = 9 if num_candidates is None else num_candidates
        candidates = [RotationSpec(ROT_DENSE, matrix=learned_rotation(H_, g_cpu).to(device)) for _ in range(nc)]
        rot_k = rot_v = candidates[0]

    key_mean = None
    if p["center"]:
        key_mean = k.to(torch.float64).mean(dim=0).to(torch.float32).contiguous()

    pages_per_seq = (T + P - 1) // P
    num_pages = B * pages_per_seq
    if p["paged"]:
        perm = torch.randperm(num_pages, generator=g_cpu).to(torch.int32)
        page_table = perm.view(B, pages_per_seq).to(device)
    else:
        page_table = torch.arange(num_pages, dtype=torch.int32).view(B, pages_per_seq).to(device)
    t_idx = torch.arange(T, device=device)
    slots = (page_table.to(torch.int64)[:, t_idx // P] * P + (t_idx % P)).reshape(-1)
    seq_lens = torch.full((B,), T, dtype=torch.int32, device=device)
    clips = CLIP_GRID
    clip_k, clip_v = (1.0, 1.0) if p["rot"].startswith("candidates") else (0.96, 0.92)
    return Workload(name=name, num_seqs=B, tokens=T, H=H_, Hq=Hq_, d_model=dm, dtype=dtype, page_size=P,
                    k=k, v=v, q=q, queries_per_seq=nq, w_o=w_o, rot_k=rot_k, rot_v=rot_v, candidates=candidates,
                    clips=clips, clip_k=clip_k, clip_v=clip_v, key_mean=key_mean, num_pages=num_pages,
                    page_table=page_table.contiguous(), slot_mapping=slots.contiguous(), seq_lens=seq_lens,
                    seed=seed)


def ragged_seq_lens(num_seqs: int, max_tokens: int, seed: int, page_size: int = 16) -> torch.Tensor:
    """Seeded ragged lengths in [1, max_tokens], including 1 and a non-multiple of the page size."""
    g = _gen(seed, 7, "cpu")
    lens = torch.randint(1, max_tokens + 1, (num_seqs,), generator=g)
    if num_seqs >= 1:
        lens[0] = 1
    if num_seqs >= 2:
        lens[1] = max(1, max_tokens - (page_size // 2 + 1))
    if num_seqs >= 3:
        lens[2] = max_tokens
    return lens.to(torch.int32)


@dataclasses.dataclass
class TraceSet:
    """Calibration traces of one layer: k, v [num_seqs][max_len][H][128] (zero
    past each length), q [num_seqs][nq][Hq][128] (the queries of each
    sequence's final nq positions), lens (host list)."""
    k: torch.Tensor
    v: torch.Tensor
    q: torch.Tensor
    lens: list


def optr_traces(seed: int, num_seqs: int, min_len: int, max_len: int, H: int, Hq: int, nq: int = 64,
                dtype: str = "bf16") -> TraceSet:
    """Synthetic calibration traces with the decode workloads' distribution
    (K, V ~ N(0,1) per channel, 4 outlier channels per head x10, key offsets
    ~ N(0, 2); queries ~ N(0, 1)) and seeded lengths in [min_len, max_len]
    (the paper keeps calibration sequences of at least 328 tokens)."""
    g = _gen(seed, 11, "cpu")
    lens = torch.randint(min_len, max_len + 1, (num_seqs,), generator=g).tolist()
    L = max(lens)
    k = torch.randn((num_seqs, L, H, D), generator=g) * _outlier_mask(H, g, "cpu")
    v = torch.randn((num_seqs, L, H, D), generator=g) * _outlier_mask(H, g, "cpu")
    k += torch.randn((H, D), generator=g) * math.sqrt(2.0)
    q = torch.randn((num_seqs, nq, Hq, D), generator=g)
    for b, n in enumerate(lens):
        k[b, n:] = 0.0
        v[b, n:] = 0.0
    return TraceSet(k=_to_dtype(k, dtype), v=_to_dtype(v, dtype), q=_to_dtype(q, dtype), lens=lens)


def optr_problem(seed: int, H: int, Hq: int, d_model: int, calib=(6, 328, 700), heldout=(5, 328, 700), nq: int = 64,
                 dtype: str = "bf16") -> dict:
    """A calibration problem: calibration and held-out traces (disjoint draws),
    W_O [Hq*128][d_model] ~ N(0, 1/(Hq*128)), and base rotations R0_K, R0_V
    (fp32 [H][128][128], learned-rotation draws: the method accepts any
    orthogonal initialization)."""
    g = _gen(seed, 12, "cpu")
    fan_in = Hq * D
    return {"calib": optr_traces(seed * 2 + 1, *calib, H, Hq, nq, dtype),
            "heldout": optr_traces(seed * 2 + 2, *heldout, H, Hq, nq, dtype),
            "w_o": _to_dtype(torch.randn((fan_in, d_model), generator=g) / math.sqrt(fan_in), dtype),
            "r0_k": learned_rotation(H, g), "r0_v": learned_rotation(H, g), "nq": nq, "H": H, "Hq": Hq}

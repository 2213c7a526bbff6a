"""OptR offline calibration, the oracle: output-aware key and value rotations
learned through the INT2 path ("Output-Aware Rotation for INT2 KV-Cache
Quantization": §4.1-§4.5, Eq. (11)-(18); Appendix "OptR Algorithm",
Algorithm 1; Appendix "Calibration details" and Table A).

TEST INFRASTRUCTURE ONLY.  Only the test suite may import this module; the
HIP library never does, and this module imports nothing from it.

Precision: fp64 PyTorch CPU ops throughout, except the INT2 quantizer, which
is the C oracle's fp32 sequence (``quantize_dequant_groups``) applied to the
rotated values rounded to fp32.  Gradients come from torch autograd with the
straight-through substitution of Eq. (18) (the quantizer passes the gradient
where the value lies inside its clipping range and blocks it elsewhere); the
optimizer is torch.optim.Adam (Kingma and Ba's algorithm) with its default
betas (0.9, 0.999) and eps 1e-8, as the paper names Adam and no other
setting.

Readings (where the pages leave a step open):
  * Traces: a set of sequences; each has keys and values of every cached
    position and the queries of its final `nq` positions (the paper computes
    the objective over the final 64 query positions, causally: query t
    attends positions s <= t).
  * BF16 windows: for a sequence of length L, positions [0, min(sink, L)) and
    [max(that, L - recent), L) are window tokens: their keys are centered but
    not rotated-and-quantized (rotation leaves their logits unchanged), their
    values are the raw values; the rest is INT2 (the cache-write path).
  * The key mean is the fp64 mean of every cached key of the calibration
    set, per KV head, rounded to fp32 (Algorithm 1: "estimate the key mean
    from D").
  * Losses are means over every (query position, query head) pair of the set
    (the expectation of Eq. (14), (16)); the per-pair post-W_O error is
    ||x W_{O,j}||^2 / d_model with W_{O,j} the query head's 128 rows of W_O
    [Hq*128, d_model] (y = concat(o) W_O).
  * Held-out selection: after every `eval_every` Adam steps the held-out
    objective of the current generator is evaluated; the first minimum over
    these checkpoints is kept (with fewer steps than eval_every, the last
    step is the only checkpoint).
  * The value phase uses the attention of the selected key rotation,
    computed once per set with the quantized keys (Algorithm 1, lines 14-15).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

from . import quantize_dequant_groups

D = 128


@dataclasses.dataclass
class TraceSet:
    """k, v: float32 [num_seqs][max_len][H][128]; q: float32
    [num_seqs][nq][Hq][128] (the queries of the final nq positions);
    lens: the sequence lengths (each >= nq)."""
    k: np.ndarray
    v: np.ndarray
    q: np.ndarray
    lens: List[int]


@dataclasses.dataclass
class Config:
    lambda_k: float = 1.0        # Table A / §5: lambda_K = 1.0
    clip_k: float = 0.96         # Table A
    clip_v: float = 0.92         # Table A
    num_sink: int = 64           # Table A
    num_recent: int = 256        # Table A
    steps: int = 80              # §5, Table A
    lr: float = 0.02             # §5, Table A
    eval_every: int = 20         # Appendix, calibration details


def key_mean(ts: TraceSet) -> np.ndarray:
    """Per-KV-head mean of every cached key of the set (fp64), as fp32 [H][128]."""
    rows = [ts.k[b, :ts.lens[b]].astype(np.float64) for b in range(len(ts.lens))]
    return np.concatenate(rows).mean(axis=0).astype(np.float32)


def _window_range(L: int, cfg: Config):
    lo = min(cfg.num_sink, L)
    hi = max(lo, L - cfg.num_recent)
    return lo, hi


def _q2_ste(z: torch.Tensor, clip: float) -> torch.Tensor:
    """Q2 of each row (a 128-group) of z with the straight-through estimator:
    forward = the dequantized fp32 Q2 of fp32(z); backward = identity where the
    value lies inside the group's clipping range, zero elsewhere (Eq. (18))."""
    if z.shape[0] == 0:
        return z
    zh, m = quantize_dequant_groups(z.detach().numpy().astype(np.float32), clip)
    zh = torch.from_numpy(zh.astype(np.float64))
    m = torch.from_numpy(m.astype(np.float64))
    zm = z * m
    return zm + (zh - zm).detach()


def rotation(a: torch.Tensor, r0: torch.Tensor) -> torch.Tensor:
    """R = R0 exp(A - A^T) (Eq. (11))."""
    return r0 @ torch.linalg.matrix_exp(a - a.T)


def _seq(ts: TraceSet, b: int, h: int, G: int, nq: int):
    L = ts.lens[b]
    k = torch.from_numpy(ts.k[b, :L, h].astype(np.float64))
    v = torch.from_numpy(ts.v[b, :L, h].astype(np.float64))
    q = torch.from_numpy(ts.q[b, :, h * G:(h + 1) * G].astype(np.float64))  # [nq][G][128]
    # query t (of the final nq) sits at position L - nq + t and attends s <= L - nq + t
    pos = torch.arange(L)[None, :]
    qpos = (L - nq + torch.arange(nq))[:, None]
    valid = (pos <= qpos)[:, None, :].expand(nq, G, L)
    return L, k, v, q, valid


def _softmax_logs(logits: torch.Tensor, valid: torch.Tensor) -> torch.Tensor:
    return torch.log_softmax(logits.masked_fill(~valid, -math.inf), dim=-1)


def _effective_keys(kc: torch.Tensor, r: torch.Tensor, L: int, cfg: Config) -> torch.Tensor:
    """Rotated effective keys: Q2((k - mu) R) for INT2 positions (straight-through),
    (k - mu) R for window positions."""
    z = kc @ r
    lo, hi = _window_range(L, cfg)
    return torch.cat([z[:lo], _q2_ste(z[lo:hi], cfg.clip_k), z[hi:]])


def key_attention(ts: TraceSet, h: int, G: int, nq: int, mu: np.ndarray, r_k: torch.Tensor, cfg: Config):
    """The attention of the quantized-key path for each sequence,
    p^K [nq][G][L] (Eq. (12))."""
    out = []
    m = torch.from_numpy(mu[h].astype(np.float64))
    for b in range(len(ts.lens)):
        L, k, v, q, valid = _seq(ts, b, h, G, nq)
        kt = _effective_keys(k - m, r_k, L, cfg)
        logits = (q @ r_k) @ kt.T / math.sqrt(D)
        out.append(torch.exp(_softmax_logs(logits, valid)).detach())
    return out


def _post_wo_err2(x: torch.Tensor, w_o: torch.Tensor, h: int, G: int) -> torch.Tensor:
    """||x_j W_{O,j}||^2 / d_model for x [nq][G][128] -> [nq][G]."""
    d_model = w_o.shape[1]
    e = torch.stack([x[:, g] @ w_o[(h * G + g) * D:(h * G + g + 1) * D] for g in range(G)], dim=1)
    return (e * e).sum(-1) / d_model


def key_loss(a: torch.Tensor, r0: torch.Tensor, ts: TraceSet, h: int, G: int, nq: int, mu: np.ndarray,
             w_o: torch.Tensor, cfg: Config) -> torch.Tensor:
    """L_K of Eq. (14) for KV head h at generator a: the mean over (t, j) of
    KL(p_t || p_t^K) + lambda_K ||e_K||^2 / d_model, with e_K of Eq. (13)
    (values unquantized) and p from the unquantized, unrotated keys."""
    r = rotation(a, r0)
    m = torch.from_numpy(mu[h].astype(np.float64))
    total, count = 0.0, 0
    for b in range(len(ts.lens)):
        L, k, v, q, valid = _seq(ts, b, h, G, nq)
        kt = _effective_keys(k - m, r, L, cfg)
        log_pk = _softmax_logs((q @ r) @ kt.T / math.sqrt(D), valid)
        log_p = _softmax_logs(q @ k.T / math.sqrt(D), valid)
        p, pk = torch.exp(log_p), torch.exp(log_pk)
        kl = torch.where(valid, p * (log_p - log_pk), torch.zeros_like(p)).sum(-1)   # [nq][G]
        e2 = _post_wo_err2((pk - p) @ v, w_o, h, G)
        total = total + (kl + cfg.lambda_k * e2).sum()
        count += nq * G
    return total / count


def value_loss(a: torch.Tensor, r0: torch.Tensor, ts: TraceSet, h: int, G: int, nq: int, p_hat: list,
               w_o: torch.Tensor, cfg: Config) -> torch.Tensor:
    """L_V of Eq. (16) for KV head h at generator a: the mean over (t, j) of
    ||e_V||^2 / d_model, e_V of Eq. (15) under the selected key attention
    p_hat (window values are kept exactly, so they contribute nothing)."""
    r = rotation(a, r0)
    total, count = 0.0, 0
    for b in range(len(ts.lens)):
        L, k, v, q, valid = _seq(ts, b, h, G, nq)
        lo, hi = _window_range(L, cfg)
        vq = _q2_ste(v[lo:hi] @ r, cfg.clip_v) @ r.T
        vt = torch.cat([v[:lo], vq, v[hi:]])
        e2 = _post_wo_err2(p_hat[b] @ (vt - v), w_o, h, G)
        total = total + e2.sum()
        count += nq * G
    return total / count


def calibrate(calib: TraceSet, heldout: TraceSet, num_q_heads: int, nq: int, w_o: np.ndarray, r0_k: np.ndarray,
              r0_v: np.ndarray, cfg: Config = Config(), mu: Optional[np.ndarray] = None) -> dict:
    """Algorithm 1 for every KV head: key mean, key rotation (Adam on L_K,
    held-out selection), then the value rotation under the selected key
    attention (Adam on L_V, held-out selection).

    Returns {"r_k", "r_v": fp64 [H][128][128], "key_mean": fp32 [H][128],
    "log": per head and phase, the training loss of every step (at the
    generator before that step's update), the held-out objective at every
    checkpoint, and the selected checkpoint step}."""
    H = calib.k.shape[2]
    G = num_q_heads // H
    if mu is None:
        mu = key_mean(calib)
    wo = torch.from_numpy(w_o.astype(np.float64))
    checkpoints = [i for i in range(1, cfg.steps + 1) if i % cfg.eval_every == 0] or [cfg.steps]
    out = {"r_k": np.zeros((H, D, D)), "r_v": np.zeros((H, D, D)), "key_mean": mu, "log": []}

    def run(loss_of, r0):
        a = torch.zeros((D, D), dtype=torch.float64, requires_grad=True)
        opt = torch.optim.Adam([a], lr=cfg.lr)
        train, held, best = [], [], None
        for i in range(1, cfg.steps + 1):
            opt.zero_grad()
            loss = loss_of(a, calib_side=True)
            loss.backward()
            opt.step()
            train.append(float(loss.detach()))
            if i in checkpoints:
                with torch.no_grad():
                    hv = float(loss_of(a, calib_side=False))
                held.append(hv)
                if best is None or hv < best[1]:
                    best = (i, hv, a.detach().clone())
        with torch.no_grad():
            r = rotation(best[2], r0)
        return r, {"train": train, "heldout": held, "checkpoints": checkpoints, "selected_step": best[0]}

    for h in range(H):
        r0k = torch.from_numpy(r0_k[h].astype(np.float64))
        r0v = torch.from_numpy(r0_v[h].astype(np.float64))
        rk, key_log = run(lambda a, calib_side: key_loss(a, r0k, calib if calib_side else heldout, h, G, nq, mu, wo,
                                                          cfg), r0k)
        p_cal = key_attention(calib, h, G, nq, mu, rk, cfg)
        p_held = key_attention(heldout, h, G, nq, mu, rk, cfg)
        rv, val_log = run(lambda a, calib_side: value_loss(a, r0v, calib if calib_side else heldout, h, G, nq,
                                                            p_cal if calib_side else p_held, wo, cfg), r0v)
        out["r_k"][h] = rk.numpy()
        out["r_v"][h] = rv.numpy()
        out["log"].append({"key": key_log, "value": val_log})
    return out

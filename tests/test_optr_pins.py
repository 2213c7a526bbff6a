"""Pins of the OptR calibration oracle (oracle/optr.py) against what the
paper and the mathematics fix, without retyping its formulas: the losses at
the base rotation recomputed from the C oracle's quantized cache with
textbook softmax attention (scipy), the straight-through gradient against
finite differences of the same surrogate, the orthogonality of exp(A - A^T),
the closed form of all-window caches, and the held-out selection rule.
("Output-Aware Rotation for INT2 KV-Cache Quantization": §4.1-§4.5, Eq.
(11)-(18); Appendix, Algorithm 1 and calibration details.)"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import synthetic

D = 128


@pytest.fixture(scope="module")
def optr(oracle):
    from oracle import optr as o
    return o


def _problem(seed=3, H=2, Hq=4, dm=96, calib=(2, 200, 260), heldout=(2, 200, 260), nq=16):
    pb = synthetic.optr_problem(seed, H=H, Hq=Hq, d_model=dm, calib=calib, heldout=heldout, nq=nq, dtype="f32")
    return pb


def _ts(optr, s):
    f = lambda t: t.float().numpy()
    return optr.TraceSet(f(s.k), f(s.v), f(s.q), list(s.lens))


def _c_oracle_keys_values(oracle, ts, b, h, mu, r0, clip_k, clip_v):
    """The C oracle's cache write of sequence b, head h (keys centered by mu,
    both sides rotated by r0), read back group by group: the dequantized
    rotated keys and values [L][128] (fp64)."""
    L = ts.lens[b]
    k = np.ascontiguousarray(ts.k[b, :L, h:h + 1])
    v = np.ascontiguousarray(ts.v[b, :L, h:h + 1])
    rot = oracle.Rotation(oracle.ROT_DENSE, matrix=r0[None].astype(np.float32))
    cache = oracle.Cache((L + 15) // 16, 16, 1)
    oracle.quantize(k, v, cache, rot, rot, key_mean=mu[h:h + 1], clip_k=clip_k, clip_v=clip_v)
    out = []
    for side in (0, 1):
        rows = []
        for t in range(L):
            c, sb, zb = oracle.read_group(cache, t, 0, side)
            s, z = np.float32(oracle.f16_bits_to_f32(sb)), np.float32(oracle.f16_bits_to_f32(zb))
            rows.append((c.astype(np.float32) * s + z).astype(np.float64))
        out.append(np.stack(rows))
    return out


def _textbook(ts, b, h, G, nq, rk0, kq_rot, mu, sink, recent):
    """Causal softmax attention of the final nq queries (scipy): the quantized
    key path p^K (rotated queries against the cache's rotated keys; window
    keys centered and rotated in fp64) and the reference p (raw keys)."""
    L = ts.lens[b]
    k = ts.k[b, :L, h].astype(np.float64)
    q = ts.q[b, :, h * G:(h + 1) * G].astype(np.float64)
    lo = min(sink, L)
    hi = max(lo, L - recent)
    kr = (k - mu[h].astype(np.float64)) @ rk0
    keff = np.concatenate([kr[:lo], kq_rot[lo:hi], kr[hi:]])
    pk = np.zeros((nq, G, L))
    p = np.zeros((nq, G, L))
    for t in range(nq):
        n = L - nq + t + 1
        for g in range(G):
            pk[t, g, :n] = scipy.special.softmax((q[t, g] @ rk0) @ keff[:n].T / math.sqrt(D))
            p[t, g, :n] = scipy.special.softmax(q[t, g] @ k[:n].T / math.sqrt(D))
    return pk, p, lo, hi


@pytest.mark.parametrize("sink,recent", [(0, 0), (16, 48)])
def test_losses_at_base_rotation_match_c_oracle_and_textbook_attention(oracle, optr, sink, recent):
    """At A = 0 (R = R0): L_K = mean KL(p || p^K) + lambda ||(p^K - p) V W_j||^2 / d_model
    and L_V = mean ||p^K (V_tilde - V) W_j||^2 / d_model, recomputed from the C
    oracle's quantized cache (pinned by its own tests) with scipy's softmax
    and relative entropy."""
    pb = _problem()
    cal = _ts(optr, pb["calib"])
    H, G, nq = pb["H"], pb["Hq"] // pb["H"], pb["nq"]
    cfg = optr.Config(lambda_k=0.7, clip_k=0.9, clip_v=0.85, num_sink=sink, num_recent=recent)
    mu = optr.key_mean(cal)
    wo = pb["w_o"].double().numpy()
    dm = wo.shape[1]
    for h in range(H):
        r0k = pb["r0_k"][h].double().numpy()
        r0v = pb["r0_v"][h].double().numpy()
        kl_sum, e2k_sum, e2v_sum, n = 0.0, 0.0, 0.0, 0
        pks = []
        for b in range(len(cal.lens)):
            L = cal.lens[b]
            kq, _ = _c_oracle_keys_values(oracle, cal, b, h, mu, r0k.astype(np.float32), cfg.clip_k, cfg.clip_v)
            _, vq = _c_oracle_keys_values(oracle, cal, b, h, mu, r0v.astype(np.float32), cfg.clip_k, cfg.clip_v)
            pk, p, lo, hi = _textbook(cal, b, h, G, nq, r0k, kq, mu, sink, recent)
            pks.append(pk)
            v = cal.v[b, :L, h].astype(np.float64)
            vt = v.copy()
            vt[lo:hi] = vq[lo:hi] @ r0v.T
            for t in range(nq):
                for g in range(G):
                    wj = wo[(h * G + g) * D:(h * G + g + 1) * D]
                    kl_sum += scipy.special.rel_entr(p[t, g], pk[t, g]).sum()
                    e2k_sum += np.sum((((pk[t, g] - p[t, g]) @ v) @ wj) ** 2) / dm
                    e2v_sum += np.sum(((pk[t, g] @ (vt - v)) @ wj) ** 2) / dm
                    n += 1
        a0 = torch.zeros((D, D), dtype=torch.float64)
        lk = float(optr.key_loss(a0, pb["r0_k"][h].double(), cal, h, G, nq, mu, torch.from_numpy(wo), cfg))
        expect_k = (kl_sum + cfg.lambda_k * e2k_sum) / n
        assert abs(lk - expect_k) <= 1e-9 * expect_k, (h, lk, expect_k)
        p_hat = [torch.from_numpy(x) for x in pks]
        lv = float(optr.value_loss(a0, pb["r0_v"][h].double(), cal, h, G, nq, p_hat, torch.from_numpy(wo), cfg))
        expect_v = e2v_sum / n
        assert abs(lv - expect_v) <= 1e-9 * expect_v, (h, lv, expect_v)
        # and the key attention the value phase uses is that same p^K
        pk_or = optr.key_attention(cal, h, G, nq, mu, pb["r0_k"][h].double(), cfg)
        for b in range(len(cal.lens)):
            assert np.abs(pk_or[b].numpy() - pks[b]).max() < 1e-12


def _frozen_ste(optr, monkeypatch, record):
    """Replace the straight-through quantizer by the surrogate frozen at the
    recorded point: value = z * m + r with the mask m and the residual r of
    the recorded call (same call order), so the surrogate's gradient is the
    straight-through gradient at that point."""
    it = iter(record)

    def frozen(z, clip):
        if z.shape[0] == 0:
            return z
        m, r = next(it)
        return z * m + r
    monkeypatch.setattr(optr, "_q2_ste", frozen)


def _record_ste(optr, monkeypatch, record):
    real = optr._q2_ste

    def rec(z, clip):
        out = real(z, clip)
        if z.shape[0]:
            from oracle import quantize_dequant_groups
            zh, m = quantize_dequant_groups(z.detach().numpy().astype(np.float32), clip)
            m = torch.from_numpy(m.astype(np.float64))
            record.append((m, torch.from_numpy(zh.astype(np.float64)) - z.detach() * m))
        return out
    monkeypatch.setattr(optr, "_q2_ste", rec)


@pytest.mark.parametrize("phase", ["key", "value"])
def test_straight_through_gradient_matches_finite_differences(oracle, optr, monkeypatch, phase):
    """The autograd gradient of L_K / L_V in A (through exp(A - A^T), the
    rotations, softmax, KL and the post-W_O error) equals central finite
    differences of the surrogate whose quantizer is frozen at A (Eq. (18):
    the straight-through estimator is that surrogate's gradient)."""
    pb = _problem(seed=4, H=1, Hq=2, dm=64, calib=(2, 150, 190))
    cal = _ts(optr, pb["calib"])
    G, nq = 2, pb["nq"]
    cfg = optr.Config(clip_k=0.9, clip_v=0.9, num_sink=16, num_recent=32)
    mu = optr.key_mean(cal)
    wo = torch.from_numpy(pb["w_o"].double().numpy())
    r0 = pb["r0_k"][0].double()
    g = torch.Generator().manual_seed(17)
    a0 = (torch.randn((D, D), generator=g, dtype=torch.float64) * 0.02)
    p_hat = optr.key_attention(cal, 0, G, nq, mu, optr.rotation(a0 * 0.5, r0), cfg)
    loss = (lambda a: optr.key_loss(a, r0, cal, 0, G, nq, mu, wo, cfg)) if phase == "key" else \
        (lambda a: optr.value_loss(a, r0, cal, 0, G, nq, p_hat, wo, cfg))
    record = []
    with monkeypatch.context() as mp:
        _record_ste(optr, mp, record)
        a = a0.clone().requires_grad_(True)
        lval = loss(a)
        lval.backward()
        grad = a.grad.clone()
    assert torch.allclose(grad, -grad.T, atol=1e-15)          # the loss depends on A - A^T only
    eps = 1e-5
    for i in range(3):
        d = torch.randn((D, D), generator=g, dtype=torch.float64)
        vals = []
        for sgn in (1.0, -1.0):
            with monkeypatch.context() as mp:
                _frozen_ste(optr, mp, record)
                vals.append(float(loss(a0 + sgn * eps * d)))
        fd = (vals[0] - vals[1]) / (2 * eps)
        an = float((grad * d).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3 * float(lval.detach())), (i, fd, an)


def test_generator_exponential_is_orthogonal_and_calibrated_rotations_stay_orthogonal(optr):
    """exp(A - A^T) is orthogonal with determinant +1 (Eq. (11)); the
    calibrated rotations are R0 times such a matrix."""
    g = torch.Generator().manual_seed(5)
    for scale in (0.01, 0.1, 1.0):
        a = torch.randn((D, D), generator=g, dtype=torch.float64) * scale
        e = optr.rotation(a, torch.eye(D, dtype=torch.float64))
        assert float((e @ e.T - torch.eye(D, dtype=torch.float64)).abs().max()) < 1e-12
        assert abs(float(torch.linalg.det(e)) - 1.0) < 1e-10
    pb = _problem(seed=6, H=1, Hq=2, dm=64, calib=(2, 150, 180), heldout=(1, 150, 180))
    res = optr.calibrate(_ts(optr, pb["calib"]), _ts(optr, pb["heldout"]), 2, pb["nq"], pb["w_o"].float().numpy(),
                         pb["r0_k"].numpy(), pb["r0_v"].numpy(),
                         optr.Config(steps=4, eval_every=2, num_sink=16, num_recent=32))
    for side in ("r_k", "r_v"):
        r0 = pb["r0_" + side[-1]][0].double().numpy()
        e = np.linalg.solve(r0, res[side][0])
        assert np.abs(e @ e.T - np.eye(D)).max() < 1e-10


def test_all_window_cache_has_zero_losses(optr):
    """With every position in the BF16 windows nothing is quantized: the key
    attention equals the reference one (centering and rotation leave the
    logits unchanged up to a shift), so L_K = 0, and the values are exact, so
    L_V = 0 (Eq. (13)-(16))."""
    pb = _problem(seed=7, H=1, Hq=2, dm=64, calib=(2, 150, 190))
    cal = _ts(optr, pb["calib"])
    cfg = optr.Config(num_sink=64, num_recent=200)
    mu = optr.key_mean(cal)
    wo = torch.from_numpy(pb["w_o"].double().numpy())
    a = (torch.randn((D, D), generator=torch.Generator().manual_seed(8), dtype=torch.float64) * 0.05)
    a.requires_grad_(True)
    lk = optr.key_loss(a, pb["r0_k"][0].double(), cal, 0, 2, pb["nq"], mu, wo, cfg)
    assert abs(float(lk)) < 1e-12
    p_hat = optr.key_attention(cal, 0, 2, pb["nq"], mu, pb["r0_k"][0].double(), cfg)
    lv = optr.value_loss(a, pb["r0_v"][0].double(), cal, 0, 2, pb["nq"], p_hat, wo, cfg)
    assert float(lv) == 0.0
    lv.backward()
    assert float(a.grad.abs().max()) == 0.0


def test_key_mean_and_checkpoint_selection(optr):
    """The key mean is the mean of every cached key of the calibration set
    (lengths respected); the kept generator is the first minimum of the
    held-out objective over the checkpoints every eval_every steps."""
    pb = _problem(seed=9, H=1, Hq=2, dm=64, calib=(3, 150, 200), heldout=(2, 150, 200))
    cal = _ts(optr, pb["calib"])
    w = np.concatenate([np.ones(n) for n in cal.lens])
    rows = np.concatenate([cal.k[b, :n, 0] for b, n in enumerate(cal.lens)]).astype(np.float64)
    assert np.array_equal(optr.key_mean(cal)[0], np.average(rows, axis=0, weights=w).astype(np.float32))
    res = optr.calibrate(cal, _ts(optr, pb["heldout"]), 2, pb["nq"], pb["w_o"].float().numpy(), pb["r0_k"].numpy(),
                         pb["r0_v"].numpy(), optr.Config(steps=6, eval_every=2, num_sink=16, num_recent=32))
    for phase in ("key", "value"):
        lg = res["log"][0][phase]
        assert lg["checkpoints"] == [2, 4, 6] and len(lg["train"]) == 6
        assert lg["selected_step"] == lg["checkpoints"][int(np.argmin(lg["heldout"]))]

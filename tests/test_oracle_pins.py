"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests retypes the oracle's formulas: each compares the oracle
with a figure the pages print, a closed form, an invariant the paper proves,
a library routine (numpy float16, scipy hadamard) or brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")
D = 128


def _gold():
    with open(GOLD) as f:
        return json.load(f)


# ---------------------------------------------------------------- fp16 metadata
def test_f16_conversion_matches_numpy(oracle):
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(20000).astype(np.float32) * np.float32(30.0))
    vals += list((rng.standard_normal(2000) * 1e-5).astype(np.float32))  # fp16 subnormal range
    # exact midpoints between adjacent fp16 values (ties go to even) and +-1 fp32 ulp around them
    h = np.arange(0, 0x7BFF, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[:-1] + np.nextafter(h[:-1].astype(np.float16), np.float16(np.inf)).astype(np.float64)) / 2)
    for m in mids[::3]:
        m32 = np.float32(m)
        vals += [m32, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf))]
    vals += [np.float32(65504.0), np.float32(-65504.0), np.float32(0.0), np.float32(-0.0), np.float32(2.0 ** -24),
             np.float32(2.0 ** -25), np.float32(3 * 2.0 ** -26), np.float32(65519.99)]
    for x in vals:
        bits = oracle.f32_to_f16_bits(float(x))
        ref = np.array([x], np.float32).astype(np.float16).view(np.uint16)[0]
        assert bits == ref, (x, hex(bits), hex(ref))
        assert oracle.f16_bits_to_f32(bits) == np.float32(np.array([bits], np.uint16).view(np.float16)[0])


def test_f16_overflow_and_nonfinite_are_errors(oracle):
    for x in (65520.0, 1e6, -70000.0):
        with pytest.raises(oracle.OracleError):
            oracle.f32_to_f16_bits(x)
    for x in (float("inf"), float("nan")):
        with pytest.raises(oracle.OracleError):
            oracle.f32_to_f16_bits(x)


# ---------------------------------------------------------------- rotations
def test_sylvester_matches_scipy(oracle):
    for n in (1, 2, 4, 16, 128):
        assert np.array_equal(oracle.sylvester(n), scipy.linalg.hadamard(n).astype(np.float64))


def test_signed_hadamard_orthogonal_and_row_convention(oracle):
    rng = np.random.default_rng(2)
    s = (rng.integers(0, 2, D) * 2 - 1).astype(np.int8)
    r = oracle.rotation_matrix(oracle.ROT_SIGNED_HADAMARD, signs=s)
    assert np.abs(r @ r.T - np.eye(D)).max() < 1e-14
    # z' = z R: rotating the unit vector e_i gives row i = s_i * H[i, :] / sqrt(128)
    hs = scipy.linalg.hadamard(D).astype(np.float64)
    x = np.zeros((D, 1, D), np.float32)
    for i in range(D):
        x[i, 0, i] = 1.0
    out = oracle.rotate(x, oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s[None, :]))
    for i in range(D):
        expect = np.float32(s[i] * hs[i] / math.sqrt(D))
        assert np.array_equal(out[i, 0], expect.astype(np.float32))


def test_dense_rotation_rows_and_learned_orthogonality(oracle):
    import torch
    import synthetic

    g = torch.Generator().manual_seed(3)
    m = synthetic.learned_rotation(2, g).numpy()
    for h in range(2):
        r = oracle.rotation_matrix(oracle.ROT_DENSE, matrix=m[h])
        assert np.abs(r @ r.T - np.eye(D)).max() < 1e-6           # fp32-rounded orthogonal matrix
        sign, _ = np.linalg.slogdet(r)
        assert sign == 1.0                                        # exp(skew) has det +1
    x = np.zeros((D, 2, D), np.float32)
    for i in range(D):
        x[i, :, i] = 1.0
    out = oracle.rotate(x, oracle.Rotation(oracle.ROT_DENSE, matrix=m))
    for h in range(2):
        assert np.array_equal(out[:, h, :], m[h])                 # e_i R = row i of R


def test_rotation_preserves_attention_and_centering_is_softmax_invariant(oracle):
    """Eq. (24) of the paper: (qR)((k-mu)R)^T = q(k-mu)^T, and subtracting mu
    from every key shifts all logits of a query by one constant (section 4.1)."""
    rng = np.random.default_rng(4)
    T, H, Hq = 64, 2, 4
    k = rng.standard_normal((T, H, D)).astype(np.float32) + 3.0
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    q = rng.standard_normal((3, Hq, D)).astype(np.float32)
    mu = rng.standard_normal((H, D)).astype(np.float32)
    s = (rng.integers(0, 2, (H, D)) * 2 - 1).astype(np.int8)
    rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s)
    base = oracle.attention_ref(q, k, v)
    kc = oracle.rotate(k, rot, mean=mu)
    vr = oracle.rotate(v, rot)
    # queries use the rotation of their KV head (G = 2)
    qr = np.zeros_like(q)
    for j in range(Hq):
        qr[:, j:j + 1, :] = oracle.rotate(q[:, j:j + 1, :], oracle.Rotation(oracle.ROT_SIGNED_HADAMARD,
                                                                            signs=s[j // 2:j // 2 + 1]))
    out = oracle.attention_ref(qr, kc, vr)
    # bring o' back: o = o' R^T per head
    for j in range(Hq):
        r = oracle.rotation_matrix(oracle.ROT_SIGNED_HADAMARD, signs=s[j // 2])
        out[:, j, :] = out[:, j, :] @ r.T
    assert np.abs(out - base).max() < 1e-5


# ---------------------------------------------------------------- quantizer
def _levels(sb, zb, oracle):
    s, z = oracle.f16_bits_to_f32(sb), oracle.f16_bits_to_f32(zb)
    return s, z, np.array([np.float32(np.float32(c) * np.float32(s) + np.float32(z)) for c in range(4)])


def test_quantizer_brute_force_tiny_groups(oracle):
    """Each code is the nearest of the 4 levels (brute force), and exhaustive
    search over all 4^n code vectors reaches the same total squared error."""
    rng = np.random.default_rng(5)
    import itertools
    for trial in range(300):
        n = int(rng.integers(2, 7))
        x = (rng.standard_normal(n) * rng.choice([0.01, 1.0, 20.0])).astype(np.float32)
        clip = float(rng.choice([1.0, 0.95, 0.9, 0.85, 0.8]))
        codes, sb, zb = oracle.quantize_group(x, clip)
        s, z, lv = _levels(sb, zb, oracle)
        assert s > 0
        for i in range(n):
            d = np.abs(x[i].astype(np.float64) - lv.astype(np.float64))
            best = d.min()
            # the chosen level is a nearest one (ties within fp32 rounding of t may go either way)
            assert d[codes[i]] <= best + 4e-7 * max(abs(s), 1e-30) * 8 + 1e-12, (trial, i, codes, d)
        err = ((x.astype(np.float64) - lv[codes].astype(np.float64)) ** 2).sum()
        brute = min(((x.astype(np.float64) - lv[list(c)].astype(np.float64)) ** 2).sum()
                    for c in itertools.product(range(4), repeat=n))
        assert err <= brute * (1 + 1e-9) + 1e-12


def test_quantizer_range_and_endpoints(oracle):
    """With c = 1 the minimum maps to code 0 and the maximum to code 3; the
    levels span [c*min, c*max] up to fp16 rounding; every value inside the
    clipped range is within s/2 of its level (plain per-group INT2 of the
    paper's Appendix B naive baseline when c = 1)."""
    rng = np.random.default_rng(6)
    for trial in range(200):
        x = (rng.standard_normal(D) * 3 + rng.standard_normal() * 5).astype(np.float32)
        x[rng.integers(0, D, 3)] *= 10
        clip = float(rng.choice([1.0, 0.96, 0.92, 0.8]))
        codes, sb, zb = oracle.quantize_group(x, clip)
        s, z, lv = _levels(sb, zb, oracle)
        lo, hi = np.float64(clip) * x.min(), np.float64(clip) * x.max()
        assert abs(lv[0] - lo) <= 2 ** -10 * abs(lo) + 2 ** -24
        assert abs(lv[3] - hi) <= 3 * 2 ** -10 * (hi - lo) + 2 ** -10 * abs(lo) + 2 ** -22
        if clip == 1.0:
            assert codes[np.argmin(x)] == 0 and codes[np.argmax(x)] == 3
        inside = (x >= lv[0]) & (x <= lv[3])
        assert np.all(np.abs(x[inside] - lv[codes[inside]]) <= s / 2 * (1 + 1e-5))
        assert np.all(codes[x < lv[0]] == 0) and np.all(codes[x > lv[3]] == 3)


def test_quantizer_degenerate_group(oracle):
    codes, sb, zb = oracle.quantize_group(np.full(D, 1.25, np.float32), 1.0)
    assert oracle.f16_bits_to_f32(sb) == 0.0 and np.all(codes == 0)
    assert oracle.f16_bits_to_f32(zb) == np.float32(1.25)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_group(np.array([1.0, np.nan], np.float32), 1.0)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_group(np.array([0.0, 2e6], np.float32), 1.0)


# ---------------------------------------------------------------- packed layout + page figures
def test_packed_payload_matches_page_figure(oracle):
    g = _gold()["packed_payload"]
    T, H = g["tokens"], g["kv_heads"]
    P = 16
    cache = oracle.Cache((T + P - 1) // P, P, H)
    rng = np.random.default_rng(7)
    k = rng.standard_normal((T, H, D)).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    oracle.quantize(k, v, cache, ident, ident)
    code_bytes = cache.pages[:, :, :64 * P].size
    meta_bytes = cache.pages[:, :, 64 * P:].size
    assert code_bytes == g["packed_kv_bytes"] == T * H * 2 * g["head_dim"] * 2 // 8
    assert meta_bytes == T * H * 2 * 4 == 131072


def test_bits_per_element_pins_fp16_scale_and_zero():
    g = _gold()["bits_per_element"]
    n, w = g["context_tokens"], g["sink_tokens"] + g["recent_tokens"]
    for meta_bits, expect_match in ((32, True), (24, False), (16, False)):
        bpe = ((n - w) * (2 + meta_bits / g["group_size"]) + w * 16) / n
        assert (round(bpe, 2) == g["bpe_printed"]) == expect_match


def test_layout_bytes_follow_header_definition(oracle):
    """Byte placement restated from the C-ABI header: K token-major, V four
    tokens interleaved, dim 4m+e of a byte in bits 2e."""
    P, H = 8, 2
    cache = oracle.Cache(2, P, H)
    rng = np.random.default_rng(8)
    k = rng.standard_normal((5, H, D)).astype(np.float32)
    v = rng.standard_normal((5, H, D)).astype(np.float32)
    slots = np.array([0, 3, 9, 14, 6], np.int64)
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    oracle.quantize(k, v, cache, ident, ident, slot_mapping=slots)
    for t, slot in enumerate(slots):
        page, p = divmod(int(slot), P)
        for h in range(H):
            blk = cache.pages[page, h]
            for kv, x in ((0, k), (1, v)):
                codes, sb, zb = oracle.quantize_group(x[t, h], 1.0)
                for i in range(D):
                    m, e = divmod(i, 4)
                    off = 32 * p + m if kv == 0 else 32 * P + 128 * (p // 4) + 4 * m + p % 4
                    assert (blk[off] >> (2 * e)) & 3 == codes[i]
                mo = (64 if kv == 0 else 68) * P + 4 * p
                assert int(blk[mo]) | (int(blk[mo + 1]) << 8) == sb and int(blk[mo + 2]) | (int(blk[mo + 3]) << 8) == zb


# ---------------------------------------------------------------- decode special cases
def _lossless_values(oracle, rng, T, H, rot):
    """Rotated values that quantize exactly: v' = code * s + z with fp16 s, z;
    v = v' R^T (fp64 -> fp32).  Rotating v again lands within ~1e-6 of v'."""
    vr = np.zeros((T, H, D), np.float64)
    for t in range(T):
        for h in range(H):
            c = rng.integers(0, 4, D)
            c[0], c[1] = 0, 3
            s = np.float16(rng.uniform(0.5, 2.0)).astype(np.float64)
            z = np.float16(rng.uniform(-3, 0)).astype(np.float64)
            vr[t, h] = c * s + z
    v = np.zeros_like(vr)
    for h in range(H):
        r = oracle.rotation_matrix(rot.kind, signs=None if rot.signs is None else rot.signs[h],
                                   matrix=None if rot.matrix is None else rot.matrix[h])
        v[:, h] = vr[:, h] @ r.T
    return v.astype(np.float32), vr


def test_decode_single_token_and_uniform_attention(oracle):
    """T = 1 gives o = v_hat R^T; identical keys give uniform p, o = mean(v_hat) R^T."""
    rng = np.random.default_rng(9)
    H, Hq, P = 2, 4, 16
    s = (rng.integers(0, 2, (H, D)) * 2 - 1).astype(np.int8)
    rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s)
    for T in (1, 37):
        k = np.repeat(rng.standard_normal((1, H, D)).astype(np.float32), T, axis=0)
        v, _ = _lossless_values(oracle, rng, T, H, rot)
        cache = oracle.Cache((T + P - 1) // P, P, H)
        oracle.quantize(k, v, cache, rot, rot)
        q = rng.standard_normal((1, Hq, D)).astype(np.float32)
        o = oracle.decode(q, cache, [T], rot, rot, num_seqs=1, max_pages=cache.num_pages, f64=True)
        for j in range(Hq):
            h = j // 2
            vh = np.stack([(lambda c, sb, zb: np.array([oracle.f16_bits_to_f32(sb) * np.float32(ci) for ci in c],
                                                       np.float32) + np.float32(oracle.f16_bits_to_f32(zb)))(
                *oracle.read_group(cache, t, h, 1)) for t in range(T)]).astype(np.float64)
            r = oracle.rotation_matrix(oracle.ROT_SIGNED_HADAMARD, signs=s[h])
            expect = vh.mean(axis=0) @ r.T
            assert np.abs(o[0, j] - expect).max() < 1e-12
            assert np.abs(o[0, j] - v[:, h].astype(np.float64).mean(0)).max() < 1e-5  # lossless values


def test_decode_rotated_query_equals_inverse_rotated_keys(oracle):
    """Appendix Eq. (22)/(26): (q R_K) k_R^T = q (k_R R_K^T)^T.  The oracle's
    decode (rotated-query form) matches softmax attention computed here with
    inverse-rotated dequantized keys and the unrotated query."""
    rng = np.random.default_rng(10)
    T, H, Hq, P = 40, 2, 2, 8
    import torch
    import synthetic
    m = synthetic.learned_rotation(H, torch.Generator().manual_seed(11)).numpy()
    rot = oracle.Rotation(oracle.ROT_DENSE, matrix=m)
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    k = (rng.standard_normal((T, H, D)) * 2).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    cache = oracle.Cache((T + P - 1) // P, P, H)
    oracle.quantize(k, v, cache, rot, ident, clip_k=0.96, clip_v=0.92)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    o = oracle.decode(q, cache, [T], rot, ident, num_seqs=1, max_pages=cache.num_pages, f64=True)
    for j in range(Hq):
        h = j
        kh, vh = [], []
        for t in range(T):
            for kv, dst in ((0, kh), (1, vh)):
                c, sb, zb = oracle.read_group(cache, t, h, kv)
                dst.append(np.array([np.float32(np.float32(ci) * np.float32(oracle.f16_bits_to_f32(sb)))
                                     + np.float32(oracle.f16_bits_to_f32(zb)) for ci in c], np.float32))
        kt = np.stack(kh).astype(np.float64) @ m[h].astype(np.float64).T   # k~ = k_R R^T
        logits = kt @ q[0, j].astype(np.float64) / math.sqrt(D)
        p = np.exp(logits - logits.max())
        p /= p.sum()
        assert np.abs(o[0, j] - p @ np.stack(vh).astype(np.float64)).max() < 1e-9


def test_value_fold_identity(oracle):
    """Appendix Eq. (28)-(31): o' R_V^T W_O-block equals o' (R_V^T W_O-block);
    decode with R_V equals decode without the inverse rotation followed by the
    folded weight matrix."""
    rng = np.random.default_rng(12)
    T, H, Hq, P, dm = 33, 2, 4, 16, 24
    s = (rng.integers(0, 2, (H, D)) * 2 - 1).astype(np.int8)
    rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s)
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    k = rng.standard_normal((T, H, D)).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    w = (rng.standard_normal((Hq * D, dm)) / 20).astype(np.float32)
    cache = oracle.Cache((T + P - 1) // P, P, H)
    oracle.quantize(k, v, cache, rot, rot)
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    o, y = oracle.decode(q, cache, [T], rot, rot, num_seqs=1, queries_per_seq=2, max_pages=cache.num_pages,
                         w_o=w, d_model=dm)
    o_rot = oracle.decode(q, cache, [T], rot, ident, num_seqs=1, queries_per_seq=2, max_pages=cache.num_pages,
                          f64=True)
    y_fold = np.zeros((2, dm))
    for j in range(Hq):
        r = oracle.rotation_matrix(oracle.ROT_SIGNED_HADAMARD, signs=s[j // 2])
        y_fold += o_rot[:, j] @ (r.T @ w[j * D:(j + 1) * D].astype(np.float64))
    assert np.abs(y - y_fold).max() < 1e-4 * np.abs(y_fold).max()


def test_key_induced_error_decomposition(oracle):
    """Section 3.2 Eq. (8): with lossless values the output error is exactly
    the key-induced term (sum_s dp_s v_s) W_O^T, computed here from the
    dequantized keys independently of the oracle's decode."""
    rng = np.random.default_rng(13)
    T, H, Hq, P, dm = 24, 1, 2, 8, 16
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    k = (rng.standard_normal((T, H, D)) * 1.5).astype(np.float32)
    v, _ = _lossless_values(oracle, rng, T, H, ident)
    w = (rng.standard_normal((Hq * D, dm)) / 10).astype(np.float32)
    cache = oracle.Cache((T + P - 1) // P, P, H)
    oracle.quantize(k, v, cache, ident, ident, clip_k=0.9)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    _, y_hat = oracle.decode(q, cache, [T], ident, ident, num_seqs=1, max_pages=cache.num_pages, w_o=w, d_model=dm)
    o_ref = oracle.attention_ref(q, k, v)
    y_ref = o_ref.reshape(1, -1) @ w.astype(np.float64)
    dk = np.stack([(lambda c, sb, zb: c.astype(np.float32) * np.float32(oracle.f16_bits_to_f32(sb))
                    + np.float32(oracle.f16_bits_to_f32(zb)))(*oracle.read_group(cache, t, 0, 0)) for t in range(T)])
    y_k = np.zeros(dm)
    for j in range(Hq):
        lt = dk.astype(np.float64) @ q[0, j].astype(np.float64) / math.sqrt(D)
        l0 = k[:, 0].astype(np.float64) @ q[0, j].astype(np.float64) / math.sqrt(D)
        pt, p0 = np.exp(lt - lt.max()), np.exp(l0 - l0.max())
        pt, p0 = pt / pt.sum(), p0 / p0.sum()
        y_k += ((pt - p0) @ v[:, 0].astype(np.float64)) @ w[j * D:(j + 1) * D].astype(np.float64)
    assert np.abs((y_hat[0] - y_ref[0]) - y_k).max() < 1e-4 * max(1e-3, np.abs(y_k).max())


# ---------------------------------------------------------------- candidate search
def test_candidate_nmse_zero_when_lossless_and_scale_invariant(oracle):
    rng = np.random.default_rng(14)
    T, H, Hq, dm = 20, 1, 1, 8
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    k, _ = _lossless_values(oracle, rng, T, H, ident)
    v, _ = _lossless_values(oracle, rng, T, H, ident)
    q = rng.standard_normal((3, Hq, D)).astype(np.float32)
    w = rng.standard_normal((Hq * D, dm)).astype(np.float32)
    nm, nq, best = oracle.candidate_nmse(k, v, q, [ident], [1.0], w, oracle.SELECT_JOINT)
    assert nm[0, 0, 0] < 1e-12
    k2 = rng.standard_normal((T, H, D)).astype(np.float32)
    a, _, _ = oracle.candidate_nmse(k2, v, q, [ident], [1.0, 0.8], w, oracle.SELECT_JOINT)
    b, _, _ = oracle.candidate_nmse(k2, v, q, [ident], [1.0, 0.8], w * 4, oracle.SELECT_JOINT)
    assert np.allclose(a, b, rtol=1e-12) and a.max() > 1e-6
    # per-head with one KV head and G = 1 is the joint objective
    c, _, _ = oracle.candidate_nmse(k2, v, q, [ident], [1.0, 0.8], w, oracle.SELECT_PER_HEAD)
    assert np.allclose(a, c, rtol=1e-12)


# ---------------------------------------------------------------- candidate search: closed forms
def _dequant_group(oracle, x, clip):
    """x_hat of one 128-group through the oracle's quantizer (pinned above by
    brute force), widened to fp64."""
    codes, sb, zb = oracle.quantize_group(x, clip)
    s, z = np.float32(oracle.f16_bits_to_f32(sb)), np.float32(oracle.f16_bits_to_f32(zb))
    return (codes.astype(np.float32) * s + z).astype(np.float64)


def _constant_value_case(rng, T, H, G, dm, zero_block=None):
    """Every token of KV head h carries the same value vector u_h, so the
    softmax weights sum the same vector: o = u_h for any keys and queries, in
    the full-precision readout, and o_hat = u_hat_h (one quantized group) in
    the quantized one [OptR, §3 Eq. (1)-(2)]."""
    Hq = H * G
    u = rng.standard_normal((H, D)).astype(np.float32)
    u[:, :4] *= 8.0                                  # outliers: the INT2 error is large
    k = (rng.standard_normal((T, H, D)) * 2).astype(np.float32)
    v = np.broadcast_to(u[None], (T, H, D)).copy()
    q = rng.standard_normal((3, Hq, D)).astype(np.float32)
    w = rng.standard_normal((Hq * D, dm)).astype(np.float32)
    for j in range(Hq):                               # head blocks of very different scale
        w[j * D:(j + 1) * D] *= np.float32(3.0 ** j)
    if zero_block is not None:
        w[zero_block * D:(zero_block + 1) * D] = 0.0
    return k, v, q, w, u


def test_candidate_nmse_constant_values_closed_form(oracle):
    """NMSE = ||(u_hat - u) W||^2 / ||u W||^2 with the denominator on the
    full-precision output ([Eval]: NMSE against the unquantized output; [OptR]
    §3.2 Eq. (10)); per KV head the squared errors and the squared norms of
    its query heads are pooled before the ratio; joint mode sums the heads'
    contributions y = sum_j o_j W_j before the norms (Eq. (3))."""
    rng = np.random.default_rng(21)
    T, H, G, dm = 40, 2, 2, 24
    k, v, q, w, u = _constant_value_case(rng, T, H, G, dm)
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    clips = [1.0, 0.7]
    w64 = w.astype(np.float64)
    blk = [w64[j * D:(j + 1) * D] for j in range(H * G)]
    for mode in (oracle.SELECT_PER_HEAD, oracle.SELECT_JOINT):
        nm, nq, _ = oracle.candidate_nmse(k, v, q, [ident], clips, w, mode)
        for ci, c in enumerate(clips):
            uh = np.stack([_dequant_group(oracle, u[h], c) for h in range(H)])
            du = uh - u.astype(np.float64)
            if mode == oracle.SELECT_PER_HEAD:
                for h in range(H):
                    js = range(h * G, (h + 1) * G)
                    num = sum(float(np.sum((du[h] @ blk[j]) ** 2)) for j in js)
                    den = sum(float(np.sum((u[h].astype(np.float64) @ blk[j]) ** 2)) for j in js)
                    expect = num / den
                    assert abs(nm[h, 0, ci] - expect) <= 1e-9 * expect
                    assert np.allclose(nq[h, 0, ci], expect, rtol=1e-9)
                    # the pins discriminate: the prediction's norm and the mean of per-head ratios differ
                    den_hat = sum(float(np.sum((uh[h] @ blk[j]) ** 2)) for j in js)
                    ratios = [float(np.sum((du[h] @ blk[j]) ** 2) / np.sum((u[h].astype(np.float64) @ blk[j]) ** 2))
                              for j in js]
                    assert abs(num / den_hat - expect) > 1e-4 * expect
                    assert abs(np.mean(ratios) - expect) > 1e-3 * expect
            else:
                dy = sum(du[j // G] @ blk[j] for j in range(H * G))
                y = sum(u[j // G].astype(np.float64) @ blk[j] for j in range(H * G))
                expect = float(np.sum(dy ** 2) / np.sum(y ** 2))
                assert abs(nm[0, 0, ci] - expect) <= 1e-9 * expect
                sep = sum(float(np.sum((du[j // G] @ blk[j]) ** 2)) for j in range(H * G)) / \
                    sum(float(np.sum((u[j // G].astype(np.float64) @ blk[j]) ** 2)) for j in range(H * G))
                assert abs(sep - expect) > 1e-4 * expect   # joint is not the pooled per-head sum


def test_candidate_nmse_zero_wo_block_is_pooled_not_averaged(oracle):
    """A query head whose W_O block is zero contributes nothing to the
    post-W_O output: the per-head objective of its KV head is the other query
    head's ratio alone (a mean of per-query-head ratios would divide 0 by 0)."""
    rng = np.random.default_rng(22)
    T, H, G, dm = 24, 1, 2, 16
    k, v, q, w, u = _constant_value_case(rng, T, H, G, dm, zero_block=1)
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    nm, _, _ = oracle.candidate_nmse(k, v, q, [ident], [0.8], w, oracle.SELECT_PER_HEAD)
    du = _dequant_group(oracle, u[0], 0.8) - u[0].astype(np.float64)
    w0 = w[:D].astype(np.float64)
    expect = float(np.sum((du @ w0) ** 2) / np.sum((u[0].astype(np.float64) @ w0) ** 2))
    assert np.isfinite(nm[0, 0, 0]) and abs(nm[0, 0, 0] - expect) <= 1e-9 * expect


def test_candidate_selection_takes_the_first_minimum(oracle):
    """Exact ties (a candidate listed twice, a clip listed twice) select the
    first of the tied entries in (candidate, clip) order, as numpy's argmin
    over the row-major grid does."""
    rng = np.random.default_rng(23)
    T, H, G, dm = 48, 2, 1, 16
    k = (rng.standard_normal((T, H, D)) * 1.5).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    v[:, :, :3] *= 6.0
    q = rng.standard_normal((2, H * G, D)).astype(np.float32)
    w = rng.standard_normal((H * G * D, dm)).astype(np.float32)
    s = np.where(rng.random((H, D)) < 0.5, -1, 1).astype(np.int8)
    sh = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s)
    clips = [0.85, 0.85, 1.0]
    for mode in (oracle.SELECT_JOINT, oracle.SELECT_PER_HEAD):
        nm, _, best = oracle.candidate_nmse(k, v, q, [sh, sh], clips, w, mode)
        assert np.array_equal(nm[:, 0], nm[:, 1]) and np.array_equal(nm[:, :, 0], nm[:, :, 1])
        for u in range(nm.shape[0]):
            flat = nm[u].reshape(-1)
            assert best[u] == int(np.argmin(flat))
            assert best[u] < len(clips) and best[u] != 1   # candidate 0, and clip 0 over its duplicate


def test_paged_decode_equals_contiguous_decode(oracle):
    """Token t of sequence b is read from page page_table[b][t / P] at
    position t % P (the cache layout of the C header): a permuted page table
    with the tokens written through the matching slots decodes exactly as the
    contiguous layout does, ragged last pages included."""
    rng = np.random.default_rng(24)
    B, H, Hq, P = 3, 2, 4, 16
    lens = [70, 33, 16]
    mp = 5
    s = np.where(rng.random((H, D)) < 0.5, -1, 1).astype(np.int8)
    rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    contig = oracle.Cache(B * mp, P, H)
    perm_pages = 2 * B * mp
    paged = oracle.Cache(perm_pages, P, H)
    table = rng.permutation(perm_pages)[:B * mp].reshape(B, mp).astype(np.int32)
    for b, L in enumerate(lens):
        k = (rng.standard_normal((L, H, D)) * 2).astype(np.float32)
        v = rng.standard_normal((L, H, D)).astype(np.float32)
        t = np.arange(L)
        oracle.quantize(k, v, contig, rot, rot, clip_k=0.9, clip_v=0.95, slot_mapping=b * mp * P + t)
        oracle.quantize(k, v, paged, rot, rot, clip_k=0.9, clip_v=0.95,
                        slot_mapping=table[b, t // P].astype(np.int64) * P + t % P)
    table[1, 3:] = -7          # entries of pages past a sequence's end are never read
    a = oracle.decode(q, contig, lens, rot, rot, num_seqs=B, max_pages=mp, f64=True)
    b2 = oracle.decode(q, paged, lens, rot, rot, num_seqs=B, page_table=table, max_pages=mp, f64=True)
    assert np.array_equal(a, b2)
    # and a wrong page in range changes the result
    bad = table.copy()
    bad[0, [0, 1]] = bad[0, [1, 0]]
    c = oracle.decode(q, paged, lens, rot, rot, num_seqs=B, page_table=bad, max_pages=mp, f64=True)
    assert not np.array_equal(a[0], c[0]) and np.array_equal(a[1:], c[1:])


def test_population_sd_matches_page_figures(oracle):
    g = _gold()["threshold_quality"]
    nq = g["queries"]
    one_pass = np.array([5.0] + [50.0] * (nq - 1))   # 1 of 10 queries under the threshold
    st = oracle.evaluation_stats(one_pass, g["threshold"])
    assert round(st["quality_mean"], 2) == g["no_rotation"]["mean"]
    assert round(st["quality_sd"], 2) == g["no_rotation"]["sd"]          # population sd: 0.30
    st = oracle.evaluation_stats(np.full(nq, 2.0), g["threshold"])
    assert (st["quality_mean"], st["quality_sd"]) == (g["rotation"]["mean"], g["rotation"]["sd"])
    sample_sd = float(np.std(np.r_[1.0, np.zeros(nq - 1)], ddof=1))
    assert round(sample_sd, 2) != g["no_rotation"]["sd"]                 # ddof = 1 would print 0.32


def test_envelope_search_sanity_band(oracle):
    """Parity unpinned (the page's generator is not given): on the envelope
    workload the best signed-Hadamard candidate's NMSE is far below the tuned
    identity's, as in the page's table."""
    import synthetic
    g = _gold()
    w = synthetic.make("envelope", "cpu")
    cands = [oracle.Rotation(c.kind, None if c.signs is None else c.signs.numpy(),
                             None if c.matrix is None else c.matrix.numpy()) for c in w.candidates]
    nm, nq, best = oracle.candidate_nmse(w.k.numpy(), w.v.numpy(), w.q[:1].numpy(), cands,
                                         list(g["search_grid"]["clips"]), w.w_o.numpy(), oracle.SELECT_JOINT)
    ident_best = nm[0, 0].min()
    sh_best = nm[0, 1:].min()
    assert nm.shape == (1, 9, 5)
    assert sh_best * 3 < ident_best
    assert best[0] >= 5          # a signed-Hadamard candidate wins


# ---------------------------------------------------------------- BF16 sink and recent windows
def test_window_bits_per_element_closed_form(oracle):
    """2.32 bits per element at a 64K context with 64 sink and 256 recent
    BF16 tokens (the paper's section 5, Implementation Details): the oracle's
    count is ((L - 320) * 2.25 + 320 * 16) / L."""
    g = _gold()["bits_per_element"]
    n, s, r = g["context_tokens"], g["sink_tokens"], g["recent_tokens"]
    bpe = oracle.bits_per_element(n, s, r)
    assert bpe == ((n - s - r) * 2.25 + (s + r) * 16.0) / n == 151856 / 65536
    assert round(bpe, 2) == g["bpe_printed"]
    assert oracle.bits_per_element(300, s, r) == 16.0      # every token in a window
    assert oracle.bits_per_element(4096, 0, 0) == 2.25    # no windows: codes + fp16 scale and zero


def test_window_bf16_rounding_ties_to_even(oracle):
    bits = oracle.f32_to_bf16_bits(np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 65504.0], np.float32))
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x4780]
    assert oracle.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] & 0x7F80 == 0x7F80


def _textbook_attention(q, k, v):
    """softmax(q k^T / sqrt(128)) v in fp64 for one (query row, head): q [128], k, v [L][128]."""
    x = (k.astype(np.float64) @ q.astype(np.float64)) / math.sqrt(D)
    p = np.exp(x - x.max())
    return (p / p.sum()) @ v.astype(np.float64)


def _bf16_values(oracle, x):
    b = oracle.f32_to_bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32)


def test_windows_only_decode_is_textbook_attention(oracle):
    """A sequence no longer than 64 + 256 tokens is all windows: the decode is
    plain softmax attention over the BF16 keys and values (their centering
    shifts every logit by the same q . mu)."""
    rng = np.random.default_rng(31)
    H, Hq, L = 2, 4, 200
    k = rng.standard_normal((L, H, D)).astype(np.float32)
    v = rng.standard_normal((L, H, D)).astype(np.float32)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    mu = rng.standard_normal((H, D)).astype(np.float32)
    win = oracle.Windows(1, H, 64, 256, key_mean=mu)
    oracle.window_write(k, v, np.zeros(L, np.int32), np.arange(L, dtype=np.int32), win)
    cache = oracle.Cache(13, 16, H)          # never read: no position is an INT2 position
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    o = oracle.decode_windows(q, cache, [L], ident, ident, win, num_seqs=1, max_pages=13)
    kb, vb = _bf16_values(oracle, k), _bf16_values(oracle, v)
    for j in range(Hq):
        ref = _textbook_attention(q[0, j], kb[:, j // 2], vb[:, j // 2])
        assert np.allclose(o[0, j], ref, rtol=1e-12, atol=1e-13)


def _grid_keys_values(rng, T, H, mu):
    """Groups on a 2-bit grid c * s + z (codes 0 and 3 present, dyadic s and z),
    keys shifted by mu (multiples of 1/4): exact in bf16, and the INT2 cache
    write (identity rotation, clip 1, keys centered by mu) reproduces them."""
    def grid():
        g = np.zeros((T, H, D))
        for t in range(T):
            for h in range(H):
                c = rng.integers(0, 4, D)
                c[0], c[1] = 0, 3
                g[t, h] = c * rng.choice([0.25, 0.5]) + rng.choice([-1.0, -0.5, 0.0])
        return g
    return (grid() + mu[None]).astype(np.float32), grid().astype(np.float32)


def test_windows_mixed_decode_lossless_is_textbook_attention(oracle):
    """Sink, INT2 middle and recent ring together, with keys centered by a
    non-zero mean: on grid inputs the INT2 part is exact, so the decode equals
    plain attention over the raw tokens.  The INT2 cache holds only the middle
    positions and each window only its own, so reading a position from the
    wrong store, or leaving the window keys uncentered, changes the result."""
    rng = np.random.default_rng(32)
    H, Hq, P = 2, 4, 16
    lens = [457, 300]                        # INT2 middle [64, 201); all windows
    mp = (max(lens) + P - 1) // P
    mu = rng.integers(-4, 5, (H, D)).astype(np.float64) / 4
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    cache = oracle.Cache(2 * mp, P, H)
    win = oracle.Windows(2, H, 64, 256, key_mean=mu)
    page_table = rng.permutation(2 * mp).astype(np.int32).reshape(2, mp)
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    ks, vs = [], []
    for b, L in enumerate(lens):
        k, v = _grid_keys_values(rng, L, H, mu)
        ks.append(k)
        vs.append(v)
        lo, hi = min(64, L), max(min(64, L), L - 256)
        mid = np.arange(lo, hi)
        if mid.size:
            slots = page_table[b, mid // P].astype(np.int64) * P + mid % P
            oracle.quantize(k[mid], v[mid], cache, ident, ident, key_mean=mu, clip_k=1.0, clip_v=1.0,
                            slot_mapping=slots)
        oracle.window_write(k, v, np.full(L, b, np.int32), np.arange(L, dtype=np.int32), win)
    o = oracle.decode_windows(q, cache, lens, ident, ident, win, num_seqs=2, page_table=page_table, max_pages=mp)
    for b, L in enumerate(lens):
        for j in range(Hq):
            ref = _textbook_attention(q[b, j], ks[b][:, j // 2], vs[b][:, j // 2])
            assert np.allclose(o[b, j], ref, rtol=1e-10, atol=1e-12), (b, j)


def test_windows_of_size_zero_reduce_to_plain_decode(oracle):
    rng = np.random.default_rng(33)
    H, Hq, P, L = 2, 4, 16, 150
    mp = (L + P - 1) // P
    s = (rng.integers(0, 2, (H, D)) * 2 - 1).astype(np.int8)
    rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s)
    k = rng.standard_normal((L, H, D)).astype(np.float32)
    v = rng.standard_normal((L, H, D)).astype(np.float32)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    cache = oracle.Cache(mp, P, H)
    oracle.quantize(k, v, cache, rot, rot, clip_k=0.96, clip_v=0.92)
    ref = oracle.decode(q, cache, [L], rot, rot, num_seqs=1, max_pages=mp, f64=True)
    got = oracle.decode_windows(q, cache, [L], rot, rot, oracle.Windows(1, H, 0, 0), num_seqs=1, max_pages=mp)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- value-rotation folding
def test_fold_identity_rotation_is_a_copy(oracle):
    rng = np.random.default_rng(51)
    w = rng.standard_normal((4 * D, 40)).astype(np.float32)
    out = oracle.fold_value_rotation(w, 2, oracle.Rotation(oracle.ROT_IDENTITY))
    assert np.array_equal(out, w)


def test_fold_preserves_column_norms_per_block(oracle):
    """R_V is orthogonal: every column of every block keeps its norm."""
    rng = np.random.default_rng(52)
    H = 2
    s = (rng.integers(0, 2, (H, D)) * 2 - 1).astype(np.int8)
    w = rng.standard_normal((4 * D, 24)).astype(np.float32)
    out = oracle.fold_value_rotation(w, 2, oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s))
    for b in range(4):
        a = np.linalg.norm(w[b * D:(b + 1) * D].astype(np.float64), axis=0)
        c = np.linalg.norm(out[b * D:(b + 1) * D].astype(np.float64), axis=0)
        assert np.allclose(a, c, rtol=1e-6)


@pytest.mark.parametrize("kind", ["sh", "dense"])
def test_fold_wo_equals_explicit_inverse_rotation(oracle, kind):
    """Eq. (31): decoding with the explicit R_V^T and W_O equals decoding in
    the rotated value domain (identity R_V at decode) with the folded W_O."""
    rng = np.random.default_rng(53)
    T, H, Hq, P, dm = 45, 2, 4, 16, 20
    if kind == "sh":
        rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=(rng.integers(0, 2, (H, D)) * 2 - 1).astype(np.int8))
    else:
        import scipy.linalg
        m = np.stack([scipy.linalg.expm((lambda a: a - a.T)(rng.normal(0, 0.1, (D, D)))) for _ in range(H)])
        rot = oracle.Rotation(oracle.ROT_DENSE, matrix=m.astype(np.float32))
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    k = rng.standard_normal((T, H, D)).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    w = (rng.standard_normal((Hq * D, dm)) / 20).astype(np.float32)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    cache = oracle.Cache((T + P - 1) // P, P, H)
    oracle.quantize(k, v, cache, rot, rot)
    _, y = oracle.decode(q, cache, [T], rot, rot, num_seqs=1, max_pages=cache.num_pages, w_o=w, d_model=dm)
    wf = oracle.fold_value_rotation(w, Hq // H, rot)
    _, y2 = oracle.decode(q, cache, [T], rot, ident, num_seqs=1, max_pages=cache.num_pages, w_o=wf, d_model=dm)
    assert np.allclose(y, y2, rtol=1e-5, atol=1e-6 * np.abs(y).max())


def test_fold_wv_equals_rotating_the_values(oracle):
    """Eq. (30): x W_V-folded^T = (x W_V^T) R_V, with W_V in [H*128][d_in]."""
    rng = np.random.default_rng(54)
    H, din = 2, 48
    s = (rng.integers(0, 2, (H, D)) * 2 - 1).astype(np.int8)
    rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s)
    wv = rng.standard_normal((H * D, din)).astype(np.float32)
    x = rng.standard_normal((5, din)).astype(np.float32)
    v = (x.astype(np.float64) @ wv.astype(np.float64).T).reshape(5, H, D).astype(np.float32)
    vr = oracle.rotate(v, rot)
    wf = oracle.fold_value_rotation(wv, 1, rot)
    vf = (x.astype(np.float64) @ wf.astype(np.float64).T).reshape(5, H, D)
    assert np.allclose(vf, vr, rtol=1e-5, atol=1e-5)


# ---------------------------------------------------------------- causal queries
def test_causal_decode_reduces_to_plain_decode(oracle):
    """The last of a sequence's causal rows, and a single causal row, attend
    the whole sequence: they equal the plain decode.  A row whose prefix is
    one token returns that token's value (v_hat R_V^T)."""
    rng = np.random.default_rng(61)
    H, Hq, P, L, nq = 2, 4, 16, 70, 5
    s = (rng.integers(0, 2, (H, D)) * 2 - 1).astype(np.int8)
    rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=s)
    k = rng.standard_normal((L, H, D)).astype(np.float32)
    v = rng.standard_normal((L, H, D)).astype(np.float32)
    q = rng.standard_normal((nq, Hq, D)).astype(np.float32)
    mp = (L + P - 1) // P
    cache = oracle.Cache(mp, P, H)
    oracle.quantize(k, v, cache, rot, rot)
    causal = oracle.decode_causal(q, cache, [L], rot, rot, num_seqs=1, queries_per_seq=nq, max_pages=mp)
    plain = oracle.decode(q, cache, [L], rot, rot, num_seqs=1, queries_per_seq=nq, max_pages=mp, f64=True)
    assert np.array_equal(causal[nq - 1], plain[nq - 1])
    for qi in range(nq - 1):                 # shorter prefixes differ from the full-cache rows
        assert not np.allclose(causal[qi], plain[qi])
    one = oracle.decode_causal(q[:1], cache, [L], rot, rot, num_seqs=1, queries_per_seq=1, max_pages=mp)
    assert np.array_equal(one[0], plain[0])
    # a 3-row chunk over a 3-token sequence: row 0 attends token 0 only
    tiny = oracle.decode_causal(q[:3], cache, [3], rot, rot, num_seqs=1, queries_per_seq=3, max_pages=mp)
    codes, sb, zb = oracle.read_group(cache, 0, 0, 1)
    vhat = np.array([oracle.f16_bits_to_f32(zb) + c * oracle.f16_bits_to_f32(sb) for c in codes], np.float64)
    r = oracle.rotation_matrix(oracle.ROT_SIGNED_HADAMARD, signs=s[0])
    assert np.allclose(tiny[0, 0], vhat @ r.T, rtol=1e-12, atol=1e-12)
    # a chunk longer than the sequence: its first rows have no token
    none = oracle.decode_causal(q, cache, [2], rot, rot, num_seqs=1, queries_per_seq=nq, max_pages=mp)
    assert np.all(none[:3] == 0.0)

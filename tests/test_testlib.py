"""The cache reader used by the GPU tests agrees with the oracle's own reader."""
import numpy as np

import oracle
from kvq_testlib import fp16_spacing, parse_cache


def test_parse_cache_matches_oracle_reader():
    rng = np.random.default_rng(7)
    T, H, P = 70, 3, 16
    num_pages = 7
    slots = rng.permutation(num_pages * P)[:T].astype(np.int64)
    k = rng.standard_normal((T, H, 128)).astype(np.float32)
    v = rng.standard_normal((T, H, 128)).astype(np.float32)
    cache = oracle.Cache(num_pages, P, H)
    ident = oracle.Rotation(oracle.ROT_IDENTITY)
    oracle.quantize(k, v, cache, ident, ident, clip_k=0.9, clip_v=0.95, slot_mapping=slots)
    got = parse_cache(cache.pages, slots, P)
    for side, kv in (("k", 0), ("v", 1)):
        codes, s, z = got[side]
        for t in range(T):
            for h in range(H):
                c, sb, zb = oracle.read_group(cache, int(slots[t]), h, kv)
                assert np.array_equal(codes[t, h], c)
                assert s[t, h] == oracle.f16_bits_to_f32(sb) and z[t, h] == oracle.f16_bits_to_f32(zb)


def test_fp16_spacing():
    assert fp16_spacing(np.array([1.0]))[0] == 2.0 ** -10
    assert fp16_spacing(np.array([-3.0]))[0] == 2.0 ** -9
    assert fp16_spacing(np.array([0.0]))[0] == 2.0 ** -24

"""The C-ABI library loads on a CPU-only host, exports every symbol that
include/kvq.h declares, and rejects bad arguments on the host before any
launch (no GPU needed: validation never touches the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    hdr = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|int|double|const char \*)\s*(kvq_\w+)\s*\(", hdr, re.M)))


@pytest.fixture(scope="module")
def lib():
    from decode_attention_int2_amd import kvq
    if not os.path.exists(kvq.LIB_PATH):
        from decode_attention_int2_amd import build
        build.build()
    return kvq.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    from decode_attention_int2_amd import kvq
    assert set(kvq.EXPORTED) == set(names)


def test_version_and_status_strings(lib):
    assert lib.kvq_version() == 1
    assert lib.kvq_status_string(0) == b"KVQ_OK"
    assert lib.kvq_status_string(3) == b"KVQ_ERR_WORKSPACE"
    assert lib.kvq_status_string(99) == b"KVQ_UNKNOWN_STATUS"


def test_cache_bytes(lib):
    # 72 bytes per (token, head): 1,152-byte blocks for 16-token pages
    assert lib.kvq_cache_bytes(32768, 16, 8) == 32768 * 8 * 1152
    assert lib.kvq_cache_bytes(-1, 16, 8) == 0


def _rot(kind=0):
    from decode_attention_int2_amd.kvq import _Rot
    return _Rot(kind, None, None)


def _cache(pages=1, P=16, H=2):
    from decode_attention_int2_amd.kvq import _Cache
    return _Cache(ctypes.c_void_p(0x1000), pages, P, H)


def test_quantize_validation(lib):
    f = ctypes.c_float
    ok_rot, c = _rot(), _cache()
    fake = ctypes.c_void_p(0x2000)
    # unknown dtype / rotation kind -> UNSUPPORTED
    assert lib.kvq_quantize(fake, fake, 7, 4, None, ctypes.byref(ok_rot), ctypes.byref(ok_rot), None, f(1), f(1),
                            ctypes.byref(c), None) == 2
    bad_kind = _rot(5)
    assert lib.kvq_quantize(fake, fake, 0, 4, None, ctypes.byref(bad_kind), ctypes.byref(ok_rot), None, f(1), f(1),
                            ctypes.byref(c), None) == 2
    # signed Hadamard without signs, clip out of range, page size not a multiple of 16 -> INVALID
    sh = _rot(1)
    assert lib.kvq_quantize(fake, fake, 0, 4, None, ctypes.byref(sh), ctypes.byref(ok_rot), None, f(1), f(1),
                            ctypes.byref(c), None) == 1
    for clip in (0.0, 1.01, float("nan")):
        assert lib.kvq_quantize(fake, fake, 0, 4, None, ctypes.byref(ok_rot), ctypes.byref(ok_rot), None,
                                f(clip), f(1), ctypes.byref(c), None) == 1
    c8 = _cache(P=8)
    assert lib.kvq_quantize(fake, fake, 0, 4, None, ctypes.byref(ok_rot), ctypes.byref(ok_rot), None, f(1), f(1),
                            ctypes.byref(c8), None) == 1
    # K or V not 16-byte aligned -> INVALID
    odd = ctypes.c_void_p(0x2008)
    assert lib.kvq_quantize(odd, fake, 0, 4, None, ctypes.byref(ok_rot), ctypes.byref(ok_rot), None, f(1), f(1),
                            ctypes.byref(c), None) == 1
    assert lib.kvq_quantize(fake, odd, 1, 4, None, ctypes.byref(ok_rot), ctypes.byref(ok_rot), None, f(1), f(1),
                            ctypes.byref(c), None) == 1
    # dense rotation matrix not 16-byte aligned -> INVALID
    from decode_attention_int2_amd.kvq import _Rot
    bad_dense = _Rot(2, None, 0x2004)
    assert lib.kvq_quantize(fake, fake, 0, 4, None, ctypes.byref(bad_dense), ctypes.byref(ok_rot), None, f(1), f(1),
                            ctypes.byref(c), None) == 1
    # nothing to do: zero tokens succeeds without touching the device
    assert lib.kvq_quantize(None, None, 0, 0, None, ctypes.byref(ok_rot), ctypes.byref(ok_rot), None, f(1), f(1),
                            ctypes.byref(c), None) == 0


def test_decode_validation(lib):
    fake = ctypes.c_void_p(0x2000)
    r, c = _rot(), _cache(pages=4, H=2)
    call = lambda **kw: lib.kvq_decode_attn(
        kw.get("q", fake), kw.get("dtype", 1), kw.get("num_seqs", 1), kw.get("qps", 1), kw.get("hq", 4),
        ctypes.byref(kw.get("cache", c)), kw.get("pt", fake), kw.get("max_pages", 4), fake, kw.get("msl", 64),
        ctypes.byref(r), ctypes.byref(r), kw.get("wo", None), kw.get("dm", 0), fake, kw.get("y", None),
        kw.get("ws", fake), kw.get("wsb", 1 << 30), 0, None, None)
    assert call(dtype=3) == 2
    assert call(hq=3) == 1                      # Hq not a multiple of H
    assert call(qps=40, hq=4) == 2              # 80 rows per KV head > 64
    assert call(msl=65) == 1                    # max_seq_len > max_pages * P
    assert call(pt=None, num_seqs=2) == 1       # contiguous table needs num_seqs * max_pages <= num_pages
    assert call(wo=fake, dm=16, y=None) == 1    # W_O without out_y
    assert call(ws=None) == 3 and call(wsb=8) == 3
    assert call(q=ctypes.c_void_p(0x2004)) == 1                       # q not 16-byte aligned
    assert call(wo=ctypes.c_void_p(0x2002), dm=16, y=fake) == 1       # W_O not 16-byte aligned
    assert call(num_seqs=0) == 0


def test_candidate_validation(lib):
    fake = ctypes.c_void_p(0x2000)
    from decode_attention_int2_amd.kvq import _Rot
    cands = (_Rot * 2)(_Rot(0, None, None), _Rot(1, None, None))
    clips = (ctypes.c_float * 2)(1.0, 0.9)
    call = lambda **kw: lib.kvq_candidate_nmse(
        fake, fake, fake, kw.get("dtype", 1), kw.get("T", 100), 2, 2, kw.get("nq", 4), kw.get("cands", cands),
        kw.get("nc", 2), kw.get("clips", clips), 2, None, fake, 16, kw.get("mode", 0), fake, None, fake,
        fake, 1 << 30, None)
    assert call(mode=5) == 2
    assert call(nq=65) == 2
    assert call() == 1                           # candidate 1 is signed Hadamard without signs
    one = (_Rot * 1)(_Rot(0, None, None))
    bad_clips = (ctypes.c_float * 2)(1.0, 0.0)
    assert call(cands=one, nc=1, clips=bad_clips) == 1
    assert lib.kvq_candidate_workspace_bytes(100, 2, 2, 4, 1, 2, 16) > 0
    # checks that come before any launch, with otherwise valid arguments
    good = (ctypes.c_float * 2)(1.0, 0.9)
    call2 = lambda k=fake, v=fake, q=fake, wo=fake, H=2, Hq=2, nq=4, mode=0: lib.kvq_candidate_nmse(
        k, v, q, 1, 100, H, Hq, nq, one, 1, good, 2, None, wo, 16, mode, fake, None, fake, fake, 1 << 30, None)
    for bad in ("k", "v", "q", "wo"):
        assert call2(**{bad: ctypes.c_void_p(0x2008)}) == 1          # not 16-byte aligned
    assert call2(H=2, Hq=128, nq=1, mode=0) == 2                      # JOINT with more than 64 query heads


def test_window_validation(lib):
    """Window entry points reject bad descriptors before any launch."""
    from decode_attention_int2_amd.kvq import _Windows
    fake = ctypes.c_void_p(0x2000)
    good = _Windows(fake, fake, fake, fake, 2, 2, 64, 256)
    seq = pos = fake
    # window write: unknown dtype, null descriptor, sink not a multiple of 16, too many window tokens,
    # unaligned buffers, negative token count
    assert lib.kvq_window_write(fake, fake, 7, 4, seq, pos, None, ctypes.byref(good), None) == 2
    assert lib.kvq_window_write(fake, fake, 1, 4, seq, pos, None, None, None) == 1
    assert lib.kvq_window_write(fake, fake, 1, 4, seq, pos, None,
                                ctypes.byref(_Windows(fake, fake, fake, fake, 2, 2, 8, 0)), None) == 2
    assert lib.kvq_window_write(fake, fake, 1, 4, seq, pos, None,
                                ctypes.byref(_Windows(fake, fake, fake, fake, 2, 2, 64, 336)), None) == 2
    assert lib.kvq_window_write(fake, fake, 1, 4, seq, pos, None,
                                ctypes.byref(_Windows(ctypes.c_void_p(0x2008), fake, fake, fake, 2, 2, 64, 256)),
                                None) == 1
    assert lib.kvq_window_write(fake, fake, 1, -1, seq, pos, None, ctypes.byref(good), None) == 1
    assert lib.kvq_window_write(None, None, 1, 0, None, None, None, ctypes.byref(good), None) == 0   # nothing to do
    # decode with windows: head count must match the cache, and the windows must cover num_seqs
    c = _cache(pages=4, H=2)
    r = _rot()
    call = lambda w: lib.kvq_decode_attn_windows(fake, 1, 1, 1, 4, ctypes.byref(c), fake, 4, fake, 64, ctypes.byref(r),
                                                 ctypes.byref(r), w, None, None, 0, fake, None, fake, 1 << 30, 0,
                                                 None)
    assert call(None) == 1
    assert call(ctypes.byref(_Windows(fake, fake, fake, fake, 1, 3, 64, 256))) == 1
    assert call(ctypes.byref(_Windows(fake, fake, fake, fake, 1, 2, 40, 0))) == 2            # sink % 16 != 0


def test_bits_per_element_closed_form(lib):
    """2.32 bits per element at 64K with 64 + 256 BF16 tokens (host function)."""
    assert lib.kvq_bits_per_element(65536, 64, 256) == 151856 / 65536
    assert round(lib.kvq_bits_per_element(65536, 64, 256), 2) == 2.32
    assert lib.kvq_bits_per_element(320, 64, 256) == 16.0
    assert lib.kvq_bits_per_element(4096, 0, 0) == 2.25

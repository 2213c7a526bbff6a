"""CPU oracle for rotated INT2 KV-cache quantization and decode attention.

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product path (the
HIP library under ``decode_attention_int2_amd``) never imports this package,
and this package imports nothing from it.

The arithmetic lives in ``kvq_oracle.c`` (plain C, fp64 except the fp32 INT2
quantizer sequence); this module only builds it with gcc and marshals numpy
arrays through ctypes.  Every function cites the passage it follows in the C
source.  Pages cited: "Output-Aware Rotation for INT2 KV-Cache Quantization"
(the paper) and "Output-aware INT2 KV-cache rotation evaluation" (the project
page with the observed 4,096-token envelope).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
# (KVQ_ORACLE_LIB points the loader at another build of the same source, e.g.
# the sanitizer build of the test suite)
_LIB_PATH = os.environ.get("KVQ_ORACLE_LIB") or os.path.join(_HERE, "libkvq_oracle.so")

ROT_IDENTITY, ROT_SIGNED_HADAMARD, ROT_DENSE = 0, 1, 2
SELECT_JOINT, SELECT_PER_HEAD = 0, 1
D = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cache(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("num_pages", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32)]


class _Rot(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("signs", ctypes.c_void_p), ("matrix", ctypes.c_void_p)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        I, P, F = ctypes.c_int, ctypes.c_void_p, ctypes.c_float
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.kvqo_f32_to_f16.argtypes = [F, P]
        lib.kvqo_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.kvqo_f16_to_f32.restype = F
        lib.kvqo_sylvester.argtypes = [I, P]
        lib.kvqo_rotation_matrix.argtypes = [I, P, P, P]
        lib.kvqo_quantize_group.argtypes = [P, I, F, P, P, P]
        lib.kvqo_quantize.argtypes = [P, P, i64, P, P, P, P, F, F, P]
        lib.kvqo_rotate.argtypes = [P, i64, i32, P, P, P]
        lib.kvqo_read_group.argtypes = [P, i64, i32, I, P, P, P]
        lib.kvqo_decode.argtypes = [P, i32, i32, i32, P, P, i32, P, P, P, P, i32, P, P]
        lib.kvqo_decode_f64.argtypes = [P, i32, i32, i32, P, P, i32, P, P, P, P]
        lib.kvqo_attention_ref.argtypes = [P, i32, i32, P, P, i64, i32, P]
        lib.kvqo_candidate_nmse.argtypes = [P, P, P, i64, i32, i32, i32, P, i32, P, i32, P, P, i32, I,
                                            P, P, P]
        lib.kvqo_f32_to_bf16.argtypes = [F]
        lib.kvqo_f32_to_bf16.restype = ctypes.c_uint16
        lib.kvqo_window_write.argtypes = [P, P, i64, i32, P, P, P, i32, P, P, P, P, i32, i32]
        lib.kvqo_decode_windows_f64.argtypes = [P, i32, i32, i32, P, P, i32, P, P, P, P, P]
        lib.kvqo_bits_per_element.argtypes = [i64, i32, i32]
        lib.kvqo_bits_per_element.restype = ctypes.c_double
        lib.kvqo_fold_value_rotation.argtypes = [P, i32, i32, i32, P, P]
        lib.kvqo_decode_causal_f64.argtypes = [P, i32, i32, i32, P, P, i32, P, P, P, P]
        lib.kvqo_quantize_dequant_groups.argtypes = [P, i64, F, P, P]
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with oracle status {rc}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


class Rotation:
    """Rotation of one side (K or V) for all heads: kind + signs [H][128] or matrix [H][128][128]."""

    def __init__(self, kind: int, signs=None, matrix=None):
        self.kind = int(kind)
        self.signs = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
        self.matrix = None if matrix is None else np.ascontiguousarray(matrix, dtype=np.float32)

    def _c(self):
        return _Rot(self.kind, _ptr(self.signs), _ptr(self.matrix))


class Cache:
    """Packed paged cache owned by the oracle: bytes [num_pages][H][72 * page_size]."""

    def __init__(self, num_pages: int, page_size: int, num_kv_heads: int):
        self.num_pages, self.page_size, self.num_kv_heads = int(num_pages), int(page_size), int(num_kv_heads)
        self.pages = np.zeros((self.num_pages, self.num_kv_heads, 72 * self.page_size), dtype=np.uint8)

    def _c(self):
        return _Cache(self.pages.ctypes.data_as(ctypes.c_void_p).value, self.num_pages, self.page_size,
                      self.num_kv_heads)


def f32_to_f16_bits(x: float) -> int:
    out = np.zeros(1, np.uint16)
    _check(_load().kvqo_f32_to_f16(ctypes.c_float(x), _ptr(out)), "f32_to_f16")
    return int(out[0])


def f16_bits_to_f32(bits: int) -> float:
    return float(np.float32(_load().kvqo_f16_to_f32(ctypes.c_uint16(bits))))


def sylvester(n: int) -> np.ndarray:
    h = np.zeros((n, n), np.float64)
    _check(_load().kvqo_sylvester(n, _ptr(h)), "sylvester")
    return h


def rotation_matrix(kind: int, signs=None, matrix=None) -> np.ndarray:
    r = np.zeros((D, D), np.float64)
    s = None if signs is None else np.ascontiguousarray(signs, np.int8)
    m = None if matrix is None else np.ascontiguousarray(matrix, np.float32)
    _check(_load().kvqo_rotation_matrix(kind, _ptr(s), _ptr(m), _ptr(r)), "rotation_matrix")
    return r


def quantize_group(x, clip: float):
    """Returns (codes uint8 [n], scale_bits, zero_bits)."""
    x = _f32(x)
    codes = np.zeros(x.size, np.uint8)
    sb = np.zeros(1, np.uint16)
    zb = np.zeros(1, np.uint16)
    _check(_load().kvqo_quantize_group(_ptr(x), x.size, ctypes.c_float(clip), _ptr(codes), _ptr(sb), _ptr(zb)),
           "quantize_group")
    return codes, int(sb[0]), int(zb[0])


def quantize_dequant_groups(x, clip: float):
    """Groups of 128 (x [n][128] fp32): (dequantized Q2 values fp32, in-range
    flags bool) -- the C oracle's quantizer, with the pass-through flags of the
    straight-through estimator."""
    x = np.ascontiguousarray(x, np.float32).reshape(-1, D)
    xh = np.zeros_like(x)
    m = np.zeros(x.shape, np.uint8)
    _check(_load().kvqo_quantize_dequant_groups(_ptr(x), x.shape[0], ctypes.c_float(clip), _ptr(xh), _ptr(m)),
           "quantize_dequant_groups")
    return xh, m.astype(bool)


def rotate(x, rot: Rotation, mean=None) -> np.ndarray:
    x = _f32(x)
    T, H, _ = x.shape
    out = np.zeros_like(x)
    r = rot._c()
    _check(_load().kvqo_rotate(_ptr(x), T, H, ctypes.byref(r), _ptr(_f32(mean)), _ptr(out)), "rotate")
    return out


def quantize(k, v, cache: Cache, rot_k: Rotation, rot_v: Rotation, key_mean=None, clip_k=1.0, clip_v=1.0,
             slot_mapping=None):
    k, v = _f32(k), _f32(v)
    sm = None if slot_mapping is None else np.ascontiguousarray(slot_mapping, np.int64)
    c = cache._c()
    rk, rv = rot_k._c(), rot_v._c()
    _check(_load().kvqo_quantize(_ptr(k), _ptr(v), k.shape[0], _ptr(sm), ctypes.byref(rk), ctypes.byref(rv),
                                 _ptr(_f32(key_mean)), ctypes.c_float(clip_k), ctypes.c_float(clip_v),
                                 ctypes.byref(c)), "quantize")


def read_group(cache: Cache, slot: int, head: int, kv: int):
    codes = np.zeros(D, np.uint8)
    sb = np.zeros(1, np.uint16)
    zb = np.zeros(1, np.uint16)
    c = cache._c()
    _check(_load().kvqo_read_group(ctypes.byref(c), slot, head, kv, _ptr(codes), _ptr(sb), _ptr(zb)), "read_group")
    return codes, int(sb[0]), int(zb[0])


def decode(q, cache: Cache, seq_lens, rot_k: Rotation, rot_v: Rotation, num_seqs: int, queries_per_seq: int = 1,
           page_table=None, max_pages: int = 0, w_o=None, d_model: int = 0, f64: bool = False):
    """Returns out_o [rows][Hq][128] (and out_y [rows][d_model] when w_o is given)."""
    q = _f32(q)
    rows, Hq, _ = q.shape
    pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    c = cache._c()
    rk, rv = rot_k._c(), rot_v._c()
    lib = _load()
    if f64:
        out = np.zeros((rows, Hq, D), np.float64)
        _check(lib.kvqo_decode_f64(_ptr(q), num_seqs, queries_per_seq, Hq, ctypes.byref(c), _ptr(pt), max_pages,
                                   _ptr(sl), ctypes.byref(rk), ctypes.byref(rv), _ptr(out)), "decode_f64")
        return out
    out_o = np.zeros((rows, Hq, D), np.float32)
    wo = _f32(w_o)
    out_y = np.zeros((rows, d_model), np.float32) if wo is not None else None
    _check(lib.kvqo_decode(_ptr(q), num_seqs, queries_per_seq, Hq, ctypes.byref(c), _ptr(pt), max_pages, _ptr(sl),
                           ctypes.byref(rk), ctypes.byref(rv), _ptr(wo), d_model, _ptr(out_o), _ptr(out_y)),
           "decode")
    return (out_o, out_y) if wo is not None else out_o


class _Windows(ctypes.Structure):
    _fields_ = [("sink_k", ctypes.c_void_p), ("sink_v", ctypes.c_void_p), ("recent_k", ctypes.c_void_p),
                ("recent_v", ctypes.c_void_p), ("num_sink", ctypes.c_int32), ("num_recent", ctypes.c_int32),
                ("key_mean", ctypes.c_void_p)]


class Windows:
    """BF16 sink and recent windows of num_seqs sequences (bf16 bits, uint16):
    sink [num_seqs][num_sink][H][128], recent [num_seqs][num_recent][H][128]
    (position p in slot p % num_recent); key_mean [H][128] centers the window
    keys as the cache write centered the INT2 keys."""

    def __init__(self, num_seqs: int, num_kv_heads: int, num_sink: int = 64, num_recent: int = 256,
                 key_mean=None):
        self.num_seqs, self.num_kv_heads = int(num_seqs), int(num_kv_heads)
        self.num_sink, self.num_recent = int(num_sink), int(num_recent)
        self.sink_k = np.zeros((num_seqs, num_sink, num_kv_heads, D), np.uint16)
        self.sink_v = np.zeros_like(self.sink_k)
        self.recent_k = np.zeros((num_seqs, num_recent, num_kv_heads, D), np.uint16)
        self.recent_v = np.zeros_like(self.recent_k)
        self.key_mean = _f32(key_mean)

    def _c(self):
        return _Windows(_ptr(self.sink_k).value, _ptr(self.sink_v).value, _ptr(self.recent_k).value,
                        _ptr(self.recent_v).value, self.num_sink, self.num_recent,
                        None if self.key_mean is None else _ptr(self.key_mean).value)


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bits (round to nearest even), elementwise."""
    x = np.ascontiguousarray(x, np.float32)
    f = _load().kvqo_f32_to_bf16
    return np.array([f(float(e)) for e in x.ravel()], np.uint16).reshape(x.shape)


def window_write(k, v, seq_idx, positions, windows: Windows, seq_lens=None):
    k, v = _f32(k), _f32(v)
    si = np.ascontiguousarray(seq_idx, np.int32)
    ps = np.ascontiguousarray(positions, np.int32)
    sl = None if seq_lens is None else np.ascontiguousarray(seq_lens, np.int32)
    w = windows
    _check(_load().kvqo_window_write(_ptr(k), _ptr(v), k.shape[0], k.shape[1], _ptr(si), _ptr(ps), _ptr(sl),
                                     w.num_seqs,
                                     _ptr(w.sink_k), _ptr(w.sink_v), _ptr(w.recent_k), _ptr(w.recent_v),
                                     w.num_sink, w.num_recent), "window_write")


def decode_windows(q, cache: Cache, seq_lens, rot_k: Rotation, rot_v: Rotation, windows: Windows, num_seqs: int,
                   queries_per_seq: int = 1, page_table=None, max_pages: int = 0) -> np.ndarray:
    """fp64 out_o [rows][Hq][128] of the decode with BF16 sink and recent windows."""
    q = _f32(q)
    rows, Hq, _ = q.shape
    pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    c = cache._c()
    rk, rv = rot_k._c(), rot_v._c()
    wc = windows._c()
    out = np.zeros((rows, Hq, D), np.float64)
    _check(_load().kvqo_decode_windows_f64(_ptr(q), num_seqs, queries_per_seq, Hq, ctypes.byref(c), _ptr(pt),
                                           max_pages, _ptr(sl), ctypes.byref(rk), ctypes.byref(rv),
                                           ctypes.byref(wc), _ptr(out)), "decode_windows_f64")
    return out


def bits_per_element(seq_len: int, num_sink: int = 64, num_recent: int = 256) -> float:
    return float(_load().kvqo_bits_per_element(seq_len, num_sink, num_recent))


def decode_causal(q, cache: Cache, seq_lens, rot_k: Rotation, rot_v: Rotation, num_seqs: int,
                  queries_per_seq: int = 1, page_table=None, max_pages: int = 0) -> np.ndarray:
    """fp64 out_o [rows][Hq][128]: row qi of a sequence attends its first L - (queries_per_seq - 1 - qi) tokens."""
    q = _f32(q)
    rows, Hq, _ = q.shape
    pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    c = cache._c()
    rk, rv = rot_k._c(), rot_v._c()
    out = np.zeros((rows, Hq, D), np.float64)
    _check(_load().kvqo_decode_causal_f64(_ptr(q), num_seqs, queries_per_seq, Hq, ctypes.byref(c), _ptr(pt),
                                          max_pages, _ptr(sl), ctypes.byref(rk), ctypes.byref(rv), _ptr(out)),
           "decode_causal_f64")
    return out


def fold_value_rotation(w, blocks_per_head: int, rot_v: Rotation) -> np.ndarray:
    """out block b = R_V[b / blocks_per_head]^T w block b (blocks of 128 rows), fp32."""
    w = _f32(w)
    nb = w.shape[0] // D
    out = np.zeros_like(w)
    rv = rot_v._c()
    _check(_load().kvqo_fold_value_rotation(_ptr(w), nb, blocks_per_head, w.shape[1], ctypes.byref(rv), _ptr(out)),
           "fold_value_rotation")
    return out


def attention_ref(q, k, v) -> np.ndarray:
    q, k, v = _f32(q), _f32(k), _f32(v)
    rows, Hq, _ = q.shape
    T, H, _ = k.shape
    out = np.zeros((rows, Hq, D), np.float64)
    _check(_load().kvqo_attention_ref(_ptr(q), rows, Hq, _ptr(k), _ptr(v), T, H, _ptr(out)), "attention_ref")
    return out


def candidate_nmse(k, v, q, candidates, clips, w_o, mode: int, key_mean=None):
    """Returns (nmse [U][C][n], nmse_per_query [U][C][n][Nq], best [U])."""
    k, v, q, w_o = _f32(k), _f32(v), _f32(q), _f32(w_o)
    T, H, _ = k.shape
    Nq, Hq, _ = q.shape
    C, n = len(candidates), len(clips)
    U = 1 if mode == SELECT_JOINT else H
    rots = (_Rot * C)(*[c._c() for c in candidates])
    cl = np.ascontiguousarray(clips, np.float32)
    nmse = np.zeros((U, C, n), np.float64)
    nmse_q = np.zeros((U, C, n, Nq), np.float64)
    best = np.zeros(U, np.int32)
    _check(_load().kvqo_candidate_nmse(_ptr(k), _ptr(v), _ptr(q), T, H, Hq, Nq, rots, C, _ptr(cl), n,
                                       _ptr(_f32(key_mean)), _ptr(w_o), w_o.shape[1], mode, _ptr(nmse),
                                       _ptr(nmse_q), _ptr(best)), "candidate_nmse")
    return nmse, nmse_q, best


def evaluation_stats(nmse_per_query, threshold: float = 10.0) -> dict:
    """Fresh-query statistics of "Output-aware INT2 KV-cache rotation evaluation"
    (results table): mean and population standard deviation (ddof = 0) of the
    per-query post-W_O NMSE, and of the bounded threshold quality 1{NMSE <= 10}."""
    x = np.asarray(nmse_per_query, dtype=np.float64)
    ok = (x <= threshold).astype(np.float64)
    n = x.size
    mean = float(x.sum() / n)
    sd = float(np.sqrt(((x - mean) ** 2).sum() / n))
    qm = float(ok.sum() / n)
    qsd = float(np.sqrt(((ok - qm) ** 2).sum() / n))
    return {"nmse_mean": mean, "nmse_sd": sd, "quality_mean": qm, "quality_sd": qsd}

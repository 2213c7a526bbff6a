"""Thin ctypes binding of libkvq (the C ABI declared in include/kvq.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of libkvq.so.  Tensors must be torch tensors on the GPU; there is no
CPU path, and a missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# (KVQ_LIB points the loader at another build of the library, e.g. the
# sanitizer build of the test suite)
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(_PKG, "libkvq.so")

KVQ_OK, KVQ_ERR_INVALID_ARGUMENT, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP = 0, 1, 2, 3, 4
KVQ_F32, KVQ_BF16 = 0, 1
KVQ_ROT_IDENTITY, KVQ_ROT_SIGNED_HADAMARD, KVQ_ROT_DENSE = 0, 1, 2
KVQ_SELECT_JOINT, KVQ_SELECT_PER_HEAD = 0, 1
HEAD_DIM = 128

EXPORTED = ("kvq_cache_bytes", "kvq_quantize", "kvq_decode_workspace_bytes", "kvq_decode_attn",
            "kvq_decode_attn_causal", "kvq_decode_attn_noalloc", "kvq_window_write", "kvq_decode_attn_windows", "kvq_bits_per_element", "kvq_fold_value_rotation",
            "kvq_candidate_workspace_bytes", "kvq_candidate_nmse", "kvq_optr_workspace_bytes", "kvq_optr_calibrate",
            "kvq_optr_loss_grad", "kvq_status_string", "kvq_version")


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class _Rot(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("signs", ctypes.c_void_p), ("matrix", ctypes.c_void_p)]


class _Cache(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("num_pages", ctypes.c_int64), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32)]


class _Events(ctypes.Structure):
    _fields_ = [("split_start", ctypes.c_void_p), ("split_stop", ctypes.c_void_p), ("attn_stop", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkvq.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libkvq.so not found at {path}; build it with `python -m decode_attention_int2_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.kvq_cache_bytes.argtypes = [i64, i32, i32]
    lib.kvq_cache_bytes.restype = sz
    lib.kvq_quantize.argtypes = [P, P, i32, i64, P, P, P, P, f32, f32, P, P]
    lib.kvq_quantize.restype = ctypes.c_int
    lib.kvq_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.kvq_decode_workspace_bytes.restype = sz
    lib.kvq_decode_attn.argtypes = [P, i32, i32, i32, i32, P, P, i32, P, i32, P, P, P, i32, P, P, P, sz, i32, P, P]
    lib.kvq_decode_attn.restype = ctypes.c_int
    lib.kvq_candidate_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32, i32]
    lib.kvq_candidate_workspace_bytes.restype = sz
    lib.kvq_candidate_nmse.argtypes = [P, P, P, i32, i64, i32, i32, i32, P, i32, P, i32, P, P, i32, i32, P, P, P, P,
                                       sz, P]
    lib.kvq_candidate_nmse.restype = ctypes.c_int
    lib.kvq_decode_attn_noalloc.argtypes = [P, i32, i32, i32, i32, P, P, i32, P, i32, P, P, P, i32, P, P, i32, P]
    lib.kvq_decode_attn_noalloc.restype = ctypes.c_int
    lib.kvq_decode_attn_causal.argtypes = [P, i32, i32, i32, i32, P, P, i32, P, i32, P, P, P, i32, P, P, P, sz, i32, P]
    lib.kvq_decode_attn_causal.restype = ctypes.c_int
    lib.kvq_window_write.argtypes = [P, P, i32, i64, P, P, P, P, P]
    lib.kvq_window_write.restype = ctypes.c_int
    lib.kvq_decode_attn_windows.argtypes = [P, i32, i32, i32, i32, P, P, i32, P, i32, P, P, P, P, P, i32, P, P, P, sz,
                                            i32, P]
    lib.kvq_decode_attn_windows.restype = ctypes.c_int
    lib.kvq_fold_value_rotation.argtypes = [P, i32, i32, i32, i32, P, P, P]
    lib.kvq_fold_value_rotation.restype = ctypes.c_int
    lib.kvq_bits_per_element.argtypes = [i64, i32, i32]
    lib.kvq_bits_per_element.restype = ctypes.c_double
    lib.kvq_optr_workspace_bytes.argtypes = [P, P, i32, i32, i32, i32]
    lib.kvq_optr_workspace_bytes.restype = sz
    lib.kvq_optr_calibrate.argtypes = [i32, P, P, i32, i32, i32, P, i32, P, P, P, P, P, P, P, P, P, sz, P]
    lib.kvq_optr_calibrate.restype = ctypes.c_int
    lib.kvq_optr_loss_grad.argtypes = [i32, i32, P, i32, i32, i32, P, i32, P, P, P, P, P, P, P, P, sz, P]
    lib.kvq_optr_loss_grad.restype = ctypes.c_int
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_version.argtypes = []
    lib.kvq_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kvq_status_string(status).decode()


def _dev_ptr(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU (libkvq has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KVQ_F32
    if t.dtype == torch.bfloat16:
        return KVQ_BF16
    raise ValueError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


# ---- argument contract of include/kvq.h, checked before any pointer is taken:
# a wrong element type or a short buffer would otherwise be read or written
# past its end by a kernel.
def _need(t, name: str, dtype=None, shape=None, min_numel: Optional[int] = None, optional: bool = False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in allowed)}, not {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")


_FLOAT_IO = (torch.float32, torch.bfloat16)


def _need_kv(k, v, H: Optional[int] = None):
    _need(k, "k", _FLOAT_IO)
    _need(v, "v", _FLOAT_IO)
    if k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError(f"k must be [tokens][H][{HEAD_DIM}], not {tuple(k.shape)}")
    if H is not None and k.shape[1] != H:
        raise ValueError(f"k has {k.shape[1]} KV heads, the cache {H}")
    _need(v, "v", k.dtype, tuple(k.shape))


def _need_rot(rot: "Rotation", H: int, name: str):
    if not isinstance(rot, Rotation):
        raise TypeError(f"{name} must be a Rotation")
    if rot.kind == KVQ_ROT_SIGNED_HADAMARD:
        _need(rot.signs, f"{name}.signs", torch.int8, (H, HEAD_DIM))
    elif rot.kind == KVQ_ROT_DENSE:
        _need(rot.matrix, f"{name}.matrix", torch.float32, (H, HEAD_DIM, HEAD_DIM))


def _need_cache(cache: "Cache"):
    _need(cache.pages, "cache.pages", torch.uint8, min_numel=cache.num_pages * cache.num_kv_heads * 72 * cache.page_size)


def _need_key_mean(key_mean, H: int):
    _need(key_mean, "key_mean", torch.float32, (H, HEAD_DIM), optional=True)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Rotation:
    """kvq_rotation: kind + signs (int8 [H][128]) or matrix (fp32 [H][128][128]) on the GPU."""

    def __init__(self, kind: int, signs: Optional[torch.Tensor] = None, matrix: Optional[torch.Tensor] = None):
        self.kind = int(kind)
        self.signs = signs
        self.matrix = matrix

    def _c(self) -> _Rot:
        return _Rot(self.kind, _dev_ptr(self.signs, "signs"), _dev_ptr(self.matrix, "matrix"))


class Cache:
    """kvq_cache: packed pages uint8 [num_pages][H][72 * page_size] on the GPU."""

    def __init__(self, num_pages: int, page_size: int, num_kv_heads: int, device="cuda",
                 pages: Optional[torch.Tensor] = None):
        self.num_pages, self.page_size, self.num_kv_heads = int(num_pages), int(page_size), int(num_kv_heads)
        if pages is None:
            pages = torch.zeros((self.num_pages, self.num_kv_heads, 72 * self.page_size), dtype=torch.uint8,
                                device=device)
        self.pages = pages

    def _c(self) -> _Cache:
        return _Cache(_dev_ptr(self.pages, "pages"), self.num_pages, self.page_size, self.num_kv_heads)

    @property
    def nbytes(self) -> int:
        return int(load_library().kvq_cache_bytes(self.num_pages, self.page_size, self.num_kv_heads))


def _check(rc: int, what: str):
    if rc != KVQ_OK:
        raise KvqError(rc, what)


def kvq_quantize(k: torch.Tensor, v: torch.Tensor, cache: Cache, rot_k: Rotation, rot_v: Rotation,
                 key_mean: Optional[torch.Tensor] = None, clip_k: float = 1.0, clip_v: float = 1.0,
                 slot_mapping: Optional[torch.Tensor] = None, stream=None) -> None:
    H = cache.num_kv_heads
    _need_kv(k, v, H)
    _need(slot_mapping, "slot_mapping", torch.int64, (k.shape[0],), optional=True)
    _need_rot(rot_k, H, "rot_k")
    _need_rot(rot_v, H, "rot_v")
    _need_key_mean(key_mean, H)
    _need_cache(cache)
    lib = load_library()
    c, rk, rv = cache._c(), rot_k._c(), rot_v._c()
    _check(lib.kvq_quantize(_dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(k), k.shape[0],
                            _dev_ptr(slot_mapping, "slot_mapping"), ctypes.byref(rk), ctypes.byref(rv),
                            _dev_ptr(key_mean, "key_mean"), clip_k, clip_v, ctypes.byref(c), _stream(stream)),
           "kvq_quantize")


def kvq_decode_workspace_bytes(num_seqs: int, queries_per_seq: int, num_q_heads: int, num_kv_heads: int,
                               max_seq_len: int, d_model: int = 0, num_splits: int = 0) -> int:
    return int(load_library().kvq_decode_workspace_bytes(num_seqs, queries_per_seq, num_q_heads, num_kv_heads,
                                                         max_seq_len, d_model, num_splits))


def _need_decode(q, num_seqs: int, queries_per_seq: int, cache: "Cache", page_table, max_pages_per_seq: int,
                 seq_lens, rot_k, rot_v, out_o, w_o, out_y):
    H = cache.num_kv_heads
    _need(q, "q", _FLOAT_IO)
    rows = int(num_seqs) * int(queries_per_seq)
    if q.dim() != 3 or q.shape[0] != rows or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [num_seqs * queries_per_seq = {rows}][Hq][{HEAD_DIM}], not {tuple(q.shape)}")
    Hq = q.shape[1]
    if Hq % H:
        raise ValueError(f"num_q_heads {Hq} is not a multiple of num_kv_heads {H}")
    _need_cache(cache)
    _need(page_table, "page_table", torch.int32, min_numel=int(num_seqs) * int(max_pages_per_seq), optional=True)
    _need(seq_lens, "seq_lens", torch.int32, min_numel=int(num_seqs))
    _need_rot(rot_k, H, "rot_k")
    _need_rot(rot_v, H, "rot_v")
    _need(out_o, "out_o", torch.float32, (rows, Hq, HEAD_DIM))
    if w_o is not None:
        _need(w_o, "w_o", q.dtype)
        if w_o.dim() != 2 or w_o.shape[0] != Hq * HEAD_DIM:
            raise ValueError(f"w_o must be [{Hq * HEAD_DIM}][d_model], not {tuple(w_o.shape)}")
        _need(out_y, "out_y", torch.float32, (rows, w_o.shape[1]))
    _need(out_y, "out_y", torch.float32, optional=True)


def kvq_decode_attn(q: torch.Tensor, num_seqs: int, queries_per_seq: int, cache: Cache,
                    page_table: Optional[torch.Tensor], max_pages_per_seq: int, seq_lens: torch.Tensor,
                    max_seq_len: int, rot_k: Rotation, rot_v: Rotation, out_o: torch.Tensor,
                    w_o: Optional[torch.Tensor] = None, out_y: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, num_splits: int = 0, stream=None,
                    split_events: Optional[tuple] = None) -> None:
    """split_events: optional (start, stop) or (start, stop, attn_stop) torch.cuda.Event tuple: start/stop
    are recorded around the split-K kernel, attn_stop after the merge (before W_O)."""
    _need_decode(q, num_seqs, queries_per_seq, cache, page_table, max_pages_per_seq, seq_lens, rot_k, rot_v, out_o,
                 w_o, out_y)
    lib = load_library()
    Hq = q.shape[1]
    d_model = int(w_o.shape[1]) if w_o is not None else 0
    c, rk, rv = cache._c(), rot_k._c(), rot_v._c()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ev = None
    if split_events is not None:
        handles = [ctypes.c_void_p(e.cuda_event) for e in split_events] + [ctypes.c_void_p(0)] * 3
        ev = ctypes.byref(_Events(*handles[:3]))
    _check(lib.kvq_decode_attn(_dev_ptr(q, "q"), _dtype_code(q), num_seqs, queries_per_seq, Hq, ctypes.byref(c),
                               _dev_ptr(page_table, "page_table"), max_pages_per_seq, _dev_ptr(seq_lens, "seq_lens"),
                               max_seq_len, ctypes.byref(rk), ctypes.byref(rv), _dev_ptr(w_o, "w_o"), d_model,
                               _dev_ptr(out_o, "out_o"), _dev_ptr(out_y, "out_y"), _dev_ptr(workspace, "workspace"),
                               ws_bytes, num_splits, ev, _stream(stream)), "kvq_decode_attn")


NOALLOC_SCRATCH_BYTES = 16 << 20  # KVQ_NOALLOC_SCRATCH_BYTES


def kvq_decode_attn_noalloc(q: torch.Tensor, num_seqs: int, queries_per_seq: int, cache: Cache,
                            page_table: Optional[torch.Tensor], max_pages_per_seq: int, seq_lens: torch.Tensor,
                            max_seq_len: int, rot_k: Rotation, rot_v: Rotation, out_o: torch.Tensor,
                            w_o: Optional[torch.Tensor] = None, out_y: Optional[torch.Tensor] = None,
                            num_splits: int = 0, stream=None) -> None:
    """kvq_decode_attn without a workspace: the library's per-GPU scratch array
    (NOALLOC_SCRATCH_BYTES) holds the partials; nothing is allocated."""
    _need_decode(q, num_seqs, queries_per_seq, cache, page_table, max_pages_per_seq, seq_lens, rot_k, rot_v, out_o,
                 w_o, out_y)
    lib = load_library()
    Hq = q.shape[1]
    d_model = int(w_o.shape[1]) if w_o is not None else 0
    c, rk, rv = cache._c(), rot_k._c(), rot_v._c()
    _check(lib.kvq_decode_attn_noalloc(_dev_ptr(q, "q"), _dtype_code(q), num_seqs, queries_per_seq, Hq,
                                       ctypes.byref(c), _dev_ptr(page_table, "page_table"), max_pages_per_seq,
                                       _dev_ptr(seq_lens, "seq_lens"), max_seq_len, ctypes.byref(rk),
                                       ctypes.byref(rv), _dev_ptr(w_o, "w_o"), d_model, _dev_ptr(out_o, "out_o"),
                                       _dev_ptr(out_y, "out_y"), num_splits, _stream(stream)),
           "kvq_decode_attn_noalloc")


def kvq_decode_attn_causal(q: torch.Tensor, num_seqs: int, queries_per_seq: int, cache: Cache,
                           page_table: Optional[torch.Tensor], max_pages_per_seq: int, seq_lens: torch.Tensor,
                           max_seq_len: int, rot_k: Rotation, rot_v: Rotation, out_o: torch.Tensor,
                           w_o: Optional[torch.Tensor] = None, out_y: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, num_splits: int = 0, stream=None) -> None:
    """Rows of a sequence are its last queries_per_seq positions: row qi attends the first
    seq_len - (queries_per_seq - 1 - qi) tokens."""
    _need_decode(q, num_seqs, queries_per_seq, cache, page_table, max_pages_per_seq, seq_lens, rot_k, rot_v, out_o,
                 w_o, out_y)
    lib = load_library()
    Hq = q.shape[1]
    d_model = int(w_o.shape[1]) if w_o is not None else 0
    c, rk, rv = cache._c(), rot_k._c(), rot_v._c()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.kvq_decode_attn_causal(_dev_ptr(q, "q"), _dtype_code(q), num_seqs, queries_per_seq, Hq,
                                      ctypes.byref(c), _dev_ptr(page_table, "page_table"), max_pages_per_seq,
                                      _dev_ptr(seq_lens, "seq_lens"), max_seq_len, ctypes.byref(rk), ctypes.byref(rv),
                                      _dev_ptr(w_o, "w_o"), d_model, _dev_ptr(out_o, "out_o"), _dev_ptr(out_y, "out_y"),
                                      _dev_ptr(workspace, "workspace"), ws_bytes, num_splits, _stream(stream)),
           "kvq_decode_attn_causal")


class _Windows(ctypes.Structure):
    _fields_ = [("sink_k", ctypes.c_void_p), ("sink_v", ctypes.c_void_p), ("recent_k", ctypes.c_void_p),
                ("recent_v", ctypes.c_void_p), ("num_seqs", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("num_sink", ctypes.c_int32), ("num_recent", ctypes.c_int32)]


class Windows:
    """kvq_windows: BF16 sink [num_seqs][num_sink][H][128] and recent [num_seqs][num_recent][H][128]
    (position p in slot p % num_recent) buffers on the GPU."""

    def __init__(self, num_seqs: int, num_kv_heads: int, num_sink: int = 64, num_recent: int = 256, device="cuda"):
        self.num_seqs, self.num_kv_heads = int(num_seqs), int(num_kv_heads)
        self.num_sink, self.num_recent = int(num_sink), int(num_recent)
        shape_s = (self.num_seqs, self.num_sink, self.num_kv_heads, 128)
        shape_r = (self.num_seqs, self.num_recent, self.num_kv_heads, 128)
        self.sink_k = torch.zeros(shape_s, dtype=torch.bfloat16, device=device)
        self.sink_v = torch.zeros(shape_s, dtype=torch.bfloat16, device=device)
        self.recent_k = torch.zeros(shape_r, dtype=torch.bfloat16, device=device)
        self.recent_v = torch.zeros(shape_r, dtype=torch.bfloat16, device=device)

    def _c(self):
        ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t.numel() else None
        return _Windows(ptr(self.sink_k), ptr(self.sink_v), ptr(self.recent_k), ptr(self.recent_v), self.num_seqs,
                        self.num_kv_heads, self.num_sink, self.num_recent)


def _need_windows(windows: Windows, H: int):
    if not isinstance(windows, Windows):
        raise TypeError("windows must be a Windows")
    if windows.num_kv_heads != H:
        raise ValueError(f"windows hold {windows.num_kv_heads} KV heads, the cache {H}")
    for name, n in (("sink", windows.num_sink), ("recent", windows.num_recent)):
        shape = (windows.num_seqs, n, H, HEAD_DIM)
        _need(getattr(windows, name + "_k"), f"windows.{name}_k", torch.bfloat16, shape)
        _need(getattr(windows, name + "_v"), f"windows.{name}_v", torch.bfloat16, shape)


def kvq_window_write(k: torch.Tensor, v: torch.Tensor, seq_idx: torch.Tensor, positions: torch.Tensor,
                     windows: Windows, seq_lens: Optional[torch.Tensor] = None, stream=None) -> None:
    _need_kv(k, v, windows.num_kv_heads)
    _need_windows(windows, windows.num_kv_heads)
    _need(seq_idx, "seq_idx", torch.int32, (k.shape[0],))
    _need(positions, "positions", torch.int32, (k.shape[0],))
    _need(seq_lens, "seq_lens", torch.int32, min_numel=windows.num_seqs, optional=True)
    w = windows._c()
    _check(load_library().kvq_window_write(_dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(k), k.shape[0],
                                           _dev_ptr(seq_idx, "seq_idx"), _dev_ptr(positions, "positions"),
                                           _dev_ptr(seq_lens, "seq_lens"), ctypes.byref(w), _stream(stream)),
           "kvq_window_write")


def kvq_decode_attn_windows(q: torch.Tensor, num_seqs: int, queries_per_seq: int, cache: Cache,
                            page_table: Optional[torch.Tensor], max_pages_per_seq: int, seq_lens: torch.Tensor,
                            max_seq_len: int, rot_k: Rotation, rot_v: Rotation, windows: Windows,
                            out_o: torch.Tensor, key_mean: Optional[torch.Tensor] = None,
                            w_o: Optional[torch.Tensor] = None, out_y: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, num_splits: int = 0, stream=None) -> None:
    _need_decode(q, num_seqs, queries_per_seq, cache, page_table, max_pages_per_seq, seq_lens, rot_k, rot_v, out_o,
                 w_o, out_y)
    _need_windows(windows, cache.num_kv_heads)
    _need_key_mean(key_mean, cache.num_kv_heads)
    lib = load_library()
    Hq = q.shape[1]
    d_model = int(w_o.shape[1]) if w_o is not None else 0
    c, rk, rv, w = cache._c(), rot_k._c(), rot_v._c(), windows._c()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.kvq_decode_attn_windows(_dev_ptr(q, "q"), _dtype_code(q), num_seqs, queries_per_seq, Hq,
                                       ctypes.byref(c), _dev_ptr(page_table, "page_table"), max_pages_per_seq,
                                       _dev_ptr(seq_lens, "seq_lens"), max_seq_len, ctypes.byref(rk),
                                       ctypes.byref(rv), ctypes.byref(w), _dev_ptr(key_mean, "key_mean"),
                                       _dev_ptr(w_o, "w_o"), d_model, _dev_ptr(out_o, "out_o"),
                                       _dev_ptr(out_y, "out_y"), _dev_ptr(workspace, "workspace"), ws_bytes,
                                       num_splits, _stream(stream)), "kvq_decode_attn_windows")


def kvq_fold_value_rotation(w: torch.Tensor, blocks_per_head: int, rot_v: Rotation, out: torch.Tensor,
                            stream=None) -> None:
    """out block b = R_V[b / blocks_per_head]^T w block b (blocks of 128 rows); out has w's shape and dtype."""
    _need(w, "w", _FLOAT_IO)
    if w.dim() != 2 or w.shape[0] % HEAD_DIM:
        raise ValueError(f"w must be [blocks * {HEAD_DIM}][cols], not {tuple(w.shape)}")
    nb = w.shape[0] // HEAD_DIM
    if blocks_per_head < 1 or nb % blocks_per_head:
        raise ValueError(f"{nb} blocks are not a multiple of blocks_per_head {blocks_per_head}")
    _need(out, "out", w.dtype, tuple(w.shape))
    _need_rot(rot_v, nb // blocks_per_head, "rot_v")
    r = rot_v._c()
    _check(load_library().kvq_fold_value_rotation(_dev_ptr(w, "w"), _dtype_code(w), w.shape[0] // 128, blocks_per_head,
                                                  w.shape[1], ctypes.byref(r), _dev_ptr(out, "out"), _stream(stream)),
           "kvq_fold_value_rotation")


def kvq_bits_per_element(seq_len: int, num_sink: int = 64, num_recent: int = 256) -> float:
    return float(load_library().kvq_bits_per_element(seq_len, num_sink, num_recent))


def kvq_candidate_workspace_bytes(num_tokens: int, num_kv_heads: int, num_q_heads: int, num_queries: int,
                                  num_candidates: int, num_clips: int, d_model: int) -> int:
    return int(load_library().kvq_candidate_workspace_bytes(num_tokens, num_kv_heads, num_q_heads, num_queries,
                                                            num_candidates, num_clips, d_model))


def kvq_candidate_nmse(k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, candidates: Sequence[Rotation],
                       clips: Sequence[float], w_o: torch.Tensor, mode: int, out_nmse: torch.Tensor,
                       out_best: torch.Tensor, out_nmse_per_query: Optional[torch.Tensor] = None,
                       key_mean: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    _need_kv(k, v)
    T, H = k.shape[0], k.shape[1]
    _need(q, "q", k.dtype)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or q.shape[1] % H:
        raise ValueError(f"q must be [queries][Hq][{HEAD_DIM}] with Hq a multiple of {H}, not {tuple(q.shape)}")
    Nq, Hq = q.shape[0], q.shape[1]
    _need(w_o, "w_o", k.dtype)
    if w_o.dim() != 2 or w_o.shape[0] != Hq * HEAD_DIM:
        raise ValueError(f"w_o must be [{Hq * HEAD_DIM}][d_model], not {tuple(w_o.shape)}")
    for i, c in enumerate(candidates):
        _need_rot(c, H, f"candidates[{i}]")
    _need_key_mean(key_mean, H)
    U = 1 if mode == KVQ_SELECT_JOINT else H
    grid = U * len(candidates) * len(clips)
    _need(out_nmse, "out_nmse", torch.float32, min_numel=grid)
    _need(out_best, "out_best", torch.int32, min_numel=U)
    _need(out_nmse_per_query, "out_nmse_per_query", torch.float32, min_numel=grid * Nq, optional=True)
    lib = load_library()
    rots = (_Rot * len(candidates))(*[c._c() for c in candidates])
    cl = (ctypes.c_float * len(clips))(*[float(x) for x in clips])
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.kvq_candidate_nmse(_dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(q, "q"), _dtype_code(k), T, H, Hq, Nq,
                                  rots, len(candidates), cl, len(clips), _dev_ptr(key_mean, "key_mean"),
                                  _dev_ptr(w_o, "w_o"), int(w_o.shape[1]), mode, _dev_ptr(out_nmse, "out_nmse"),
                                  _dev_ptr(out_nmse_per_query, "out_nmse_per_query"), _dev_ptr(out_best, "out_best"),
                                  _dev_ptr(workspace, "workspace"), ws_bytes, _stream(stream)),
           "kvq_candidate_nmse")


class _TraceSet(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("max_len", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("q", ctypes.c_void_p)]


class _OptrConfig(ctypes.Structure):
    _fields_ = [("lambda_k", ctypes.c_double), ("clip_k", ctypes.c_float), ("clip_v", ctypes.c_float),
                ("num_sink", ctypes.c_int32), ("num_recent", ctypes.c_int32), ("steps", ctypes.c_int32),
                ("lr", ctypes.c_double), ("eval_every", ctypes.c_int32)]


OPTR_DEFAULTS = dict(lambda_k=1.0, clip_k=0.96, clip_v=0.92, num_sink=64, num_recent=256, steps=80, lr=0.02,
                     eval_every=20)


class _Traces:
    """A kvq_trace_set built from an object with k, v [S][L][H][128], q [S][nq][Hq][128]
    (GPU tensors of one dtype) and lens (host list); keeps the host length array alive."""

    def __init__(self, t, H: int, Hq: int):
        _need(t.k, "traces.k", _FLOAT_IO)
        if t.k.dim() != 4 or t.k.shape[2] != H or t.k.shape[3] != HEAD_DIM:
            raise ValueError(f"traces.k must be [seqs][max_len][{H}][{HEAD_DIM}], not {tuple(t.k.shape)}")
        _need(t.v, "traces.v", t.k.dtype, tuple(t.k.shape))
        S, Lm = t.k.shape[0], t.k.shape[1]
        _need(t.q, "traces.q", t.k.dtype)
        if t.q.dim() != 4 or t.q.shape[0] != S or t.q.shape[2] != Hq or t.q.shape[3] != HEAD_DIM:
            raise ValueError(f"traces.q must be [{S}][queries][{Hq}][{HEAD_DIM}], not {tuple(t.q.shape)}")
        self.nq = int(t.q.shape[1])
        lens = [int(x) for x in t.lens]
        if len(lens) != S or any(not (self.nq <= n <= Lm) for n in lens):
            raise ValueError(f"lens must hold {S} lengths in [{self.nq}, {Lm}]")
        self.dtype = t.k.dtype
        self._lens = (ctypes.c_int32 * S)(*lens)
        self.c = _TraceSet(S, Lm, ctypes.cast(self._lens, ctypes.c_void_p), _dev_ptr(t.k, "traces.k"),
                           _dev_ptr(t.v, "traces.v"), _dev_ptr(t.q, "traces.q"))


def _optr_config(cfg: Optional[dict]) -> _OptrConfig:
    c = dict(OPTR_DEFAULTS, **(cfg or {}))
    return _OptrConfig(c["lambda_k"], c["clip_k"], c["clip_v"], c["num_sink"], c["num_recent"], c["steps"], c["lr"],
                       c["eval_every"])


def kvq_optr_workspace_bytes(calib, heldout, num_kv_heads: int, num_q_heads: int, d_model: int) -> int:
    a = _Traces(calib, num_kv_heads, num_q_heads)
    b = _Traces(heldout, num_kv_heads, num_q_heads) if heldout is not None else None
    return int(load_library().kvq_optr_workspace_bytes(ctypes.byref(a.c), ctypes.byref(b.c) if b else None,
                                                       num_kv_heads, num_q_heads, a.nq, d_model))


def kvq_optr_calibrate(calib, heldout, num_kv_heads: int, num_q_heads: int, w_o: torch.Tensor, r0_k: torch.Tensor,
                       r0_v: torch.Tensor, out_r_k: torch.Tensor, out_r_v: torch.Tensor, cfg: Optional[dict] = None,
                       key_mean: Optional[torch.Tensor] = None, out_key_mean: Optional[torch.Tensor] = None,
                       out_log: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """OptR calibration (Algorithm 1) of one layer; cfg overrides OPTR_DEFAULTS (the paper's Table A)."""
    H, Hq = int(num_kv_heads), int(num_q_heads)
    a = _Traces(calib, H, Hq)
    b = _Traces(heldout, H, Hq)
    if b.nq != a.nq or b.dtype != a.dtype:
        raise ValueError("held-out traces must have the calibration traces' query count and dtype")
    _need(w_o, "w_o", a.dtype)
    if w_o.dim() != 2 or w_o.shape[0] != Hq * HEAD_DIM:
        raise ValueError(f"w_o must be [{Hq * HEAD_DIM}][d_model], not {tuple(w_o.shape)}")
    for name, t in (("r0_k", r0_k), ("r0_v", r0_v), ("out_r_k", out_r_k), ("out_r_v", out_r_v)):
        _need(t, name, torch.float32, (H, HEAD_DIM, HEAD_DIM))
    _need_key_mean(key_mean, H)
    _need(out_key_mean, "out_key_mean", torch.float32, (H, HEAD_DIM), optional=True)
    c = _optr_config(cfg)
    n_ck = max(1, c.steps // c.eval_every)
    _need(out_log, "out_log", torch.float64, (H, 2, c.steps + n_ck + 1), optional=True)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().kvq_optr_calibrate(
        _dtype_code(w_o), ctypes.byref(a.c), ctypes.byref(b.c), H, Hq, a.nq, _dev_ptr(w_o, "w_o"), int(w_o.shape[1]),
        _dev_ptr(r0_k, "r0_k"), _dev_ptr(r0_v, "r0_v"), _dev_ptr(key_mean, "key_mean"), ctypes.byref(c),
        _dev_ptr(out_r_k, "out_r_k"), _dev_ptr(out_r_v, "out_r_v"), _dev_ptr(out_key_mean, "out_key_mean"),
        _dev_ptr(out_log, "out_log"), _dev_ptr(workspace, "workspace"), ws_bytes, _stream(stream)),
        "kvq_optr_calibrate")


def kvq_optr_loss_grad(phase: int, traces, num_kv_heads: int, num_q_heads: int, w_o: torch.Tensor, r0: torch.Tensor,
                       a: torch.Tensor, key_mean: torch.Tensor, out_loss: torch.Tensor, out_grad: torch.Tensor,
                       r_k_hat: Optional[torch.Tensor] = None, cfg: Optional[dict] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """L_K (phase 0) or L_V (phase 1) and dL/dA at generator a (fp64 [H][128][128]), per KV head."""
    H, Hq = int(num_kv_heads), int(num_q_heads)
    t = _Traces(traces, H, Hq)
    _need(w_o, "w_o", t.dtype)
    if w_o.dim() != 2 or w_o.shape[0] != Hq * HEAD_DIM:
        raise ValueError(f"w_o must be [{Hq * HEAD_DIM}][d_model], not {tuple(w_o.shape)}")
    _need(r0, "r0", torch.float32, (H, HEAD_DIM, HEAD_DIM))
    _need(a, "a", torch.float64, (H, HEAD_DIM, HEAD_DIM))
    _need(r_k_hat, "r_k_hat", torch.float32, (H, HEAD_DIM, HEAD_DIM), optional=phase == 0)
    _need(key_mean, "key_mean", torch.float32, (H, HEAD_DIM))
    _need(out_loss, "out_loss", torch.float64, (H,))
    _need(out_grad, "out_grad", torch.float64, (H, HEAD_DIM, HEAD_DIM))
    c = _optr_config(cfg)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().kvq_optr_loss_grad(
        _dtype_code(w_o), phase, ctypes.byref(t.c), H, Hq, t.nq, _dev_ptr(w_o, "w_o"), int(w_o.shape[1]),
        _dev_ptr(r0, "r0"), _dev_ptr(a, "a"), _dev_ptr(r_k_hat, "r_k_hat"), _dev_ptr(key_mean, "key_mean"),
        ctypes.byref(c), _dev_ptr(out_loss, "out_loss"), _dev_ptr(out_grad, "out_grad"),
        _dev_ptr(workspace, "workspace"), ws_bytes, _stream(stream)), "kvq_optr_loss_grad")


def kvq_version() -> int:
    return int(load_library().kvq_version())

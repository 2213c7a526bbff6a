"""The Python binding checks every tensor's element type, shape and size
against the C header's contract before it takes a pointer (CPU only: each
bad case raises before any launch, and a well-formed call on CPU tensors
reaches the device check, which runs last)."""
import pytest
import torch

from decode_attention_int2_amd import kvq

D = 128
H, HQ, T, P = 2, 8, 32, 16


def _cache(pages=None):
    return kvq.Cache(T // P, P, H, device="cpu", pages=pages)


def _kv(dtype=torch.bfloat16, heads=H):
    return torch.zeros((T, heads, D), dtype=dtype), torch.zeros((T, heads, D), dtype=dtype)


def _rot():
    return kvq.Rotation(kvq.KVQ_ROT_SIGNED_HADAMARD, signs=torch.ones((H, D), dtype=torch.int8))


def test_quantize_checks():
    k, v = _kv()
    with pytest.raises(ValueError, match="slot_mapping must have dtype"):
        kvq.kvq_quantize(k, v, _cache(), _rot(), _rot(), slot_mapping=torch.arange(T, dtype=torch.int32))
    with pytest.raises(ValueError, match="KV heads"):
        k3, v3 = _kv(heads=3)
        kvq.kvq_quantize(k3, v3, _cache(), _rot(), _rot())
    with pytest.raises(ValueError, match="v must have dtype"):
        kvq.kvq_quantize(k, v.float(), _cache(), _rot(), _rot())
    with pytest.raises(ValueError, match="cache.pages holds"):
        kvq.kvq_quantize(k, v, _cache(torch.zeros(100, dtype=torch.uint8)), _rot(), _rot())
    with pytest.raises(ValueError, match="rot_k.signs must have shape"):
        kvq.kvq_quantize(k, v, _cache(), kvq.Rotation(kvq.KVQ_ROT_SIGNED_HADAMARD,
                                                      signs=torch.ones((1, D), dtype=torch.int8)), _rot())
    with pytest.raises(ValueError, match="rot_v.matrix must have dtype"):
        kvq.kvq_quantize(k, v, _cache(), _rot(), kvq.Rotation(kvq.KVQ_ROT_DENSE,
                                                              matrix=torch.zeros((H, D, D), dtype=torch.float64)))
    with pytest.raises(ValueError, match="key_mean must have"):
        kvq.kvq_quantize(k, v, _cache(), _rot(), _rot(), key_mean=torch.zeros((H, D), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must live on the GPU"):
        kvq.kvq_quantize(k, v, _cache(), _rot(), _rot())


def _decode_args(**over):
    a = dict(q=torch.zeros((2, HQ, D), dtype=torch.float32), num_seqs=2, queries_per_seq=1, cache=_cache(),
             page_table=torch.zeros((2, 2), dtype=torch.int32), max_pages_per_seq=2,
             seq_lens=torch.zeros(2, dtype=torch.int32), max_seq_len=T, rot_k=_rot(), rot_v=_rot(),
             out_o=torch.zeros((2, HQ, D), dtype=torch.float32), w_o=torch.zeros((HQ * D, 64), dtype=torch.float32),
             out_y=torch.zeros((2, 64), dtype=torch.float32))
    a.update(over)
    return a


@pytest.mark.parametrize("fn", [kvq.kvq_decode_attn, kvq.kvq_decode_attn_causal])
def test_decode_checks(fn):
    cases = [
        (dict(w_o=torch.zeros((HQ * D, 64), dtype=torch.bfloat16)), "w_o must have dtype"),
        (dict(out_o=torch.zeros((1, HQ, D), dtype=torch.float32)), "out_o must have shape"),
        (dict(out_o=torch.zeros((2, HQ, D), dtype=torch.float64)), "out_o must have dtype"),
        (dict(out_y=torch.zeros((2, 32), dtype=torch.float32)), "out_y must have shape"),
        (dict(page_table=torch.zeros((2, 2), dtype=torch.int64)), "page_table must have dtype"),
        (dict(page_table=torch.zeros((2, 1), dtype=torch.int32)), "page_table holds"),
        (dict(seq_lens=torch.zeros(2, dtype=torch.int64)), "seq_lens must have dtype"),
        (dict(seq_lens=torch.zeros(1, dtype=torch.int32)), "seq_lens holds"),
        (dict(q=torch.zeros((3, HQ, D), dtype=torch.float32)), "q must be"),
        (dict(q=torch.zeros((2, 3, D), dtype=torch.float32), out_o=torch.zeros((2, 3, D))), "not a multiple"),
        (dict(cache=_cache(torch.zeros(10, dtype=torch.uint8))), "cache.pages holds"),
    ]
    for over, msg in cases:
        with pytest.raises(ValueError, match=msg):
            fn(**_decode_args(**over))
    with pytest.raises(ValueError, match="must live on the GPU"):
        fn(**_decode_args())


def test_window_and_fold_checks():
    k, v = _kv()
    win = kvq.Windows(2, H, 16, 32, device="cpu")
    i32 = torch.zeros(T, dtype=torch.int32)
    with pytest.raises(ValueError, match="positions must have dtype"):
        kvq.kvq_window_write(k, v, i32, i32.long(), win)
    with pytest.raises(ValueError, match="seq_idx must have shape"):
        kvq.kvq_window_write(k, v, i32[:5], i32, win)
    win.sink_k = win.sink_k.float()
    with pytest.raises(ValueError, match="windows.sink_k must have dtype"):
        kvq.kvq_window_write(k, v, i32, i32, win)
    w = torch.zeros((HQ * D, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must have dtype"):
        kvq.kvq_fold_value_rotation(w, HQ // H, _rot(), torch.zeros((HQ * D, 64), dtype=torch.float32))
    with pytest.raises(ValueError, match="not a multiple of blocks_per_head"):
        kvq.kvq_fold_value_rotation(w, 3, _rot(), torch.zeros_like(w))


def test_candidate_checks():
    k, v = _kv()
    q = torch.zeros((4, HQ, D), dtype=torch.bfloat16)
    w_o = torch.zeros((HQ * D, 64), dtype=torch.bfloat16)
    ok = dict(out_nmse=torch.zeros((H, 1, 2), dtype=torch.float32), out_best=torch.zeros(H, dtype=torch.int32))
    args = lambda **o: dict(dict(k=k, v=v, q=q, candidates=[_rot()], clips=[1.0, 0.9], w_o=w_o,
                                 mode=kvq.KVQ_SELECT_PER_HEAD), **dict(ok, **o))
    with pytest.raises(ValueError, match="out_best must have dtype"):
        kvq.kvq_candidate_nmse(**args(out_best=torch.zeros(H, dtype=torch.int64)))
    with pytest.raises(ValueError, match="out_nmse holds"):
        kvq.kvq_candidate_nmse(**args(out_nmse=torch.zeros(3, dtype=torch.float32)))
    with pytest.raises(ValueError, match="q must have dtype"):
        kvq.kvq_candidate_nmse(**args(q=q.float()))
    with pytest.raises(ValueError, match="w_o must be"):
        kvq.kvq_candidate_nmse(**args(w_o=w_o[:D]))
    with pytest.raises(ValueError, match="out_nmse_per_query holds"):
        kvq.kvq_candidate_nmse(**args(out_nmse_per_query=torch.zeros(7, dtype=torch.float32)))
    with pytest.raises(ValueError, match="must live on the GPU"):
        kvq.kvq_candidate_nmse(**args())

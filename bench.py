"""Benchmark of the rotated-INT2 KV-cache hot path on one MI355X.

One step = cache write of the whole batch (kvq_quantize: rotation, clip,
INT2 quantize, pack, paged write) + one decode step over it (kvq_decode_attn:
query rotation, split-K attention straight from the packed cache, merge,
inverse value rotation, W_O), on the paged batched-decode workload:
16 sequences x 32,768 tokens, 16-token pages with a permuted page table,
32 query / 8 KV heads, head_dim 128, bf16 K/V/q/W_O, signed-Hadamard rotation
per head, W_O [4096, 4096].  Inputs are seeded synthetic data resident in HBM
before the timed region.

Three cache buffers rotate: step i writes cache i%3 and decodes cache
(i+1)%3, written earlier and followed by >2 GB of other traffic, so the
decode reads its 302 MB from HBM, not from the 256 MB Infinity Cache.

Timed regions, each a run of back-to-back calls on one stream between two
HIP events (an event recorded between two kernels leaves the GPU idle for
several microseconds, so none is recorded inside a region), each preceded by
an untimed run of the same calls:
  * steps: K full steps (cache write + decode with W_O) -> ms_per_step;
  * attention: K decode calls without W_O (query rotation, split-K attention,
    split merge and inverse value rotation: one kernel launch with a signed
    Hadamard R_K) over the rotating caches -> decode_attn_us;
  * cache write: K kvq_quantize calls -> quantize_us;
  * decode call: K decode calls with W_O -> decode_call_us.

Prints one JSON line.  value = effective KV GB/s of decode attention: 72
bytes per cached token per KV head / decode_attn_us.  roofline = the decode
kernel (decode_mfma_kernel, the only launch of the attention region).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor peak
BYTES_PER_TOKEN_HEAD = 72      # 2 x 32 B codes + 2 x 4 B fp16 scale/zero
WORKLOAD = "paged16x32k"


def progress(msg: str) -> None:
    """One line per finished phase on stderr (a long profiled run stays visibly alive)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true", help="skip the calibration-search measurement")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the decode figures of the batch-1 and long-context workloads")
    ap.add_argument("--calibration-only", action="store_true",
                    help="only time the calibration search (calib64k) and print its figures")
    ap.add_argument("--num-splits", type=int, default=0, help="split-K parts per sequence (0 = library default)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (calibrates HBM byte counters)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "decode_split_paged16x32k_traffic.json"))
    return ap.parse_args()


# the decode kernel's device code: its own file and the shared device helpers it includes
SPLIT_KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_int2_amd", "csrc", f)
                        for f in ("decode_mfma.hip", "kvq_internal.h")]


def kernel_source_digest() -> str:
    """sha256 of the split kernel's sources (concatenated in the order above):
    counter figures taken from another version of the kernel are not
    reported."""
    import hashlib
    h = hashlib.sha256()
    for path in SPLIT_KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path: str):
    """HBM bytes per split-kernel launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None if there is
    none for the current kernel source."""
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return d.get("hbm_bytes_per_launch")


def host_cpu():
    """(threads this process may use, logical CPUs of the host, CPU model)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return usable, os.cpu_count(), model


def cpu_baseline_threaded(w_cpu, threads: int) -> dict:
    """The same oracle calls on `threads` sequences at once (one sequence per
    thread, its own cache; the oracle's C routines keep no shared state and
    release the interpreter lock): cache writes, then decode steps."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    T = w_cpu["tokens"]
    S = w_cpu["k"].shape[0] // T
    H = w_cpu["k"].shape[1]
    P = 16
    pages = (T + P - 1) // P
    rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=w_cpu["signs"])
    caches = [oracle.Cache(pages, P, H) for _ in range(S)]
    slots = np.arange(T, dtype=np.int64)

    def write(s):
        oracle.quantize(w_cpu["k"][s * T:(s + 1) * T], w_cpu["v"][s * T:(s + 1) * T], caches[s], rot, rot,
                        clip_k=0.96, clip_v=0.92, slot_mapping=slots)

    def read(s):
        oracle.decode(w_cpu["q"][s:s + 1], caches[s], [T], rot, rot, num_seqs=1, max_pages=pages)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(write, range(S)))
        t1 = time.perf_counter()
        list(ex.map(read, range(S)))
        t2 = time.perf_counter()
    usable, logical, model = host_cpu()
    return {"value": S * T * H * BYTES_PER_TOKEN_HEAD / (t2 - t1) / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": f"{S} of 16 sequences x {H} KV heads x {T} tokens, one sequence per thread: "
                                        f"oracle cache write {t1 - t0:.2f} s, oracle decode {t2 - t1:.2f} s",
            "quantize_mtok_s": S * T / (t1 - t0) / 1e6, "host_logical_cpus": logical, "usable_cpus": usable,
            "cpu_model": model}


def cpu_baseline(w_cpu) -> dict:
    """The oracle as it stands, timed on this host on a bounded sample of the
    same workload (about 10-20 s single-threaded): two of the 16 sequences,
    all 8 KV heads (32 query heads), 32,768 tokens each: cache write of the
    sample, then one decode step over it."""
    import numpy as np
    import oracle

    S = 2
    T = w_cpu["tokens"]
    H = w_cpu["k"].shape[1]
    k = w_cpu["k"][:S * T].astype(np.float32)
    v = w_cpu["v"][:S * T].astype(np.float32)
    q = w_cpu["q"][:S].astype(np.float32)
    P = 16
    pages_per_seq = (T + P - 1) // P
    rot = oracle.Rotation(oracle.ROT_SIGNED_HADAMARD, signs=w_cpu["signs"])
    cache = oracle.Cache(S * pages_per_seq, P, H)
    slots = np.concatenate([s * pages_per_seq * P + np.arange(T) for s in range(S)]).astype(np.int64)
    t0 = time.perf_counter()
    oracle.quantize(k, v, cache, rot, rot, clip_k=0.96, clip_v=0.92, slot_mapping=slots)
    t1 = time.perf_counter()
    oracle.decode(q, cache, [T] * S, rot, rot, num_seqs=S, max_pages=pages_per_seq)
    t2 = time.perf_counter()
    dec_gbs = S * T * H * BYTES_PER_TOKEN_HEAD / (t2 - t1) / 1e9
    return {"value": dec_gbs, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{S} of 16 sequences x {H} KV heads x {T} tokens: oracle cache write {t1 - t0:.2f} s, "
                      f"oracle decode ({q.shape[1]} query heads) {t2 - t1:.2f} s",
            "quantize_mtok_s": S * T / (t1 - t0) / 1e6}


def decode_workload(name, dev, timed, median_of, min_bytes=0):
    """Decode attention (no W_O) of another decode workload: average GPU time
    of one call, from 50 calls captured in a HIP graph (median of 5 replays),
    and of 50 eager back-to-back calls (median of 5 runs).  With min_bytes, the calls
    rotate through enough cache copies that the caches together exceed it
    (each call then reads its cache from HBM, not the 256 MB Infinity Cache)."""
    import torch
    import synthetic
    from decode_attention_int2_amd import kvq
    w = synthetic.make(name, dev)
    B, T, H, Hq = w.num_seqs, w.tokens, w.H, w.Hq
    rot = kvq.Rotation(w.rot_k.kind, signs=w.rot_k.signs, matrix=w.rot_k.matrix)
    kv_bytes = B * T * H * BYTES_PER_TOKEN_HEAD
    n = max(3, -(-min_bytes // kv_bytes))
    caches = [kvq.Cache(w.num_pages, w.page_size, H, device=dev) for _ in range(n)]
    write = lambda i: kvq.kvq_quantize(w.k, w.v, caches[i % n], rot, rot, key_mean=w.key_mean, clip_k=w.clip_k,
                                       clip_v=w.clip_v, slot_mapping=w.slot_mapping)
    for i in range(n):
        write(i)
    # the cache write of the whole batch (dense rotation for the learned-rotation workloads)
    wr_ms = median_of(lambda: timed(write, 10), 3)
    n_tok = B * T
    in_bytes = n_tok * H * 2 * 128 * w.k.element_size()
    wr_bytes = in_bytes + kv_bytes
    write_rec = {"rotation": {0: "identity", 1: "signed_hadamard", 2: "dense"}[w.rot_k.kind],
                 "key_centering": w.key_mean is not None, "cache_write_us": round(wr_ms * 1e3, 2),
                 "cache_write_mtok_s": round(n_tok / (wr_ms * 1e-3) / 1e6, 1),
                 "cache_write_gbs": round(wr_bytes / (wr_ms * 1e-3) / 1e9, 1),
                 "cache_write_pct_hbm_peak": round(100.0 * wr_bytes / (wr_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                 "cache_write_input_source": "hbm" if in_bytes > 2 * 256e6 else "mall-resident"}
    del w.k, w.v
    out_o = torch.empty((B * w.queries_per_seq, Hq, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.kvq_decode_workspace_bytes(B, w.queries_per_seq, Hq, H, T, 0, 0), dtype=torch.uint8,
                     device=dev)
    dec = lambda i: kvq.kvq_decode_attn(w.q, B, w.queries_per_seq, caches[i % n], w.page_table,
                                        w.page_table.shape[1], w.seq_lens, T, rot, rot, out_o, workspace=ws)
    eager_ms = median_of(lambda: timed(dec, 50))
    # the same 50 calls captured once in a HIP graph and replayed: the GPU time
    # of a call without the host's per-call cost (which bounds back-to-back
    # eager calls when the kernel is short)
    ms = graph_timed(dec, 50)
    return {"workload": name, "description": synthetic.DESCRIPTIONS[name], "cache_copies": n,
            "source": "hbm" if n * kv_bytes > 2 * 256e6 else "mall-resident", "decode_attn_us": round(ms * 1e3, 2),
            "timing": "hip graph of 50 calls, replayed", "decode_call_us_eager": round(eager_ms * 1e3, 2),
            "gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2), **write_rec}


def graph_timed(fn, n, repeats=5):
    """Average GPU time (ms) of one of n calls fn(i) captured in one HIP graph:
    the median over `repeats` timed replays, after an untimed one.  Every call
    of the path is capturable (no allocation, no synchronization, no memset)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    vals = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        vals.append(e0.elapsed_time(e1) / n)
    del g
    return sorted(vals)[len(vals) // 2]


def envelope_protocol(dev, timed, median_of):
    """The evaluation page's protocol on its own workload (4,096 tokens x 4 KV
    heads x 128, fp32, W_O [512, 128]): the joint search of identity + 8
    signed-Hadamard candidates x 5 clips on 1 calibration query, the cache
    write at the selected variant, then the decode of each of the 10 fresh
    queries (one query per call, W_O included) and their post-W_O NMSE
    statistics.  The page's own figures (host reference math next to an
    NVIDIA L4) are quoted beside them for context."""
    import torch
    import synthetic
    from decode_attention_int2_amd import kvq
    w = synthetic.make("envelope", dev)
    T, H, Hq, dm = w.tokens, w.H, w.Hq, w.d_model
    clips, C = list(w.clips), len(w.candidates)
    rots = [kvq.Rotation(c.kind, signs=c.signs, matrix=c.matrix) for c in w.candidates]
    q_cal, q_eval = w.q[:1].contiguous(), w.q[1:].contiguous()
    out = torch.empty((1, C, len(clips)), dtype=torch.float32, device=dev)
    best = torch.empty((1,), dtype=torch.int32, device=dev)
    ws = torch.empty(kvq.kvq_candidate_workspace_bytes(T, H, Hq, 1, C, len(clips), dm), dtype=torch.uint8, device=dev)
    search = lambda i: kvq.kvq_candidate_nmse(w.k, w.v, q_cal, rots, clips, w.w_o, kvq.KVQ_SELECT_JOINT, out, best,
                                              workspace=ws)
    search_ms = median_of(lambda: timed(search, 5), 3)
    b = int(best.item())
    r, ci = divmod(b, len(clips))
    cache = kvq.Cache(w.num_pages, w.page_size, H, device=dev)
    write = lambda i: kvq.kvq_quantize(w.k, w.v, cache, rots[r], rots[r], clip_k=clips[ci], clip_v=clips[ci],
                                       slot_mapping=w.slot_mapping)
    write_ms = median_of(lambda: timed(write, 20), 3)
    out_o = torch.empty((1, Hq, 128), dtype=torch.float32, device=dev)
    out_y = torch.empty((1, dm), dtype=torch.float32, device=dev)
    dws = torch.empty(kvq.kvq_decode_workspace_bytes(1, 1, Hq, H, T, dm, 0), dtype=torch.uint8, device=dev)
    one = lambda i: kvq.kvq_decode_attn(q_eval[i % 10:i % 10 + 1], 1, 1, cache, w.page_table, w.page_table.shape[1],
                                        w.seq_lens, T, rots[r], rots[r], out_o, w_o=w.w_o, out_y=out_y, workspace=dws)
    dec_ms = median_of(lambda: timed(one, 50))
    # per-query NMSE of the 10 fresh queries at the selected variant (C = 1, one clip)
    e_out = torch.empty((1, 1, 1), dtype=torch.float32, device=dev)
    e_q = torch.empty((1, 1, 1, 10), dtype=torch.float32, device=dev)
    e_best = torch.empty((1,), dtype=torch.int32, device=dev)
    e_ws = torch.empty(kvq.kvq_candidate_workspace_bytes(T, H, Hq, 10, 1, 1, dm), dtype=torch.uint8, device=dev)
    kvq.kvq_candidate_nmse(w.k, w.v, q_eval, [rots[r]], [clips[ci]], w.w_o, kvq.KVQ_SELECT_JOINT, e_out, e_best,
                           out_nmse_per_query=e_q, workspace=e_ws)
    torch.cuda.synchronize()
    x = e_q.double().cpu().flatten()
    mean = float(x.mean())
    sd = float(((x - mean) ** 2).mean().sqrt())
    ok = (x <= 10.0).double()
    qm = float(ok.mean())
    qsd = float(((ok - qm) ** 2).mean().sqrt())
    ident = out[0, 0].min().item()
    return {"workload": "envelope", "description": synthetic.DESCRIPTIONS["envelope"],
            "search_ms": round(search_ms, 4), "selected": {"candidate": r, "clip": clips[ci]},
            "search_nmse_selected": round(float(out[0].flatten()[b]), 6), "search_nmse_identity_best": round(ident, 6),
            "cache_write_us_selected": round(write_ms * 1e3, 2),
            "calibration_plus_quantize_ms": round(search_ms + write_ms, 4),
            "decode_us_per_query": round(dec_ms * 1e3, 2),
            "fresh_queries": {"nmse_mean": round(mean, 6), "nmse_sd_population": round(sd, 6),
                              "threshold_quality_mean": round(qm, 2), "threshold_quality_sd": round(qsd, 2)},
            "packed_kv_code_bytes": T * H * 2 * 32, "metadata_bytes": T * H * 2 * 4,
            "page_figures_for_context": {"calibration_plus_quantize_ms": 319.27, "decode_ms_per_query": 19.19,
                                         "hardware": "host reference math beside one NVIDIA L4"}}


def cpu_baseline_search(threads: int) -> dict:
    """The oracle's candidate search as it stands, timed on this host: the
    envelope's whole joint search (9 x 5 variants, 1 query, 4,096 tokens x 4
    heads), and a bounded sample of the calibration search (one KV head x one
    candidate x 5 clips x 64 queries x 65,536 tokens; the full search is 8
    heads x 9 candidates of such work) single-threaded and with one head per
    thread."""
    import numpy as np
    import oracle
    import synthetic
    from concurrent.futures import ThreadPoolExecutor
    w = synthetic.make("envelope", "cpu")
    f = lambda t: t.float().numpy()
    cands = [oracle.Rotation(c.kind, None if c.signs is None else c.signs.numpy(),
                             None if c.matrix is None else c.matrix.numpy()) for c in w.candidates]
    t0 = time.perf_counter()
    oracle.candidate_nmse(f(w.k), f(w.v), f(w.q[:1]), cands, list(w.clips), f(w.w_o), oracle.SELECT_JOINT)
    env_s = time.perf_counter() - t0
    wc = synthetic.make("calib64k", "cpu")
    k, v, q, wo = f(wc.k), f(wc.v), f(wc.q), f(wc.w_o)
    heads = min(threads, wc.H)

    def one(h):
        c = [oracle.Rotation(wc.candidates[0].kind, matrix=wc.candidates[0].matrix.numpy()[h:h + 1])]
        oracle.candidate_nmse(np.ascontiguousarray(k[:, h:h + 1]), np.ascontiguousarray(v[:, h:h + 1]),
                              np.ascontiguousarray(q[:, h:h + 1]), c, list(wc.clips), wo[h * 128:(h + 1) * 128],
                              oracle.SELECT_JOINT)
    t0 = time.perf_counter()
    one(0)
    one_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=heads) as ex:
        list(ex.map(one, range(heads)))
    thr_s = time.perf_counter() - t0
    full_units = wc.H * len(wc.candidates)
    return {"envelope_search": {"value_s": round(env_s, 3), "cores": 1, "kind": "oracle",
                                "sample": "whole joint search: 9 candidates x 5 clips, 1 query, 4,096 x 4 heads"},
            "calibration_search": {"value_s_estimated_full": round(one_s * full_units, 1), "cores": 1, "kind": "oracle",
                                   "sample": f"1 KV head x 1 candidate x 5 clips (x {full_units} for the full "
                                             f"search): {one_s:.2f} s"},
            "calibration_search_threaded": {"value_s_estimated_full": round(thr_s * full_units / heads, 1),
                                            "cores": heads, "kind": "oracle",
                                            "sample": f"{heads} KV heads x 1 candidate x 5 clips, one head per "
                                                      f"thread: {thr_s:.2f} s"}}


def optr_calibration(dev, cpu_sample: bool) -> dict:
    """The OptR offline calibration (Algorithm 1) of one synthetic layer at the
    paper's settings: 8 KV heads, 32 query heads, d_model 4096, 6 calibration
    and 5 held-out bf16 sequences of 328-700 tokens, the final 64 query
    positions, 80 Adam steps per phase, held-out checks every 20 steps; one
    timed call after an untimed one.  With cpu_sample, the oracle's time for a
    bounded sample (one KV head, 4 steps per phase, one checkpoint each),
    scaled by 8 heads x 20 to the full calibration."""
    import types
    import torch
    import synthetic
    from decode_attention_int2_amd import kvq
    H, Hq, dm = 8, 32, 4096
    pb = synthetic.optr_problem(11, H=H, Hq=Hq, d_model=dm)
    g = lambda ts: types.SimpleNamespace(k=ts.k.to(dev), v=ts.v.to(dev), q=ts.q.to(dev), lens=list(ts.lens))
    cal, hel = g(pb["calib"]), g(pb["heldout"])
    ws = torch.empty(kvq.kvq_optr_workspace_bytes(cal, hel, H, Hq, dm), dtype=torch.uint8, device=dev)
    rk = torch.empty((H, 128, 128), dtype=torch.float32, device=dev)
    rv = torch.empty_like(rk)
    args = (cal, hel, H, Hq, pb["w_o"].to(dev), pb["r0_k"].to(dev), pb["r0_v"].to(dev), rk, rv)
    kvq.kvq_optr_calibrate(*args, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    kvq.kvq_optr_calibrate(*args, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    out = {"workload": "one layer, 8/32 heads, d_model 4096, 6 + 5 sequences of 328-700 tokens, 64 queries, "
                       "80 + 80 Adam steps", "ms": round(ms, 2), "arithmetic": "fp64 (INT2 quantizer in fp32)",
           "workspace_mb": round(ws.numel() / 2 ** 20, 1),
           "page_figures_for_context": {"calibration_min_per_model": [6.25, 7.05, 11.03],
                                        "models": ["Qwen3-4B", "Qwen3-8B", "Phi4-14B"], "hardware": "one A100"}}
    del ws
    if cpu_sample:
        import numpy as np
        from oracle import optr
        G = Hq // H
        f = lambda t: t.float().numpy()
        sub = lambda ts: optr.TraceSet(np.ascontiguousarray(f(ts.k)[:, :, :1]), np.ascontiguousarray(f(ts.v)[:, :, :1]),
                                       np.ascontiguousarray(f(ts.q)[:, :, :G]), list(ts.lens))
        t0 = time.perf_counter()
        optr.calibrate(sub(pb["calib"]), sub(pb["heldout"]), G, pb["nq"], f(pb["w_o"])[:G * 128],
                       pb["r0_k"].numpy()[:1], pb["r0_v"].numpy()[:1], optr.Config(steps=4, eval_every=4))
        s = time.perf_counter() - t0
        out["cpu_baseline"] = {"value_s_estimated_full": round(s * H * 20, 1), "cores": torch.get_num_threads(),
                               "kind": "oracle",
                               "sample": f"1 KV head x 4 steps per phase ({s:.2f} s), x 8 heads x 20 for the full "
                                         f"calibration (fp64 torch ops, {torch.get_num_threads()} threads)"}
    return out


def calibration_search(dev, timed):
    """Time one kvq_candidate_nmse call on calib64k (65,536 tokens x 8 KV
    heads, 9 dense candidates x 5 clips, 64 queries, per-head selection)."""
    import torch
    import synthetic
    from decode_attention_int2_amd import kvq
    wc = synthetic.make("calib64k", dev)
    C, n = len(wc.candidates), len(wc.clips)
    T5, H5, Nq5, Hq5 = wc.tokens, wc.H, wc.q.shape[0], wc.Hq
    out5 = torch.empty((H5, C, n), dtype=torch.float32, device=dev)
    best5 = torch.empty((H5,), dtype=torch.int32, device=dev)
    ws5 = torch.empty(kvq.kvq_candidate_workspace_bytes(T5, H5, Hq5, Nq5, C, n, wc.d_model), dtype=torch.uint8,
                      device=dev)
    rots5 = [kvq.Rotation(cd.kind, signs=cd.signs, matrix=cd.matrix) for cd in wc.candidates]
    search = lambda i: kvq.kvq_candidate_nmse(wc.k, wc.v, wc.q, rots5, list(wc.clips), wc.w_o,
                                              kvq.KVQ_SELECT_PER_HEAD, out5, best5, workspace=ws5)
    cal_ms = timed(search, 3)
    # work of one search: attention of every variant (QK^T and PV) and the rotations
    att_flop = C * n * Nq5 * Hq5 * T5 * 128 * 2 * 2
    rot_flop = C * T5 * H5 * 2 * 128 * 128 * 2
    return {"workload": "calib64k", "description": synthetic.DESCRIPTIONS["calib64k"], "ms": round(cal_ms, 3),
            "variants": C * n, "attention_gflop": round(att_flop / 1e9, 1), "rotation_gflop": round(rot_flop / 1e9, 1),
            "tflop_s": round((att_flop + rot_flop) / (cal_ms * 1e-3) / 1e12, 2),
            "best": [int(x) for x in best5.cpu().tolist()]}


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (every box here has one GPU).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synthetic
    from decode_attention_int2_amd import kvq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.profile_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": 1 << 30, "copy_bytes_written_per_launch": 1 << 30}))
        return
    kvq.load_library()
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        """Average GPU time (ms) of n back-to-back calls fn(i), one event pair
        around them, after an untimed pass of the same n calls (the GPU's clock
        settles over the first tens of kernels of a kind)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        timed.wall_s = time.perf_counter() - w0
        return e0.elapsed_time(e1) / n

    def median_of(fn, repeats=5):
        """Median over repeats of fn() (each an average over a run of calls)."""
        vals = sorted(fn() for _ in range(repeats))
        return vals[len(vals) // 2]

    if a.calibration_only:
        print(json.dumps({"calibration_search": calibration_search(dev, timed)}))
        return
    w = synthetic.make(WORKLOAD, dev)
    B, T, H, Hq, dm, P = w.num_seqs, w.tokens, w.H, w.Hq, w.d_model, w.page_size
    rot = kvq.Rotation(w.rot_k.kind, signs=w.rot_k.signs)
    NC = 3
    caches = [kvq.Cache(w.num_pages, P, H, device=dev) for _ in range(NC)]
    max_pages = w.page_table.shape[1]
    rows = B * w.queries_per_seq
    out_o = torch.empty((rows, Hq, 128), dtype=torch.float32, device=dev)
    out_y = torch.empty((rows, dm), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.kvq_decode_workspace_bytes(B, 1, Hq, H, T, dm, a.num_splits), dtype=torch.uint8,
                     device=dev)

    def quantize(i):
        kvq.kvq_quantize(w.k, w.v, caches[i % NC], rot, rot, clip_k=w.clip_k, clip_v=w.clip_v,
                         slot_mapping=w.slot_mapping)

    def decode(i, with_wo=True):
        kvq.kvq_decode_attn(w.q, B, 1, caches[i % NC], w.page_table, max_pages, w.seq_lens, T, rot, rot, out_o,
                            w_o=w.w_o if with_wo else None, out_y=out_y if with_wo else None, workspace=ws,
                            num_splits=a.num_splits)

    def step(i):
        quantize(i)
        decode(i + 1)

    for i in range(NC):                     # every cache buffer holds a valid cache before warmup
        quantize(i)
    for i in range(a.warmup):
        step(i)
        decode(i, with_wo=False)
    torch.cuda.synchronize()
    step_ms = timed(lambda i: step(a.warmup + i), a.steps)
    wall = timed.wall_s
    progress(f"steps: {step_ms:.3f} ms per step")
    # decode attention and the cache write: median of 5 runs of >= 50 (>= 20) calls
    attn_ms = median_of(lambda: timed(lambda i: decode(i, with_wo=False), max(50, a.steps)))
    quant_ms = median_of(lambda: timed(quantize, max(20, a.steps)))
    decode_ms = median_of(lambda: timed(decode, max(50, a.steps)))
    # the same decode calls captured in a HIP graph (reported beside value)
    attn_graph_ms = graph_timed(lambda i: decode(i, with_wo=False), 48)
    progress(f"decode attention {attn_ms * 1e3:.2f} us (graph {attn_graph_ms * 1e3:.2f} us), cache write "
             f"{quant_ms * 1e3:.2f} us, call {decode_ms * 1e3:.2f} us")

    kv_bytes = B * T * H * BYTES_PER_TOKEN_HEAD
    attn_gbs = kv_bytes / (attn_ms * 1e-3) / 1e9
    tokens = B * T
    quant_bytes = tokens * H * (2 * 128 * 2 + BYTES_PER_TOKEN_HEAD)
    quant_gbs = quant_bytes / (quant_ms * 1e-3) / 1e9

    traffic = measured_traffic(a.traffic_json)

    # the same decode with 64 sink and 256 recent BF16 tokens per sequence
    # (INT2 for the rest): algorithmic bytes = INT2 bytes of the middle + bf16
    # K and V of the windows
    windows = None
    if not a.no_other_workloads:
        S_w, W_w = 64, 256
        seq_idx = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(T)
        pos = torch.arange(T, dtype=torch.int32, device=dev).repeat(B)
        gws = []
        for i in range(NC):
            gw = kvq.Windows(B, H, S_w, W_w, device=dev)
            kvq.kvq_window_write(w.k, w.v, seq_idx, pos, gw, seq_lens=w.seq_lens)
            gws.append(gw)
        wr_ms = median_of(lambda: timed(lambda i: kvq.kvq_window_write(w.k, w.v, seq_idx, pos, gws[i % NC],
                                                                        seq_lens=w.seq_lens), 5))
        dec_w = lambda i: kvq.kvq_decode_attn_windows(w.q, B, 1, caches[i % NC], w.page_table, max_pages, w.seq_lens,
                                                      T, rot, rot, gws[i % NC], out_o, workspace=ws,
                                                      num_splits=a.num_splits)
        win_ms = median_of(lambda: timed(dec_w, 50))
        win_bytes = B * H * ((T - S_w - W_w) * BYTES_PER_TOKEN_HEAD + (S_w + W_w) * 2 * 128 * 2)
        windows = {"num_sink": S_w, "num_recent": W_w, "decode_attn_us": round(win_ms * 1e3, 2),
                   "algorithmic_bytes": win_bytes, "gbs": round(win_bytes / (win_ms * 1e-3) / 1e9, 1),
                   "pct_hbm_peak": round(100.0 * win_bytes / (win_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                   "bits_per_element": round(kvq.kvq_bits_per_element(T, S_w, W_w), 4),
                   "window_write_us_all_tokens": round(wr_ms * 1e3, 2)}
        del gws
        progress(f"windows decode {win_ms * 1e3:.2f} us")

    clip_k, clip_v, desc = w.clip_k, w.clip_v, synthetic.DESCRIPTIONS[WORKLOAD]
    w_cpu = None
    if not a.no_cpu_baseline:   # the oracle's sample: 2 of the 16 sequences, copied to the host
        # threaded run: one sequence per usable CPU, at most 16 (this GPU's share of the host)
        n_thr = max(1, min(16, host_cpu()[0], B))
        n_cpu = max(2, n_thr)
        w_cpu = {"tokens": T, "k": w.k[:n_cpu * T].float().cpu().numpy(), "v": w.v[:n_cpu * T].float().cpu().numpy(),
                 "q": w.q[:n_cpu].float().cpu().numpy(), "signs": w.rot_k.signs.cpu().numpy(), "threads": n_thr}
    del caches, ws, w
    torch.cuda.empty_cache()
    # the other decode workloads: batch 1 x 32K (from HBM, and as measured with
    # 3 copies that stay in the Infinity Cache) and 4 x 131K tokens
    others = None
    if not a.no_other_workloads:
        others = []
        for name, mb in (("gqa32k", 600 << 20), ("gqa32k", 0), ("long131k", 0)):
            others.append(decode_workload(name, dev, timed, median_of, min_bytes=mb))
            progress(f"{name}: decode {others[-1]['decode_attn_us']} us, cache write {others[-1]['cache_write_us']} us")
        torch.cuda.empty_cache()
    # calibration search (a separate workload of the same path) and the
    # evaluation page's own protocol
    cal = env = optr_cal = None
    if not a.no_calibration:
        cal = calibration_search(dev, timed)
        progress(f"calibration search {cal['ms']} ms")
        env = envelope_protocol(dev, timed, median_of)
        progress(f"envelope protocol: search {env['search_ms']} ms")
        optr_cal = optr_calibration(dev, not a.no_cpu_baseline)
        progress(f"OptR calibration {optr_cal['ms']} ms")

    base = None
    if w_cpu is not None:
        base = cpu_baseline(w_cpu)
        progress("cpu baseline")
        base["threaded"] = cpu_baseline_threaded(w_cpu, w_cpu["threads"])
        base["cpu_model"] = host_cpu()[2]
        if not a.no_calibration:
            base["search"] = cpu_baseline_search(w_cpu["threads"])

    out = {
        "metric": "INT2 decode-attn effective KV GB/s (% HBM peak) + quantize Mtok/s, 32K ctx",
        "value": round(attn_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "arithmetic": "INT2 codes on the int8 matrix cores (exact int32 sums) + fp32 softmax and merge",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "description": desc, "batch": B,
                   "context": T, "kv_heads": H, "q_heads": Hq, "head_dim": 128, "page_size": P, "d_model": dm,
                   "kv_input_dtype": "bf16", "cache": "int2 group-128 + fp16 scale/zero",
                   "rotation": "signed_hadamard", "clip_k": clip_k, "clip_v": clip_v},
        "pct_hbm_peak": round(100.0 * attn_gbs / HBM_PEAK_GBS, 2),
        "decode_attn_us": round(attn_ms * 1e3, 2),
        "decode_attn_us_graph": round(attn_graph_ms * 1e3, 2),
        "decode_call_us": round(decode_ms * 1e3, 2),
        "quantize_mtok_s": round(tokens / (quant_ms * 1e-3) / 1e6, 2),
        "quantize_gbs": round(quant_gbs, 1),
        "quantize_us": round(quant_ms * 1e3, 2),
        "wall_ms_per_step": round(wall * 1e3 / a.steps, 4),
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_mfma_kernel", "algorithmic_bytes_per_launch": kv_bytes},
        "cpu_baseline": base,
        "bf16_windows": windows,
        "other_decode_workloads": others,
        "calibration_search": cal,
        "envelope_protocol": env,
        "optr_calibration": optr_cal,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

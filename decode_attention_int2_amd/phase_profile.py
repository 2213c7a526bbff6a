"""Per-phase breakdown of decode_mfma_kernel launches, from the diagnostic
library with phase timestamps (libkvq_phases.so: the same kernels as
libkvq.so, plus a wall-clock read at each phase boundary of every wave).

Build the library on the build host first:
    python -m decode_attention_int2_amd.build --phase-timestamps
then, on a GPU:
    python -m decode_attention_int2_amd.phase_profile [--workload paged16x32k] [--launches 5] [--windows 64,256]

The workload's cache is written into three rotating buffers (as bench.py
does, so that each decode reads its cache from HBM); after untimed launches,
each recorded launch is the last of a run of back-to-back kvq_decode_attn
calls (no W_O), as in a decode loop.  Per launch, with
times relative to the first wave's entry:
  * entry: when the last workgroup started;
  * blocks issued: when each wave had issued its first two blocks' loads
    (their page-table entries read);
  * query row loaded: when each wave's query row had arrived;
  * query ready: when each wave's workgroup had its query digits;
  * first block: when each wave's first block of cache data had arrived;
  * loop start: when each wave began its main loop (query rows ready, first
    blocks in flight);
  * loop end: when each workgroup's last wave left its main loop (the
    spread across workgroups, overall and per XCD);
  * arrived: when each workgroup had stored its partials and counted its
    arrival;
  * merge: in each merging workgroup (the last split of a row group), the
    time from its arrival to its partials merged, to the value rotation
    applied, and to its outputs stored;
  * end: when the last merge ended (the launch's last instruction).
Prints one JSON object: the median over the recorded launches of each
statistic, in microseconds.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PHASE_WAVES, PHASE_FIELDS, WAVES = 8192, 14, 8
# record fields: hw id, xcc id, blocks, t entry, t loop, t loop end, t arrived, t merged, t rotated, t stored,
# t query digits ready, t first block's data, t first blocks' loads issued, t query row loaded
HW, XCC, NB, T0, T1, T2, T3, T4, T5, T6, TQ, TB, TI, TQL = range(14)


def _pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(p * (len(xs) - 1)))))]


def launch_stats(rec, khz):
    """rec: list of per-wave records (fields above, then the workgroup index) of one launch."""
    us = lambda t: t * 1e3 / khz
    t0 = min(r[T0] for r in rec)
    wgs = {}
    for r in rec:
        wgs.setdefault(r[-1], []).append(r)
    entry = [us(r[T0] - t0) for r in rec]
    loop0 = [us(r[T1] - t0) for r in rec]
    loop_wave = [us(r[T2] - r[T1]) for r in rec]
    wg_end = {k: us(max(r[T2] for r in v) - t0) for k, v in wgs.items()}
    wg_arr = {k: us(max(r[T3] for r in v) - t0) for k, v in wgs.items()}
    wg_xcc = {k: v[0][XCC] for k, v in wgs.items()}
    mergers = [v for v in wgs.values() if any(r[T6] for r in v)]
    # merging workgroups: from their arrival to partials merged / rotated / stored (slowest wave)
    m_merge = [us(max(r[T4] for r in v) - max(r[T3] for r in v)) for v in mergers]
    m_rot = [us(max(r[T5] for r in v) - max(r[T4] for r in v)) for v in mergers]
    m_store = [us(max(r[T6] for r in v) - max(r[T5] for r in v)) for v in mergers]
    ends = list(wg_end.values())
    per_xcc = {}
    for k, e in wg_end.items():
        per_xcc.setdefault(int(wg_xcc[k]), []).append(e)
    return {
        "workgroups": len(wgs),
        "entry_last_us": max(entry),
        "blocks_issued_median_us": statistics.median(us(r[TI] - t0) for r in rec),
        "query_row_loaded_median_us": statistics.median(us(r[TQL] - t0) for r in rec),
        "query_ready_median_us": statistics.median(us(r[TQ] - t0) for r in rec),
        "first_block_median_us": statistics.median(us(r[TB] - t0) for r in rec),
        "loop_start_median_us": statistics.median(loop0),
        "loop_start_max_us": max(loop0),
        "loop_wave_median_us": statistics.median(loop_wave),
        "loop_end_min_us": min(ends),
        "loop_end_p10_us": _pct(ends, 0.1),
        "loop_end_median_us": statistics.median(ends),
        "loop_end_p90_us": _pct(ends, 0.9),
        "loop_end_max_us": max(ends),
        "arrived_max_us": max(wg_arr.values()),
        "end_us": max(us(r[T6] - t0) for v in mergers for r in v) if mergers else None,
        "merge_partials_median_us": statistics.median(m_merge) if mergers else None,
        "merge_rotate_median_us": statistics.median(m_rot) if mergers else None,
        "merge_store_median_us": statistics.median(m_store) if mergers else None,
        "loop_end_median_by_xcd_us": {str(x): statistics.median(v) for x, v in sorted(per_xcc.items())},
        "entry_median_by_xcd_us": {str(x): statistics.median(us(min(r[T0] for r in wgs[k]) - t0)
                                                             for k in wgs if wg_xcc[k] == x)
                                   for x in sorted(per_xcc)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="paged16x32k")
    ap.add_argument("--launches", type=int, default=5)
    ap.add_argument("--run", type=int, default=20, help="back-to-back launches per record (the last is recorded)")
    ap.add_argument("--raw", default=None, help="also write every wave's record of every launch here (JSON lines)")
    ap.add_argument("--windows", default=None, help="SINK,RECENT: decode with BF16 sink and recent windows of these sizes")
    a = ap.parse_args()
    import torch
    import synthetic
    from decode_attention_int2_amd import build, kvq
    if not os.path.exists(build.PHASES_LIB):
        raise SystemExit(f"{build.PHASES_LIB} is missing: python -m decode_attention_int2_amd.build --phase-timestamps")
    lib = kvq.load_library(build.PHASES_LIB)
    lib.kvq_phase_timestamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.kvq_phase_timestamps.restype = ctypes.c_int
    lib.kvq_phase_clock_khz.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    w = synthetic.make(a.workload, dev)
    B, T, H, Hq = w.num_seqs, w.tokens, w.H, w.Hq
    rot = kvq.Rotation(w.rot_k.kind, signs=w.rot_k.signs, matrix=w.rot_k.matrix)
    n = 3
    caches = [kvq.Cache(w.num_pages, w.page_size, H, device=dev) for _ in range(n)]
    for c in caches:
        kvq.kvq_quantize(w.k, w.v, c, rot, rot, key_mean=w.key_mean, clip_k=w.clip_k, clip_v=w.clip_v,
                         slot_mapping=w.slot_mapping)
    out_o = torch.empty((B * w.queries_per_seq, Hq, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(kvq.kvq_decode_workspace_bytes(B, w.queries_per_seq, Hq, H, T, 0, 0), dtype=torch.uint8,
                     device=dev)
    dec = lambda i: kvq.kvq_decode_attn(w.q, B, w.queries_per_seq, caches[i % n], w.page_table,
                                        w.page_table.shape[1], w.seq_lens, T, rot, rot, out_o, workspace=ws)
    if a.windows:
        # the windows' bf16 copies of the same K, V (one set per cache buffer)
        S_w, W_w = (int(x) for x in a.windows.split(","))
        seq_idx = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(T)
        pos = torch.arange(T, dtype=torch.int32, device=dev).repeat(B)
        gws = []
        for i in range(n):
            gw = kvq.Windows(B, H, S_w, W_w, device=dev)
            kvq.kvq_window_write(w.k, w.v, seq_idx, pos, gw, seq_lens=w.seq_lens)
            gws.append(gw)
        dec = lambda i: kvq.kvq_decode_attn_windows(w.q, B, w.queries_per_seq, caches[i % n], w.page_table,
                                                    w.page_table.shape[1], w.seq_lens, T, rot, rot, gws[i % n],
                                                    out_o, workspace=ws)
    for i in range(30):
        dec(i)
    buf = (ctypes.c_ulonglong * (PHASE_WAVES * PHASE_FIELDS))()
    if lib.kvq_phase_timestamps(ctypes.addressof(buf), ctypes.sizeof(buf)) != 0:
        raise SystemExit("kvq_phase_timestamps failed")
    khz = lib.kvq_phase_clock_khz()
    per = []
    for i in range(a.launches):
        # a run of back-to-back launches; the records are the last one's (each
        # wave overwrites its own), taken in steady state: a launch right
        # after an idle GPU starts its XCDs up to ~4 us apart
        for j in range(a.run):
            dec(30 + i * a.run + j)
        if lib.kvq_phase_timestamps(ctypes.addressof(buf), ctypes.sizeof(buf)) != 0:
            raise SystemExit("kvq_phase_timestamps failed")
        rec = []
        for wv in range(PHASE_WAVES):
            f = buf[wv * PHASE_FIELDS:(wv + 1) * PHASE_FIELDS]
            if f[T0]:
                rec.append(tuple(f) + (wv // WAVES,))
        per.append(launch_stats(rec, khz))
        if a.raw:
            with open(a.raw, "a") as f:
                f.write(json.dumps({"launch": i, "khz": khz, "waves": rec}) + "\n")
        print(f"launch {i}: {json.dumps(per[-1])}", file=sys.stderr, flush=True)
    keys = [k for k in per[0] if not k.endswith("_by_xcd_us")]
    out = {"workload": a.workload + (f" windows {a.windows}" if a.windows else ""), "launches": a.launches,
           "clock_khz": khz, "kv_bytes": B * T * H * 72}
    for k in keys:
        vals = [p[k] for p in per if p[k] is not None]
        out[k] = round(statistics.median(vals), 2) if vals else None
    for key in ("entry_median_by_xcd_us", "loop_end_median_by_xcd_us"):
        out[key] = {x: round(statistics.median(p[key][x] for p in per), 2) for x in per[0][key]}
    print(json.dumps(out))


if __name__ == "__main__":
    main()

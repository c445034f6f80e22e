"""Per-workgroup timeline of cold partial launches, read from the
measurement build libmla_fp8_timeline.so: the partial kernel with
wall-clock marks (s_memrealtime, 100 MHz, one counter for every CU) at each
workgroup's start and end, at the phases of its first two pieces and of its
last epilogue (csrc/decode_partial.hip lists them at g_timeline).

    python -m mla_latent_kv_fp8_amd.build --timeline
    python -m mla_latent_kv_fp8_amd.timeline [--config batch] [--write separate|fused] [--launches 3] [--warm]

Each timed launch follows 0.1 s of back-to-back launches (the clocks up)
and a read of a separate 512 MiB buffer (L2 and the Infinity Cache then
hold nothing of the launch); --warm leaves that read out, so the launch
finds in the caches what the one before it left.  One JSON line per launch: times in us from
the first workgroup's start, means over the workgroups unless named
otherwise.  The marks cost a few instructions each, so the launch runs a
little slower than the plain build's.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import time

import numpy as np
import torch

from . import build as _build
from . import lib, synth, use_library
from .step import DeviceStep


def _stats(g: np.ndarray, event_us: float) -> dict:
    g = g[g[:, 0] > 0].astype(np.int64)  # workgroups that found no unit leave no record
    t0 = g[:, 0].min()

    def us(x):
        return (x - t0) / 100.0

    start, end, npc = us(g[:, 0]), us(g[:, 1]), g[:, 2]
    one, two = npc >= 1, npc >= 2
    mean = lambda x, m: round(float(np.mean(x[m])), 2) if m.any() else None
    r = {"event_us": round(event_us, 1), "workgroups": int(len(g)), "span": round(float(end.max()), 1),
         "start_max": round(float(start.max()), 2), "end_min": round(float(end.min()), 1),
         "end_median": round(float(np.median(end)), 1), "end_p90": round(float(np.percentile(end, 90)), 1),
         "pieces": np.bincount(npc, minlength=4).tolist()}
    # the first piece: its start, its cache indices, its first ready tile, and the
    # loop's time per tile
    r["piece1_start"] = mean(us(g[:, 3]) - start, one)
    r["indices_landed"] = mean(us(g[:, 15]) - start, one)
    r["first_tile_ready"] = mean(us(g[:, 4]) - start, one)
    r["tile_us"] = round(float(np.sum((us(g[:, 5]) - us(g[:, 4]))[one]) / max(1, np.sum(g[one, 6]))), 3)
    if two.any():
        r["piece2_gap"] = mean(us(g[:, 7]) - us(g[:, 5]), two)  # first piece's loop end -> second's start
        r["piece2_first_tile"] = mean(us(g[:, 8]) - us(g[:, 7]), two)
        r["piece2_tile_us"] = round(float(np.sum((us(g[:, 9]) - us(g[:, 8]))[two]) / max(1, np.sum(g[two, 10]))),
                                    3)
    # the last epilogue, for workgroups whose last piece is one of the two marked
    last = np.where(npc == 2, us(g[:, 9]), us(g[:, 5]))
    m12 = (npc == 1) | (npc == 2)
    r["epilogue_exchange"] = mean(us(g[:, 11]) - last, m12)
    r["epilogue_normalise"] = mean(us(g[:, 12]) - us(g[:, 11]), m12)
    r["epilogue_stores"] = mean(us(g[:, 13]) - us(g[:, 12]), m12)
    r["epilogue_to_end"] = mean(end - us(g[:, 13]), m12)
    late = g[:, 14] > 0
    if late.any():
        r["late_rows_stored"] = mean(us(g[:, 14]) - us(g[:, 3]), late)  # from the first piece's start
        r["late_rows_workgroups"] = int(late.sum())
        r["first_tile_ready_late"] = mean(us(g[:, 4]) - start, one & late)
        r["first_tile_ready_other"] = mean(us(g[:, 4]) - start, one & ~late)
    tiles = g[:, 6] + np.where(two, g[:, 10], 0)
    r["tiles_min_median_max"] = [int(tiles.min()), float(np.median(tiles)), int(tiles.max())]
    slow = np.argsort(end)[-5:]
    r["slowest"] = [{"end": round(float(end[i]), 1), "pieces": int(npc[i]), "tiles": int(tiles[i])} for i in slow]
    return r


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="batch")
    ap.add_argument("--write", choices=("separate", "fused"), default="separate",
                    help="the plain partial launch, or the one with the new tokens' cache write in it")
    ap.add_argument("--launches", type=int, default=3)
    ap.add_argument("--warm", action="store_true", help="no eviction read before the timed launch")
    args = ap.parse_args()
    use_library(_build.TIMELINE_LIB)
    L = lib()
    if not hasattr(L, "mla_wg_timeline"):
        raise SystemExit("%s is not the timeline build" % _build.TIMELINE_LIB)
    L.mla_wg_timeline.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    L.mla_wg_timeline.restype = ctypes.c_int
    L.mla_wg_timeline_clear.argtypes = []
    L.mla_wg_timeline_clear.restype = ctypes.c_int

    w = synth.make(args.config)
    st = DeviceStep(w)
    st.fused_write = args.write == "fused"
    evict = torch.ones(128 << 20, dtype=torch.float32, device="cuda")  # 512 MiB
    M = w.qlen * w.heads
    rows = 16 if M <= 16 else (32 if M <= 32 else 48)
    n_rb = (M + rows - 1) // rows
    n = 8 * ((st.num_workers + 7) // 8) * n_rb  # every workgroup of the launch grid
    if n > 4096:
        raise SystemExit("the launch has %d workgroups; the timeline holds 4096" % n)
    print(json.dumps({"config": args.config, "write": args.write, "warm": args.warm, "workers": st.num_workers,
                      "row_blocks": n_rb}), flush=True)
    for _ in range(args.launches):
        t_end = time.perf_counter() + 0.1
        while time.perf_counter() < t_end:
            for _ in range(10):
                evict.sum()
                st.partials()
            torch.cuda.synchronize()
        assert L.mla_wg_timeline_clear() == 0
        if not args.warm:
            evict.sum()
        else:
            st.partials()  # the launch before the timed one, with nothing between them
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        st.partials()
        b.record()
        torch.cuda.synchronize()
        buf = np.zeros((n, 16), np.uint64)
        assert L.mla_wg_timeline(buf.ctypes.data_as(ctypes.c_void_p), n) == 0
        print(json.dumps(_stats(buf, a.elapsed_time(b) * 1e3)), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the MLA fp8-KV decode step on one MI355X.

A step is the whole hot path over one batch of synthetic input already
resident in HBM: kv_write (the step's new tokens) -> decode_partial ->
merge_lse -> value_gate, where the cache write runs inside the partials'
launch (mla_kv_write_decode_partial_hostplan) when each request has at most 4 new
tokens (--write auto: every workload but spec_q8).  Measured, the fused
steps are 2-8 us faster; with spec_q8's 8 new tokens per request, whose
encodes every row block's workgroup repeats, it comes out even.
Default workload: the batch-decode configuration
(64 requests, qlen 1, 96 heads in a 128-head query buffer, fp8 KV with
kv_scale 0.05, context lengths uniform in [1024, 8192], 4 empty requests,
bf16 W_UV).

Each timed step is preceded (outside its HIP events) by a read of a separate
512 MiB buffer, which evicts the KV cache and everything else the step
touched from L2 and the 256 MB Infinity Cache, so `value` is a cold-cache,
HBM-served figure.  The eviction reads rather than writes: a 512 MiB write
would leave as many dirty lines in the caches, to be written back to HBM
during the timed step (measured: it halves the rate of a plain gather of the
same cache rows).  Warm back-to-back numbers are reported alongside.

The host must stay ahead of the GPU, or a step's GPU time includes waits
for its own launches (the Python binding takes about 55 us of host time
per step, the eviction read only about 70 us of GPU time).  Two things
broke that and made the slow-step tail (mean several microseconds above the
median over a short run): the first step of a loop started from an idle
GPU, and Python's cyclic garbage collector paused the host for up to ~40 ms
in mid-loop (measured: one pause turned a 200-step warm loop from 82 to 270
us per step).  So every timed loop starts behind a short spin kernel (about
0.4 ms) and runs with the collector off (collected once before the
warm-up: a GPU left idle for a few tens of milliseconds runs its next
launches at lower clocks, so nothing idles it between a warm-up and its
timed loop).

The partial kernel's own duration (the `roofline` figures; with the cache
write in it when the step fuses it) is what its
dispatch records in the start and stop events it is given
(mla_time_next_partial), the same span a kernel trace reports; events
recorded around the call (`us_queued`) also hold the launch's dispatch and
completion.

Besides the headline workload, the line carries the partial kernel's
roofline on the other configurations (a short cold partial-only loop each):
batch_8k (64 requests of exactly 8192 tokens), spec_q4, spec_q8 and long
against bf16 MFMA, rank_share against HBM, and the fp8-query call on the
batch workload and on the rank share against the peaks of its mix (QK on
the fp8 MFMA, PV on the bf16 MFMA).  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP8_MFMA_PEAK_TFLOPS = 5000.0
LEAD_CYCLES = 1_000_000  # the spin kernel ahead of a timed loop (about 0.4 ms)
WARM_S = 0.3  # the least warm-up before a timed loop, in seconds of back-to-back launches


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="batch")
    ap.add_argument("--fp8-query", action="store_true",
                    help="the fp8-query path: each step quantises the bf16 query to fp8 E4M3 with a "
                         "per-tensor scale (mla_concat_quant_fp8) and attends on it "
                         "(mla_decode_partial_fp8q)")
    ap.add_argument("--post", choices=("fused", "separate"), default="separate",
                    help="merge + W_UV + gate as mla_merge_lse then mla_value_gate (the faster, measured), "
                         "or as one call (mla_merge_value_gate; needs value heads == attention heads)")
    ap.add_argument("--write", choices=("auto", "fused", "separate"), default="auto",
                    help="the new tokens' cache write inside the partials' launch "
                         "(mla_kv_write_decode_partial_hostplan) or as mla_kv_write before it; auto: fused "
                         "for up to 4 new tokens per request (measured faster there), separate for more")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-config-rooflines", action="store_true",
                    help="skip the partial kernel's rooflines on the other configurations")
    ap.add_argument("--config-iters", type=int, default=50)
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (the known-size "
                         "kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


class Evict:
    """Evicts L2 and the Infinity Cache by reading a 512 MiB buffer that no
    timed work touches; the caches are left clean (no pending write-backs)."""

    def __init__(self, torch):
        self.buf = torch.ones(128 << 20, dtype=torch.float32, device="cuda")  # 512 MiB

    def __call__(self):
        self.buf.sum()  # a float reduction reads the buffer as is (no cast, no temporary)


def copy_probe():
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        flush.zero_()
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}))


def algorithmic(w):
    """KV bytes and MFMA flops of the partial kernel per launch (QK 2*576
    and PV 2*512 flops per visible (row, token) pair)."""
    L = w.lengths.astype(np.int64)
    kv_bytes = int(L.sum()) * 576
    visible = 0
    for j in range(w.qlen):
        visible += int(np.maximum(L - w.qlen + j + 1, 0)[L > 0].sum())
    flops = 2176 * w.heads * visible
    return kv_bytes, flops


def mixed_peak_tflops():
    """The MFMA peak of the fp8-query call: its 1152 QK flops per pair on
    the fp8 MFMA, its 1024 PV flops on the bf16 MFMA."""
    return 2176.0 / (1152.0 / FP8_MFMA_PEAK_TFLOPS + 1024.0 / BF16_MFMA_PEAK_TFLOPS)


def roof_of(flops, kv_bytes, us, mfma_peak):
    """Both roofs of one partial launch and the one that bounds it (MFMA
    when its flops per KV byte exceed the chip's balance, else HBM)."""
    tflops = flops / (us * 1e-6) / 1e12
    gbs = kv_bytes / (us * 1e-6) / 1e9
    mfma = {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(mfma_peak, 1), "unit": "TFLOP/s",
            "frac": round(tflops / mfma_peak, 4)}
    hbm = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if flops / max(kv_bytes, 1) > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        return mfma, hbm
    return hbm, mfma


def step_bytes_kv_write(w):
    """The cache write's algorithmic bytes: each new token's bf16 row and
    slot read, its fp8 row written."""
    return int((w.slot_mapping >= 0).sum()) * (2 * 576 + 8 + 576)


def step_bytes(w, num_workers, split_min):
    """Algorithmic bytes of one whole step, by tensor: each byte a kernel must
    read or write once.  Live partial entries (splits that hold tokens for a
    row) come from the library's host-side split plan."""
    import mla_latent_kv_fp8_amd as m

    S, H, VH = w.S, w.heads, w.value_heads
    bounds, _ = m.split_plan(w.indptr, w.num_splits, num_workers, split_min)
    live = 0
    for r in range(w.batch):
        L = int(w.lengths[r])
        for j in range(w.qlen):
            vis = max(0, L - w.qlen + j + 1)
            b = np.minimum(bounds[r], vis)
            live += int((np.diff(b) > 0).sum())
    w_bytes = VH * 128 * 512 * 2 if w.w_format == "bf16" else VH * 128 * (256 + 16)
    parts = {
        "kv_write": step_bytes_kv_write(w),
        "query": S * H * 576 * 2,
        "kv_cache": int(w.total_tokens) * (576 + 4),
        "partials": 2 * live * H * (512 * 2 + 4),  # written by the partial kernel, read by the merge
        "latent": 2 * S * H * 512 * 2,             # written by the merge, read by W_UV
        "w_uv": w_bytes,
        "gate_and_out": 2 * S * VH * 128 * 2,
    }
    parts["total"] = sum(parts.values())
    return parts


def measured_traffic(config, fused_write=False):
    """HBM bytes per launch of the partial kernel (with the cache write in
    it: fused_write) from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-probe calibration), or None when that
    summary was taken on other kernel source."""
    import hashlib

    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "partial_kernel_%s%s_hbm_traffic.md"
                        % ("kv_write_fused_" if fused_write else "", config))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_launch", "source_sha256"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    h = hashlib.sha256()
    for src in ("decode_partial.hip", "common.hpp"):
        with open(os.path.join(here, "mla_latent_kv_fp8_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def host_cpu():
    """The host's CPU model and its logical CPU count, from /proc/cpuinfo."""
    model, n = "unknown", 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name") and model == "unknown":
                    model = line.split(":", 1)[1].strip()
                elif line.startswith("processor"):
                    n += 1
    except OSError:
        pass
    return "%s (%d logical CPUs visible; %d usable by this process)" % (model, n, len(os.sched_getaffinity(0)))


def warm_up(torch, launch, n):
    """n launches, and at least WARM_S seconds of them, ending on a
    synchronisation; a timed loop follows at once.  A GPU left idle for a
    few tens of milliseconds (a garbage collection, a workload's synthesis)
    runs its next launches at lower clocks: after 33 ms idle, 20 cold partial
    launches on the long workload averaged 330 us against 270 us without the
    gap, and after 100 ms idle the first 40-60 batch steps took 93-96 us
    against 89 us."""
    t_end = time.perf_counter() + WARM_S
    done = 0
    while done < n or time.perf_counter() < t_end:
        for _ in range(10):
            launch()
        done += 10
        torch.cuda.synchronize()


def cold_partial_us(torch, evict, st, n):
    """n cold launches of the step's partial kernel alone (st.partials(),
    each after the eviction read), twice.  Returns (kernel, queued): the mean of the durations the
    kernel records itself (its dispatch takes the start and stop events),
    and, from a second loop of plain launches, the mean of events recorded
    on its stream around each call, which also hold the launch's dispatch
    and completion (about 3 us more on the batch workload)."""
    import mla_latent_kv_fp8_amd as m

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for e in ev:  # created on first use
        for x in e:
            x.record()
    torch.cuda.synchronize()
    torch.cuda._sleep(LEAD_CYCLES)
    for k0, k1 in ev:
        evict()
        m.time_next_partial(k0, k1)
        st.partials()
    torch.cuda.synchronize()
    kern = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    torch.cuda._sleep(LEAD_CYCLES)
    for q0, q1 in ev:
        evict()
        q0.record()
        st.partials()
        q1.record()
    torch.cuda.synchronize()
    queued = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    return kern, queued


def config_roofline(torch, evict, name, fp8_query, iters):
    """The partial kernel's cold roofline on one more configuration: a short
    partial-only loop, each launch after the eviction read, with its own
    events."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    w = synth.make(name)
    print("[bench] partial roofline on %s%s: B=%d qlen=%d H=%d tokens=%d" %
          (name, " (fp8 query)" if fp8_query else "", w.batch, w.qlen, w.heads, w.total_tokens),
          file=sys.stderr, flush=True)
    st = DeviceStep(w)
    if fp8_query:
        st.use_fp8_query(1.0 / 16.0)
        st.quantize_query()
    st.write_new_tokens()
    gc.collect()
    gc.disable()
    warm_up(torch, lambda: (evict(), st.attend()), 3)
    us, us_queued = cold_partial_us(torch, evict, st, iters)
    gc.enable()
    kv_bytes, flops = algorithmic(w)
    roof, other = roof_of(flops, kv_bytes, us, mixed_peak_tflops() if fp8_query else BF16_MFMA_PEAK_TFLOPS)
    roof.update({"us": round(us, 2), "us_queued": round(us_queued, 2), "other": other, "flops_per_launch": flops,
                 "kv_bytes_per_launch": kv_bytes,
                 "workload": "%s: B=%d qlen=%d heads=%d tokens=%d%s" % (name, w.batch, w.qlen, w.heads,
                                                                        w.total_tokens,
                                                                        ", fp8 query" if fp8_query else "")})
    del st
    torch.cuda.empty_cache()
    return roof


def cpu_baseline(w, budget_s):
    """The oracle (as it stands) on a bounded sample of the same workload:
    the first requests of the batch until about `budget_s` of CPU work."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle

    oracle.lib()
    H = w.heads
    nonempty = [r for r in range(w.batch) if w.lengths[r] > 0]
    done_bytes, t_total, n_req = 0, 0.0, 0
    for r in nonempty:
        L = int(w.lengths[r])
        rows = w.indices[w.indptr[r]:w.indptr[r + 1]]
        x = w.kv_rows[w.indptr[r]:w.indptr[r + 1]]
        t0 = time.perf_counter()
        cache = oracle.kv_write(x[:, :512], x[:, 512:], np.arange(L, dtype=np.int64),
                                np.zeros((L, 576), np.uint8), w.kv_scale)
        ip = np.array([0, L], np.int32)
        b, _ = oracle.split_bounds(ip, 1, 1, 1)
        q = np.ascontiguousarray(w.q[r * w.qlen:(r + 1) * w.qlen, :H])
        o, l = oracle.decode_partial(q, cache, ip, np.arange(L, dtype=np.int32), b, w.qlen, w.sm_scale,
                                     w.kv_scale)
        lat = oracle.bf16_round(o[0])
        oracle.value_gate(lat, w.gate[r * w.qlen:(r + 1) * w.qlen, :H * 128], w.lengths[r:r + 1], w.qlen,
                          w_bf16=None if w.w_uv is None else w.w_uv[:H],
                          w_fp4=None if w.w_fp4 is None else w.w_fp4[:H],
                          w_scale=None if w.w_scale is None else w.w_scale[:H])
        t_total += time.perf_counter() - t0
        done_bytes += L * 576
        n_req += 1
        if t_total >= budget_s:
            break
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "host_cpu": host_cpu(),
            "sample": "%d of %d requests of the workload (all %d heads, whole contexts, %d KV tokens): "
                      "cache write + exact attention + W_UV/gate, %.1f s" %
                      (n_req, w.batch, H, done_bytes // 576, t_total)}


# the configurations whose partial-kernel rooflines join the bench line
CONFIG_ROOFLINES = (("batch_8k", False), ("rank_share", False), ("spec_q4", False), ("spec_q8", False), ("long", False),
                    ("batch", True), ("rank_share", True))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    import torch

    import mla_latent_kv_fp8_amd as m
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    m.lib()
    w = synth.make(args.config)
    print("[bench] workload %s: B=%d qlen=%d H=%d tokens=%d" % (w.name, w.batch, w.qlen, w.heads, w.total_tokens),
          file=sys.stderr, flush=True)
    st = DeviceStep(w)
    if args.fp8_query:
        # the runtime's fp8 path: each step quantises the bf16 query (q_scale
        # 1/16 for the N(0,1) synthetic query), then attends on the fp8 codes
        st.use_fp8_query(1.0 / 16.0)
    st.fused_post = fused_post = args.post == "fused" and w.value_heads == w.heads
    new_per_request = len(w.slot_mapping) // w.batch
    st.fused_write = fused_write = args.write == "fused" or (args.write == "auto" and new_per_request <= 4)
    evict = Evict(torch)
    torch.cuda.synchronize()

    # collected before the warm-up steps, not between them and the timed
    # loop: a GPU left idle that long starts the timed steps at lower clocks
    gc.collect()
    gc.disable()  # no collector pause inside a timed loop (re-enabled after them)
    for _ in range(args.warmup):
        evict()
        st.run()
    torch.cuda.synchronize()

    K = args.steps
    # one event pair per step and none inside it: an event recorded between
    # two launches can hold the second one back
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    torch.cuda._sleep(LEAD_CYCLES)  # the host gets ahead of the GPU before the first step
    for i in range(K):
        evict()  # L2 and Infinity Cache hold nothing of the step (outside its events)
        ev[i][0].record()
        st.run()
        ev[i][1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    # the step's first part (new rows written, query quantised, partials), cold
    ea = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda._sleep(LEAD_CYCLES)
    for i in range(K):
        evict()
        ea[i][0].record()
        if not fused_write:
            st.write_new_tokens()
        if st.q_bf16 is not None:
            st.quantize_query()
        st.partials()
        ea[i][1].record()
    torch.cuda.synchronize()
    attn_ms = [a.elapsed_time(b) for a, b in ea]
    # warm: the same steps back to back
    wa, wb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(LEAD_CYCLES)
    wa.record()
    for _ in range(K):
        st.run()
    wb.record()
    torch.cuda.synchronize()
    warm_ms = wa.elapsed_time(wb) / K

    # the partial kernel alone, cold
    partial_us, partial_us_queued = cold_partial_us(torch, evict, st, K)
    partial_ms = partial_us * 1e-3
    gc.enable()

    kv_bytes, flops = algorithmic(w)
    ms = float(np.mean(step_ms))
    value = kv_bytes / (ms * 1e-3) / 1e9
    # the fused launch also reads the new rows and slots and writes their
    # cache rows
    write_bytes = step_bytes_kv_write(w) if fused_write else 0
    sb = step_bytes(w, st.num_workers, st.split_min)
    # the partial kernel's bound: MFMA when its flops per KV byte exceed the
    # chip's balance (2.5 PFLOP/s / 8 TB/s = 312.5 flop/B), else HBM
    traffic = None if args.fp8_query else measured_traffic(args.config, fused_write)
    common = {"traffic": traffic,
              "kernel": ("partial_kernel (kv_write fused into decode_partial)" if fused_write
                         else "partial_kernel (decode_partial)"),
              "us": round(partial_ms * 1e3, 2), "us_queued": round(partial_us_queued, 2),
              "flops_per_launch": flops, "kv_bytes_per_launch": kv_bytes + write_bytes,
              "flop_per_byte": round(flops / max(kv_bytes + write_bytes, 1), 1)}
    if fused_write:
        common["kv_write_bytes_per_launch"] = write_bytes
    roof, other = roof_of(flops, kv_bytes + write_bytes, partial_ms * 1e3,
                          mixed_peak_tflops() if args.fp8_query else BF16_MFMA_PEAK_TFLOPS)
    roof = dict(roof, **common)
    other_key = "roofline_hbm" if roof["bound"] == "mfma" else "roofline_mfma"
    by_config = None
    if not args.no_config_rooflines:
        del st
        torch.cuda.empty_cache()
        by_config = {}
        for name, fq in CONFIG_ROOFLINES:
            if (name, fq) == (args.config, args.fp8_query):
                continue
            by_config[name + ("_fp8_query" if fq else "")] = config_roofline(torch, evict, name, fq, args.config_iters)
    out = {
        "metric": "MLA decode: fp8-KV GB/s + MFMA TFLOP/s vs peak; us/step at B=64, H=128",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "us_per_step_median": round(float(np.median(step_ms)) * 1e3, 2),
        "us_per_step_p90": round(float(np.percentile(step_ms, 90)) * 1e3, 2),
        "us_per_step_max": round(float(np.max(step_ms)) * 1e3, 2),
        "us_per_step_warm": round(warm_ms * 1e3, 2),
        "step_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8-e4m3 KV and query, fp8 MFMA QK + bf16 MFMA PV (f32 accumulate)" if args.fp8_query
                  else "fp8-e4m3 KV, bf16 MFMA (f32 accumulate)"),
        "data": "synthetic (seeded; no dataset or weights)",
        "config": {"workload": "%s: B=%d qlen=%d heads=%d (query buffer %d%s) tokens=%d kv_scale=%g "
                               "splits<=%d workers=%d W_UV=%s" % (w.name, w.batch, w.qlen, w.heads, w.heads_pad,
                                                                  ", fp8 E4M3 + per-tensor scale" if args.fp8_query
                                                                  else " bf16", w.total_tokens, w.kv_scale,
                                                                  w.num_splits, w.num_workers, w.w_format),
                   "post": "merge+W_UV+gate fused" if fused_post else "merge, then W_UV+gate",
                   "cache_write": ("fused into the partials' launch" if fused_write
                                   else "mla_kv_write before the partials"),
                   "global_batch": w.batch, "seq_len": int(w.lengths.max())},
        "roofline": roof,
        # the other roof of the same kernel, for reference
        other_key: other,
        # the same kernel on the other configurations (cold partial-only loops)
        "roofline_by_config": by_config,
        "step_bytes": sb,
        "step_gbs_all_bytes": round(sb["total"] / (ms * 1e-3) / 1e9, 1),
        "attend_us_in_step": round(float(np.mean(attn_ms)) * 1e3, 2),
        "wall_s_timed_region": round(t_wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    print(json.dumps(out))


if __name__ == "__main__":
    main()

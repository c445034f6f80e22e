"""CPU checks of the C ABI: the library loads and exports every entry point
the header declares, the host split plan matches the oracle's partition,
and argument errors are reported before any device work."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_fp8.h")


@pytest.fixture(scope="module")
def mlib():
    import mla_latent_kv_fp8_amd as m

    if not os.path.exists(m.LIB_PATH):
        from mla_latent_kv_fp8_amd import build

        build.build()
    return m


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(mla_\w+)\(", text, flags=re.M)))


def test_header_declares_the_path():
    names = declared_functions()
    for n in ["mla_kv_write", "mla_absorb_query", "mla_concat_quant_fp8", "mla_decode_partial", "mla_decode_partial_fp8q",
              "mla_decode_partial_hostplan", "mla_decode_partial_fp8q_hostplan", "mla_merge_lse", "mla_value_gate", "mla_merge_value_gate", "mla_split_plan", "mla_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol(mlib):
    L = mlib.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings(mlib):
    L = mlib.lib()
    assert L.mla_status_string(0) == b"ok"
    assert L.mla_status_string(1) == b"invalid argument"
    assert L.mla_status_string(99) == b"unknown status"


@pytest.mark.parametrize("lens,ns,W,mn", [
    ([37, 64], 2, 256, 1),
    ([1024, 8192, 0, 4000, 17], 16, 256, 256),
    ([5, 0, 0, 9], 3, 4, 1),
    ([100000, 3, 64000], 64, 256, 256),
    ([10, 20, 30], 1, 256, 1),
    ([0, 0], 4, 8, 1),
])
def test_split_plan_matches_oracle(mlib, oracle, lens, ns, W, mn):
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    b, chunk = mlib.split_plan(indptr, ns, W, mn)
    ob, ochunk = oracle.split_bounds(indptr, ns, W, mn)
    assert chunk == ochunk and np.array_equal(b, ob)


def test_split_plan_random_matches_oracle(mlib, oracle):
    rng = np.random.default_rng(0)
    for _ in range(200):
        B = int(rng.integers(1, 40))
        lens = rng.integers(0, 5000, B)
        lens[rng.random(B) < 0.2] = 0
        indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ns, W, mn = int(rng.integers(1, 70)), int(rng.integers(1, 300)), int(rng.integers(1, 600))
        b, chunk = mlib.split_plan(indptr, ns, W, mn)
        ob, ochunk = oracle.split_bounds(indptr, ns, W, mn)
        assert chunk == ochunk and np.array_equal(b, ob)


def test_argument_errors_before_device_work(mlib):
    L = mlib.lib()
    null = ctypes.c_void_p(0)
    # null pointers / bad sizes are rejected on the host (no launch happens)
    assert L.mla_kv_write(null, 512, null, 64, null, 4, null, 10, 1.0, null) == 1
    assert L.mla_kv_write(null, 512, null, 64, null, 0, null, 10, 1.0, null) == 0  # n = 0: no-op
    assert L.mla_decode_partial(null, 576, 576, 2, 1, 16, null, 10, null, null, 0.1, 1.0, 2, 8, 1,
                                null, 0, 0, 0, null, 0, 0, 0, null) == 1
    assert L.mla_decode_partial(null, 576, 576, 2, 0, 16, null, 10, null, null, 0.1, 1.0, 2, 8, 1,
                                null, 0, 0, 0, null, 0, 0, 0, null) == 1  # qlen 0
    assert L.mla_decode_partial_fp8q(null, 576, 576, 0.5, 2, 1, 16, null, 10, null, null, 0.1, 1.0, 2, 8,
                                     1, null, 0, 0, 0, null, 0, 0, 0, null) == 1
    # (never dereferenced: every case below is rejected before a launch)
    fake = ctypes.c_void_p(1 << 20)
    args = lambda qs, sr: (fake, sr, 576, qs, 2, 1, 16, fake, 10, fake, fake, 0.1, 1.0, 2, 8, 1, fake, 0, 0, 0,
                           fake, 0, 0, 0, null)
    assert L.mla_decode_partial_fp8q(*args(0.0, 576)) == 1            # q_scale must be > 0
    assert L.mla_decode_partial_fp8q(*args(float("nan"), 576)) == 1
    assert L.mla_decode_partial_fp8q(*args(float("inf"), 576)) == 1
    assert L.mla_decode_partial_fp8q(*args(0.5, 584)) == 2            # fp8 row stride not 16-B aligned
    sc = lambda sm, kv: (fake, 576, 576, 2, 1, 16, fake, 10, fake, fake, sm, kv, 2, 8, 1, fake, 0, 0, 0, fake, 0,
                         0, 0, null)
    for sm, kv in ((float("inf"), 1.0), (0.1, float("inf")), (float("nan"), 1.0), (0.1, -1.0)):
        assert L.mla_decode_partial(*sc(sm, kv)) == 1                 # scales must be positive and finite
    gw = lambda nw: (fake, 576, 576, 2, 1, 16, fake, 10, fake, fake, 0.1, 1.0, 2, nw, 1, fake, 0, 0, 0, fake, 0,
                     0, 0, null)
    assert L.mla_decode_partial(*gw(524288)) == 2   # ceil(workers / 8) = 65536: past one launch grid
    assert L.mla_decode_partial(*gw(524281)) == 2   # also 65536 (the last z holds one worker)
    cq = lambda qs, lr, rows: (fake, lr, 512, fake, 192 * 4, 192, qs, rows, 4, fake, 2304, 576, null)
    assert L.mla_concat_quant_fp8(*cq(0.5, 2048, 0)) == 0            # rows = 0: no-op
    assert L.mla_concat_quant_fp8(null, 2048, 512, null, 768, 192, 0.5, 2, 4, null, 2304, 576, null) == 1
    assert L.mla_concat_quant_fp8(*cq(0.0, 2048, 2)) == 1            # q_scale must be > 0
    assert L.mla_concat_quant_fp8(*cq(float("inf"), 2048, 2)) == 1
    assert L.mla_concat_quant_fp8(*cq(0.5, 2044, 2)) == 2            # bf16 stride not 16-B aligned
    assert L.mla_merge_lse(null, 0, 0, 0, null, 0, 0, 0, 2, 0, 4, null, 0, 0, null, 0, 0, null) == 0
    assert L.mla_value_gate(null, 0, 0, 0, null, 0, 0, null, 0, 0, null, 0, null, 6, 4, 2, null, 0,
                            null) == 1  # rows not a multiple of qlen
    assert L.mla_value_gate(null, 0, 0, 7, null, 0, 0, null, 0, 0, null, 0, null, 8, 4, 2, null, 0,
                            null) == 1
    mv = lambda rows, qlen, fmt, op: (op, 0, 0, 0, fake, 0, 0, 0, 2, fmt, fake, 65536, 512, null, 0, 0, fake,
                                      512, fake, rows, qlen, 4, fake, 512, null, 0, 0, null)
    assert L.mla_merge_value_gate(*mv(0, 1, 0, fake)) == 0                 # rows = 0: no-op
    assert L.mla_merge_value_gate(*mv(6, 4, 0, fake)) == 1                 # rows not a multiple of qlen
    assert L.mla_merge_value_gate(*mv(8, 4, 7, fake)) == 1                 # unknown weight format
    assert L.mla_merge_value_gate(*mv(8, 4, 0, null)) == 1                 # null partials
    indptr = np.array([0, 5, 3], dtype=np.int32)  # negative length
    bounds = np.zeros((2, 3), np.int32)
    assert L.mla_split_plan(indptr.ctypes.data_as(ctypes.c_void_p), 2, 2, 4, 1,
                            bounds.ctypes.data_as(ctypes.c_void_p), null) == 1


def test_bench_refuses_more_than_one_gpu():
    # the bench measures one GPU; asking for more exits with a message and
    # status 2 before anything touches a device
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_step_bytes_counts_live_splits():
    # the whole-step byte count: one partial entry per (row, split) that holds
    # tokens for the row, no more than num_splits per row, and at least one
    # for every row that sees a token
    import bench
    from mla_latent_kv_fp8_amd import synth

    w = synth.make("rank_share", seed=5, batch=6, draw_kv=False)
    sb = bench.step_bytes(w, w.num_workers, w.split_min_tokens)
    assert w.num_splits > 1
    live = sb["partials"] // (2 * w.heads * (512 * 2 + 4))
    seen = sum(1 for r in range(w.batch) for j in range(w.qlen) if int(w.lengths[r]) - w.qlen + j + 1 > 0)
    assert seen <= live <= w.num_splits * w.S
    assert sb["kv_cache"] == int(w.total_tokens) * 580
    assert sb["total"] == sum(v for k, v in sb.items() if k != "total")


def test_bench_roofline_bound_and_mixed_peak():
    # the bound of a partial launch follows its flop per KV byte against the
    # chip's balance for the MFMA peak in play; the fp8-query call's peak is
    # the harmonic mix of its QK flops on the fp8 MFMA and its PV flops on
    # the bf16 MFMA (2176 / (1152 / 5000 + 1024 / 2500) = 3400 TFLOP/s)
    import bench

    assert abs(bench.mixed_peak_tflops() - 3400.0) < 1e-9
    # batch-like: 363 flop/B > 312.5 -> MFMA-bound against bf16, HBM-bound against the mix (425)
    roof, other = bench.roof_of(53.16e9, 146.59e6, 70.0, bench.BF16_MFMA_PEAK_TFLOPS)
    assert roof["bound"] == "mfma" and other["bound"] == "hbm"
    assert abs(roof["achieved"] - 53.16e9 / 70e-6 / 1e12) < 0.01
    assert abs(roof["frac"] - roof["achieved"] / 2500.0) < 1e-4
    roof, other = bench.roof_of(53.16e9, 146.59e6, 70.0, bench.mixed_peak_tflops())
    assert roof["bound"] == "hbm" and other["bound"] == "mfma"
    assert abs(roof["achieved"] - 146.59e6 / 70e-6 / 1e9) < 0.1


def test_bench_host_cpu_names_the_model():
    import bench

    h = bench.host_cpu()
    assert "logical CPUs visible" in h and "usable by this process" in h


def test_hostplan_argument_errors(mlib):
    # the host-plan entry point: a null host copy of the offsets, or a
    # decreasing one, is rejected before anything is enqueued
    import numpy as np

    L = mlib.lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every case is rejected on the host

    def call(ih, batch=2):
        return L.mla_decode_partial_hostplan(fake, 576, 576, batch, 1, 16, fake, 10, fake, fake, 0.1, 1.0, 2, 8,
                                             1, fake, 0, 0, 0, fake, 0, 0, 0, ih, null)

    assert call(null) == 1
    assert call(null, batch=0) == 0  # no requests: a no-op
    assert L.mla_decode_partial_fp8q_hostplan(fake, 576, 576, 0.5, 2, 1, 16, fake, 10, fake, fake, 0.1, 1.0, 2,
                                              8, 1, fake, 0, 0, 0, fake, 0, 0, 0, null, null) == 1
    bad = np.array([0, 5, 3], dtype=np.int32)
    assert call(bad.ctypes.data_as(ctypes.c_void_p)) == 1



def test_hostplan_partition_runs_on_the_host(mlib):
    # Valid calls of the host-plan entry points reach the host-built split
    # partition (argument checks, the partition, the kernel arguments) and
    # only then the launch, which fails without a device: status 3.  This
    # runs the host code over many shapes (and under the sanitizer build, in
    # test_sanitizers.py).  Only without a visible GPU: the device pointers
    # here are fakes.
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the fake device pointers must not reach a launch")
    L = mlib.lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(1 << 20)
    rng = np.random.default_rng(11)
    for it in range(60):
        B = int(rng.integers(1, 400))
        lens = rng.integers(0, 20000, B)
        lens[rng.random(B) < 0.1] = 0
        ih = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        nw = int(rng.choice([1, 7, 64, 128, 256, 300]))
        ns = int(rng.integers(1, 65))
        for fp8 in (False, True):
            if fp8:
                st = L.mla_decode_partial_fp8q_hostplan(fake, 576, 576, 0.5, B, 1, 16, fake, 1 << 30, fake, fake,
                                                        0.1, 1.0, ns, nw, 256, fake, 0, 0, 0, fake, 0, 0, 0,
                                                        ih.ctypes.data_as(ctypes.c_void_p), null)
            else:
                st = L.mla_decode_partial_hostplan(fake, 576, 576, B, 1, 96, fake, 1 << 30, fake, fake, 0.1, 1.0,
                                                   ns, nw, 256, fake, 0, 0, 0, fake, 0, 0, 0,
                                                   ih.ctypes.data_as(ctypes.c_void_p), null)
            assert st == 3, (it, st)
    # a decreasing host offset is refused for any worker count
    bad = np.array([0, 5, 3], dtype=np.int32)
    for nw in (8, 256, 300, 4096):
        assert L.mla_decode_partial_hostplan(fake, 576, 576, 2, 1, 16, fake, 10, fake, fake, 0.1, 1.0, 2, nw, 1,
                                             fake, 0, 0, 0, fake, 0, 0, 0, bad.ctypes.data_as(ctypes.c_void_p),
                                             null) == 1


def test_fused_write_argument_errors(mlib):
    # the cache write fused into the partials' launch: its own arguments are
    # checked before anything is enqueued, also for batch = 0
    import torch

    L = mlib.lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced by the rejected cases
    ih = np.array([0, 40, 90], dtype=np.int32)

    def call(kv_c=fake, kv_c_stride=512, k_pe=fake, k_pe_stride=64, slots=fake, k=1, batch=2, fp8=False,
             host=ih.ctypes.data_as(ctypes.c_void_p)):
        new = (kv_c, kv_c_stride, k_pe, k_pe_stride, slots, k)
        if fp8:
            return L.mla_kv_write_decode_partial_fp8q_hostplan(*new, fake, 576, 576, 0.5, batch, 1, 16, fake, 10,
                                                               fake, fake, 0.1, 1.0, 2, 8, 1, fake, 0, 0, 0, fake,
                                                               0, 0, 0, host, null)
        return L.mla_kv_write_decode_partial_hostplan(*new, fake, 576, 576, batch, 1, 16, fake, 10, fake, fake, 0.1,
                                                      1.0, 2, 8, 1, fake, 0, 0, 0, fake, 0, 0, 0, host, null)

    for fp8 in (False, True):
        assert call(k=0, fp8=fp8) == 1
        assert call(k=9, fp8=fp8) == 1
        assert call(k=0, batch=0, fp8=fp8) == 1
        assert call(kv_c=null, fp8=fp8) == 1
        assert call(k_pe=null, fp8=fp8) == 1
        assert call(slots=null, fp8=fp8) == 1
        assert call(kv_c_stride=511, fp8=fp8) == 1
        assert call(k_pe_stride=63, fp8=fp8) == 1
        assert call(host=null, fp8=fp8) == 1
        assert call(kv_c=ctypes.c_void_p((1 << 20) + 8), fp8=fp8) == 2  # not 16-byte aligned
        assert call(k_pe_stride=68, fp8=fp8) == 2                        # rows 8 bytes apart
        assert call(batch=0, k=8, fp8=fp8) == 0                          # no requests: a no-op
        if torch.cuda.device_count() == 0:
            # valid arguments reach the launch, which fails without a device
            assert call(k=8, fp8=fp8) == 3


def test_absorb_query_argument_errors(mlib):
    L = mlib.lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every case is rejected (or a no-op) on the host

    def call(rows=4, heads=2, fp8=0, qs=1.0, qn=fake, qn_row=256, wk_n=64, out_row=1152, out=fake):
        return L.mla_absorb_query(qn, qn_row, 128, fake, 128, 64, fake, 512 * 64, wk_n, fake, 512 * 4, 4, rows,
                                  heads, fp8, qs, out, out_row, 576, null)

    assert call(rows=0) == 0                   # no rows: a no-op
    assert call(rows=-1) == 1
    assert call(heads=0) == 1
    assert call(fp8=2) == 1                    # unknown output format
    assert call(qn=null) == 1
    assert call(out=null) == 1
    assert call(fp8=1, qs=0.0) == 1            # the fp8 path needs q_scale > 0 and finite
    assert call(fp8=1, qs=float("inf")) == 1
    assert call(qn_row=260) == 2               # bf16 rows in 16-byte chunks
    assert call(wk_n=66) == 2                  # W_K code words are 4-byte aligned
    assert call(fp8=1, out_row=1160) == 2      # fp8 output rows in 16-byte chunks


def test_timeline_build_exports_its_reader(mlib):
    # the measurement build carries the partial kernel's per-workgroup marks
    # and their reader; the product library has neither
    from mla_latent_kv_fp8_amd import build

    if not os.path.exists(build.TIMELINE_LIB):
        pytest.skip("the timeline build is not built (python -m mla_latent_kv_fp8_amd.build --timeline)")
    T = ctypes.CDLL(build.TIMELINE_LIB)
    assert hasattr(T, "mla_wg_timeline") and hasattr(T, "mla_wg_timeline_clear")
    assert not hasattr(mlib.lib(), "mla_wg_timeline")

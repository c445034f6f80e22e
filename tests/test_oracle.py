"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a library routine that
computes the same definition (torch's fp8 / e8m0 / bf16 casts, torch's
scaled-dot-product attention and logsumexp, numpy matmul, scipy's expit),
brute force on tiny inputs, or an invariant of the method.  The pages print
no worked example (tests/golden/README.md), so no pin quotes a printed value.
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

from mla_latent_kv_fp8_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ codecs

def test_fp8_decode_matches_torch_e4m3fn(oracle):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_fp8_named_points_from_spec(oracle):
    for line in open(os.path.join(GOLDEN, "ocp_fp8_e4m3.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = oracle.fp8_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_fp8_encode_roundtrip_all_finite_codes(oracle):
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.fp8_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(oracle.fp8_encode(vals[fin]), codes[fin])


def _nearest_even_bruteforce(v, table_vals, table_codes):
    """Nearest finite fp8 value, ties to the even code, saturating: brute
    force over the finite positive codes."""
    a = abs(v)
    if a >= 448:
        c = 0x7E
    else:
        d = np.abs(table_vals - a)
        best = np.flatnonzero(d == d.min())
        c = int(table_codes[best[0]]) if len(best) == 1 else int(
            [table_codes[i] for i in best if table_codes[i] % 2 == 0][0])
    return c | (0x80 if np.signbit(v) else 0)


def test_fp8_encode_bruteforce_midpoints_and_saturation(oracle):
    pos = np.arange(0, 0x7F, dtype=np.uint8)
    pv = oracle.fp8_decode(pos)
    mids = (pv[:-1] + pv[1:]) / 2.0
    rng = np.random.default_rng(0)
    probes = np.concatenate([mids, -mids, pv * 1.0001, pv * 0.9999, rng.uniform(-500, 500, 2000),
                             [449.0, 464.0, 465.0, 1e6, -1e6, 0.0, -0.0, 1e-30]])
    got = oracle.fp8_encode(probes)
    want = np.array([_nearest_even_bruteforce(v, pv, pos) for v in probes], dtype=np.uint8)
    assert np.array_equal(got, want)
    assert oracle.fp8_encode(np.array([np.nan]))[0] == 0x7F


def test_fp8_encode_matches_torch_cast_in_range(oracle):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 30, rng.uniform(-448, 448, 20000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_encode(x.astype(np.float64)), ref)


def test_bf16_round_matches_torch_for_binary32_inputs(oracle):
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # ties: low 16 bits exactly 0x8000
    ties = ((rng.integers(0, 2**16, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_direct_not_double_rounded(oracle):
    # 1 + 2^-8 + 2^-30 lies just above a bf16 tie: direct rounding goes up,
    # rounding through binary32 first would land on the tie and go to even.
    x = 1.0 + 2.0**-8 + 2.0**-30
    assert oracle.bf16_decode(oracle.bf16_round(np.array([x])))[0] == 1.0 + 2.0**-7
    assert oracle.bf16_round(np.array([np.nan]))[0] == 0x7FC0


def test_e2m1_table_from_spec(oracle):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "ocp_mx_e2m1.txt")) if l.strip() and l[0] != "#"]
    for code, val in rows:
        c = int(code)
        assert oracle.e2m1_decode(np.array([c]))[0] == float(val)
        neg = oracle.e2m1_decode(np.array([c | 8]))[0]
        assert neg == -float(val) and np.signbit(neg)


def test_e8m0_matches_torch(oracle):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


# ------------------------------------------------------------- kv write

def test_kv_write_bruteforce_and_skip(oracle):
    rng = np.random.default_rng(3)
    n, slots, kv_scale = 7, 13, 0.05
    rows = synth.to_bf16_bits(rng.standard_normal((n, 576)).astype(np.float32) * 0.5)
    slot_map = np.array([3, 0, -1, 12, 7, 5, 9], dtype=np.int64)
    cache = np.full((slots, 576), 0x7F, dtype=np.uint8)
    out = oracle.kv_write(rows[:, :512], rows[:, 512:], slot_map, cache, kv_scale)
    pos = np.arange(0, 0x7F, dtype=np.uint8)
    pv = oracle.fp8_decode(pos)
    for i, s in enumerate(slot_map):
        if s < 0:
            continue
        x = oracle.bf16_decode(rows[i]).astype(np.float32)
        scaled = (x / np.float32(kv_scale)).astype(np.float64)  # binary32 division
        want = [_nearest_even_bruteforce(v, pv, pos) for v in scaled]
        assert np.array_equal(out[s], np.array(want, dtype=np.uint8))
    untouched = sorted(set(range(slots)) - set(int(s) for s in slot_map if s >= 0))
    assert (out[untouched] == 0x7F).all()


# ---------------------------------------------------------- split bounds

def test_split_bounds_tiny_worked_example(oracle):
    indptr = np.array([0, 37, 101], dtype=np.int32)
    b, chunk = oracle.split_bounds(indptr, 2, 256, 1)
    lines = [l for l in open(os.path.join(GOLDEN, "split_bounds_tiny.txt")) if l[0] != "#"]
    want = np.array([[int(v) for v in l.split(":")[1].split()] for l in lines], dtype=np.int32)
    assert chunk == 64
    assert np.array_equal(b, want)


def test_split_bounds_weighted_worked_example(oracle):
    """A worked example where the per-request stream positions move the cuts
    (tests/golden/split_bounds_weighted.txt, derived by hand)."""
    lens = [100, 0, 250]
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    b, chunk = oracle.split_bounds(indptr, 4, 4, 1)
    lines = [l for l in open(os.path.join(GOLDEN, "split_bounds_weighted.txt")) if l[0] != "#"]
    want = np.array([[int(v) for v in l.split(":")[1].split()] for l in lines], dtype=np.int32)
    assert chunk == 328
    assert np.array_equal(b, want)


@pytest.mark.parametrize("lens,ns,W,mn", [
    ([1024, 8192, 0, 4000, 17], 16, 256, 256),
    ([5, 0, 0, 9], 3, 4, 1),
    ([100000, 3, 64000], 64, 256, 256),
    ([10, 20, 30], 1, 256, 1),
    ([0, 0], 4, 8, 1),
])
def test_split_bounds_properties(oracle, lens, ns, W, mn):
    lens = np.array(lens)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    b, chunk = oracle.split_bounds(indptr, ns, W, mn)
    T = int(lens.sum())
    assert chunk >= max(1, mn)
    for r, L in enumerate(lens):
        br = b[r]
        assert br[0] == 0 and br[-1] == L and (np.diff(br) >= 0).all()
        # stream position of the request's first token
        P = int(indptr[r]) + oracle.PIECE_TOKENS * (r + 1)
        for k in range(ns):
            lo, hi = int(br[k]), int(br[k + 1])
            if hi > lo:
                # a piece never crosses a multiple of chunk in stream coordinates
                assert (P + lo) // chunk == (P + hi - 1) // chunk
                if k > 0:
                    assert (P + lo) % chunk == 0
        # pieces are maximal: consecutive non-empty pieces sit in consecutive chunks
        if L > 0:
            n_pieces = (P + L - 1) // chunk - P // chunk + 1
            assert n_pieces <= ns
            assert int((np.diff(br) > 0).sum()) == n_pieces


# ------------------------------------------------------------- attention

def _decode_kv(kv):
    return torch.from_numpy(np.ascontiguousarray(kv)).view(torch.float8_e4m3fn).to(torch.float64)


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def _sdpa_reference(q_bits, kv_bytes, indptr, indices, qlen, sm_scale, kv_scale, q_real=None):
    """Library attention: torch SDPA (float64, CPU) with a boolean causal
    window mask, and torch.logsumexp for the LSE.  q_real (float64
    [S, H, 576]) replaces the bf16 query when given."""
    S, H, _ = q_bits.shape
    B = len(indptr) - 1
    o = np.zeros((S, H, 512))
    lse = np.full((S, H), -np.inf)
    for r in range(B):
        L = int(indptr[r + 1] - indptr[r])
        if L == 0:
            continue
        rows = indices[indptr[r]:indptr[r + 1]]
        kv = _decode_kv(kv_bytes[rows])           # [L, 576]
        if q_real is None:
            q = _bf16(q_bits[r * qlen:(r + 1) * qlen])  # [qlen, H, 576]
        else:
            q = torch.from_numpy(np.ascontiguousarray(q_real[r * qlen:(r + 1) * qlen]))
        vis = torch.tensor([[i < L - qlen + j + 1 for i in range(L)] for j in range(qlen)])
        qq = q.permute(1, 0, 2).unsqueeze(0)       # [1, H, qlen, 576]
        k = kv.unsqueeze(0).unsqueeze(0)           # [1, 1, L, 576]
        v = kv[:, :512].unsqueeze(0).unsqueeze(0) * kv_scale
        scale = sm_scale * kv_scale
        out = torch.nn.functional.scaled_dot_product_attention(
            qq, k.expand(1, H, L, 576), v.expand(1, H, L, 512), attn_mask=vis, scale=scale)
        scores = torch.matmul(qq, k.expand(1, H, L, 576).transpose(-1, -2)) * scale
        scores = scores.masked_fill(~vis, -math.inf)
        l = torch.logsumexp(scores, dim=-1)        # [1, H, qlen]
        o[r * qlen:(r + 1) * qlen] = out[0].permute(1, 0, 2).numpy()
        lse[r * qlen:(r + 1) * qlen] = l[0].permute(1, 0).numpy()
    return o, lse


def _tiny_problem(rng, lens, H, qlen, kv_scale=1.0, std=0.5):
    lens = np.array(lens)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(lens.sum())
    nslots = max(1, int(T * 1.25) + 3)
    indices = rng.permutation(nslots)[:T].astype(np.int32)
    kv = np.full((nslots, 576), 0x7F, dtype=np.uint8)  # unused rows are NaN
    xs = synth.to_bf16_bits(rng.standard_normal((T, 576)).astype(np.float32) * std)
    scaled = _bf16(xs).to(torch.float32) / kv_scale   # library fp8 cast makes the test cache
    kv[indices] = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q = synth.to_bf16_bits(rng.standard_normal((len(lens) * qlen, H, 576)).astype(np.float32))
    return q, kv, indptr, indices


@pytest.mark.parametrize("lens,H,qlen,kv_scale", [
    ([37, 64], 16, 1, 1.0),
    ([5, 1, 0, 33], 3, 1, 0.05),
    ([9, 16, 4], 2, 4, 0.05),
    ([20, 8], 4, 8, 0.5),
])
def test_attention_matches_library_sdpa(oracle, lens, H, qlen, kv_scale):
    rng = np.random.default_rng(len(lens) * 100 + H)
    q, kv, indptr, indices = _tiny_problem(rng, lens, H, qlen, kv_scale)
    sm = 1 / math.sqrt(192)
    b, _ = oracle.split_bounds(indptr, 1, 1, 1)
    o, lse = oracle.decode_partial(q, kv, indptr, indices, b, qlen, sm, kv_scale)
    ro, rl = _sdpa_reference(q, kv, indptr, indices, qlen, sm, kv_scale)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse[0]), fin)
    np.testing.assert_allclose(lse[0][fin], rl[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0][fin], ro[fin], rtol=0, atol=1e-12)
    assert (o[0][~fin] == 0).all()


def test_attention_closed_forms(oracle):
    rng = np.random.default_rng(7)
    sm, kv_scale = 0.1, 0.25
    # L = 1: o = kv_scale * v0, LSE = s0
    q, kv, indptr, indices = _tiny_problem(rng, [1], 4, 1, kv_scale)
    b, _ = oracle.split_bounds(indptr, 1, 1, 1)
    o, lse = oracle.decode_partial(q, kv, indptr, indices, b, 1, sm, kv_scale)
    row = oracle.fp8_decode(kv[indices[0]])
    qd = oracle.bf16_decode(q[0])
    np.testing.assert_allclose(o[0, 0], kv_scale * row[None, :512].repeat(4, 0), atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], sm * kv_scale * (qd @ row), atol=1e-12)
    # q = 0: uniform weights, o = kv_scale * mean(v), LSE = ln n
    q, kv, indptr, indices = _tiny_problem(rng, [11], 2, 1, kv_scale)
    q[:] = 0
    b, _ = oracle.split_bounds(indptr, 1, 1, 1)
    o, lse = oracle.decode_partial(q, kv, indptr, indices, b, 1, sm, kv_scale)
    v = oracle.fp8_decode(kv[indices])[:, :512]
    np.testing.assert_allclose(o[0, 0, 0], kv_scale * v.mean(0), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(11), atol=1e-14)
    # identical keys on the scored dims: q zero on the latent, rows sharing
    # their rope bytes -> equal scores -> o = mean of the latents, LSE = s + ln n
    q, kv, indptr, indices = _tiny_problem(rng, [9], 3, 1, kv_scale)
    q[:, :, :512] = 0
    kv[indices, 512:] = kv[indices[0], 512:]
    b, _ = oracle.split_bounds(indptr, 1, 1, 1)
    o, lse = oracle.decode_partial(q, kv, indptr, indices, b, 1, sm, kv_scale)
    v = oracle.fp8_decode(kv[indices])
    s0 = sm * kv_scale * (oracle.bf16_decode(q[0]) @ v[0])
    np.testing.assert_allclose(o[0, 0], kv_scale * v[:, :512].mean(0)[None].repeat(3, 0), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], s0 + np.log(9), atol=1e-12)
    # empty request: LSE = -inf and o = 0
    q, kv, indptr, indices = _tiny_problem(rng, [0, 3], 2, 1, kv_scale)
    o, lse = oracle.decode_partial(q, kv, indptr, indices, oracle.split_bounds(indptr, 1, 1, 1)[0], 1, sm,
                                   kv_scale)
    assert np.isneginf(lse[0, 0]).all() and (o[0, 0] == 0).all() and np.isfinite(lse[0, 1]).all()


def test_causal_window_rows_see_prefix(oracle):
    # row j of a qlen window equals a qlen=1 query over the first L-qlen+j+1 tokens
    rng = np.random.default_rng(8)
    qlen, L, H = 4, 10, 2
    q, kv, indptr, indices = _tiny_problem(rng, [L], H, qlen)
    sm = 0.07
    o, lse = oracle.decode_partial(q, kv, indptr, indices, oracle.split_bounds(indptr, 1, 1, 1)[0], qlen,
                                   sm, 1.0)
    for j in range(qlen):
        n = L - qlen + j + 1
        ip = np.array([0, n], dtype=np.int32)
        o1, l1 = oracle.decode_partial(q[j:j + 1], kv, ip, indices[:n], oracle.split_bounds(ip, 1, 1, 1)[0],
                                       1, sm, 1.0)
        np.testing.assert_array_equal(o1[0, 0], o[0, j])
        np.testing.assert_array_equal(l1[0, 0], lse[0, j])


# --------------------------------------------------- fp8 query (q8, q_scale)

def _q8_codes(rng, shape, std=16.0):
    """E4M3 codes of N(0, std^2) draws by torch's cast (all finite: the draws
    stay far below the format's 448)."""
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * np.float32(std))
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("lens,H,qlen,q_scale", [
    ([37, 64], 16, 1, 0.0625),
    ([5, 1, 0, 33], 3, 1, 0.03),
    ([9, 16, 4], 2, 4, 0.07),
])
def test_attention_q8_matches_library_sdpa(oracle, lens, H, qlen, q_scale):
    # the fp8 query stands for q_scale * D(q8): torch's fp8 decode times the
    # scale, then torch SDPA
    rng = np.random.default_rng(len(lens) * 10 + H)
    _, kv, indptr, indices = _tiny_problem(rng, lens, H, qlen, 0.05)
    q8 = _q8_codes(rng, (len(lens) * qlen, H, 576))
    sm = 1 / math.sqrt(192)
    b, _ = oracle.split_bounds(indptr, 1, 1, 1)
    o, lse = oracle.decode_partial(q8, kv, indptr, indices, b, qlen, sm, 0.05, q_scale=q_scale)
    q_real = _decode_kv(q8).numpy() * q_scale
    ro, rl = _sdpa_reference(q8, kv, indptr, indices, qlen, sm, 0.05, q_real=q_real)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse[0]), fin)
    np.testing.assert_allclose(lse[0][fin], rl[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0][fin], ro[fin], rtol=0, atol=1e-12)


def test_q8_power_of_two_scale_is_the_bf16_query(oracle):
    # 2^-4 * D(code) has at most 4 significant bits: it is exactly a bf16
    # value, and the fp8 query must give bit-identical partials to that bf16
    # query (the query decode is the only difference between the two paths)
    rng = np.random.default_rng(11)
    _, kv, indptr, indices = _tiny_problem(rng, [21, 0, 40], 5, 2, 0.05)
    q8 = _q8_codes(rng, (6, 5, 576))
    real = (_decode_kv(q8).numpy() * 0.0625).astype(np.float32)
    w = real.view(np.uint32)
    assert (w & 0xFFFF == 0).all()
    qb = (w >> 16).astype(np.uint16)
    b, _ = oracle.split_bounds(indptr, 3, 1, 8)
    o8, l8 = oracle.decode_partial(q8, kv, indptr, indices, b, 2, 0.08, 0.05, q_scale=0.0625)
    ob, lb = oracle.decode_partial(qb, kv, indptr, indices, b, 2, 0.08, 0.05)
    np.testing.assert_array_equal(o8, ob)
    np.testing.assert_array_equal(l8, lb)
    # a scale that is not a power of two multiplies every score: the same as
    # the unscaled query with sm_scale * q_scale
    real1 = _decode_kv(q8).numpy().astype(np.float32)
    qb1 = (real1.view(np.uint32) >> 16).astype(np.uint16)
    o3, l3 = oracle.decode_partial(q8, kv, indptr, indices, b, 2, 0.08, 0.05, q_scale=0.03)
    o1, l1 = oracle.decode_partial(qb1, kv, indptr, indices, b, 2, 0.08 * 0.03, 0.05)
    fin = np.isfinite(l1)
    assert np.array_equal(np.isfinite(l3), fin)
    np.testing.assert_allclose(l3[fin], l1[fin], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o3, o1, rtol=0, atol=1e-13)


def test_q8_zero_query_closed_form(oracle):
    # q8 = 0: every score is 0, so LSE = ln n and o = kv_scale * mean(v)
    rng = np.random.default_rng(12)
    _, kv, indptr, indices = _tiny_problem(rng, [13], 2, 1, 0.25)
    q8 = np.zeros((1, 2, 576), dtype=np.uint8)
    o, lse = oracle.decode_partial(q8, kv, indptr, indices, oracle.split_bounds(indptr, 1, 1, 1)[0], 1,
                                   0.1, 0.25, q_scale=0.5)
    v = oracle.fp8_decode(kv[indices])[:, :512]
    np.testing.assert_allclose(lse[0, 0], np.log(13), atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 1], 0.25 * v.mean(0), atol=1e-14)


def _merge_f64(o, lse):
    """merge in double of unrounded partials (an invariant check, not a pin
    of the bf16 merge)."""
    lse = np.asarray(lse, dtype=np.float64)
    m = lse.max(0)
    out = np.zeros(o.shape[1:])
    tot = np.full(lse.shape[1:], -np.inf)
    fin = np.isfinite(m)
    w = np.where(np.isfinite(lse), np.exp(lse - np.where(fin, m, 0)[None]), 0.0)
    ssum = w.sum(0)
    tot[fin] = m[fin] + np.log(ssum[fin])
    out[fin] = (w[:, fin, None] * o[:, fin]).sum(0) / ssum[fin, None]
    return out, tot


@pytest.mark.parametrize("ns,W,mn", [(2, 256, 1), (4, 8, 3), (7, 16, 2)])
def test_split_partials_merge_to_unsplit(oracle, ns, W, mn):
    rng = np.random.default_rng(9 + ns)
    lens, H, qlen = [37, 64, 0, 19], 3, 2
    q, kv, indptr, indices = _tiny_problem(rng, lens, H, qlen, 0.05)
    sm = 1 / math.sqrt(192)
    b1, _ = oracle.split_bounds(indptr, 1, 1, 1)
    o1, l1 = oracle.decode_partial(q, kv, indptr, indices, b1, qlen, sm, 0.05)
    b, chunk = oracle.split_bounds(indptr, ns, W, mn)
    assert (np.diff(b, axis=1) > 0).sum(1).max() > 1  # some request really is split
    o, l = oracle.decode_partial(q, kv, indptr, indices, b, qlen, sm, 0.05)
    om, lm = _merge_f64(o, l)
    np.testing.assert_allclose(lm[np.isfinite(lm)], l1[0][np.isfinite(lm)], atol=1e-12)
    assert np.array_equal(np.isfinite(lm), np.isfinite(l1[0]))
    np.testing.assert_allclose(om, o1[0], atol=1e-13)


def test_page_table_permutation_invariance(oracle):
    rng = np.random.default_rng(10)
    q, kv, indptr, indices = _tiny_problem(rng, [23, 40], 4, 1)
    b, _ = oracle.split_bounds(indptr, 3, 4, 1)
    o, l = oracle.decode_partial(q, kv, indptr, indices, b, 1, 0.08, 1.0)
    perm = rng.permutation(kv.shape[0])      # move every row ...
    kv2 = np.empty_like(kv)
    kv2[perm] = kv
    idx2 = perm[indices].astype(np.int32)    # ... and its index with it
    o2, l2 = oracle.decode_partial(q, kv2, indptr, idx2, b, 1, 0.08, 1.0)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


# ------------------------------------------------------------------ merge

def test_merge_single_split_passes_through(oracle):
    rng = np.random.default_rng(11)
    o, l = synth.random_partials(rng, 1, 5, 3, p_empty=0.2)
    mo, ml = oracle.merge_lse(o, l)
    fin = np.isfinite(l[0])
    np.testing.assert_array_equal(oracle.bf16_round(mo[fin]), o[0][fin])
    np.testing.assert_array_equal(ml[fin], l[0][fin].astype(np.float64))
    assert (mo[~fin] == 0).all() and np.isneginf(ml[~fin]).all()


def test_merge_two_splits_closed_form(oracle):
    # equal LSEs: o = mean, LSE = lse + ln 2; a -inf split is ignored (NaN o)
    o = np.zeros((3, 1, 1, 512), dtype=np.uint16)
    a = synth.to_bf16_bits(np.linspace(-1, 1, 512).astype(np.float32))
    bb = synth.to_bf16_bits(np.linspace(2, -3, 512).astype(np.float32))
    o[0, 0, 0], o[1, 0, 0], o[2, 0, 0] = a, bb, synth.BF16_NAN
    lse = np.array([0.5, 0.5, -np.inf], dtype=np.float32).reshape(3, 1, 1)
    mo, ml = oracle.merge_lse(o, lse)
    np.testing.assert_allclose(mo[0, 0], (oracle.bf16_decode(a) + oracle.bf16_decode(bb)) / 2, atol=1e-15)
    np.testing.assert_allclose(ml[0, 0], 0.5 + np.log(2), atol=1e-15)
    # unequal: weights e^{l_k} / sum
    lse = np.array([0.0, math.log(3.0), -np.inf], dtype=np.float32).reshape(3, 1, 1)
    mo, ml = oracle.merge_lse(o, lse)
    e1 = math.exp(float(np.float32(math.log(3.0))))
    np.testing.assert_allclose(mo[0, 0], (oracle.bf16_decode(a) + e1 * oracle.bf16_decode(bb)) / (1 + e1),
                               atol=1e-14)
    np.testing.assert_allclose(ml[0, 0], math.log(1 + e1), atol=1e-14)


def test_merge_all_empty_and_associativity(oracle):
    rng = np.random.default_rng(12)
    o, l = synth.random_partials(rng, 4, 6, 2, p_empty=0.3)
    l[:, 0, 0] = -np.inf
    mo, ml = oracle.merge_lse(o, l)
    assert (mo[0, 0] == 0).all() and np.isneginf(ml[0, 0])
    assert not np.isnan(mo).any()
    # merging (0,1) and (2,3) separately in double, then merging the results
    # in double, equals merging all four
    f = lambda oo, ll: _merge_f64(np.where(np.isfinite(ll)[..., None], oracle.bf16_decode(oo), 0.0), ll)
    a_o, a_l = f(o[:2], l[:2])
    b_o, b_l = f(o[2:], l[2:])
    c_o, c_l = _merge_f64(np.stack([a_o, b_o]), np.stack([a_l, b_l]))
    fin = np.isfinite(ml)
    np.testing.assert_allclose(c_o[fin], mo[fin], atol=1e-13)
    np.testing.assert_allclose(c_l[fin], ml[fin], atol=1e-13)


# ----------------------------------------------------------- value + gate

def test_value_bf16_matches_numpy_matmul_and_gate(oracle):
    w = synth.make("tiny")
    rng = np.random.default_rng(13)
    S, H = w.S, w.heads
    lat = synth.to_bf16_bits(rng.standard_normal((S, H, 512)).astype(np.float32) * 0.3)
    acc, out = oracle.value_gate(lat, w.gate, w.lengths, w.qlen, w_bf16=w.w_uv)
    L = oracle.bf16_decode(lat)
    W = oracle.bf16_decode(w.w_uv)                         # [H, 128, 512]
    ref = np.einsum("shl,hvl->shv", L, W).reshape(S, H * 128)  # numpy contraction in double
    np.testing.assert_allclose(acc, ref, rtol=1e-12, atol=1e-12)
    g = oracle.bf16_decode(w.gate).astype(np.float32).astype(np.float64)
    val = oracle.bf16_decode(oracle.bf16_round(ref))
    want = oracle.bf16_round(val * expit(g))
    assert np.array_equal(out, want)


def test_value_mxfp4_matches_table_expansion(oracle):
    w = synth.make("rank_share", batch=2, len_range=(5, 9))
    rng = np.random.default_rng(14)
    S, H = w.S, w.value_heads
    lat = synth.to_bf16_bits(rng.standard_normal((S, H, 512)).astype(np.float32) * 0.3)
    acc, _ = oracle.value_gate(lat, w.gate, w.lengths, w.qlen, w_fp4=w.w_fp4, w_scale=w.w_scale)
    table = {int(l.split()[0]): float(l.split()[1]) for l in open(os.path.join(GOLDEN, "ocp_mx_e2m1.txt"))
             if l[0] != "#" and l.strip()}
    mag = np.array([table[c & 7] for c in range(16)]) * np.where(np.arange(16) >= 8, -1, 1)
    codes = np.stack([w.w_fp4 & 0xF, w.w_fp4 >> 4], -1).reshape(H, 128, 512)
    scale = 2.0 ** (w.w_scale.astype(np.float64) - 127)
    W = mag[codes] * np.repeat(scale, 32, axis=-1)
    ref = np.einsum("shl,hvl->shv", oracle.bf16_decode(lat), W).reshape(S, H * 128)
    np.testing.assert_allclose(acc, ref, rtol=1e-12, atol=1e-12)


def test_gate_closed_forms_and_empty_rows(oracle):
    rng = np.random.default_rng(15)
    B, qlen, H = 3, 2, 2
    lengths = np.array([4, 0, 1], dtype=np.int32)
    lat = synth.to_bf16_bits(rng.standard_normal((B * qlen, H, 512)).astype(np.float32))
    wuv = synth.to_bf16_bits(rng.standard_normal((H, 128, 512)).astype(np.float32) * 0.05)
    gate = np.zeros((B * qlen, H * 128), dtype=np.uint16)  # logit +0 -> sigmoid 1/2 exactly
    gate[2:4] = synth.BF16_NAN                             # empty request's rows
    lat[2:4] = synth.BF16_NAN
    acc, out = oracle.value_gate(lat, gate, lengths, qlen, w_bf16=wuv)
    keep = np.ones(B * qlen, bool)
    keep[2:4] = False
    half = oracle.bf16_decode(oracle.bf16_round(acc[keep])) / 2   # exact halving
    assert np.array_equal(oracle.bf16_decode(out[keep]), half)
    assert (out[~keep] == 0).all()                                  # +0 bits


# ------------------------------------------- query concat + fp8 quant (q8)

def _bf16_bits(x):
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_concat_quant_matches_torch_cast_in_range(oracle):
    # in range, E is torch's float8_e4m3fn cast of the binary32 quotient
    # (library routine); the layout is [ql_nope | q_pe] per (row, head)
    rng = np.random.default_rng(31)
    ql = _bf16_bits(rng.standard_normal((5, 3, 512)).astype(np.float32) * 2.0)
    pe = _bf16_bits(rng.standard_normal((5, 3, 64)).astype(np.float32) * 2.0)
    for q_scale in (0.0625, 0.03, 1.7):
        got = oracle.concat_quant_fp8(ql, pe, q_scale)
        x = torch.cat([_bf16(ql), _bf16(pe)], -1).to(torch.float32) / torch.tensor(q_scale, dtype=torch.float32)
        assert float(x.abs().max()) < 448
        want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got, want), q_scale


def test_concat_quant_is_the_cache_write_of_the_same_row(oracle):
    # the query row and a cache row of the same 576 values quantise alike
    rng = np.random.default_rng(32)
    ql = _bf16_bits(rng.standard_normal((4, 2, 512)).astype(np.float32) * 30.0)
    pe = _bf16_bits(rng.standard_normal((4, 2, 64)).astype(np.float32) * 30.0)
    got = oracle.concat_quant_fp8(ql, pe, 0.05)
    cache = oracle.kv_write(ql.reshape(8, 512), pe.reshape(8, 64), np.arange(8, dtype=np.int64),
                            np.zeros((8, 576), np.uint8), 0.05)
    assert np.array_equal(got.reshape(8, 576), cache)


def test_concat_quant_closed_forms(oracle):
    # a power-of-two scale round-trips every finite code; beyond 448 the code
    # saturates; NaN gives 0x7F; the rope part lands at columns 512..575
    codes = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.fp8_decode(codes) * 0.25
    ql = np.zeros((1, 1, 512), np.uint16)
    ql[0, 0, :codes.size] = _bf16_bits(vals)
    pe = _bf16_bits(np.array([1e6, -1e6, np.nan, 448.0 * 0.25 * 1.0625] + [0.0] * 60, np.float32))
    got = oracle.concat_quant_fp8(ql, pe.reshape(1, 1, 64), 0.25)
    assert np.array_equal(got[0, 0, :codes.size], codes)
    assert list(got[0, 0, 512:516]) == [0x7E, 0xFE, 0x7F, 0x7E]
    assert (got[0, 0, 516:] == 0).all()


# ------------------------------------------- absorbed query (W_UK, MXFP4)

def _e2m1_grid():
    """E2M1 magnitudes by code, from the OCP MX table in tests/golden."""
    table = {int(l.split()[0]): float(l.split()[1]) for l in open(os.path.join(GOLDEN, "ocp_mx_e2m1.txt"))
             if l[0] != "#" and l.strip()}
    return np.array([table[c] for c in range(8)])


def test_mxfp4_block_is_the_nearest_grid_point(oracle):
    # Every element is the E2M1 value nearest to v / 2^X (brute force over
    # the table; a tie takes the even code), times 2^X, with the OCP shared
    # exponent X = floor(log2(max |v|)) - 2 (frexp gives the exponent).
    grid = _e2m1_grid()
    rng = np.random.default_rng(41)
    for it in range(300):
        scale = 2.0 ** rng.integers(-20, 20)
        v = rng.standard_normal(32) * scale
        if it % 3 == 0:  # exact ties: midpoints of the grid at the block's exponent
            amax_exp = int(np.frexp(np.abs(v).max())[1]) - 1
            X = amax_exp - 2
            mids = (grid[:-1] + grid[1:]) / 2
            v[:7] = mids * 2.0 ** X * np.sign(rng.standard_normal(7))
            v[7] = np.abs(v).max()  # keep the block maximum
        out = oracle.mxfp4_block(v)
        X = int(np.frexp(np.abs(v).max())[1]) - 1 - 2
        a = np.abs(v) / 2.0 ** X
        q = np.abs(out) / 2.0 ** X
        for ai, qi in zip(a, q):
            d = np.abs(grid - ai)
            best = np.flatnonzero(d == d.min())
            code = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert qi == grid[code], (ai, qi)
        assert np.all((np.signbit(out) == np.signbit(v)) | (out == 0))


def test_mxfp4_block_closed_forms(oracle):
    # values on the grid of their block come back unchanged; the largest
    # element beyond 6 * 2^X is clamped to 6 * 2^X; ties go to the even code
    # (worked by hand from the OCP table: at X = 0, 0.25 -> 0, 0.75 -> 1,
    # 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4); powers of two scale
    # through; zero and non-finite blocks.
    assert np.array_equal(oracle.mxfp4_block(np.ones(32)), np.ones(32))
    on_grid = np.array([6, 4, 3, 2, 1.5, 1, 0.5, 0] * 4) * 2.0 ** -5
    assert np.array_equal(oracle.mxfp4_block(on_grid), on_grid)
    v = np.zeros(32)
    v[0] = 7.0                      # max 7: X = 0, 7 -> 6
    v[1:8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = np.zeros(32)
    want[0:8] = [6, 0, 1, 1, 2, 2, 4, 4]
    assert np.array_equal(oracle.mxfp4_block(v), want)
    rng = np.random.default_rng(42)
    x = rng.standard_normal(32)
    base = oracle.mxfp4_block(x)
    for j in (-30, -3, 5, 40):
        assert np.array_equal(oracle.mxfp4_block(x * 2.0 ** j), base * 2.0 ** j)
    assert np.array_equal(oracle.mxfp4_block(-x), -base)
    assert np.array_equal(oracle.mxfp4_block(np.zeros(32)), np.zeros(32))
    bad = x.copy()
    bad[3] = np.nan
    assert np.isnan(oracle.mxfp4_block(bad)).all()
    bad[3] = np.inf
    assert np.isnan(oracle.mxfp4_block(bad)).all()
    # a block below the E8M0 range: X is held at -127, so elements are
    # multiples of 2^-128 (the smallest E2M1 step times 2^-127)
    tiny = rng.standard_normal(32) * 2.0 ** -135
    t = oracle.mxfp4_block(tiny)
    assert np.all(np.abs(t / 2.0 ** -128 - np.round(t / 2.0 ** -128)) == 0) and np.abs(t).max() <= 6 * 2.0 ** -127


def _absorb_inputs(rng, rows, heads, scale_lo=118, scale_hi=125):
    qn = synth.to_bf16_bits(rng.standard_normal((rows, heads, 128)).astype(np.float32))
    qp = synth.to_bf16_bits(rng.standard_normal((rows, heads, 64)).astype(np.float32))
    wk = rng.integers(0, 256, (heads, 512, 64), dtype=np.uint8)
    ws = rng.integers(scale_lo, scale_hi + 1, (heads, 512, 4)).astype(np.uint8)
    return qn, qp, wk, ws


def test_absorb_query_matches_matmul_on_table_expanded_weights(oracle):
    # y = (MXFP4-quantised q_nope) @ W_K^T per head, with W_K expanded from
    # the OCP E2M1 table and 2^(s-127): numpy einsum (library routine) on the
    # block quantiser's output (pinned above); the bf16 output is y rounded,
    # q_pe is copied bit for bit
    rng = np.random.default_rng(43)
    rows, heads = 5, 3
    qn, qp, wk, ws = _absorb_inputs(rng, rows, heads)
    y, out = oracle.absorb_query(qn, qp, wk, ws)
    grid = _e2m1_grid()
    mag = np.concatenate([grid, -grid])
    W = mag[np.stack([wk & 0xF, wk >> 4], -1).reshape(heads, 512, 128)] * \
        np.repeat(2.0 ** (ws.astype(np.float64) - 127), 32, axis=-1)
    x = oracle.bf16_decode(qn)
    xq = np.stack([oracle.mxfp4_block(x[t, h, 32 * b:32 * b + 32])
                   for t in range(rows) for h in range(heads) for b in range(4)]).reshape(rows, heads, 128)
    ref = np.einsum("thk,hnk->thn", xq, W)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=0)
    assert np.array_equal(out[..., :512], oracle.bf16_round(y))
    assert np.array_equal(out[..., 512:], qp)


def test_absorb_query_fp8_matches_torch_cast_in_range(oracle):
    # the fp8 path: E(f32(y) / q_scale) and E(q_pe / q_scale) are torch's
    # float8_e4m3fn cast of the binary32 quotients (in range)
    rng = np.random.default_rng(44)
    qn, qp, wk, ws = _absorb_inputs(rng, 4, 2, 121, 125)
    for q_scale in (1.0, 0.5, 3.0):
        y, out = oracle.absorb_query(qn, qp, wk, ws, fp8=True, q_scale=q_scale)
        yq = torch.from_numpy(y.astype(np.float32)) / torch.tensor(q_scale, dtype=torch.float32)
        assert float(yq.abs().max()) < 448
        ref = yq.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(out[..., :512], ref)
        pe = torch.from_numpy(oracle.bf16_decode(qp).astype(np.float32)) / torch.tensor(q_scale, dtype=torch.float32)
        assert np.array_equal(out[..., 512:], pe.to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_absorb_query_identity_weights(oracle):
    # W_K rows that pick one k (code 2 = 1.0 at k = n % 128, scale 2^0, all
    # other codes 0): y[n] is the quantised q_nope element n % 128 itself
    rng = np.random.default_rng(45)
    rows, heads = 3, 2
    qn, qp, _, _ = _absorb_inputs(rng, rows, heads)
    wk = np.zeros((heads, 512, 64), np.uint8)
    for n in range(512):
        k = n % 128
        wk[:, n, k // 2] = 2 << (4 * (k & 1))
    ws = np.full((heads, 512, 4), 127, np.uint8)
    y, _ = oracle.absorb_query(qn, qp, wk, ws)
    x = oracle.bf16_decode(qn)
    for t in range(rows):
        for h in range(heads):
            xq = np.concatenate([oracle.mxfp4_block(x[t, h, 32 * b:32 * b + 32]) for b in range(4)])
            assert np.array_equal(y[t, h], np.tile(xq, 4))

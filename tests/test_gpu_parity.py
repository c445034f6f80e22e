"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bars: kv_write bytes and split indexing bit-exact; partial o within 1e-2
(abs, after bf16 rounding) and LSE within 1e-3 (-inf must match); merged
latent the same; gated output max|err| <= 2e-2 * max|ref|.
"""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL, OUT_REL_TOL = 1e-2, 1e-3, 2e-2


def o_err_ok(got, ref):
    """|got - ref| <= max(1e-2, 2^-7 |ref|), elementwise.  o is bf16 (and so
    is P inside the kernel), so beyond |ref| ~ 1.3 a correct result can
    differ from the rounded exact value by one bf16 ulp at its magnitude;
    below that the bound is the plain 1e-2."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return bool(np.all(np.abs(got - ref) <= np.maximum(O_TOL, np.abs(ref) * 2.0 ** -7)))


def lse_err_ok(got, ref):
    """|got - ref| <= 1e-3 plus 8 f32 ulps of |ref|: the LSE output is f32, so
    for very large scores (|LSE| ~ 1e4) its own resolution exceeds 1e-3."""
    tol = LSE_TOL + 8 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    return bool(np.all(np.abs(got - ref) <= tol))


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_fp8_amd as m

    m.lib()  # raises if the HIP library is missing: no fallback
    return m


def _np_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _announce(msg):
    print("[case]", msg, flush=True)


# ------------------------------------------------------------------ kv_write

@pytest.mark.parametrize("aligned", [True, False])
def test_kv_write_bitexact_edge_values(ops, oracle, aligned):
    """Strided views of a fused projection: 16-byte aligned sources with
    strides of a multiple of 8 (the 16-byte load path) and odd ones (the
    2-byte load path)."""
    _announce(f"kv_write edge values, aligned={aligned}")
    rng = np.random.default_rng(100)
    n, slots = 300, 401
    x = (rng.standard_normal((n, 576)) * 40).astype(np.float32)
    # ties of E4M3 at several binades, saturation, NaN, tiny values, -0
    pos = np.arange(0, 0x7F, dtype=np.uint8)
    pv = oracle.fp8_decode(pos)
    mids = ((pv[:-1] + pv[1:]) / 2).astype(np.float32)
    x[0, :len(mids)] = mids
    x[1, :len(mids)] = -mids
    x[2, :8] = [448, 449, 464, 465, 1e30, -1e30, np.inf, -np.inf]
    x[2, 8:12] = [np.nan, -0.0, 1e-30, -1e-6]
    from mla_latent_kv_fp8_amd.synth import to_bf16_bits
    bits = to_bf16_bits(x)
    o = 1536 if aligned else 1537
    fused = np.zeros((n, 2112 if aligned else 2115), dtype=np.uint16)  # strided views of a fused projection
    fused[:, o:o + 512] = bits[:, :512]
    fused[:, o + 512:o + 576] = bits[:, 512:]
    slot_map = rng.permutation(slots)[:n].astype(np.int64)
    slot_map[5] = -1
    for kv_scale in (1.0, 0.05, 3.0):
        cache = torch.full((slots, 576), 0x7F, dtype=torch.uint8, device="cuda")
        f = _bf16_dev(fused)
        ops.kv_write(f[:, o:o + 512], f[:, o + 512:o + 576], torch.from_numpy(slot_map).cuda(), cache, kv_scale)
        torch.cuda.synchronize()
        want = oracle.kv_write(fused[:, o:o + 512], fused[:, o + 512:o + 576], slot_map,
                               np.full((slots, 576), 0x7F, np.uint8), kv_scale)
        assert np.array_equal(cache.cpu().numpy(), want), kv_scale


# ----------------------------------------------------------- helpers

def _oracle_cache(oracle, w, requests=None):
    """Cache bytes the oracle writes (all rows, or only the rows of the
    given requests), then the step's new tokens."""
    cache = np.full((w.num_slots, 576), 0x7F, np.uint8)
    if requests is None:
        sel = np.arange(w.total_tokens)
    else:
        sel = np.concatenate([np.arange(w.indptr[r], w.indptr[r + 1]) for r in requests] + [np.zeros(0, int)])
    rows = w.kv_rows[sel]
    cache = oracle.kv_write(rows[:, :512], rows[:, 512:], w.indices[sel].astype(np.int64), cache, w.kv_scale)
    sm = w.slot_mapping.copy()
    if requests is not None:
        keep = np.zeros(len(sm), bool)
        per = len(sm) // w.batch
        for r in requests:
            keep[r * per:(r + 1) * per] = True
        sm[~keep] = -1
    cache = oracle.kv_write(w.new_rows[:, :512], w.new_rows[:, 512:], sm, cache, w.kv_scale)
    return cache


def _run_step(ops, w, **kw):
    from mla_latent_kv_fp8_amd.step import DeviceStep

    st = DeviceStep(w, **kw)
    st.run()
    torch.cuda.synchronize()
    return st


def _check_partials(oracle, w, st, cache, q8=None, q_scale=None):
    """Partials against the oracle's; q8 / q_scale: the fp8 query the step ran on."""
    H = w.heads
    bounds, chunk = oracle.split_bounds(w.indptr, w.num_splits, st.num_workers, st.split_min)
    import mla_latent_kv_fp8_amd as m

    lib_bounds, lib_chunk = m.split_plan(w.indptr, w.num_splits, st.num_workers, st.split_min)
    assert lib_chunk == chunk and np.array_equal(lib_bounds, bounds)
    q = np.ascontiguousarray((w.q if q8 is None else q8)[:, :H])
    o_ref, l_ref = oracle.decode_partial(q, cache, w.indptr, w.indices, bounds, w.qlen, w.sm_scale, w.kv_scale,
                                         q_scale=q_scale)
    lse = st.lse_part.cpu().numpy().astype(np.float64)
    o = oracle.bf16_decode(_np_bf16(st.o_part))
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(lse), ~fin), "empty-split pattern differs"
    assert lse_err_ok(lse[fin], l_ref[fin])
    o_ref_b = oracle.bf16_decode(oracle.bf16_round(o_ref))
    assert o_err_ok(o[fin], o_ref_b[fin]), np.abs(o[fin] - o_ref_b[fin]).max(initial=0)
    return bounds


def _check_merge_and_value(oracle, w, st):
    H, VH = w.heads, w.value_heads
    o_part = _np_bf16(st.o_part)
    lse_part = st.lse_part.cpu().numpy()
    # merge, on the GPU's own partials (same inputs on both sides)
    mo, ml = oracle.merge_lse(np.where(np.isfinite(lse_part)[..., None], o_part, 0), lse_part)
    lat = _np_bf16(st.latent)
    got = oracle.bf16_decode(lat[:, :H])
    want = oracle.bf16_decode(oracle.bf16_round(mo))
    assert o_err_ok(got, want), np.abs(got - want).max(initial=0)
    gl = st.lse.cpu().numpy()
    assert np.array_equal(np.isneginf(gl), np.isneginf(ml))
    fin = np.isfinite(ml)
    assert lse_err_ok(gl[fin], ml[fin])
    # value + gate, on the GPU's latent
    _, out_ref = oracle.value_gate(lat, w.gate, w.lengths, w.qlen, w_bf16=w.w_uv, w_fp4=w.w_fp4,
                                   w_scale=w.w_scale)
    out = _np_bf16(st.out)
    ref = oracle.bf16_decode(out_ref)
    dev = oracle.bf16_decode(out)
    scale = np.abs(ref).max()
    assert np.abs(dev - ref).max() <= OUT_REL_TOL * scale
    empty_rows = np.repeat(w.lengths == 0, w.qlen)
    assert (out[empty_rows] == 0).all(), "rows of empty requests must be +0"
    assert not np.isnan(dev[~empty_rows]).any()


# ------------------------------------------------------- small full parity

SMALL = [
    # name, batch override, length range, num_workers, split_min
    ("tiny", None, None, None, None),
    ("batch", 6, (100, 700), 8, 16),
    ("batch", 5, (1, 70), 16, 1),
    ("spec_q4", 3, (60, 300), 4, 16),
    ("spec_q8", 2, (64, 200), 4, 8),
    ("long", 2, (900, 1500), 16, 64),
    ("rank_share", 4, (100, 500), 8, 32),
]


@pytest.mark.parametrize("name,batch,lr,nw,smin", SMALL)
def test_step_parity_small(ops, oracle, name, batch, lr, nw, smin):
    from mla_latent_kv_fp8_amd import synth

    _announce(f"step parity {name} batch={batch} lengths={lr} workers={nw} min={smin}")
    w = synth.make(name, batch=batch, len_range=lr)
    st = _run_step(ops, w, num_workers=nw, split_min_tokens=smin)
    cache = _oracle_cache(oracle, w)
    assert np.array_equal(st.kv_cache.cpu().numpy(), cache), "cache bytes differ"
    _check_partials(oracle, w, st, cache)
    _check_merge_and_value(oracle, w, st)


# ------------------------------------------------------ fp8 query (q8)

Q8_SMALL = [
    # name, batch override, length range, num_workers, split_min, q_scale
    ("tiny", None, None, None, None, 0.0625),
    ("batch", 6, (100, 700), 8, 16, 0.03),
    ("batch", 5, (1, 70), 16, 1, 0.0625),
    ("spec_q4", 3, (60, 300), 4, 16, 0.07),
    ("spec_q8", 2, (64, 200), 4, 8, 0.0625),
    ("rank_share", 4, (100, 500), 8, 32, 0.05),
]


@pytest.mark.parametrize("name,batch,lr,nw,smin,q_scale", Q8_SMALL)
def test_fp8_query_parity_small(ops, oracle, name, batch, lr, nw, smin, q_scale):
    """mla_decode_partial_fp8q against the oracle on the same fp8 query
    codes and scale (16-, 32- and 48-row workgroups, ragged tails)."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"fp8 query parity {name} batch={batch} lengths={lr} q_scale={q_scale}")
    w = synth.make(name, batch=batch, len_range=lr)
    q8, _ = synth.fp8_query(np.random.default_rng(300 + (batch or 0)), w.q.shape, w.heads)
    st = DeviceStep(w, num_workers=nw, split_min_tokens=smin)
    st.q, st.q_scale = torch.from_numpy(q8).cuda(), q_scale
    st.run()
    torch.cuda.synchronize()
    cache = _oracle_cache(oracle, w)
    _check_partials(oracle, w, st, cache, q8=q8, q_scale=q_scale)
    _check_merge_and_value(oracle, w, st)


@pytest.mark.parametrize("heads", [16, 32, 96])
def test_fp8_query_power_of_two_scale_is_the_bf16_query(ops, heads, monkeypatch):
    """With q_scale = 2^-4 every decoded query element q_scale * fp8(code) is
    exactly a bf16 value, so the two entry points see the same exact
    products.  The fp8-query call forms each score on the scaled fp8 MFMA
    (128 products per instruction) and the bf16 call on the bf16 MFMA (32 per
    instruction): only the order of the f32 additions differs, and a score
    that moves in its last bits can round its bf16 P to the neighbouring
    value, which moves O by an absolute amount.  The partial LSE must agree
    to 1e-4 (f32 sums of 576 products; measured <= 1e-5), O within the
    tolerance the oracle tests use, and at least 90% of the O elements bit
    for bit (measured 97%); the empty-split pattern must be the same."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"fp8 query vs bf16 query at q_scale 2^-4 ({heads} heads)")
    spec = dict(synth.SPECS["batch"], heads=heads, heads_pad=128 if heads == 96 else heads)
    monkeypatch.setitem(synth.SPECS, "batch", spec)
    w = synth.make("batch", batch=4, len_range=(50, 900))
    q8, _ = synth.fp8_query(np.random.default_rng(17), w.q.shape, w.heads)
    real = torch.from_numpy(q8).view(torch.float8_e4m3fn).float() * 0.0625
    a = DeviceStep(w, num_workers=16, split_min_tokens=16)
    a.q, a.q_scale = torch.from_numpy(q8).cuda(), 0.0625
    b = DeviceStep(w, num_workers=16, split_min_tokens=16)
    b.q = real.to(torch.bfloat16).cuda()
    assert torch.equal(b.q.float().cpu()[:, :heads], real[:, :heads])  # exactly representable
    a.attend()
    b.attend()
    torch.cuda.synchronize()
    la, lb = a.lse_part.cpu().numpy(), b.lse_part.cpu().numpy()
    fin = np.isfinite(lb)
    assert np.array_equal(np.isfinite(la), fin) and np.array_equal(np.isneginf(la), np.isneginf(lb))
    assert np.abs(la[fin].astype(np.float64) - lb[fin]).max(initial=0) <= 1e-4
    oa, ob = _np_bf16(a.o_part)[fin], _np_bf16(b.o_part)[fin]
    fa = (oa.astype(np.uint32) << 16).view(np.float32)
    fb = (ob.astype(np.uint32) << 16).view(np.float32)
    assert o_err_ok(fa, fb), np.abs(fa.astype(np.float64) - fb).max(initial=0)
    assert (oa == ob).mean() >= 0.9


@pytest.mark.parametrize("heads", [16, 96])
def test_fp8_query_restart_on_late_spike(ops, oracle, heads, monkeypatch):
    """fp8 query: a late token aligned with one head's query outgrows the
    reference by far more than 2^64, so the piece restarts; the query codes
    held in registers must survive the restart.  Exact attention still
    holds."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"fp8 query restart on a late spike ({heads} heads)")
    spec = dict(synth.SPECS["batch"], heads=heads, heads_pad=128 if heads == 96 else heads)
    monkeypatch.setitem(synth.SPECS, "batch", spec)
    w = synth.make("batch", batch=2, len_range=(3000, 3000))
    q8, _ = synth.fp8_query(np.random.default_rng(23), w.q.shape, w.heads)
    qd = oracle.fp8_decode(q8)
    for r, tok, h in ((0, 2600, 5), (1, 1500, heads - 2)):
        row = w.indptr[r] + tok
        sign = np.where(qd[r, h] >= 0, 1.0, -1.0).astype(np.float32)
        w.kv_rows[row] = synth.to_bf16_bits(448.0 * sign)
    w.slot_mapping[:] = -1  # keep the spike rows (no new-token overwrite)
    st = DeviceStep(w, num_workers=2, split_min_tokens=1)
    st.q, st.q_scale = torch.from_numpy(q8).cuda(), 0.0625
    st.run()
    torch.cuda.synchronize()
    cache = _oracle_cache(oracle, w)
    _check_partials(oracle, w, st, cache, q8=q8, q_scale=0.0625)
    _check_merge_and_value(oracle, w, st)


@pytest.mark.parametrize("rows,heads", [(7, 5), (64, 12), (1, 96)])
def test_concat_quant_bitexact(ops, oracle, rows, heads):
    """mla_concat_quant_fp8 byte for byte against the oracle, on strided views
    (ql_nope inside a padded buffer, q_pe the rope slice of a [rows, H, 192]
    projection output, q8 with padded heads), with ties, saturation, NaN, -0
    and subnormals among the values."""
    from mla_latent_kv_fp8_amd.synth import to_bf16_bits

    _announce(f"concat_quant rows={rows} heads={heads}")
    rng = np.random.default_rng(rows * 7 + heads)
    x = (rng.standard_normal((rows, heads, 576)) * 6).astype(np.float32)
    mids = ((oracle.fp8_decode(np.arange(0, 0x7F, dtype=np.uint8))[:-1] +
             oracle.fp8_decode(np.arange(1, 0x7F, dtype=np.uint8))) / 2 * 0.25).astype(np.float32)
    flat = x.reshape(-1)
    flat[:mids.size] = mids
    flat[mids.size:2 * mids.size] = -mids
    flat[2 * mids.size:2 * mids.size + 8] = [1e9, -1e9, np.nan, -0.0, 1e-6, 113.0, 116.0, 448 * 0.25 * 1.03]
    bits = to_bf16_bits(x)
    ql_buf = np.zeros((rows, heads + 1, 528), np.uint16)
    ql_buf[:, :heads, :512] = bits[..., :512]
    proj = np.zeros((rows, heads, 192), np.uint16)
    proj[..., 128:] = bits[..., 512:]
    ql_dev = _bf16_dev(ql_buf)[:, :heads, :512]
    pe_dev = _bf16_dev(proj)[..., 128:]
    q8 = torch.full((rows, heads + 2, 584), 0x7F, dtype=torch.uint8, device="cuda")
    for q_scale in (0.25, 0.037):
        ops.concat_quant_fp8(ql_dev, pe_dev, q_scale, q8[:, :heads, :576])
        torch.cuda.synchronize()
        want = oracle.concat_quant_fp8(bits[..., :512], bits[..., 512:], q_scale)
        got = q8.cpu().numpy()
        assert np.array_equal(got[:, :heads, :576], want), q_scale
        assert (got[:, heads:] == 0x7F).all() and (got[:, :, 576:] == 0x7F).all()  # pads untouched


def test_fp8_query_chain_from_bf16_query(ops, oracle):
    """The fp8 query path of the runtime's pre/attend/post: the bf16 absorbed
    query is quantised by mla_concat_quant_fp8, then attended by
    mla_decode_partial_fp8q, merged and projected; every stage against the
    oracle (its own concat + quant, its fp8-query partials)."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("fp8 query chain: concat_quant -> partial_fp8q -> merge -> value")
    w = synth.make("batch", batch=5, len_range=(100, 900))
    H, q_scale = w.heads, 0.0625
    st = DeviceStep(w, num_workers=16, split_min_tokens=32)
    st.use_fp8_query(q_scale)  # each step: ql_nope = dims 0..511, q_pe = 512..575 of the bf16 query
    st.run()
    torch.cuda.synchronize()
    q8 = st.q
    q8_ref = oracle.concat_quant_fp8(w.q[:, :H, :512], w.q[:, :H, 512:], q_scale)
    assert np.array_equal(q8.cpu().numpy()[:, :H], q8_ref)
    cache = _oracle_cache(oracle, w)
    _check_partials(oracle, w, st, cache, q8=q8_ref, q_scale=q_scale)
    _check_merge_and_value(oracle, w, st)


@pytest.mark.parametrize("heads,qlen,fp8_q", [(7, 3, False), (40, 1, False), (5, 4, True), (40, 1, True)])
def test_rows_not_a_multiple_of_16(ops, oracle, heads, qlen, fp8_q, monkeypatch):
    """qlen * heads rows per request that leave a row group partly empty
    (21, 40, 20 rows: the 32-, 48- and 32-row blocks compute rows past the
    end on a copy of a real row and never store them), with bf16 and fp8
    queries; partials, merge and value against the oracle."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"rows not a multiple of 16: heads={heads} qlen={qlen} fp8 query={fp8_q}")
    spec = dict(synth.SPECS["spec_q4"], heads=heads, heads_pad=heads + 3, qlen=qlen, value_heads=heads)
    monkeypatch.setitem(synth.SPECS, "spec_q4", spec)
    w = synth.make("spec_q4", batch=3, len_range=(70, 400))
    st = DeviceStep(w, num_workers=6, split_min_tokens=16)
    q8, q_scale = None, None
    if fp8_q:
        q8, q_scale = synth.fp8_query(np.random.default_rng(heads), w.q.shape, w.heads)
        st.q, st.q_scale = torch.from_numpy(q8).cuda(), q_scale
    st.run()
    torch.cuda.synchronize()
    cache = _oracle_cache(oracle, w)
    _check_partials(oracle, w, st, cache, q8=q8, q_scale=q_scale)
    _check_merge_and_value(oracle, w, st)


@pytest.mark.parametrize("case", ["heads_128", "splits_1024"])
def test_maximum_sizes(ops, oracle, case, monkeypatch):
    """The largest padded head count (128 heads, no pad: row blocks of 48, 48
    and 32) and the largest split count (1024 splits of about four tokens,
    750 and 1000 of them live, so the merge takes its multi-pass path);
    partials, merge and value against the oracle."""
    from mla_latent_kv_fp8_amd import synth

    _announce(f"maximum sizes: {case}")
    if case == "heads_128":
        spec = dict(synth.SPECS["batch"], heads=128, heads_pad=128, value_heads=128, empty=1)
        monkeypatch.setitem(synth.SPECS, "batch", spec)
        w = synth.make("batch", batch=3, len_range=(100, 700))
        st = _run_step(ops, w, num_workers=8, split_min_tokens=16)
    else:
        spec = dict(synth.SPECS["batch"], batch=2, heads=16, heads_pad=16, value_heads=16, num_splits=1024,
                    fixed_lengths=[3000, 4000], empty=0)
        monkeypatch.setitem(synth.SPECS, "batch", spec)
        w = synth.make("batch")
        st = _run_step(ops, w, num_workers=4096, split_min_tokens=1)
        live = (st.lse_part.cpu().numpy() > -np.inf).sum(axis=0)
        assert live.min() == 750 and live.max() == 1000
    cache = _oracle_cache(oracle, w)
    assert np.array_equal(st.kv_cache.cpu().numpy(), cache), "cache bytes differ"
    _check_partials(oracle, w, st, cache)
    _check_merge_and_value(oracle, w, st)


HOSTPLAN = [
    # name, batch override, length range, num_workers, split_min
    ("tiny", None, None, None, None),
    ("batch", 6, (100, 700), 8, 16),      # 4 of 6 requests empty: units that start on an empty one
    ("batch", 8, (30, 60), 32, 1),
    ("batch", 5, (1, 70), 16, 1),
    ("spec_q4", 3, (60, 300), 4, 16),
    ("spec_q8", 2, (64, 200), 4, 8),
    ("long", 2, (900, 1500), 16, 64),
    ("rank_share", 4, (100, 500), 8, 32),
    ("batch", 300, (1, 12), 2, 1),       # units of more than 128 requests
    ("batch", None, None, 128, 256),     # the whole batch workload
    ("rank_share", 64, (2048, 4096), 256, 256),  # 256 workers: the largest plan
]


@pytest.mark.parametrize("name,batch,lr,nw,smin", HOSTPLAN)
def test_hostplan_is_the_in_kernel_partition_bit_for_bit(ops, name, batch, lr, nw, smin):
    """mla_decode_partial_hostplan (the partition built on the host and passed
    in the kernel arguments) against mla_decode_partial on the same cache:
    every o_part and lse_part byte equal."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"host plan vs in-kernel partition: {name} batch={batch} lengths={lr} workers={nw} min={smin}")
    w = synth.make(name, batch=batch, len_range=lr)
    st = DeviceStep(w, num_workers=nw, split_min_tokens=smin)
    st.write_new_tokens()
    got = []
    for hp in (False, True):
        st.host_plan = hp
        st.o_part.fill_(0)
        st.lse_part.fill_(0)
        st.attend()
        torch.cuda.synchronize()
        got.append((_np_bf16(st.o_part), st.lse_part.cpu().numpy().view(np.uint32)))
    assert np.array_equal(got[0][1], got[1][1]), "lse_part differs"
    assert np.array_equal(got[0][0], got[1][0]), "o_part differs"


@pytest.mark.parametrize("name,batch,lr,nw,smin", [HOSTPLAN[1], HOSTPLAN[4], HOSTPLAN[8], HOSTPLAN[9]])
def test_hostplan_fp8_query_is_the_in_kernel_partition_bit_for_bit(ops, name, batch, lr, nw, smin):
    """mla_decode_partial_fp8q_hostplan against mla_decode_partial_fp8q on the
    same fp8 query and cache: every o_part and lse_part byte equal."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"host plan vs in-kernel partition, fp8 query: {name} batch={batch} lengths={lr} workers={nw}")
    w = synth.make(name, batch=batch, len_range=lr)
    st = DeviceStep(w, num_workers=nw, split_min_tokens=smin)
    q8, q_scale = synth.fp8_query(np.random.default_rng(7), w.q.shape, w.heads)
    st.q, st.q_scale = torch.from_numpy(q8).cuda(), q_scale
    st.write_new_tokens()
    got = []
    for hp in (False, True):
        st.host_plan = hp
        st.o_part.fill_(0)
        st.lse_part.fill_(0)
        st.attend()
        torch.cuda.synchronize()
        got.append((_np_bf16(st.o_part), st.lse_part.cpu().numpy().view(np.uint32)))
    assert np.array_equal(got[0][1], got[1][1]), "lse_part differs"
    assert np.array_equal(got[0][0], got[1][0]), "o_part differs"


@pytest.mark.parametrize("host_plan", [False, True])
def test_timed_launch_is_the_untimed_launch(ops, host_plan):
    """mla_time_next_partial: the launch that takes the events writes the
    same o_part and lse_part bytes as an untimed one, its recorded duration
    is positive and within the events recorded around the call, and the pair
    is taken by that one launch (the next launch records nothing)."""
    import mla_latent_kv_fp8_amd as m
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"timed partial launch, host plan={host_plan}")
    w = synth.make("batch", batch=6, len_range=(100, 900))
    st = DeviceStep(w, num_workers=8)
    st.host_plan = host_plan
    st.write_new_tokens()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    got = []
    for timed in (False, True):
        st.o_part.fill_(0)
        st.lse_part.fill_(0)
        if timed:
            ev[2].record()
            m.time_next_partial(ev[0], ev[1])
        st.attend()
        if timed:
            ev[3].record()
        torch.cuda.synchronize()
        got.append((_np_bf16(st.o_part), st.lse_part.cpu().numpy().view(np.uint32)))
    assert np.array_equal(got[0][1], got[1][1]), "lse_part differs"
    assert np.array_equal(got[0][0], got[1][0]), "o_part differs"
    kern, outer = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    assert 0.0 < kern <= outer, (kern, outer)
    # taken: a second launch leaves the events where the first put them
    st.attend()
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == kern
    m.time_next_partial(None, None)


def test_requests_shorter_than_the_window(ops, oracle):
    """qlen 4 with requests of 1, 2, 3, 0 and 6 tokens: row j of a window
    sees max(0, L - qlen + j + 1) tokens, so the first rows of the short
    requests see none (LSE -inf in every split, latent zero), the others a
    prefix.  Partials, merge and value against the oracle."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("requests shorter than the speculative window (qlen 4)")
    w = synth.make("spec_q4", batch=5, len_range=(8, 12))
    new_len = np.array([1, 2, 3, 0, 6], dtype=np.int64)
    keep = np.concatenate([np.arange(w.indptr[r], w.indptr[r] + new_len[r]) for r in range(w.batch)])
    w.kv_rows = w.kv_rows[keep]
    w.indices = w.indices[keep]
    w.lengths = new_len.astype(np.int32)
    w.indptr = np.concatenate([[0], np.cumsum(new_len)]).astype(np.int32)
    w.slot_mapping[:] = -1  # the cache already holds every row
    st = DeviceStep(w, num_workers=3, split_min_tokens=1)
    st.run()
    torch.cuda.synchronize()
    cache = _oracle_cache(oracle, w)
    _check_partials(oracle, w, st, cache)
    _check_merge_and_value(oracle, w, st)
    lat = oracle.bf16_decode(_np_bf16(st.latent[:, :w.heads]))
    for r in range(w.batch):
        for j in range(w.qlen):
            t = r * w.qlen + j
            if new_len[r] - w.qlen + j + 1 <= 0:
                assert (lat[t] == 0).all() and torch.isneginf(st.lse[t]).all(), (r, j)


def test_end_to_end_chain_tiny(ops, oracle):
    """The oracle's own chain (its partials -> its merge -> its value) against
    the GPU chain, from the same inputs."""
    from mla_latent_kv_fp8_amd import synth

    _announce("end-to-end chain tiny")
    w = synth.make("tiny")
    st = _run_step(ops, w)
    cache = _oracle_cache(oracle, w)
    bounds, _ = oracle.split_bounds(w.indptr, w.num_splits, st.num_workers, st.split_min)
    o, l = oracle.decode_partial(w.q, cache, w.indptr, w.indices, bounds, w.qlen, w.sm_scale, w.kv_scale)
    ob = oracle.bf16_round(o)
    mo, ml = oracle.merge_lse(ob, l.astype(np.float32))
    lat = oracle.bf16_round(mo)
    _, out_ref = oracle.value_gate(lat, w.gate, w.lengths, w.qlen, w_bf16=w.w_uv)
    ref = oracle.bf16_decode(out_ref)
    got = oracle.bf16_decode(_np_bf16(st.out))
    assert np.abs(got - ref).max() <= OUT_REL_TOL * np.abs(ref).max()


# ------------------------------------------------------------- merge alone

@pytest.mark.parametrize("ns,rows,heads", [(1, 7, 3), (2, 5, 16), (16, 9, 12), (64, 3, 5), (70, 2, 4)])
def test_merge_parity(ops, oracle, ns, rows, heads):
    from mla_latent_kv_fp8_amd import synth

    _announce(f"merge ns={ns} rows={rows} heads={heads}")
    rng = np.random.default_rng(ns * 31 + rows)
    o, l = synth.random_partials(rng, ns, rows, heads, p_empty=0.3)
    l[:, 0, 0] = -np.inf  # a fully empty (row, head)
    # strided device views: pad heads and the split stride
    o_dev = torch.zeros((ns, rows, heads + 3, 512), dtype=torch.bfloat16, device="cuda")
    o_dev[:, :, :heads] = _bf16_dev(o)
    l_dev = torch.zeros((ns, rows, heads + 1), dtype=torch.float32, device="cuda")
    l_dev[:, :, :heads] = torch.from_numpy(l).cuda()
    out = torch.full((rows, heads, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
    ops.merge_lse(o_dev[:, :, :heads], l_dev[:, :, :heads], out, lse)
    torch.cuda.synchronize()
    mo, ml = oracle.merge_lse(np.where(np.isfinite(l)[..., None], o, 0), l)
    got = _np_bf16(out)
    if ns == 1:  # a single split passes through bit-exactly
        fin = np.isfinite(l[0])
        assert np.array_equal(got[fin], o[0][fin])
        assert np.array_equal(lse.cpu().numpy()[fin], l[0][fin])
    err = np.abs(oracle.bf16_decode(got) - oracle.bf16_decode(oracle.bf16_round(mo))).max()
    assert err <= O_TOL
    g = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(g), np.isneginf(ml))
    fin = np.isfinite(ml)
    assert np.abs(g[fin] - ml[fin]).max() <= LSE_TOL
    assert (got[~fin] == 0).all()


# -------------------------------------------------------------- value alone

@pytest.mark.parametrize("fmt,rows,qlen,heads", [("bf16", 64, 1, 96), ("bf16", 13, 1, 5), ("mxfp4", 256, 4, 96),
                                                 ("mxfp4", 20, 4, 3)])
def test_value_gate_parity(ops, oracle, fmt, rows, qlen, heads):
    from mla_latent_kv_fp8_amd.synth import to_bf16_bits, BF16_NAN

    _announce(f"value_gate {fmt} rows={rows} qlen={qlen} heads={heads}")
    rng = np.random.default_rng(rows + heads)
    B = rows // qlen
    lengths = rng.integers(0, 5, B).astype(np.int32)
    lengths[0] = 0
    lat = to_bf16_bits(rng.standard_normal((rows, heads, 512)).astype(np.float32) * 0.3)
    gate = to_bf16_bits(rng.standard_normal((rows, heads * 128)).astype(np.float32))
    gate[:, :7] = 0  # logit 0: the output is exactly bf16(acc) / 2
    empty = np.repeat(lengths == 0, qlen)
    gate[empty] = BF16_NAN
    lat[empty] = BF16_NAN
    out = torch.full((rows, heads * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    if fmt == "bf16":
        wuv = to_bf16_bits(rng.standard_normal((heads, 128, 512)).astype(np.float32) * 0.044)
        ops.value_gate(_bf16_dev(lat), _bf16_dev(gate), torch.from_numpy(lengths).cuda(), out, qlen=qlen,
                       w_uv=_bf16_dev(wuv))
        acc, ref = oracle.value_gate(lat, gate, lengths, qlen, w_bf16=wuv)
    else:
        w4 = rng.integers(0, 256, (heads, 128, 256), dtype=np.uint8)
        ws = rng.integers(118, 125, (heads, 128, 16)).astype(np.uint8)
        ops.value_gate(_bf16_dev(lat), _bf16_dev(gate), torch.from_numpy(lengths).cuda(), out, qlen=qlen,
                       w_fp4=torch.from_numpy(w4).cuda(), w_scale=torch.from_numpy(ws).cuda())
        acc, ref = oracle.value_gate(lat, gate, lengths, qlen, w_fp4=w4, w_scale=ws)
    torch.cuda.synchronize()
    got = _np_bf16(out)
    assert (got[empty] == 0).all()
    g, r = oracle.bf16_decode(got[~empty]), oracle.bf16_decode(ref[~empty])
    assert np.abs(g - r).max() <= OUT_REL_TOL * np.abs(r).max()
    # gate logit 0: sigma = 1/2 exactly, so out = bf16(acc) / 2 with no second
    # rounding.  The GPU accumulates in f32 in its own order, so bf16(acc)
    # is compared bit for bit where the oracle's exact acc lies farther from
    # a bf16 rounding midpoint than any f32 accumulation error can move it
    # (2^-18 of the sum of |terms|: 16 K-steps of 32 exact products each
    # add at most about 2^-19 of it), and within one bf16 ulp elsewhere.
    acc0 = acc[~empty][:, :7]
    if fmt == "bf16":
        w_dec = oracle.bf16_decode(wuv)
    else:
        w_dec = (oracle.e2m1_decode(np.stack([w4 & 15, w4 >> 4], -1).reshape(heads, 128, 512))
                 * np.repeat(oracle.e8m0_decode(ws), 32, axis=-1))
    lat_ne = oracle.bf16_decode(lat[~empty])
    abs_terms = np.abs(lat_ne[:, 0]) @ np.abs(w_dec[0, :7]).T  # head 0, outputs 0..6
    want = oracle.bf16_round(oracle.bf16_decode(oracle.bf16_round(acc0)) * 0.5)
    half = got[~empty][:, :7]
    mag = np.abs(acc0)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7)
    frac = mag / ulp - np.floor(mag / ulp)
    far = np.abs(frac - 0.5) * ulp > 2.0 ** -18 * abs_terms
    assert far.mean() > 0.5  # the exact check covers most entries
    assert np.array_equal(half[far], want[far])
    near_err = np.abs(oracle.bf16_decode(half[~far]) - oracle.bf16_decode(want[~far]))
    assert np.all(near_err <= ulp[~far] / 2 * 1.0000001)


def test_value_gate_mxfp4_edge_scales(ops, oracle):
    """MXFP4 W_UV with E8M0 scale bytes at the edges of the format, against
    the oracle's exact decode (e2m1 * 2^(s-127)):
      head 0: every scale 0x00 (2^-127, so most decoded weights are bf16
              subnormals), latent scaled by 2^100;
      head 1: some 32-element blocks with scale 0xFF (NaN): exactly the
              outputs whose weight row holds such a block are NaN (rows of
              non-empty requests), all others finite;
      head 2: scales 250 and 252 (weights up to 6 * 2^125, the largest that
              bf16 holds for every code), latent scaled by 2^-110;
      head 3: scales drawn over [1, 200] per block, a plain latent.
    Each head is compared against its own largest reference output."""
    from mla_latent_kv_fp8_amd.synth import to_bf16_bits, BF16_NAN

    _announce("value_gate mxfp4 edge scales")
    rng = np.random.default_rng(4242)
    heads, qlen, B = 4, 1, 24
    rows = B * qlen
    lengths = rng.integers(1, 5, B).astype(np.int32)
    lengths[3] = 0
    latf = rng.standard_normal((rows, heads, 512)) * 0.3
    latf[:, 0] *= 2.0 ** 100
    latf[:, 2] *= 2.0 ** -110
    lat = to_bf16_bits(latf.astype(np.float32))
    gate = to_bf16_bits(rng.standard_normal((rows, heads * 128)).astype(np.float32))
    empty = np.repeat(lengths == 0, qlen)
    gate[empty] = BF16_NAN
    w4 = rng.integers(0, 256, (heads, 128, 256), dtype=np.uint8)
    ws = np.empty((heads, 128, 16), np.uint8)
    ws[0] = 0
    ws[1] = rng.integers(118, 125, (128, 16))
    nan_blocks = rng.random((128, 16)) < 0.03
    nan_blocks[5, 3] = True
    ws[1][nan_blocks] = 0xFF
    ws[2] = rng.choice(np.array([250, 252], np.uint8), (128, 16))
    ws[3] = rng.integers(1, 201, (128, 16))
    out = torch.full((rows, heads * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ops.value_gate(_bf16_dev(lat), _bf16_dev(gate), torch.from_numpy(lengths).cuda(), out, qlen=qlen,
                   w_fp4=torch.from_numpy(w4).cuda(), w_scale=torch.from_numpy(ws).cuda())
    _, ref = oracle.value_gate(lat, gate, lengths, qlen, w_fp4=w4, w_scale=ws)
    torch.cuda.synchronize()
    got = _np_bf16(out)
    assert (got[empty] == 0).all()
    g = oracle.bf16_decode(got[~empty]).reshape(-1, heads, 128)
    r = oracle.bf16_decode(ref[~empty]).reshape(-1, heads, 128)
    nan_rows = nan_blocks.any(axis=1)  # output v of head 1 is NaN
    assert np.array_equal(np.isnan(r[:, 1]), np.broadcast_to(nan_rows, r[:, 1].shape))
    assert np.array_equal(np.isnan(g), np.isnan(r))
    for h in range(heads):
        fin = ~np.isnan(r[:, h])
        assert np.all(np.isfinite(g[:, h][fin])), h
        scale = np.abs(r[:, h][fin]).max()
        assert scale > 0, h
        assert np.abs(g[:, h][fin] - r[:, h][fin]).max() <= OUT_REL_TOL * scale, h


# ------------------------------------------------ absorbed query (W_UK)

def _ulp_far(x, margin, mant_bits, emin):
    """True where x lies farther than `margin` from a rounding midpoint of a
    binary format with `mant_bits` fraction bits and least exponent emin."""
    mag = np.abs(x)
    e = np.floor(np.log2(np.maximum(mag, 1e-300)))
    ulp = 2.0 ** (np.maximum(e, emin) - mant_bits)
    frac = mag / ulp - np.floor(mag / ulp)
    return np.abs(frac - 0.5) * ulp > margin, ulp


@pytest.mark.parametrize("rows,heads,fp8,q_scale", [(5, 3, False, None), (37, 12, True, 0.5), (256, 96, False, None),
                                                    (256, 96, True, 1.0 / 16), (16, 1, True, 2.0)])
def test_absorb_query_parity(ops, oracle, rows, heads, fp8, q_scale):
    """mla_absorb_query against the oracle: q_nope and q_pe are strided
    slices of one [rows, heads, 192] projection output, the result goes into
    a query buffer with 4 pad heads (left untouched).  Blocks with a NaN,
    all zeros, values below the binary32 normal range and exact E2M1 ties
    are included.  The rope part is bit-exact; each product is compared bit
    for bit (bf16, or the fp8 code) where the exact value lies farther from a
    rounding midpoint than a binary32 sum of 128 exact products can move it
    (2^-18 of the sum of |terms|), within one unit elsewhere."""
    from mla_latent_kv_fp8_amd.synth import to_bf16_bits

    _announce(f"absorb_query rows={rows} heads={heads} fp8={fp8}")
    rng = np.random.default_rng(rows * 7 + heads)
    proj = rng.standard_normal((rows, heads, 192)).astype(np.float32)
    proj[0, 0, 5] = np.nan                          # a NaN block: its row's products are NaN
    proj[rows - 1, heads - 1, 32:64] = 0.0          # an all-zero block
    proj[rows // 2, 0, 64:96] *= 2.0 ** -130        # values below the binary32 normal range
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mids = (grid[:-1] + grid[1:]) / 2
    proj[min(1, rows - 1), heads // 2, 96:103] = mids * 0.25   # exact ties at X = -2
    proj[min(1, rows - 1), heads // 2, 103] = 1.5              # the block maximum: X = -2
    pb = to_bf16_bits(proj)
    wk = rng.integers(0, 256, (heads, 512, 64), dtype=np.uint8)
    ws = rng.integers(119, 126, (heads, 512, 4)).astype(np.uint8)
    qn, qp = pb[..., :128], pb[..., 128:]
    y, ref = oracle.absorb_query(qn, qp, wk, ws, fp8=fp8, q_scale=q_scale if fp8 else 1.0)
    hp = heads + 4
    pd = _bf16_dev(pb)
    if fp8:
        out = torch.full((rows, hp, 576), 0x5A, dtype=torch.uint8, device="cuda")
    else:
        out = torch.full((rows, hp, 576), 1234.0, dtype=torch.bfloat16, device="cuda")
    ops.absorb_query(pd[..., :128], pd[..., 128:], torch.from_numpy(wk).cuda(), torch.from_numpy(ws).cuda(), out,
                     q_scale=q_scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy() if fp8 else _np_bf16(out)
    pad = got[:, heads:]
    assert (pad == (0x5A if fp8 else to_bf16_bits(np.float32(1234.0)))).all()
    got = got[:, :heads]
    assert np.array_equal(got[..., 512:], ref[..., 512:])            # rope part: bit-exact
    # sum of |terms| per product, from the oracle's quantised rows and the
    # table-expanded weights
    mag = np.concatenate([grid, -grid])
    W = mag[np.stack([wk & 0xF, wk >> 4], -1).reshape(heads, 512, 128)] * \
        np.repeat(2.0 ** (ws.astype(np.float64) - 127), 32, axis=-1)
    x = oracle.bf16_decode(qn)
    xq = np.stack([oracle.mxfp4_block(x[t, h, 32 * b:32 * b + 32])
                   for t in range(rows) for h in range(heads) for b in range(4)]).reshape(rows, heads, 128)
    nan_th = np.isnan(xq).any(-1)
    xq = np.nan_to_num(xq)
    abs_terms = np.einsum("thk,hnk->thn", np.abs(xq), np.abs(W))
    margin = 2.0 ** -18 * abs_terms
    g, r = got[..., :512], ref[..., :512]
    if fp8:
        assert (g[nan_th] == 0x7F).all() and (r[nan_th] == 0x7F).all()
        v = y.astype(np.float32).astype(np.float64) / q_scale
        far, _ = _ulp_far(v, margin / q_scale, 3, -6)
        keep = ~nan_th[..., None] & np.ones_like(far)
        assert np.array_equal(g[keep & far], r[keep & far])
        gd, rd = oracle.fp8_decode(g[keep & ~far]), oracle.fp8_decode(r[keep & ~far])
        _, ulp = _ulp_far(rd, 0, 3, -6)
        assert np.all(np.abs(gd - rd) <= ulp * 1.0000001)
    else:
        assert np.isnan(oracle.bf16_decode(g[nan_th])).all()
        far, ulp = _ulp_far(y, margin, 7, -126)
        keep = ~nan_th[..., None] & np.ones_like(far)
        assert far[keep].mean() > 0.5
        assert np.array_equal(g[keep & far], r[keep & far])
        assert np.all(np.abs(oracle.bf16_decode(g[keep & ~far]) - oracle.bf16_decode(r[keep & ~far]))
                      <= ulp[keep & ~far] * 1.0000001)


# ------------------------------------------- fused merge + value + gate

@pytest.mark.parametrize("fmt,ns,rows,qlen,heads", [("bf16", 16, 64, 1, 96), ("bf16", 3, 13, 1, 5),
                                                    ("mxfp4", 5, 40, 4, 12), ("bf16", 1, 20, 4, 3),
                                                    ("mxfp4", 70, 9, 1, 9)])
def test_merge_value_gate_equals_the_two_calls(ops, oracle, fmt, ns, rows, qlen, heads):
    """mla_merge_value_gate bit for bit against mla_merge_lse followed by
    mla_value_gate on the same partials (empty splits, fully empty rows,
    empty requests with NaN gates, ragged row blocks, one split and more than
    64), and the output against the oracle's merge + value + gate."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.synth import BF16_NAN, to_bf16_bits

    _announce(f"merge_value_gate {fmt} splits={ns} rows={rows} qlen={qlen} heads={heads}")
    rng = np.random.default_rng(ns * 13 + rows + heads)
    o, l = synth.random_partials(rng, ns, rows, heads, p_empty=0.3)
    l[:, 0, 0] = -np.inf  # a fully empty (row, head)
    B = rows // qlen
    lengths = rng.integers(1, 5, B).astype(np.int32)
    lengths[0] = 0
    empty = np.repeat(lengths == 0, qlen)
    l[:, empty] = -np.inf  # an empty request has no live split
    gate = to_bf16_bits(rng.standard_normal((rows, heads * 128)).astype(np.float32))
    gate[empty] = BF16_NAN
    o_dev = torch.zeros((ns, rows, heads + 1, 512), dtype=torch.bfloat16, device="cuda")
    o_dev[:, :, :heads] = _bf16_dev(o)
    o_dev = o_dev[:, :, :heads]
    l_dev = torch.from_numpy(l).cuda()
    g_dev, len_dev = _bf16_dev(gate), torch.from_numpy(lengths).cuda()
    if fmt == "bf16":
        wkw = dict(w_uv=_bf16_dev(to_bf16_bits(rng.standard_normal((heads, 128, 512)).astype(np.float32) * 0.044)))
        okw = dict(w_bf16=ops_np(wkw["w_uv"]))
    else:
        w4 = rng.integers(0, 256, (heads, 128, 256), dtype=np.uint8)
        ws = rng.integers(118, 125, (heads, 128, 16)).astype(np.uint8)
        wkw = dict(w_fp4=torch.from_numpy(w4).cuda(), w_scale=torch.from_numpy(ws).cuda())
        okw = dict(w_fp4=w4, w_scale=ws)
    # the two calls
    lat = torch.full((rows, heads, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse2 = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
    out2 = torch.full((rows, heads * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ops.merge_lse(o_dev, l_dev, lat, lse2)
    ops.value_gate(lat, g_dev, len_dev, out2, qlen=qlen, **wkw)
    # the fused call
    lse1 = torch.full((rows, heads), 7.0, dtype=torch.float32, device="cuda")
    out1 = torch.full((rows, heads * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ops.merge_value_gate(o_dev, l_dev, g_dev, len_dev, out1, qlen=qlen, lse=lse1, **wkw)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.isneginf(), lse2.isneginf())
    fin = torch.isfinite(lse2)
    assert torch.equal(lse1[fin], lse2[fin])
    # against the oracle: its merge of the same partials, then its value + gate
    mo, _ = oracle.merge_lse(np.where(np.isfinite(l)[..., None], o, 0), l)
    _, ref = oracle.value_gate(oracle.bf16_round(mo), gate, lengths, qlen, **okw)
    got, want = oracle.bf16_decode(_np_bf16(out1)), oracle.bf16_decode(ref)
    assert (_np_bf16(out1)[empty] == 0).all()
    assert np.abs(got - want).max() <= OUT_REL_TOL * np.abs(want).max()


def ops_np(t):
    return _np_bf16(t)


@pytest.mark.parametrize("name,batch,lr,nw,smin", [("batch", 6, (100, 700), 8, 16), ("spec_q4", 3, (60, 300), 4, 16)])
def test_step_with_fused_post(ops, oracle, name, batch, lr, nw, smin):
    """The whole step with the fused merge + value + gate: outputs against
    the oracle, and bit for bit against the step with the two calls."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"step with fused post {name} batch={batch} lengths={lr}")
    w = synth.make(name, batch=batch, len_range=lr)
    a = DeviceStep(w, num_workers=nw, split_min_tokens=smin)
    a.run()
    b = DeviceStep(w, num_workers=nw, split_min_tokens=smin)
    b.fused_post = True
    b.run()
    torch.cuda.synchronize()
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    assert torch.equal(a.lse, b.lse)
    lat = _np_bf16(a.latent)
    _, out_ref = oracle.value_gate(lat, w.gate, w.lengths, w.qlen, w_bf16=w.w_uv)
    ref, got = oracle.bf16_decode(out_ref), oracle.bf16_decode(_np_bf16(b.out))
    assert np.abs(got - ref).max() <= OUT_REL_TOL * np.abs(ref).max()


# ------------------------------------------------------- invariants / edges

def test_page_table_permutation_bitwise(ops):
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("page-table permutation")
    w = synth.make("batch", batch=4, len_range=(200, 600))
    a = DeviceStep(w, num_workers=8, split_min_tokens=32)
    a.attend(); a.merge()
    rng = np.random.default_rng(5)
    perm = torch.from_numpy(rng.permutation(w.num_slots)).cuda()
    b = DeviceStep(w, num_workers=8, split_min_tokens=32)
    kv2 = torch.empty_like(b.kv_cache)
    kv2[perm] = b.kv_cache
    b.kv_cache = kv2
    b.indices = perm[b.indices.long()].to(torch.int32)
    b.attend(); b.merge()
    torch.cuda.synchronize()
    assert torch.equal(a.latent.view(torch.int16), b.latent.view(torch.int16))
    assert torch.equal(a.lse_part, b.lse_part)


def test_determinism_and_canaries(ops):
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("determinism + NaN canaries (batch config, reduced lengths)")
    w = synth.make("batch", batch=16, len_range=(1, 3000))
    st = DeviceStep(w, num_workers=64, split_min_tokens=64)
    st.run()
    o1 = st.out.clone(); l1 = st.lse_part.clone()
    st.run(write_new=False)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), st.out.view(torch.int16))
    assert torch.equal(l1, st.lse_part)
    live = torch.from_numpy(np.repeat(w.lengths > 0, w.qlen)).cuda()
    assert not torch.isnan(st.out[live].float()).any()       # padded heads 96..127 (NaN) never read
    assert (st.out[~live].view(torch.int16) == 0).all()


def test_bad_index_poisons_not_faults(ops):
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("out-of-range cache index reads as NaN")
    w = synth.make("tiny")
    st = DeviceStep(w)
    idx = st.indices.clone()
    idx[3] = w.num_slots + 1000
    st.indices = idx
    st.attend(); st.merge()
    torch.cuda.synchronize()
    assert torch.isnan(st.latent[0, :w.heads].float()).all()     # request 0 uses the bad row
    assert not torch.isnan(st.latent[1, :w.heads].float()).any()


def test_empty_inputs_and_all_empty_requests(ops):
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("empty batch / all requests empty")
    w = synth.make("tiny")
    w.lengths[:] = 0
    w.indptr[:] = 0
    w.indices = w.indices[:1]  # never read: every request is empty
    w.kv_rows = w.kv_rows[:0]
    w.slot_mapping[:] = -1
    st = DeviceStep(w)
    st.o_part.fill_(float("nan"))
    st.run()
    torch.cuda.synchronize()
    assert torch.isneginf(st.lse_part).all()
    assert (st.latent.view(torch.int16) == 0).all()
    assert (st.out.view(torch.int16) == 0).all()
    # zero-size calls are no-ops
    ops.kv_write(st.new_rows[:0, :512], st.new_rows[:0, 512:], st.slot_mapping[:0], st.kv_cache, 1.0)
    ops.merge_lse(st.o_part[:, :0], st.lse_part[:, :0], st.latent[:0, :w.heads])


def test_single_split_and_one_token(ops, oracle):
    from mla_latent_kv_fp8_amd import synth

    _announce("num_splits=1, L=1 requests")
    w = synth.make("batch", batch=3, len_range=(1, 1))
    w.num_splits = 1
    st = _run_step(ops, w, num_workers=4, split_min_tokens=1)
    cache = _oracle_cache(oracle, w)
    _check_partials(oracle, w, st, cache)
    # L = 1: o equals kv_scale times the (only) value row
    row = oracle.fp8_decode(cache[w.indices[0]])[:512] * w.kv_scale
    got = oracle.bf16_decode(_np_bf16(st.latent)[0, 0])
    assert o_err_ok(got, row)


# ------------------------------------------- full size, sampled (bench launch)

@pytest.mark.parametrize("name,fp8_q", [("batch", None), ("batch_8k", None), ("long", None), ("spec_q4", None),
                                         ("spec_q8", None), ("rank_share", None), ("batch", "codes"),
                                         ("batch", "quantised"), ("spec_q8", "codes"), ("long", "codes"),
                                         ("rank_share", "codes")])
def test_full_size_sampled(ops, oracle, name, fp8_q):
    """The bench configuration at full size; the oracle recomputes a few
    sampled requests (their cache rows written by the oracle itself).  With
    fp8_q the step runs on an fp8 query with a per-tensor scale: drawn codes,
    or the bf16 query quantised each step by mla_concat_quant_fp8 (the
    bench's --fp8-query step)."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"full-size sampled {name} fp8 query={fp8_q}")
    w = synth.make(name)
    st = DeviceStep(w)
    q_all, q_scale = w.q, None
    if fp8_q == "codes":
        q_all, q_scale = synth.fp8_query(np.random.default_rng(78), w.q.shape, w.heads)
        st.q, st.q_scale = torch.from_numpy(q_all).cuda(), q_scale
    elif fp8_q == "quantised":
        q_scale = 1.0 / 16.0
        st.use_fp8_query(q_scale)
        q_all = np.full(w.q.shape, 0x7F, np.uint8)
        q_all[:, :w.heads] = oracle.concat_quant_fp8(w.q[:, :w.heads, :512], w.q[:, :w.heads, 512:], q_scale)
    st.run()
    if fp8_q == "quantised":
        torch.cuda.synchronize()
        assert np.array_equal(st.q.cpu().numpy()[:, :w.heads], q_all[:, :w.heads])
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    nonempty = np.flatnonzero(w.lengths > 0)
    n_sample = 1 if name == "long" else 2
    sample = sorted(rng.choice(nonempty, size=min(n_sample, len(nonempty)), replace=False).tolist())
    empty = np.flatnonzero(w.lengths == 0)
    if len(empty):
        sample.append(int(empty[0]))
    cache = _oracle_cache(oracle, w, requests=sample)
    gcache = st.kv_cache.cpu().numpy()
    for r in sample:
        rows = w.indices[w.indptr[r]:w.indptr[r + 1]]
        assert np.array_equal(gcache[rows], cache[rows])
    bounds, _ = oracle.split_bounds(w.indptr, w.num_splits, st.num_workers, st.split_min)
    H = w.heads
    # sub-problem of the sampled requests, with the full problem's split bounds
    sub_ptr = np.concatenate([[0], np.cumsum([w.lengths[r] for r in sample])]).astype(np.int32)
    sub_idx = np.concatenate([w.indices[w.indptr[r]:w.indptr[r + 1]] for r in sample]).astype(np.int32)
    rows_t = np.concatenate([np.arange(r * w.qlen, (r + 1) * w.qlen) for r in sample])
    q = np.ascontiguousarray(q_all[rows_t][:, :H])
    o_ref, l_ref = oracle.decode_partial(q, cache, sub_ptr, sub_idx, bounds[sample], w.qlen, w.sm_scale,
                                         w.kv_scale, q_scale=q_scale)
    lse = st.lse_part.cpu().numpy()[:, rows_t].astype(np.float64)
    o = oracle.bf16_decode(_np_bf16(st.o_part[:, torch.from_numpy(rows_t).cuda()]))
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(lse), ~fin)
    assert np.abs(lse[fin] - l_ref[fin]).max(initial=0) <= LSE_TOL
    assert o_err_ok(o[fin], oracle.bf16_decode(oracle.bf16_round(o_ref))[fin])
    # merged latent of the sampled rows against the oracle's unsplit attention
    one = np.stack([np.zeros(len(sample), np.int32), sub_ptr[1:] - sub_ptr[:-1]], 1).astype(np.int32)
    o1, l1 = oracle.decode_partial(q, cache, sub_ptr, sub_idx, one, w.qlen, w.sm_scale, w.kv_scale,
                                   q_scale=q_scale)
    lat = oracle.bf16_decode(_np_bf16(st.latent[torch.from_numpy(rows_t).cuda(), :H]))
    f1 = np.isfinite(l1[0])
    assert o_err_ok(lat[f1], o1[0][f1])
    assert (lat[~f1] == 0).all()
    # gated output rows: oracle value+gate on the GPU latent rows
    latb = _np_bf16(st.latent[torch.from_numpy(rows_t).cuda()])
    _, out_ref = oracle.value_gate(latb, w.gate[rows_t], w.lengths[sample], w.qlen, w_bf16=w.w_uv,
                                   w_fp4=w.w_fp4, w_scale=w.w_scale)
    got = oracle.bf16_decode(_np_bf16(st.out[torch.from_numpy(rows_t).cuda()]))
    ref = oracle.bf16_decode(out_ref)
    assert np.abs(got - ref).max() <= OUT_REL_TOL * max(np.abs(ref).max(), 1e-30)


def test_rebase_on_late_spike(ops, oracle):
    """A late token whose key is aligned with a head's query: its score
    exceeds everything before it by far more than 2^64, so the running
    reference must be rebased mid-piece.  Exact attention still holds."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("late score spike (rebase path)")
    w = synth.make("tiny")
    qd = oracle.bf16_decode(w.q)
    for r, tok in ((0, 30), (1, 50)):
        row = w.indptr[r] + tok
        sign = np.where(qd[r, r % w.heads] >= 0, 1.0, -1.0).astype(np.float32)
        w.kv_rows[row] = synth.to_bf16_bits(448.0 * sign)
    w.slot_mapping[:] = -1  # keep the spike rows (no new-token overwrite)
    st = DeviceStep(w, num_workers=2, split_min_tokens=1)
    st.run()
    torch.cuda.synchronize()
    cache = _oracle_cache(oracle, w)
    _check_partials(oracle, w, st, cache)
    _check_merge_and_value(oracle, w, st)


@pytest.mark.parametrize("heads", [16, 32, 96])
def test_restart_in_a_later_segment(ops, oracle, heads, monkeypatch):
    """A score spike in the third index segment of a 5000-token piece: the
    piece restarts from its first segment (the indices are staged again)
    with the new reference.  Exact attention still holds.  16, 32 and 96
    heads run the 16-, 32- and 48-row workgroup variants."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce(f"restart from a later segment (5000-token pieces, {heads} heads)")
    spec = dict(synth.SPECS["batch"], heads=heads, heads_pad=128 if heads == 96 else heads)
    monkeypatch.setitem(synth.SPECS, "batch", spec)
    w = synth.make("batch", batch=2, len_range=(5000, 5000))
    qd = oracle.bf16_decode(w.q)
    for r, tok in ((0, 4500), (1, 2100)):
        row = w.indptr[r] + tok
        h = 7 + r
        sign = np.where(qd[r, h] >= 0, 1.0, -1.0).astype(np.float32)
        w.kv_rows[row] = synth.to_bf16_bits(448.0 * sign)
    w.slot_mapping[:] = -1  # keep the spike rows (no new-token overwrite)
    st = DeviceStep(w, num_workers=2, split_min_tokens=1)
    st.run()
    torch.cuda.synchronize()
    cache = _oracle_cache(oracle, w)
    _check_partials(oracle, w, st, cache)
    _check_merge_and_value(oracle, w, st)


def test_unit_with_many_requests(ops, oracle):
    """Units that cover more than 64 requests (short requests, two workers):
    the request offsets past the first 64 of a unit are read from global
    memory instead of the LDS cache."""
    from mla_latent_kv_fp8_amd import synth

    _announce("units of more than 64 requests")
    w = synth.make("batch", batch=180, len_range=(1, 24))
    st = _run_step(ops, w, num_workers=2, split_min_tokens=1)
    cache = _oracle_cache(oracle, w)
    assert np.array_equal(st.kv_cache.cpu().numpy(), cache)
    bounds = _check_partials(oracle, w, st, cache)
    _check_merge_and_value(oracle, w, st)


def test_restart_inside_the_speculative_window(ops, oracle):
    """qlen = 4: a spike on the second-to-last token of each request, which
    only the window's last two rows see.  Those rows restart the piece with
    a new reference; the earlier rows keep the token masked."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("restart inside the speculative window (qlen 4)")
    w = synth.make("spec_q4", batch=2, len_range=(3000, 3000))
    qd = oracle.bf16_decode(w.q)
    for r in range(2):
        row = w.indptr[r + 1] - 2
        t = r * w.qlen + w.qlen - 1  # the window's last row sees it
        h = 11 + r
        sign = np.where(qd[t, h] >= 0, 1.0, -1.0).astype(np.float32)
        w.kv_rows[row] = synth.to_bf16_bits(448.0 * sign)
    w.slot_mapping[:] = -1  # keep the spike rows (no new-token overwrite)
    st = DeviceStep(w, num_workers=2, split_min_tokens=1)
    st.run()
    torch.cuda.synchronize()
    cache = _oracle_cache(oracle, w)
    _check_partials(oracle, w, st, cache)
    _check_merge_and_value(oracle, w, st)

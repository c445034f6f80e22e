"""The cache write fused into the partials' launch
(mla_kv_write_decode_partial_hostplan and its fp8-query form) against the two
calls it replaces, mla_kv_write then mla_decode_partial_hostplan: the same
cache bytes, the same LSE bits and the same partial rows wherever the LSE is
finite (elsewhere a partial row is unspecified).  The two calls are checked
against the oracle elsewhere."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def ops():
    import mla_latent_kv_fp8_amd as m

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()
    return m


def _both(w, nw, fp8=False, smin=None):
    """Run the two calls on one DeviceStep and the fused call on another
    (same starting cache); returns both steps."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    steps = []
    for fused in (False, True):
        st = DeviceStep(w, num_workers=nw, split_min_tokens=smin)
        if fp8:
            q8, q_scale = synth.fp8_query(np.random.default_rng(5), w.q.shape, w.heads)
            st.q, st.q_scale = torch.from_numpy(q8).cuda(), q_scale
        st.o_part.fill_(0)
        st.lse_part.fill_(0)
        if fused:
            st.attend(write_new=True)
        else:
            st.write_new_tokens()
            st.host_plan = True
            st.attend()
        steps.append(st)
    torch.cuda.synchronize()
    return steps


def _assert_same(a, b):
    assert np.array_equal(a.kv_cache.cpu().numpy(), b.kv_cache.cpu().numpy()), "cache bytes differ"
    la, lb = a.lse_part.cpu().numpy(), b.lse_part.cpu().numpy()
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), "lse_part differs"
    fin = np.isfinite(la)
    oa = a.o_part.view(torch.int16).cpu().numpy()[fin]
    ob = b.o_part.view(torch.int16).cpu().numpy()[fin]
    assert np.array_equal(oa, ob), "o_part differs"


CASES = [  # name, batch, lengths, workers, split_min
    ("batch", 10, (60, 3000), 8, 1),
    ("batch", 6, (1, 200), 16, 1),
    ("spec_q4", 4, (40, 700), 8, 1),
    ("spec_q8", 3, (30, 900), 8, 16),
    ("rank_share", 6, (50, 1500), 8, 1),
    ("batch", 2, (5000, 6000), 2, 1),  # one piece per request, three index segments
    ("batch", 12, (60, 3000), 300, 1),  # more workers than the host plan takes: the in-kernel partition
    ("spec_q4", 5, (40, 900), 300, 1),
]


@pytest.mark.parametrize("name,batch,lr,nw,smin", CASES)
@pytest.mark.parametrize("fp8", [False, True])
def test_fused_write_is_the_two_calls(ops, name, batch, lr, nw, smin, fp8):
    from mla_latent_kv_fp8_amd import synth

    _announce(f"fused cache write: {name} batch={batch} lengths={lr} workers={nw} fp8={fp8}")
    w = synth.make(name, batch=batch, len_range=lr)
    a, b = _both(w, nw, fp8, smin)
    _assert_same(a, b)


def _spare_slots(w, n):
    used = np.zeros(w.num_slots, bool)
    used[w.indices] = True
    spare = np.flatnonzero(~used)
    assert spare.size >= n
    return spare[:n]


def test_fused_write_short_and_empty_requests(ops):
    """k = 4 new tokens per request: a request of 2 tokens (its first two new
    tokens precede the request: written, not attended), an empty request
    (all four written), an invalid slot (-1) and one past the cache (both
    skipped), and a new token whose cache index is not its slot."""
    from mla_latent_kv_fp8_amd import synth

    _announce("fused cache write: short and empty requests, bad slots, index mismatch")
    w = synth.make("spec_q4", batch=5, len_range=(40, 300))
    lengths = w.lengths.astype(np.int64).copy()
    # request 1 keeps 2 tokens, request 3 none
    keep, rows = [], []
    for r in range(w.batch):
        lo, hi = w.indptr[r], w.indptr[r + 1]
        n = {1: 2, 3: 0}.get(r, hi - lo)
        keep.append(w.indices[lo:lo + n])
        rows.append(w.kv_rows[lo:lo + n])
        lengths[r] = n
    w.indices = np.concatenate(keep).astype(np.int32)
    w.kv_rows = np.concatenate(rows)
    w.indptr = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    w.lengths = lengths.astype(np.int32)
    k = w.qlen
    spare = _spare_slots(w, 8)
    sm = np.full(w.batch * k, -1, np.int64)
    for r in range(w.batch):
        L = int(lengths[r])
        for j in range(k):
            pos = L - k + j
            if pos >= 0:
                sm[r * k + j] = w.indices[w.indptr[r] + pos]
    sm[1 * k + 0], sm[1 * k + 1] = spare[0], spare[1]      # before request 1's first token
    sm[3 * k:3 * k + 4] = spare[2:6]                        # the empty request
    sm[0 * k + 3] = -1                                      # skipped
    sm[2 * k + 3] = w.num_slots + 5                         # past the cache: skipped
    sm[4 * k + 2] = spare[6]                                # its cache index is not this slot
    w.slot_mapping = sm
    a, b = _both(w, 4, False, 1)
    _assert_same(a, b)
    cache = b.kv_cache.cpu().numpy()
    assert not np.array_equal(cache[spare[:7]], np.full((7, 576), 0x7F, np.uint8))


def test_fused_write_restart_on_a_new_spike(ops):
    """The new token's row is a spike aligned with a head's query, so the
    piece restarts with a new reference; both passes substitute the staged
    row."""
    from mla_latent_kv_fp8_amd import synth

    _announce("fused cache write: restart on a spike in a new token")
    w = synth.make("batch", batch=3, len_range=(800, 2500))
    qd = (w.q[:, :w.heads].astype(np.uint32) << 16).view(np.float32)
    for r in range(w.batch):
        h = (5 * r) % w.heads
        sign = np.where(qd[r, h] >= 0, 1.0, -1.0).astype(np.float32)
        w.new_rows[r] = synth.to_bf16_bits(sign * 400.0 * w.kv_scale)
    a, b = _both(w, 4, False, 1)
    _assert_same(a, b)


def test_fused_step_is_the_step(ops):
    """DeviceStep.run() with fused_write against the plain step: the same
    merged latent and output, bit for bit."""
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("fused cache write: whole step")
    w = synth.make("batch", batch=12, len_range=(100, 4000))
    outs = []
    for fused in (False, True):
        st = DeviceStep(w, num_workers=16)
        st.fused_write = fused
        st.run()
        torch.cuda.synchronize()
        outs.append((st.kv_cache.cpu().numpy(), st.latent.view(torch.int16).cpu().numpy(),
                     st.out.view(torch.int16).cpu().numpy()))
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


SCALES = [1.0, 0.5, 1024.0, 0.0173, 3.7, 1e-3, 300.0, 1.9999999, 1.0000001, 0.33333334, 7.0e-30, 3.0e+30,
          float(np.float32(np.uint32(0x3FFFFFFF).view(np.float32))), float(np.float32(np.uint32(0x3F7FFFFF).view(np.float32))),
          # 1 / scale subnormal, or infinite (a subnormal scale): the division decides
          2.0 ** 127, float(np.finfo(np.float32).max), 1e-39]


@pytest.mark.parametrize("length", [400, 20])  # new tokens past tile 2 (stored late) / in tile 0 (stored early)
def test_fused_write_encodes_every_bf16_value(ops, length):
    """Every bf16 bit pattern (NaNs, infinities, zeros and subnormals
    included) as a new token's value, under scales of every kind: the cache
    bytes the fused call writes are mla_kv_write's."""
    _announce(f"fused cache write: every bf16 value, request length {length}")
    B, k, H = 15, 8, 16
    n_new = B * k
    rng = np.random.default_rng(77)
    vals = np.concatenate([np.arange(65536, dtype=np.uint32),
                           rng.integers(0, 65536, n_new * 576 - 65536, dtype=np.uint32)]).astype(np.uint16)
    rng.shuffle(vals)
    rows = torch.from_numpy(vals.view(np.int16).reshape(n_new, 576)).cuda().view(torch.bfloat16)
    num_slots = B * length + 64
    perm = rng.permutation(num_slots).astype(np.int64)
    indices = perm[:B * length].astype(np.int32)
    slots = np.empty(n_new, np.int64)
    for r in range(B):
        slots[r * k:(r + 1) * k] = indices[r * length + length - k:(r + 1) * length]
    indptr = (np.arange(B + 1) * length).astype(np.int32)
    q = torch.zeros((B, H, 576), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((2, B, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, B, H), dtype=torch.float32, device="cuda")
    d_indptr, d_idx = torch.from_numpy(indptr).cuda(), torch.from_numpy(indices).cuda()
    d_slots = torch.from_numpy(slots).cuda()
    base = torch.randint(0, 256, (num_slots, 576), dtype=torch.uint8, device="cuda")
    for scale in SCALES:
        ref, got = base.clone(), base.clone()
        ops.kv_write(rows[:, :512], rows[:, 512:], d_slots, ref, scale)
        ops.kv_write_decode_partial_hostplan(rows[:, :512], rows[:, 512:], d_slots, q, got, d_indptr, d_idx, o, lse,
                                             indptr, qlen=1, heads=H, sm_scale=1e-30, kv_scale=scale, num_workers=8,
                                             split_min_tokens=1)
        torch.cuda.synchronize()
        assert torch.equal(ref, got), f"scale {scale!r}: {int((ref != got).sum())} bytes differ"

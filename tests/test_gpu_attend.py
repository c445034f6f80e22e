"""GPU tests of mla_decode_attend (the partials and their LSE merge in one
launch): bit for bit the partials of mla_decode_partial_hostplan followed by
mla_merge_lse, and within tolerance of the oracle's attention."""
import numpy as np
import pytest
import torch

from test_gpu_parity import _announce, _np_bf16, _oracle_cache, lse_err_ok, o_err_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_fp8_amd as m

    m.lib()  # raises if the HIP library is missing: no fallback
    return m


def _two_ways(w, nw, smin, calls=2):
    """The merged latent and LSE from attend() + merge() and from the fused
    call (run `calls` times on one workspace, every result kept)."""
    from mla_latent_kv_fp8_amd.step import DeviceStep

    st = DeviceStep(w, num_workers=nw, split_min_tokens=smin)
    st.write_new_tokens()
    H = w.heads
    st.attend()
    st.merge()
    torch.cuda.synchronize()
    ref = (_np_bf16(st.latent[:, :H]), st.lse.cpu().numpy())
    got = []
    for _ in range(calls):
        st.latent.fill_(float("nan"))
        st.lse.fill_(3.0)
        st.attend_merged()
        torch.cuda.synchronize()
        got.append((_np_bf16(st.latent[:, :H]), st.lse.cpu().numpy()))
    return st, ref, got


def _same_lse(a, b):
    """Equal f32 bits, NaN matching NaN."""
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))


FUSED = [
    # name, batch override, length range, num_workers, split_min
    ("tiny", None, None, 8, 1),
    ("batch", 6, (100, 700), 8, 16),
    ("batch", 5, (1, 70), 16, 1),
    ("spec_q4", 3, (60, 300), 4, 16),
    ("spec_q8", 2, (64, 200), 4, 8),
    ("long", 2, (900, 1500), 16, 64),
    ("rank_share", 4, (100, 500), 8, 32),
    ("batch", 300, (1, 12), 2, 1),        # units of more than 128 requests
    ("batch", None, None, 128, 256),      # the whole batch workload (4 empty requests)
    ("rank_share", 64, (2048, 4096), 256, 256),  # 256 workers: the largest plan
    ("long", 1, (20000, 20000), 128, 16),  # one request in 128 splits: the merge's multi-pass path
]


@pytest.mark.parametrize("name,batch,lr,nw,smin", FUSED)
def test_attend_is_partials_then_merge_bit_for_bit(ops, name, batch, lr, nw, smin):
    from mla_latent_kv_fp8_amd import synth

    _announce(f"fused attend vs partials + merge: {name} batch={batch} lengths={lr} workers={nw} min={smin}")
    w = synth.make(name, batch=batch, len_range=lr)
    if name == "long" and batch == 1:
        w.num_splits = 128
    _, ref, got = _two_ways(w, nw, smin)
    empty = np.repeat(w.lengths == 0, w.qlen)
    if empty.any():  # an empty request's merged rows: 0 and -inf
        assert (ref[0][empty] == 0).all() and np.isneginf(ref[1][empty]).all()
    for i, (lat, lse) in enumerate(got):
        assert np.array_equal(lat, ref[0]), f"latent differs (call {i})"
        assert _same_lse(lse, ref[1]), f"lse differs (call {i})"


def test_attend_against_the_oracle(ops, oracle):
    from mla_latent_kv_fp8_amd import synth

    _announce("fused attend vs oracle: spec_q4 batch=3 (60, 300)")
    w = synth.make("spec_q4", batch=3, len_range=(60, 300))
    st, _, got = _two_ways(w, 4, 16, calls=1)
    cache = _oracle_cache(oracle, w)
    assert np.array_equal(st.kv_cache.cpu().numpy(), cache)
    H = w.heads
    L = np.diff(w.indptr)
    bounds = np.stack([np.zeros_like(L), L], axis=1).astype(np.int32)  # one split: the whole context
    o_ref, l_ref = oracle.decode_partial(np.ascontiguousarray(w.q[:, :H]), cache, w.indptr, w.indices, bounds,
                                         w.qlen, w.sm_scale, w.kv_scale)
    lat, lse = got[0]
    fin = np.isfinite(l_ref[0])
    assert np.array_equal(np.isneginf(lse), ~fin)
    assert lse_err_ok(lse[fin], l_ref[0][fin])
    want = oracle.bf16_decode(oracle.bf16_round(o_ref[0]))
    assert o_err_ok(oracle.bf16_decode(lat)[fin], want[fin])


def test_attend_bad_index_poisons_its_request(ops):
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    _announce("fused attend: an out-of-range cache index poisons its request only")
    w = synth.make("tiny")
    st = DeviceStep(w)
    idx = st.indices.clone()
    idx[3] = w.num_slots + 1000
    st.indices = idx
    st.latent.fill_(1.0)
    st.attend_merged()
    torch.cuda.synchronize()
    H = w.heads
    lat = _np_bf16(st.latent[:, :H])
    assert (lat[0] == 0x7FC0).all(), "the poisoned request's rows are the canonical NaN"
    assert np.isnan(st.lse[0, :H].cpu().numpy()).all()
    assert not np.isnan(_bf16_to_f32(lat[1])).any()


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)

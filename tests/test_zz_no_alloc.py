"""mla_decode_attend_noalloc (the fused attention on the library's own
workspace, for callers that cannot allocate) against mla_decode_attend with
a caller's workspace: the same bits, on two calls in a row, the second
smaller; sizes beyond the library's workspace are refused."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _np_bf16(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _same_lse(a, b):
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_fp8_amd as m

    m.lib()  # raises if the HIP library is missing: no fallback
    return m


def _both(ops, name, batch, lr, nw, smin):
    from mla_latent_kv_fp8_amd import synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    print(f"[case] no-alloc attend {name} batch={batch} lengths={lr} workers={nw}", flush=True)
    w = synth.make(name, batch=batch, len_range=lr)
    st = DeviceStep(w, num_workers=nw, split_min_tokens=smin)
    st.write_new_tokens()
    H = w.heads
    st.attend_merged()  # the workspace call
    torch.cuda.synchronize()
    ref = (_np_bf16(st.latent[:, :H]), st.lse.cpu().numpy())
    lat = torch.full_like(st.latent[:, :H], float("nan"))
    lse = torch.full_like(st.lse, 3.0)
    ops.decode_attend_noalloc(st.q, st.kv_cache, st.indptr, st.indices, lat, lse, st.indptr_host, qlen=w.qlen,
                              heads=H, sm_scale=w.sm_scale, kv_scale=w.kv_scale, num_splits=w.num_splits,
                              num_workers=nw, split_min_tokens=smin)
    torch.cuda.synchronize()
    assert np.array_equal(_np_bf16(lat), ref[0]), "latent differs"
    assert _same_lse(lse.cpu().numpy(), ref[1]), "lse differs"


def test_noalloc_attend_two_calls_second_smaller(ops):
    _both(ops, "batch", 12, (500, 3000), 64, 64)  # split requests: the workspace's counters and slots are used
    _both(ops, "spec_q4", 2, (60, 200), 8, 16)     # smaller: what the first call left must not leak into it


def test_noalloc_attend_refuses_sizes_beyond_its_workspace(ops):
    from mla_latent_kv_fp8_amd import MlaError, synth
    from mla_latent_kv_fp8_amd.step import DeviceStep

    print("[case] no-alloc attend: workspace beyond the library's", flush=True)
    w = synth.make("spec_q8", batch=2, len_range=(64, 128))
    need = ops.decode_attend_workspace_bytes(w.batch, w.qlen, w.heads, 256)
    assert need > (32 << 20)
    st = DeviceStep(w, num_workers=256, split_min_tokens=8)
    lat = torch.zeros_like(st.latent[:, :w.heads])
    with pytest.raises(MlaError, match="unsupported"):
        ops.decode_attend_noalloc(st.q, st.kv_cache, st.indptr, st.indices, lat, None, st.indptr_host, qlen=w.qlen,
                                  heads=w.heads, sm_scale=w.sm_scale, kv_scale=w.kv_scale, num_splits=w.num_splits,
                                  num_workers=256, split_min_tokens=8)

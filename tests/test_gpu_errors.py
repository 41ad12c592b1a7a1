"""Error paths of the C ABI that need a device: handles used after they were
freed or destroyed (SEKV_ESTATE, checked without touching the freed object),
an index used on another context (SEKV_ESTATE), and an allocation the device
cannot satisfy (SEKV_ENOMEM, nothing left behind).  Every failing call is
refused on the host before any kernel is launched."""
import ctypes as C

import numpy as np
import pytest
import torch

from compressed_kv_cache_sekv_amd import synth
from tests import sekv_cases as SC

pytestmark = pytest.mark.gpu

ESTATE, ENOMEM = 5, 2


@pytest.fixture(scope="module")
def sl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from compressed_kv_cache_sekv_amd import lib
    return lib


@pytest.fixture(scope="module")
def case():
    return SC.make_case(synth.WORKLOADS["tiny_2k"])


def _decode_args(idx, w):
    q = torch.zeros(w.B, w.L, w.Hq, w.d, dtype=torch.bfloat16, device="cuda")
    tau = torch.zeros(w.L, w.Hq, device="cuda")
    mask = torch.zeros(w.B, w.L, w.Hq, idx.mask_words, dtype=torch.int64, device="cuda")
    out = torch.zeros(w.B, w.L, w.Hq, w.d, device="cuda")
    return q, tau, mask, out


def test_freed_index_is_refused(sl, case):
    w = case.w
    ctx = sl.Context(0)
    idx = ctx.import_index(sl.build_params(w), SC.import_arrays(case))
    q, tau, mask, out = _decode_args(idx, w)
    h = idx.h
    idx.free()
    L = sl.lib()
    assert L.sekv_route(ctx.h, h, 0, w.L, q.data_ptr(), tau.data_ptr(), 0, mask.data_ptr(), None) == ESTATE
    assert L.sekv_decode_attend(ctx.h, h, 0, w.L, q.data_ptr(), mask.data_ptr(), out.data_ptr(), None) == ESTATE
    info = sl.IndexInfo()
    assert L.sekv_index_get_info(h, C.byref(info)) == ESTATE
    L.sekv_index_free(h)           # a second free is a no-op
    # the context is unaffected
    idx2 = ctx.import_index(sl.build_params(w), SC.import_arrays(case))
    idx2.route(0, w.L, q, tau, 0, mask)
    torch.cuda.synchronize()
    idx2.free()
    ctx.close()


def test_destroyed_context_is_refused(sl, case):
    w = case.w
    ctx = sl.Context(0)
    idx = ctx.import_index(sl.build_params(w), SC.import_arrays(case))
    q, tau, mask, out = _decode_args(idx, w)
    hc = ctx.h
    ctx.close()
    L = sl.lib()
    assert L.sekv_route(hc, idx.h, 0, w.L, q.data_ptr(), tau.data_ptr(), 0, mask.data_ptr(), None) == ESTATE
    p = sl.build_params(w)
    hx = C.c_void_p()
    arr = {k: np.ascontiguousarray(v) for k, v in SC.import_arrays(case).items()}
    hi = sl.HostIndex(**{k: v.ctypes.data for k, v in arr.items()})
    assert L.sekv_index_import(hc, C.byref(p), C.byref(hi), C.byref(hx)) == ESTATE
    assert not hx.value
    L.sekv_destroy(hc)             # a second destroy is a no-op
    idx.free()                     # the index outlives its context and still frees


def test_index_on_another_context_is_refused(sl, case):
    w = case.w
    a, b = sl.Context(0), sl.Context(0)
    idx = a.import_index(sl.build_params(w), SC.import_arrays(case))
    q, tau, mask, out = _decode_args(idx, w)
    assert sl.lib().sekv_route(b.h, idx.h, 0, w.L, q.data_ptr(), tau.data_ptr(), 0, mask.data_ptr(),
                               None) == ESTATE
    idx.free()
    a.close()
    b.close()


def test_ring_larger_than_the_device_is_enomem(sl, case):
    """A pinned-tier ring of 1 PiB cannot be allocated: SEKV_ENOMEM, no index,
    and the context keeps working."""
    w = case.w
    ctx = sl.Context(0)
    with pytest.raises(sl.SekvError) as e:
        ctx.import_index(sl.build_params(w, tier=sl.TIER_PINNED_HOST, ring_bytes=1 << 50), SC.import_arrays(case))
    assert e.value.status == ENOMEM
    idx = ctx.import_index(sl.build_params(w, tier=sl.TIER_PINNED_HOST), SC.import_arrays(case))
    q, tau, mask, out = _decode_args(idx, w)
    idx.route(0, w.L, q, tau, 0, mask)
    idx.decode_attend(0, w.L, q, mask, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    idx.free()
    ctx.close()


def test_misaligned_inputs_are_refused(sl, case):
    """The kernels read q, K, V and W with 16-byte loads and the masks as
    64-bit words: a pointer off that alignment is SEKV_EINVAL, refused on the
    host before any work, and the context keeps working."""
    EINVAL = 1
    w = case.w
    ctx = sl.Context(0)
    idx = ctx.import_index(sl.build_params(w), SC.import_arrays(case))
    q, tau, mask, out = _decode_args(idx, w)
    qb = torch.zeros(q.numel() + 8, dtype=torch.bfloat16, device="cuda")   # q at +2 bytes
    mb = torch.zeros(mask.numel() + 1, dtype=torch.int64, device="cuda")    # mask at +4 bytes
    L = sl.lib()
    assert L.sekv_route(ctx.h, idx.h, 0, w.L, qb.data_ptr() + 2, tau.data_ptr(), 0, mask.data_ptr(), None) == EINVAL
    assert b"aligned" in L.sekv_last_error()
    assert L.sekv_route(ctx.h, idx.h, 0, w.L, q.data_ptr(), tau.data_ptr(), 0, mb.data_ptr() + 4, None) == EINVAL
    assert L.sekv_route_pooled(ctx.h, idx.h, 0, w.L, qb.data_ptr() + 2, tau.data_ptr(), 0, mask.data_ptr(),
                               None) == EINVAL
    assert L.sekv_decode_attend(ctx.h, idx.h, 0, w.L, qb.data_ptr() + 2, mask.data_ptr(), out.data_ptr(),
                                None) == EINVAL
    assert L.sekv_decode_attend_noalloc(ctx.h, idx.h, 0, w.L, q.data_ptr(), mb.data_ptr() + 4, out.data_ptr(),
                                        None) == EINVAL
    assert L.sekv_calibrate_tau(ctx.h, idx.h, 0, w.L, qb.data_ptr() + 2, C.c_float(0.1), tau.data_ptr()) == EINVAL
    # the build: K off by 2 bytes
    H, K, V, W, _ = SC.make_inputs(w)
    Kb = torch.zeros(K.numel() + 8, dtype=torch.bfloat16, device="cuda")
    Vd, Hd, Wd = V.cuda().contiguous(), H.cuda().contiguous(), W.cuda().contiguous()
    hx = C.c_void_p()
    p = sl.build_params(w)
    assert L.sekv_build_index(ctx.h, C.byref(p), C.c_void_p(Kb.data_ptr() + 2), C.c_void_p(Vd.data_ptr()),
                              C.c_void_p(Hd.data_ptr()), C.c_void_p(Wd.data_ptr()), None, C.byref(hx)) == EINVAL
    assert not hx.value
    # aligned calls still work
    idx.route(0, w.L, q, tau, 0, mask)
    idx.decode_attend(0, w.L, q, mask, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    idx.free()
    ctx.close()

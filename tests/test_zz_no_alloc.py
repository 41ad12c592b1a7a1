"""sekv_decode_attend_noalloc (the decode entry point that allocates nothing:
its partials live in the library's static device scratch) against
sekv_decode_attend on the same inputs, through the C ABI: two calls in a row,
the second smaller (fewer layers, then a smaller index), bit-identical
outputs; a call whose partials exceed the scratch is refused."""
import math

import numpy as np
import pytest
import torch

from compressed_kv_cache_sekv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from compressed_kv_cache_sekv_amd import lib
    return lib


@pytest.fixture(scope="module")
def ctx(sl):
    c = sl.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


def _built(ctx, sl, w):
    H, K, V = synth.kv_cache(w, device="cuda")
    W = torch.stack([synth.routing_w(w, l, "cuda") for l in range(w.L)])
    return ctx.build_index(sl.build_params(w, tier=sl.TIER_HBM), K, V, H, W, None)


def _routed(idx, w, step):
    tau = torch.zeros(w.L, w.Hq, device="cuda")
    idx.calibrate_tau(0, w.L, synth.calibration_query(w, "cuda"), 0.1, tau)
    q = synth.query(w, step, "cuda")
    mask = torch.zeros(w.B, w.L, w.Hq, idx.mask_words, dtype=torch.int64, device="cuda")
    cap = int(math.floor(0.1 * int(idx.n_spans.min())))
    idx.route(0, w.L, q, tau, cap, mask, None)
    return q, mask


def _both(idx, w, q, mask, lb, lc):
    ref = torch.zeros(w.B, lc, w.Hq, w.d, device="cuda")
    got = torch.full((w.B, lc, w.Hq, w.d), float("nan"), device="cuda")
    qs, ms = q[:, lb:lb + lc].contiguous(), mask[:, lb:lb + lc].contiguous()
    idx.decode_attend(lb, lc, qs, ms, ref)
    idx.decode_attend_noalloc(lb, lc, qs, ms, got)
    torch.cuda.synchronize()
    return ref.cpu(), got.cpu()


def test_noalloc_matches_decode_attend(ctx, sl):
    w = synth.WORKLOADS["llama8b_l32_128k"].scaled(L=2, T=16384, tier="hbm")
    idx = _built(ctx, sl, w)
    q, mask = _routed(idx, w, 0)
    assert int(mask.count_nonzero()) > 0
    # call 1: both layers; call 2: the second layer alone (a smaller call)
    for lb, lc in ((0, 2), (1, 1)):
        ref, got = _both(idx, w, q, mask, lb, lc)
        assert torch.isfinite(got).all()
        assert torch.equal(ref, got), (lb, lc)
        print(f"[noalloc] layers [{lb}, {lb + lc}): identical to sekv_decode_attend", flush=True)
    # a smaller index right after: the scratch holds the last call's partials
    w2 = synth.WORKLOADS["llama8b_l1_32k"].scaled(T=4096)
    idx2 = _built(ctx, sl, w2)
    q2, mask2 = _routed(idx2, w2, 1)
    ref, got = _both(idx2, w2, q2, mask2, 0, 1)
    assert torch.equal(ref, got)
    print("[noalloc] smaller index: identical to sekv_decode_attend", flush=True)
    idx2.free()
    idx.free()


def test_noalloc_refuses_more_than_its_scratch(ctx, sl):
    """64 sequences x 8 KV heads of one item each over 48 layers: 48 x 512
    items x 4 heads x 130 floats = 51 MB of partials, above the 40 MiB
    scratch.  The call is refused before any device work; sekv_decode_attend
    serves it."""
    w = synth.WORKLOADS["llama8b_l32_128k"].scaled(L=48, T=512, B=64, tier="hbm")
    idx = _built(ctx, sl, w)
    q = synth.query(w, 0, "cuda")
    mask = torch.zeros(w.B, w.L, w.Hq, idx.mask_words, dtype=torch.int64, device="cuda")
    out = torch.zeros(w.B, w.L, w.Hq, w.d, device="cuda")
    with pytest.raises(sl.SekvError) as e:
        idx.decode_attend_noalloc(0, w.L, q, mask, out)
    assert e.value.status == 4 and "scratch" in str(e.value)
    assert not out.count_nonzero()
    idx.decode_attend(0, w.L, q, mask, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    idx.free()

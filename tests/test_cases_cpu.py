"""CPU checks of the test machinery itself: the conversion of exported index
arrays back into oracle indexes, and the score-window exclusion rules."""
import numpy as np

from compressed_kv_cache_sekv_amd import synth
from tests import sekv_cases as SC


def test_index_from_export_round_trip():
    """The import layout the oracle's index is written in converts back to
    the same oracle index, whole and one KV head at a time."""
    w = synth.WORKLOADS["llama8b_l1_32k"].scaled(T=1500, B=2, L=2, Hq=8, Hkv=2, d=32, R=16, dprime=8)
    c = SC.make_case(w)
    arr = SC.import_arrays(c)
    ns, nr = [i.n_spans for i in c.idxs], [i.n_raw for i in c.idxs]
    ix = SC.index_from_export(arr, ns, nr, w.L, w.Hq, w.Hkv, w.d, w.R, w.dprime)
    for a, b in zip(ix, c.idxs):
        for f in ("kres", "vres", "s", "uk", "uv", "vkt", "vvt", "smk", "smv"):
            assert np.array_equal(getattr(a, f), getattr(b, f)), f
        assert np.array_equal(a.split.spans, b.split.spans) and np.array_equal(a.split.raw, b.split.raw)
    G = w.Hq // w.Hkv
    ix1 = SC.index_from_export(arr, ns, nr, w.L, w.Hq, w.Hkv, w.d, w.R, w.dprime, kv_head=1)
    for a, b in zip(ix1, c.idxs):
        assert np.array_equal(a.kres[:, 0], b.kres[:, 1]) and np.array_equal(a.uk[:, 0], b.uk[:, 1])
        assert np.array_equal(a.s, b.s[:, G:2 * G]) and np.array_equal(a.vvt[:, 0], b.vvt[:, 1])


def test_score_window_bounds_fp32_arithmetic():
    """The score window holds the fp32 score, computed in a few summation
    orders, within its bound of the fp64 score."""
    rng = np.random.default_rng(3)
    dp, d, N = 64, 128, 400
    W = (rng.standard_normal((dp, d)) / np.sqrt(d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    s = (rng.standard_normal((dp, N)) * 4).astype(np.float32)
    exact = (W.astype(np.float64) @ q.astype(np.float64)) @ s.astype(np.float64)
    win = SC.score_window(W, q, s)
    u32 = (W @ q).astype(np.float32)                                # one order
    u_rev = np.array([np.float32(sum(np.float32(W[j, k]) * q[k] for k in range(d)[::-1]))
                      for j in range(dp)], np.float32)             # a sequential order
    for u in (u32, u_rev):
        a32 = np.array([np.float32(sum((u * s[:, n]).astype(np.float32))) for n in range(N)])
        assert np.all(np.abs(a32 - exact) <= win)


def test_boundary_uncertain_only_near_the_boundary():
    a = np.array([10.0, 9.0, 8.0, 7.0, 6.9999, 3.0])
    win = np.full(6, 1e-3)
    routed = np.array([True, True, True, True, True, False])
    kept = np.array([True, True, True, True, False, False])
    # last kept 7.0, first dropped 6.9999: both within the windows of each other
    ex = SC.boundary_uncertain(a, win, routed, kept, (7.0, 1e-3, 6.9999, 1e-3))
    assert ex.tolist() == [False, False, False, True, True, False]
    # a clear gap excludes nothing
    kept2 = np.array([True, True, True, False, False, False])
    ex2 = SC.boundary_uncertain(a, win, routed, kept2, (8.0, 1e-3, 7.0, 1e-3))
    assert not ex2.any()

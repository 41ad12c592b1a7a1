"""Budget-cap selection paths of the routing kernels, on one 8B-shaped layer at
131072 tokens (N_S = 2628 spans) whose index the library builds on the GPU.

The cap rule (SeKV article, section 기술 상세 (Technical details): spans taken
in descending alpha until the budget holds; here the cap largest scores
a = (W q) . s, the order of alpha, ties to the lower span index) is checked
against the oracle routing the library's own exported summary keys, masks
bit-exact outside the score windows.  This file makes every selection path
of the cap kernel run:
  bin     one histogram over the candidates' key range (boundary bin kept
          whole, or its keys ranked against each other)
  radix   a boundary bin of more than 256 keys (a group of spans with equal
          summary keys, so equal scores on both sides, split by the cap)
  global  more than 2048 candidates
"""
import math
import types

import numpy as np
import pytest
import torch

from compressed_kv_cache_sekv_amd import synth
from oracle import sekv_oracle as O
from tests import sekv_cases as SC

pytestmark = pytest.mark.gpu

CAP_LIST, CAP_BINS, CAP_RANK = 2048, 1024, 256


@pytest.fixture(scope="module")
def setup():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from compressed_kv_cache_sekv_amd import lib as sl
    ctx = sl.Context(0)
    w = synth.WORKLOADS["llama8b_l32_128k"].scaled(L=1, tier="hbm")
    print("[cap paths] building the 128K layer index on the GPU", flush=True)
    H, K, V = synth.kv_cache(w, device="cuda")
    W = torch.stack([synth.routing_w(w, 0, "cuda")])
    idx = ctx.build_index(sl.build_params(w), K, V, H, W, None)
    del H, K, V
    yield sl, ctx, w, idx, W.cpu()
    torch.cuda.synchronize()
    idx.free()
    ctx.close()


def _keys_of(idx, w):
    """The library's summary keys as the oracle reads them (one sequence)."""
    n = int(idx.n_spans[0])
    s = idx.export(fields=("s",))["s"].reshape(w.L, w.Hq, w.dprime, n).astype(np.float64)
    return [types.SimpleNamespace(s=s)]


def _route(idx, w, q, tau, cap):
    Wd = idx.mask_words
    mask = torch.zeros(w.B, 1, w.Hq, Wd, dtype=torch.int64, device="cuda")
    idx.route(0, 1, q.cuda(), torch.as_tensor(tau, dtype=torch.float32).reshape(1, w.Hq).cuda(), cap, mask, None)
    torch.cuda.synchronize()
    return mask.cpu().numpy().view(np.uint64)


def _order_keys(a):
    """Order keys of the scores rounded to fp32 (the kernel's key, up to the
    score window), for the path census only."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.int64)
    return np.where(u >> 31, u ^ 0xFFFFFFFF, u | 0x80000000)


def _path(a, z, cap):
    """Which selection the kernel takes for this head (for coverage only)."""
    nc = int(z.sum())
    if nc <= cap:
        return "none"
    if nc > CAP_LIST:
        return "global"
    bits = _order_keys(a[z])
    lo, hi = int(bits.min()), int(bits.max())
    sh = max(0, (hi - lo).bit_length() - 10)
    cnt = np.bincount((bits - lo) >> sh, minlength=CAP_BINS)[::-1]
    cum = np.cumsum(cnt)
    i = int(np.searchsorted(cum, cap))
    m, r = int(cnt[i]), cap - (int(cum[i - 1]) if i else 0)
    if r == m:
        return "bin-whole"
    return "bin-rank" if m <= CAP_RANK else "radix"


def _tau_quantile(idxs, W, q, frac):
    """Per head: the alpha threshold midway (in score) between the k-th and
    (k+1)-th largest score, k = frac * N_S, as fp32 values."""
    out = []
    for h in range(W.shape[1]):
        a = np.sort(O.routing_score(W[0, h].double().numpy(), q[0, 0, h].double().numpy(), idxs[0].s[0, h]))[::-1]
        k = int(frac * len(a))
        t = 0.5 * (a[k - 1] + a[k])
        out.append(float(np.float32(1.0 / (1.0 + math.exp(-t)))))
    return np.array(out)[None]


def _check(idx, idxs, w, W, q, tau, cap, paths, label, boundary_windows=True):
    words = _route(idx, w, q, tau[0], cap)
    ref = SC.route_ref(idxs, W, q, tau, cap, boundary_windows=boundary_windows)
    SC.check_masks(lambda k: words[k], ref, label)
    for k, z in ref.z_pre.items():
        p = _path(ref.score[k], z, cap)
        paths[p] = paths.get(p, 0) + 1
    print(f"[cap paths] {label}: cap {cap}, paths so far {paths}", flush=True)
    return ref


def test_cap_selection_paths(setup):
    sl, ctx, w, idx, W = setup
    n = int(idx.n_spans[0])
    cap = int(np.floor(w.cap_frac * n))
    assert n > CAP_LIST
    q = synth.query(w, 0)
    idxs = _keys_of(idx, w)
    paths = {}
    # bin: about 20% routed, twice the cap
    _check(idx, idxs, w, W, q, _tau_quantile(idxs, W, q, 0.2), cap, paths, "20% routed")
    # global: everything routed
    _check(idx, idxs, w, W, q, np.full((1, w.Hq), -np.inf), cap, paths, "all routed")
    # radix: 300 spans of every head share one summary key whose score lies
    # above all the others, so the cap splits a group of exactly equal scores
    ex = idx.export()
    arr = dict(ex, n_spans=idx.n_spans.copy(), n_raw=idx.n_raw.copy(), W=W.numpy().astype(np.float32).ravel())
    s = idxs[0].s.copy()
    group = np.arange(5, 5 + 8 * 300, 8)
    for h in range(w.Hq):
        u = W[0, h].double().numpy() @ q[0, 0, h].double().numpy()
        top = float(np.max(u @ s[0, h]))
        v = (u * (top + 8.0) / float(u @ u)).astype(np.float32).astype(np.float64)
        s[0, h][:, group] = v[:, None]
    arr["s"] = s.astype(np.float32).ravel()
    tie = ctx.import_index(sl.build_params(w), arr)
    tidx = [types.SimpleNamespace(s=s)]
    tau = _tau_quantile(tidx, W, q, 0.2)
    ref = _check(tie, tidx, w, W, q, tau, cap, paths, "300 equal scores per head", boundary_windows=False)
    for k in ref.score:
        others = np.delete(ref.score[k], group)
        assert np.all(np.abs(others - ref.score[k][group[0]]) > 1.0)
        assert len(set(ref.score[k][group].tolist())) == 1
        assert ref.z[k][group].sum() == cap and ref.z[k][group[:cap]].all()
    tie.free()
    assert paths.get("global", 0) >= 1
    assert paths.get("bin-whole", 0) + paths.get("bin-rank", 0) >= 1
    assert paths.get("radix", 0) >= 1


def test_cap_repeated_calls(setup):
    """The cap over the library's own score scratch, in consecutive calls
    whose queries differ: each call's capped mask must follow that call's
    scores, never values left in the scratch by the call before."""
    sl, ctx, w, idx, W = setup
    n = int(idx.n_spans[0])
    cap = int(np.floor(w.cap_frac * n))
    idxs = _keys_of(idx, w)
    cases = []
    for s in (0, 1, 2):
        q = synth.query(w, s)
        tau = _tau_quantile(idxs, W, q, 0.2)
        cases.append((q, tau, SC.route_ref(idxs, W, q, tau, cap)))
    mask = torch.zeros(w.B, 1, w.Hq, idx.mask_words, dtype=torch.int64, device="cuda")
    for rep in range(3):
        for i, (q, tau, ref) in enumerate(cases):
            idx.route(0, 1, q.cuda(), torch.as_tensor(tau, dtype=torch.float32).cuda(), cap, mask, None)
            torch.cuda.synchronize()
            got = mask.cpu().numpy().view(np.uint64)
            SC.check_masks(lambda k: got[k], ref, f"repeat {rep} query {i}")
